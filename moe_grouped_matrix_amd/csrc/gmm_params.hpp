// gmm_params.hpp -- kernel arguments and constants shared by the host
// launchers and the device code of the gfx950 grouped matmul.
#pragma once

#include <stdint.h>

namespace gmmk {

// Operand type fed to the matrix cores.
enum class Op { F32, BF16, FP8, I8 };

constexpr int kMaxGroups = 1024;
constexpr int kQueues = 8;  // one per XCD
// The transposed product's counter block (int32 words, all zero between
// calls): [0, kQueues) the dynamic schedule's tile counters, [kQueues,
// 2 kQueues) finished workgroups per queue, kGangNext the gang schedule's
// next group, kGangDone finished workgroups of the grid, and from
// kGangMeet one 64-bit meet word per queue (8-byte aligned).
constexpr int kGangNext = 2 * kQueues, kGangDone = kGangNext + 1;
constexpr int kGangMeet = kGangNext + 4;
constexpr int kQueueWords = kGangMeet + 2 * kQueues;
constexpr uint32_t kFlagNegative = 0x1u;
constexpr uint32_t kFlagExceed = 0x2u;
constexpr uint32_t kFlagBadOffset = 0x4u;
constexpr uint32_t kFlagSchedule = 0x8u;
// What the rows outside the active groups receive.
enum Fill : int32_t { kFillZero = 0, kFillCopy = 1, kFillKeep = 2 };
// Bytes of inactive rows filled by one work item.
constexpr int kZeroChunk = 64 * 1024;
// dword 3 of a raw buffer resource on gfx9-family parts (32-bit data format).
constexpr int kBufferRsrcWord3 = 0x00020000;

struct Params {
  const void* lhs;
  const void* rhs;
  const int32_t* group_sizes;
  const int32_t* group_offset;  // device scalar or nullptr
  const float* rhs_scale;       // [Ga, nb, 1, N] or nullptr
  const void* rhs_bias;         // [Ga, 1, N] or nullptr
  const float* lhs_scale;       // [M, nb] or nullptr
  void* out;                    // [M, N]
  // rows outside the active groups: zeros (kFillZero), the rows of
  // `existing` (kFillCopy), or left as they are (kFillKeep: existing is out)
  const void* existing;         // [M, N] like out, or nullptr
  int32_t fill;
  uint32_t* flags;
  // the transposed product's counter block (kQueueWords int32, zero between
  // calls)
  int32_t* queue;
  int32_t M, K, N, G, Ga, nb, blk;
  int32_t bias_f32, out_f32;
};

}  // namespace gmmk
