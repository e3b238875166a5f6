// gmm_tgmm.hpp -- the transposed grouped matmul on gfx950: for each active
// group h, out[h] = lhs_g^T . rhs_g over the group's rows (g = s + h), the
// weight gradient of gmm; an empty group's output is zero.  The Megablox
// metadata builder keeps a tile for every empty group for exactly this
// operation (tpu-inference wheel diff page, megablox/gmm.py,
// make_group_metadata, visit_empty_groups).
//
// An output tile is 256 (k) x 256 (n) of one group, computed by the big
// kernel's machinery (gmm_big.hpp): eight waves of 128 x 64 (64 x 64 over
// the valid half of a tile with at most 128 valid rows or columns),
// 32x32x16 bf16 MFMAs with the column-side fragment as the first operand,
// a four-stage ring of direct-to-LDS loads running three steps ahead across
// the workgroup's tiles, and the same epilogue.  The contraction runs over
// the group's rows, 32 per step.  Both operands are row-major with the
// contraction as their row index, so both are staged like the big kernel's
// [G,K,N] weight -- 512-byte rows of 256 columns -- and both fragments come
// from LDS transpose reads.  The step's row offset is part of the
// range-checked vector offset, so the rows past the group's end (the
// contraction tail) read as zeros; a tile runs at least five steps (the
// phased loop's minimum), the extra ones reading zeros.
//
// Tiles are handed out dynamically, per XCD: the active groups, largest
// first, are dealt to eight queues (one per XCD) so that each queue gets the
// same number of contraction steps (each to the least-loaded queue), and the
// workgroups of an XCD take their queue's tiles in order with an atomic
// counter, so a group's tiles share that XCD's L2 and the long contractions
// are spread first, the short ones filling in behind.  The counters are the
// caller's (Params::queue: a block of the handle's per stream); the last
// workgroup of a queue to finish resets its counters for the next call.
#pragma once

#include "gmm_big.hpp"

namespace gmmk {

template <bool OUT_F32_>
struct TgCfg {
  static constexpr bool OUT_F32 = OUT_F32_;
  static constexpr int BM = 256, BN = 256;  // output tile: k rows x n columns
  static constexpr int WM = 2, WN = 4, NWAVES = WM * WN, T = 64 * NWAVES;
  static constexpr int FM = 4, FN = 2;      // 32 x 32 blocks of a full-tile wave (128 x 64)
  static constexpr int BK = 32;             // contraction rows per step
  static constexpr int ROWB = 512;          // bytes of one 256-column operand row
  static constexpr int A_BYTES = BK * ROWB, B_BYTES = BK * ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int S = 4;  // stages in the ring
  static constexpr int RING = S * STAGE;
  static constexpr int DMA_STEP = 4;  // 1 KB direct-to-LDS loads per wave and step (two per operand)
  static constexpr int MIN_STEPS = 5;
  static constexpr int es_out = OUT_F32 ? 4 : 2;
  // epilogue stores per wave and tile (as in the big kernel)
  static constexpr int ST_BLOCK = OUT_F32 ? 4 : 2;
  static constexpr int E = FM * FN * ST_BLOCK;
  static_assert(A_BYTES == NWAVES * 2 * 1024, "two 1 KB loads per wave and operand");
};

struct TgItem {
  int h;           // active group
  int rlo, nrow;   // the group's first row and row count (the contraction)
  int steps;       // contraction steps of this tile (at least MIN_STEPS)
  BigItem out;     // output tile as rows h * K + k0 .. of the [Ga*K, N] output
};

// Scheduling units: a group's tiles, or, for a group whose tiles are long,
// one of the four quadrants of its tile grid (k-tiles [0, ka) or [ka, nkt),
// n-tiles [0, na) or [na, nnt)), so that its tiles can spread over several
// queues.  A unit is an int: the active group in bits 0..9, the quadrant in
// bits 10 (upper k half) and 11 (upper n half), bit 12 set for a quadrant.
constexpr int kMaxSplit = 128;                          // groups split at most
constexpr int kMaxUnits = kMaxGroups + 3 * kMaxSplit;  // units at most

struct TgGrid {
  int nkt, nnt, ka, na;
};

// The unit of queue tile L: the last of the queue's units [*cur, u_end) whose
// first tile (ustart, increasing along a queue) is at most L, 64 at a time
// with a ballot.  A workgroup's tile indices only grow, so the search starts
// from its previous unit (*cur).
__device__ __forceinline__ int tg_find_unit(const int* ustart, int* cur, int u_end, int L, int lane) {
  int u = *cur;
  while (true) {
    const int k = u + 1 + lane;
    const bool le = k < u_end && ustart[k] <= L;
    const int c = __popcll(__ballot(le));
    u += c;
    if (c < 64) break;
  }
  *cur = u;
  return u;
}

// Tile L of a queue: its unit, then k-tile, then n-tile within the unit.
template <class C>
__device__ __forceinline__ TgItem decode_tg(const Plan& pl, const int* units, const int* ustart, int* cur,
                                            int u_end, int L, const TgGrid& gr, int K, int N, int w, int lane) {
  TgItem it;
  const int u = tg_find_unit(ustart, cur, u_end, L, lane);
  const int d = __builtin_amdgcn_readfirstlane(units[u]);
  const int t = L - __builtin_amdgcn_readfirstlane(ustart[u]);
  const int h = d & 1023;
  int kt, nt;
  if (d & 4096) {
    const int k0 = (d & 1024) ? gr.ka : 0, n0 = (d & 2048) ? gr.na : 0;
    const int bw = (d & 2048) ? gr.nnt - gr.na : gr.na;
    kt = k0 + t / bw;
    nt = n0 + t % bw;
  } else {
    kt = t / gr.nnt;
    nt = t % gr.nnt;
  }
  it.h = h;
  it.rlo = __builtin_amdgcn_readfirstlane(pl.row_start[h]);
  it.nrow = __builtin_amdgcn_readfirstlane(pl.row_start[h + 1] - pl.row_start[h]);
  const int st = (it.nrow + C::BK - 1) / C::BK;
  it.steps = st < C::MIN_STEPS ? C::MIN_STEPS : st;
  BigItem& o = it.out;
  const int k0 = kt * C::BM;
  o.h = it.h;
  o.row0 = it.h * K + k0;
  o.rows = K - k0 < C::BM ? K - k0 : C::BM;
  o.n0 = nt * C::BN;
  o.ncols = N - o.n0 < C::BN ? N - o.n0 : C::BN;
  const bool half_m = o.rows <= C::BM / 2, half_n = o.ncols <= C::BN / 2;
  o.half = half_m || half_n;
  if (!o.half) {  // 2 x 4 waves of 128 x 64
    o.rbase = (w / C::WN) * 128;
    o.cbase = (w % C::WN) * 64;
  } else if (!half_n) {  // 2 x 4 waves of 64 x 64 over 128 x 256
    o.rbase = (w / 4) * 64;
    o.cbase = (w % 4) * 64;
  } else {  // 4 x 2 waves of 64 x 64 over 256 x 128
    o.rbase = (w / 2) * 64;
    o.cbase = (w % 2) * 64;
  }
  return it;
}

// Direct-to-LDS sources of one tile: buffer resources over the group's rows
// from the tile's first column (zero-size past the end of the stream).
// Columns past the tile's valid part are loaded too (the next columns of
// the row, or zeros past the group): they only feed output rows and columns
// that the epilogue's range check drops.
struct TgDma {
  __amdgpu_buffer_rsrc_t ra, rb;
};

template <class C>
__device__ __forceinline__ TgDma tg_dma(const Params& p, const TgItem& it, bool live) {
  const int K = p.K, N = p.N;
  TgDma d;
  const BigItem& o = it.out;
  const int k0 = o.row0 - it.h * K;
  const char* a = reinterpret_cast<const char*>(p.lhs) + ((long long)it.rlo * K + k0) * 2;
  const char* b = reinterpret_cast<const char*>(p.rhs) + ((long long)it.rlo * N + o.n0) * 2;
  const int abytes = it.nrow * K * 2 - k0 * 2, bbytes = it.nrow * N * 2 - o.n0 * 2;
  d.ra = uniform_rsrc(a, live && abytes > 0 ? abytes : 0);
  d.rb = uniform_rsrc(b, live && bbytes > 0 ? bbytes : 0);
  return d;
}

// This lane's offsets: instruction i of a wave fills contraction row
// 4 w + 2 i + lane / 32 of the step, 16-byte chunk lane % 32 of the row,
// which holds the tile's columns 8 c .. 8 c + 7 with c = (lane % 32) ^
// swz_nn(row).
struct TgOff {
  int a[2], b[2];
};

__device__ __forceinline__ TgOff tg_offsets(int K, int N, int w, int lane) {
  TgOff o;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * w + 2 * i + (lane >> 5);
    const int c = (lane & 31) ^ swz_nn(r);
    o.a[i] = r * K * 2 + c * 16;
    o.b[i] = r * N * 2 + c * 16;
  }
  return o;
}

// lane + uniform, added where it is used: the compiler would otherwise
// turn the per-step offsets into per-lane induction variables that stay live
// across the loop (registers the kernel does not have to spare)
__device__ __forceinline__ int add_at_use(int lane_part, int uniform) {
  int r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(uniform), "v"(lane_part));
  return r;
}

// Direct-to-LDS operation J of contraction step k into stage `st`: J = 0, 1
// the lhs, J = 2, 3 the other operand (1 KB each per wave).  The step's row
// offset (sa, sb bytes per step) goes into the range-checked vector offset,
// so rows past the group read as zeros.
template <class C, int J>
__device__ __forceinline__ void tg_dma_op(const TgDma& d, const TgOff& o, int k, int sa, int sb, char* st, int w) {
  if constexpr (J < 2) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (lds_ptr_t)(st + w * 2048 + J * 1024), 16,
                                             add_at_use(o.a[J], k * sa), 0, 0, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rb, (lds_ptr_t)(st + C::A_BYTES + w * 2048 + (J - 2) * 1024), 16,
                                             add_at_use(o.b[J - 2], k * sb), 0, 0, 0);
  }
}

// Per K half the refills issue twelve LDS transpose reads in a fixed order
// (four lhs-side fragments, then two of the other side, two reads each), so
// a half's fragments have completed once at most the twelve reads of the
// following half are outstanding.
__device__ __forceinline__ void tg_frags_ready() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (12 << 8) | (0x3 << 14));
}

// Group order for the tiles: active groups by row count, largest first
// (ties by index).  One thread per group counts the groups ahead of it.
template <int T>
__device__ void tg_order(const Plan& pl, int* order) {
  const int ga = pl.ga;
  for (int h = threadIdx.x; h < ga; h += T) {
    const int sz = pl.row_start[h + 1] - pl.row_start[h];
    int rank = 0;
    for (int j = 0; j < ga; ++j) {
      const int sj = pl.row_start[j + 1] - pl.row_start[j];
      rank += (sj > sz) || (sj == sz && j < h);
    }
    order[rank] = h;
  }
}

// LDS areas.  While the tiles are scheduled, before the first load, the
// ring holds the group order and the deal's per-unit records; past the ring
// lie the queues' unit lists (each queue's units in order, queue after
// queue), the first tile of each unit within its queue, scheduling words, and
// the plan.
template <class C>
struct TgLds {
  static constexpr int ORDER = 0;                        // int[kMaxGroups], in the ring
  static constexpr int REC_UNIT = ORDER + kMaxGroups * 4;  // int[kMaxUnits], in the ring
  static constexpr int REC_POS = REC_UNIT + kMaxUnits * 4;  // int[kMaxUnits], in the ring
  static constexpr int REC_START = REC_POS + kMaxUnits * 4;  // int[kMaxUnits], in the ring
  static_assert(REC_START + kMaxUnits * 4 <= C::RING, "deal records fit the ring");
  static constexpr int UNITS = C::RING;                  // int[kMaxUnits]
  static constexpr int USTART = UNITS + kMaxUnits * 4;   // int[kMaxUnits]
  static constexpr int SCHED = USTART + kMaxUnits * 4;   // int[32], see the kernel
  static constexpr int PLAN = SCHED + 128;
  static constexpr int BYTES = PLAN + sizeof(Plan);
  static_assert(PLAN % 16 == 0, "plan alignment");
};
// scheduling words: the first unit of each queue [0, kQueues], the tiles of
// each queue, and the hand-over slot of a grabbed tile index
constexpr int kSchedOff = 0, kSchedTiles = 12, kSchedSlot = 24;

// Deal the units to nq queues, each to the queue with the least work so far
// (the lowest index on ties), in the group order (largest first), so each
// queue's units are in that order too.  A tile's work is its contraction
// steps plus two for the epilogue.  A group is split into quadrants when its
// tiles take more than a quarter of a workgroup's share of all the work (at
// most kMaxSplit groups, the largest).  Wave 0 runs it: the greedy choice is
// made in scalar registers, unit after unit, recording each unit's queue,
// place in the queue and first tile; the lists are then written in parallel.
template <class C>
__device__ inline void tg_deal(const Plan& pl, const int* order, char* smem, int* units, int* ustart, int* sched,
                               int nq, int P, const TgGrid& gr, int lane) {
  using Lds = TgLds<C>;
  int* const rec_unit = reinterpret_cast<int*>(smem + Lds::REC_UNIT);
  int* const rec_pos = reinterpret_cast<int*>(smem + Lds::REC_POS);
  int* const rec_start = reinterpret_cast<int*>(smem + Lds::REC_START);
  const int ga = pl.ga;
  const int per = gr.nnt * gr.nkt;
  auto tile_cost = [&](int i) {
    const int h = order[i];
    const int st = (pl.row_start[h + 1] - pl.row_start[h] + C::BK - 1) / C::BK;
    return (st < C::MIN_STEPS ? C::MIN_STEPS : st) + 2;
  };
  // all the work, and the scale that keeps the queue loads in 31 bits
  long long total = 0;
  for (int c = 0; c < ga; c += 64) {
    const int cost = c + lane < ga ? tile_cost(c + lane) : 0;
    const int n = ga - c < 64 ? ga - c : 64;
    for (int jj = 0; jj < n; ++jj) total += __builtin_amdgcn_readlane(cost, jj);
  }
  total *= per;
  int shift = 0;
  while ((total >> shift) >= (1ll << 30)) ++shift;
  int load[kQueues], cnt[kQueues], tiles[kQueues];
#pragma unroll
  for (int q = 0; q < kQueues; ++q) {
    load[q] = q < nq ? 0 : 0x7fffffff;
    cnt[q] = 0;
    tiles[q] = 0;
  }
  int k = 0, nsplit = 0;
  for (int c = 0; c < ga; c += 64) {
    const int cost = c + lane < ga ? tile_cost(c + lane) : 0;
    const int h = c + lane < ga ? order[c + lane] : 0;
    const int n = ga - c < 64 ? ga - c : 64;
    for (int jj = 0; jj < n; ++jj) {
      const int cj = __builtin_amdgcn_readlane(cost, jj);
      const int hj = __builtin_amdgcn_readlane(h, jj);
      // a tile longer than a quarter of a workgroup's share: cost > total / (4 P)
      const bool split = per > 1 && nsplit < kMaxSplit && 4ll * P * cj > total;
      nsplit += split;
      for (int qd = 0; qd < (split ? 4 : 1); ++qd) {
        const int nk = !split ? gr.nkt : (qd & 1) ? gr.nkt - gr.ka : gr.ka;
        const int nn = !split ? gr.nnt : (qd & 2) ? gr.nnt - gr.na : gr.na;
        const int nt = nk * nn;
        if (nt == 0) continue;
        int q = 0, best = load[0];
#pragma unroll
        for (int t = 1; t < kQueues; ++t)
          if (load[t] < best) {
            best = load[t];
            q = t;
          }
        const int add = (int)(((long long)cj * nt) >> shift) + 1;
        int pos = 0, first = 0;
#pragma unroll
        for (int t = 0; t < kQueues; ++t) {
          pos = t == q ? cnt[t] : pos;
          first = t == q ? tiles[t] : first;
          load[t] += t == q ? add : 0;
          cnt[t] += t == q ? 1 : 0;
          tiles[t] += t == q ? nt : 0;
        }
        if (lane == 0) {
          rec_unit[k] = hj | (split ? 4096 | qd << 10 : 0);
          rec_pos[k] = q | pos << 4;
          rec_start[k] = first;
        }
        ++k;
      }
    }
  }
  int base[kQueues];
  int acc = 0;
#pragma unroll
  for (int q = 0; q < kQueues; ++q) {
    base[q] = acc;
    if (lane == 0) {
      sched[kSchedOff + q] = acc;
      sched[kSchedTiles + q] = tiles[q];
    }
    acc += cnt[q];
  }
  if (lane == 0) sched[kSchedOff + kQueues] = acc;
  for (int i = lane; i < k; i += 64) {
    const int qp = rec_pos[i];
    const int q = qp & 15;
    int b = 0;
#pragma unroll
    for (int t = 0; t < kQueues; ++t) b = t == q ? base[t] : b;
    units[b + (qp >> 4)] = rec_unit[i];
    ustart[b + (qp >> 4)] = rec_start[i];
  }
}

// atomicAdd(counter, 1) as one instruction of a whole wave that takes part
// (`live`): a buffer atomic over the counter's four bytes, so only lane 0 is
// in range (the other lanes' adds are dropped) and returns the old value.  A
// wave that does not take part issues the same instruction over zero bytes:
// every lane is dropped, but the wave still counts one memory operation, so
// the waits after it are the same in every wave, with no branch around it.
__device__ __forceinline__ int tg_grab_wave(int* counter, int lane, bool live) {
  const __amdgpu_buffer_rsrc_t r = uniform_rsrc(reinterpret_cast<const char*>(counter), live ? 4 : 0);
  return __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, r, lane * 4, 0, 0);
}

template <class C>
__global__ __launch_bounds__(C::T) void gmm_tgmm_kernel(Params p) {
  using Lds = TgLds<C>;
  // one LDS array: the ring, the scheduling tables and the plan
  __shared__ __attribute__((aligned(1024))) char smem[Lds::BYTES];
  int* const order = reinterpret_cast<int*>(smem + Lds::ORDER);
  int* const units = reinterpret_cast<int*>(smem + Lds::UNITS);
  int* const ustart = reinterpret_cast<int*>(smem + Lds::USTART);
  int* const sched = reinterpret_cast<int*>(smem + Lds::SCHED);
  Plan& pl = *reinterpret_cast<Plan*>(smem + Lds::PLAN);
  if (threadIdx.x == 0) pl.flags = 0;
  __syncthreads();
  build_plan<C::T>(p, pl, C::BM);
  report_flags(p, pl);
  tg_order<C::T>(pl, order);
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = lane >> 5, r32 = lane & 31;
  const int K = p.K, N = p.N;
  const int P = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, P);
  TgGrid gr;
  gr.nkt = (K + C::BM - 1) / C::BM;
  gr.nnt = (N + C::BN - 1) / C::BN;
  gr.ka = (gr.nkt + 1) / 2;
  gr.na = (gr.nnt + 1) / 2;
  // queues: one per XCD (workgroup b runs on XCD b % 8) when the grid
  // divides evenly and there are groups enough to deal, else one
  const int nq = P % kQueues == 0 && pl.ga >= 2 * kQueues ? kQueues : 1;
  const int x = blockIdx.x % nq;
  if (w == 0) tg_deal<C>(pl, order, smem, units, ustart, sched, nq, P, gr, lane);
  __syncthreads();
  // this queue's units [ucur, u_end) and tiles [0, n_items)
  int ucur = __builtin_amdgcn_readfirstlane(sched[kSchedOff + x]);
  const int u_end = __builtin_amdgcn_readfirstlane(sched[kSchedOff + x + 1]);
  const int n_items = __builtin_amdgcn_readfirstlane(sched[kSchedTiles + x]);
  int* const counter = p.queue + x;
  const int W = P / nq, j = blockIdx.x / nq;  // workgroups of the queue, this one's place
  // Output groups the plan dropped (a group offset past G - Ga, which is
  // flagged) are zero.  K * N is a multiple of 64, so 16-byte stores tile it.
  {
    const long long b0 = (long long)pl.ga * K * N * C::es_out, b1 = (long long)p.Ga * K * N * C::es_out;
    char* o = reinterpret_cast<char*>(p.out);
    for (long long off = b0 + ((long long)slot * C::T + tid) * 16; off < b1; off += (long long)P * C::T * 16)
      *reinterpret_cast<i32x4*>(o + off) = i32x4{0, 0, 0, 0};
  }
  // The last workgroup of the queue to get here resets its counters; every
  // index this workgroup grabbed has returned by then (each was used).
  auto finish = [&]() {
    if (tid == 0) {
      const int prev = atomicAdd(p.queue + kQueues + x, 1);
      if (prev == W - 1) {
        atomicExch(counter, 0);
        atomicExch(p.queue + kQueues + x, 0);
      }
    }
  };

  // Tile indices: the queue's first two rounds are fixed, workgroup j of the
  // queue's W taking tiles j and 2W-1-j (had each grabbed its first two, the
  // first workgroups would take two of the longest tiles each); afterwards
  // each tile grabs the index of the tile after next during its first steps
  // (so the next tile is known before its loads start), from 2W on.
  int L_cur = j;
  int L_nxt = 2 * W - 1 - j;
  if (L_cur >= n_items) {
    finish();
    return;
  }

  TgItem cur = decode_tg<C>(pl, units, ustart, &ucur, u_end, L_cur, gr, K, N, w, lane);
  bool last_item = L_nxt >= n_items;
  TgItem nxt = cur;
  if (!last_item) nxt = decode_tg<C>(pl, units, ustart, &ucur, u_end, L_nxt, gr, K, N, w, lane);
  TgDma dcur = tg_dma<C>(p, cur, true);
  TgDma dnxt = tg_dma<C>(p, nxt, !last_item);
  const TgOff off = tg_offsets(K, N, w, lane);
  const int sa = C::BK * K * 2, sb = C::BK * N * 2;  // bytes per contraction step

  // Prologue: the first tile's steps 0..2; every older memory operation is
  // complete after the wait, so the loop's counts start from an empty queue.
#pragma unroll
  for (int s = 0; s < C::S - 1; ++s) {
    tg_dma_op<C, 0>(dcur, off, s, sa, sb, smem + s * C::STAGE, w);
    tg_dma_op<C, 1>(dcur, off, s, sa, sb, smem + s * C::STAGE, w);
    tg_dma_op<C, 2>(dcur, off, s, sa, sb, smem + s * C::STAGE, w);
    tg_dma_op<C, 3>(dcur, off, s, sa, sb, smem + s * C::STAGE, w);
  }
  wait_vmcnt<0>();
  __syncthreads();

  // lane part of a fragment address for the first 32 columns of a
  // 128-column half; the next 32 are the same XOR 64 (chunk bit 2, which the
  // K-row swizzle leaves alone) and a block 64 columns on XORs 128
  const int lo0 = nn_lane_off(lane, 0);
  // fragment f of K half h from an operand area: 32 rows (lhs side) or
  // columns (other side) starting 32 f past the wave's first one `base`
  // The XOR is formed at each use (volatile, so it is not hoisted): hoisted,
  // the lane parts of every fragment of both tile layouts stay live across
  // the loop and push the kernel past its register budget into spills.
  auto frag = [&](const char* area, int base, int f, int h) __attribute__((always_inline)) {
    const int cb = base * 2 + f * 64;  // byte offset of the block in a K row
    int lane_part;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(lane_part) : "v"(lo0), "s"(cb & 192));
    const unsigned addr = (unsigned)(size_t)(lds_ptr_t)(area + (cb & ~192)) + (unsigned)lane_part;
    return h ? nn_frag<1>(addr) : nn_frag<0>(addr);
  };
  auto a_frag = [&](const char* st, const TgItem& it, int f, int h) __attribute__((always_inline)) {
    return frag(st, it.out.rbase, f, h);
  };
  auto b_frag = [&](const char* st, const TgItem& it, int f, int h) __attribute__((always_inline)) {
    return frag(st + C::A_BYTES, it.out.cbase, f, h);
  };

  i32x4 a[C::FM][2], b[C::FN][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int f = 0; f < C::FM; ++f) a[f][h] = a_frag(smem, cur, f, h);
#pragma unroll
    for (int f = 0; f < C::FN; ++f) b[f][h] = b_frag(smem, cur, f, h);
  }

  // The transpose reads write their registers when the data arrives, but the
  // compiler takes an asm output as written when the asm issues: a fragment
  // it sees no later use of (a[2..3] in a half tile, or every refill after
  // the last step) would have its registers handed to other values, which
  // the arriving data then overwrites.  Each fragment is therefore used here,
  // after the wait that guarantees its data has arrived.
  auto hold = [&](int h) __attribute__((always_inline)) {
    asm volatile("" ::"v"(a[0][h]), "v"(a[1][h]), "v"(a[2][h]), "v"(a[3][h]), "v"(b[0][h]), "v"(b[1][h]));
  };

  f32x16 acc[C::FM][C::FN];
  int stage = 0;
  int L_new = 0;  // the grabbed index handed over during the current tile

  // One contraction step s (as the big kernel's K step, without a bias
  // row): step s+1's operands are complete once at most WAIT newer
  // operations are outstanding -- step s+2's four loads and, in a tile's
  // first two steps, the previous tile's E stores (and in the second, the
  // tile-index grab issued after the first).  The barrier frees the
  // stage step s-1 used, which takes step s+3 (this tile's step kd, or the
  // next tile's when NEXT); fragments are refilled with step s+1's right
  // after their last use.
  auto kstep = [&](auto full_tag, auto wait_tag, auto next_tag, auto last_tag, int kd)
      __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int WAIT = decltype(wait_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value, LAST = decltype(last_tag)::value;
    constexpr int FMA = FULL ? C::FM : C::FM / 2;
    constexpr int NM = 2 * FMA * C::FN;  // MFMAs per step
    wait_vmcnt<WAIT>();
    if constexpr (LAST) __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    ring_barrier();
    const TgDma& d = NEXT ? dnxt : dcur;
    char* st3 = smem + ((stage + 3) & (C::S - 1)) * C::STAGE;
    const char* st1 = smem + ((stage + 1) & (C::S - 1)) * C::STAGE;
    const TgItem& it1 = LAST ? nxt : cur;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      tg_frags_ready();
      hold(h);
#pragma unroll
      for (int fm = 0; fm < FMA; ++fm) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b[fn][h]),
                                                                __builtin_bit_cast(bf16x8, a[fm][h]),
                                                                acc[fm][fn], 0, 0, 0);
          const int m = (h * FMA + fm) * C::FN + fn;
          if (m == 0 * NM / 4) tg_dma_op<C, 0>(d, off, kd, sa, sb, st3, w);
          if (m == 1 * NM / 4) tg_dma_op<C, 1>(d, off, kd, sa, sb, st3, w);
          if (m == 2 * NM / 4) tg_dma_op<C, 2>(d, off, kd, sa, sb, st3, w);
          if (m == 3 * NM / 4) tg_dma_op<C, 3>(d, off, kd, sa, sb, st3, w);
          __builtin_amdgcn_sched_barrier(0);  // keep this order
        }
        a[fm][h] = a_frag(st1, it1, fm, h);
      }
#pragma unroll
      for (int fm = FMA; fm < C::FM; ++fm) a[fm][h] = a_frag(st1, it1, fm, h);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) b[fn][h] = b_frag(st1, it1, fn, h);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage = (stage + 1) & (C::S - 1);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // a tile's first two steps: the previous tile's E stores are also
  // outstanding, and in the second step the grab too
  using W0 = std::integral_constant<int, C::DMA_STEP + C::E>;
  using W0G = std::integral_constant<int, C::DMA_STEP + C::E + 1>;
  using W1 = std::integral_constant<int, C::DMA_STEP>;
  // One tile of cur.steps >= 5 steps.
  auto ktile = [&](auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int FMA = FULL ? C::FM : C::FM / 2;
    const int KT = cur.steps;
    kstep(full_tag, W0{}, F_{}, F_{}, 3);
    // the grab of the tile after next, by wave 0 unless this tile has no
    // successor: exactly one counted operation in every wave
    const int g = tg_grab_wave(counter, lane, w == 0 && !last_item);
    kstep(full_tag, W0G{}, F_{}, F_{}, 4);
    for (int kt = 2; kt + 3 < KT; ++kt) kstep(full_tag, W1{}, F_{}, F_{}, kt + 3);
    kstep(full_tag, W1{}, T_{}, F_{}, 0);  // kt = KT-3: the next tile's step 0
    // the grab has returned (this step's wait left only the loads of the
    // step before outstanding); hand it to every wave, which reads it after
    // the last step's barrier
    if (w == 0 && lane == 0 && !last_item) sched[kSchedSlot] = g;
    kstep(full_tag, W1{}, T_{}, F_{}, 1);
    kstep(full_tag, W1{}, T_{}, T_{}, 2);
    // every refill has landed before the epilogue takes registers of its own
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    hold(0);
    hold(1);
    L_new = 2 * W + __builtin_amdgcn_readfirstlane(sched[kSchedSlot]);
    // the last step's stage holds the epilogue's staging slices, 4 KB per wave
    big_epilogue<C, FMA, false>(p, acc, cur.out, smem, smem + ((stage + 3) & (C::S - 1)) * C::STAGE + w * 4096, kh, r32,
                         lane);
  };

  while (true) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int z = 0; z < 16; ++z) acc[i][j][z] = 0.f;
    if (!cur.out.half)
      ktile(std::true_type{});
    else
      ktile(std::false_type{});
    if (last_item) break;
    L_nxt = L_new;
    last_item = L_nxt >= n_items;
    cur = nxt;
    dcur = dnxt;
    if (!last_item) nxt = decode_tg<C>(pl, units, ustart, &ucur, u_end, L_nxt, gr, K, N, w, lane);
    dnxt = tg_dma<C>(p, nxt, !last_item);
  }
  finish();
}

}  // namespace gmmk
