// gmm_tgmm.hpp -- the transposed grouped matmul on gfx950: for each active
// group h, out[h] = lhs_g^T . rhs_g over the group's rows (g = s + h), the
// weight gradient of gmm; an empty group's output is zero.  The Megablox
// metadata builder keeps a tile for every empty group for exactly this
// operation (tpu-inference wheel diff page, megablox/gmm.py,
// make_group_metadata, visit_empty_groups).
//
// The contraction runs over the group's rows, 32 per step.  Both operands
// are row-major with the contraction as their row index, so a step stages
// 32 rows of each operand's column slices in LDS and the MFMA fragments come
// from LDS transpose reads.  A stage is four areas of 32 rows x 128 columns
// (256-byte rows); an output tile takes its lhs columns from the first `na`
// areas and its rhs columns from the rest: 256 x 256 tiles two and two,
// 384 x 128 tiles three and one, 128 x 384 tiles one and three.  Eight
// waves, two per SIMD, compute 128 x 64 (96 x 64, 64 x 96) each with
// 32x32x16 bf16 MFMAs, the rhs-side fragment first; a four-stage ring of
// direct-to-LDS loads runs three steps ahead, across the workgroup's tiles;
// the epilogue is the big kernel's, staged through LDS.  The step's row
// offset is part of the range-checked vector offset, so the rows past the
// group's end (the contraction tail) read as zeros; a tile runs at least
// five steps (the phased loop's minimum), the extra ones reading zeros.
//
// Two schedules, both with one work queue per XCD (workgroup b runs on XCD
// b mod 8) when the grid is a multiple of 8 and there are at least 16
// groups:
//  - Gang: when a group's output splits into T <= W tiles of the shapes in
//    gmm_tgmm_tiles.hpp, T >= 3/4 of the W workgroups of a queue: the
//    queues take the groups (largest first) one at a time, each next group
//    going to the queue that needs one first, and workgroup j of a queue
//    computes tile j of each of its queue's groups in turn.  All of a
//    group's tiles then run side by side on one XCD and read each
//    contraction row of both operands at about the same time, once from
//    HBM into that XCD's L2.  The workgroups drift apart as they go; so
//    that none runs ahead into the next group alone, each workgroup, before
//    it queues the next group's first loads, meets the queue's other
//    workgroups (tg_gang_meet), where the queue's leader also hands out the
//    group after it.  Taking groups as they are needed lets an XCD that
//    runs faster take more of them (measured: the XCDs of one GPU ran the
//    same number of steps and group boundaries up to 4% apart, the same
//    XCDs from run to run).
//  - Dynamic (otherwise): 256 x 256 tiles handed out through the queues'
//    atomic counters, largest groups first.
// The counters are the caller's (Params::queue: a block of the handle's per
// stream, or the library's static scratch); in either schedule the last
// workgroup of a queue to finish resets them for the next call.
#pragma once

#include "gmm_big.hpp"
#include "gmm_tgmm_tiles.hpp"

namespace gmmk {

template <bool OUT_F32_>
struct TgCfg {
  static constexpr bool OUT_F32 = OUT_F32_;
  static constexpr int BM = 256, BN = 256;  // dynamic-schedule tile: k rows x n columns
  static constexpr int NWAVES = 8, T = 64 * NWAVES;
  static constexpr int BK = 32;             // contraction rows per step
  static constexpr int AREA_ROW = 256;      // bytes of 128 columns
  static constexpr int AREA = BK * AREA_ROW;
  static constexpr int NAREA = 4;
  static constexpr int STAGE = NAREA * AREA;
  static constexpr int S = 4;  // stages in the ring
  static constexpr int RING = S * STAGE;
  static constexpr int DMA_STEP = 4;  // 1 KB direct-to-LDS loads per wave and step
  static constexpr int MIN_STEPS = 5;
  static constexpr int NSLOT = 6;     // fragment slots per K half
  static constexpr int NACC = 8;      // 32 x 32 accumulator blocks
  static constexpr int es_out = OUT_F32 ? 4 : 2;
  // epilogue stores per wave and tile: the full tile's (the others pad)
  static constexpr int ST_BLOCK = OUT_F32 ? 4 : 2;
  static constexpr int E = NACC * ST_BLOCK;
  static_assert(STAGE == NWAVES * DMA_STEP * 1024, "each wave fills half an area per step");
};

// Per-shape compile-time layout: FM x FN accumulator blocks per wave and the
// first rhs-side fragment slot BS (slots [0, BS) hold lhs-side fragments).
template <int SH>
struct TgShapeCfg {
  static constexpr int FM = SH == kTgFull ? 4 : SH == kTgTall ? 3 : 2;
  static constexpr int FN = SH == kTgWide ? 3 : 2;
  static constexpr int BS = SH == kTgTall ? 3 : SH == kTgWide ? 2 : 4;
  static_assert(FM * FN <= 8 && BS + FN <= 6, "shape fits the accumulators and slots");
};

// Gang schedule meets.  The T workgroups of a queue take the queue's groups
// together; meet m (m = 0, 1, ... in every one of them) comes before the
// loads of their (m+1)-th group.  The queue's leader (workgroup 0) brings to
// meet m the list index of the queue's (m+2)-th group, which it takes from
// the grid's counter (the first two groups of queue x are list items x and
// 2 kQueues - 1 - x, so the counter starts at item 2 kQueues): an XCD that
// runs faster takes more groups.  One 64-bit word per queue carries both:
// the arrivals in bits 0..23 and, in the 20-bit field 24 + 20 (m % 2), the
// sum of the indices published at meets m, m - 2, ...  At meet m lane 0 of
// wave 0 adds 1 (the leader also its index into the field), then polls
// until all T (m + 1) arrivals are in -- at most kGangSpin polls: that wait
// only keeps the workgroups in step (shared L2 reads) -- and until the field
// has moved past the value this workgroup saw at meet m - 2; the difference
// is the index.  Meet m + 2's leader cannot add to the field before this
// workgroup has arrived at meet m + 1, so the difference is exactly meet
// m's index.  The results depend on that index, so its wait is bounded only
// by kGangLeaderSpin polls (about a second: it ends early only when the
// grid's workgroups cannot all run at once); past it the workgroup sets
// kFlagSchedule and takes no further group.  The atomics' returns and the
// polls are waited for by the compiler (vmcnt 0), which only makes the
// loop's later constant waits hold sooner.
constexpr int kGangSpin = 2048;
constexpr int kGangLeaderSpin = 1 << 20;
constexpr int kGangNone = 0x7fffffff;  // no further group

__device__ __forceinline__ int tg_gang_meet(unsigned long long* word, int* next, uint32_t* flags, int m, int T,
                                            bool leader, int& seen0, int& seen1, int lane) {
  int idx = kGangNone, seen = (m & 1) ? seen1 : seen0;
  if (lane == 0) {
    const int sh = 24 + 20 * (m & 1);
    unsigned long long add = 1;
    if (leader) {
      const int mine = 2 * kQueues + __hip_atomic_fetch_add(next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      add += (unsigned long long)mine << sh;
    }
    unsigned long long v = __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
    const unsigned long long target = (unsigned long long)T * (unsigned long long)(m + 1);
    for (int spin = 0; (v & 0xFFFFFFull) < target && spin < kGangSpin; ++spin) {
      __builtin_amdgcn_s_sleep(4);
      v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    int f = (int)((v >> sh) & 0xFFFFFull);
    for (int spin = 0; f == seen && spin < kGangLeaderSpin; ++spin) {
      __builtin_amdgcn_s_sleep(4);
      v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      f = (int)((v >> sh) & 0xFFFFFull);
    }
    if (f == seen) {
      atomicOr(flags, kFlagSchedule);
    } else {
      idx = f - seen;
      seen = f;
    }
  }
  seen = __builtin_amdgcn_readlane(seen, 0);
  if (m & 1)
    seen1 = seen;
  else
    seen0 = seen;
  return __builtin_amdgcn_readlane(idx, 0);
}

// A tile as the loop and the epilogue see it.  The kernel keeps two (the
// current and the next), in scalar registers, so the fields that outlive
// the decode are packed two to a word where they fit in 16 bits.
struct TgItem {
  // decode-time only (the loads' source is formed from them)
  int h;              // active group
  int rlo, nrow;      // the group's first row and row count (the contraction)
  int k0, n0;         // origin in the group's K x N output
  int rows;           // valid rows from the origin
  int na;             // areas holding lhs columns
  // used by the loop and the epilogue
  int steps;          // contraction steps of this tile (at least MIN_STEPS)
  int shape;          // TgShape
  int ncols;          // valid columns from the origin
  int skip;           // skip_r | skip_c << 16: [0, skip_r) x [0, skip_c) is another tile's (not stored)
  int rc;             // rbase | cbase << 16: this wave's first row / column in the tile
  int sofs[3];        // fragment slot 2i (low half) and 2i+1 (high half): area * AREA | block << 6
  long long obase;    // byte offset of the tile's origin in the output
  int nrec;           // output bytes from the origin to the end of the valid part
};

template <int S>
__device__ __forceinline__ int tg_slot_off(const TgItem& it) {
  return (it.sofs[S >> 1] >> (16 * (S & 1))) & 0xFFFF;
}

// Scheduling units of the dynamic schedule: a group's tiles, or, for a group
// whose tiles are long, one of the four quadrants of its tile grid (k-tiles
// [0, ka) or [ka, nkt), n-tiles [0, na) or [na, nnt)), so that its tiles can
// spread over several queues.  A unit is an int: the active group in bits
// 0..9, the quadrant in bits 10 (upper k half) and 11 (upper n half), bit 12
// set for a quadrant.  The gang schedule's list holds whole groups, largest
// first.
constexpr int kMaxSplit = 128;                          // groups split at most
constexpr int kMaxUnits = kMaxGroups + 3 * kMaxSplit;  // units at most

struct TgGrid {
  int nkt, nnt, ka, na;
};

// The tile's rows, steps, wave layout and fragment slots.
template <class C>
__device__ __forceinline__ void tg_finish(const Params& p, const Plan& pl, TgItem& it, int skip_r, int skip_c,
                                          int w) {
  it.rlo = __builtin_amdgcn_readfirstlane(pl.row_start[it.h]);
  it.nrow = __builtin_amdgcn_readfirstlane(pl.row_start[it.h + 1] - pl.row_start[it.h]);
  const int st = (it.nrow + C::BK - 1) / C::BK;
  it.steps = st < C::MIN_STEPS ? C::MIN_STEPS : st;
  int bs, fnx, rbase, cbase;
  if (it.shape == kTgTall) {  // 4 x 2 waves of 96 x 64
    rbase = (w >> 1) * 96;
    cbase = (w & 1) * 64;
    it.na = 3;
    bs = 3;
    fnx = 2;
  } else if (it.shape == kTgWide) {  // 2 x 4 waves of 64 x 96
    rbase = (w >> 2) * 64;
    cbase = (w & 3) * 96;
    it.na = 1;
    bs = 2;
    fnx = 3;
  } else {
    it.na = 2;
    bs = 4;
    fnx = 2;
    if (it.shape == kTgFull) {  // 2 x 4 waves of 128 x 64
      rbase = (w >> 2) * 128;
      cbase = (w & 3) * 64;
    } else if (it.rows <= C::BM / 2) {  // 2 x 4 waves of 64 x 64 over 128 x 256
      rbase = (w >> 2) * 64;
      cbase = (w & 3) * 64;
    } else {  // 4 x 2 waves of 64 x 64 over 256 x 128
      rbase = (w >> 1) * 64;
      cbase = (w & 1) * 64;
    }
  }
  it.rc = rbase | cbase << 16;
  it.skip = skip_r | skip_c << 16;
  it.obase = ((long long)(it.h * p.K + it.k0) * p.N + it.n0) * C::es_out;
  it.nrec = ((it.rows - 1) * p.N + it.ncols) * C::es_out;
  // Slot s < bs: the lhs-side fragment at tile row rbase + 32 s; slot s >=
  // bs: the rhs-side one at column cbase + 32 (s - bs).  Slots past the
  // shape's fragments repeat the first rhs-side one (read, never used).
#pragma unroll
  for (int i = 0; i < 3; ++i) it.sofs[i] = 0;
#pragma unroll
  for (int s = 0; s < C::NSLOT; ++s) {
    int area, col;
    if (s < bs) {
      col = rbase + 32 * s;
      area = col >> 7;
    } else {
      const int fn = s - bs < fnx ? s - bs : 0;
      col = cbase + 32 * fn;
      area = it.na + (col >> 7);
    }
    it.sofs[s >> 1] |= (area * C::AREA | ((col & 127) >> 5) << 6) << (16 * (s & 1));
  }
}

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

// Dynamic schedule: tile L of a queue -- its unit, then k-tile, then n-tile
// within the unit.
template <class C>
__device__ __forceinline__ TgItem decode_tg(const Params& p, const Plan& pl, const int* units, const int* ustart,
                                            int* cur, int u_end, int L, const TgGrid& gr, int w, int lane) {
  const int K = p.K, N = p.N;
  TgItem it;
  const int u = tg_find_unit(ustart, cur, u_end, L, lane);
  const int d = __builtin_amdgcn_readfirstlane(units[u]);
  const int t = L - __builtin_amdgcn_readfirstlane(ustart[u]);
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
  it.h = d & 1023;
  it.k0 = kt * C::BM;
  it.n0 = nt * C::BN;
  it.rows = K - it.k0 < C::BM ? K - it.k0 : C::BM;
  it.ncols = N - it.n0 < C::BN ? N - it.n0 : C::BN;
  it.shape = (it.rows <= C::BM / 2 || it.ncols <= C::BN / 2) ? kTgHalf : kTgFull;
  tg_finish<C>(p, pl, it, 0, 0, w);
  return it;
}

// Gang schedule: list item L (a group) of workgroup j of a queue is tile j
// (t) of that group.
template <class C>
__device__ __forceinline__ TgItem decode_gang(const Params& p, const Plan& pl, const int* units, int L,
                                              const TgTile& t, int w) {
  TgItem it;
  it.h = __builtin_amdgcn_readfirstlane(units[L]) & 1023;
  it.shape = t.shape;
  it.k0 = t.k0;
  it.n0 = t.n0;
  it.rows = t.rows;
  it.ncols = t.ncols;
  tg_finish<C>(p, pl, it, t.skip_r, t.skip_c, w);
  return it;
}

// This wave's direct-to-LDS source for a tile: wave w fills rows
// 16 (w % 2) .. + 16 of area w / 2, whose columns are the lhs's from k0 +
// 128 a (a < na) or the rhs's from n0 + 128 (a - na), over the group's rows
// (zero-size past the end of the stream).  Instruction i of a step fills 4
// rows (1 KB); lane l takes row 16 (w % 2) + 4 i + l / 16 and 16-byte chunk
// (l % 16) ^ swz_nn(row) of it (the row's low two bits are l / 16's).
// Columns past the tile's valid part are loaded too (the next columns of the
// row, or zeros past the group): they only feed output rows and columns that
// the epilogue drops.
struct TgDma {
  __amdgpu_buffer_rsrc_t r;
  int s2;  // bytes per operand row
  int lo;  // lane part of the offset
};

template <class C>
__device__ __forceinline__ TgDma tg_dma(const Params& p, const TgItem& it, bool live, int w, int lane) {
  const int a = w >> 1;
  const bool lhs = a < it.na;
  const int col = lhs ? it.k0 + 128 * a : it.n0 + 128 * (a - it.na);
  const int width = lhs ? p.K : p.N;
  const char* src = reinterpret_cast<const char*>(lhs ? p.lhs : p.rhs);
  const long long off = ((long long)it.rlo * width + col) * 2;
  const long long bytes = (long long)it.nrow * width * 2 - (long long)col * 2;
  TgDma d;
  d.r = uniform_rsrc(src + off, live && bytes > 0 ? (int)bytes : 0);
  d.s2 = __builtin_amdgcn_readfirstlane(width * 2);
  const int q = lane >> 4;
  d.lo = q * d.s2 + (((lane & 15) ^ swz_nn(q)) << 4);
  return d;
}

// lane + uniform, added where it is used: the compiler would otherwise
// turn the per-step offsets into per-lane induction variables that stay live
// across the loop (registers the kernel does not have to spare)
__device__ __forceinline__ int add_at_use(int lane_part, int uniform) {
  int r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(uniform), "v"(lane_part));
  return r;
}

// Direct-to-LDS instruction J (0..3) of contraction step k into stage `st`.
template <class C, int J>
__device__ __forceinline__ void tg_dma_op(const TgDma& d, int k, char* st, int w) {
  const int row = 16 * (w & 1) + 4 * J + C::BK * k;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.r, (lds_ptr_t)(st + (w >> 1) * C::AREA + (w & 1) * 4096 + J * 1024), 16,
                                           add_at_use(d.lo, row * d.s2), 0, 0, 0);
}

// Lane part of a fragment's LDS address in a 256-byte-row area, for the
// 32-column block at column 0 of the area and K half 0: in transpose read t,
// lane l (q = l / 16, j = l % 16) points at row 8 (q / 2) + 4 t + j / 4 and
// columns 16 (q % 2) + 4 (j % 4) + [0, 4) of the block; the read hands lane
// l column l % 32 at rows 8 (l / 32) + 4 t + [0, 4).  Block b of the area
// flips chunk bits 2-3 (byte bits 6-7), which the row swizzle also flips, so
// it is an XOR of b << 6; the area and the K half add (bits 12 and up).  The
// 32 lanes of an LDS cycle read four rows by four chunks, which the swizzle
// puts in the four quarters of the 64 banks.
__device__ __forceinline__ int tg_lane_off(int lane) {
  const int q = lane >> 4, j = lane & 15;
  const int row = 8 * (q >> 1) + (j >> 2);
  const int chunk = (2 * (q & 1) + ((j >> 1) & 1)) ^ swz_nn(j >> 2);
  return row * 256 + chunk * 16 + (j & 1) * 8;
}

template <int H>
__device__ __forceinline__ i32x4 tg_frag(unsigned addr) {
  const i32x2 lo = ds_read_tr16<H * 16 * 256>(addr);
  const i32x2 hi = ds_read_tr16<H * 16 * 256 + 4 * 256>(addr);
  return i32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Per K half the refills issue twelve LDS transpose reads in slot order (six
// slots, two reads each), so a half's fragments have completed once at most
// the twelve reads of the following half are outstanding.
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

// Deal the units of the dynamic schedule to nq queues, each to the queue
// with the least work so far (the lowest index on ties), in the group order
// (largest first), so each queue's units are in that order too.  A tile's
// work is its contraction steps plus two for the epilogue.  A group's tiles
// are its nkt x nnt grid, and a group is split into quadrants when its tiles
// take more than a quarter of a workgroup's share of all the work (at most
// kMaxSplit groups, the largest).  Wave 0 runs it: the greedy choice is made
// in scalar registers, unit after unit, recording each unit's queue, place
// in the queue and first tile; the lists are then written in parallel.
template <class C>
__device__ inline void tg_deal(const Plan& pl, const int* order, char* smem, int* units, int* ustart, int* sched,
                               int nq, int P, const TgGrid& gr, int lane) {
  using Lds = TgLds<C>;
  int* const rec_unit = reinterpret_cast<int*>(smem + Lds::REC_UNIT);
  int* const rec_pos = reinterpret_cast<int*>(smem + Lds::REC_POS);
  int* const rec_start = reinterpret_cast<int*>(smem + Lds::REC_START);
  const int ga = pl.ga;
  const int per = gr.nnt * gr.nkt;
  // a tile's epilogue overlaps other tiles' steps and costs about two
  const int boundary = 2;
  auto tile_cost = [&](int i) {
    const int h = order[i];
    const int st = (pl.row_start[h + 1] - pl.row_start[h] + C::BK - 1) / C::BK;
    return (st < C::MIN_STEPS ? C::MIN_STEPS : st) + boundary;
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

// Epilogue of one tile, as the big kernel's (big_epilogue): block (fm, fn)
// of the wave is accumulator fm * FN + fn; lane (kh, r32) holds row
// rbase + 32 fm + r32 and, in register 4 g + i, column cbase + 32 fn + 8 g +
// 4 kh + i.  The permlane32 swap of groups (g, g+1) leaves each lane eight
// consecutive columns, and each 32-row block passes through the wave's 4 KB
// staging slice so that a store writes eight whole 128-byte row segments.
// With bf16 output a staging row holds 64 columns: two column blocks, or the
// last block of a three-block wave alone (the other half of the row is not
// stored).  Stores outside the tile's valid rows and columns are dropped by
// the range check, those in its skipped part by an out-of-range offset, and
// a tile with fewer blocks pads to the full tile's store count E.
template <class C, int FM, int FN>
__device__ __forceinline__ void tg_epilogue(const Params& p, const f32x16 (&acc)[C::NACC], const TgItem& it, char* stg,
                                            int kh, int r32, int lane) {
  const int N = p.N;
  const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(reinterpret_cast<char*>(p.out) + it.obase, it.nrec);
  const int rbase = it.rc & 0xFFFF, cbase = it.rc >> 16;
  const int skip_r = it.skip & 0xFFFF, skip_c = it.skip >> 16;
  const int srow = lane >> 3, schunk = lane & 7;  // store phase: row and chunk of this lane
  const int wr_row = r32 * 128;                   // write phase: this lane's staging row
  // rows srow + 8 i of the staged block back out, as whole row segments;
  // col0: the block's first column in the tile, cw: columns per chunk, nch:
  // chunks of the row that hold data
  auto drain = [&](int fm, int col0, int cw, int nch) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = srow + 8 * i;
      const i32x4 d = *reinterpret_cast<const i32x4*>(stg + row * 128 + ((schunk ^ swz_out(row)) << 4));
      const int col = col0 + cw * schunk;
      const int trow = rbase + fm * 32 + row;
      const bool keep = col < it.ncols && schunk < nch && !(trow < skip_r && col < skip_c);
      const int voff = keep ? trow * N * C::es_out + col * C::es_out : (int)0x80000000;
      __builtin_amdgcn_raw_buffer_store_b128(d, ro, voff, 0, 0);
    }
  };
  auto stage_write = [&](int chunk, i32x4 v) __attribute__((always_inline)) {
    *reinterpret_cast<i32x4*>(stg + wr_row + ((chunk ^ swz_out(r32)) << 4)) = v;
  };
  // bf16: columns 32 fn + [0, 32) of row block fm into chunks 4 (fn % 2) + ...
  auto stage_bf16 = [&](int fm, int fn) __attribute__((always_inline)) {
#pragma unroll
    for (int gp = 0; gp < 4; gp += 2) {
      uint32_t x0[2], x1[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const f32x16& a = acc[fm * FN + fn];
        x0[x] = pk_bf16_rne(a[4 * (gp + x) + 0], a[4 * (gp + x) + 1]);
        x1[x] = pk_bf16_rne(a[4 * (gp + x) + 2], a[4 * (gp + x) + 3]);
      }
      const auto r0 = __builtin_amdgcn_permlane32_swap(x0[0], x0[1], false, false);
      const auto r1 = __builtin_amdgcn_permlane32_swap(x1[0], x1[1], false, false);
      stage_write(4 * (fn & 1) + gp + kh, i32x4{(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1]});
    }
  };
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    if constexpr (C::OUT_F32) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
        for (int gp = 0; gp < 4; gp += 2) {
          int lo[4], hi[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[fm * FN + fn][4 * gp + i]),
                                                            __float_as_uint(acc[fm * FN + fn][4 * (gp + 1) + i]),
                                                            false, false);
            lo[i] = (int)r[0];
            hi[i] = (int)r[1];
          }
          // 32 columns of 4 bytes per staging row: chunks 2 (gp + kh) + {0, 1}
          stage_write(2 * (gp + kh), i32x4{lo[0], lo[1], lo[2], lo[3]});
          stage_write(2 * (gp + kh) + 1, i32x4{hi[0], hi[1], hi[2], hi[3]});
        }
        drain(fm, cbase + fn * 32, 4, 8);
      }
    } else {
#pragma unroll
      for (int fn = 0; fn < FN; fn += 2) {
        stage_bf16(fm, fn);
        if (fn + 1 < FN) stage_bf16(fm, fn + 1);
        drain(fm, cbase + fn * 32, 8, fn + 1 < FN ? 8 : 4);
      }
    }
  }
  // pad to the full tile's store count with range-dropped stores, each to
  // an address of its own: the compiler deletes a store that repeats an
  // earlier one, and every dropped one would leave the K loop's constant
  // waits one operation short
  constexpr int kIssued = C::OUT_F32 ? FM * FN * 4 : FM * ((FN + 1) / 2) * 4;
  static_assert(kIssued <= C::E, "store count");
#pragma unroll
  for (int i = kIssued; i < C::E; ++i)
    __builtin_amdgcn_raw_buffer_store_b128(i32x4{0, 0, 0, 0}, ro, (int)0x80000000, 64 * i, 0);
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
  const int W = P / nq, j = blockIdx.x / nq;  // workgroups of the queue, this one's place
  const TgGang gg = tg_gang_plan(K, N);
  const bool gang = nq == kQueues && gg.T <= W && 4 * gg.T >= 3 * W;
  // the gang schedule's tile of this workgroup, the same in every group
  const TgTile tj = tg_gang_tile(gg, K, N, j < gg.T ? j : 0);
  const int gang_tiles = gg.T;
  if (w == 0) {
    if (gang) {
      for (int i = lane; i < pl.ga; i += 64) units[i] = order[i];  // the list, largest group first
    } else {
      tg_deal<C>(pl, order, smem, units, ustart, sched, nq, P, gr, lane);
    }
  }
  __syncthreads();
  // dynamic: this queue's units [ucur, u_end) and tiles [0, n_items); gang:
  // list items [0, n_items) (none for a workgroup past the tile count)
  int ucur = gang ? 0 : __builtin_amdgcn_readfirstlane(sched[kSchedOff + x]);
  const int u_end = gang ? 0 : __builtin_amdgcn_readfirstlane(sched[kSchedOff + x + 1]);
  const int n_items = gang ? (j < gang_tiles ? pl.ga : 0) : __builtin_amdgcn_readfirstlane(sched[kSchedTiles + x]);
  int* const counter = p.queue + x;
  unsigned long long* const meet_word = reinterpret_cast<unsigned long long*>(p.queue + kGangMeet + 2 * x);
  // Output groups the plan dropped (a group offset past G - Ga, which is
  // flagged) are zero.  K * N is a multiple of 64, so 16-byte stores tile it.
  {
    const long long b0 = (long long)pl.ga * K * N * C::es_out, b1 = (long long)p.Ga * K * N * C::es_out;
    char* o = reinterpret_cast<char*>(p.out);
    for (long long off = b0 + ((long long)slot * C::T + tid) * 16; off < b1; off += (long long)P * C::T * 16)
      *reinterpret_cast<i32x4*>(o + off) = i32x4{0, 0, 0, 0};
  }
  // The last workgroup of the queue to get here resets the queue's counters,
  // and the last of the grid the grid's; every index grabbed and every
  // arrival counted has returned by then.
  auto finish = [&]() {
    if (tid == 0) {
      const int prev = atomicAdd(p.queue + kQueues + x, 1);
      if (prev == W - 1) {
        atomicExch(counter, 0);
        atomicExch(meet_word, 0ull);
        atomicExch(p.queue + kQueues + x, 0);
      }
      const int all = atomicAdd(p.queue + kGangDone, 1);
      if (all == P - 1) {
        atomicExch(p.queue + kGangNext, 0);
        atomicExch(p.queue + kGangDone, 0);
      }
    }
  };

  // Item indices.  Gang: list items x and 2 kQueues - 1 - x, then the
  // leader's grabs (tg_gang_meet).  Dynamic: the queue's first two rounds
  // are fixed, workgroup j of the queue's W taking tiles j and 2W-1-j (had
  // each grabbed its first two, the first workgroups would take two of the
  // longest tiles each); afterwards each tile grabs the index of the tile
  // after next during its first steps (so the next tile is known before its
  // loads start), from 2W on.
  int L_cur = gang ? x : j;
  int L_nxt = gang ? 2 * kQueues - 1 - x : 2 * W - 1 - j;
  if (L_cur >= n_items) {
    finish();
    return;
  }
  auto decode = [&](int L) __attribute__((always_inline)) {
    return gang ? decode_gang<C>(p, pl, units, L, tj, w)
                : decode_tg<C>(p, pl, units, ustart, &ucur, u_end, L, gr, w, lane);
  };

  TgItem cur = decode(L_cur);
  bool last_item = L_nxt >= n_items;
  TgItem nxt = cur;
  if (!last_item) nxt = decode(L_nxt);
  TgDma dcur = tg_dma<C>(p, cur, true, w, lane);
  TgDma dnxt = tg_dma<C>(p, nxt, !last_item, w, lane);

  // Prologue: the first tile's steps 0..2; every older memory operation is
  // complete after the wait, so the loop's counts start from an empty queue.
#pragma unroll
  for (int s = 0; s < C::S - 1; ++s) {
    tg_dma_op<C, 0>(dcur, s, smem + s * C::STAGE, w);
    tg_dma_op<C, 1>(dcur, s, smem + s * C::STAGE, w);
    tg_dma_op<C, 2>(dcur, s, smem + s * C::STAGE, w);
    tg_dma_op<C, 3>(dcur, s, smem + s * C::STAGE, w);
  }
  wait_vmcnt<0>();
  __syncthreads();

  const int lo0 = tg_lane_off(lane);
  // fragment slot s of K half h of the step in stage `st`, for the layout of
  // `it`.  The XOR is formed at each use (volatile, so it is not hoisted):
  // hoisted, the lane parts of every slot of both tiles stay live across the
  // loop and push the kernel past its register budget into spills.
  auto frag = [&](const char* st, const TgItem& it, int s, int h) __attribute__((always_inline)) {
    int lane_part;
    int so;
    switch (s) {
      case 0: so = tg_slot_off<0>(it); break;
      case 1: so = tg_slot_off<1>(it); break;
      case 2: so = tg_slot_off<2>(it); break;
      case 3: so = tg_slot_off<3>(it); break;
      case 4: so = tg_slot_off<4>(it); break;
      default: so = tg_slot_off<5>(it); break;
    }
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(lane_part) : "v"(lo0), "s"(so));
    const unsigned addr = (unsigned)(size_t)(lds_ptr_t)st + (unsigned)lane_part;
    return h ? tg_frag<1>(addr) : tg_frag<0>(addr);
  };

  i32x4 f[C::NSLOT][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int s = 0; s < C::NSLOT; ++s) f[s][h] = frag(smem, cur, s, h);

  // The transpose reads write their registers when the data arrives, but the
  // compiler takes an asm output as written when the asm issues: a slot it
  // sees no later use of (a slot the shape does not use, or every refill
  // after the last step) would have its registers handed to other values,
  // which the arriving data then overwrites.  Each slot is therefore used
  // here, after the wait that guarantees its data has arrived.
  auto hold = [&](int h) __attribute__((always_inline)) {
    asm volatile("" ::"v"(f[0][h]), "v"(f[1][h]), "v"(f[2][h]), "v"(f[3][h]), "v"(f[4][h]), "v"(f[5][h]));
  };

  f32x16 acc[C::NACC];
  int stage = 0;
  int arrivals = 0;  // gang: this workgroup's meets so far (every workgroup of the queue meets as often)
  int seen0 = 0, seen1 = 0;  // gang: the meet word's two index fields as last seen
  int L_new = 0;  // the grabbed index handed over during the current tile

  // One contraction step (as the big kernel's K step, without a bias row):
  // the next step's operands are complete once at most WAIT newer
  // operations are outstanding -- the step after's four loads and, in a
  // tile's first two steps, the previous tile's E stores (and in the second,
  // the tile-index grab issued after the first).  The barrier frees the
  // stage the step before last used, which takes step kd (this tile's, or
  // the next tile's when NEXT); slots are refilled with the next step's
  // fragments right after their last use, in slot order.
  auto kstep = [&](auto shape_tag, auto wait_tag, auto next_tag, auto last_tag, int kd)
      __attribute__((always_inline)) {
    using SC = TgShapeCfg<decltype(shape_tag)::value>;
    constexpr int WAIT = decltype(wait_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value, LAST = decltype(last_tag)::value;
    constexpr int NMH = SC::FM * SC::FN;  // MFMAs per K half
    constexpr int NM = 2 * NMH;
    wait_vmcnt<WAIT>();
    if constexpr (LAST) __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    ring_barrier();
    const TgDma& d = NEXT ? dnxt : dcur;
    char* st3 = smem + ((stage + 3) & (C::S - 1)) * C::STAGE;
    const char* st1 = smem + ((stage + 1) & (C::S - 1)) * C::STAGE;
    const TgItem& it1 = LAST ? nxt : cur;
    auto dma_at = [&](int m) __attribute__((always_inline)) {
      if (m == 0 * NM / 4) tg_dma_op<C, 0>(d, kd, st3, w);
      if (m == 1 * NM / 4) tg_dma_op<C, 1>(d, kd, st3, w);
      if (m == 2 * NM / 4) tg_dma_op<C, 2>(d, kd, st3, w);
      if (m == 3 * NM / 4) tg_dma_op<C, 3>(d, kd, st3, w);
    };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      tg_frags_ready();
      hold(h);
      int m = h * NMH;
#pragma unroll
      for (int fm = 0; fm < SC::FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < SC::FN; ++fn) {
          acc[fm * SC::FN + fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, f[SC::BS + fn][h]), __builtin_bit_cast(bf16x8, f[fm][h]),
              acc[fm * SC::FN + fn], 0, 0, 0);
          dma_at(m++);
          __builtin_amdgcn_sched_barrier(0);  // keep this order
        }
        f[fm][h] = frag(st1, it1, fm, h);
      }
#pragma unroll
      for (int s = SC::FM; s < C::NSLOT; ++s) f[s][h] = frag(st1, it1, s, h);
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
  auto ktile = [&](auto shape_tag) __attribute__((always_inline)) {
    using SC = TgShapeCfg<decltype(shape_tag)::value>;
#pragma unroll
    for (int i = 0; i < SC::FM * SC::FN; ++i)
#pragma unroll
      for (int z = 0; z < 16; ++z) acc[i][z] = 0.f;
    const int KT = cur.steps;
    kstep(shape_tag, W0{}, F_{}, F_{}, 3);
    // the grab of the tile after next, by wave 0 unless this tile has no
    // successor (or the schedule is the gang's): exactly one counted
    // operation in every wave
    const int g = tg_grab_wave(counter, lane, w == 0 && !last_item && !gang);
    kstep(shape_tag, W0G{}, F_{}, F_{}, 4);
    for (int kt = 2; kt + 3 < KT; ++kt) kstep(shape_tag, W1{}, F_{}, F_{}, kt + 3);
    // gang: meet the queue's other workgroups before the next group's
    // loads, and learn the group after it
    int after = kGangNone;
    if (gang && !last_item && w == 0)
      after = tg_gang_meet(meet_word, p.queue + kGangNext, p.flags, arrivals++, gang_tiles, j == 0, seen0, seen1,
                           lane);
    kstep(shape_tag, W1{}, T_{}, F_{}, 0);  // kt = KT-3: the next tile's step 0
    // the grab has returned (this step's wait left only the loads of the
    // step before outstanding); hand it to every wave, which reads it after
    // the last step's barrier
    if (w == 0 && lane == 0 && !last_item) sched[kSchedSlot] = gang ? after : g;
    kstep(shape_tag, W1{}, T_{}, F_{}, 1);
    kstep(shape_tag, W1{}, T_{}, T_{}, 2);
    // every refill has landed before the epilogue takes registers of its own
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    hold(0);
    hold(1);
    L_new = gang ? __builtin_amdgcn_readfirstlane(sched[kSchedSlot])
                 : 2 * W + __builtin_amdgcn_readfirstlane(sched[kSchedSlot]);
    // the last step's stage holds the epilogue's staging slices, 4 KB per wave
    tg_epilogue<C, SC::FM, SC::FN>(p, acc, cur, smem + ((stage + 3) & (C::S - 1)) * C::STAGE + w * 4096, kh, r32,
                                   lane);
  };

  while (true) {
    if (cur.shape == kTgFull)
      ktile(std::integral_constant<int, kTgFull>{});
    else if (cur.shape == kTgHalf)
      ktile(std::integral_constant<int, kTgHalf>{});
    else if (cur.shape == kTgTall)
      ktile(std::integral_constant<int, kTgTall>{});
    else
      ktile(std::integral_constant<int, kTgWide>{});
    if (last_item) break;
    L_nxt = L_new;
    last_item = L_nxt >= n_items;
    cur = nxt;
    dcur = dnxt;
    if (!last_item) nxt = decode(L_nxt);
    dnxt = tg_dma<C>(p, nxt, !last_item, w, lane);
  }
  finish();
}

}  // namespace gmmk
