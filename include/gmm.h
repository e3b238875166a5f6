/*
 * gmm.h -- C ABI of the MI355X (gfx950) grouped matrix multiplication library
 * (libgmm.so).
 *
 * The operation is the Megablox grouped matmul (tpu-inference 0.13.2 wheel
 * diff page, megablox/gmm.py, gmm()): a row-sorted lhs [M,K] is cut into
 * contiguous row groups by an int32 group_sizes[G]; the rows of group g are
 * [o[g], o[g+1]) with o[0] = 0 and o[g+1] = o[g] + group_sizes[g]
 * (make_group_metadata, group offsets).  Groups s .. s+Ga-1 are active, where
 * s is the group offset and Ga = rhs.shape[0]; each active row r of group g is
 *
 *   out[r,n] = sum_b rhs_scale[g-s,b,0,n] * lhs_scale[r,b] *
 *                    sum_{k in block b} lhs[r,k] * W(g-s,n,k)
 *              + rhs_bias[g-s,0,n]
 *
 * accumulated in fp32 and rounded once, to nearest even, to the output type
 * (gmm() kernel body: the accumulator is reset per quantisation block and
 * scaled by that block's rhs_scale; the bias is added once).  An absent scale
 * is 1, an absent bias 0, and with neither scale the whole of K is one block.
 * W(h,n,k) = rhs[h,n,k] when transpose_rhs == 0 (rhs [Ga,N,K], an NT product)
 * and rhs[h,k,n] when transpose_rhs == 1 (rhs [Ga,K,N], an NN product that
 * reads the forward weight in place -- MaxText PR "Megablox: transposed-RHS
 * gmm_v2 kernel for the backward dlhs", Context).  lhs_scale is the
 * per-token activation scale of the block-scaled W8A8 GEMM (metrale
 * gemm_quant.rs page, fp8_gemm_t_blockscaled).  Every output row outside
 * [o[s], o[s+Ga]) is written as +0.0 (gmm(), _zero_uninitialized_memory).
 *
 * Conventions
 *  - Every tensor is a dense, row-major view of device memory that the caller
 *    owns and keeps alive until the work queued on `stream` has finished.
 *    Pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  gmm_run only
 *    queues work: it never synchronises and never copies group_sizes or the
 *    group offset to the host.
 *  - A handle is used by one host thread at a time.
 *  - No exception crosses this boundary.  Every call returns a gmm_status;
 *    gmm_last_error() gives the text of the last failure on a handle.
 */
#ifndef GMM_MI355X_GMM_H
#define GMM_MI355X_GMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GMM_F32 = 0,       /* IEEE binary32 */
  GMM_BF16 = 1,      /* bfloat16 */
  GMM_F8E4M3FN = 2,  /* OCP e4m3fn: bias 7, max 448, no infinities */
  GMM_I32 = 3,       /* int32 (group_sizes only) */
  GMM_F8E5M2 = 4,    /* OCP e5m2: bias 15, max 57344, with infinities and NaN */
  GMM_E8M0 = 5,      /* 8-bit power-of-two scale byte (block scales only) */
  GMM_I8 = 6,        /* two's-complement int8 */
  GMM_I4 = 7,        /* two's-complement int4, two to a byte (element i in the low
                        nibble of byte i/2 when i is even, the high nibble when odd) */
  GMM_U4 = 8,        /* unsigned int4, packed as GMM_I4 */
  GMM_F4E2M1 = 9     /* OCP fp4 e2m1 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6), packed as GMM_I4 */
} gmm_dtype;

typedef enum {
  GMM_OK = 0,
  GMM_E_INVALID = -1,     /* inconsistent shapes, ranks, dtypes or pointers */
  GMM_E_UNSUPPORTED = -2, /* a valid problem this library does not run */
  GMM_E_HIP = -3,         /* a HIP runtime call or kernel launch failed */
  GMM_E_DEVICE_DATA = -4  /* device-resident data was invalid (gmm_device_flags) */
} gmm_status;

/* A dense row-major device tensor view (caller-owned). */
typedef struct {
  const void* data;
  int32_t dtype;     /* gmm_dtype */
  int32_t ndim;      /* 1..4 */
  int64_t shape[4];
} gmm_tensor;

typedef struct gmm_handle gmm_handle;

/* Bits reported by gmm_device_flags.  The kernels clamp the offending value
 * so every access stays in bounds, compute with the clamped value and set the
 * bit. */
#define GMM_FLAG_NEGATIVE_SIZE 0x1u  /* some group_sizes[g] < 0 (taken as 0) */
#define GMM_FLAG_SIZES_EXCEED_M 0x2u /* o[G] > M (offsets clamped to M) */
#define GMM_FLAG_BAD_OFFSET 0x4u     /* group offset < 0 or s + Ga > G (clamped) */
/* Not a data error: a gmm_tgmm_run workgroup waited past its bound (about a
 * second) for its XCD's next group, which only happens when the call's
 * workgroups cannot all run at once (the GPU shared with other work); the
 * groups it did not learn of were not computed.  Run the call again. */
#define GMM_FLAG_SCHEDULE_TIMEOUT 0x8u

/*
 * gmm_create: make a handle on HIP device `device` (must be gfx950).
 * Allocates a 16-byte device block for the data-error flags.  The first
 * gmm_tgmm_run on each stream allocates that stream's 144-byte block of
 * work-queue counters (kept until gmm_destroy); no other call allocates.
 * Returns GMM_E_UNSUPPORTED on another architecture, GMM_E_HIP on a HIP
 * failure, GMM_E_INVALID when h is NULL.
 */
gmm_status gmm_create(gmm_handle** h, int device);

/* gmm_destroy: free the handle, its flag word and its counter blocks.  Work
 * queued with the handle must have finished.  NULL is allowed. */
gmm_status gmm_destroy(gmm_handle* h);

/* gmm_last_error: text of the last failure on h ("" when none; never NULL). */
const char* gmm_last_error(const gmm_handle* h);

/*
 * gmm_run: queue out = gmm(lhs, rhs, group_sizes, ...) on `stream`.
 *
 *   lhs          [M,K]; F32, BF16, F8E4M3FN, F8E5M2, I8, or the four-bit I4,
 *                U4 and F4E2M1 (two to a byte; the shape counts elements, the
 *                data holds M*K/2 bytes).
 *   rhs          [Ga,N,K] (transpose_rhs == 0) or [Ga,K,N] (== 1).
 *                Supported (lhs, rhs) pairs: (F32,F32), (BF16,BF16),
 *                (BF16, F8E4M3FN or F8E5M2: the weight is widened exactly
 *                to bf16), (F8E4M3FN or F8E5M2, F8E4M3FN or F8E5M2: fp8 x
 *                fp8 products, either format on either side; e5m2 is one of
 *                the dtypes of the Megablox gmm's whitelist on the
 *                tpu-inference wheel diff page), (BF16, I8: the weight is
 *                widened exactly to bf16), (I8, I8: exact int32 products
 *                and sums, converted to f32 per scale block, or once when
 *                there is no scale; K, or K/nb with scales, at most 2^17).
 *                (BF16, I4 / U4 / F4E2M1: four-bit weights, two to a byte,
 *                widened exactly to bf16; the tensor's shape counts
 *                elements, [Ga,N,K], and its data holds Ga*N*K/2 bytes).
 *                Four-bit activations (the Megablox gmm's dtype list holds
 *                for lhs as for rhs): (I8 / I4 / U4, I8 / I4 / U4: int8
 *                products, four-bit values widened exactly to int8, exact
 *                int32 sums as for (I8, I8)), and (F8E4M3FN / F8E5M2 /
 *                F4E2M1, F8E4M3FN / F8E5M2 / F4E2M1: products on the
 *                f8f6f4 matrix instruction with each side in its own
 *                format, fp4 e2m1 read packed).  K % 128 == 0 for these.
 *                fp8, int8 and four-bit weights need transpose_rhs == 0.
 *                Infinite or NaN e5m2 codes are outside the contract.
 *   group_sizes  [G] I32 on the device, 1 <= G <= 1024.
 *   rhs_scale    NULL or F32 [Ga,nb,1,N]; K % nb == 0.
 *   rhs_bias     NULL or [Ga,1,N], F32 or BF16.
 *   lhs_scale    NULL or F32 [M,nb] (its nb must equal rhs_scale's when both
 *                are given).
 *                Either scale may instead be E8M0 bytes (then every given
 *                scale is): microscaling block scales of 32 K elements
 *                (nb = K/32), byte e meaning 2^(e-127) as in the metrale
 *                gemm_quant.rs page's E8M0 widening, applied by the gfx950
 *                scaled f8f6f4 matrix instruction itself, for any pair of
 *                F8E4M3FN / F8E5M2 / F4E2M1 operands.  Byte 255 (NaN in the
 *                microscaling encoding) is outside the contract.
 *   group_offset NULL (s = 0) or a device pointer to one int32 s.
 *   out          [M,N], F32 or BF16.  All M rows are written.  out must not
 *                overlap any input.
 *
 * Size limits: M < 2^31; N % 8 == 0; K % 64 == 0 for BF16 products,
 * K % 128 == 0 for fp8 x fp8, K % 32 == 0 for F32, and the block length K/nb
 * must be a multiple of the same number; Ga <= G; one group's weight, a
 * 256-row lhs tile and a 256-row output tile each below 2 GiB.  Outside them the call
 * returns GMM_E_UNSUPPORTED and queues nothing.  Shape or dtype
 * inconsistencies return GMM_E_INVALID and queue nothing.  A launch failure
 * returns GMM_E_HIP.  Invalid device-resident values (negative sizes, a total
 * beyond M, an offset outside [0, G-Ga]) are clamped and reported through
 * gmm_device_flags.
 */
gmm_status gmm_run(gmm_handle* h,
                   const gmm_tensor* lhs,
                   const gmm_tensor* rhs,
                   const gmm_tensor* group_sizes,
                   const gmm_tensor* rhs_scale,
                   const gmm_tensor* rhs_bias,
                   const gmm_tensor* lhs_scale,
                   const int32_t* group_offset,
                   int transpose_rhs,
                   const gmm_tensor* out,
                   void* stream);

/*
 * gmm_run_existing_out: gmm_run, except that the rows outside the active
 * groups (rows before the first active group's, and from the end of the last
 * active group's on) are those of existing_out instead of zeros.  This is
 * the existing_out argument of gmm() on the tpu-inference wheel diff pages
 * (megablox/gmm.py): the kernel starts each output tile from existing_out
 * and stores only its group's rows over it, and no zero fill follows.  With
 * expert shards it merges one shard's rows into an output the other shards
 * have written.
 *
 *   existing_out [M,N], the dtype of out (as the pages require of the
 *                preferred element type).  Either out itself (the active
 *                rows are written in place, the others are not touched) or
 *                a buffer that does not overlap out (the other rows are
 *                copied from it).  Read-only; it may overlap an input.
 *   Every other argument, limit and error is as for gmm_run; existing_out
 *   NULL returns GMM_E_INVALID (gmm_run is that call), as does an
 *   existing_out of another shape or dtype, or one that partly overlaps out.
 */
gmm_status gmm_run_existing_out(gmm_handle* h,
                                const gmm_tensor* lhs,
                                const gmm_tensor* rhs,
                                const gmm_tensor* group_sizes,
                                const gmm_tensor* rhs_scale,
                                const gmm_tensor* rhs_bias,
                                const gmm_tensor* lhs_scale,
                                const int32_t* group_offset,
                                int transpose_rhs,
                                const gmm_tensor* existing_out,
                                const gmm_tensor* out,
                                void* stream);

/*
 * gmm_quant_fp8_run: queue the per-token activation quantiser on `stream`:
 * per_token_group_quant_fp8 of the metrale gemm_quant.rs page, bf16 x [M,K]
 * to e4m3fn q [M,K] and an f32 scale per 128-element block of each row,
 * scale [M,K/128] -- the lhs and lhs_scale that gmm_run takes for fp8 x fp8
 * products (the page's fp8_gemm_t_blockscaled activation scale, x ~ q *
 * scale).  The page gives the shapes only; the arithmetic is
 *   scale[r,b] = amax / 448 over x[r, 128b .. 128b+127] in binary32
 *                (1 when the block is all zero),
 *   q[r,k]     = the e4m3fn value nearest to clamp(x[r,k] / scale[r,b],
 *                -448, 448), the quotient one correctly rounded binary32
 *                division, ties to the even mantissa, the sign kept (a
 *                negative value that rounds to zero is 0x80).
 *
 *   x      [M,K] BF16, K % 128 == 0 (GMM_E_INVALID otherwise).
 *   q      [M,K] F8E4M3FN, written.
 *   scale  [M,K/128] F32, written.
 *   All three on the device, 16-byte aligned, caller-owned, not overlapping
 *   (GMM_E_INVALID otherwise).  Values outside the finite bf16 range (NaN,
 *   infinity) are outside the contract.  A launch failure returns GMM_E_HIP.
 */
gmm_status gmm_quant_fp8_run(gmm_handle* h,
                             const gmm_tensor* x,
                             const gmm_tensor* q,
                             const gmm_tensor* scale,
                             void* stream);

/*
 * gmm_widen_scales_run: queue the widening of a block-scale tensor to f32
 * on `stream`: widen_block_scale_f32 of the metrale gemm_quant.rs page, so
 * that bf16 or E8M0 block scales can be passed to gmm_run (which reads f32
 * rhs_scale and lhs_scale).
 *   src  any shape, BF16 (widened exactly), F32 (copied) or E8M0 (a byte e
 *        becomes the binary32 with bit pattern e << 23, i.e. 2^(e - 127);
 *        as the page states, e = 0 becomes 2^-127 and e = 255 becomes 0.0 --
 *        not the NaN of the OCP encoding).
 *   dst  F32 with src's number of elements (any shape), written.
 *   Both on the device, 16-byte aligned, caller-owned and not overlapping;
 *   otherwise GMM_E_INVALID.  A launch failure returns GMM_E_HIP.
 */
gmm_status gmm_widen_scales_run(gmm_handle* h, const gmm_tensor* src, const gmm_tensor* dst, void* stream);

/*
 * gmm_tgmm_run: queue the transposed grouped matmul, the weight gradient of
 * gmm, on `stream`.  For each active group h = g - s (g = s .. s+Ga-1),
 *
 *   out[h,k,n] = sum over rows r in [o[g], o[g+1]) of lhs[r,k] * rhs[r,n],
 *
 * accumulated in fp32 and rounded once, to nearest even, to the output type;
 * an empty group's out[h] is all +0.0.  For the forward gmm with an NN
 * weight W [Ga,K,N] and output gradient dout, tgmm(lhs, dout) is dW; for an
 * NT weight [Ga,N,K], tgmm(dout, lhs) is dW.  The Megablox metadata builder
 * keeps a tile for every empty group because this product must still write
 * its output (tpu-inference 0.13.2 wheel diff page, megablox/gmm.py,
 * make_group_metadata, visit_empty_groups); the MaxText PR "Megablox:
 * transposed-RHS gmm_v2 kernel for the backward dlhs" keeps it as the
 * weight-gradient step (drhs) of the custom VJP.
 *
 *   lhs          [M,K] BF16.
 *   rhs          [M,N] BF16 (the same rows as lhs).
 *   group_sizes  [G] I32 on the device, 1 <= G <= 1024.
 *   group_offset NULL (s = 0) or a device pointer to one int32 s.
 *   out          [Ga,K,N], F32 or BF16, Ga <= G.  Every element is written.
 *                out must not overlap an input.
 *
 * Size limits: K % 8 == 0, N % 8 == 0, M*K*2 and M*N*2 below 2 GiB, Ga*K
 * below 2^31, 384*N*(output element size) below 2 GiB.  Outside them the
 * call returns GMM_E_UNSUPPORTED and queues nothing; shape or dtype
 * inconsistencies return GMM_E_INVALID; a launch failure returns GMM_E_HIP
 * (as does a failed allocation of a new stream's counters).  Invalid
 * device-resident sizes or offset are clamped and reported through
 * gmm_device_flags, as for gmm_run.
 *
 * Scheduling state: the kernel hands out its tiles from work-queue counters
 * that the call's last workgroup resets.  The handle keeps one counter block
 * per stream (allocated on the first call on that stream), so calls on one
 * stream run one after another on their own counters and calls on different
 * streams may overlap.  When each group's tiles fit one XCD's workgroups
 * (the gang schedule), an XCD's workgroups take the groups together, one
 * after another, and the next group comes from a grid-wide counter at each
 * group boundary: that needs every workgroup of the call resident at once,
 * and a call that waits too long for it sets GMM_FLAG_SCHEDULE_TIMEOUT.
 */
gmm_status gmm_tgmm_run(gmm_handle* h,
                        const gmm_tensor* lhs,
                        const gmm_tensor* rhs,
                        const gmm_tensor* group_sizes,
                        const int32_t* group_offset,
                        const gmm_tensor* out,
                        void* stream);

/*
 * gmm_tgmm_run_noalloc: gmm_tgmm_run for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The same kernel and result (bit for bit); the
 * work-queue counters live in the library's static device scratch instead
 * of a per-stream block of the handle, so the call never allocates, also on
 * a stream the handle has not seen.  The handle must exist (gmm_create,
 * which looks the scratch up once per device, is the only allocating call).
 *
 *   Arguments, limits and errors are those of gmm_tgmm_run.  The scratch is
 *   256 bytes per device, held until the process ends; the counters use 144
 *   of them for every problem size, so no size is rejected for want of
 *   scratch.  Each call first clears the counters on `stream` (a one-
 *   workgroup kernel) and then queues the tgmm kernel.
 *
 *   All calls on one device share that device's scratch: two calls that
 *   overlap in time on one GPU (different streams, or several host threads)
 *   race on the counters and give wrong results.  Serialise them.
 */
gmm_status gmm_tgmm_run_noalloc(gmm_handle* h,
                                const gmm_tensor* lhs,
                                const gmm_tensor* rhs,
                                const gmm_tensor* group_sizes,
                                const int32_t* group_offset,
                                const gmm_tensor* out,
                                void* stream);

/*
 * gmm_device_flags: synchronise `stream`, return the GMM_FLAG_* bits that
 * runs on this handle have set since the last call, and clear them.
 * Returns GMM_E_DEVICE_DATA when any bit was set, GMM_OK otherwise.
 */
gmm_status gmm_device_flags(gmm_handle* h, void* stream, uint32_t* flags);

/*
 * gmm_set_tile_policy: choose the output tile family of later gmm_run calls
 * on h.  0 (the default) picks from the problem shape; 1 forces the small
 * decode tiles (32 x 64); 2 forces the big tiles (256 x 128).  The result
 * differs only in the order of fp32 additions.  Returns GMM_E_INVALID for
 * another value.  For tests and tuning.
 */
gmm_status gmm_set_tile_policy(gmm_handle* h, int policy);

/*
 * gmm_set_grid_limit: launch at most `limit` workgroups for the gmm and tgmm
 * kernels of later calls on h (0, the default, lets each kernel take its own
 * count, normally one per compute unit).  Every kernel walks its output
 * tiles with a grid stride, so the result does not change; with few
 * workgroups each one runs many tiles back to back, carrying its operand
 * pipeline from one tile into the next.  Returns GMM_E_INVALID for a
 * negative limit.  For tests.
 */
gmm_status gmm_set_grid_limit(gmm_handle* h, int limit);

/*
 * gmm_debug_worklist: run the device code that turns group_sizes and the
 * group offset into group-aligned m-tiles -- the same device functions every
 * gmm_run kernel starts with -- and write the tiles it finds.
 *
 *   group_sizes  [G] I32 on the device.
 *   group_offset NULL or a device int32 (as in gmm_run).
 *   num_active   Ga.
 *   M            number of lhs rows (offsets are clamped to it).
 *   tm           m-tile height, 1..4096.
 *   tiles        device int32 [capacity, 3]: (group, first_row, rows) per tile,
 *                in group order.
 *   count        device int32 [4]: tile count, first active row, end of the
 *                active rows, and the flag bits of this call.
 * Queues one kernel on `stream`.  Tiles beyond `capacity` are counted but not
 * written.
 */
gmm_status gmm_debug_worklist(gmm_handle* h,
                              const gmm_tensor* group_sizes,
                              const int32_t* group_offset,
                              int64_t num_active,
                              int64_t M,
                              int32_t tm,
                              int32_t* tiles,
                              int64_t capacity,
                              int32_t* count,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GMM_MI355X_GMM_H */
