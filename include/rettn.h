/*
 * rettn.h -- C ABI of the Re-ttention static block-sparse attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (Re-ttention: Ultra Sparse Visual Generation via Attention
 * Statistical Reshape; summary page, section "Approach"; review thread,
 * authors' replies to W1 of the first three reviews):
 *   - a full-attention calibration step records, per (batch, head, query
 *     token), rho = sparse-window softmax denominator / full denominator,
 *     and the residual R = attention output of the masked (out-of-window)
 *     keys normalised by the full denominator;
 *   - each later sparse step attends only to the kept key blocks, rescales
 *     the window-normalised output by the cached rho (ramped up by lambda)
 *     and adds the cached R.
 *
 * Conventions shared by every entry point
 *   - Q, K, V, O, R are [B, H, L, d] tensors in device memory with d
 *     contiguous; element strides stride_b, stride_h, stride_l are given in
 *     the descriptor and apply to all five.  rho is a contiguous float32
 *     [B, H, L] device array.  The element type is the descriptor's dtype
 *     (float32 or bfloat16); rho is always float32.
 *   - The caller owns every buffer.  The library allocates no device
 *     memory and keeps no state between calls besides its code objects
 *     (one of which holds the static scratch array of
 *     rettn_dynamic_index_noalloc, with its device address cached per GPU).
 *   - Launches are asynchronous on the given HIP stream (NULL = the null
 *     stream); results are valid once the stream is ordered after them.
 *   - Errors are returned as status codes; nothing throws or aborts.  All
 *     arguments are validated before anything is launched; a rejected call
 *     launches nothing and writes nothing.
 *   - Outputs must not alias inputs.
 */
#ifndef RETTN_H
#define RETTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RETTN_OK = 0,
    RETTN_EINVAL = 1,        /* a bad argument: null pointer, size, stride, alignment, mismatch */
    RETTN_EUNSUPPORTED = 2,  /* a valid request outside what the kernels implement */
    RETTN_EHIP = 3,          /* a HIP runtime call or kernel launch failed */
    RETTN_ESCRATCH = 4       /* the request needs more than the library's static scratch
                                (rettn_dynamic_index_noalloc only) */
} rettn_status;

typedef enum { RETTN_F32 = 0, RETTN_BF16 = 1 } rettn_dtype;

/* Shape and layout of Q, K, V, O and R (all five share it).
 *   B, H >= 1; L >= 1; 1 <= d <= 128; block in {32, 64, 128}.
 *   bfloat16: d % 8 == 0 and every stride a multiple of 8 elements (16 bytes).
 *   float32:  d % 4 == 0 and every stride a multiple of 4 elements (16 bytes).
 *   Every row must fit: stride_l >= d. */
typedef struct {
    int32_t B, H, L, d, block;
    int32_t dtype;                      /* rettn_dtype */
    int64_t stride_b, stride_h, stride_l;
} rettn_desc;

/* Static block-mask generators (the mask is the same at every denoising
 * step: summary page, "Limitations"; review thread, reply to W2 of the
 * first review).  The pages print no geometry; these are the readings used:
 *   RETTN_MASK_DIAG        query block qb keeps key block qb.
 *   RETTN_MASK_BAND        keeps w consecutive key blocks starting at
 *                          clamp(qb - (w-1)/2, 0, nb - w)  (1 <= w <= nb).
 *   RETTN_MASK_COGVIDEO3D  keeps text blocks [0, text_blocks) and the blocks
 *                          {qb-1, qb, qb+1, qb-tshift, qb+tshift} inside [0, nb).
 *   RETTN_MASK_FULL        keeps every block (0% sparsity). */
typedef enum {
    RETTN_MASK_DIAG = 0,
    RETTN_MASK_BAND = 1,
    RETTN_MASK_COGVIDEO3D = 2,
    RETTN_MASK_FULL = 3
} rettn_mask_kind;

typedef struct {
    int32_t kind;          /* rettn_mask_kind */
    int32_t nb;            /* blocks per side, >= 1 */
    int32_t w;             /* BAND width */
    int32_t text_blocks;   /* COGVIDEO3D: leading text blocks, >= 0 */
    int32_t tshift;        /* COGVIDEO3D: temporal offset in blocks, >= 1 */
} rettn_mask_spec;

/* The compacted block mask, all arrays in device memory and owned by the caller.
 *   mask     uint8 [nqb * nkb] row-major; nonzero = key block kept.
 *   row_ptr  int32 [nqb + 1]; col_idx int32 [nnz], ascending within a row.
 *
 * One index may also hold a mask per head or per (batch, head) slice (heads
 * keep their own statistics: review thread, answer to Q2 of the first review):
 *   slices      0 or 1: one mask shared by every slice (the layout above);
 *               H: one per head, shared by the batch elements;
 *               B*H: one per (batch b, head h), slice b*H + h.
 *   col_stride  slices > 1: elements from one slice's col_idx to the next's.
 * Slice s then has its mask at mask + s*nqb*nkb, its row_ptr at
 * row_ptr + s*(nqb+1) and its col_idx at col_idx + s*col_stride; nnz is the
 * largest slice's count (nnz <= col_stride).  A zero-initialised tail (slices =
 * col_stride = 0) is the shared layout. */
typedef struct {
    int32_t nqb, nkb, nnz;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const uint8_t* mask;
    int32_t slices;
    int32_t col_stride;
} rettn_index;

/* Build a static block mask on the host.
 * mask_host: caller-owned host buffer of spec->nb * spec->nb bytes, filled
 * with 0/1.  Returns RETTN_EINVAL for a null pointer, nb < 1 or nb > 65536,
 * an unknown kind, or generator parameters out of range. */
rettn_status rettn_mask_build(const rettn_mask_spec* spec, uint8_t* mask_host);

/* Compact a device block mask into its CSR block index (kept key blocks of
 * each query block, ascending).
 *   mask_dev    uint8 [nqb * nkb], device.
 *   row_ptr_dev int32 [nqb + 1], device, written.
 *   col_idx_dev int32 capacity nqb * nkb, device; the first nnz entries are written.
 *   nnz_host    host int32, written with the number of kept pairs.
 * The one call in the library that synchronises: it waits on `stream` to
 * read nnz back.  The result is unique, so it is bit-exact by construction. */
rettn_status rettn_index_build(const uint8_t* mask_dev, int32_t nqb, int32_t nkb,
                               int32_t* row_ptr_dev, int32_t* col_idx_dev,
                               int32_t* nnz_host, hipStream_t stream);

/* rettn_index_build for `slices` masks at once (one per head or per slice).
 *   mask_dev    uint8 [slices * nqb * nkb], device.
 *   row_ptr_dev int32 [slices * (nqb + 1)], device, written.
 *   col_idx_dev int32 [slices * nqb * nkb], device: slice s's ids start at
 *               s * nqb * nkb (the index's col_stride is nqb * nkb).
 *   nnz_host    host int32, written with the largest slice's count.
 * Synchronises on `stream` once.  RETTN_EINVAL for a null pointer, slices < 1
 * or sizes beyond 2^31 - 1 elements. */
rettn_status rettn_index_build_sliced(const uint8_t* mask_dev, int32_t slices, int32_t nqb, int32_t nkb,
                                      int32_t* row_ptr_dev, int32_t* col_idx_dev, int32_t* nnz_host,
                                      hipStream_t stream);

/* Dynamic block masks: a mask computed afresh from each step's Q and K, one
 * per (batch, head) slice.  The pages report applying Re-ttention to such
 * masks (review thread, answers to W2 and Q1 of the first review: rho stays
 * predictable, the cached residual no longer matches) but print no rule; the
 * rule implemented is:
 *   - every block of query and of key tokens is summarised by its mean (the
 *     last block by the mean of its tokens < L), in float32;
 *   - query block a scores key block b by the dot product of the two means;
 *   - query block a keeps block a itself and the keep - 1 other key blocks with
 *     the highest scores (all blocks when keep >= nkb); equal scores go to the
 *     lower block and a score that is not a number ranks below all others.
 * Every row therefore keeps exactly kk = min(keep, nkb) blocks.
 *
 * rettn_dynamic_workspace_bytes: device workspace the call needs for `desc`
 * (the block means: 2 * B * H * nb * d float32).
 *
 * rettn_dynamic_index: writes, for every slice s = b*H + h,
 *   mask_out    uint8 [B*H * nb * nb], the slice's mask;
 *   row_ptr_out int32 [B*H * (nb + 1)], row a of slice s at s*(nb+1) + a holds a*kk;
 *   col_idx_out int32 [B*H * nb * kk], the kept blocks of each row, ascending;
 * so the matching rettn_index is {nb, nb, nb*kk, row_ptr_out, col_idx_out,
 * mask_out, slices = B*H, col_stride = nb*kk}.  Q and K follow `desc` (only
 * B, H, L, d, block, dtype and the strides are used).  Asynchronous: nothing
 * waits on the host.  RETTN_EINVAL for bad descriptors or pointers, keep < 1,
 * or a workspace that is null, misaligned (16 bytes) or smaller than the size
 * above; RETTN_EUNSUPPORTED for more than 2048 blocks per side. */
rettn_status rettn_dynamic_workspace_bytes(const rettn_desc* desc, size_t* bytes);
rettn_status rettn_dynamic_index(const rettn_desc* desc, const void* Q, const void* K, int32_t keep,
                                 void* workspace, size_t workspace_bytes, uint8_t* mask_out,
                                 int32_t* row_ptr_out, int32_t* col_idx_out, hipStream_t stream);

/* rettn_dynamic_index without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc).  The block means live in a static device
 * array of RETTN_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends; its device address is looked up once per device on
 * the first call made with that device current.  The call itself allocates
 * nothing.  Outputs, validation and results are those of rettn_dynamic_index
 * (bit for bit).  A request whose block means exceed the array
 * (rettn_dynamic_workspace_bytes > RETTN_NOALLOC_SCRATCH_BYTES) returns
 * RETTN_ESCRATCH and launches nothing; a failed symbol lookup returns
 * RETTN_EHIP.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams, or from different threads without
 * ordering) race and must be serialised by the caller.  Nothing in the array
 * needs to start at zero (every mean is written before it is read). */
#define RETTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
rettn_status rettn_dynamic_index_noalloc(const rettn_desc* desc, const void* Q, const void* K, int32_t keep,
                                         uint8_t* mask_out, int32_t* row_ptr_out, int32_t* col_idx_out,
                                         hipStream_t stream);

/* Full-attention calibration step.  For each (b, h) and query row i < L,
 * over every key j < L, with s_j = <q_i, k_j> / sqrt(d) and W(i) the kept keys:
 *   O_i   = softmax(s) V                                  (full attention)
 *   rho_i = sum_{j in W(i)} e^{s_j} / sum_j e^{s_j}
 *   R_i   = sum_{j not in W(i)} e^{s_j} v_j / sum_j e^{s_j}
 * (review thread, replies to W1 of the first and second reviews: rho is the
 * denominator ratio, R holds only the masked tokens' attention; answer to Q2
 * of the first review: both per head and per token).
 * Writes O and R (dtype, descriptor layout) and rho (float32 [B,H,L]).
 * idx must describe a mask of ceil(L/block) x ceil(L/block) blocks (only
 * idx->mask is read; one per head or slice if idx->slices says so).  For bfloat16, the P*V products run with P and V in
 * float16: V converts exactly for 2^-14 <= |V| <= 65504 (and zero), values
 * below 2^-14 round to float16's subnormal grid (steps of 2^-24), and values
 * beyond 65504 overflow to infinity in O and R. */
rettn_status rettn_calibrate(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                             const rettn_index* idx, void* O, float* rho, void* R,
                             hipStream_t stream);

/* Which residual a calibration writes into R. */
typedef enum {
    /* Re-ttention's residual: the masked keys' share of full attention,
     * R_i = sum_{j not in W(i)} e^{s_j} v_j / sum_j e^{s_j}. */
    RETTN_RESIDUAL_MASKED = 0,
    /* The DiTFastAttn comparator's residual: full attention minus window
     * attention, R_i = O_i - softmax_{W(i)}(s) V_{W(i)} (O_i when W(i) is
     * empty); its later steps add it to plain window attention (review
     * thread, reply to W1 of the first review, on how the two residuals
     * differ). */
    RETTN_RESIDUAL_DIFFERENCE = 1
} rettn_residual;

/* rettn_calibrate with a choice of residual: identical O and rho; R as
 * `kind` says, computed from the float32 accumulators and rounded once to
 * the I/O type.  rettn_calibrate is this call with RETTN_RESIDUAL_MASKED.
 * An unknown `kind` gives RETTN_EINVAL with nothing launched. */
rettn_status rettn_calibrate_residual(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                                      const rettn_index* idx, void* O, float* rho, void* R,
                                      rettn_residual kind, hipStream_t stream);

/* rettn_calibrate_residual with a device workspace (the same step, Re-ttention
 * summary page, "Approach"; review thread, replies to W1 of the first and
 * second reviews).  For bfloat16 calibrations with 64- or 128-token blocks:
 *   - V is first converted to float16 into the workspace, in V's own layout,
 *     by one pass over V; the attention kernel then streams the float16 tiles
 *     instead of re-encoding every V tile in every work-group.  The conversion
 *     is the one the kernel applies otherwise;
 *   - when the work-groups fill at least one round of the current device and
 *     leave a last round at most half full, the last round's groups are cut
 *     into parts along the key range (up to 8, at least two key tiles each);
 *     each part leaves its partial softmax state (reference, both
 *     denominators, both P*V sums) in the workspace and a second pass merges
 *     them into O, rho and R.
 * Without a split, O, rho and R are bit for bit those of
 * rettn_calibrate_residual; the rows of split groups differ from them only by
 * the order of float32 additions.
 *
 * rettn_calibrate_workspace_bytes: the workspace the call needs for `desc` on
 * the current device: V's extent in float16,
 * ((B-1) stride_b + (H-1) stride_h + (L-1) stride_l + d) * 2 bytes, rounded up
 * to 256 and followed by parts * rows * (4 + 2 * dp) * 4 bytes of partial
 * states when a split is planned (dp = d rounded up to 32, 64, 96 or 128;
 * rows = 128 or 256 per group); 0 when the call takes neither (float32,
 * 32-token blocks, or a slice too large for 32-bit offsets).  RETTN_EINVAL for
 * a bad descriptor, RETTN_EUNSUPPORTED for an extent beyond 2^50 elements.
 *
 * rettn_calibrate_ws: as rettn_calibrate_residual, with the size queried while
 * the same device is current.  When that size is not 0 the workspace must be
 * 16-byte aligned, at least that size and overlap none of Q, K, V, O and R
 * (each taken over V's extent) nor rho (B H L floats), else RETTN_EINVAL with
 * nothing launched; when
 * it is 0 the workspace is ignored (it may be null).  The caller owns the
 * workspace; its contents before and after the call mean nothing.  Two or
 * three launches on `stream`, no allocation and no host wait, so the call can
 * be captured in a HIP graph. */
rettn_status rettn_calibrate_workspace_bytes(const rettn_desc* desc, size_t* bytes);
rettn_status rettn_calibrate_ws(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                                const rettn_index* idx, void* workspace, size_t workspace_bytes,
                                void* O, float* rho, void* R, rettn_residual kind, hipStream_t stream);

/* Sparse step `step` (>= 1 sparse steps since the last calibration):
 *   O'_i = min(1, rho_i (1 + lambda step)) * softmax_{W(i)}(s') V'_{W(i)} + R_i
 * over the kept key blocks only (review thread, replies to W1 of the first
 * and third reviews; the ramp-up lambda: answer to W1 of the fourth review;
 * the pages print no ramp formula: this multiplicative, clamped ramp is the
 * reading used).  A row with no kept block gets O'_i = R_i.  Reads rho and R
 * cached by rettn_calibrate; idx->row_ptr and idx->col_idx are walked (those
 * of the row's own head or slice if idx->slices says so).  The mask need not
 * be the calibration's: with a dynamic mask the cached rho and R describe
 * the calibration step's window, as in the pages' trial of dynamic masks.
 * lambda must be finite and >= 0.  For bfloat16, P*V runs in float16 with
 * V converted as in rettn_calibrate. */
rettn_status rettn_sparse(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                          const rettn_index* idx, const float* rho, const void* R,
                          float lambda, int32_t step, void* O, hipStream_t stream);

/* rettn_sparse with a device workspace, into which V is first converted to
 * float16 (V's own layout, one pass over V) so that the sparse kernel streams
 * float16 tiles instead of re-encoding each V tile in every query block that
 * keeps it.  The pass pays when many query blocks keep each key block: it is
 * taken for bfloat16 with 128-token blocks when idx->nnz is at least 24 times
 * nkb (each key block kept by 24 query blocks on average); the conversion is
 * the kernel's own, so O' is bit for bit that of rettn_sparse.
 * rettn_sparse_workspace_bytes: V's extent in float16 (as for
 * rettn_calibrate_workspace_bytes, without the 256-byte rounding) when the
 * pass is taken, else 0; RETTN_EINVAL for a bad descriptor or index.
 * rettn_sparse_ws: as rettn_sparse; the workspace rules are those of
 * rettn_calibrate_ws (aligned, large enough, disjoint from Q, K, V, O, R and
 * rho; ignored when the size is 0). */
rettn_status rettn_sparse_workspace_bytes(const rettn_desc* desc, const rettn_index* idx, size_t* bytes);
rettn_status rettn_sparse_ws(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                             const rettn_index* idx, const float* rho, const void* R, float lambda, int32_t step,
                             void* workspace, size_t workspace_bytes, void* O, hipStream_t stream);

/* A static string naming a status code. */
const char* rettn_status_str(rettn_status status);

#ifdef __cplusplus
}
#endif

#endif /* RETTN_H */
