// Launchers of the attention kernels (their argument block is in args.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "args.h"

namespace rettn {

// v16: null, or device memory covering V's extent that receives V in float16 first (bfloat16
// calibrations on the 64/128-token-block kernel; ignored by the other paths).  part: null, or
// calib_split_bytes(a, block) bytes for the partial states of a split last round (with v16 only).
hipError_t launch_calibrate_bf16(AttnArgs a, int block, void* v16, void* part, hipStream_t s);
// v16: null, or device memory covering V's extent for the float16 copy of V (the 128-token-block
// sparse kernel streams it; the other paths ignore it).
hipError_t launch_sparse_bf16(AttnArgs a, int block, void* v16, hipStream_t s);
hipError_t launch_calibrate_f32(AttnArgs a, int block, hipStream_t s);
hipError_t launch_sparse_f32(AttnArgs a, int block, hipStream_t s);

// One-wave-per-query-block sparse step for 64-token blocks (bfloat16, d <= 64).
bool sparse64_supported(const AttnArgs& a, int block);
hipError_t launch_sparse64(AttnArgs a, hipStream_t s);

// Sparse step for 128-token blocks (bfloat16, d <= 128) and 64-token blocks with d > 64: one
// work-group of block / 32 waves per query block.
bool sparse_wg_supported(const AttnArgs& a, int block);
hipError_t launch_sparse_wg(AttnArgs a, int block, void* v16, hipStream_t s);

// V (bfloat16, a's layout) converted to float16 into v16, same offsets: one pass over V.
hipError_t launch_v16(const AttnArgs& a, void* v16, hipStream_t s);

// Calibration for 64- and 128-token blocks (bfloat16): 128 or 256 query rows per work-group.  With
// v16 set, V is first converted to float16 into v16 (same layout) and streamed from there; with
// part set too, a last round of work-groups at most half full is split along the key range and
// merged by a second pass (calib_split_bytes: the partial states' size on the current device,
// 0 when no split is planned).
bool calib_supported(const AttnArgs& a, int block);
size_t calib_split_bytes(const AttnArgs& a, int block);
hipError_t launch_calib(AttnArgs a, int block, void* v16, void* part, hipStream_t s);

// CSR of `slices` masks [slices, nqb, nkb]; slice s's ids start at col_idx + s * nqb * nkb.
hipError_t launch_index_build(const uint8_t* mask, int slices, int nqb, int nkb, int32_t* row_ptr, int32_t* col_idx,
                              hipStream_t s);

// Dynamic block masks (block means -> scores -> per-row top-kk), one per (batch, head) slice.
// ws holds 2 * B * H * nb * d floats.
hipError_t launch_dynamic_index(const void* Q, const void* K, bool bf16, int B, int H, int L, int d, int block,
                                int64_t sb, int64_t sh, int64_t sl, int keep, float* ws, uint8_t* mask,
                                int32_t* row_ptr, int32_t* col_idx, hipStream_t s);

}  // namespace rettn
