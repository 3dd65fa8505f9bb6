// Kernel-side argument block and launchers of the attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rettn {

struct AttnArgs {
    const void* Q;
    const void* K;
    const void* V;
    void* O;
    // calibration writes R and rho; the sparse step reads them
    void* R_out;
    float* rho_out;
    const void* R_in;
    const float* rho_in;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const uint8_t* mask;
    int64_t sb, sh, sl;       // element strides of Q, K, V, O, R
    int32_t B, H, L, d;
    int32_t nqb, nkb;
    float c;                  // log2(e) / sqrt(d): scores enter exp2 pre-scaled
    float ramp;               // 1 + lambda * step (sparse step only)
    int32_t G;                // work-groups in the launch
    int32_t residual;         // calibration's R: 0 masked keys' share of O (Re-ttention), 1 full minus window
                              // attention (the DiTFastAttn comparator)
    // One index per head or per (batch, head) slice: slice bh % slice_mod (1 = one shared index) has its
    // mask at mask + slice * nqb * nkb, row_ptr at row_ptr + slice * (nqb + 1), col_idx at
    // col_idx + slice * col_stride.
    int32_t slice_mod;
    int64_t col_stride;
};

// d is padded to DP in {32, 64, 96, 128} inside the kernels.
inline int pad_d(int d) { return d <= 32 ? 32 : d <= 64 ? 64 : d <= 96 ? 96 : 128; }

hipError_t launch_calibrate_bf16(AttnArgs a, int block, hipStream_t s);
hipError_t launch_sparse_bf16(AttnArgs a, int block, hipStream_t s);
hipError_t launch_calibrate_f32(AttnArgs a, int block, hipStream_t s);
hipError_t launch_sparse_f32(AttnArgs a, int block, hipStream_t s);

// One-wave-per-query-block sparse step for 64-token blocks (bfloat16, d <= 64).
bool sparse64_supported(const AttnArgs& a, int block);
hipError_t launch_sparse64(AttnArgs a, hipStream_t s);

// Sparse step for 128-token blocks (bfloat16, d <= 128) and 64-token blocks with d > 64: one
// work-group of block / 32 waves per query block.
bool sparse_wg_supported(const AttnArgs& a, int block);
hipError_t launch_sparse_wg(AttnArgs a, int block, hipStream_t s);

// Calibration for 64- and 128-token blocks (bfloat16): 128 or 256 query rows per work-group.
bool calib_supported(const AttnArgs& a, int block);
hipError_t launch_calib(AttnArgs a, int block, hipStream_t s);

// CSR of `slices` masks [slices, nqb, nkb]; slice s's ids start at col_idx + s * nqb * nkb.
hipError_t launch_index_build(const uint8_t* mask, int slices, int nqb, int nkb, int32_t* row_ptr, int32_t* col_idx,
                              hipStream_t s);

// Dynamic block masks (block means -> scores -> per-row top-kk), one per (batch, head) slice.
// ws holds 2 * B * H * nb * d floats.
hipError_t launch_dynamic_index(const void* Q, const void* K, bool bf16, int B, int H, int L, int d, int block,
                                int64_t sb, int64_t sh, int64_t sl, int keep, float* ws, uint8_t* mask,
                                int32_t* row_ptr, int32_t* col_idx, hipStream_t s);

}  // namespace rettn
