// Kernel argument block of the attention kernels and the host-side rules that pick a kernel.
// Plain C++ (no HIP headers), so that the host-only code can be compiled and checked on its own.
#pragma once

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
    // Calibration only (64/128-token-block kernel): the last, partial round of work-groups may be
    // split along the key range.  Work items at or past split_from are (group, part) pairs: part p
    // of nsplit walks key tiles [p * nkt / nsplit, (p + 1) * nkt / nsplit) and stores its partial
    // softmax state in `part` (see calib.hip) instead of O, rho and R; a merge pass combines them.
    int32_t split_from;       // first split group; no split when nsplit <= 1
    int32_t nsplit;
    float* part;
};

// d is padded to DP in {32, 64, 96, 128} inside the kernels.
inline int pad_d(int d) { return d <= 32 ? 32 : d <= 64 ? 64 : d <= 96 ? 96 : 128; }

// The fast kernels address one (batch, head) slice through a buffer resource with 32-bit
// offsets: a row offset (row * stride_l * 2 bytes, rows up to the slice's length rounded up to
// a whole work tile) plus, for padded 16-byte chunks, an out-of-range offset of 2^31.  A sum
// that passed 2^32 would wrap onto a valid row, so a slice is taken by these kernels only if
// every such sum stays below 2^32: rows rounded up to 256, times the row pitch, below
// 2^31 - 256.  Other slices take the general kernels, which use 64-bit addresses.
inline bool slice_offsets_fit(const AttnArgs& a) {
    const int64_t rows = ((int64_t)a.L + 255) / 256 * 256;
    return rows * a.sl * 2 <= ((int64_t)1 << 31) - 256;
}

// The calibration kernel for 64- and 128-token blocks (bfloat16, d <= 128) takes a slice when its
// 32-bit offsets fit; other calibrations run on the general kernels.
inline bool calib_fast_path(const AttnArgs& a, int block) {
    return (block == 64 || block == 128) && a.d <= 128 && slice_offsets_fit(a);
}

}  // namespace rettn
