// Host-side part of the C ABI: argument validation, the static mask generators and the
// bookkeeping around the kernels.  Plain C++ with no device code, so that it can be built and
// exercised on its own (with the address and undefined-behaviour sanitizers) without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/rettn.h"
#include "args.h"

namespace rettn {
namespace host {

int64_t cdiv(int64_t a, int64_t b);

// Checks of rettn_calibrate_residual; on RETTN_OK, *args holds the kernel arguments.
rettn_status prepare_calibrate(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                               const rettn_index* idx, void* O, float* rho, void* R, rettn_residual kind,
                               AttnArgs* args);

// Workspace of rettn_calibrate_ws for `desc`: the float16 copy of V in V's own layout when the
// calibration kernel for 64/128-token blocks takes the call (bfloat16), else 0.  RETTN_EINVAL for a
// bad descriptor.
rettn_status calibrate_workspace(const rettn_desc* desc, size_t* bytes);

// Workspace of rettn_sparse_ws: the float16 copy of V when the 128-token-block sparse kernel takes
// the call (bfloat16) and each key block is kept, on average, by at least kSparseV16Readers query
// blocks (idx->nnz >= that many times nkb), else 0.  RETTN_EINVAL for a bad descriptor or index.
constexpr int64_t kSparseV16Readers = 24;
rettn_status sparse_workspace(const rettn_desc* desc, const rettn_index* idx, size_t* bytes);

// Checks of rettn_calibrate_ws's workspace: when need > 0 it must be 16-byte aligned, at least need
// bytes, and [workspace, workspace + need) must overlap none of the tensors, each tensor_bytes long.
// A workspace the call does not need (need == 0) is ignored.
rettn_status check_calibrate_workspace(const void* workspace, size_t workspace_bytes, size_t need,
                                       size_t tensor_bytes, std::initializer_list<const void*> tensors);

// Checks of rettn_sparse; on RETTN_OK, *args holds the kernel arguments (ramp = 1 + lambda step).
rettn_status prepare_sparse(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                            const rettn_index* idx, const float* rho, const void* R, float lambda, int32_t step,
                            void* O, AttnArgs* args);

// Checks shared by both dynamic-index entry points; on RETTN_OK, *need is the block means' size.
rettn_status prepare_dynamic(const rettn_desc* desc, const void* Q, const void* K, int32_t keep,
                             const uint8_t* mask_out, const int32_t* row_ptr_out, const int32_t* col_idx_out,
                             size_t* need);

// Checks of rettn_index_build_sliced (before any launch).
rettn_status check_index_build(const uint8_t* mask_dev, int32_t slices, int32_t nqb, int32_t nkb,
                               const int32_t* row_ptr_dev, const int32_t* col_idx_dev, const int32_t* nnz_host);

// The index's nnz: the largest of the slices' kept-pair counts (each slice's last row pointer).
int32_t largest_total(const int32_t* totals, int32_t slices);

// 16-byte aligned and not null.
bool tensor_ok(const void* p);

}  // namespace host
}  // namespace rettn
