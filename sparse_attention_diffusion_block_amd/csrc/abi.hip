// C ABI of librettn: the entry points that launch the gfx950 kernels.  Their
// arguments are checked first by the host-only code in host.cpp (which also holds
// the static mask generators); a rejected call launches nothing.
#include <mutex>
#include <vector>

#include "../../include/rettn.h"
#include "attn.h"
#include "host.h"

namespace {

using rettn::AttnArgs;
namespace host = rettn::host;

// Scratch of the no-allocation entry point: a static device array, one copy per GPU.  Host code
// never uses the array's name as an address (on the host it is only a stand-in); it uses the
// device address looked up once per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[RETTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on its first use (null on failure).
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

// Layout of rettn_calibrate_ws's workspace: V in float16 over V's extent, then (256-byte aligned)
// the partial states of a split last round, when one is planned on the current device.
struct CalibWorkspace {
    size_t v16 = 0, part_offset = 0, part = 0, total = 0;
};

rettn_status calib_workspace(const rettn_desc* desc, CalibWorkspace* w) {
    rettn_status st = host::calibrate_workspace(desc, &w->v16);
    if (st != RETTN_OK || w->v16 == 0) return st;
    AttnArgs a{};
    a.B = desc->B;
    a.H = desc->H;
    a.L = desc->L;
    a.d = desc->d;
    a.sl = desc->stride_l;
    w->part_offset = (w->v16 + 255) / 256 * 256;
    w->part = rettn::calib_split_bytes(a, desc->block);
    w->total = w->part ? w->part_offset + w->part : w->v16;
    return RETTN_OK;
}

// bytes of rho: one float per (batch, head, row); the descriptor has been validated (B H L < 2^40)
size_t rho_bytes(const rettn_desc* desc) { return (size_t)desc->B * desc->H * desc->L * sizeof(float); }

}  // namespace

extern "C" {

rettn_status rettn_index_build(const uint8_t* mask_dev, int32_t nqb, int32_t nkb, int32_t* row_ptr_dev,
                               int32_t* col_idx_dev, int32_t* nnz_host, hipStream_t stream) {
    return rettn_index_build_sliced(mask_dev, 1, nqb, nkb, row_ptr_dev, col_idx_dev, nnz_host, stream);
}

rettn_status rettn_index_build_sliced(const uint8_t* mask_dev, int32_t slices, int32_t nqb, int32_t nkb,
                                      int32_t* row_ptr_dev, int32_t* col_idx_dev, int32_t* nnz_host,
                                      hipStream_t stream) {
    const rettn_status st = host::check_index_build(mask_dev, slices, nqb, nkb, row_ptr_dev, col_idx_dev, nnz_host);
    if (st != RETTN_OK) return st;
    if (rettn::launch_index_build(mask_dev, slices, nqb, nkb, row_ptr_dev, col_idx_dev, stream) != hipSuccess)
        return RETTN_EHIP;
    // each slice's total is its last row pointer: gather them (pitch nqb + 1) and take the largest
    std::vector<int32_t> totals((size_t)slices, 0);
    if (hipMemcpy2DAsync(totals.data(), sizeof(int32_t), row_ptr_dev + nqb, sizeof(int32_t) * ((size_t)nqb + 1),
                         sizeof(int32_t), (size_t)slices, hipMemcpyDeviceToHost, stream) != hipSuccess)
        return RETTN_EHIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return RETTN_EHIP;
    *nnz_host = host::largest_total(totals.data(), slices);
    return RETTN_OK;
}

static rettn_status launch_dynamic(const rettn_desc* desc, const void* Q, const void* K, int32_t keep, float* ws,
                                   uint8_t* mask_out, int32_t* row_ptr_out, int32_t* col_idx_out,
                                   hipStream_t stream) {
    const hipError_t e = rettn::launch_dynamic_index(Q, K, desc->dtype == RETTN_BF16, desc->B, desc->H, desc->L,
                                                     desc->d, desc->block, desc->stride_b, desc->stride_h,
                                                     desc->stride_l, keep, ws, mask_out, row_ptr_out, col_idx_out,
                                                     stream);
    return e == hipSuccess ? RETTN_OK : RETTN_EHIP;
}

rettn_status rettn_dynamic_index(const rettn_desc* desc, const void* Q, const void* K, int32_t keep, void* workspace,
                                 size_t workspace_bytes, uint8_t* mask_out, int32_t* row_ptr_out,
                                 int32_t* col_idx_out, hipStream_t stream) {
    size_t need = 0;
    rettn_status st = host::prepare_dynamic(desc, Q, K, keep, mask_out, row_ptr_out, col_idx_out, &need);
    if (st != RETTN_OK) return st;
    if (!host::tensor_ok(workspace) || workspace_bytes < need) return RETTN_EINVAL;
    return launch_dynamic(desc, Q, K, keep, (float*)workspace, mask_out, row_ptr_out, col_idx_out, stream);
}

rettn_status rettn_dynamic_index_noalloc(const rettn_desc* desc, const void* Q, const void* K, int32_t keep,
                                         uint8_t* mask_out, int32_t* row_ptr_out, int32_t* col_idx_out,
                                         hipStream_t stream) {
    size_t need = 0;
    rettn_status st = host::prepare_dynamic(desc, Q, K, keep, mask_out, row_ptr_out, col_idx_out, &need);
    if (st != RETTN_OK) return st;
    if (need > RETTN_NOALLOC_SCRATCH_BYTES) return RETTN_ESCRATCH;
    void* ws = scratch_for_current_device();
    if (!ws) return RETTN_EHIP;
    return launch_dynamic(desc, Q, K, keep, (float*)ws, mask_out, row_ptr_out, col_idx_out, stream);
}

rettn_status rettn_calibrate(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                             const rettn_index* idx, void* O, float* rho, void* R, hipStream_t stream) {
    return rettn_calibrate_residual(desc, Q, K, V, idx, O, rho, R, RETTN_RESIDUAL_MASKED, stream);
}

rettn_status rettn_calibrate_residual(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                                      const rettn_index* idx, void* O, float* rho, void* R, rettn_residual kind,
                                      hipStream_t stream) {
    AttnArgs a{};
    const rettn_status st = host::prepare_calibrate(desc, Q, K, V, idx, O, rho, R, kind, &a);
    if (st != RETTN_OK) return st;
    const hipError_t e = desc->dtype == RETTN_BF16
                             ? rettn::launch_calibrate_bf16(a, desc->block, nullptr, nullptr, stream)
                             : rettn::launch_calibrate_f32(a, desc->block, stream);
    return e == hipSuccess ? RETTN_OK : RETTN_EHIP;
}

rettn_status rettn_calibrate_workspace_bytes(const rettn_desc* desc, size_t* bytes) {
    if (!bytes) return RETTN_EINVAL;
    CalibWorkspace w;
    const rettn_status st = calib_workspace(desc, &w);
    if (st == RETTN_OK) *bytes = w.total;
    return st;
}

rettn_status rettn_calibrate_ws(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                                const rettn_index* idx, void* workspace, size_t workspace_bytes, void* O, float* rho,
                                void* R, rettn_residual kind, hipStream_t stream) {
    AttnArgs a{};
    rettn_status st = host::prepare_calibrate(desc, Q, K, V, idx, O, rho, R, kind, &a);
    if (st != RETTN_OK) return st;
    CalibWorkspace w;
    st = calib_workspace(desc, &w);
    if (st != RETTN_OK) return st;
    st = host::check_calibrate_workspace(workspace, workspace_bytes, w.total, w.v16, {Q, K, V, O, R});
    if (st != RETTN_OK) return st;
    st = host::check_calibrate_workspace(workspace, workspace_bytes, w.total, rho_bytes(desc), {rho});
    if (st != RETTN_OK) return st;
    void* v16 = w.total ? workspace : nullptr;
    void* part = w.part ? (char*)workspace + w.part_offset : nullptr;
    const hipError_t e = desc->dtype == RETTN_BF16 ? rettn::launch_calibrate_bf16(a, desc->block, v16, part, stream)
                                                   : rettn::launch_calibrate_f32(a, desc->block, stream);
    return e == hipSuccess ? RETTN_OK : RETTN_EHIP;
}

rettn_status rettn_sparse(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                          const rettn_index* idx, const float* rho, const void* R, float lambda, int32_t step,
                          void* O, hipStream_t stream) {
    AttnArgs a{};
    const rettn_status st = host::prepare_sparse(desc, Q, K, V, idx, rho, R, lambda, step, O, &a);
    if (st != RETTN_OK) return st;
    const hipError_t e = desc->dtype == RETTN_BF16 ? rettn::launch_sparse_bf16(a, desc->block, nullptr, stream)
                                                   : rettn::launch_sparse_f32(a, desc->block, stream);
    return e == hipSuccess ? RETTN_OK : RETTN_EHIP;
}

rettn_status rettn_sparse_workspace_bytes(const rettn_desc* desc, const rettn_index* idx, size_t* bytes) {
    return host::sparse_workspace(desc, idx, bytes);
}

rettn_status rettn_sparse_ws(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                             const rettn_index* idx, const float* rho, const void* R, float lambda, int32_t step,
                             void* workspace, size_t workspace_bytes, void* O, hipStream_t stream) {
    AttnArgs a{};
    rettn_status st = host::prepare_sparse(desc, Q, K, V, idx, rho, R, lambda, step, O, &a);
    if (st != RETTN_OK) return st;
    size_t need = 0;
    st = host::sparse_workspace(desc, idx, &need);
    if (st != RETTN_OK) return st;
    st = host::check_calibrate_workspace(workspace, workspace_bytes, need, need, {Q, K, V, O, R});
    if (st != RETTN_OK) return st;
    st = host::check_calibrate_workspace(workspace, workspace_bytes, need, rho_bytes(desc), {rho});
    if (st != RETTN_OK) return st;
    const hipError_t e = desc->dtype == RETTN_BF16
                             ? rettn::launch_sparse_bf16(a, desc->block, need ? workspace : nullptr, stream)
                             : rettn::launch_sparse_f32(a, desc->block, stream);
    return e == hipSuccess ? RETTN_OK : RETTN_EHIP;
}

}  // extern "C"
