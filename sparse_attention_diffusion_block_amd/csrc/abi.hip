// C ABI of librettn: argument validation, the host-side static mask
// generators and dispatch to the gfx950 kernels.  Every argument is checked
// before anything is launched; a rejected call launches nothing.
#include <math.h>
#include <string.h>

#include <initializer_list>
#include <vector>

#include "../../include/rettn.h"
#include "attn.h"

namespace {

using rettn::AttnArgs;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape, dtype, stride and pointer checks common to both attention steps.
rettn_status check_desc(const rettn_desc* d, const rettn_index* idx) {
    if (!d || !idx) return RETTN_EINVAL;
    if (d->B < 1 || d->H < 1 || d->L < 1) return RETTN_EINVAL;
    if (d->d < 1 || d->d > 128) return RETTN_EINVAL;
    if (d->block != 32 && d->block != 64 && d->block != 128) return RETTN_EINVAL;
    if (d->dtype != RETTN_F32 && d->dtype != RETTN_BF16) return RETTN_EINVAL;
    const int64_t gran = d->dtype == RETTN_BF16 ? 8 : 4;   // elements per 16 bytes
    if (d->d % gran != 0) return RETTN_EINVAL;
    if (d->stride_l < d->d || d->stride_h < 1 || d->stride_b < 1) return RETTN_EINVAL;
    if (d->stride_l % gran || d->stride_h % gran || d->stride_b % gran) return RETTN_EINVAL;
    const int64_t nb = cdiv(d->L, d->block);
    if (idx->nqb != nb || idx->nkb != nb) return RETTN_EINVAL;
    // one shared index, one per head, or one per (batch, head) slice
    const int64_t S = (int64_t)d->B * d->H;
    if (idx->slices < 0 || (idx->slices > 1 && idx->slices != d->H && idx->slices != S)) return RETTN_EINVAL;
    if (idx->slices > 1 && (idx->col_stride < 0 || idx->nnz > idx->col_stride)) return RETTN_EINVAL;
    if ((int64_t)d->B * d->H * nb > 0x7fffffff) return RETTN_EUNSUPPORTED;
    if ((int64_t)d->B * d->H * d->L > ((int64_t)1 << 40)) return RETTN_EUNSUPPORTED;
    return RETTN_OK;
}

// Tensors are read and written in 16-byte chunks; rho and the index arrays element-wise.
rettn_status check_tensors(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p || !aligned16(p)) return RETTN_EINVAL;
    return RETTN_OK;
}

rettn_status check_words(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p || ((uintptr_t)p & 3u) != 0) return RETTN_EINVAL;
    return RETTN_OK;
}

AttnArgs make_args(const rettn_desc* d, const void* Q, const void* K, const void* V, const rettn_index* idx, void* O) {
    AttnArgs a{};
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = O;
    a.row_ptr = idx->row_ptr;
    a.col_idx = idx->col_idx;
    a.mask = idx->mask;
    a.sb = d->stride_b;
    a.sh = d->stride_h;
    a.sl = d->stride_l;
    a.B = d->B;
    a.H = d->H;
    a.L = d->L;
    a.d = d->d;
    a.nqb = idx->nqb;
    a.nkb = idx->nkb;
    // slice of (batch, head) bh: bh % slice_mod (bh < B*H, so B*H gives bh itself)
    a.slice_mod = idx->slices <= 1 ? 1 : idx->slices == d->H ? d->H : d->B * d->H;
    a.col_stride = idx->slices <= 1 ? 0 : idx->col_stride;
    a.c = (float)(1.4426950408889634 / sqrt((double)d->d));
    a.ramp = 1.f;
    return a;
}

}  // namespace

extern "C" {

const char* rettn_status_str(rettn_status s) {
    switch (s) {
        case RETTN_OK: return "RETTN_OK";
        case RETTN_EINVAL: return "RETTN_EINVAL: invalid argument";
        case RETTN_EUNSUPPORTED: return "RETTN_EUNSUPPORTED: outside the implemented shapes";
        case RETTN_EHIP: return "RETTN_EHIP: HIP runtime or launch failure";
    }
    return "unknown rettn_status";
}

rettn_status rettn_mask_build(const rettn_mask_spec* spec, uint8_t* mask) {
    if (!spec || !mask) return RETTN_EINVAL;
    const int nb = spec->nb;
    if (nb < 1 || nb > 65536) return RETTN_EINVAL;
    switch (spec->kind) {
        case RETTN_MASK_DIAG:
        case RETTN_MASK_FULL: break;
        case RETTN_MASK_BAND:
            if (spec->w < 1 || spec->w > nb) return RETTN_EINVAL;
            break;
        case RETTN_MASK_COGVIDEO3D:
            if (spec->text_blocks < 0 || spec->text_blocks > nb || spec->tshift < 1) return RETTN_EINVAL;
            break;
        default: return RETTN_EINVAL;
    }
    memset(mask, 0, (size_t)nb * (size_t)nb);
    for (int qb = 0; qb < nb; ++qb) {
        uint8_t* row = mask + (size_t)qb * nb;
        switch (spec->kind) {
            case RETTN_MASK_DIAG: row[qb] = 1; break;
            case RETTN_MASK_FULL: memset(row, 1, (size_t)nb); break;
            case RETTN_MASK_BAND: {
                int lo = qb - (spec->w - 1) / 2;
                if (lo > nb - spec->w) lo = nb - spec->w;
                if (lo < 0) lo = 0;
                memset(row + lo, 1, (size_t)spec->w);
                break;
            }
            case RETTN_MASK_COGVIDEO3D: {
                memset(row, 1, (size_t)spec->text_blocks);
                const int nbr[5] = {qb - 1, qb, qb + 1, qb - spec->tshift, qb + spec->tshift};
                for (int k : nbr)
                    if (k >= 0 && k < nb) row[k] = 1;
                break;
            }
        }
    }
    return RETTN_OK;
}

rettn_status rettn_index_build(const uint8_t* mask_dev, int32_t nqb, int32_t nkb, int32_t* row_ptr_dev,
                               int32_t* col_idx_dev, int32_t* nnz_host, hipStream_t stream) {
    return rettn_index_build_sliced(mask_dev, 1, nqb, nkb, row_ptr_dev, col_idx_dev, nnz_host, stream);
}

rettn_status rettn_index_build_sliced(const uint8_t* mask_dev, int32_t slices, int32_t nqb, int32_t nkb,
                                      int32_t* row_ptr_dev, int32_t* col_idx_dev, int32_t* nnz_host,
                                      hipStream_t stream) {
    if (!mask_dev || !row_ptr_dev || !col_idx_dev || !nnz_host) return RETTN_EINVAL;
    if (nqb < 1 || nkb < 1 || (int64_t)nqb * nkb > 0x7fffffff) return RETTN_EINVAL;
    if (slices < 1 || slices > 65535) return RETTN_EINVAL;
    if (rettn::launch_index_build(mask_dev, slices, nqb, nkb, row_ptr_dev, col_idx_dev, stream) != hipSuccess)
        return RETTN_EHIP;
    // each slice's total is its last row pointer: gather them (pitch nqb + 1) and take the largest
    std::vector<int32_t> totals((size_t)slices, 0);
    if (hipMemcpy2DAsync(totals.data(), sizeof(int32_t), row_ptr_dev + nqb, sizeof(int32_t) * ((size_t)nqb + 1),
                         sizeof(int32_t), (size_t)slices, hipMemcpyDeviceToHost, stream) != hipSuccess)
        return RETTN_EHIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return RETTN_EHIP;
    int32_t nnz = 0;
    for (int32_t t : totals) nnz = t > nnz ? t : nnz;
    *nnz_host = nnz;
    return RETTN_OK;
}

rettn_status rettn_dynamic_workspace_bytes(const rettn_desc* desc, size_t* bytes) {
    if (!desc || !bytes) return RETTN_EINVAL;
    if (desc->B < 1 || desc->H < 1 || desc->L < 1 || desc->d < 1 || desc->d > 128) return RETTN_EINVAL;
    if (desc->block != 32 && desc->block != 64 && desc->block != 128) return RETTN_EINVAL;
    *bytes = 2 * sizeof(float) * (size_t)desc->B * (size_t)desc->H * (size_t)cdiv(desc->L, desc->block) *
             (size_t)desc->d;
    return RETTN_OK;
}

rettn_status rettn_dynamic_index(const rettn_desc* desc, const void* Q, const void* K, int32_t keep, void* workspace,
                                 size_t workspace_bytes, uint8_t* mask_out, int32_t* row_ptr_out,
                                 int32_t* col_idx_out, hipStream_t stream) {
    if (!desc) return RETTN_EINVAL;
    const int64_t nb = cdiv(desc->L > 0 ? desc->L : 1, desc->block > 0 ? desc->block : 1);
    // the index that the outputs form: its checks are the attention calls' own
    rettn_index idx{};
    idx.nqb = idx.nkb = (int32_t)(nb > 0x7fffffff ? 0 : nb);
    rettn_status st = check_desc(desc, &idx);
    if (st != RETTN_OK) return st;
    st = check_tensors({Q, K, workspace});
    if (st != RETTN_OK) return st;
    if (!mask_out || check_words({row_ptr_out, col_idx_out}) != RETTN_OK) return RETTN_EINVAL;
    if (keep < 1) return RETTN_EINVAL;
    if (nb > 2048 || (int64_t)desc->B * desc->H > 65535) return RETTN_EUNSUPPORTED;
    size_t need = 0;
    st = rettn_dynamic_workspace_bytes(desc, &need);
    if (st != RETTN_OK) return st;
    if (workspace_bytes < need) return RETTN_EINVAL;
    const hipError_t e = rettn::launch_dynamic_index(Q, K, desc->dtype == RETTN_BF16, desc->B, desc->H, desc->L,
                                                     desc->d, desc->block, desc->stride_b, desc->stride_h,
                                                     desc->stride_l, keep, (float*)workspace, mask_out, row_ptr_out,
                                                     col_idx_out, stream);
    return e == hipSuccess ? RETTN_OK : RETTN_EHIP;
}

rettn_status rettn_calibrate(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                             const rettn_index* idx, void* O, float* rho, void* R, hipStream_t stream) {
    return rettn_calibrate_residual(desc, Q, K, V, idx, O, rho, R, RETTN_RESIDUAL_MASKED, stream);
}

rettn_status rettn_calibrate_residual(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                                      const rettn_index* idx, void* O, float* rho, void* R, rettn_residual kind,
                                      hipStream_t stream) {
    if (kind != RETTN_RESIDUAL_MASKED && kind != RETTN_RESIDUAL_DIFFERENCE) return RETTN_EINVAL;
    rettn_status st = check_desc(desc, idx);
    if (st != RETTN_OK) return st;
    st = check_tensors({Q, K, V, O, R});
    if (st != RETTN_OK) return st;
    st = check_words({rho});
    if (st != RETTN_OK) return st;
    if (!idx->mask) return RETTN_EINVAL;
    AttnArgs a = make_args(desc, Q, K, V, idx, O);
    a.R_out = R;
    a.rho_out = rho;
    a.residual = kind == RETTN_RESIDUAL_DIFFERENCE ? 1 : 0;
    const hipError_t e = desc->dtype == RETTN_BF16 ? rettn::launch_calibrate_bf16(a, desc->block, stream)
                                                   : rettn::launch_calibrate_f32(a, desc->block, stream);
    return e == hipSuccess ? RETTN_OK : RETTN_EHIP;
}

rettn_status rettn_sparse(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                          const rettn_index* idx, const float* rho, const void* R, float lambda, int32_t step,
                          void* O, hipStream_t stream) {
    rettn_status st = check_desc(desc, idx);
    if (st != RETTN_OK) return st;
    st = check_tensors({Q, K, V, O, R});
    if (st != RETTN_OK) return st;
    st = check_words({rho, idx->row_ptr});
    if (st != RETTN_OK) return st;
    if (idx->nnz > 0 && check_words({idx->col_idx}) != RETTN_OK) return RETTN_EINVAL;
    if (!(lambda >= 0.f) || !isfinite(lambda) || step < 0) return RETTN_EINVAL;
    if (idx->nnz < 0 || (int64_t)idx->nnz > (int64_t)idx->nqb * idx->nkb) return RETTN_EINVAL;
    AttnArgs a = make_args(desc, Q, K, V, idx, O);
    a.R_in = R;
    a.rho_in = rho;
    a.ramp = (float)(1.0 + (double)lambda * (double)step);
    const hipError_t e = desc->dtype == RETTN_BF16 ? rettn::launch_sparse_bf16(a, desc->block, stream)
                                                   : rettn::launch_sparse_f32(a, desc->block, stream);
    return e == hipSuccess ? RETTN_OK : RETTN_EHIP;
}

}  // extern "C"
