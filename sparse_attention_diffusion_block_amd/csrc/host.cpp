// Host-side part of the C ABI (see host.h): validation, the static mask generators, and the
// entry points that need no GPU.  Every argument is checked before anything is launched.
#include "host.h"

#include <math.h>
#include <string.h>

#include <initializer_list>

namespace rettn {
namespace host {

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

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
    // S < 2^62; once S <= 2^31 - 1, S * nb and S * L stay below 2^62 (no overflow in 64 bits)
    if (S > 0x7fffffff || S * nb > 0x7fffffff) return RETTN_EUNSUPPORTED;
    if (S * d->L > ((int64_t)1 << 40)) return RETTN_EUNSUPPORTED;
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

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool tensor_ok(const void* p) { return p && aligned16(p); }

rettn_status prepare_calibrate(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                               const rettn_index* idx, void* O, float* rho, void* R, rettn_residual kind,
                               AttnArgs* args) {
    if (!args) return RETTN_EINVAL;
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
    *args = a;
    return RETTN_OK;
}

rettn_status calibrate_workspace(const rettn_desc* desc, size_t* bytes) {
    if (!desc || !bytes) return RETTN_EINVAL;
    const int64_t nb = desc->block > 0 ? cdiv(desc->L, desc->block) : 0;
    rettn_index idx{};
    idx.nqb = idx.nkb = (int32_t)nb;
    rettn_status st = check_desc(desc, &idx);
    if (st != RETTN_OK) return st;
    *bytes = 0;
    if (desc->dtype != RETTN_BF16) return RETTN_OK;
    AttnArgs a{};
    a.L = desc->L;
    a.d = desc->d;
    a.sl = desc->stride_l;
    if (!calib_fast_path(a, desc->block)) return RETTN_OK;
    // V's extent in elements: the last (batch, head, row)'s d elements end there.  The strides are
    // unbounded int64 values, so the sum is formed in 128 bits and must stay below 2^50.
    const __int128 last = (__int128)(desc->B - 1) * desc->stride_b + (__int128)(desc->H - 1) * desc->stride_h +
                          (__int128)(desc->L - 1) * desc->stride_l + desc->d;
    if (last > ((__int128)1 << 50)) return RETTN_EUNSUPPORTED;
    *bytes = (size_t)last * 2u;
    return RETTN_OK;
}

rettn_status sparse_workspace(const rettn_desc* desc, const rettn_index* idx, size_t* bytes) {
    if (!desc || !idx || !bytes) return RETTN_EINVAL;
    rettn_status st = check_desc(desc, idx);
    if (st != RETTN_OK) return st;
    *bytes = 0;
    if (desc->dtype != RETTN_BF16 || desc->block != 128 || idx->nnz < 0) return RETTN_OK;
    if ((int64_t)idx->nnz < kSparseV16Readers * idx->nkb) return RETTN_OK;
    size_t v16 = 0;
    st = calibrate_workspace(desc, &v16);       // V's extent in float16 on the 128-token-block kernel
    if (st != RETTN_OK) return st;
    *bytes = v16;
    return RETTN_OK;
}

rettn_status check_calibrate_workspace(const void* workspace, size_t workspace_bytes, size_t need,
                                       size_t tensor_bytes, std::initializer_list<const void*> tensors) {
    if (need == 0) return RETTN_OK;
    if (!tensor_ok(workspace) || workspace_bytes < need) return RETTN_EINVAL;
    const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + need;
    for (const void* t : tensors) {
        const uintptr_t t0 = (uintptr_t)t, t1 = t0 + tensor_bytes;
        if (w0 < t1 && t0 < w1) return RETTN_EINVAL;
    }
    return RETTN_OK;
}

rettn_status prepare_sparse(const rettn_desc* desc, const void* Q, const void* K, const void* V,
                            const rettn_index* idx, const float* rho, const void* R, float lambda, int32_t step,
                            void* O, AttnArgs* args) {
    if (!args) return RETTN_EINVAL;
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
    *args = a;
    return RETTN_OK;
}

rettn_status prepare_dynamic(const rettn_desc* desc, const void* Q, const void* K, int32_t keep,
                             const uint8_t* mask_out, const int32_t* row_ptr_out, const int32_t* col_idx_out,
                             size_t* need) {
    if (!desc || !need) return RETTN_EINVAL;
    const int64_t nb = cdiv(desc->L > 0 ? desc->L : 1, desc->block > 0 ? desc->block : 1);
    // the index that the outputs form: its checks are the attention calls' own
    rettn_index idx{};
    idx.nqb = idx.nkb = (int32_t)(nb > 0x7fffffff ? 0 : nb);
    rettn_status st = check_desc(desc, &idx);
    if (st != RETTN_OK) return st;
    st = check_tensors({Q, K});
    if (st != RETTN_OK) return st;
    if (!mask_out || check_words({row_ptr_out, col_idx_out}) != RETTN_OK) return RETTN_EINVAL;
    if (keep < 1) return RETTN_EINVAL;
    if (nb > 2048 || (int64_t)desc->B * desc->H > 65535) return RETTN_EUNSUPPORTED;
    return rettn_dynamic_workspace_bytes(desc, need);
}

rettn_status check_index_build(const uint8_t* mask_dev, int32_t slices, int32_t nqb, int32_t nkb,
                               const int32_t* row_ptr_dev, const int32_t* col_idx_dev, const int32_t* nnz_host) {
    if (!mask_dev || !row_ptr_dev || !col_idx_dev || !nnz_host) return RETTN_EINVAL;
    if (nqb < 1 || nkb < 1 || (int64_t)nqb * nkb > 0x7fffffff) return RETTN_EINVAL;
    if (slices < 1 || slices > 65535) return RETTN_EINVAL;
    // every slice's arrays must be addressable with 32-bit element indices
    if ((int64_t)slices * nqb * nkb > 0x7fffffff || (int64_t)slices * ((int64_t)nqb + 1) > 0x7fffffff)
        return RETTN_EINVAL;
    return RETTN_OK;
}

int32_t largest_total(const int32_t* totals, int32_t slices) {
    int32_t nnz = 0;
    for (int32_t s = 0; s < slices; ++s) nnz = totals[s] > nnz ? totals[s] : nnz;
    return nnz;
}

}  // namespace host
}  // namespace rettn

extern "C" {

const char* rettn_status_str(rettn_status s) {
    switch (s) {
        case RETTN_OK: return "RETTN_OK";
        case RETTN_EINVAL: return "RETTN_EINVAL: invalid argument";
        case RETTN_EUNSUPPORTED: return "RETTN_EUNSUPPORTED: outside the implemented shapes";
        case RETTN_EHIP: return "RETTN_EHIP: HIP runtime or launch failure";
        case RETTN_ESCRATCH: return "RETTN_ESCRATCH: request exceeds the static scratch of the no-allocation entry point";
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
                // neighbours in 64-bit arithmetic: qb + tshift must not overflow for any tshift
                const int64_t nbr[5] = {(int64_t)qb - 1, qb, (int64_t)qb + 1, (int64_t)qb - spec->tshift,
                                        (int64_t)qb + spec->tshift};
                for (int64_t k : nbr)
                    if (k >= 0 && k < nb) row[k] = 1;
                break;
            }
        }
    }
    return RETTN_OK;
}

rettn_status rettn_dynamic_workspace_bytes(const rettn_desc* desc, size_t* bytes) {
    if (!desc || !bytes) return RETTN_EINVAL;
    if (desc->B < 1 || desc->H < 1 || desc->L < 1 || desc->d < 1 || desc->d > 128) return RETTN_EINVAL;
    if (desc->block != 32 && desc->block != 64 && desc->block != 128) return RETTN_EINVAL;
    // the attention calls' own size limit; it also keeps the product below 2^51 bytes
    const int64_t S = (int64_t)desc->B * desc->H;   // < 2^62
    if (S > 0x7fffffff || S * desc->L > ((int64_t)1 << 40)) return RETTN_EUNSUPPORTED;
    *bytes = 2 * sizeof(float) * (size_t)desc->B * (size_t)desc->H *
             (size_t)rettn::host::cdiv(desc->L, desc->block) * (size_t)desc->d;
    return RETTN_OK;
}

}  // extern "C"
