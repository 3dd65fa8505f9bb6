// float32 attention kernels for gfx950: calibration and sparse step with
// float32 operands on the matrix cores (v_mfma_f32_32x32x2f32), for callers
// whose tensors are float32.  Same structure as the bfloat16 kernels: the
// transposed products S^T = K Q^T and O^T += V^T P^T give one query row per
// lane; the calibration routes each key block's mass and P*V into the
// in-window or the masked accumulator by the static mask bit, the sparse step
// walks the CSR row and fuses  O' = min(1, rho * ramp) * acc / D' + R.
// (Re-ttention summary page, "Approach"; review thread, replies to W1 of the
// first three reviews and to W1 of the fourth review.)
//
// Fragment maps of v_mfma_f32_32x32x2f32 (lane l, n = l % 32, h = l / 32):
//   A[m][k]: A[n][h]     B[k][n]: B[h][n]     C[i][n]: acc[4 b + r] = C[8 b + 4 h + r][n]
// The P^T operand of k-step j is the lane's own acc[j] (key 8 (j/4) + 4 h + j%4),
// so the matching V^T operand is V[that key][d = 32 dt + n]: no transposition.
#include "attn.h"
#include "common.h"

namespace rettn {

template <int BLOCK, int DP, bool CALIB>
struct F32Cfg {
    static constexpr int NW = CALIB ? 4 : BLOCK / 32;
    static constexpr int NT = NW * 64;
    static constexpr int QT = NW * 32;
    static constexpr int NS = DP / 2;        // k-steps of S^T over d
    static constexpr int NDT = DP / 32;
    static constexpr int KT = BLOCK / 32;
    static constexpr int RSF = DP + 1;       // odd LDS row stride: column reads hit 32 distinct banks
    static constexpr int CPR = DP / 4;       // 16-byte chunks per key row
    static constexpr int TOTAL = BLOCK * CPR;
    static constexpr int CPT = (TOTAL + NT - 1) / NT;
};

template <int BLOCK, int DP, bool CALIB>
__global__ void __launch_bounds__((F32Cfg<BLOCK, DP, CALIB>::NT))
attn_f32_kernel(const AttnArgs a) {
    using C = F32Cfg<BLOCK, DP, CALIB>;
    __shared__ float sk[BLOCK * C::RSF];
    __shared__ float sv[BLOCK * C::RSF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, n = lane & 31;

    const int ntile = CALIB ? (a.L + C::QT - 1) / C::QT : a.nqb;
    const int work = xcd_remap(blockIdx.x, a.G);
    const int bh = work / ntile;
    const int tile = work - bh * ntile;
    const int bi = bh / a.H, hi = bh - bi * a.H;
    const int sl = bh % a.slice_mod;                        // this slice's index
    const int32_t* rp = a.row_ptr + (int64_t)sl * (a.nqb + 1);
    const int32_t* ci = a.col_idx + (int64_t)sl * a.col_stride;
    const int64_t base = (int64_t)bi * a.sb + (int64_t)hi * a.sh;
    const int q0 = tile * C::QT + wave * 32;
    const int qb = min(q0 / BLOCK, a.nqb - 1);
    const int row = q0 + n;
    const bool row_ok = row < a.L;

    const float* Qp = (const float*)a.Q + base;
    const float* Kp = (const float*)a.K + base;
    const float* Vp = (const float*)a.V + base;

    float qf[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        const int dd = 2 * s + h;
        qf[s] = (row_ok && dd < a.d) ? Qp[(int64_t)row * a.sl + dd] : 0.f;
    }

    float rho_c = 0.f;
    f32x4 rres[C::NDT][4];
    if constexpr (!CALIB) {
        if (row_ok) rho_c = a.rho_in[(int64_t)bh * a.L + row];
        const float* Rp = (const float*)a.R_in + base + (int64_t)row * a.sl;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int d0 = 32 * dt + 8 * bb + 4 * h;
                f32x4 w = {0.f, 0.f, 0.f, 0.f};
                if (row_ok && d0 < a.d) w = *(const f32x4*)(Rp + d0);
                rres[dt][bb] = w;
            }
    }

    int e0 = 0, nit;
    if constexpr (CALIB) {
        nit = a.nkb;
    } else {
        e0 = scalar_load(rp, qb);
        nit = scalar_load(rp, qb + 1) - e0;
    }
    const int64_t mrow = ((int64_t)sl * a.nqb + qb) * a.nkb;   // this wave's mask row (calibration)

    f32x16 acc[C::NDT];
    f32x16 acc2[CALIB ? C::NDT : 1];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        acc[dt] = f32x16{};
        if constexpr (CALIB) acc2[dt] = f32x16{};
    }
    float mx = -INFINITY, dsum = 0.f, dsum2 = 0.f;

    f32x4 kr[C::CPT], vr[C::CPT];
    auto load_tile = [&](int kb) {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            const int id = tid + i * C::NT;
            const int key = id / C::CPR, c = id - key * C::CPR;
            const int krow = kb * BLOCK + key;
            const bool ok = (C::CPT * C::NT == C::TOTAL || id < C::TOTAL) && krow < a.L && c * 4 < a.d;
            f32x4 zk = {0.f, 0.f, 0.f, 0.f}, zv = {0.f, 0.f, 0.f, 0.f};
            if (ok) {
                zk = *(const f32x4*)(Kp + (int64_t)krow * a.sl + c * 4);
                zv = *(const f32x4*)(Vp + (int64_t)krow * a.sl + c * 4);
            }
            kr[i] = zk;
            vr[i] = zv;
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            const int id = tid + i * C::NT;
            if (C::CPT * C::NT == C::TOTAL || id < C::TOTAL) {
                const int key = id / C::CPR, c = id - key * C::CPR;
                float* pk = sk + key * C::RSF + 4 * c;
                float* pv = sv + key * C::RSF + 4 * c;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pk[j] = kr[i][j];
                    pv[j] = vr[i][j];
                }
            }
        }
    };
    auto kb_of = [&](int it) -> int {
        if constexpr (CALIB) return it;
        else return scalar_load(ci, e0 + it);
    };

    if (nit > 0) {
        load_tile(kb_of(0));
        store_tile();
    }
    __syncthreads();

    for (int it = 0; it < nit; ++it) {
        const int kb = kb_of(it);
        if (it + 1 < nit) load_tile(kb_of(it + 1));

        f32x16 sacc[C::KT];
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt) {
            sacc[kt] = f32x16{};
            const float* kp = sk + (kt * 32 + n) * C::RSF + h;
#pragma unroll
            for (int s = 0; s < C::NS; ++s)
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kp[2 * s], qf[s], sacc[kt], 0, 0, 0);
        }
        if ((kb + 1) * BLOCK > a.L) {
#pragma unroll
            for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = kb * BLOCK + kt * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
                    if (key >= a.L) sacc[kt][j] = -INFINITY;
                }
        }

        float bm = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
            for (int j = 0; j < 16; ++j) bm = fmaxf(bm, sacc[kt][j]);
        bm = xhalf_max(bm);
        const float mnew = fmaxf(mx, bm);
        const float alpha = fast_exp2((mx - mnew) * a.c);
        mx = mnew;
        const float msc = mnew * a.c;
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float p = fast_exp2(fmaf(sacc[kt][j], a.c, -msc));
                sacc[kt][j] = p;
                psum += p;
            }
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            acc[dt] *= alpha;
            if constexpr (CALIB) acc2[dt] *= alpha;
        }
        dsum *= alpha;
        dsum2 *= alpha;
        bool in_window = true;
        if constexpr (CALIB) in_window = mask_byte(a.mask, mrow + kb) != 0;
        if (in_window) dsum += psum;
        else dsum2 += psum;

        auto pv = [&](f32x16 (&dst)[C::NDT]) {
#pragma unroll
            for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = kt * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
                    const float* vp = sv + key * C::RSF + n;
#pragma unroll
                    for (int dt = 0; dt < C::NDT; ++dt)
                        dst[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[32 * dt], sacc[kt][j], dst[dt], 0, 0, 0);
                }
        };
        if constexpr (CALIB) {
            if (in_window) pv(acc);
            else pv(acc2);
        } else {
            pv(acc);
        }

        __syncthreads();
        if (it + 1 < nit) store_tile();
        __syncthreads();
    }

    float* Op = (float*)a.O + base + (int64_t)row * a.sl;
    if constexpr (CALIB) {
        const float din = xhalf_sum(dsum), dout = xhalf_sum(dsum2);
        const float inv = 1.f / (din + dout);
        // window attention's normaliser for the difference residual (no kept key: the window output is 0)
        const float inv_in = din > 0.f ? 1.f / din : 0.f;
        const bool diff = a.residual != 0;
        if (row_ok && h == 0) a.rho_out[(int64_t)bh * a.L + row] = din * inv;
        float* Rp = (float*)a.R_out + base + (int64_t)row * a.sl;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int d0 = 32 * dt + 8 * bb + 4 * h;
                if (row_ok && d0 < a.d) {
                    f32x4 ov, rv;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float ai = acc[dt][4 * bb + r], ao = acc2[dt][4 * bb + r];
                        ov[r] = (ai + ao) * inv;
                        rv[r] = diff ? ov[r] - ai * inv_in : ao * inv;
                    }
                    *(f32x4*)(Op + d0) = ov;
                    *(f32x4*)(Rp + d0) = rv;
                }
            }
    } else {
        const float dtot = xhalf_sum(dsum);
        const float scale = nit > 0 ? fminf(1.f, rho_c * a.ramp) / dtot : 0.f;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int d0 = 32 * dt + 8 * bb + 4 * h;
                if (row_ok && d0 < a.d) {
                    f32x4 ov;
#pragma unroll
                    for (int r = 0; r < 4; ++r) ov[r] = fmaf(scale, acc[dt][4 * bb + r], rres[dt][bb][r]);
                    *(f32x4*)(Op + d0) = ov;
                }
            }
    }
}

template <int BLOCK, int DP, bool CALIB>
static hipError_t launch_one(AttnArgs a, hipStream_t s) {
    using C = F32Cfg<BLOCK, DP, CALIB>;
    const int64_t ntile = CALIB ? (a.L + C::QT - 1) / C::QT : a.nqb;
    const int64_t G = (int64_t)a.B * a.H * ntile;
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidValue;
    a.G = (int32_t)G;
    hipLaunchKernelGGL((attn_f32_kernel<BLOCK, DP, CALIB>), dim3((unsigned)G), dim3(C::NT), 0, s, a);
    return hipGetLastError();
}

template <bool CALIB>
static hipError_t dispatch(AttnArgs a, int block, hipStream_t s) {
    const int dp = pad_d(a.d);
#define RETTN_CASE(BL, D) \
    if (block == BL && dp == D) return launch_one<BL, D, CALIB>(a, s);
    RETTN_CASE(32, 32) RETTN_CASE(32, 64) RETTN_CASE(32, 96) RETTN_CASE(32, 128)
    RETTN_CASE(64, 32) RETTN_CASE(64, 64) RETTN_CASE(64, 96) RETTN_CASE(64, 128)
    RETTN_CASE(128, 32) RETTN_CASE(128, 64) RETTN_CASE(128, 96) RETTN_CASE(128, 128)
#undef RETTN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_calibrate_f32(AttnArgs a, int block, hipStream_t s) { return dispatch<true>(a, block, s); }
hipError_t launch_sparse_f32(AttnArgs a, int block, hipStream_t s) { return dispatch<false>(a, block, s); }

}  // namespace rettn
