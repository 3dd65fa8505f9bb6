// bfloat16 attention kernels for gfx950: the full-attention calibration step
// and the block-sparse step of Re-ttention.
//
// Both are flash-style single-pass kernels.  Per work-group: a tile of query
// rows (32 per wave) held in registers; the key blocks it attends to are
// staged one at a time into LDS (K and V, BLOCK keys each) and contracted on
// the matrix cores with v_mfma_f32_32x32x16 in the transposed orientation
//     S^T = K Q^T      (A = K fragment from LDS, B = Q^T fragment in registers)
//     O^T += V^T P^T   (A = V^T via the gfx950 transposing LDS read, B = P^T)
// so that every lane owns exactly one query row: the row max, the row sums
// and the epilogue scale are per-lane scalars, and the lane pair (l, l^32)
// that splits a row's keys is joined with one v_permlane32_swap.
//
// Calibration (Re-ttention summary page, "Approach"; review thread, replies
// to W1 of the first and second reviews): every key block is visited; the
// static mask bit of (query block, key block) routes the block's softmax
// mass and its P*V product into the in-window or the masked accumulator,
// under one shared running max, so
//     O = (N_in + N_out) / D,  rho = D_in / D,  R = N_out / D,  D = D_in + D_out.
// In both kernels P*V runs in float16 (P and V both; V is re-encoded exactly
// when it is staged): rounding the probabilities to bfloat16 alone costs about
// 1.3e-3 relative L1 on a dense row, which with the output's own bfloat16
// rounding exceeds a 2e-3 budget; float16 rounds P 8x finer.
//
// Sparse step (same sources; ramp-up: review thread, answer to W1 of the
// fourth review): only the kept key blocks of the CSR row are visited, with
// a plain online softmax, and the epilogue fuses the statistical reshape and
// the residual add:  O' = min(1, rho * ramp) * acc / D' + R.
#include "attn.h"
#include "common.h"

namespace rettn {

template <int BLOCK, int DP, bool CALIB>
struct Bf16Cfg {
    static constexpr int NW = CALIB ? 4 : BLOCK / 32;   // waves per work-group, 32 query rows each
    static constexpr int NT = NW * 64;
    static constexpr int QT = NW * 32;                  // query rows per work-group
    static constexpr int NS = DP / 16;                  // k-steps of S^T = K Q^T over d
    static constexpr int NDT = DP / 32;                 // 32-wide d tiles of O^T
    static constexpr int KT = BLOCK / 32;               // 32-key tiles per key block
    static constexpr int NKC = BLOCK / 16;              // 16-key k-steps of O^T
    static constexpr int RS = DP <= 64 ? 64 : 128;      // LDS row stride in elements
    static constexpr int CPR = DP / 8;                  // staged 16-byte chunks per key row
    static constexpr int TOTAL = BLOCK * CPR;           // staged chunks per tensor tile
    static constexpr int CPT = (TOTAL + NT - 1) / NT;   // staged chunks per thread
};

template <int BLOCK, int DP, bool CALIB>
__global__ void __launch_bounds__((Bf16Cfg<BLOCK, DP, CALIB>::NT))
attn_bf16_kernel(const AttnArgs a) {
    using C = Bf16Cfg<BLOCK, DP, CALIB>;
    __shared__ __attribute__((aligned(16))) uint16_t sk[BLOCK * C::RS];
    __shared__ __attribute__((aligned(16))) uint16_t sv[BLOCK * C::RS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;      // which half of the keys of a 32-key tile this lane holds
    const int n = lane & 31;      // query row within the wave

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
    // query block of this wave (wave-uniform); a calibration wave wholly past L
    // reads the last mask row and stores nothing
    const int qb = min(q0 / BLOCK, a.nqb - 1);
    const int row = q0 + n;
    const bool row_ok = row < a.L;

    const uint16_t* Qp = (const uint16_t*)a.Q + base;
    const uint16_t* Kp = (const uint16_t*)a.K + base;
    const uint16_t* Vp = (const uint16_t*)a.V + base;

    // B operand of S^T = K Q^T: lane holds Q[row][16 s + 8 h .. +7]; zero past d.
    bf16x8 qf[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        const int d0 = 16 * s + 8 * h;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (row_ok && d0 < a.d) w = *(const u32x4*)(Qp + (int64_t)row * a.sl + d0);
        qf[s] = __builtin_bit_cast(bf16x8, w);
    }

    // Sparse step: cached rho and R of this row are read up front.
    float rho_c = 0.f;
    u32x2 rres[C::NDT][4];
    if constexpr (!CALIB) {
        if (row_ok) rho_c = a.rho_in[(int64_t)bh * a.L + row];
        const uint16_t* Rp = (const uint16_t*)a.R_in + base + (int64_t)row * a.sl;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int d0 = 32 * dt + 8 * bb + 4 * h;
                u32x2 w = {0u, 0u};
                if (row_ok && d0 < a.d) w = *(const u32x2*)(Rp + d0);
                rres[dt][bb] = w;
            }
    }

    // Key blocks to visit.
    int e0 = 0, nit;
    if constexpr (CALIB) {
        nit = a.nkb;
    } else {
        e0 = scalar_load(rp, qb);
        nit = scalar_load(rp, qb + 1) - e0;
    }
    const int64_t mrow = ((int64_t)sl * a.nqb + qb) * a.nkb;   // this wave's mask row (calibration)

    f32x16 acc[C::NDT];
    f32x16 acc2[CALIB ? C::NDT : 1];   // calibration: masked-key accumulator
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        acc[dt] = f32x16{};
        if constexpr (CALIB) acc2[dt] = f32x16{};
    }
    float mx = -INFINITY, dsum = 0.f, dsum2 = 0.f;

    // Staging: global -> registers -> swizzled LDS tile.
    u32x4 kr[C::CPT], vr[C::CPT];
    auto load_tile = [&](int kb) {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            const int id = tid + i * C::NT;
            const int key = id / C::CPR, c = id - key * C::CPR;
            const int krow = kb * BLOCK + key;
            const bool ok = (C::CPT * C::NT == C::TOTAL || id < C::TOTAL) && krow < a.L && c * 8 < a.d;
            u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
            if (ok) {
                zk = *(const u32x4*)(Kp + (int64_t)krow * a.sl + c * 8);
                zv = *(const u32x4*)(Vp + (int64_t)krow * a.sl + c * 8);
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
                const int off = key * C::RS + ((c ^ swz(key)) << 3);
                *(u32x4*)(sk + off) = kr[i];
                *(u32x4*)(sv + off) = bf16x8_to_f16x8(vr[i]);
            }
        }
    };
    auto kb_of = [&](int it) -> int {
        if constexpr (CALIB) return it;
        else return scalar_load(ci, e0 + it);
    };

    // Lane-constant parts of the LDS fragment addresses.
    const int swn = swz(n);
    const int s16 = lane & 15, g = lane >> 4;
    const int fv = ((s16 >> 2) << 1) | h;                 // swizzle of the 4 keys a tr-read group touches
    const int vrow = (4 * h + (s16 >> 2)) * C::RS;        // key row of the first tr read (t = 0)

    if (nit > 0) {
        load_tile(kb_of(0));
        store_tile();
    }
    __syncthreads();

    for (int it = 0; it < nit; ++it) {
        const int kb = kb_of(it);
        if (it + 1 < nit) load_tile(kb_of(it + 1));

        // S^T = K Q^T for this key block: KT tiles of 32 keys x 32 query rows.
        f32x16 sacc[C::KT];
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt) {
            sacc[kt] = f32x16{};
            const uint16_t* krow_p = sk + (kt * 32 + n) * C::RS;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const u32x4 w = *(const u32x4*)(krow_p + (((2 * s + h) ^ swn) << 3));
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), qf[s],
                                                                   sacc[kt], 0, 0, 0);
            }
        }
        // Keys past the end of the sequence do not exist.
        if ((kb + 1) * BLOCK > a.L) {
#pragma unroll
            for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = kb * BLOCK + kt * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
                    if (key >= a.L) sacc[kt][j] = -INFINITY;
                }
        }

        // Online softmax with one running max per row.
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

        // O^T += V^T P^T over the block's 16-key chunks, into `dst`.
        auto pv = [&](f32x16 (&dst)[C::NDT]) {
#pragma unroll
            for (int t = 0; t < C::NKC; ++t) {
                const f32x16& sp = sacc[t >> 1];
                const int o8 = 8 * (t & 1);
                u32x4 pw;
                pw[0] = pack_f16(sp[o8 + 0], sp[o8 + 1]);
                pw[1] = pack_f16(sp[o8 + 2], sp[o8 + 3]);
                pw[2] = pack_f16(sp[o8 + 4], sp[o8 + 5]);
                pw[3] = pack_f16(sp[o8 + 6], sp[o8 + 7]);
                const uint16_t* vbase = sv + vrow + 16 * t * C::RS;
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt) {
                    const int c = 4 * dt + 2 * (g & 1) + ((s16 & 3) >> 1);
                    const int off = ((c ^ fv) << 3) + ((s16 & 1) << 2);
                    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vbase + off));
                    const i16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vbase + off + 8 * C::RS));
                    u32x4 vw;
                    vw[0] = (uint32_t)(uint16_t)r1[0] | ((uint32_t)(uint16_t)r1[1] << 16);
                    vw[1] = (uint32_t)(uint16_t)r1[2] | ((uint32_t)(uint16_t)r1[3] << 16);
                    vw[2] = (uint32_t)(uint16_t)r2[0] | ((uint32_t)(uint16_t)r2[1] << 16);
                    vw[3] = (uint32_t)(uint16_t)r2[2] | ((uint32_t)(uint16_t)r2[3] << 16);
                    dst[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vw),
                                                                     __builtin_bit_cast(f16x8, pw), dst[dt], 0, 0, 0);
                }
            }
        };
        if constexpr (CALIB) {
            if (in_window) pv(acc);
            else pv(acc2);
        } else {
            pv(acc);
        }

        __syncthreads();            // every wave is done with this tile
        if (it + 1 < nit) store_tile();
        __syncthreads();            // the next tile is visible
    }

    // Epilogue.  Lane (n, h) owns d = 32 dt + 8 bb + 4 h + r, r = 0..3, of row `row`.
    uint16_t* Op = (uint16_t*)a.O + base + (int64_t)row * a.sl;
    if constexpr (CALIB) {
        const float din = xhalf_sum(dsum), dout = xhalf_sum(dsum2);
        const float inv = 1.f / (din + dout);
        // window attention's normaliser for the difference residual (no kept key: the window output is 0)
        const float inv_in = din > 0.f ? 1.f / din : 0.f;
        const bool diff = a.residual != 0;
        if (row_ok && h == 0) a.rho_out[(int64_t)bh * a.L + row] = din * inv;
        uint16_t* Rp = (uint16_t*)a.R_out + base + (int64_t)row * a.sl;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int d0 = 32 * dt + 8 * bb + 4 * h;
                if (row_ok && d0 < a.d) {
                    float ov[4], rv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float ai = acc[dt][4 * bb + r], ao = acc2[dt][4 * bb + r];
                        ov[r] = (ai + ao) * inv;
                        rv[r] = diff ? ov[r] - ai * inv_in : ao * inv;
                    }
                    u32x2 ow, rw;
                    ow[0] = pack_bf16(ov[0], ov[1]);
                    ow[1] = pack_bf16(ov[2], ov[3]);
                    rw[0] = pack_bf16(rv[0], rv[1]);
                    rw[1] = pack_bf16(rv[2], rv[3]);
                    *(u32x2*)(Op + d0) = ow;
                    *(u32x2*)(Rp + d0) = rw;
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
                    const int j = 4 * bb;
                    const u32x2 rw = rres[dt][bb];
                    u32x2 ow;
                    ow[0] = pack_bf16(fmaf(scale, acc[dt][j], bf16_lo(rw[0])), fmaf(scale, acc[dt][j + 1], bf16_hi(rw[0])));
                    ow[1] = pack_bf16(fmaf(scale, acc[dt][j + 2], bf16_lo(rw[1])), fmaf(scale, acc[dt][j + 3], bf16_hi(rw[1])));
                    *(u32x2*)(Op + d0) = ow;
                }
            }
    }
}

template <int BLOCK, int DP, bool CALIB>
static hipError_t launch_one(AttnArgs a, hipStream_t s) {
    using C = Bf16Cfg<BLOCK, DP, CALIB>;
    const int64_t ntile = CALIB ? (a.L + C::QT - 1) / C::QT : a.nqb;
    const int64_t G = (int64_t)a.B * a.H * ntile;
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidValue;
    a.G = (int32_t)G;
    hipLaunchKernelGGL((attn_bf16_kernel<BLOCK, DP, CALIB>), dim3((unsigned)G), dim3(C::NT), 0, s, a);
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

hipError_t launch_calibrate_bf16(AttnArgs a, int block, void* v16, void* part, hipStream_t s) {
    if (calib_supported(a, block)) return launch_calib(a, block, v16, part, s);
    return dispatch<true>(a, block, s);
}
hipError_t launch_sparse_bf16(AttnArgs a, int block, void* v16, hipStream_t s) {
    if (sparse64_supported(a, block)) return launch_sparse64(a, s);
    if (sparse_wg_supported(a, block)) return launch_sparse_wg(a, block, v16, s);
    return dispatch<false>(a, block, s);
}

}  // namespace rettn
