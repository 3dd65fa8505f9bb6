// Calibration step of Re-ttention for bfloat16 (64- and 128-token blocks).
//
// A full-attention step that also records, per (batch, head, query token),
//     rho = D_in / D   and   R = N_out / D,
// where D_in, N_in are the softmax mass and P*V of the kept (in-window) key
// blocks and D_out, N_out those of the masked ones, all against one shared
// reference, and O = (N_in + N_out) / D, D = D_in + D_out  (Re-ttention
// summary page, "Approach"; review thread, replies to W1 of the first and
// second reviews: rho is the denominator ratio and the residual holds only the
// masked tokens' attention, normalised by the full denominator).
//
// Design for gfx950 (dense, matrix-core bound):
//   * a work-group of 4 waves (d <= 64; 8 for d = 96) covers 128 (256) query
//     rows, 32 per wave, and walks all key tiles of 64 keys, so each K/V tile
//     fetched from L2 feeds 128 (256) rows; at d <= 64 three work-groups share
//     a CU, which keeps three waves per SIMD issuing the softmax's vector work;
//   * K tiles arrive by coalesced direct-to-LDS loads; V tiles by coalesced
//     16-byte loads that are re-encoded to float16 once per work-group and
//     written to LDS; both double buffered, one barrier per tile;
//   * S^T = K Q^T and O^T += V^T P^T on 32x32x16 MFMA (bf16, then fp16), one
//     query row per lane; V^T fragments come from the transposing LDS read;
//   * the static mask bit of (query block, key block) is wave-uniform and
//     routes the tile's P*V and mass into the in-window or the masked
//     accumulators;
//   * softmax against a running reference per row: a tile is redone against
//     its true max only when a row's packed float16 sum is non-finite or
//     above 2^14 (then all four accumulators are rescaled).
#include "attn.h"
#include "common.h"

namespace rettn {

namespace {

constexpr uint32_t kOOB = 0x80000000u;   // a buffer offset past every record: reads as zero

__device__ __forceinline__ float dot2_f16(uint32_t a, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), one, acc, false);
}

}  // namespace

template <int DP>
struct CalCfg {
    // waves per work-group, 32 query rows each.  d <= 64: 4 waves in 168 registers, so three
    // work-groups share a CU (3 waves per SIMD; the vector work of the softmax issues faster with
    // more resident waves); d = 96 needs more registers: 8 waves, one work-group per CU.
    static constexpr int NW = DP <= 64 ? 4 : 8;
    static constexpr int WPS = DP <= 32 ? 4 : DP <= 64 ? 3 : 2;   // resident waves per SIMD to fit
    static constexpr int NT = NW * 64;
    static constexpr int QT = NW * 32;             // query rows per work-group
    static constexpr int NS = DP / 16;             // k-steps of S^T over d
    static constexpr int NDT = DP / 32;            // 32-row d tiles of O^T
    static constexpr int RS = DP <= 64 ? 64 : 128; // LDS row stride (elements)
    static constexpr int CPR = RS / 8;             // 16-byte chunks per LDS row
    static constexpr int TILE = 64 * RS;           // elements per 64-key tile
    static constexpr int KL = TILE / 512 / NW;     // 1 KiB K loads per wave per tile
    static constexpr int VC = TILE / 8 / NT;       // 16-byte V chunks per thread per tile
    // d = 128: the Q fragments (32 registers) would leave no room for the two accumulator sets at
    // 2 waves per SIMD, so the group's Q rows sit in LDS (swizzled like K) and are read per tile
    static constexpr bool QLDS = DP > 96;
    static constexpr int QSLOT = QLDS ? QT * RS : 8;
};

template <int BLOCK, int DP>
__global__ void __launch_bounds__(CalCfg<DP>::NT, CalCfg<DP>::WPS) calib_kernel(const AttnArgs a) {
    using C = CalCfg<DP>;
    // [buffer][K | V][64 keys][RS]
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * 2 * C::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t qlds[C::QSLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, n = lane & 31;

    const int ntile = (a.L + C::QT - 1) / C::QT;
    const int work = xcd_remap(blockIdx.x, a.G);
    const int bh = work / ntile;
    const int tile = work - bh * ntile;
    const int bi = bh / a.H, hi = bh - bi * a.H;
    const int64_t base = (int64_t)bi * a.sb + (int64_t)hi * a.sh;
    const int q0 = tile * C::QT + wave * 32;
    const int qb = min(q0 / BLOCK, a.nqb - 1);     // a wave wholly past L reads the last mask row, stores nothing
    const int64_t mrow = ((int64_t)(bh % a.slice_mod) * a.nqb + qb) * a.nkb;   // this wave's mask row
    const int row = q0 + n;
    const bool row_ok = row < a.L;
    const uint32_t row_bytes = (uint32_t)a.sl * 2u;
    const uint32_t nrec = (uint32_t)(a.L - 1) * row_bytes + (uint32_t)a.d * 2u;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.Q + base), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.K + base), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.V + base), 0, nrec, 0x00020000);

    // B operand of S^T = K Q^T: Q[row][16 s + 8 h .. +7] (read once per wave)
    u32x4 qf[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        const int d0 = 16 * s + 8 * h;
        const uint32_t off = d0 < a.d ? (uint32_t)row * row_bytes + 2u * d0 : kOOB;
        qf[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
    // this wave's rows of the Q slot: row 32 wave + n, logical chunk 2 s + h at chunk (2 s + h) ^ swz(n)
    uint32_t qoff = (uint32_t)(wave * 32 + n) * C::RS;
    if constexpr (C::QLDS) {
#pragma unroll
        for (int s = 0; s < C::NS; ++s) *(u32x4*)(qlds + qoff + (((2 * s + h) ^ swz(n)) << 3)) = qf[s];
    }

    // Tile staging.  K: direct-to-LDS, wave w fills 1 KiB pieces w, w + NW, ...; lane -> (row, physical chunk).
    // V: thread t holds 16-byte chunks t, t + NT, ... in registers until they are re-encoded and stored.
    // (plain expressions only inside these lambdas: see the note in sparse64.hip)
    const int nkt = (a.L + 63) / 64;
    u32x4 vreg[C::VC];
    auto issue_k = [&](int kt, int buf) {
#pragma unroll
        for (int j = 0; j < C::KL; ++j) {
            const int piece = wave + j * C::NW;                  // 1 KiB piece of the tile
            const int r = piece * (64 / C::CPR) + lane / C::CPR; // key row within the tile
            const int c = (lane % C::CPR) ^ swz(r);              // logical chunk loaded into this slot
            const uint32_t off = c * 8 < a.d ? (uint32_t)(kt * 64 + r) * row_bytes + 16u * c : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (__attribute__((address_space(3))) void*)(lds + buf * 2 * C::TILE + piece * 512), 16, off, 0, 0, 0);
        }
    };
    auto issue_v = [&](int kt) {
#pragma unroll
        for (int j = 0; j < C::VC; ++j) {
            const int id = tid + j * C::NT;
            const int r = id / C::CPR;
            const int c = (id % C::CPR) ^ swz(r);
            const uint32_t off = c * 8 < a.d ? (uint32_t)(kt * 64 + r) * row_bytes + 16u * c : kOOB;
            vreg[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
        }
    };
    auto store_v = [&](int buf) {
#pragma unroll
        for (int j = 0; j < C::VC; ++j) {
            const int id = tid + j * C::NT;
            *(u32x4*)(lds + buf * 2 * C::TILE + C::TILE + id * 8) = bf16x8_to_f16x8(vreg[j]);
        }
    };

    f32x16 acc_in[C::NDT], acc_out[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) acc_in[dt] = acc_out[dt] = f32x16{};
    float mref = -INFINITY, d_in = 0.f, d_out = 0.f;

    const int swn = swz(n);
    const int s16 = lane & 15, g = lane >> 4;
    const int fv = ((s16 >> 2) << 1) | h;
    const int vrow = (4 * h + (s16 >> 2)) * C::RS;

    issue_k(0, 0);
    issue_v(0);
    store_v(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();

    for (int kt64 = 0; kt64 < nkt; ++kt64) {
        const int buf = kt64 & 1;
        const bool more = kt64 + 1 < nkt;
        if (more) {
            issue_k(kt64 + 1, buf ^ 1);
            issue_v(kt64 + 1);
        }
        const uint16_t* ks = lds + buf * 2 * C::TILE;
        const uint16_t* vs = ks + C::TILE;
        if constexpr (C::QLDS) asm volatile("" : "+v"(qoff));   // re-read Q every tile, not kept in registers

        // S^T for the tile's two 32-key halves
        f32x16 sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sacc[kt] = f32x16{};
            const uint16_t* kr = ks + (kt * 32 + n) * C::RS;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const u32x4 w = *(const u32x4*)(kr + (((2 * s + h) ^ swn) << 3));
                u32x4 qv;
                if constexpr (C::QLDS) qv = *(const u32x4*)(qlds + qoff + (((2 * s + h) ^ swn) << 3));
                else qv = qf[s];
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                                   __builtin_bit_cast(bf16x8, qv), sacc[kt], 0, 0, 0);
            }
        }
        if (__builtin_expect((kt64 + 1) * 64 > a.L, 0)) {
            int lim = a.L - kt64 * 64 - 4 * h;
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (kt * 32 + 8 * (j >> 2) + (j & 3) >= lim) sacc[kt][j] = -INFINITY;
        }

        u32x4 pf[4];
        float bsum;
        auto make_p = [&]() {
            float sum = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x16& sp = sacc[t >> 1];
                const int o8 = 8 * (t & 1);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float p0 = fast_exp2(fmaf(sp[o8 + 2 * w], a.c, -mref));
                    const float p1 = fast_exp2(fmaf(sp[o8 + 2 * w + 1], a.c, -mref));
                    pf[t][w] = pack_f16(p0, p1);
                    sum = dot2_f16(pf[t][w], sum);
                }
            }
            bsum = sum;
        };
        make_p();
        if (__builtin_amdgcn_ballot_w64(!(bsum <= 16384.f)) != 0) {
            float bm = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) bm = fmaxf(bm, sacc[kt][j]);
            bm = xhalf_max(bm) * a.c;
            const float mnew = fmaxf(mref, bm);
            const float alpha = fast_exp2(mref - mnew);
            mref = mnew;
            d_in *= alpha;
            d_out *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
                acc_in[dt] *= alpha;
                acc_out[dt] *= alpha;
            }
            make_p();
        }

        const bool in_window = mask_byte(a.mask, mrow + (kt64 * 64) / BLOCK) != 0;
        auto pv = [&](f32x16 (&dst)[C::NDT]) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint16_t* vb = vs + vrow + 16 * t * C::RS;
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt) {
                    const int c = 4 * dt + 2 * (g & 1) + ((s16 & 3) >> 1);
                    const uint16_t* p = vb + ((c ^ fv) << 3) + ((s16 & 1) << 2);
                    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)p);
                    const i16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p + 8 * C::RS));
                    const u32x2 w1 = __builtin_bit_cast(u32x2, r1), w2 = __builtin_bit_cast(u32x2, r2);
                    const u32x4 vw = {w1[0], w1[1], w2[0], w2[1]};
                    dst[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vw),
                                                                     __builtin_bit_cast(f16x8, pf[t]), dst[dt], 0, 0, 0);
                }
            }
        };
        if (in_window) {
            d_in += bsum;
            pv(acc_in);
        } else {
            d_out += bsum;
            pv(acc_out);
        }

        if (more) store_v(buf ^ 1);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // Epilogue.  Lane (n, h) owns d = 32 dt + 8 bb + 4 h + r of row `row`.
    const float din = xhalf_sum(d_in), dout = xhalf_sum(d_out);
    const float inv = 1.f / (din + dout);
    // window attention's normaliser for the difference residual (no kept key: the window output is 0)
    const float inv_in = din > 0.f ? 1.f / din : 0.f;
    const bool diff = a.residual != 0;
    if (row_ok && h == 0) a.rho_out[(int64_t)bh * a.L + row] = din * inv;
    uint16_t* Op = (uint16_t*)a.O + base + (int64_t)row * a.sl;
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
                    const float ai = acc_in[dt][4 * bb + r], ao = acc_out[dt][4 * bb + r];
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
}

template <int BLOCK, int DP>
static hipError_t launch(AttnArgs a, hipStream_t s) {
    using C = CalCfg<DP>;
    const int64_t ntile = (a.L + C::QT - 1) / C::QT;
    const int64_t G = (int64_t)a.B * a.H * ntile;
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidValue;
    a.G = (int32_t)G;
    hipLaunchKernelGGL((calib_kernel<BLOCK, DP>), dim3((unsigned)G), dim3(C::NT), 0, s, a);
    return hipGetLastError();
}

bool calib_supported(const AttnArgs& a, int block) {
    // every d up to 128: two accumulator sets fit at 2 waves per SIMD (Q in LDS at d = 128)
    const int64_t slice = ((int64_t)a.L - 1) * a.sl * 2 + (int64_t)a.d * 2;
    return (block == 64 || block == 128) && a.d <= 128 && slice < ((int64_t)1 << 31);
}

hipError_t launch_calib(AttnArgs a, int block, hipStream_t s) {
    const int dp = pad_d(a.d);
#define RETTN_CASE(BL, D) \
    if (block == BL && dp == D) return launch<BL, D>(a, s);
    RETTN_CASE(64, 32) RETTN_CASE(64, 64) RETTN_CASE(64, 96) RETTN_CASE(64, 128)
    RETTN_CASE(128, 32) RETTN_CASE(128, 64) RETTN_CASE(128, 96) RETTN_CASE(128, 128)
#undef RETTN_CASE
    return hipErrorInvalidValue;
}

}  // namespace rettn
