// Sparse step of Re-ttention for bfloat16 with 128-token blocks (any d <= 128)
// and 64-token blocks with 64 < d <= 128.
//
// The step (Re-ttention summary page, "Approach"; review thread, replies to
// W1 of the first and third reviews; ramp-up: answer to W1 of the fourth
// review) attends each query block only to its kept key blocks, then applies
// the statistical reshape and the residual:
//     O' = min(1, rho * (1 + lambda step)) * softmax_W(s) V_W + R.
//
// Design for gfx950: one work-group of 4 waves per 128-row query block, 32
// rows per wave, walks the block's CSR row 64 keys at a time.  K tiles arrive
// by coalesced direct-to-LDS loads; V tiles by coalesced 16-byte loads that are
// re-encoded to float16 once per work-group, or, when many query blocks keep
// each key block and the caller supplies a workspace, direct-to-LDS from a
// float16 copy of V made by one pass over it; both double buffered, one barrier
// per tile.  One accumulator set and Q in registers keep a wave at about 200
// registers, so two work-groups share a CU (2 waves per SIMD, 128 KiB of LDS):
// a SIMD issues the softmax's vector work faster the more waves it holds.  The
// products, the swizzled LDS tiles, the float16 P*V and the running-reference
// softmax are those of the calibration kernel.  Also used for 64-token blocks
// with d > 64 (2-wave groups), where it beats the general kernel; at d <= 64
// the one-wave-per-query-block sparse64 kernel is faster (with ~9 kept blocks
// per query block, the per-tile barrier and the per-lane prologue and epilogue
// weigh more than the extra resident waves).  At 64-token blocks and d > 64
// the group keeps a single K and V slot (32 KiB instead of 64) and is compiled
// for two waves per SIMD, so four groups share a CU: with two or four kept
// blocks per row there is little to double buffer, and the doubled residency
// pays more than the exposed K transfer of each later tile.  For d > 64 each
// lane fetches the residual of its epilogue elements together with Q, so that
// the epilogue does not wait for HBM at the end of such short work-groups.
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

template <int BLOCK_, int DP>
struct SwgCfg {
    static constexpr int BLOCK = BLOCK_;
    static constexpr int TPB = BLOCK / 64;         // 64-key tiles per key block
    static constexpr int NW = BLOCK / 32;          // waves per work-group, 32 query rows each
    static constexpr int NT = NW * 64;
    static constexpr int NS = DP / 16;             // k-steps of S^T over d
    static constexpr int NDT = DP / 32;            // 32-row d tiles of O^T
    static constexpr int RS = DP <= 64 ? 64 : 128; // LDS row stride (elements)
    static constexpr int CPR = RS / 8;             // 16-byte chunks per LDS row
    static constexpr int TILE = 64 * RS;           // elements per 64-key tile
    static constexpr int KL = TILE / 512 / NW;     // 1 KiB K loads per wave per tile
    static constexpr int VC = TILE / 8 / NT;       // 16-byte V chunks per thread per tile
    // 64-token blocks at d > 64: a 2-wave group with one K and one V slot (32 KiB), so that four
    // groups share a CU (two waves per SIMD); the next tile's V still comes ahead into registers,
    // its K after the group has read the current one.  Otherwise both slots are double buffered.
    static constexpr bool SB = BLOCK == 64 && DP >= 96;
    static constexpr int NBUF = SB ? 1 : 2;
    static constexpr int WPE = SB ? 2 : 1;          // resident waves per SIMD to compile for (at least)
};

template <int BLOCK, int DP, bool V16>
__global__ void __launch_bounds__((SwgCfg<BLOCK, DP>::NT), 2) __attribute__((amdgpu_waves_per_eu(SwgCfg<BLOCK, DP>::WPE)))
sparse_wg_kernel(const AttnArgs a) {
    using C = SwgCfg<BLOCK, DP>;
    static_assert(!(V16 && C::SB), "float16 V tiles are streamed only into double-buffered slots");
    // [buffer][K | V][64 keys][RS]
    __shared__ __attribute__((aligned(1024))) uint16_t lds[C::NBUF * 2 * C::TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, n = lane & 31;

    const int work = xcd_remap(blockIdx.x, a.G);
    const int bh = work / a.nqb;
    const int qb = work - bh * a.nqb;
    const int bi = bh / a.H, hi = bh - bi * a.H;
    const int sl = bh % a.slice_mod;                        // this slice's CSR
    const int32_t* rp = a.row_ptr + (int64_t)sl * (a.nqb + 1);
    const int32_t* ci = a.col_idx + (int64_t)sl * a.col_stride;
    const int64_t base = (int64_t)bi * a.sb + (int64_t)hi * a.sh;
    const int row = qb * C::BLOCK + wave * 32 + n;
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
    const float rho_c = row_ok ? a.rho_in[(int64_t)bh * a.L + row] : 0.f;
    // The residual of this lane's epilogue elements.  For d > 64 it is fetched here, so that its
    // latency hides behind the tiles (the registers it holds leave the occupancy unchanged there);
    // for d <= 64 the epilogue reads it, which keeps one more work-group per CU.
    constexpr bool R_EARLY = DP >= 96;
    u32x2 rreg[R_EARLY ? C::NDT : 1][4];
    if constexpr (R_EARLY) {
        const __amdgpu_buffer_rsrc_t rr =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.R_in + base), 0, nrec, 0x00020000);
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int d0 = 32 * dt + 8 * bb + 4 * h;
                const uint32_t off = d0 < a.d ? (uint32_t)row * row_bytes + 2u * d0 : kOOB;
                rreg[dt][bb] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, 0));
            }
    }

    // 64-key tiles: tile t is part t % TPB of kept block t / TPB of this query block's CSR row
    const int e0 = scalar_load(rp, qb);
    const int ntiles = C::TPB * (scalar_load(rp, qb + 1) - e0);
    auto key0 = [&](int t) -> int { return scalar_load(ci, e0 + t / C::TPB) * C::BLOCK + 64 * (t % C::TPB); };

    // Tile staging.  K: direct-to-LDS, wave w fills 1 KiB pieces w, w + NW, ...; lane -> (row, physical chunk).
    // V, bfloat16: thread t holds 16-byte chunks t, t + NT, ... in registers until they are re-encoded and
    // stored.  V16 (V already converted to float16 by one pass over it): direct-to-LDS like K.
    // A lane's byte offset within a tile is the same for every tile (a padded chunk takes an offset
    // past every record); the tile's row offset k0 * row_bytes rides in the scalar offset.  (Each
    // offset array is declared right before the lambda that reads it: other placements kept the
    // host compiler from emitting the launch stubs.)
    u32x4 vreg[V16 ? 1 : C::VC];
    uint32_t k_off[C::KL];
#pragma unroll
    for (int j = 0; j < C::KL; ++j) {
        const int piece = wave + j * C::NW;
        const int r = piece * (64 / C::CPR) + lane / C::CPR;
        const int c = (lane % C::CPR) ^ swz(r);
        k_off[j] = c * 8 < a.d ? (uint32_t)r * row_bytes + 16u * c : kOOB;
    }
    auto issue_k = [&](int k0, int buf) {
#pragma unroll
        for (int j = 0; j < C::KL; ++j) {
            const int piece = wave + j * C::NW;
            const uint32_t off = k_off[j];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (__attribute__((address_space(3))) void*)(lds + buf * 2 * C::TILE + piece * 512), 16, off,
                (uint32_t)k0 * row_bytes, 0, 0);
        }
    };
    uint32_t v_off[V16 ? 1 : C::VC];
#pragma unroll
    for (int j = 0; j < (V16 ? 0 : C::VC); ++j) {
        const int id = tid + j * C::NT;
        const int r = id / C::CPR;
        const int c = (id % C::CPR) ^ swz(r);
        v_off[j] = c * 8 < a.d ? (uint32_t)r * row_bytes + 16u * c : kOOB;
    }
    // V tile at key k0 towards slot buf (bfloat16: into registers now, into the slot at store_v)
    auto issue_v = [&](int k0, int buf) {
        if constexpr (V16) {
#pragma unroll
            for (int j = 0; j < C::KL; ++j) {
                const int piece = wave + j * C::NW;
                const uint32_t off = k_off[j];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rv, (__attribute__((address_space(3))) void*)(lds + buf * 2 * C::TILE + C::TILE + piece * 512), 16,
                    off, (uint32_t)k0 * row_bytes, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < C::VC; ++j) {
                const uint32_t off = v_off[j];
                vreg[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, (uint32_t)k0 * row_bytes, 0));
            }
        }
    };
    auto store_v = [&](int buf) {
        if constexpr (!V16) {
#pragma unroll
            for (int j = 0; j < C::VC; ++j) {
                const int id = tid + j * C::NT;
                *(u32x4*)(lds + buf * 2 * C::TILE + C::TILE + id * 8) = bf16x8_to_f16x8(vreg[j]);
            }
        }
    };

    f32x16 acc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) acc[dt] = f32x16{};
    float mref = -INFINITY, dsum = 0.f;

    const int swn = swz(n);
    const int s16 = lane & 15, g = lane >> 4;
    const int fv = ((s16 >> 2) << 1) | h;
    const int vrow = (4 * h + (s16 >> 2)) * C::RS;

    int kcur = 0;
    if (ntiles > 0) {
        kcur = key0(0);
        issue_k(kcur, 0);
        issue_v(kcur, 0);
        store_v(0);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
    }

    for (int t = 0; t < ntiles; ++t) {
        const int buf = C::SB ? 0 : t & 1;
        const bool more = t + 1 < ntiles;
        const int knext = more ? key0(t + 1) : 0;
        if (more) {
            if constexpr (!C::SB) issue_k(knext, buf ^ 1);
            issue_v(knext, buf ^ 1);                // (single slot: into registers, stored after the barrier)
        }
        const uint16_t* ks = lds + buf * 2 * C::TILE;
        const uint16_t* vs = ks + C::TILE;

        // S^T for the tile's two 32-key halves
        f32x16 sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sacc[kt] = f32x16{};
            const uint16_t* kr = ks + (kt * 32 + n) * C::RS;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const u32x4 w = *(const u32x4*)(kr + (((2 * s + h) ^ swn) << 3));
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                                   __builtin_bit_cast(bf16x8, qf[s]), sacc[kt], 0, 0, 0);
            }
        }
        // keys at or past L (the tail of the sequence's last block) do not exist
        if (__builtin_expect(kcur + 64 > a.L, 0)) {
            int lim = a.L - kcur - 4 * h;
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (kt * 32 + 8 * (j >> 2) + (j & 3) >= lim) sacc[kt][j] = -INFINITY;
        }
        auto row_max = [&]() -> float {
            float bm = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) bm = fmaxf(bm, sacc[kt][j]);
            return xhalf_max(bm) * a.c;
        };
        // the first tile holds at least one key < L (its block starts below L): anchor there
        if (t == 0) mref = row_max();

        u32x4 pf[4];
        float bsum;
        auto make_p = [&]() {
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x16& sp = sacc[q >> 1];
                const int o8 = 8 * (q & 1);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float p0 = fast_exp2(fmaf(sp[o8 + 2 * w], a.c, -mref));
                    const float p1 = fast_exp2(fmaf(sp[o8 + 2 * w + 1], a.c, -mref));
                    pf[q][w] = pack_f16(p0, p1);
                    sum = dot2_f16(pf[q][w], sum);
                }
            }
            bsum = sum;
        };
        make_p();
        if (__builtin_amdgcn_ballot_w64(!(bsum <= 16384.f)) != 0) {
            const float mnew = fmaxf(mref, row_max());
            const float alpha = fast_exp2(mref - mnew);
            mref = mnew;
            dsum *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) acc[dt] *= alpha;
            make_p();
        }
        dsum += bsum;

#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint16_t* vb = vs + vrow + 16 * q * C::RS;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
                const int c = 4 * dt + 2 * (g & 1) + ((s16 & 3) >> 1);
                const uint16_t* p = vb + ((c ^ fv) << 3) + ((s16 & 1) << 2);
                const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)p);
                const i16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p + 8 * C::RS));
                const u32x2 w1 = __builtin_bit_cast(u32x2, r1), w2 = __builtin_bit_cast(u32x2, r2);
                const u32x4 vw = {w1[0], w1[1], w2[0], w2[1]};
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vw),
                                                                 __builtin_bit_cast(f16x8, pf[q]), acc[dt], 0, 0, 0);
            }
        }

        if constexpr (C::SB) {
            if (more) {
                // every wave has read this tile's K and V: refill the slots
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __syncthreads();
                issue_k(knext, 0);
                store_v(0);
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                __syncthreads();
            }
        } else {
            if (more) store_v(buf ^ 1);
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            __syncthreads();
        }
        kcur = knext;
    }

    // Epilogue.  Lane (n, h) owns d = 32 dt + 8 bb + 4 h + r of row `row`:
    // O' = min(1, rho * ramp) * acc / D' + R  (O' = R for a row with no kept block).
    const float dtot = xhalf_sum(dsum);
    const float scale = ntiles > 0 ? fminf(1.f, rho_c * a.ramp) / dtot : 0.f;
    const uint16_t* Rp = (const uint16_t*)a.R_in + base + (int64_t)row * a.sl;
    uint16_t* Op = (uint16_t*)a.O + base + (int64_t)row * a.sl;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int d0 = 32 * dt + 8 * bb + 4 * h;
            if (row_ok && d0 < a.d) {
                u32x2 rw;
                if constexpr (R_EARLY) rw = rreg[dt][bb];
                else rw = *(const u32x2*)(Rp + d0);
                const int j = 4 * bb;
                u32x2 ow;
                ow[0] = pack_bf16(fmaf(scale, acc[dt][j], bf16_lo(rw[0])), fmaf(scale, acc[dt][j + 1], bf16_hi(rw[0])));
                ow[1] = pack_bf16(fmaf(scale, acc[dt][j + 2], bf16_lo(rw[1])), fmaf(scale, acc[dt][j + 3], bf16_hi(rw[1])));
                *(u32x2*)(Op + d0) = ow;
            }
        }
}

template <int BLOCK, int DP, bool V16>
static hipError_t launch(AttnArgs a, hipStream_t s) {
    using C = SwgCfg<BLOCK, DP>;
    const int64_t G = (int64_t)a.B * a.H * a.nqb;
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidValue;
    a.G = (int32_t)G;
    hipLaunchKernelGGL((sparse_wg_kernel<BLOCK, DP, V16>), dim3((unsigned)G), dim3(C::NT), 0, s, a);
    return hipGetLastError();
}

bool sparse_wg_supported(const AttnArgs& a, int block) {
    // 64-token blocks at d <= 64 belong to sparse64_kernel (faster there)
    return (block == 128 || (block == 64 && a.d > 64)) && a.d <= 128 && slice_offsets_fit(a);
}

hipError_t launch_sparse_wg(AttnArgs a, int block, void* v16, hipStream_t s) {
    if (block == 64) return pad_d(a.d) <= 96 ? launch<64, 96, false>(a, s) : launch<64, 128, false>(a, s);
    if (v16) {
        const hipError_t e = launch_v16(a, v16, s);
        if (e != hipSuccess) return e;
        a.V = v16;
        switch (pad_d(a.d)) {
            case 32: return launch<128, 32, true>(a, s);
            case 64: return launch<128, 64, true>(a, s);
            case 96: return launch<128, 96, true>(a, s);
            default: return launch<128, 128, true>(a, s);
        }
    }
    switch (pad_d(a.d)) {
        case 32: return launch<128, 32, false>(a, s);
        case 64: return launch<128, 64, false>(a, s);
        case 96: return launch<128, 96, false>(a, s);
        default: return launch<128, 128, false>(a, s);
    }
}

}  // namespace rettn
