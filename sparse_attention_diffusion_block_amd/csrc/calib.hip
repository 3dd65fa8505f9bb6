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
//   * K tiles arrive by coalesced direct-to-LDS loads; V tiles either the same
//     way from a float16 copy of V made by one pass over it (v16_kernel, when
//     the caller supplies a workspace), or by coalesced 16-byte loads that are
//     re-encoded to float16 once per work-group and written to LDS; both double
//     buffered, one barrier per tile;
//   * with a workspace, a last round of work-groups at most half full is split
//     along the key range: each part stores its partial softmax state and
//     calib_merge_kernel combines them (a tail of 12% of a round otherwise
//     costs a whole round);
//   * S^T = K Q^T and O^T += V^T P^T on 32x32x16 MFMA (bf16, then fp16), one
//     query row per lane; V^T fragments come from the transposing LDS read;
//   * the static mask bit of (query block, key block) is wave-uniform and
//     routes the tile's P*V and mass into the in-window or the masked
//     accumulators;
//   * softmax against a running reference per row: a tile is redone against
//     its true max only when a row's packed float16 sum is non-finite or
//     above 2^14 (then all four accumulators are rescaled).
#include <algorithm>

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

template <int BLOCK, int DP, bool V16>
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
    const int nkt = (a.L + 63) / 64;
    // Work-groups are dispatched in order, round-robin over the XCDs.  With a split last round the
    // whole groups come first and the parts after them, each run spread evenly over the XCDs (so
    // that every XCD gets its share of both), each XCD taking a contiguous range of either.
    const int blk = blockIdx.x;
    const int work = a.nsplit <= 1 ? xcd_remap(blk, a.G)
                     : blk < a.split_from ? xcd_remap(blk, a.split_from)
                                          : a.split_from + xcd_remap(blk - a.split_from, a.G - a.split_from);
    // a work item of the split last round is part `part` of group `grp`, over key tiles [kt_lo, kt_hi)
    int grp = work, part = -1, kt_lo = 0, kt_hi = nkt;
    if (a.nsplit > 1 && work >= a.split_from) {
        const int t = work - a.split_from;
        grp = a.split_from + t / a.nsplit;
        part = t - (t / a.nsplit) * a.nsplit;
        kt_lo = (int)((int64_t)part * nkt / a.nsplit);
        kt_hi = (int)((int64_t)(part + 1) * nkt / a.nsplit);
    }
    const int bh = grp / ntile;
    const int tile = grp - bh * ntile;
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
    // V, bfloat16: thread t holds 16-byte chunks t, t + NT, ... in registers until they are re-encoded and
    // stored.  V16 (V already converted to float16 by v16_kernel): direct-to-LDS like K.
    // (plain expressions only inside these lambdas: see the note in sparse64.hip; a buffer-load
    // argument taken straight from an array element also suppressed the stub, hence the locals)
    u32x4 vreg[V16 ? 1 : C::VC];
    // A lane's byte offset within a tile is the same for every tile (a padded chunk takes an offset
    // past every record); the tile's row offset kt * 64 * row_bytes rides in the scalar offset.
    // (Each offset array is declared right before the lambda that reads it: other placements
    // kept the host compiler from emitting the launch stubs.)
    uint32_t k_off[C::KL];
#pragma unroll
    for (int j = 0; j < C::KL; ++j) {
        const int piece = wave + j * C::NW;                  // 1 KiB piece of the tile
        const int r = piece * (64 / C::CPR) + lane / C::CPR; // key row within the tile
        const int c = (lane % C::CPR) ^ swz(r);              // logical chunk loaded into this slot
        k_off[j] = c * 8 < a.d ? (uint32_t)r * row_bytes + 16u * c : kOOB;
    }
    auto issue_k = [&](int kt, int buf) {
#pragma unroll
        for (int j = 0; j < C::KL; ++j) {
            const int piece = wave + j * C::NW;
            const uint32_t off = k_off[j];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (__attribute__((address_space(3))) void*)(lds + buf * 2 * C::TILE + piece * 512), 16, off,
                (uint32_t)kt * 64u * row_bytes, 0, 0);
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
    // V tile kt towards slot buf (bfloat16: into registers now, into the slot at store_v)
    auto issue_v = [&](int kt, int buf) {
        if constexpr (V16) {
#pragma unroll
            for (int j = 0; j < C::KL; ++j) {
                const int piece = wave + j * C::NW;
                const uint32_t off = k_off[j];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rv, (__attribute__((address_space(3))) void*)(lds + buf * 2 * C::TILE + C::TILE + piece * 512), 16,
                    off, (uint32_t)kt * 64u * row_bytes, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < C::VC; ++j) {
                const uint32_t off = v_off[j];
                vreg[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, (uint32_t)kt * 64u * row_bytes, 0));
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

    f32x16 acc_in[C::NDT], acc_out[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) acc_in[dt] = acc_out[dt] = f32x16{};
    float mref = -INFINITY, d_in = 0.f, d_out = 0.f;

    const int swn = swz(n);
    // d within the first DP - 16 elements: the last 16-element k-step of S^T holds only zeros
    const bool short_d = __builtin_amdgcn_readfirstlane(a.d) <= DP - 16;
    const int s16 = lane & 15, g = lane >> 4;
    const int fv = ((s16 >> 2) << 1) | h;
    const int vrow = (4 * h + (s16 >> 2)) * C::RS;

    issue_k(kt_lo, 0);
    issue_v(kt_lo, 0);
    store_v(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();

    for (int kt64 = kt_lo; kt64 < kt_hi; ++kt64) {
        const int buf = (kt64 - kt_lo) & 1;
        const bool more = kt64 + 1 < kt_hi;
        if (more) {
            issue_k(kt64 + 1, buf ^ 1);
            issue_v(kt64 + 1, buf ^ 1);
        }
        const uint16_t* ks = lds + buf * 2 * C::TILE;
        const uint16_t* vs = ks + C::TILE;
        if constexpr (C::QLDS) asm volatile("" : "+v"(qoff));   // re-read Q every tile, not kept in registers

        // S^T for the tile's two 32-key halves: two independent MFMA chains, issued alternately
        // (the last k-step is skipped when it covers only padding: d = 72 at DP = 96)
        f32x16 sacc[2];
        sacc[0] = sacc[1] = f32x16{};
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            if (s == C::NS - 1 && short_d) break;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const uint16_t* kr = ks + (kt * 32 + n) * C::RS;
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
    if (part >= 0) {
        // partial state of this part, against its own reference mref (log2 units):
        // {mref, D_in, D_out, 0}, then N_in[DP], then N_out[DP], per row of the split groups
        if (!row_ok) return;
        const int64_t tail_rows = (int64_t)(a.G - a.split_from) / a.nsplit * C::QT;
        const int64_t trow = (int64_t)(grp - a.split_from) * C::QT + wave * 32 + n;
        float* rec = a.part + ((int64_t)part * tail_rows + trow) * (4 + 2 * DP);
        if (h == 0) *(f32x4*)rec = f32x4{mref, din, dout, 0.f};
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int d0 = 32 * dt + 8 * bb + 4 * h;
                f32x4 vi, vo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    vi[r] = acc_in[dt][4 * bb + r];
                    vo[r] = acc_out[dt][4 * bb + r];
                }
                *(f32x4*)(rec + 4 + d0) = vi;
                *(f32x4*)(rec + 4 + DP + d0) = vo;
            }
        return;
    }
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

// V converted once to float16 in V's own layout (exactly as the kernel's per-tile re-encoding would):
// every (batch, head, row)'s d elements, 16 bytes per thread and step.
__global__ void __launch_bounds__(256) v16_kernel(const AttnArgs a, uint16_t* __restrict__ out) {
    const int64_t cpr = a.d / 8;                          // 16-byte chunks per row
    const int64_t total = (int64_t)a.B * a.H * a.L * cpr;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = i % cpr, rowid = i / cpr;
        const int64_t r = rowid % a.L, bh = rowid / a.L;
        const int64_t b = bh / a.H, hd = bh - b * a.H;
        const int64_t off = b * a.sb + hd * a.sh + r * a.sl + 8 * c;
        const u32x4 w = *(const u32x4*)((const uint16_t*)a.V + off);
        *(u32x4*)(out + off) = bf16x8_to_f16x8(w);
    }
}

// Combines the nsplit partial states of every row of the split groups (written by the parts'
// epilogue) into O, rho and R: the parts' sums are brought to the largest of their references and
// added, then the calibration's own epilogue arithmetic follows.  One thread per 4 elements of a row.
template <int DP>
__global__ void __launch_bounds__(256) calib_merge_kernel(const AttnArgs a) {
    using C = CalCfg<DP>;
    constexpr int REC = 4 + 2 * DP;
    const int ntile = (a.L + C::QT - 1) / C::QT;
    const int64_t tail_rows = (int64_t)(a.G - a.split_from) / a.nsplit * C::QT;
    const int cpr = a.d / 4;
    const int64_t total = tail_rows * cpr;
    const bool diff = a.residual != 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t trow = i / cpr;
        const int c4 = (int)(i - trow * cpr);
        const int grp = a.split_from + (int)(trow / C::QT);
        const int bh = grp / ntile;
        const int row = (grp - bh * ntile) * C::QT + (int)(trow % C::QT);
        if (row >= a.L) continue;
        float M = -INFINITY;
        for (int p = 0; p < a.nsplit; ++p) M = fmaxf(M, a.part[((int64_t)p * tail_rows + trow) * REC]);
        float din = 0.f, dout = 0.f;
        f32x4 ni = {0.f, 0.f, 0.f, 0.f}, no = {0.f, 0.f, 0.f, 0.f};
        for (int p = 0; p < a.nsplit; ++p) {
            const float* rec = a.part + ((int64_t)p * tail_rows + trow) * REC;
            const f32x4 hd = *(const f32x4*)rec;
            const float w = hd[0] == -INFINITY ? 0.f : fast_exp2(hd[0] - M);
            din += w * hd[1];
            dout += w * hd[2];
            ni += w * *(const f32x4*)(rec + 4 + 4 * c4);
            no += w * *(const f32x4*)(rec + 4 + DP + 4 * c4);
        }
        const float inv = 1.f / (din + dout);
        const float inv_in = din > 0.f ? 1.f / din : 0.f;
        const int bi = bh / a.H, hi = bh - bi * a.H;
        const int64_t off = (int64_t)bi * a.sb + (int64_t)hi * a.sh + (int64_t)row * a.sl + 4 * c4;
        float ov[4], rv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ov[r] = (ni[r] + no[r]) * inv;
            rv[r] = diff ? ov[r] - ni[r] * inv_in : no[r] * inv;
        }
        u32x2 ow, rw;
        ow[0] = pack_bf16(ov[0], ov[1]);
        ow[1] = pack_bf16(ov[2], ov[3]);
        rw[0] = pack_bf16(rv[0], rv[1]);
        rw[1] = pack_bf16(rv[2], rv[3]);
        *(u32x2*)((uint16_t*)a.O + off) = ow;
        *(u32x2*)((uint16_t*)a.R_out + off) = rw;
        if (c4 == 0) a.rho_out[(int64_t)bh * a.L + row] = din * inv;
    }
}

// How the last round is split.  slots = work-groups resident on the whole device at once.  When
// the groups fill at least one round and leave a last round at most half full, each group of that
// round is cut into nsplit parts along the key range (at least two key tiles per part, at most
// 8 parts), so that the last round holds nsplit times as many, shorter, work items.
struct SplitPlan {
    int from = 0, nsplit = 1;
    int64_t groups = 0, tail = 0;
};

template <int BLOCK, int DP>
static SplitPlan split_plan(const AttnArgs& a) {
    using C = CalCfg<DP>;
    SplitPlan sp;
    sp.groups = (int64_t)a.B * a.H * ((a.L + C::QT - 1) / C::QT);
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, calib_kernel<BLOCK, DP, true>, C::NT, 0) != hipSuccess)
        return sp;
    const int64_t slots = (int64_t)cus * per_cu;
    if (slots <= 0 || sp.groups < slots) return sp;
    const int64_t tail = sp.groups % slots;
    const int64_t nkt = (a.L + 63) / 64;
    if (tail == 0 || 2 * tail > slots) return sp;
    const int64_t n = std::min<int64_t>(std::min<int64_t>(slots / tail, 8), nkt / 2);
    if (n < 2 || sp.groups - tail + tail * n > 0x7fffffff) return sp;
    sp.from = (int)(sp.groups - tail);
    sp.nsplit = (int)n;
    sp.tail = tail;
    return sp;
}

template <int BLOCK, int DP>
static size_t split_bytes(const AttnArgs& a) {
    const SplitPlan sp = split_plan<BLOCK, DP>(a);
    if (sp.nsplit <= 1) return 0;
    return (size_t)sp.nsplit * (size_t)sp.tail * CalCfg<DP>::QT * (4 + 2 * DP) * sizeof(float);
}

template <int BLOCK, int DP, bool V16>
static hipError_t launch(AttnArgs a, float* part, hipStream_t s) {
    using C = CalCfg<DP>;
    const int64_t ntile = (a.L + C::QT - 1) / C::QT;
    int64_t G = (int64_t)a.B * a.H * ntile;
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidValue;
    a.nsplit = 1;
    a.split_from = 0;
    a.part = nullptr;
    if (V16 && part) {
        const SplitPlan sp = split_plan<BLOCK, DP>(a);
        if (sp.nsplit > 1) {
            a.split_from = sp.from;
            a.nsplit = sp.nsplit;
            a.part = part;
            G = sp.from + sp.tail * sp.nsplit;
        }
    }
    a.G = (int32_t)G;
    hipLaunchKernelGGL((calib_kernel<BLOCK, DP, V16>), dim3((unsigned)G), dim3(C::NT), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit <= 1) return e;
    hipLaunchKernelGGL((calib_merge_kernel<DP>), dim3(1024), dim3(256), 0, s, a);
    return hipGetLastError();
}

bool calib_supported(const AttnArgs& a, int block) {
    // every d up to 128: two accumulator sets fit at 2 waves per SIMD (Q in LDS at d = 128)
    return calib_fast_path(a, block);
}

#define RETTN_CALIB_CASES(X)                                                                    \
    X(64, 32) X(64, 64) X(64, 96) X(64, 128) X(128, 32) X(128, 64) X(128, 96) X(128, 128)

size_t calib_split_bytes(const AttnArgs& a, int block) {
    const int dp = pad_d(a.d);
#define RETTN_CASE(BL, D) \
    if (block == BL && dp == D) return split_bytes<BL, D>(a);
    RETTN_CALIB_CASES(RETTN_CASE)
#undef RETTN_CASE
    return 0;
}

hipError_t launch_v16(const AttnArgs& a, void* v16, hipStream_t s) {
    hipLaunchKernelGGL(v16_kernel, dim3(2048), dim3(256), 0, s, a, (uint16_t*)v16);
    return hipGetLastError();
}

hipError_t launch_calib(AttnArgs a, int block, void* v16, void* part, hipStream_t s) {
    const int dp = pad_d(a.d);
    if (v16) {
        const hipError_t e = launch_v16(a, v16, s);
        if (e != hipSuccess) return e;
        a.V = v16;
    }
#define RETTN_CASE(BL, D)                                                                         \
    if (block == BL && dp == D)                                                                   \
        return v16 ? launch<BL, D, true>(a, (float*)part, s) : launch<BL, D, false>(a, nullptr, s);
    RETTN_CALIB_CASES(RETTN_CASE)
#undef RETTN_CASE
    return hipErrorInvalidValue;
}

}  // namespace rettn
