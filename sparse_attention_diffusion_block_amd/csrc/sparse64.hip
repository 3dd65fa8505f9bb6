// Sparse step of Re-ttention for bfloat16 with 64-token blocks, one wave per
// query block.
//
// The step (Re-ttention summary page, "Approach"; review thread, replies to
// W1 of the first and third reviews; ramp-up: answer to W1 of the fourth
// review) attends each 64-row query block only to its kept key blocks (the
// CSR row), then applies the statistical reshape and the residual:
//     O' = min(1, rho * (1 + lambda step)) * softmax_W(s) V_W + R.
//
// Design for gfx950 (at 96.9% sparsity the step is bound by memory latency
// and by the vector work of the softmax, not by the matrix cores):
//   * one wave owns all 64 rows of a query block, so the K and V of a key
//     block are fetched once per query block and no barrier is ever needed;
//   * every tile (Q, K, V, R) streams straight into LDS (buffer_load ... lds,
//     1 KiB per instruction); padding and keys past L read as zero through
//     the buffer bounds.  K comes back as the A fragments of S^T = K Q^T, V
//     through the transposing LDS read as the V^T fragments of
//     O^T += V^T P^T.  Each slot is refilled with the next key block as soon
//     as its fragments are in registers.  Q, R and O, touched once, move as
//     non-temporal whole rows; K and V keep the default policy, since L2
//     serves their reuse across query blocks;
//   * the MFMAs of one row tile are interleaved with independent vector work
//     (the float16 re-encoding of V, the probabilities of the other row
//     tile), which a wave issues while its MFMAs execute;
//   * P*V runs in float16 (P rounds 8x finer than in bfloat16); V is
//     re-encoded exactly as its fragments are read;
//   * the softmax keeps a running reference per row instead of a per-block
//     max: the first kept block sets it to its row max, later blocks'
//     probabilities are computed against it, and only if a row's packed
//     float16 sum is non-finite or above 2^14 is the block redone against
//     its true max (rescaling the accumulators).  Any reference gives the same mathematics; the bound
//     keeps every float16 probability finite.
#include "attn.h"
#include "common.h"

namespace rettn {

namespace {

constexpr uint32_t kOOB = 0x80000000u;   // a buffer offset past every record: reads as zero
// Cache policy of the streamed tiles: Q and R are read once and O written once, as whole 128-byte
// rows, so they move non-temporally (the nt bit) and leave the L2 to the K and V blocks that later
// query blocks of the head read again.
constexpr int kStream = 2;
constexpr int kReused = 0;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t f16x2_from_bf16x2(uint32_t w) { return pack_f16(bf16_lo(w), bf16_hi(w)); }

__device__ __forceinline__ float dot2_f16(uint32_t a, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), one, acc, false);
}

}  // namespace

template <int DP>
struct S64Cfg {
    static constexpr int NS = DP / 16;             // k-steps of S^T over d
    static constexpr int NDT = DP / 32;            // 32-row d tiles of O^T
    static constexpr int RS = 64;                  // LDS row stride (elements): one 128-byte row
    static constexpr int SLOT = 64 * RS;           // elements per 64-row LDS slot (8 KiB)
    static constexpr int NL = 8;                   // 1 KiB transfers per 64-row tile
};

// All global traffic moves as 64-row tiles of 128-byte rows, 1 KiB per
// instruction: lane l carries 16 bytes of row 8 i + l / 8, so each group of
// 8 lanes covers one contiguous row.  In LDS, logical 16-byte chunk c of row
// r sits at physical chunk c ^ swz(r) (see common.h).  A tile transfer of a
// padded chunk or of a row at or past L uses an offset past the buffer
// records: loads read zeros, stores are dropped.
template <int DP>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) sparse64_kernel(const AttnArgs a) {
    using C = S64Cfg<DP>;
    // Two separate LDS objects: the compiler can then tell that a transfer into one
    // slot never overlaps reads of the other, and does not wait for it.
    __shared__ __attribute__((aligned(1024))) uint16_t kslot[C::SLOT];   // K tiles
    __shared__ __attribute__((aligned(1024))) uint16_t vslot[C::SLOT];   // V tiles; Q at the start, R / O at the end

    const int lane = threadIdx.x;
    const int h = lane >> 5, n = lane & 31;
    const int work = xcd_remap(blockIdx.x, a.G);
    const int bh = work / a.nqb;
    const int qb = work - bh * a.nqb;
    const int bi = bh / a.H, hi = bh - bi * a.H;
    const int sl = bh % a.slice_mod;                        // this slice's CSR
    const int32_t* rp = a.row_ptr + (int64_t)sl * (a.nqb + 1);
    const int32_t* ci = a.col_idx + (int64_t)sl * a.col_stride;
    const int64_t base = (int64_t)bi * a.sb + (int64_t)hi * a.sh;
    const int q0 = qb * 64;
    const uint32_t row_bytes = (uint32_t)a.sl * 2u;
    // one (batch, head) slice: rows [0, L) of d elements
    const uint32_t nrec = (uint32_t)(a.L - 1) * row_bytes + (uint32_t)a.d * 2u;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.Q + base), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.K + base), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.V + base), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.R_in + base), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)((uint16_t*)a.O + base), 0, nrec, 0x00020000);

    // lane -> (row within an 8-row group, physical chunk) of a tile transfer.  Row 8 i + trow
    // has the same swizzle as row trow, so a lane's byte offset within every 8-row group is
    // a constant; the group's row offset goes in the scalar offset.  Both offsets count in
    // the buffer range check, so rows at or past L read as zero (and stores to them are
    // dropped), and a padded chunk (d <= 16 c) takes an offset past every record.
    const int trow = lane >> 3, tpc = lane & 7;
    const uint32_t lane_off = (tpc ^ swz(trow)) * 8 < a.d
                                  ? (uint32_t)trow * row_bytes + 16u * (uint32_t)(tpc ^ swz(trow)) : kOOB;
#define RETTN_ROW_OFF(ROW0, I) ((uint32_t)((ROW0) + 8 * (I)) * row_bytes)
    // (plain expressions only inside these loaders: a lambda called from another
    // lambda here, a buffer-resource lambda parameter or a generic pointer cast to
    // the LDS address space keeps the host compiler from emitting the launch stub)
#define RETTN_TILE_LOADER(NAME, RSRC, SLOT, POLICY)                                                           \
    auto NAME = [&](int row0) {                                                                                  \
        _Pragma("unroll") for (int i = 0; i < C::NL; ++i)                                                         \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(RSRC, (__attribute__((address_space(3))) void*)(SLOT + i * 512), \
                                                     16, lane_off, RETTN_ROW_OFF(row0, i), 0, POLICY);          \
    };
    RETTN_TILE_LOADER(load_q, rq, vslot, kStream)
    RETTN_TILE_LOADER(load_k, rk, kslot, kReused)
    RETTN_TILE_LOADER(load_v, rv, vslot, kReused)
    RETTN_TILE_LOADER(load_r, rr, vslot, kStream)
#undef RETTN_TILE_LOADER
    // fragment of row r, logical chunk c (16 bytes)
    auto frag = [&](const uint16_t* slot, int r, int c) -> u32x4 {
        return *(const u32x4*)(slot + r * C::RS + ((c ^ swz(r)) << 3));
    };

    const int e0 = scalar_load(rp, qb);
    const int nit = scalar_load(rp, qb + 1) - e0;

    // Q tile -> registers: B operand of S^T = K Q^T, Q[q0 + 32 rt + n][16 s + 8 h .. +7]
    // rho of this wave's rows (used in the epilogue; issued first so it is long done by then)
    float rho_r[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int row = q0 + 32 * rt + n;
        rho_r[rt] = row < a.L ? a.rho_in[(int64_t)bh * a.L + row] : 0.f;
    }
    // Q tile into the V slot and the first K tile into the K slot, together
    int kbn = nit > 0 ? scalar_load(ci, e0) : 0;
    load_q(q0);
    if (nit > 0) {
        load_k(kbn * 64);
        wait_vmcnt<C::NL>();                  // Q has landed (K may still be in flight)
    } else {
        wait_vmcnt<0>();
    }
    u32x4 qf[2][C::NS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int s = 0; s < C::NS; ++s) qf[rt][s] = frag(vslot, 32 * rt + n, 2 * s + h);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (nit > 0) load_v(kbn * 64);         // in flight now: K(0), then V(0)
    else load_r(q0);

    f32x16 acc[C::NDT][2];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) acc[dt][0] = acc[dt][1] = f32x16{};
    // Running reference per row, log2 units: the max of the row's first kept block, raised
    // only when a later block would overflow the float16 probabilities.
    float mref[2] = {-INFINITY, -INFINITY};
    float dsum[2] = {0.f, 0.f};

    // lane-constant parts of the transposing V reads
    const int s16 = lane & 15, g = lane >> 4;
    const int fv = ((s16 >> 2) << 1) | h;
    const int vrow = (4 * h + (s16 >> 2)) * C::RS;

    f32x16 sacc[2][2];                            // [row tile][key tile]
    u32x4 pf[2][4];                               // P^T fragments (float16) of both row tiles
    float bsum[2];
    // probabilities of pairs [p0, p1) of row tile rt (pair 4 t + w covers the two
    // scores that pack into pf[rt][t][w]) against the running reference, in float16;
    // their float16 sum accumulates into bsum[rt]
    auto make_p = [&](int rt, int p0, int p1) {
#pragma unroll
        for (int pi = p0; pi < p1; ++pi) {
            const int t = pi >> 2, w = pi & 3;
            const f32x16& sp = sacc[rt][t >> 1];
            const int o = 8 * (t & 1) + 2 * w;
            const float e0 = fast_exp2(fmaf(sp[o], a.c, -mref[rt]));
            const float e1 = fast_exp2(fmaf(sp[o + 1], a.c, -mref[rt]));
            pf[rt][t][w] = pack_f16(e0, e1);
            bsum[rt] = dot2_f16(pf[rt][t][w], bsum[rt]);
        }
    };
    // max of the current block's scores over each row of row tile rt, log2 units
    auto row_max = [&](int rt) -> float {
        float m[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) m[j] = fmaxf(sacc[rt][0][j], sacc[rt][1][j]);
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
            for (int j = 0; j < w; ++j) m[j] = fmaxf(m[j], m[j + w]);
        return xhalf_max(m[0]) * a.c;
    };
    // re-anchor the reference of row tile rt at the true running max (rescaling what is
    // accumulated), then redo its probabilities
    auto reanchor = [&](int rt) {
        const float mnew = fmaxf(mref[rt], row_max(rt));
        const float alpha = fast_exp2(mref[rt] - mnew);
        mref[rt] = mnew;
        dsum[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) acc[dt][rt] *= alpha;
        bsum[rt] = 0.f;
        make_p(rt, 0, 16);
    };
    // keys at or past L in the last key block take -inf scores
    auto mask_tail = [&](int rt, int kb) {
        int lim = a.L - kb * 64 - 4 * h;   // keys at local index >= lim do not exist
        asm volatile("" : "+v"(lim));      // keeps the compares inside the rarely taken branch
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (kt * 32 + 8 * (j >> 2) + (j & 3) >= lim) sacc[rt][kt][j] = -INFINITY;
    };

    // MFMAs per phase and the share of vector work issued behind each of them
    constexpr int NA = 2 * C::NS;                 // S^T MFMAs of one row tile
    constexpr int NC = 4 * C::NDT;                // P*V MFMAs of one row tile
    constexpr int VA = 16 * C::NDT / NA;          // V registers re-encoded per MFMA of phase A
    constexpr int PB = 16 / NA, PC = 16 / NC;     // probability pairs per MFMA of phases B and C
    static_assert(VA * NA == 16 * C::NDT && PB * NA == 16 && PC * NC == 16, "phase split");

    // In flight at the top of iteration it: K(it), then V(it).  Each iteration runs in
    // four phases; in each, every MFMA is followed by a fixed share of independent
    // vector work of the same wave, which issues while the MFMA executes:
    //   A  S^T of row tile 0            | V(it) fragments re-encoded to float16
    //      (then the K and V slots are refilled with the next key block, or the V slot
    //       with this query block's residual R after the last one)
    //   B  S^T of row tile 1            | probabilities of row tile 0
    //   C  O^T += V^T P^T of row tile 0 | probabilities of row tile 1
    //   D  O^T += V^T P^T of row tile 1
    // A row tile whose packed float16 row sum overflows is re-anchored between phases.
    for (int it = 0; it < nit; ++it) {
        const int kb = kbn;
        const bool more = it + 1 < nit;
        const bool tail = (kb + 1) * 64 > a.L;
        kbn = more ? scalar_load(ci, e0 + it + 1) : 0;

        wait_vmcnt<0>();                          // K(it) and V(it) have landed
        // The next block id comes from a scalar load, and scalar and LDS reads share one counter
        // that scalar reads may decrement out of order: while it is outstanding the compiler can
        // only wait for all fragment reads below before the first MFMA.  Consuming it here, behind
        // the transfer wait, lets each MFMA wait for just the fragments it needs.
        asm volatile("" ::"s"(kbn));
        u32x4 vf[C::NDT][4];
        {
            u32x4 kf[2][C::NS];                   // A operand: K[64 kb + 32 kt + n][16 s + 8 h .. +7]
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int s = 0; s < C::NS; ++s) kf[kt][s] = frag(kslot, 32 * kt + n, 2 * s + h);
            u32x2 vr[C::NDT][4][2];               // raw bfloat16 V^T fragments
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt) {
                    const int c = 4 * dt + 2 * (g & 1) + ((s16 & 3) >> 1);
                    const uint16_t* p = vslot + vrow + 16 * t * C::RS + ((c ^ fv) << 3) + ((s16 & 1) << 2);
                    vr[dt][t][0] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)p));
                    vr[dt][t][1] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p + 8 * C::RS)));
                }
            // phase A
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) sacc[0][kt] = sacc[1][kt] = f32x16{};
#pragma unroll
            for (int mi = 0; mi < NA; ++mi) {
                const int s = mi >> 1, kt = mi & 1;
                sacc[0][kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, kf[kt][s]), __builtin_bit_cast(bf16x8, qf[0][s]), sacc[0][kt], 0, 0, 0);
#pragma unroll
                for (int x = 0; x < VA; ++x) {
                    const int f = mi * VA + x, dt = f >> 4, t = (f >> 2) & 3, w = f & 3;
                    vf[dt][t][w] = f16x2_from_bf16x2(vr[dt][t][w >> 1][w & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // The K and V slots have been read into registers: refill them.  (The empty
            // statement keeps the re-encoding in this phase instead of next to its use.)
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(vf[dt][t]));
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (more) {
                load_k(kbn * 64);
                load_v(kbn * 64);
            } else {
                load_r(q0);
            }
            if (__builtin_expect(tail, 0)) mask_tail(0, kb);
            if (it == 0) mref[0] = row_max(0);    // first kept block: nothing accumulated yet
            // phase B
            bsum[0] = bsum[1] = 0.f;
#pragma unroll
            for (int mi = 0; mi < NA; ++mi) {
                const int s = mi >> 1, kt = mi & 1;
                sacc[1][kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, kf[kt][s]), __builtin_bit_cast(bf16x8, qf[1][s]), sacc[1][kt], 0, 0, 0);
                make_p(0, mi * PB, (mi + 1) * PB);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(bsum[0] <= 16384.f)) != 0, 0)) reanchor(0);
        dsum[0] += bsum[0];
        if (__builtin_expect(tail, 0)) mask_tail(1, kb);
        if (it == 0) mref[1] = row_max(1);
        // phase C
#pragma unroll
        for (int mi = 0; mi < NC; ++mi) {
            const int t = mi / C::NDT, dt = mi % C::NDT;
            acc[dt][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, vf[dt][t]), __builtin_bit_cast(f16x8, pf[0][t]), acc[dt][0], 0, 0, 0);
            make_p(1, mi * PC, (mi + 1) * PC);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(bsum[1] <= 16384.f)) != 0, 0)) reanchor(1);
        dsum[1] += bsum[1];
        // phase D
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
                acc[dt][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(f16x8, vf[dt][t]), __builtin_bit_cast(f16x8, pf[1][t]), acc[dt][1], 0, 0, 0);
    }

    // Epilogue: O' = min(1, rho * ramp) * acc / D' + R, transposed through LDS so
    // that R is read and O written as whole 128-byte rows.
    float scale[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const float dtot = xhalf_sum(dsum[rt]);
        scale[rt] = nit > 0 ? fminf(1.f, rho_r[rt] * a.ramp) / dtot : 0.f;
    }
    wait_vmcnt<0>();                          // R has landed in the V slot
    // lane (n, h) owns d = 32 dt + 8 bb + 4 h + r of rows 32 rt + n: read R there, write O there
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int r = 32 * rt + n;
                uint16_t* p = vslot + r * C::RS + (((4 * dt + bb) ^ swz(r)) << 3) + 4 * h;
                const u32x2 rw = *(const u32x2*)p;
                const int j = 4 * bb;
                u32x2 ow;
                ow[0] = pack_bf16(fmaf(scale[rt], acc[dt][rt][j], bf16_lo(rw[0])),
                                  fmaf(scale[rt], acc[dt][rt][j + 1], bf16_hi(rw[0])));
                ow[1] = pack_bf16(fmaf(scale[rt], acc[dt][rt][j + 2], bf16_lo(rw[1])),
                                  fmaf(scale[rt], acc[dt][rt][j + 3], bf16_hi(rw[1])));
                *(u32x2*)p = ow;
            }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < C::NL; ++i) {
        const u32x4 w = *(const u32x4*)(vslot + (8 * i + trow) * C::RS + tpc * 8);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), ro, lane_off, RETTN_ROW_OFF(q0, i), kStream);
    }
#undef RETTN_ROW_OFF
}

template <int DP>
static hipError_t launch(AttnArgs a, hipStream_t s) {
    const int64_t G = (int64_t)a.B * a.H * a.nqb;
    if (G <= 0 || G > 0x7fffffff) return hipErrorInvalidValue;
    a.G = (int32_t)G;
    hipLaunchKernelGGL((sparse64_kernel<DP>), dim3((unsigned)G), dim3(64), 0, s, a);
    return hipGetLastError();
}

bool sparse64_supported(const AttnArgs& a, int block) {
    return block == 64 && a.d <= 64 && slice_offsets_fit(a);
}

hipError_t launch_sparse64(AttnArgs a, hipStream_t s) {
    return pad_d(a.d) <= 32 ? launch<32>(a, s) : launch<64>(a, s);
}

}  // namespace rettn
