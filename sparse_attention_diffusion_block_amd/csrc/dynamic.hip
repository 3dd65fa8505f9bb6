// Dynamic block masks: a mask computed from each step's own Q and K, one per
// (batch, head) slice.  Re-ttention's authors tried their method on masks
// recomputed at every step (review thread, answers to W2 and Q1 of the first
// review) without printing how the masks were made; the rule here is the
// plainest block-level one:
//   block means  every block of query and of key tokens is summarised by the
//                mean of its tokens (the last block: its tokens < L only);
//   scores       query block a scores key block b by <mean q_a, mean k_b>;
//   selection    row a keeps block a, then the kk - 1 other blocks with the
//                highest scores; ties go to the lower block, NaN ranks last.
// Two launches:
//   dyn_pool_kernel  one work-group per (block, slice) reads the block's Q and
//                    K rows once (16-byte loads) and writes both means (fp32);
//                    the whole pass is one read of Q and K: HBM-bound.
//   dyn_topk_kernel  one wave per query block: lane j scores key blocks
//                    j, j + 64, ... against the key means staged 64 at a time
//                    in LDS, then kk - 1 rounds of a wave-wide arg-max pick the
//                    blocks; the row's mask bytes, CSR row pointer and ascending
//                    column ids are written directly (every row holds exactly
//                    kk blocks, so no count or scan is needed).
#include "attn.h"
#include "common.h"

namespace rettn {

template <bool BF16>
__global__ void __launch_bounds__(256) dyn_pool_kernel(const void* __restrict__ Q, const void* __restrict__ K, int H,
                                                       int L, int d, int block, int64_t sb, int64_t sh, int64_t sl,
                                                       int nb, float* __restrict__ qm, float* __restrict__ km) {
    constexpr int EPC = BF16 ? 8 : 4;   // elements per 16-byte chunk
    __shared__ __attribute__((aligned(16))) float red[2][256 * EPC];
    const int blk = blockIdx.x, s = blockIdx.y;
    const int bi = s / H, hi = s - bi * H;
    const int64_t base = (int64_t)bi * sb + (int64_t)hi * sh;
    const int cpr = d / EPC;            // chunks per row
    const int rp = 256 / cpr;           // rows per pass
    const int t = threadIdx.x;
    const int c = t % cpr, r0 = t / cpr;
    const int row0 = blk * block;
    const int nrows = min(block, L - row0);
    float sq[EPC], sk[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) sq[e] = sk[e] = 0.f;
    if (r0 < rp) {
        for (int r = r0; r < nrows; r += rp) {
            const int64_t off = base + (int64_t)(row0 + r) * sl + c * EPC;
            if constexpr (BF16) {
                const u32x4 wq = *(const u32x4*)((const uint16_t*)Q + off);
                const u32x4 wk = *(const u32x4*)((const uint16_t*)K + off);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sq[2 * i] += bf16_lo(wq[i]);
                    sq[2 * i + 1] += bf16_hi(wq[i]);
                    sk[2 * i] += bf16_lo(wk[i]);
                    sk[2 * i + 1] += bf16_hi(wk[i]);
                }
            } else {
                const f32x4 wq = *(const f32x4*)((const float*)Q + off);
                const f32x4 wk = *(const f32x4*)((const float*)K + off);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sq[i] += wq[i];
                    sk[i] += wk[i];
                }
            }
        }
    }
    // partial sums of (row group r0, column c * EPC + e) at r0 * d + c * EPC + e
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        red[0][t * EPC + e] = sq[e];
        red[1][t * EPC + e] = sk[e];
    }
    __syncthreads();
    // threads 0..d-1 finish Q's column t, threads 128..128+d-1 K's column t - 128
    const int which = t >> 7, col = t & 127;
    if (col < d) {
        const int groups = min(rp, nrows);
        float sum = 0.f;
        for (int g = 0; g < groups; ++g) sum += red[which][g * d + col];
        float* dst = which ? km : qm;
        dst[((int64_t)s * nb + blk) * d + col] = sum / (float)nrows;
    }
}

template <int MM>   // score registers per lane: nb <= 64 * MM
__global__ void __launch_bounds__(256) dyn_topk_kernel(const float* __restrict__ qm, const float* __restrict__ km,
                                                       int nb, int d, int kk, uint8_t* __restrict__ mask,
                                                       int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx) {
    // 64 key means (row stride d + 1: the lanes' reads of one column fall in distinct banks) and the
    // 4 query means of the work-group
    __shared__ float kt[64 * 129];
    __shared__ float qs[4 * 128];
    const int s = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int a = blockIdx.x * 4 + wave;   // this wave's query block (>= nb: idle, but joins every barrier)
    const int ldk = d + 1;
    const float* qms = qm + (int64_t)s * nb * d;
    const float* kms = km + (int64_t)s * nb * d;
    for (int e = threadIdx.x; e < 4 * d; e += 256) {
        const int w = e / d, cc = e - w * d;
        const int ab = blockIdx.x * 4 + w;
        qs[e] = ab < nb ? qms[(int64_t)ab * d + cc] : 0.f;
    }
    float sc[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        sc[m] = -INFINITY;
        if (m * 64 < nb) {   // uniform over the work-group
            __syncthreads();
            for (int e = threadIdx.x; e < 64 * d; e += 256) {
                const int r = e / d, cc = e - r * d;
                const int j = m * 64 + r;
                kt[r * ldk + cc] = j < nb ? kms[(int64_t)j * d + cc] : 0.f;
            }
            __syncthreads();
            const float* kr = kt + lane * ldk;
            const float* qr = qs + wave * d;
            float acc = 0.f;
            for (int cc = 0; cc < d; ++cc) acc = fmaf(qr[cc], kr[cc], acc);
            sc[m] = acc == acc ? acc : -INFINITY;   // NaN ranks below everything
        }
    }
    if (a >= nb) return;

    // bit m of `selb`: block lane + 64 m is kept
    uint32_t selb = lane == (a & 63) ? 1u << (a >> 6) : 0u;
    for (int round = 1; round < kk; ++round) {
        float bs = -INFINITY;
        int bj = 0x7fffffff;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int j = lane + 64 * m;
            const bool cand = j < nb && ((selb >> m) & 1u) == 0u;
            if (cand && (sc[m] > bs || (sc[m] == bs && j < bj))) {
                bs = sc[m];
                bj = j;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float os = __shfl_xor(bs, off, 64);
            const int oj = __shfl_xor(bj, off, 64);
            if (os > bs || (os == bs && oj < bj)) {
                bs = os;
                bj = oj;
            }
        }
        if (bj < nb && lane == (bj & 63)) selb |= 1u << (bj >> 6);
    }

    const int64_t mrow = ((int64_t)s * nb + a) * nb;
    int32_t* ci = col_idx + ((int64_t)s * nb + a) * kk;
    int out = 0;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        const int j = lane + 64 * m;
        const bool keep = j < nb && ((selb >> m) & 1u) != 0u;
        if (j < nb) mask[mrow + j] = keep ? 1 : 0;
        const uint64_t bal = __ballot(keep);
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (keep) ci[out + rank] = j;
        out += __popcll(bal);
    }
    if (lane == 0) {
        int32_t* rp = row_ptr + (int64_t)s * (nb + 1);
        rp[a] = a * kk;
        if (a == nb - 1) rp[nb] = nb * kk;
    }
}

template <int MM>
static void launch_topk(dim3 grid, const float* qm, const float* km, int nb, int d, int kk, uint8_t* mask,
                        int32_t* row_ptr, int32_t* col_idx, hipStream_t s) {
    hipLaunchKernelGGL(dyn_topk_kernel<MM>, grid, dim3(256), 0, s, qm, km, nb, d, kk, mask, row_ptr, col_idx);
}

hipError_t launch_dynamic_index(const void* Q, const void* K, bool bf16, int B, int H, int L, int d, int block,
                                int64_t sb, int64_t sh, int64_t sl, int keep, float* ws, uint8_t* mask,
                                int32_t* row_ptr, int32_t* col_idx, hipStream_t s) {
    const int nb = (L + block - 1) / block;
    const int S = B * H;
    const int kk = keep < nb ? keep : nb;
    float* qm = ws;
    float* km = ws + (int64_t)S * nb * d;
    if (bf16) {
        hipLaunchKernelGGL(dyn_pool_kernel<true>, dim3(nb, S), dim3(256), 0, s, Q, K, H, L, d, block, sb, sh, sl, nb,
                           qm, km);
    } else {
        hipLaunchKernelGGL(dyn_pool_kernel<false>, dim3(nb, S), dim3(256), 0, s, Q, K, H, L, d, block, sb, sh, sl, nb,
                           qm, km);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((nb + 3) / 4, S);
    const int mm = (nb + 63) / 64;
    if (mm <= 1) launch_topk<1>(grid, qm, km, nb, d, kk, mask, row_ptr, col_idx, s);
    else if (mm <= 2) launch_topk<2>(grid, qm, km, nb, d, kk, mask, row_ptr, col_idx, s);
    else if (mm <= 4) launch_topk<4>(grid, qm, km, nb, d, kk, mask, row_ptr, col_idx, s);
    else if (mm <= 8) launch_topk<8>(grid, qm, km, nb, d, kk, mask, row_ptr, col_idx, s);
    else if (mm <= 16) launch_topk<16>(grid, qm, km, nb, d, kk, mask, row_ptr, col_idx, s);
    else if (mm <= 32) launch_topk<32>(grid, qm, km, nb, d, kk, mask, row_ptr, col_idx, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace rettn
