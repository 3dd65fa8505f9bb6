// Exercises the host-only half of the C ABI (sparse_attention_diffusion_block_amd/csrc/host.cpp)
// under the address and undefined-behaviour sanitizers: the static mask generators over a sweep
// of valid and invalid specs, the status strings, the workspace size, and the argument checks of
// every entry point, with edge values (zero, negative, INT32_MAX, misaligned and null pointers).
// Each result is also checked against what the checks must decide.  Exits non-zero on the first
// wrong result; a sanitizer finding aborts the program.
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "host.h"

using rettn::AttnArgs;
namespace host = rettn::host;

static int g_checks = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        ++g_checks;                                                               \
        if (!(cond)) {                                                            \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

static void check_masks() {
    const int nbs[] = {1, 2, 3, 5, 17, 64, 278, 1000};
    for (int nb : nbs) {
        std::vector<uint8_t> m((size_t)nb * nb + 16, 0xAB);         // 16 guard bytes after the mask
        for (int kind = -1; kind <= 4; ++kind) {
            const int ws[] = {-1, 0, 1, 2, nb / 2, nb, nb + 1};
            for (int w : ws)
                for (int text : {-1, 0, 1, nb, nb + 1})
                    for (int tshift : {INT_MIN, -1, 0, 1, 21, nb, INT_MAX}) {
                        rettn_mask_spec spec = {kind, nb, w, text, tshift};
                        memset(m.data(), 0xAB, m.size());
                        const rettn_status st = rettn_mask_build(&spec, m.data());
                        bool valid = kind >= 0 && kind <= 3;
                        if (kind == RETTN_MASK_BAND) valid = w >= 1 && w <= nb;
                        if (kind == RETTN_MASK_COGVIDEO3D) valid = text >= 0 && text <= nb && tshift >= 1;
                        EXPECT(st == (valid ? RETTN_OK : RETTN_EINVAL));
                        for (int i = 0; i < 16; ++i) EXPECT(m[(size_t)nb * nb + i] == 0xAB);   // nothing past the mask
                        if (!valid) continue;
                        for (int qb = 0; qb < nb; ++qb) {
                            int cnt = 0;
                            for (int kb = 0; kb < nb; ++kb) {
                                const uint8_t b = m[(size_t)qb * nb + kb];
                                EXPECT(b == 0 || b == 1);
                                cnt += b;
                            }
                            if (kind == RETTN_MASK_DIAG) EXPECT(cnt == 1 && m[(size_t)qb * nb + qb] == 1);
                            if (kind == RETTN_MASK_FULL) EXPECT(cnt == nb);
                            if (kind == RETTN_MASK_BAND) EXPECT(cnt == w);
                            if (kind == RETTN_MASK_COGVIDEO3D) EXPECT(cnt >= (text > 0 ? text : 1) && cnt <= text + 5);
                        }
                    }
        }
    }
    rettn_mask_spec spec = {RETTN_MASK_DIAG, 4, 0, 0, 0};
    uint8_t small[16];
    EXPECT(rettn_mask_build(nullptr, small) == RETTN_EINVAL);
    EXPECT(rettn_mask_build(&spec, nullptr) == RETTN_EINVAL);
    for (int nb : {0, -1, 65537, INT_MAX, INT_MIN}) {
        spec.nb = nb;
        EXPECT(rettn_mask_build(&spec, small) == RETTN_EINVAL);
    }
}

static void check_status_strings() {
    for (int s = -3; s <= 8; ++s) {
        const char* t = rettn_status_str((rettn_status)s);
        EXPECT(t != nullptr && strlen(t) > 0);
        EXPECT((s >= 0 && s <= 4) == (strncmp(t, "RETTN_", 6) == 0));
    }
}

static rettn_desc good_desc() { return rettn_desc{2, 3, 200, 64, 64, RETTN_BF16, 3 * 200 * 64, 200 * 64, 64}; }

static void check_workspace() {
    rettn_desc d = good_desc();
    size_t n = 0;
    EXPECT(rettn_dynamic_workspace_bytes(&d, &n) == RETTN_OK && n == 2 * 4 * 2 * 3 * 4 * 64);
    EXPECT(rettn_dynamic_workspace_bytes(nullptr, &n) == RETTN_EINVAL);
    EXPECT(rettn_dynamic_workspace_bytes(&d, nullptr) == RETTN_EINVAL);
    // sizes beyond what any call accepts are refused instead of wrapping
    rettn_desc big = {INT_MAX, INT_MAX, INT_MAX, 128, 32, RETTN_BF16, 1, 1, 128};
    EXPECT(rettn_dynamic_workspace_bytes(&big, &n) == RETTN_EUNSUPPORTED);
    for (int v : {0, -1, INT_MIN}) {
        rettn_desc e = good_desc();
        e.B = v;
        EXPECT(rettn_dynamic_workspace_bytes(&e, &n) == RETTN_EINVAL);
        e = good_desc();
        e.L = v;
        EXPECT(rettn_dynamic_workspace_bytes(&e, &n) == RETTN_EINVAL);
    }
}

// A fake device address: aligned or not, never dereferenced by the checks.
static void* addr(uintptr_t a) { return (void*)a; }

// The calibration workspace: V's extent in float16 on the 64/128-token-block path, 0 elsewhere,
// computed without overflow for any stride; its checks refuse null, misaligned, short and
// overlapping workspaces.
static void check_calib_workspace() {
    rettn_desc d = good_desc();
    size_t n = 1;
    EXPECT(host::calibrate_workspace(&d, &n) == RETTN_OK && n == (size_t)2 * 3 * 200 * 64 * 2);
    EXPECT(host::calibrate_workspace(nullptr, &n) == RETTN_EINVAL);
    EXPECT(host::calibrate_workspace(&d, nullptr) == RETTN_EINVAL);
    rettn_desc f = good_desc();
    f.dtype = RETTN_F32;
    EXPECT(host::calibrate_workspace(&f, &n) == RETTN_OK && n == 0);
    f = good_desc();
    f.block = 32;
    EXPECT(host::calibrate_workspace(&f, &n) == RETTN_OK && n == 0);
    for (int64_t big : {(int64_t)1 << 40, (int64_t)1 << 55, INT64_MAX - 7}) {
        rettn_desc e = good_desc();
        e.stride_b = big & ~(int64_t)7;
        const rettn_status st = host::calibrate_workspace(&e, &n);
        EXPECT(st == RETTN_OK || st == RETTN_EUNSUPPORTED);
        if (st == RETTN_OK) EXPECT(n == (size_t)((e.stride_b + 2 * e.stride_h + 199 * e.stride_l + 64) * 2));
    }
    const size_t need = (size_t)2 * 3 * 200 * 64 * 2 + 4096, tbytes = (size_t)2 * 3 * 200 * 64 * 2;
    const uintptr_t base = (uintptr_t)1 << 40, gap = (uintptr_t)1 << 30;
    const void* t5[5] = {addr(base), addr(base + gap), addr(base + 2 * gap), addr(base + 3 * gap), addr(base + 4 * gap)};
    auto check = [&](uintptr_t ws, size_t bytes) {
        return host::check_calibrate_workspace(addr(ws), bytes, need, tbytes, {t5[0], t5[1], t5[2], t5[3], t5[4]});
    };
    EXPECT(check(base + 8 * gap, need) == RETTN_OK);
    EXPECT(check(base + 8 * gap, need - 1) == RETTN_EINVAL);
    EXPECT(check(base + 8 * gap + 4, need) == RETTN_EINVAL);
    EXPECT(check(0, need) == RETTN_EINVAL);
    EXPECT(check(base + 2 * gap, need) == RETTN_EINVAL);                 // V itself
    EXPECT(check(base + gap - need + 16, need) == RETTN_EINVAL);         // ends inside the second tensor
    EXPECT(check(base + 3 * gap + tbytes - 16, need) == RETTN_EINVAL);   // starts inside the fourth
    EXPECT(check(base + gap - need, need) == RETTN_OK);                  // just before the second
    EXPECT(check(base + 3 * gap + tbytes, need) == RETTN_OK);            // just after the fourth
    EXPECT(host::check_calibrate_workspace(nullptr, 0, 0, tbytes, {t5[0]}) == RETTN_OK);   // not needed: ignored

    // the sparse step's pass: 128-token blocks whose key blocks are kept by enough query blocks
    rettn_desc s128 = {1, 2, 128 * 60, 128, 128, RETTN_BF16, 2 * 128 * 60 * 128, 128 * 60 * 128, 128};
    rettn_index ix{};
    ix.nqb = ix.nkb = 60;
    ix.nnz = (int32_t)(host::kSparseV16Readers * 60);
    EXPECT(host::sparse_workspace(&s128, &ix, &n) == RETTN_OK && n == (size_t)2 * 128 * 60 * 128 * 2);
    ix.nnz -= 1;
    EXPECT(host::sparse_workspace(&s128, &ix, &n) == RETTN_OK && n == 0);
    ix.nnz = INT32_MAX;
    EXPECT(host::sparse_workspace(&s128, &ix, &n) == RETTN_OK && n == (size_t)2 * 128 * 60 * 128 * 2);
    s128.block = 64;
    ix.nqb = ix.nkb = 120;
    EXPECT(host::sparse_workspace(&s128, &ix, &n) == RETTN_OK && n == 0);
    EXPECT(host::sparse_workspace(nullptr, &ix, &n) == RETTN_EINVAL);
    EXPECT(host::sparse_workspace(&s128, nullptr, &n) == RETTN_EINVAL);
    EXPECT(host::sparse_workspace(&s128, &ix, nullptr) == RETTN_EINVAL);
}

static void check_attention_args() {
    const uintptr_t A = 0x100000;              // 16-byte aligned
    int32_t rp[8], ci[8];
    uint8_t mk[16];
    rettn_index idx = {4, 4, 8, rp, ci, mk, 0, 0};
    AttnArgs a{};
    rettn_desc d = good_desc();
    // valid calls, and the arguments they produce
    EXPECT(host::prepare_calibrate(&d, addr(A), addr(A), addr(A), &idx, addr(A), (float*)addr(A), addr(A),
                                   RETTN_RESIDUAL_MASKED, &a) == RETTN_OK);
    EXPECT(a.nqb == 4 && a.slice_mod == 1 && a.residual == 0 && fabsf(a.c - 1.4426950f / 8.f) < 1e-6f);
    EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), &idx, (const float*)addr(A), addr(A), 0.04f, 3,
                                addr(A), &a) == RETTN_OK);
    EXPECT(fabsf(a.ramp - 1.12f) < 1e-6f);
    // per-head and per-slice indexes
    rettn_index per = idx;
    per.slices = 3;
    per.col_stride = 16;
    EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), &per, (const float*)addr(A), addr(A), 0.f, 1, addr(A),
                                &a) == RETTN_OK && a.slice_mod == 3 && a.col_stride == 16);
    per.slices = 6;
    EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), &per, (const float*)addr(A), addr(A), 0.f, 1, addr(A),
                                &a) == RETTN_OK && a.slice_mod == 6);
    for (int s : {2, 4, 5, 7, -1}) {
        per.slices = s;
        EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), &per, (const float*)addr(A), addr(A), 0.f, 1,
                                    addr(A), &a) == RETTN_EINVAL);
    }
    per.slices = 6;
    per.nnz = 17;                                                      // more than col_stride
    EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), &per, (const float*)addr(A), addr(A), 0.f, 1, addr(A),
                                &a) == RETTN_EINVAL);
    // descriptor fields one at a time
    struct Bad { int field; int64_t value; rettn_status want; };
    const Bad bads[] = {
        {0, 0, RETTN_EINVAL}, {0, -5, RETTN_EINVAL}, {1, 0, RETTN_EINVAL}, {2, 0, RETTN_EINVAL},
        {2, INT_MIN, RETTN_EINVAL}, {3, 0, RETTN_EINVAL}, {3, 129, RETTN_EINVAL}, {3, 60, RETTN_EINVAL},
        {4, 48, RETTN_EINVAL}, {4, 0, RETTN_EINVAL}, {5, 7, RETTN_EINVAL}, {6, 0, RETTN_EINVAL},
        {7, -8, RETTN_EINVAL}, {8, 56, RETTN_EINVAL}, {8, 68, RETTN_EINVAL},
    };
    for (const Bad& b : bads) {
        rettn_desc e = good_desc();
        switch (b.field) {
            case 0: e.B = (int32_t)b.value; break;
            case 1: e.H = (int32_t)b.value; break;
            case 2: e.L = (int32_t)b.value; break;
            case 3: e.d = (int32_t)b.value; break;
            case 4: e.block = (int32_t)b.value; break;
            case 5: e.dtype = (int32_t)b.value; break;
            case 6: e.stride_b = b.value; break;
            case 7: e.stride_h = b.value; break;
            case 8: e.stride_l = b.value; break;
        }
        EXPECT(host::prepare_calibrate(&e, addr(A), addr(A), addr(A), &idx, addr(A), (float*)addr(A), addr(A),
                                       RETTN_RESIDUAL_MASKED, &a) == b.want);
    }
    // huge shapes: refused without overflow
    rettn_desc huge = {INT_MAX, INT_MAX, INT_MAX, 128, 32, RETTN_BF16, 8, 8, 128};
    rettn_index hidx = {INT_MAX / 32 + 1, INT_MAX / 32 + 1, 0, rp, ci, mk, 0, 0};
    EXPECT(host::prepare_sparse(&huge, addr(A), addr(A), addr(A), &hidx, (const float*)addr(A), addr(A), 0.f, 1,
                                addr(A), &a) == RETTN_EUNSUPPORTED);
    // index of the wrong size, pointers, ramp
    rettn_index wrong = idx;
    wrong.nqb = 5;
    EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), &wrong, (const float*)addr(A), addr(A), 0.f, 1, addr(A),
                                &a) == RETTN_EINVAL);
    EXPECT(host::prepare_calibrate(&d, addr(A + 8), addr(A), addr(A), &idx, addr(A), (float*)addr(A), addr(A),
                                   RETTN_RESIDUAL_MASKED, &a) == RETTN_EINVAL);
    EXPECT(host::prepare_calibrate(&d, addr(A), addr(A), addr(A), &idx, addr(A), (float*)addr(A + 2), addr(A),
                                   RETTN_RESIDUAL_MASKED, &a) == RETTN_EINVAL);
    EXPECT(host::prepare_calibrate(&d, addr(A), addr(A), addr(A), &idx, addr(A), (float*)addr(A), addr(A),
                                   (rettn_residual)7, &a) == RETTN_EINVAL);
    rettn_index nomask = idx;
    nomask.mask = nullptr;
    EXPECT(host::prepare_calibrate(&d, addr(A), addr(A), addr(A), &nomask, addr(A), (float*)addr(A), addr(A),
                                   RETTN_RESIDUAL_MASKED, &a) == RETTN_EINVAL);
    for (float lam : {-1.f, NAN, INFINITY})
        EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), &idx, (const float*)addr(A), addr(A), lam, 1,
                                    addr(A), &a) == RETTN_EINVAL);
    EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), &idx, (const float*)addr(A), addr(A), 0.f, -1, addr(A),
                                &a) == RETTN_EINVAL);
    rettn_index bad_nnz = idx;
    bad_nnz.nnz = 17;
    EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), &bad_nnz, (const float*)addr(A), addr(A), 0.f, 1,
                                addr(A), &a) == RETTN_EINVAL);
    EXPECT(host::prepare_sparse(nullptr, addr(A), addr(A), addr(A), &idx, (const float*)addr(A), addr(A), 0.f, 1,
                                addr(A), &a) == RETTN_EINVAL);
    EXPECT(host::prepare_sparse(&d, addr(A), addr(A), addr(A), nullptr, (const float*)addr(A), addr(A), 0.f, 1,
                                addr(A), &a) == RETTN_EINVAL);
}

static void check_dynamic_and_index_build() {
    const uintptr_t A = 0x200000;
    rettn_desc d = good_desc();
    size_t need = 0;
    EXPECT(host::prepare_dynamic(&d, addr(A), addr(A), 3, (uint8_t*)addr(A), (int32_t*)addr(A), (int32_t*)addr(A),
                                 &need) == RETTN_OK && need == 2 * 4 * 2 * 3 * 4 * 64);
    EXPECT(host::prepare_dynamic(&d, addr(A), addr(A), 0, (uint8_t*)addr(A), (int32_t*)addr(A), (int32_t*)addr(A),
                                 &need) == RETTN_EINVAL);
    rettn_desc many = d;
    many.L = 2049 * 64;
    many.stride_h = (int64_t)many.L * 64;
    many.stride_b = 3 * many.stride_h;
    EXPECT(host::prepare_dynamic(&many, addr(A), addr(A), 3, (uint8_t*)addr(A), (int32_t*)addr(A), (int32_t*)addr(A),
                                 &need) == RETTN_EUNSUPPORTED);
    int32_t nnz = 0;
    EXPECT(host::check_index_build((uint8_t*)addr(A), 1, 278, 278, (int32_t*)addr(A), (int32_t*)addr(A), &nnz) ==
           RETTN_OK);
    EXPECT(host::check_index_build((uint8_t*)addr(A), 0, 4, 4, (int32_t*)addr(A), (int32_t*)addr(A), &nnz) ==
           RETTN_EINVAL);
    EXPECT(host::check_index_build((uint8_t*)addr(A), 65535, 2048, 2048, (int32_t*)addr(A), (int32_t*)addr(A),
                                   &nnz) == RETTN_EINVAL);              // slices x nqb x nkb beyond 2^31 - 1
    EXPECT(host::check_index_build((uint8_t*)addr(A), 1, INT_MAX, INT_MAX, (int32_t*)addr(A), (int32_t*)addr(A),
                                   &nnz) == RETTN_EINVAL);
    EXPECT(host::check_index_build(nullptr, 1, 4, 4, (int32_t*)addr(A), (int32_t*)addr(A), &nnz) == RETTN_EINVAL);
    const int32_t totals[5] = {3, 9, 0, 9, 4};
    EXPECT(host::largest_total(totals, 5) == 9 && host::largest_total(totals, 0) == 0);
}

int main() {
    check_masks();
    check_status_strings();
    check_workspace();
    check_calib_workspace();
    check_attention_args();
    check_dynamic_and_index_build();
    printf("host checks passed: %d expectations\n", g_checks);
    return 0;
}
