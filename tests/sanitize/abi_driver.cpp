// abi_driver.cpp -- calls every entry point of libfa_mi355x.so's C ABI with
// arguments its validation must refuse (and a few empty requests it must
// accept without launching), under AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code.  Built with the library's
// HIP sources compiled for the host only and run by tests/test_sanitize.py.
//
// No call here reaches the HIP runtime: every request is either refused by
// the argument checks or empty, both of which return before any launch or
// device query, so the driver needs no GPU and never touches one.  The
// pointers are stand-ins that are never dereferenced on the host (only
// their alignment is read); the per-head window arrays are real host
// arrays of exactly H entries, so reading past them is reported.
// Exit status 0 when every call returns the documented status.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa_mi355x.h"

static int failures = 0;

static void expect(int got, int want, const char *what, int line) {
    if (got != want) {
        fprintf(stderr, "FAIL line %d: %s returned %d (%s), expected %d\n", line, what, got, fa_status_string(got),
                want);
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

// Stand-in device pointers: 256-byte aligned addresses nobody dereferences.
static void *P(uintptr_t slot) { return reinterpret_cast<void *>((uintptr_t)0x10000000u + slot * 0x100000u); }
static float *F(uintptr_t slot) { return static_cast<float *>(P(slot)); }
static void *off(void *p, uintptr_t bytes) { return static_cast<char *>(p) + bytes; }
static float *offf(float *p, uintptr_t bytes) { return reinterpret_cast<float *>(reinterpret_cast<char *>(p) + bytes); }

static const float kNaN = NAN, kInf = INFINITY;

static void fwd_family() {
    void *q = P(1), *k = P(2), *v = P(3), *o = P(4);
    float *lse = F(5);
    const float s = 0.088f;
    // Sizes and flags.
    EXPECT(fa_fwd(q, k, v, o, lse, -1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, -4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 0, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 6, 4, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, -8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, -8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, 8, -128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, kNaN, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, kInf, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, s, 1, 0, -1.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, s, 1, 0, kInf, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, s, 1, -3, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, s, 0, 3, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    // Pointers.
    EXPECT(fa_fwd(nullptr, k, v, o, lse, 1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, nullptr, lse, 1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, nullptr, v, o, lse, 1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, nullptr, o, lse, 1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(off(q, 2), k, v, o, lse, 1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, off(k, 8), v, o, lse, 1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, off(v, 14), o, lse, 1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, off(o, 4), lse, 1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd(q, k, v, o, offf(lse, 2), 1, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    // Limits.
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, 8, 48, s, 1, 0, 0.0f, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, (int64_t)1 << 24, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_fwd(q, k, v, o, lse, 1, 4, 2, 8, (int64_t)1 << 24, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_fwd(q, k, v, o, lse, (int64_t)1 << 30, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_ERR_UNSUPPORTED);
    // Products far beyond int64 saturate instead of wrapping.
    EXPECT(fa_fwd(q, k, v, o, lse, INT64_MAX / 3, 4, 2, INT64_MAX / 5, 8, 128, s, 1, 0, 0.0f, nullptr),
           FA_ERR_UNSUPPORTED);
    // Empty requests are accepted without a launch.
    EXPECT(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_OK);
    EXPECT(fa_fwd(nullptr, k, v, nullptr, nullptr, 1, 4, 2, 0, 8, 128, s, 1, 0, 0.0f, nullptr), FA_OK);
    EXPECT(fa_fwd(nullptr, k, v, nullptr, nullptr, 1, 0, 2, 8, 8, 128, s, 1, 0, 0.0f, nullptr), FA_OK);
    // fp32 variant shares the checks.
    EXPECT(fa_fwd_f32(F(1), F(2), F(3), F(4), lse, 1, 4, 2, 8, 8, 128, s, 0, 5, 0.0f, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_f32(F(1), F(2), F(3), F(4), lse, 1, 4, 2, 8, 8, 96, s, 1, 0, 0.0f, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_fwd_f32(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 2, 8, 8, 64, s, 1, 0, 0.0f, nullptr), FA_OK);
}

static fa_fwd_args args(int64_t H, const int32_t *hw, int causal, int64_t B = 1, int64_t d = 128) {
    fa_fwd_args a;
    memset(&a, 0, sizeof a);
    a.dtype = FA_DTYPE_BF16;
    a.q = P(1);
    a.k = P(2);
    a.v = P(3);
    a.o = P(4);
    a.lse = F(5);
    a.B = B;
    a.H = H;
    a.Hkv = 1;
    a.Nq = 16;
    a.Nk = 16;
    a.d = d;
    a.scale = 0.1f;
    a.causal = causal;
    a.head_window = hw;
    return a;
}

static void fwd_ex() {
    EXPECT(fa_fwd_ex(nullptr), FA_ERR_INVALID_ARG);
    // Exactly H entries on the heap: any read past entry H-1 is reported.
    for (int64_t H : {1, 7, 32, FA_MAX_HEAD_WINDOWS}) {
        int32_t *hw = static_cast<int32_t *>(malloc(sizeof(int32_t) * H));
        for (int64_t h = 0; h < H; ++h) hw[h] = (h % 2) ? 0 : 64;
        fa_fwd_args a = args(H, hw, 1, 0);  // B = 0: validated, then nothing to launch
        EXPECT(fa_fwd_ex(&a), FA_OK);
        a = args(H, hw, 1, 1, 48);  // all H entries read, then refused for d
        EXPECT(fa_fwd_ex(&a), FA_ERR_UNSUPPORTED);
        a = args(H, hw, 0);  // a positive entry without causal
        EXPECT(fa_fwd_ex(&a), FA_ERR_INVALID_ARG);
        hw[H - 1] = -1;  // the last entry is read and refused
        a = args(H, hw, 1);
        EXPECT(fa_fwd_ex(&a), FA_ERR_INVALID_ARG);
        free(hw);
    }
    int32_t *big = static_cast<int32_t *>(calloc(FA_MAX_HEAD_WINDOWS + 1, sizeof(int32_t)));
    fa_fwd_args a = args(FA_MAX_HEAD_WINDOWS + 1, big, 1);
    EXPECT(fa_fwd_ex(&a), FA_ERR_UNSUPPORTED);
    free(big);
    a = args(4, nullptr, 1);
    a.dtype = 9;
    EXPECT(fa_fwd_ex(&a), FA_ERR_INVALID_ARG);
}

static void fp8() {
    void *q = P(1), *k = P(2), *v = P(3), *o = P(4);
    float *lse = F(5);
    EXPECT(fa_fwd_fp8(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, 0.1f, 0.0f, 1.0f, 1.0f, 1, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_fp8(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, 0.1f, 1.0f, -1.0f, 1.0f, 1, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_fp8(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, 0.1f, 1.0f, 1.0f, kNaN, 1, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_fp8(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, 0.1f, 1.0f, 1.0f, kInf, 1, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_fp8(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, 3e38f, 3e38f, 3e38f, 1.0f, 1, 0, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_fp8(q, k, v, o, lse, 1, 4, 2, 8, 8, 32, 0.1f, 1.0f, 1.0f, 1.0f, 1, 0, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_fwd_fp8(q, k, v, o, lse, 1, 4, 2, 8, 8, 128, 0.1f, 1.0f, 1.0f, 1.0f, 0, 7, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_fp8(off(q, 1), k, v, o, lse, 1, 4, 2, 8, 8, 128, 0.1f, 1.0f, 1.0f, 1.0f, 1, 0, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_fp8(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 2, 8, 8, 128, 0.1f, 1.0f, 1.0f, 1.0f, 1, 0,
                      nullptr),
           FA_OK);
}

static void splitkv_and_combine() {
    void *q = P(1), *k = P(2), *v = P(3);
    float *op = F(6), *mp = F(7), *lp = F(8);
    EXPECT(fa_fwd_splitkv(q, k, v, op, mp, lp, 2, 8, 2, 1, 1000, 128, 0.1f, 0, 0, 0.0f, 0, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_splitkv(q, k, v, op, nullptr, lp, 2, 8, 2, 1, 1000, 128, 0.1f, 0, 0, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_splitkv(q, k, v, op, mp, nullptr, 2, 8, 2, 1, 1000, 128, 0.1f, 0, 0, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_splitkv(q, k, v, nullptr, mp, lp, 2, 8, 2, 1, 1000, 128, 0.1f, 0, 0, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_splitkv(q, k, v, op, offf(mp, 2), lp, 2, 8, 2, 1, 1000, 128, 0.1f, 0, 0, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_splitkv(q, k, v, op, mp, lp, 2, 8, 2, 1, 1000, 48, 0.1f, 0, 0, 0.0f, 4, nullptr),
           FA_ERR_UNSUPPORTED);
    EXPECT(fa_fwd_splitkv(q, k, v, op, mp, lp, 2, 8, 3, 1, 1000, 128, 0.1f, 0, 0, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_fwd_splitkv(nullptr, k, v, nullptr, nullptr, nullptr, 0, 8, 2, 1, 1000, 128, 0.1f, 0, 0, 0.0f, 4,
                          nullptr),
           FA_OK);

    void *o = P(4);
    float *lse = F(5);
    EXPECT(fa_combine(op, mp, lp, o, lse, 2, 8, 1, 128, 0, FA_DTYPE_BF16, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_combine(op, mp, lp, o, lse, -2, 8, 1, 128, 4, FA_DTYPE_BF16, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_combine(op, mp, lp, o, lse, 2, 8, 1, 128, 4, 5, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_combine(op, mp, lp, nullptr, lse, 2, 8, 1, 128, 4, FA_DTYPE_BF16, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_combine(nullptr, mp, lp, o, lse, 2, 8, 1, 128, 4, FA_DTYPE_BF16, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_combine(op, mp, lp, off(o, 2), lse, 2, 8, 1, 128, 4, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_combine(op, mp, lp, off(o, 1), lse, 2, 8, 1, 128, 4, FA_DTYPE_BF16, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_combine(op, mp, offf(lp, 1), o, lse, 2, 8, 1, 128, 4, FA_DTYPE_BF16, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_combine(op, mp, lp, o, lse, 2, 8, 1, 100, 4, FA_DTYPE_BF16, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_combine(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 8, 1, 128, 4, FA_DTYPE_BF16, nullptr), FA_OK);
}

static void rolling_cache() {
    void *kn = P(1), *vn = P(2), *kc = P(3), *vc = P(4);
    EXPECT(fa_kv_append(kn, vn, kc, vc, 2, 8, 1, 128, -1, 4096, 4, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_kv_append(kn, vn, kc, vc, 2, 8, 1, 128, 10, 0, 4, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_kv_append(kn, vn, kc, vc, 2, 8, 1, 128, 10, 4096, -4, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_kv_append(kn, vn, kc, vc, 2, 8, 1, 128, 10, (int64_t)1 << 40, 4, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_kv_append(kn, vn, kc, vc, 2, 8, 1, 128, INT64_MAX, 4096, 4, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_kv_append(kn, vn, kc, vc, -2, 8, 1, 128, 10, 4096, 4, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_kv_append(kn, vn, nullptr, vc, 2, 8, 1, 128, 10, 4096, 4, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_kv_append(kn, off(vn, 2), kc, vc, 2, 8, 1, 128, 10, 4096, 4, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_kv_append(kn, vn, kc, vc, 2, 8, 1, 80, 10, 4096, 4, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_kv_append(kn, vn, kc, vc, (int64_t)1 << 20, 8, 1 << 20, 128, 10, 4096, 4, nullptr), FA_ERR_UNSUPPORTED);

    void *q = P(5);
    float *op = F(6), *mp = F(7), *lp = F(8);
    EXPECT(fa_decode_rolling(q, kc, vc, op, mp, lp, 2, 32, 8, 128, 100, 4096, 4, 0.1f, 0.0f, 0, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_decode_rolling(q, kc, vc, op, mp, lp, 2, 32, 8, 128, -1, 4096, 4, 0.1f, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_decode_rolling(q, kc, vc, op, mp, lp, 2, 30, 8, 128, 100, 4096, 4, 0.1f, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_decode_rolling(q, kc, vc, op, mp, lp, 2, 32, 8, 128, 100, 4096, 4, kNaN, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_decode_rolling(q, kc, vc, op, mp, lp, 2, 32, 8, 128, 100, 4096, 4, 0.1f, -2.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_decode_rolling(q, kc, vc, op, nullptr, lp, 2, 32, 8, 128, 100, 4096, 4, 0.1f, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_decode_rolling(q, kc, vc, op, mp, offf(lp, 2), 2, 32, 8, 128, 100, 4096, 4, 0.1f, 0.0f, 4, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_decode_rolling(q, kc, vc, op, mp, lp, 2, 32, 8, 40, 100, 4096, 4, 0.1f, 0.0f, 4, nullptr),
           FA_ERR_UNSUPPORTED);
    EXPECT(fa_decode_rolling(q, kc, vc, op, mp, lp, 2, 32, 8, 128, 100, (int64_t)1 << 30, 4, 0.1f, 0.0f, 4, nullptr),
           FA_ERR_UNSUPPORTED);
    EXPECT(fa_decode_rolling(nullptr, kc, vc, nullptr, nullptr, nullptr, 0, 32, 8, 128, 100, 4096, 4, 0.1f, 0.0f, 4,
                             nullptr),
           FA_OK);
}

static void softmax() {
    void *x = P(1), *y = P(2);
    float *lse = F(3), *probs = F(4);
    int32_t *idx = static_cast<int32_t *>(P(5));
    EXPECT(fa_softmax(x, y, lse, -1, 100, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(x, y, lse, 4, -100, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(x, y, lse, 4, 100, 3, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(nullptr, y, lse, 4, 100, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(x, nullptr, lse, 4, 100, FA_DTYPE_BF16, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(x, y, lse, (int64_t)1 << 31, 100, FA_DTYPE_FP32, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_softmax_topk(x, probs, idx, lse, 4, 100, 0, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax_topk(x, probs, idx, lse, 4, 100, FA_MAX_TOPK + 1, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax_topk(x, probs, idx, lse, 4, 5, 8, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax_topk(x, probs, nullptr, lse, 4, 100, 8, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax_topk(x, nullptr, idx, lse, 4, 100, 8, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax_topk(x, probs, idx, lse, 4, 100, 8, -1, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax_topk(x, probs, idx, lse, 4, -3, 8, FA_DTYPE_FP32, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax_topk(x, probs, idx, lse, 4, (int64_t)1 << 31, 8, FA_DTYPE_FP32, nullptr), FA_ERR_UNSUPPORTED);
}

static void static_scratch() {
    void *q = P(1), *k = P(2), *v = P(3), *o = P(4);
    float *lse = F(5);
    EXPECT(fa_splitkv_attention_static(q, k, v, o, lse, 16, 32, 8, 1, 32768, 128, 0.1f, 0, 0, 0.0f, 0, FA_DTYPE_BF16,
                                       nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_splitkv_attention_static(q, k, v, o, lse, 16, 32, 8, 1, 32768, 128, 0.1f, 0, 0, 0.0f, 4, 2, nullptr),
           FA_ERR_INVALID_ARG);
    EXPECT(fa_splitkv_attention_static(q, k, v, off(o, 2), lse, 16, 32, 8, 1, 32768, 128, 0.1f, 0, 0, 0.0f, 4,
                                       FA_DTYPE_FP32, nullptr),
           FA_ERR_INVALID_ARG);
    // Partials beyond FA_STATIC_SCRATCH_BYTES are refused before any device work.
    EXPECT(fa_splitkv_attention_static(q, k, v, o, lse, 16, 32, 8, 1, 32768, 128, 0.1f, 0, 0, 0.0f, 1024,
                                       FA_DTYPE_BF16, nullptr),
           FA_ERR_SCRATCH_LIMIT);
    EXPECT(fa_splitkv_attention_static(q, k, v, o, lse, 1, 1, 1, (int64_t)1 << 22, 16, 64, 0.1f, 1, 0, 0.0f, 1,
                                       FA_DTYPE_FP32, nullptr),
           FA_ERR_SCRATCH_LIMIT);
    EXPECT(fa_splitkv_attention_static(q, k, v, o, lse, INT64_MAX / 2, 4, 4, 1, 16, 64, 0.1f, 0, 0, 0.0f, 1 << 30,
                                       FA_DTYPE_FP32, nullptr),
           FA_ERR_UNSUPPORTED);
    EXPECT(fa_splitkv_attention_static(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 32, 8, 1, 32768, 128, 0.1f, 0,
                                       0, 0.0f, 4, FA_DTYPE_BF16, nullptr),
           FA_OK);
}

int main() {
    fwd_family();
    fwd_ex();
    fp8();
    splitkv_and_combine();
    rolling_cache();
    softmax();
    static_scratch();
    for (int s = -6; s <= 2; ++s) {
        const char *t = fa_status_string(s);
        if (!t || !t[0]) {
            fprintf(stderr, "FAIL: empty status string for %d\n", s);
            ++failures;
        }
    }
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi_driver: all checks passed\n");
    return 0;
}
