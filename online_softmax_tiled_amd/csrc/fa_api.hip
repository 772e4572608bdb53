// fa_api.hip -- the extern "C" entry points of libfa_mi355x.so declared in
// include/fa_mi355x.h: argument validation, then one or two kernel launches
// on the caller's stream.  No allocation, no synchronisation, no state.
#include <math.h>
#include <string.h>

#include <mutex>

#include "fa_device.h"
#include "fa_kernels.h"

namespace {

using fa::FwdParams;

bool supported_d(int64_t d) { return d == 32 || d == 64 || d == 128; }

// The kernels move 16 bytes per lane from and to the tensor base pointers
// (vector loads, direct-to-LDS buffer loads, vector stores), and 4 bytes
// for the fp32 row arrays; a misaligned base pointer (say a view with an
// odd element offset) is refused instead of faulting or being rounded down.
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b for non-negative sizes, saturated at INT64_MAX: a product of
// absurd caller sizes then fails the limits below instead of wrapping.
int64_t mul(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

// Checks shared by every forward entry point.  Fills p on success.
int validate_fwd(const fa_fwd_args &a, FwdParams &p) {
    if (a.B < 0 || a.H < 0 || a.Hkv < 1 || a.Nq < 0 || a.Nk < 0 || a.d < 0) return FA_ERR_INVALID_ARG;
    if (a.H % a.Hkv != 0) return FA_ERR_INVALID_ARG;
    if (!isfinite(a.scale)) return FA_ERR_INVALID_ARG;
    if (!isfinite(a.softcap) || a.softcap < 0.0f) return FA_ERR_INVALID_ARG;
    if (a.window < 0) return FA_ERR_INVALID_ARG;
    if (a.window > 0 && !a.causal) return FA_ERR_INVALID_ARG;
    if (a.dtype != FA_DTYPE_BF16 && a.dtype != FA_DTYPE_FP32) return FA_ERR_INVALID_ARG;
    if (a.head_window) {
        if (a.H > FA_MAX_HEAD_WINDOWS) return FA_ERR_UNSUPPORTED;
        for (int64_t h = 0; h < a.H; ++h) {
            if (a.head_window[h] < 0) return FA_ERR_INVALID_ARG;
            if (a.head_window[h] > 0 && !a.causal) return FA_ERR_INVALID_ARG;
        }
    }
    const bool q_nonempty = mul(mul(mul(a.B, a.H), a.Nq), a.d) > 0;
    const bool kv_nonempty = mul(mul(mul(a.B, a.Hkv), a.Nk), a.d) > 0;
    if (q_nonempty && (!a.q || !a.o)) return FA_ERR_INVALID_ARG;
    if (kv_nonempty && (!a.k || !a.v)) return FA_ERR_INVALID_ARG;
    if (!aligned(a.q, 16) || !aligned(a.o, 16) || !aligned(a.k, 16) || !aligned(a.v, 16) || !aligned(a.lse, 4))
        return FA_ERR_INVALID_ARG;
    if (!supported_d(a.d)) return FA_ERR_UNSUPPORTED;
    // Per-head element offsets are 32-bit inside the kernels.
    if (mul(a.Nq, a.d) > 0x7fffffff || mul(a.Nk, a.d) > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    // Query and K/V head counts over the batch are 32-bit inside the kernels.
    if (mul(a.B, a.H) > 0x7fffffff) return FA_ERR_UNSUPPORTED;

    memset(&p, 0, sizeof p);
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.lse = a.lse;
    p.B = a.B;
    p.H = a.H;
    p.Hkv = a.Hkv;
    p.Nq = a.Nq;
    p.Nk = a.Nk;
    p.kv_rows = a.Nk;
    p.group = (int)(a.H / a.Hkv);
    p.num_splits = 1;
    p.split_len = 0;
    p.scale = a.scale;
    p.softcap = a.softcap;
    p.causal = a.causal ? 1 : 0;
    p.window = a.window;
    if (a.head_window) {
        p.has_head_window = 1;
        for (int64_t h = 0; h < a.H; ++h) p.head_window[h] = a.head_window[h];
    }
    return FA_OK;
}

int run_fwd(const fa_fwd_args &a) {
    FwdParams p;
    const int rc = validate_fwd(a, p);
    if (rc != FA_OK) return rc;
    if (a.B == 0 || a.H == 0 || a.Nq == 0) return FA_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(a.stream);
    if (a.dtype == FA_DTYPE_FP32) return fa::launch_fwd_f32(p, (int)a.d, s);
    if (fa::fwd_bf16_wide_applies(p, (int)a.d)) return fa::launch_fwd_bf16_wide(p, s);
    if (fa::fwd_bf16_splitk_applies(p, (int)a.d)) return fa::launch_fwd_bf16_splitk(p, (int)a.d, s);
    return fa::launch_fwd_bf16(p, (int)a.d, false, s);
}

// First pass of split-KV attention for validated parameters p (num_splits
// >= 1, partial pointers checked): the decode kernel when few query rows
// share a K/V head, the MFMA kernel in split mode otherwise.
int run_splitkv(FwdParams &p, float *o_part, float *m_part, float *l_part, int num_splits, int64_t d,
                fa_stream_t stream) {
    if (p.B == 0 || p.H == 0 || p.Nq == 0) return FA_OK;
    const int64_t split_len = (p.Nk + num_splits - 1) / num_splits;
    if (split_len > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    p.o = nullptr;
    p.o_part = o_part;
    p.m_part = m_part;
    p.l_part = l_part;
    p.num_splits = num_splits;
    p.split_len = (int)split_len;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((int64_t)p.group * p.Nq <= fa::splitkv_decode_max_rows()) return fa::launch_splitkv_decode(p, (int)d, s);
    return fa::launch_fwd_bf16(p, (int)d, true, s);
}

// Rolling-cache geometry: window >= 1, sinks >= 0, pos >= 0, and sizes that
// keep row indices in range.
bool valid_rolling(int64_t pos, int64_t window, int64_t sinks) {
    const int64_t lim = (int64_t)1 << 40;
    return pos >= 0 && window >= 1 && sinks >= 0 && window < lim && sinks < lim && pos < ((int64_t)1 << 62);
}

fa_fwd_args make_args(int dtype, const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                      int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                      int window, float softcap, fa_stream_t stream) {
    fa_fwd_args a;
    memset(&a, 0, sizeof a);
    a.dtype = dtype;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.Nq = Nq;
    a.Nk = Nk;
    a.d = d;
    a.scale = scale;
    a.causal = causal;
    a.window = window;
    a.softcap = softcap;
    a.head_window = nullptr;
    a.stream = stream;
    return a;
}

// Split-KV partials of fa_splitkv_attention_static: a fixed device array,
// one copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` names a host-side stand-in: its device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchFloats = FA_STATIC_SCRATCH_BYTES / sizeof(float);
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_address(float **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_HIP;
        g_scratch_dev[dev] = static_cast<float *>(ptr);
    }
    *out = g_scratch_dev[dev];
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H, int64_t Hkv,
           int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int window, float softcap,
           fa_stream_t stream) {
    return run_fwd(make_args(FA_DTYPE_BF16, q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, softcap,
                             stream));
}

int fa_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, int64_t B, int64_t H,
               int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int window, float softcap,
               fa_stream_t stream) {
    return run_fwd(make_args(FA_DTYPE_FP32, q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, softcap,
                             stream));
}

int fa_fwd_ex(const fa_fwd_args *args) {
    if (!args) return FA_ERR_INVALID_ARG;
    return run_fwd(*args);
}

int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H, int64_t Hkv,
               int64_t Nq, int64_t Nk, int64_t d, float scale, float q_descale, float k_descale, float v_descale,
               int causal, int window, fa_stream_t stream) {
    FwdParams p;
    const int rc = validate_fwd(
        make_args(FA_DTYPE_BF16, q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window, 0.0f, stream), p);
    if (rc != FA_OK) return rc;
    for (float f : {q_descale, k_descale, v_descale})
        if (!isfinite(f) || !(f > 0.0f)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    // Scores in base-2 units: dot(q8, k8) * scale * q_descale * k_descale *
    // log2(e).  A negative factor is applied as a sign flip of Q (exact in
    // fp8), a zero one as the smallest normal float: every |dot| <= 448^2 *
    // 128, so every weight is then exactly 1 (all visible keys equal).
    double c = (double)scale * q_descale * k_descale * 1.4426950408889634;
    if (!isfinite(c) || fabs(c) > 3.0e38) return FA_ERR_INVALID_ARG;
    const uint32_t qflip = c < 0.0 ? 0x80808080u : 0u;
    float c_log2 = (float)fabs(c);
    if (c_log2 < 1.17549435e-38f) c_log2 = 1.17549435e-38f;
    if (B == 0 || H == 0 || Nq == 0) return FA_OK;
    return fa::launch_fwd_fp8(p, (int)d, c_log2, v_descale, qflip, reinterpret_cast<hipStream_t>(stream));
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, float *o_part, float *m_part, float *l_part,
                   int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                   int window, float softcap, int num_splits, fa_stream_t stream) {
    if (num_splits < 1) return FA_ERR_INVALID_ARG;
    // o is not written by this pass; validate with a stand-in so only the
    // partial pointers are required.
    fa_fwd_args a = make_args(FA_DTYPE_BF16, q, k, v, o_part, nullptr, B, H, Hkv, Nq, Nk, d, scale, causal,
                              window, softcap, stream);
    FwdParams p;
    const int rc = validate_fwd(a, p);
    if (rc != FA_OK) return rc;
    if (mul(mul(B, H), Nq) > 0 && (!o_part || !m_part || !l_part)) return FA_ERR_INVALID_ARG;
    if (!aligned(m_part, 4) || !aligned(l_part, 4)) return FA_ERR_INVALID_ARG;
    return run_splitkv(p, o_part, m_part, l_part, num_splits, d, stream);
}

int fa_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache, int64_t B, int64_t Hkv,
                 int64_t T, int64_t d, int64_t pos, int64_t window, int64_t sinks, fa_stream_t stream) {
    if (B < 0 || Hkv < 0 || T < 0 || d < 0 || !valid_rolling(pos, window, sinks)) return FA_ERR_INVALID_ARG;
    const int64_t n_rows = mul(mul(B, Hkv), T);
    if (n_rows > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    if (n_rows > 0 && d > 0 && (!k_new || !v_new || !k_cache || !v_cache)) return FA_ERR_INVALID_ARG;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
        return FA_ERR_INVALID_ARG;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    return fa::launch_kv_append(k_new, v_new, k_cache, v_cache, n_rows, T, pos, window, sinks, (int)d,
                                reinterpret_cast<hipStream_t>(stream));
}

int fa_decode_rolling(const void *q, const void *k_cache, const void *v_cache, float *o_part, float *m_part,
                      float *l_part, int64_t B, int64_t H, int64_t Hkv, int64_t d, int64_t pos, int64_t window,
                      int64_t sinks, float scale, float softcap, int num_splits, fa_stream_t stream) {
    if (num_splits < 1 || !valid_rolling(pos, window, sinks)) return FA_ERR_INVALID_ARG;
    const int64_t rows = sinks + window;                  // cache rows per (batch, K/V head)
    const int64_t n = pos + 1 < rows ? pos + 1 : rows;    // filled rows: sinks and the window
    // Every filled row is visible to this query: no causal or window mask
    // over the cache rows.  o is not written by this pass (stand-in).
    fa_fwd_args a = make_args(FA_DTYPE_BF16, q, k_cache, v_cache, o_part, nullptr, B, H, Hkv, 1, n, d, scale, 0, 0,
                              softcap, stream);
    FwdParams p;
    const int rc = validate_fwd(a, p);
    if (rc != FA_OK) return rc;
    if (rows * d > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    if (mul(B, H) > 0 && (!o_part || !m_part || !l_part)) return FA_ERR_INVALID_ARG;
    if (!aligned(m_part, 4) || !aligned(l_part, 4)) return FA_ERR_INVALID_ARG;
    p.kv_rows = rows;
    return run_splitkv(p, o_part, m_part, l_part, num_splits, d, stream);
}

int fa_combine(const float *o_part, const float *m_part, const float *l_part, void *o, float *lse, int64_t B,
               int64_t H, int64_t Nq, int64_t d, int num_splits, int out_dtype, fa_stream_t stream) {
    if (B < 0 || H < 0 || Nq < 0 || d < 0 || num_splits < 1) return FA_ERR_INVALID_ARG;
    if (out_dtype != FA_DTYPE_BF16 && out_dtype != FA_DTYPE_FP32) return FA_ERR_INVALID_ARG;
    const int64_t rows = mul(mul(B, H), Nq);
    if (rows > 0 && d > 0 && (!o_part || !m_part || !l_part || !o)) return FA_ERR_INVALID_ARG;
    if (!aligned(o_part, 4) || !aligned(m_part, 4) || !aligned(l_part, 4) || !aligned(lse, 4) ||
        !aligned(o, out_dtype == FA_DTYPE_BF16 ? 2 : 4))
        return FA_ERR_INVALID_ARG;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if (rows == 0) return FA_OK;
    return fa::launch_combine(o_part, m_part, l_part, o, lse, rows, num_splits, (int)d, out_dtype,
                              reinterpret_cast<hipStream_t>(stream));
}

int fa_softmax(const void *x, void *y, float *lse, int64_t rows, int64_t n, int dtype, fa_stream_t stream) {
    if (rows < 0 || n < 0) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP32) return FA_ERR_INVALID_ARG;
    if (rows > 0 && n > 0 && (!x || !y)) return FA_ERR_INVALID_ARG;
    if (rows > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    return fa::launch_softmax(x, y, lse, rows, n, dtype, reinterpret_cast<hipStream_t>(stream));
}

int fa_softmax_topk(const void *x, float *probs, int32_t *indices, float *lse, int64_t rows, int64_t n, int k,
                    int dtype, fa_stream_t stream) {
    if (rows < 0 || n < 0 || k < 1 || k > FA_MAX_TOPK) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP32) return FA_ERR_INVALID_ARG;
    if (rows > 0 && (k > n || !x || !probs || !indices)) return FA_ERR_INVALID_ARG;
    if (rows > 0x7fffffff || n > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    return fa::launch_softmax_topk(x, probs, indices, lse, rows, n, k, dtype, reinterpret_cast<hipStream_t>(stream));
}

int fa_splitkv_attention_static(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                                int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                                int window, float softcap, int num_splits, int out_dtype, fa_stream_t stream) {
    if (num_splits < 1) return FA_ERR_INVALID_ARG;
    if (out_dtype != FA_DTYPE_BF16 && out_dtype != FA_DTYPE_FP32) return FA_ERR_INVALID_ARG;
    fa_fwd_args a = make_args(FA_DTYPE_BF16, q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, window,
                              softcap, stream);
    FwdParams p;
    const int rc = validate_fwd(a, p);
    if (rc != FA_OK) return rc;
    if (!aligned(o, out_dtype == FA_DTYPE_BF16 ? 2 : 4)) return FA_ERR_INVALID_ARG;
    const int64_t rows = mul(mul(B, H), Nq);
    if (rows == 0) return FA_OK;
    // Partials: o_part [rows, S, d], then m_part and l_part [rows, S].
    const int64_t parts = mul(rows, num_splits);
    if (mul(parts, d + 2) > (int64_t)kScratchFloats) return FA_ERR_SCRATCH_LIMIT;
    float *base = nullptr;
    const int src = scratch_address(&base);
    if (src != FA_OK) return src;
    float *o_part = base, *m_part = base + parts * d, *l_part = m_part + parts;
    const int r1 = run_splitkv(p, o_part, m_part, l_part, num_splits, d, stream);
    if (r1 != FA_OK) return r1;
    return fa::launch_combine(o_part, m_part, l_part, o, lse, rows, num_splits, (int)d, out_dtype,
                              reinterpret_cast<hipStream_t>(stream));
}

const char *fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: no kernel for this head size or shape";
        case FA_ERR_HIP: return "FA_ERR_HIP: HIP kernel launch failed";
        case FA_ERR_SCRATCH_LIMIT: return "FA_ERR_SCRATCH_LIMIT: partials exceed the static scratch";
        default: return "unknown fa_status";
    }
}

}  // extern "C"
