// fa_cache.hip -- writes tokens into a rolling KV cache for streaming
// decode: rows [0, sinks) keep the first tokens for good (attention sinks,
// Transformers & Math section 16.6) and rows [sinks, sinks + window) are a
// ring holding the window of the latest tokens (section 16.3: a local
// layer's cache never exceeds its window).
//
// Token t goes to row t when t < sinks, else to row sinks + (t - sinks) %
// window.  One call writes T consecutive tokens; a token that a later token
// of the same call would replace is skipped, so the cache ends up as if the
// tokens had been written one at a time.  Copy work only: every lane moves
// 16 bytes of K and 16 of V, d/8 lanes per row, so a wave moves whole rows
// with 16-byte loads and stores.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int NT = 256;

template <int D>
__global__ __launch_bounds__(NT) void kv_append_kernel(const uint16_t *k_new, const uint16_t *v_new,
                                                       uint16_t *k_cache, uint16_t *v_cache, int64_t n_rows,
                                                       int64_t T, int64_t pos, int64_t window, int64_t sinks) {
    constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
    const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
    const int64_t row = gid / LPR;  // (b * Hkv + g) * T + t
    if (row >= n_rows) return;
    const int c = (int)(gid % LPR) * 8;
    const int64_t t = row % T, bg = row / T;
    const int64_t a = pos + t;  // absolute position of this token
    if (a >= sinks && a + window <= pos + T - 1) return;  // a later token of this call takes the row
    const int64_t crow = a < sinks ? a : sinks + (a - sinks) % window;
    const int64_t src = row * D + c;
    const int64_t dst = (bg * (sinks + window) + crow) * D + c;
    *reinterpret_cast<u32x4 *>(k_cache + dst) = *reinterpret_cast<const u32x4 *>(k_new + src);
    *reinterpret_cast<u32x4 *>(v_cache + dst) = *reinterpret_cast<const u32x4 *>(v_new + src);
}

template <int D>
int launch_append_d(const void *k_new, const void *v_new, void *k_cache, void *v_cache, int64_t n_rows, int64_t T,
                    int64_t pos, int64_t window, int64_t sinks, hipStream_t stream) {
    const int64_t threads = n_rows * (D / 8);
    const int64_t blocks = (threads + NT - 1) / NT;
    if (blocks > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((kv_append_kernel<D>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                       static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new),
                       static_cast<uint16_t *>(k_cache), static_cast<uint16_t *>(v_cache), n_rows, T, pos, window,
                       sinks);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

int launch_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache, int64_t n_rows, int64_t T,
                     int64_t pos, int64_t window, int64_t sinks, int d, hipStream_t stream) {
    if (n_rows == 0) return FA_OK;
    switch (d) {
        case 32: return launch_append_d<32>(k_new, v_new, k_cache, v_cache, n_rows, T, pos, window, sinks, stream);
        case 64: return launch_append_d<64>(k_new, v_new, k_cache, v_cache, n_rows, T, pos, window, sinks, stream);
        case 128: return launch_append_d<128>(k_new, v_new, k_cache, v_cache, n_rows, T, pos, window, sinks, stream);
        default: return FA_ERR_UNSUPPORTED;
    }
}

}  // namespace fa
