// fa_softmax.hip -- row softmax with the online normaliser, and the top-k of
// the softmax fused into one read of the input (gfx950).
//
// The method ("Online normalizer calculation for softmax", abstract; the
// notebook "Online Softmax Without the Attention Matrix", streaming cell):
// the maximum and the normaliser of a row are built in ONE pass with the
// running recurrence m' = max(m, x), d' = d e^(m - m') + e^(x - m'), instead
// of one pass for the maximum and another for the sum.  The softmax then
// needs two reads of the row and one write (the classical safe softmax
// needs three reads); when only the k largest probabilities are wanted,
// the running top-k is kept in the same pass and the row is read once.
//
// Layout: one workgroup per row (16 waves for the softmax, 8 for the top-k); lanes stream the row in 16-byte
// vectors (4 fp32 or 8 bf16 values; rows whose start is not 16-byte aligned
// use single elements), several loads in flight per lane.  The softmax's
// second read walks the row backwards, so that much of it is served by the
// caches the first read filled.  Every lane keeps
// its own (m, d) in fp32 with a lazily moved reference maximum (moved only
// when a value exceeds it by more than TAU, so each term is <= e^TAU); the
// lanes' states are merged with the two-block rule of Transformers & Math
// section 16.2 (d = e^(m1-m) d1 + e^(m2-m) d2).  Exponentials are exp2 of
// (x - m) log2 e: the difference first, so that rounding a large reference
// m log2 e does not reach every weight.
//
// Top-k: every wave keeps a sorted list of its k best (value, column) pairs
// spread over its lanes (lane j holds the j-th best, j < k <= 64).  A loaded
// vector is compared with the list's k-th value; only values at or above it
// (rare once the list has filled) are inserted, one at a time: the
// candidate is broadcast, its rank is the number of list entries ahead of
// it (a ballot), and the entries behind it move down one lane (DPP wave
// shift).  Order: larger value first, equal values lower column first.  The
// 8 wave lists are merged through LDS by wave 0 the same way.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int NT_SOFTMAX = 1024;  // threads per workgroup (one row) of the softmax
constexpr int NT_TOPK = 512;      // ... of the top-k (its wave lists are merged serially)
constexpr int UNROLL = 4;         // vectors in flight per lane (softmax passes)
constexpr int UNROLL_TOPK = 8;    // ... of the top-k pass (4: 3% slower; 12 or 16: no faster)
constexpr float TAU = 8.0f;      // lazy move threshold of the reference maximum (natural units)

// EPV values at element offset e of a row, as fp32.  A load that nothing
// reads again is non-temporal (NTL, streamed past the caches: +11% measured
// on the top-k and the softmax's second read); the softmax's first read is
// an ordinary load, so that its lines stay in the Infinity Cache for the
// second read (see softmax_kernel).
template <bool BF16, int EPV, bool NTL = true>
__device__ __forceinline__ void load_vec(const void *row, int64_t e, float (&x)[EPV]) {
    if constexpr (BF16) {
        const uint16_t *p = static_cast<const uint16_t *>(row) + e;
        if constexpr (EPV == 8) {
            const u32x4 w = NTL ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p))
                                : *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t wi = w[i];
                x[2 * i] = bf16lo_to_f32(wi);
                x[2 * i + 1] = bf16hi_to_f32(wi);
            }
        } else {
            x[0] = __uint_as_float((uint32_t)p[0] << 16);
        }
    } else {
        const float *p = static_cast<const float *>(row) + e;
        if constexpr (EPV == 4) {
            const f32x4 v = NTL ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p))
                                : *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = v[i];
        } else {
            x[0] = p[0];
        }
    }
}

template <bool BF16, int EPV>
__device__ __forceinline__ void store_vec(void *row, int64_t e, const float (&y)[EPV]) {
    if constexpr (BF16) {
        uint16_t *p = static_cast<uint16_t *>(row) + e;
        if constexpr (EPV == 8) {
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
        } else {
            p[0] = (uint16_t)(pack_bf16x2(y[0], 0.0f) & 0xffffu);
        }
    } else {
        float *p = static_cast<float *>(row) + e;
        if constexpr (EPV == 4) {
            const f32x4 v = {y[0], y[1], y[2], y[3]};
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
        } else {
            p[0] = y[0];
        }
    }
}

// Running (m, d) of one lane: d = sum of e^(x - m) over the values seen.
struct Norm {
    float m = kNegInf, d = 0.0f;

    template <int EPV>
    __device__ __forceinline__ void add(const float (&x)[EPV]) {
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < EPV; ++i) mx = fmaxf(mx, x[i]);
        const float mn = mx > m + TAU ? mx : m;  // move the reference only by more than TAU
        const float mu = mn == kNegInf ? 0.0f : mn;
        float s = d * fast_exp2((m - mu) * kLog2e);
        // x - mu first: exact for the values that carry weight (Sterbenz),
        // so the error does not grow with |x| as a rounded mu * log2(e)
        // reference would make it (2^-24 |mu| log2(e) in every exponent).
#pragma unroll
        for (int i = 0; i < EPV; ++i) s += fast_exp2((x[i] - mu) * kLog2e);
        m = mn;
        d = s;
    }

    // Merge another state into this one (Transformers & Math 16.2).
    __device__ __forceinline__ void merge(float m2, float d2) {
        const float mn = fmaxf(m, m2);
        if (mn == kNegInf) return;
        d = d * fast_exp2((m - mn) * kLog2e) + d2 * fast_exp2((m2 - mn) * kLog2e);
        m = mn;
    }
};

// (m, d) of the whole workgroup (NWAVE waves), returned to every thread.
template <int NWAVE>
__device__ __forceinline__ Norm block_norm(Norm s, float *sm, float *sd) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s.merge(__shfl_xor(s.m, o), __shfl_xor(s.d, o));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sm[wave] = s.m;
        sd[wave] = s.d;
    }
    __syncthreads();
    Norm t;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) t.merge(sm[w], sd[w]);
    return t;
}

template <bool BF16, int EPV>
__global__ __launch_bounds__(NT_SOFTMAX) void softmax_kernel(const void *x, void *y, float *lse, int64_t n) {
    constexpr int NT = NT_SOFTMAX, NWAVE = NT / 64;
    __shared__ float sm[NWAVE], sd[NWAVE];
    constexpr int ES = BF16 ? 2 : 4;
    const int64_t r = blockIdx.x;
    const char *xr = static_cast<const char *>(x) + r * n * ES;
    char *yr = static_cast<char *>(y) + r * n * ES;
    const int64_t nvec = n / EPV;  // n % EPV == 0 for the vector instantiations
    const int tid = threadIdx.x;

    // Pass 1: the online normaliser, with cached loads.
    Norm s;
    for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)NT * UNROLL) {
        float xv[UNROLL][EPV];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t v = v0 + (int64_t)u * NT + tid;
            if (v < nvec) {
                load_vec<BF16, EPV, false>(xr, v * EPV, xv[u]);
            } else {
#pragma unroll
                for (int i = 0; i < EPV; ++i) xv[u][i] = kNegInf;
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) s.add<EPV>(xv[u]);
    }
    const Norm t = block_norm<NWAVE>(s, sm, sd);
    const float mref = t.m == kNegInf ? 0.0f : t.m;
    const float inv = 1.0f / t.d;
    if (lse && tid == 0) lse[r] = t.m + __logf(t.d);

    // Pass 2: y = e^(x - m) / d, walking the row backwards: the part read
    // last in pass 1 is read again first, while it is still in the L2 or
    // the Infinity Cache (with 256 rows of 1 MB in flight, a forward pass
    // finds little of its row left there).  284 -> 245 us on 512 x 256000
    // fp32 together with the cached first pass (cached loads alone: 259).
    const int64_t step = (int64_t)NT * UNROLL;
    for (int64_t v0 = nvec > 0 ? ((nvec - 1) / step) * step : -1; v0 >= 0; v0 -= step) {
        float xv[UNROLL][EPV];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t v = v0 + (int64_t)u * NT + tid;
            if (v < nvec) load_vec<BF16, EPV>(xr, v * EPV, xv[u]);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t v = v0 + (int64_t)u * NT + tid;
            if (v < nvec) {
                float yv[EPV];
#pragma unroll
                for (int i = 0; i < EPV; ++i) yv[i] = fast_exp2((xv[u][i] - mref) * kLog2e) * inv;
                store_vec<BF16, EPV>(yr, v * EPV, yv);
            }
        }
    }
}

// ---------------------------------------------------------------- top-k
// Does (v1, i1) rank ahead of (v2, i2)?  Larger value first, then lower column.
__device__ __forceinline__ bool ahead(float v1, int i1, float v2, int i2) {
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

__device__ __forceinline__ float shift_down(float x, float fill) {
    // lane j receives lane j-1's value, lane 0 receives `fill`
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), 0x138, 0xF, 0xF, false));
}
__device__ __forceinline__ int shift_down(int x, int fill) {
    return __builtin_amdgcn_update_dpp(fill, x, 0x138, 0xF, 0xF, false);
}

// A wave's sorted list: lane j < k holds the j-th best (lv, li); lanes >= k
// hold (-inf, INT_MAX), which ranks after every element.
struct TopList {
    float lv = kNegInf;
    int li = 0x7fffffff;

    // Insert the wave-uniform candidate (v, i) if it ranks among the best k.
    __device__ __forceinline__ void insert(float v, int i, int k, int lane) {
        const uint64_t before = __builtin_amdgcn_ballot_w64(ahead(lv, li, v, i));
        const int pos = __builtin_popcountll(before);  // entries ahead of the candidate
        if (pos >= k) return;
        const float sv = shift_down(lv, kNegInf);
        const int si = shift_down(li, 0x7fffffff);
        if (lane > pos && lane < k) {
            lv = sv;
            li = si;
        } else if (lane == pos) {
            lv = v;
            li = i;
        }
    }
    // The k-th best entry (the bar a new value has to reach).
    __device__ __forceinline__ void kth(int k, float &v, int &i) const {
        v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), k - 1));
        i = __builtin_amdgcn_readlane(li, k - 1);
    }
};

// k-th largest of the 64 lanes' x (1 <= k <= 64): bitonic sort across the wave.
__device__ __forceinline__ float wave_kth_largest(float x, int k, int lane) {
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const float y = __shfl_xor(x, stride);
            const bool asc = (lane & size) == 0 || size == 64;  // ascending overall
            const bool low = (lane & stride) == 0;
            x = (low == asc) ? fminf(x, y) : fmaxf(x, y);
        }
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 64 - k));
}

template <bool BF16, int EPV>
__global__ __launch_bounds__(NT_TOPK) void softmax_topk_kernel(const void *x, float *probs, int32_t *idx, float *lse,
                                                               int64_t n, int k) {
    constexpr int NT = NT_TOPK, NWAVE = NT / 64;
    __shared__ float sm[NWAVE], sd[NWAVE];
    __shared__ float cv[NWAVE * 64];
    __shared__ int ci[NWAVE * 64];
    constexpr int ES = BF16 ? 2 : 4;
    const int64_t r = blockIdx.x;
    const char *xr = static_cast<const char *>(x) + r * n * ES;
    const int64_t nvec = n / EPV;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    Norm s;
    TopList top;
    float bar_v = kNegInf;      // a value must rank at or ahead of (bar_v, bar_i) to be inserted
    int bar_i = 0x7fffffff;
    float floor_v = kNegInf;    // lower bound of the wave's final k-th value
    for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)NT * UNROLL_TOPK) {
        float xv[UNROLL_TOPK][EPV];
#pragma unroll
        for (int u = 0; u < UNROLL_TOPK; ++u) {
            const int64_t v = v0 + (int64_t)u * NT + tid;
            if (v < nvec) {
                load_vec<BF16, EPV>(xr, v * EPV, xv[u]);
            } else {
#pragma unroll
                for (int i = 0; i < EPV; ++i) xv[u][i] = kNegInf;
            }
        }
        if (v0 == 0) {
            // Starting bar: the k-th largest of the lanes' maxima of this
            // first batch.  At least k loaded values reach it, so no value
            // below it can end in the wave's top k; without it the empty
            // list would take almost every value of the batch one by one.
            float mx = kNegInf;
#pragma unroll
            for (int u = 0; u < UNROLL_TOPK; ++u)
#pragma unroll
                for (int i = 0; i < EPV; ++i) mx = fmaxf(mx, xv[u][i]);
            floor_v = wave_kth_largest(mx, k, lane);
            bar_v = floor_v;
        }
#pragma unroll
        for (int u = 0; u < UNROLL_TOPK; ++u) {
            s.add<EPV>(xv[u]);
            const int64_t v = v0 + (int64_t)u * NT + tid;
            const int col0 = (int)(v * EPV);
            // Values at or above the bar that exist in the row.
            uint32_t pend = 0;
#pragma unroll
            for (int i = 0; i < EPV; ++i)
                if (v < nvec && xv[u][i] >= bar_v) pend |= 1u << i;
            uint64_t lanes = __builtin_amdgcn_ballot_w64(pend != 0);
            while (lanes) {
                const int src = __builtin_ctzll(lanes);
                // this lane's first pending value, broadcast from lane src
                const int e = pend ? __builtin_ctz(pend) : 0;
                float mine = xv[u][0];
#pragma unroll
                for (int i = 1; i < EPV; ++i) mine = e == i ? xv[u][i] : mine;
                const float cand = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), src));
                const int cidx = __builtin_amdgcn_readlane(col0 + e, src);
                top.insert(cand, cidx, k, lane);
                top.kth(k, bar_v, bar_i);
                if (bar_v < floor_v) {  // the list is not full yet: keep the starting bar
                    bar_v = floor_v;
                    bar_i = 0x7fffffff;
                }
                if (lane == src) pend &= pend - 1;
                // drop pending values that no longer reach the bar
#pragma unroll
                for (int i = 0; i < EPV; ++i)
                    if ((pend >> i) & 1u)
                        if (!ahead(xv[u][i], col0 + i, bar_v, bar_i)) pend &= ~(1u << i);
                lanes = __builtin_amdgcn_ballot_w64(pend != 0);
            }
        }
    }
    const Norm t = block_norm<NWAVE>(s, sm, sd);

    // Merge the wave lists in wave 0.
    cv[wave * 64 + lane] = top.lv;
    ci[wave * 64 + lane] = top.li;
    __syncthreads();
    if (wave != 0) return;
    for (int w = 1; w < NWAVE; ++w) {
        for (int j = 0; j < k; ++j) {
            const float v = cv[w * 64 + j];
            const int i = ci[w * 64 + j];
            top.kth(k, bar_v, bar_i);
            if (!ahead(v, i, bar_v, bar_i)) break;  // the rest of this sorted list ranks lower still
            top.insert(v, i, k, lane);
        }
    }
    if (lane < k) {
        const float mref = t.m == kNegInf ? 0.0f : t.m;
        probs[r * k + lane] = fast_exp2((top.lv - mref) * kLog2e) / t.d;
        idx[r * k + lane] = top.li;
    }
    if (lse && lane == 0) lse[r] = t.m + __logf(t.d);
}

template <bool BF16>
bool aligned16(const void *p, int64_t n) {
    return (reinterpret_cast<uintptr_t>(p) % 16) == 0 && (n * (BF16 ? 2 : 4)) % 16 == 0;
}

template <bool BF16>
int launch_softmax_t(const void *x, void *y, float *lse, int64_t rows, int64_t n, hipStream_t stream) {
    constexpr int EPV = BF16 ? 8 : 4;
    if (aligned16<BF16>(x, n) && aligned16<BF16>(y, n))
        hipLaunchKernelGGL((softmax_kernel<BF16, EPV>), dim3((unsigned)rows), dim3(NT_SOFTMAX), 0, stream, x, y, lse,
                           n);
    else
        hipLaunchKernelGGL((softmax_kernel<BF16, 1>), dim3((unsigned)rows), dim3(NT_SOFTMAX), 0, stream, x, y, lse, n);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <bool BF16>
int launch_topk_t(const void *x, float *probs, int32_t *idx, float *lse, int64_t rows, int64_t n, int k,
                  hipStream_t stream) {
    constexpr int EPV = BF16 ? 8 : 4;
    if (aligned16<BF16>(x, n))
        hipLaunchKernelGGL((softmax_topk_kernel<BF16, EPV>), dim3((unsigned)rows), dim3(NT_TOPK), 0, stream, x, probs,
                           idx, lse, n, k);
    else
        hipLaunchKernelGGL((softmax_topk_kernel<BF16, 1>), dim3((unsigned)rows), dim3(NT_TOPK), 0, stream, x, probs, idx,
                           lse, n, k);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

int launch_softmax(const void *x, void *y, float *lse, int64_t rows, int64_t n, int dtype, hipStream_t stream) {
    if (rows == 0 || n == 0) return FA_OK;
    if (rows > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    return dtype == FA_DTYPE_BF16 ? launch_softmax_t<true>(x, y, lse, rows, n, stream)
                                  : launch_softmax_t<false>(x, y, lse, rows, n, stream);
}

int launch_softmax_topk(const void *x, float *probs, int32_t *idx, float *lse, int64_t rows, int64_t n, int k,
                        int dtype, hipStream_t stream) {
    if (rows == 0) return FA_OK;
    if (rows > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    return dtype == FA_DTYPE_BF16 ? launch_topk_t<true>(x, probs, idx, lse, rows, n, k, stream)
                                  : launch_topk_t<false>(x, probs, idx, lse, rows, n, k, stream);
}

}  // namespace fa
