// fa_splitkv.hip -- split-KV attention for decode-shaped inputs and the
// combine step that merges per-split results.
//
// Split-KV cuts the key axis into chunks; each chunk's block of work
// produces its own (m, l, O): the maximum score, the sum of exp(s - m) and
// the chunk's normalised output.  fa_combine merges them with the two-block
// rule of Transformers & Math, Module 16, section 16.2 (l = e^(m1-m) l1 +
// e^(m2-m) l2, outputs weighted by their share of l), applied to all splits
// at once ("more blocks repeat the same update").
//
// Decode kernel (few query rows per K/V head; HBM-bound, 4 FLOP per byte):
//   * one workgroup per (batch, K/V head, split); all query heads of the
//     group are handled together so K and V are read from HBM once;
//   * a key row of d bf16 is read by d/8 lanes, 16 bytes each, so one wave
//     load instruction covers 64*16 = 1 KiB of consecutive keys; each group
//     of d/8 lanes is an independent online-softmax stream over its keys;
//   * dot products are VALU FMAs reduced across the d/8 lanes with DPP row
//     permutes; the streams of the workgroup are merged in LDS at the end
//     with the same merge rule as fa_combine.
#include <math.h>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int NT = 256;
constexpr int U = 8;          // key rows per stream per iteration
constexpr int MAX_ROWS = 4;   // query rows per pass of the decode kernel

__device__ __forceinline__ float dpp_f(float x, int ctrl);

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPK lanes (LPK in {4, 8, 16}); every lane of
// the group receives the total.
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xB1>(x);                   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);                   // quad_perm [2,3,0,1]
    if (LPK >= 8) x += dpp<0x141>(x);    // row_half_mirror
    if (LPK >= 16) x += dpp<0x140>(x);   // row_mirror
    return x;
}

template <int D, int R>
__global__ __launch_bounds__(NT) void splitkv_decode_kernel(const FwdParams p) {
    constexpr int LPK = D / 8;           // lanes per key row
    constexpr int KPW = 64 / LPK;        // keys (streams) per wave instruction
    constexpr int NSTREAM = 4 * KPW;     // streams per workgroup
    constexpr int KPI = 4 * U * KPW;     // keys per iteration per workgroup
    __shared__ float Sm[NSTREAM * R], Sl[NSTREAM * R];
    __shared__ __attribute__((aligned(16))) float Sacc[NSTREAM * R * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sid = lane / LPK, dl = (lane % LPK) * 8;
    const int st = wave * KPW + sid;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int64_t Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    const int64_t s_lo = (int64_t)split * p.split_len < Nk ? (int64_t)split * p.split_len : Nk;
    const int64_t s_hi = s_lo + p.split_len < Nk ? s_lo + p.split_len : Nk;
    const int GR = p.group * (int)Nq;

    const uint16_t *K = static_cast<const uint16_t *>(p.k) + ((int64_t)b * p.Hkv + g) * Nk * D;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + ((int64_t)b * p.Hkv + g) * Nk * D;
    const bool capped = p.softcap > 0.0f;

    for (int r0 = 0; r0 < GR; r0 += R) {
        float q[R][8], acc[R][8], m[R], l[R];
        int64_t kmin[R], kmax[R];
        int64_t kb = s_hi, ke = s_lo;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = r0 + r;
            m[r] = kNegInf;
            l[r] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
            kmin[r] = 0;
            kmax[r] = 0;
            if (rr < GR) {
                const int hg = rr / (int)Nq;
                const int64_t i = rr % Nq;
                const int h = g * p.group + hg;
                const u32x4 x = *reinterpret_cast<const u32x4 *>(
                    static_cast<const uint16_t *>(p.q) + (((int64_t)b * p.H + h) * Nq + i) * D + dl);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    q[r][2 * e] = bf16lo_to_f32(x[e]) * p.scale;
                    q[r][2 * e + 1] = bf16hi_to_f32(x[e]) * p.scale;
                }
                int64_t lo, hi;
                key_bounds(i + off, Nk, p.causal, head_window_of(p, h), lo, hi);
                kmin[r] = lo > s_lo ? lo : s_lo;
                kmax[r] = hi < s_hi ? hi : s_hi;
                if (kmax[r] > kmin[r]) {
                    kb = kmin[r] < kb ? kmin[r] : kb;
                    ke = kmax[r] > ke ? kmax[r] : ke;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) q[r][e] = 0.0f;
            }
        }

        for (int64_t kt = kb; kt < ke; kt += KPI) {
            u32x4 kr[U], vr[U];
            int64_t key[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                key[u] = kt + (int64_t)(wave * U + u) * KPW + sid;
                const bool in = key[u] < ke;
                kr[u] = in ? *reinterpret_cast<const u32x4 *>(K + key[u] * D + dl) : u32x4{0u, 0u, 0u, 0u};
                vr[u] = in ? *reinterpret_cast<const u32x4 *>(V + key[u] * D + dl) : u32x4{0u, 0u, 0u, 0u};
            }
            float s[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kf[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kf[2 * e] = bf16lo_to_f32(kr[u][e]);
                    kf[2 * e + 1] = bf16hi_to_f32(kr[u][e]);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float d0 = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) d0 = fmaf(q[r][e], kf[e], d0);
                    d0 = group_sum<LPK>(d0);
                    if (capped) d0 = p.softcap * tanhf(d0 / p.softcap);
                    s[u][r] = (key[u] >= kmin[r] && key[u] < kmax[r]) ? d0 : kNegInf;
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float mx = s[0][r];
#pragma unroll
                for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][r]);
                const float m_new = fmaxf(m[r], mx);
                const float m_use = m_new == kNegInf ? 0.0f : m_new;
                const float alpha = fast_exp2((m[r] - m_use) * kLog2e);
                l[r] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float pu = fast_exp2((s[u][r] - m_use) * kLog2e);
                    l[r] += pu;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[r][2 * e] = fmaf(pu, bf16lo_to_f32(vr[u][e]), acc[r][2 * e]);
                        acc[r][2 * e + 1] = fmaf(pu, bf16hi_to_f32(vr[u][e]), acc[r][2 * e + 1]);
                    }
                }
                m[r] = m_new;
            }
        }

        // Merge the NSTREAM streams of this workgroup.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if ((lane % LPK) == 0) {
                Sm[st * R + r] = m[r];
                Sl[st * R + r] = l[r];
            }
            float *dst = Sacc + (st * R + r) * D + dl;
            *reinterpret_cast<f32x4 *>(dst) = f32x4{acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
            *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{acc[r][4], acc[r][5], acc[r][6], acc[r][7]};
        }
        __syncthreads();
        for (int idx = tid; idx < R * D; idx += NT) {
            const int r = idx / D, dd = idx % D;
            const int rr = r0 + r;
            if (rr >= GR) continue;
            float M = kNegInf;
            for (int t = 0; t < NSTREAM; ++t) M = fmaxf(M, Sm[t * R + r]);
            const float M_use = M == kNegInf ? 0.0f : M;
            float Lsum = 0.0f, O = 0.0f;
            for (int t = 0; t < NSTREAM; ++t) {
                const float wgt = fast_exp2((Sm[t * R + r] - M_use) * kLog2e);
                Lsum = fmaf(wgt, Sl[t * R + r], Lsum);
                O = fmaf(wgt, Sacc[(t * R + r) * D + dd], O);
            }
            const int hg = rr / (int)Nq;
            const int64_t i = rr % Nq;
            const int h = g * p.group + hg;
            const int64_t prow = (((int64_t)b * p.H + h) * Nq + i) * p.num_splits + split;
            p.o_part[prow * D + dd] = Lsum > 0.0f ? O / Lsum : 0.0f;
            if (dd == 0) {
                p.m_part[prow] = Lsum > 0.0f ? M : kNegInf;
                p.l_part[prow] = Lsum;
            }
        }
        __syncthreads();
    }
}

template <int D>
int launch_decode_d(const FwdParams &p, hipStream_t stream) {
    const int GR = p.group * (int)p.Nq;
    dim3 grid((unsigned)p.num_splits, (unsigned)p.Hkv, (unsigned)p.B);
    if (GR <= 1)
        hipLaunchKernelGGL((splitkv_decode_kernel<D, 1>), grid, dim3(NT), 0, stream, p);
    else if (GR <= 2)
        hipLaunchKernelGGL((splitkv_decode_kernel<D, 2>), grid, dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((splitkv_decode_kernel<D, MAX_ROWS>), grid, dim3(NT), 0, stream, p);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// One wave per output row: m = max_s m_s over non-empty splits, weights
// w_s = exp(m_s - m) l_s, O = sum_s w_s O_s / sum_s w_s, lse = m + ln sum_s w_s.
template <int D>
__global__ __launch_bounds__(NT) void combine_kernel(const float *__restrict__ o_part, const float *__restrict__ m_part,
                                                     const float *__restrict__ l_part, void *o, float *lse,
                                                     const int64_t rows, const int S, const int out_bf16) {
    constexpr int PER = D >= 64 ? D / 64 : 1;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *mr = m_part + row * S;
    const float *lr = l_part + row * S;
    float M = kNegInf;
    for (int s = 0; s < S; ++s)
        if (lr[s] > 0.0f) M = fmaxf(M, mr[s]);
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
    float Lsum = 0.0f;
    if (M != kNegInf) {
        for (int s = 0; s < S; ++s) {
            const float ls = lr[s];
            if (!(ls > 0.0f)) continue;
            const float wgt = expf(mr[s] - M) * ls;
            Lsum += wgt;
            const float *os = o_part + (row * S + s) * D;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int dd = lane + 64 * k;
                if (dd < D) acc[k] = fmaf(wgt, os[dd], acc[k]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int dd = lane + 64 * k;
        if (dd >= D) continue;
        const float val = Lsum > 0.0f ? acc[k] / Lsum : 0.0f;
        if (out_bf16) {
            const uint32_t w = pack_bf16x2(val, 0.0f);
            static_cast<uint16_t *>(o)[row * D + dd] = (uint16_t)(w & 0xffffu);
        } else {
            static_cast<float *>(o)[row * D + dd] = val;
        }
    }
    if (lse && lane == 0) lse[row] = Lsum > 0.0f ? M + logf(Lsum) : kNegInf;
}

template <int D>
int launch_combine_d(const float *o_part, const float *m_part, const float *l_part, void *o, float *lse,
                     int64_t rows, int S, int out_dtype, hipStream_t stream) {
    const int64_t blocks = (rows + 3) / 4;
    if (blocks == 0) return FA_OK;
    if (blocks > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)blocks), dim3(NT), 0, stream, o_part, m_part, l_part, o,
                       lse, rows, S, out_dtype == FA_DTYPE_BF16 ? 1 : 0);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

int splitkv_decode_max_rows() { return 2 * MAX_ROWS; }

int launch_splitkv_decode(const FwdParams &p, int d, hipStream_t stream) {
    if (p.B == 0 || p.H == 0 || p.Nq == 0) return FA_OK;
    if (p.B > 65535 || p.Hkv > 65535) return FA_ERR_UNSUPPORTED;
    switch (d) {
        case 32: return launch_decode_d<32>(p, stream);
        case 64: return launch_decode_d<64>(p, stream);
        case 128: return launch_decode_d<128>(p, stream);
        default: return FA_ERR_UNSUPPORTED;
    }
}

int launch_combine(const float *o_part, const float *m_part, const float *l_part, void *o, float *lse,
                   int64_t rows, int num_splits, int d, int out_dtype, hipStream_t stream) {
    switch (d) {
        case 32: return launch_combine_d<32>(o_part, m_part, l_part, o, lse, rows, num_splits, out_dtype, stream);
        case 64: return launch_combine_d<64>(o_part, m_part, l_part, o, lse, rows, num_splits, out_dtype, stream);
        case 128: return launch_combine_d<128>(o_part, m_part, l_part, o, lse, rows, num_splits, out_dtype, stream);
        default: return FA_ERR_UNSUPPORTED;
    }
}

}  // namespace fa
