// fa_splitkv.hip -- split-KV attention for decode-shaped inputs and the
// combine step that merges per-split results.
//
// Split-KV cuts the key axis into chunks; each chunk's block of work
// produces its own (m, l, O): the maximum score, the sum of exp(s - m) and
// the chunk's normalised output.  fa_combine merges them with the two-block
// rule of Transformers & Math, Module 16, section 16.2 (l = e^(m1-m) l1 +
// e^(m2-m) l2, outputs weighted by their share of l), applied to all splits
// at once (folding further blocks in one by one gives the same result).
//
// Decode kernel (few query rows per K/V head; HBM-bound, 4 FLOP per byte):
//   * one workgroup per (batch, K/V head, split); all query heads of the
//     group are handled together so K and V are read from HBM once;
//   * a key row of d bf16 is read by d/8 lanes, 16 bytes each, so one wave
//     load instruction covers 64*16 = 1 KiB of consecutive keys; each group
//     of d/8 lanes is an independent online-softmax stream over its keys;
//   * the rows of the next iteration are loaded before the current rows are
//     used, so each wave keeps loads in flight through its compute (at two
//     workgroups per CU little else hides the HBM latency);
//   * dot products use v_dot2_f32_bf16 on the raw bf16 pairs (two products,
//     fp32 accumulation), reduced across the d/8 lanes with DPP row
//     permutes; P.V pairs two keys held by the same lane so each output
//     element costs one dot2 per row, with P rounded to bf16 as in the
//     prefill kernel; the streams of the workgroup are merged in LDS at the
//     end with the same merge rule as fa_combine.
#include <math.h>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int NT = 256;
constexpr int U = 4;          // key rows per stream per iteration; the next
                              // iteration's rows load during this one's compute
                              // (U = 8 without that overlap: 9% slower on 4100-key
                              // splits, 1.5% on 2048-key ones; U = 6 or 8 with it
                              // exceed 256 VGPRs and halve the occupancy)
constexpr int MAX_ROWS = 4;   // query rows per pass of the decode kernel

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

template <int D, int R, bool CAP>
__global__ __launch_bounds__(NT) void splitkv_decode_kernel(const FwdParams p) {
    constexpr int LPK = D / 8;           // lanes per key row
    constexpr int KPW = 64 / LPK;        // keys (streams) per wave instruction
    constexpr int NSTREAM = 4 * KPW;     // streams per workgroup
    constexpr int KPI = 4 * U * KPW;     // keys per iteration per workgroup
    constexpr float TAU = 8.0f;          // lazy-rescale threshold, log2 units
    __shared__ float Sm[NSTREAM * R], Sl[NSTREAM * R], St[NSTREAM * R];
    __shared__ __attribute__((aligned(16))) float Sacc[NSTREAM * R * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sid = lane / LPK, dl = (lane % LPK) * 8;
    const int st = wave * KPW + sid;
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int64_t Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    const int64_t s_lo = (int64_t)split * p.split_len < Nk ? (int64_t)split * p.split_len : Nk;
    const int64_t s_hi = s_lo + p.split_len < Nk ? s_lo + p.split_len : Nk;
    const int GR = p.group * (int)Nq;

    const uint16_t *K = static_cast<const uint16_t *>(p.k) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;
    const float c_log2 = p.scale * kLog2e;

    for (int r0 = 0; r0 < GR; r0 += R) {
        u32x4 qb[R];              // this lane's 8 dims of each query row, bf16 pairs
        float acc[R][8], m[R], l[R];
        float mtrue[R];           // exact running maximum (m is a lazy reference)
        int64_t kmin[R], kmax[R];
        int64_t kb = s_hi, ke = s_lo;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = r0 + r;
            m[r] = kNegInf;
            mtrue[r] = kNegInf;
            l[r] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
            kmin[r] = 0;
            kmax[r] = 0;
            qb[r] = u32x4{0u, 0u, 0u, 0u};
            if (rr < GR) {
                const int hg = rr / (int)Nq;
                const int64_t i = rr % Nq;
                const int h = g * p.group + hg;
                qb[r] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.q) +
                                                         (((int64_t)b * p.H + h) * Nq + i) * D + dl);
                int64_t lo, hi;
                key_bounds(i + off, Nk, p.causal, head_window_of(p, h), lo, hi);
                kmin[r] = lo > s_lo ? lo : s_lo;
                kmax[r] = hi < s_hi ? hi : s_hi;
                if (kmax[r] > kmin[r]) {
                    kb = kmin[r] < kb ? kmin[r] : kb;
                    ke = kmax[r] > ke ? kmax[r] : ke;
                }
            }
        }

        // Rows of the next iteration are loaded before this one's compute.
        auto load = [&](int64_t kt, u32x4 (&kr)[U], u32x4 (&vr)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t key_u = kt + (int64_t)(wave * U + u) * KPW + sid;
                const bool in = key_u < ke;
                // Each key row is read once per launch: non-temporal loads
                // stream it past the caches (+9% HBM rate measured).
                kr[u] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(K + key_u * D + dl))
                           : u32x4{0u, 0u, 0u, 0u};
                vr[u] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(V + key_u * D + dl))
                           : u32x4{0u, 0u, 0u, 0u};
            }
        };
        auto step = [&](int64_t kt, const u32x4 (&kr)[U], const u32x4 (&vr)[U]) {
            int64_t key[U];
#pragma unroll
            for (int u = 0; u < U; ++u) key[u] = kt + (int64_t)(wave * U + u) * KPW + sid;
            // Scores in log2 units: dot2 on bf16 pairs, reduced over the d/8
            // lanes of the key, scaled (and capped) once.
            float t[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float d0 = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        d0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qb[r][e]), as_bf16x2(kr[u][e]), d0, false);
                    d0 = group_sum<LPK>(d0);
                    d0 = CAP ? softcap_log2(d0 * p.scale, p.softcap) : d0 * c_log2;
                    t[u][r] = (key[u] >= kmin[r] && key[u] < kmax[r]) ? d0 : kNegInf;
                }
            // Move each stream's reference maximum only when it grew by more
            // than TAU (the result is the same for any reference point).
            float mx[R];
            bool grow = false;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                mx[r] = t[0][r];
#pragma unroll
                for (int u = 1; u < U; ++u) mx[r] = fmaxf(mx[r], t[u][r]);
                mtrue[r] = fmaxf(mtrue[r], mx[r]);
                grow = grow || (mx[r] > m[r] + TAU);
            }
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float m_new = fmaxf(m[r], mx[r]);
                    const float alpha = fast_exp2(m[r] - (m_new == kNegInf ? 0.0f : m_new));
                    l[r] *= alpha;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
                    m[r] = m_new;
                }
            }
            // P V over key pairs (u, u+1) held by this lane: one dot2 per output
            // element and row on (V_u[e], V_u+1[e]) . (p_u, p_u+1), p rounded to bf16.
#pragma unroll
            for (int u = 0; u < U; u += 2) {
                uint32_t vp[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vp[2 * e] = (vr[u][e] & 0xffffu) | (vr[u + 1][e] << 16);
                    vp[2 * e + 1] = (vr[u][e] >> 16) | (vr[u + 1][e] & 0xffff0000u);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float m_use = m[r] == kNegInf ? 0.0f : m[r];
                    const float p0 = fast_exp2(t[u][r] - m_use), p1 = fast_exp2(t[u + 1][r] - m_use);
                    l[r] += p0 + p1;
                    const bf16x2 pp = as_bf16x2(pack_bf16x2(p0, p1));
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[r][e] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vp[e]), pp, acc[r][e], false);
                }
            }
        };
        u32x4 ka[U], va[U], kn[U], vn[U];
        int64_t kt = kb;
        if (kt < ke) load(kt, ka, va);
        while (kt < ke) {
            if (kt + KPI < ke) load(kt + KPI, kn, vn);
            step(kt, ka, va);
            kt += KPI;
            if (kt >= ke) break;
            if (kt + KPI < ke) load(kt + KPI, ka, va);
            step(kt, kn, vn);
            kt += KPI;
        }

        // Merge the NSTREAM streams of this workgroup.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if ((lane % LPK) == 0) {
                Sm[st * R + r] = m[r];
                Sl[st * R + r] = l[r];
                St[st * R + r] = mtrue[r];
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
            float M = kNegInf, Mt = kNegInf;
            for (int t2 = 0; t2 < NSTREAM; ++t2) {
                M = fmaxf(M, Sm[t2 * R + r]);
                Mt = fmaxf(Mt, St[t2 * R + r]);
            }
            const float M_use = M == kNegInf ? 0.0f : M;
            float Lsum = 0.0f, O = 0.0f;
            for (int t2 = 0; t2 < NSTREAM; ++t2) {
                const float wgt = fast_exp2(Sm[t2 * R + r] - M_use);
                Lsum = fmaf(wgt, Sl[t2 * R + r], Lsum);
                O = fmaf(wgt, Sacc[(t2 * R + r) * D + dd], O);
            }
            const int hg = rr / (int)Nq;
            const int64_t i = rr % Nq;
            const int h = g * p.group + hg;
            const int64_t prow = (((int64_t)b * p.H + h) * Nq + i) * p.num_splits + split;
            p.o_part[prow * D + dd] = Lsum > 0.0f ? O / Lsum : 0.0f;
            if (dd == 0) {
                // Report the split's exact maximum, with l relative to it.
                p.m_part[prow] = Lsum > 0.0f ? Mt * kLn2 : kNegInf;
                p.l_part[prow] = Lsum > 0.0f ? Lsum * fast_exp2(M - Mt) : 0.0f;
            }
        }
        __syncthreads();
    }
}

template <int D, bool CAP>
int launch_decode_dc(const FwdParams &p, hipStream_t stream) {
    const int GR = p.group * (int)p.Nq;
    dim3 grid((unsigned)p.num_splits, (unsigned)p.Hkv, (unsigned)p.B);
    if (GR <= 1)
        hipLaunchKernelGGL((splitkv_decode_kernel<D, 1, CAP>), grid, dim3(NT), 0, stream, p);
    else if (GR <= 2)
        hipLaunchKernelGGL((splitkv_decode_kernel<D, 2, CAP>), grid, dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((splitkv_decode_kernel<D, MAX_ROWS, CAP>), grid, dim3(NT), 0, stream, p);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int D>
int launch_decode_d(const FwdParams &p, hipStream_t stream) {
    return p.softcap > 0.0f ? launch_decode_dc<D, true>(p, stream) : launch_decode_dc<D, false>(p, stream);
}

// Wave-wide reductions (all 64 lanes receive the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// One 64-lane workgroup per output row.  Lanes first take one split each
// (64 at a time): m = max_s m_s over non-empty splits, weights
// w_s = exp(m_s - m) l_s, l = sum_s w_s, kept in LDS.  Then each lane
// accumulates O[d] = sum_s w_s O_s[d] / l for its D/64 columns (or one
// column for D < 64), with the split loop unrolled so several partial rows
// are in flight.  lse = m + ln l.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const float *__restrict__ o_part, const float *__restrict__ m_part,
                                                     const float *__restrict__ l_part, void *o, float *lse,
                                                     const int S, const int out_bf16) {
    constexpr int PER = D >= 64 ? D / 64 : 1;
    constexpr int MAXS = 256;  // splits whose weights stay in LDS; more use several passes
    __shared__ float wsh[MAXS];
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    const float *mr = m_part + row * S;
    const float *lr = l_part + row * S;

    float M = kNegInf;
    for (int s = lane; s < S; s += 64)
        if (lr[s] > 0.0f) M = fmaxf(M, mr[s]);
    M = wave_max(M);

    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
    float Lsum = 0.0f;
    if (M != kNegInf) {
        for (int s0 = 0; s0 < S; s0 += MAXS) {
            const int ns = S - s0 < MAXS ? S - s0 : MAXS;
            float part = 0.0f;
            for (int s = lane; s < ns; s += 64) {
                const float ls = lr[s0 + s];
                const float wgt = ls > 0.0f ? expf(mr[s0 + s] - M) * ls : 0.0f;
                wsh[s] = wgt;
                part += wgt;
            }
            Lsum += wave_sum(part);
            __syncthreads();
            const float *os = o_part + (row * S + s0) * D;
            int s = 0;
            for (; s + 4 <= ns; s += 4) {
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    const int dd = lane + 64 * k;
                    if (dd < D) {
                        const float x0 = os[(s + 0) * D + dd], x1 = os[(s + 1) * D + dd];
                        const float x2 = os[(s + 2) * D + dd], x3 = os[(s + 3) * D + dd];
                        acc[k] = fmaf(wsh[s], x0, acc[k]);
                        acc[k] = fmaf(wsh[s + 1], x1, acc[k]);
                        acc[k] = fmaf(wsh[s + 2], x2, acc[k]);
                        acc[k] = fmaf(wsh[s + 3], x3, acc[k]);
                    }
                }
            }
            for (; s < ns; ++s) {
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    const int dd = lane + 64 * k;
                    if (dd < D) acc[k] = fmaf(wsh[s], os[s * D + dd], acc[k]);
                }
            }
            __syncthreads();
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

// Few splits (S <= SF): every load of the row is issued at once -- lane s
// takes (m_s, l_s), and each lane the partial outputs of all S splits for
// its columns -- so the merge costs one memory round trip instead of three.
// Same arithmetic, in the same order, as combine_kernel: M over non-empty
// splits, w_s = exp(m_s - M) l_s (lane s), l = the wave sum of w, and
// O[d] = sum_s w_s O_s[d] / l with w_s broadcast from lane s.
template <int D, int SF>
__global__ __launch_bounds__(64) void combine_few_kernel(const float *__restrict__ o_part,
                                                         const float *__restrict__ m_part,
                                                         const float *__restrict__ l_part, void *o, float *lse,
                                                         const int S, const int out_bf16) {
    constexpr int PER = D >= 64 ? D / 64 : 1;
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    float ms = kNegInf, ls = 0.0f;
    if (lane < S) {
        ms = m_part[row * S + lane];
        ls = l_part[row * S + lane];
    }
    float x[SF][PER];
    const float *os = o_part + row * S * D;
#pragma unroll
    for (int s = 0; s < SF; ++s)
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int dd = lane + 64 * k;
            x[s][k] = (s < S && dd < D) ? os[s * D + dd] : 0.0f;
        }
    const float M = wave_max(ls > 0.0f ? ms : kNegInf);
    const float w = (M != kNegInf && ls > 0.0f) ? expf(ms - M) * ls : 0.0f;
    const float Lsum = M != kNegInf ? wave_sum(w) : 0.0f;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
    // Splits s >= S have w = 0 and x = 0: their FMAs leave acc unchanged.
#pragma unroll
    for (int s = 0; s < SF; ++s) {
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = fmaf(ws, x[s][k], acc[k]);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int dd = lane + 64 * k;
        if (dd >= D) continue;
        const float val = Lsum > 0.0f ? acc[k] / Lsum : 0.0f;
        if (out_bf16) {
            const uint32_t wb = pack_bf16x2(val, 0.0f);
            static_cast<uint16_t *>(o)[row * D + dd] = (uint16_t)(wb & 0xffffu);
        } else {
            static_cast<float *>(o)[row * D + dd] = val;
        }
    }
    if (lse && lane == 0) lse[row] = Lsum > 0.0f ? M + logf(Lsum) : kNegInf;
}

template <int D>
int launch_combine_d(const float *o_part, const float *m_part, const float *l_part, void *o, float *lse,
                     int64_t rows, int S, int out_dtype, hipStream_t stream) {
    if (rows == 0) return FA_OK;
    if (rows > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    const int ob = out_dtype == FA_DTYPE_BF16 ? 1 : 0;
    if (S <= 16)
        hipLaunchKernelGGL((combine_few_kernel<D, 16>), dim3((unsigned)rows), dim3(64), 0, stream, o_part, m_part,
                           l_part, o, lse, S, ob);
    else
        hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)rows), dim3(64), 0, stream, o_part, m_part, l_part, o,
                           lse, S, ob);
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
