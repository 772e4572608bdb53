// fa_fwd_f32.hip -- fp32 tiled forward attention with an online softmax.
//
// The same method as the bf16 kernel (Transformers & Math, Module 16,
// sections 16.1-16.2), kept in fp32 end to end for workloads whose tolerance
// is set by fp32 rounding: 64 query rows per workgroup, four lanes per row
// (each owns a quarter of the head dimension, interleaved in 4-float groups
// so the lanes of one row read adjacent LDS words), key tiles of 32 staged
// in LDS.  The running maximum is kept in natural units and the weights are
// exp2((s - m) * log2 e): the difference is formed before scaling, so large
// scores (the notebook's 1000 + ln i) lose no accuracy to the log2 e factor.
#include <math.h>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int BM = 64;   // query rows per workgroup
constexpr int BN = 32;   // keys per tile
constexpr int NT = 256;  // threads per workgroup

template <int D>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(const FwdParams p) {
    constexpr int DC = D / 16;  // float4 groups per lane
    __shared__ __attribute__((aligned(16))) float Ks[BN * D];
    __shared__ __attribute__((aligned(16))) float Vs[BN * D];

    const int tid = threadIdx.x;
    const int qi = tid >> 2, part = tid & 3;
    const int h = blockIdx.y, b = blockIdx.z;
    const int g = h / p.group;
    const int64_t Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    const int W = head_window_of(p, h);
    const int64_t q0 = (int64_t)blockIdx.x * BM;
    const int64_t qrow = q0 + qi;
    const int64_t qlast = (q0 + BM < Nq ? q0 + BM : Nq) - 1;

    int64_t lo_first, hi_first, lo_last, hi_last, kmin, kmax;
    key_bounds(q0 + off, Nk, p.causal, W, lo_first, hi_first);
    key_bounds(qlast + off, Nk, p.causal, W, lo_last, hi_last);
    key_bounds(qrow + off, Nk, p.causal, W, kmin, kmax);
    const int64_t kbeg = lo_first, kend = hi_last;

    const float *Q = static_cast<const float *>(p.q) + ((int64_t)b * p.H + h) * Nq * D;
    const float *K = static_cast<const float *>(p.k) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;
    const float *V = static_cast<const float *>(p.v) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;

    f32x4 qv[DC], acc[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        qv[c] = qrow < Nq ? *reinterpret_cast<const f32x4 *>(Q + qrow * D + c * 16 + part * 4)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m = kNegInf, l = 0.0f;
    const bool capped = p.softcap > 0.0f;

    for (int64_t kt = kbeg; kt < kend; kt += BN) {
        __syncthreads();
        for (int e = tid; e < BN * D / 4; e += NT) {
            const int64_t key = kt + e / (D / 4);
            const int col = (e % (D / 4)) * 4;
            f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
            if (key < Nk) {
                kx = *reinterpret_cast<const f32x4 *>(K + key * D + col);
                vx = *reinterpret_cast<const f32x4 *>(V + key * D + col);
            }
            *reinterpret_cast<f32x4 *>(Ks + e * 4) = kx;
            *reinterpret_cast<f32x4 *>(Vs + e * 4) = vx;
        }
        __syncthreads();

        float s[BN];
        float mt = kNegInf;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            float dot = 0.0f;
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const f32x4 kx = *reinterpret_cast<const f32x4 *>(Ks + j * D + c * 16 + part * 4);
                dot = fmaf(qv[c][0], kx[0], dot);
                dot = fmaf(qv[c][1], kx[1], dot);
                dot = fmaf(qv[c][2], kx[2], dot);
                dot = fmaf(qv[c][3], kx[3], dot);
            }
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            float sj = dot * p.scale;
            if (capped) sj = p.softcap * tanhf(sj / p.softcap);
            const int64_t key = kt + j;
            if (key < kmin || key >= kmax) sj = kNegInf;
            s[j] = sj;
            mt = fmaxf(mt, sj);
        }
        const float m_new = fmaxf(m, mt);
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        const float alpha = fast_exp2((m - m_use) * kLog2e);
        float rs = 0.0f;
#pragma unroll
        for (int c = 0; c < DC; ++c) acc[c] *= alpha;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            const float pj = fast_exp2((s[j] - m_use) * kLog2e);
            rs += pj;
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const f32x4 vx = *reinterpret_cast<const f32x4 *>(Vs + j * D + c * 16 + part * 4);
                acc[c][0] = fmaf(pj, vx[0], acc[c][0]);
                acc[c][1] = fmaf(pj, vx[1], acc[c][1]);
                acc[c][2] = fmaf(pj, vx[2], acc[c][2]);
                acc[c][3] = fmaf(pj, vx[3], acc[c][3]);
            }
        }
        l = l * alpha + rs;
        m = m_new;
    }

    if (qrow >= Nq) return;
    const int64_t row = ((int64_t)b * p.H + h) * Nq + qrow;
    float *O = static_cast<float *>(p.o) + row * D;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (l > 0.0f) x = f32x4{acc[c][0] / l, acc[c][1] / l, acc[c][2] / l, acc[c][3] / l};
        *reinterpret_cast<f32x4 *>(O + c * 16 + part * 4) = x;
    }
    if (p.lse && part == 0) p.lse[row] = l > 0.0f ? m + logf(l) : kNegInf;
}

template <int D>
int launch_one(const FwdParams &p, hipStream_t stream) {
    const int64_t nq = (p.Nq + BM - 1) / BM;
    if (nq == 0 || p.B == 0 || p.H == 0) return FA_OK;
    if (nq > 0x7fffffff || p.H > 65535 || p.B > 65535) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((unsigned)nq, (unsigned)p.H, (unsigned)p.B), dim3(NT), 0, stream, p);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

int launch_fwd_f32(const FwdParams &p, int d, hipStream_t stream) {
    switch (d) {
        case 32: return launch_one<32>(p, stream);
        case 64: return launch_one<64>(p, stream);
        case 128: return launch_one<128>(p, stream);
        default: return FA_ERR_UNSUPPORTED;
    }
}

}  // namespace fa
