// fa_device.h -- device helpers and launch parameters shared by the HIP
// kernels of libfa_mi355x.so (gfx950 / CDNA4 only).
//
// Numerics of the online softmax (Transformers & Math, Module 16, section
// 16.2; the notebook "Online Softmax Without the Attention Matrix"): every
// query row keeps a running maximum m, a normaliser l and an unnormalised
// fp32 output; when a tile raises the maximum, l and the output are
// multiplied by exp(m_old - m_new).  The kernels work in base 2: scores are
// carried as t = s * log2(e), so exp(s - m) = exp2(t - m2), one v_exp_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_mi355x.h"

namespace fa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Everything a forward kernel needs; passed by value as the kernel argument.
struct FwdParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    float *o_part, *m_part, *l_part;  // split-KV outputs (NULL otherwise)
    int64_t B, H, Hkv, Nq, Nk;
    int64_t kv_rows;   // rows per (batch, K/V head) in the K and V buffers (>= Nk)
    int group;         // H / Hkv
    int num_splits;    // 1 unless split-KV
    int split_len;     // keys per split (ceil(Nk / num_splits))
    float scale;       // multiplies q.k
    float softcap;     // 0: off
    int causal;
    int window;        // used when has_head_window == 0
    int has_head_window;
    int32_t head_window[FA_MAX_HEAD_WINDOWS];
};

__device__ __forceinline__ int head_window_of(const FwdParams &p, int h) {
    return p.has_head_window ? p.head_window[h] : p.window;
}

// bf16 <-> fp32.  bf16 -> fp32 is exact (the high half of the fp32 word);
// fp32 -> bf16 uses the hardware round-to-nearest-even pack.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Reinterpret a 32-bit word as two bf16.  Takes the word by value: applying
// __builtin_bit_cast directly to an ext_vector element (v[e]) reads element
// 0 whatever e is with this compiler, so vector elements must pass through a
// scalar first.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// kappa * tanh(z / kappa) returned in base-2 units (times log2 e).
// tanh(u) = 1 - 2 / (exp(2u) + 1); the exp saturates to inf/0 for large |u|,
// which gives exactly +-1.
__device__ __forceinline__ float softcap_log2(float z, float kappa) {
    float e = fast_exp2(z * (2.0f * kLog2e / kappa));
    float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
    return (kappa * kLog2e) * t;
}

// The same from the raw product s, with the constants folded once per
// launch: c2 = scale * 2 log2(e) / kappa, kl = kappa log2(e), nkl2 = -2 kl.
// kl * tanh(u) = kl - 2 kl / (e^(2u) + 1): one multiply, exp2, add,
// reciprocal and fused multiply-add per score.
__device__ __forceinline__ float softcap_log2_pre(float s, float c2, float kl, float nkl2) {
    return fmaf(__builtin_amdgcn_rcpf(fast_exp2(s * c2) + 1.0f), nkl2, kl);
}

// Visible-key interval [lo, hi) of a query at absolute position pos.
__device__ __forceinline__ void key_bounds(int64_t pos, int64_t Nk, int causal, int window,
                                           int64_t &lo, int64_t &hi) {
    hi = causal ? (pos + 1 < Nk ? pos + 1 : Nk) : Nk;
    lo = (window > 0) ? (pos - window + 1 > 0 ? pos - window + 1 : 0) : 0;
    if (hi < lo) hi = lo;
}

}  // namespace fa
