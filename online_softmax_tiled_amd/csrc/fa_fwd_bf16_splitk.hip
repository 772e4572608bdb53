// fa_fwd_bf16_splitk.hip -- bf16 forward attention for grids too small to
// fill the GPU: the waves of a workgroup (8 for d <= 64, 4 for d = 128)
// share 32 query rows and split their keys among them, then merge.
//
// The method is the tiled online softmax of the other bf16 kernels
// (Transformers & Math, Module 16, section 16.1 flow), and the merge of the
// four per-wave results is the two-block merge rule of section 16.2 applied
// to all waves: m = max_w m_w, l = sum_w e^(m_w - m) l_w, O = sum_w e^(m_w
// - m) O_w / l.  With B*H*Nq/32 workgroups a problem such as B = 1, H = 8,
// 1024 x 1024, d = 64 puts two waves on each of the 1024 SIMDs in a single
// launch, where workgroups of 128 or 256 query rows would occupy a quarter
// of them, and it needs no workspace: the partial results meet in LDS.
//
// Per wave and 32-key step: the step's K and V rows go from HBM / L2
// straight into the wave's own LDS slots (coalesced 1 KiB loads; K rows
// swizzled so that the operand reads are free of bank conflicts), S^T = K
// Q^T with K operands read back from LDS, the online softmax of its 32 x 32
// block (lazily moved reference maximum, as in the other kernels), P
// rounded to bf16, and O^T += V^T P^T with the V^T operands read from the
// row-major V rows (transposing reads, ds_read_b64_tr_b16).  The next
// step's K and V are in flight while a step computes.  (K loaded straight
// into registers in operand layout touches 32 rows per load instruction;
// through LDS the B=1, H=8, 1024^2, d=64 launch went from 11.5 to 9.1 us.)
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_tile.h"

namespace fa {

namespace {

// Key splits per workgroup, one per wave: 8 for d <= 64 (two waves per
// SIMD), 4 for d = 128 (its staging and merge buffers are twice as large).
template <int D>
constexpr int sk_waves() { return D == 128 ? 4 : 8; }
constexpr int SK_ROWS = 32;  // query rows per workgroup
constexpr int SK_STEP = 32;  // keys per step

typedef short sk_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) sk_i16x4 sk_lds_i16x4;

constexpr float kSkTau = 8.0f;  // lazy-rescale threshold, log2 units

__device__ __forceinline__ float sk_max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Maximum of a lane's 16 scores (v_max3_f32: no quieting of the inputs).
__device__ __forceinline__ float sk_max16(const f32x16 &s) {
    const float a = sk_max3(s[0], s[1], s[2]), b = sk_max3(s[3], s[4], s[5]), c = sk_max3(s[6], s[7], s[8]);
    const float d = sk_max3(s[9], s[10], s[11]), e = sk_max3(s[12], s[13], s[14]);
    return sk_max3(sk_max3(a, b, c), sk_max3(d, e, s[15]), a);
}

__device__ __forceinline__ int sk_lane() {
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

template <int D>
struct SkLayout {
    static constexpr int SK_WAVES = sk_waves<D>();
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int VBUF = SK_STEP * ROW_BYTES;              // one step of V (or K) rows (bytes)
    static constexpr int SLOTS = 2;                               // steps of K and V in flight
    static constexpr int WAVE_BYTES = SLOTS * 2 * VBUF;           // K slots, then V slots
    static constexpr int CPR = D / 8;                             // 16-byte chunks per row
    static constexpr int RPL_LOG2 = D == 128 ? 0 : (D == 64 ? 1 : 2);  // log2(rows per 256-byte bank line)
    // K: chunk c of row r in slot c ^ ((r >> RPL_LOG2) % CPR): the 16 rows
    // of one 16-lane pass of an operand read land on distinct bank groups.
    __device__ static int kslot(int r, int c) { return c ^ ((r >> RPL_LOG2) & (CPR - 1)); }
    static constexpr int STAGE = SK_WAVES * WAVE_BYTES;           // all waves
    // A wave's partial result (O [32][D], m [32], l [32], fp32) goes into its
    // own staging region once its last step has read it.
    static constexpr int PART = SK_ROWS * (D + 2) * 4;
    static_assert(PART <= WAVE_BYTES, "the partial result must fit in the wave's staging region");
    static constexpr int BYTES = STAGE;
    static constexpr int LOADS = SK_STEP * D / 8 / 64;            // 16-byte V loads per lane per step
};

template <int D, bool EXPLICIT, bool CAP>
__global__ __launch_bounds__(64 * sk_waves<D>()) void fwd_bf16_splitk_kernel(const FwdParams p, const int n_qtiles) {
    using SL = SkLayout<D>;
    constexpr int SK_WAVES = SL::SK_WAVES;
    // s_waitcnt vmcnt(n * D / 8) (low four bits of the count in [3:0], the
    // rest in [15:14]): n steps' loads (D/16 K + D/16 V each) may stay in flight.
    constexpr int kV1 = 0x0f70 | ((D / 8) & 15) | (((D / 8) >> 4) << 14);
    constexpr int kV2 = 0x0f70 | ((D / 4) & 15) | (((D / 4) >> 4) << 14);
    constexpr int kV3 = 0x0f70 | ((3 * D / 8) & 15) | (((3 * D / 8) >> 4) << 14);
    __shared__ __attribute__((aligned(1024))) char lds[SL::BYTES];

    const int tid = threadIdx.x;
    const int lane = sk_lane();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;

    const int qtile = (int)(blockIdx.x % n_qtiles);
    const int bh = (int)(blockIdx.x / n_qtiles);
    const int b = bh / (int)p.H, h = bh % (int)p.H;
    const int g = h / p.group;
    const int64_t Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    const int W = head_window_of(p, h);

    const int64_t q0 = (int64_t)qtile * SK_ROWS;
    const int64_t qlast = (q0 + SK_ROWS < Nq ? q0 + SK_ROWS : Nq) - 1;
    int64_t lo_first, hi_first, lo_last, hi_last;
    key_bounds(q0 + off, Nk, p.causal, W, lo_first, hi_first);
    key_bounds(qlast + off, Nk, p.causal, W, lo_last, hi_last);
    const int64_t kbeg = lo_first, kend = hi_last > lo_first ? hi_last : lo_first;
    // This wave's keys: a quarter of [kbeg, kend) in whole steps.
    const int64_t chunk = (((kend - kbeg) + SK_WAVES - 1) / SK_WAVES + SK_STEP - 1) / SK_STEP * SK_STEP;
    int64_t wbeg = kbeg + w * chunk, wend = wbeg + chunk;
    if (wbeg > kend) wbeg = kend;
    if (wend > kend) wend = kend;
    const int nsteps = (int)((wend - wbeg + SK_STEP - 1) / SK_STEP);

    const uint16_t *Q = static_cast<const uint16_t *>(p.q) + ((int64_t)b * p.H + h) * Nq * D;
    const uint16_t *K = static_cast<const uint16_t *>(p.k) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;
    const uint32_t head_bytes = (uint32_t)(Nk * D * 2);

    // Q^T operands: lane l holds row q0 + l % 32, dims 16 ds + 8 hf .. +7.
    bf16x8 qf[D / 16];
    {
        const int64_t qrow = q0 + l32;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qrow < Nq) x = *reinterpret_cast<const u32x4 *>(Q + qrow * D + ds * 16 + hf * 8);
            qf[ds] = __builtin_bit_cast(bf16x8, x);
        }
    }
    const float c_log2 = p.scale * kLog2e;
    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
    float m = kNegInf, l = 0.0f;  // running maximum (log2 units); this lane's half of the normaliser
    int64_t rlo, rhi;             // this lane's row's visible keys
    key_bounds(q0 + l32 + off, Nk, p.causal, W, rlo, rhi);

    char *const wl = lds + w * SL::WAVE_BYTES;
    const uint32_t wl_at = (uint32_t)reinterpret_cast<uintptr_t>((lds_void *)lds) + (uint32_t)(w * SL::WAVE_BYTES);

    // K operands of a step: lane l holds key k0 + l % 32, dims 16 ds + 8 hf
    // .. +7.  Buffer loads: keys past the end of the head read as zero (the
    // scalar offset counts toward the range check), and no lane branches.
    // K rows k0 .. k0 + 31 into K slot `slot`: load u fills slot bytes
    // 1024 u + 16 lane, i.e. row r = (1024 u + 16 lane) / (2 D) and chunk
    // slot sl, which holds chunk sl ^ swizzle(r) of the row.
    auto load_k = [&](int64_t k0, int slot) {
#pragma unroll
        for (int u = 0; u < SL::LOADS; ++u) {
            const int b = 1024 * u + 16 * lane;
            const int r = b / SL::ROW_BYTES, sl = (b % SL::ROW_BYTES) / 16;
            buffer_load_lds16_at(K, head_bytes, wl_at + (uint32_t)(slot * SL::VBUF + 1024 * u),
                                 r * SL::ROW_BYTES + 16 * SL::kslot(r, sl), (uint32_t)(k0 * (D * 2)));
        }
    };
    // V rows k0 .. k0 + 31 into buffer slot, row-major (16-byte chunk c of
    // the step at byte 16 c); rows past the end of the head read as zero.
    auto load_v = [&](int64_t k0, int slot) {
#pragma unroll
        for (int u = 0; u < SL::LOADS; ++u) {
            const int c = 64 * u + lane;
            buffer_load_lds16_at(V, head_bytes, wl_at + (uint32_t)((SL::SLOTS + slot) * SL::VBUF + 1024 * u), c * 16,
                                 (uint32_t)(k0 * (D * 2)));
        }
    };

    // Step t computes with K and V in slot t % 2 and then refills that
    // slot with step t + 2; step t + 1's loads stay in flight meanwhile.
    auto step = [&](int t) {
        const int64_t k0 = wbeg + (int64_t)t * SK_STEP;
        const int slot = t & 1;
        if (t + 1 < nsteps)
            __builtin_amdgcn_s_waitcnt(kV1);  // step t's loads, not step t + 1's
        else
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        // S^T = K Q^T: key 8 (j / 4) + 4 hf + j % 4 of the step, row l % 32.
        f32x16 s = {};
        const char *kb = wl + slot * SL::VBUF;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(kb + l32 * SL::ROW_BYTES + 16 * SL::kslot(l32, 2 * ds + hf));
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ds], s, 0, 0, 0);
        }
        // Scale / soft-cap into log2 units; masks unless every row sees the
        // whole step (element j is key 8 (j / 4) + j % 4 + 4 hf of the step).
#pragma unroll
        for (int j = 0; j < 16; ++j)
            s[j] = EXPLICIT ? (CAP ? softcap_log2(s[j] * p.scale, p.softcap) : s[j] * c_log2) : s[j] * c_log2;
        const int64_t base = rlo - k0 - 4 * hf, top = rhi - k0 - 4 * hf;
        if (__builtin_amdgcn_ballot_w64(!(base <= 0 && top >= 28)) != 0) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int c = 8 * (j / 4) + (j % 4);
                if (!(c >= base && c < top)) s[j] = kNegInf;
            }
        }
        // Lazy reference maximum: it moves (and O, l are rescaled) only when
        // a weight against it would exceed 2^TAU; weights stay in fp32 range.
        const float x = sk_max16(s);
        if (__builtin_amdgcn_ballot_w64(x - m > kSkTau) != 0) {
            const float m_new = fmaxf(m, row_max(x));
            const float alpha = fast_exp2(m - (m_new == kNegInf ? 0.0f : m_new));  // 0 while m is -inf
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        }
        const float m_use = m == kNegInf ? 0.0f : m;
#pragma unroll
        for (int j = 0; j < 16; ++j) s[j] = fast_exp2(s[j] - m_use);
        float r4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) r4[q] = (s[4 * q] + s[4 * q + 1]) + (s[4 * q + 2] + s[4 * q + 3]);
        l += (r4[0] + r4[1]) + (r4[2] + r4[3]);
        // P^T operands of the two 16-key k-steps, in the accumulator's key order.
        u32x4 pk[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) pk[ks][e] = pack_bf16x2(s[8 * ks + 2 * e], s[8 * ks + 2 * e + 1]);
        // O^T += V^T P^T.  Transposing read: in lane group gq = l / 16, lane
        // i = 4 e + jj addresses key row 16 ks + 8 rd + 4 (gq / 2) + e, dims
        // 32 db + 16 (gq % 2) + 4 jj .. +3, and receives dim 32 db + 16 (gq %
        // 2) + i of the group's 4 keys: rd = 0 gives keys 4 hf + [0, 4) of
        // the k-step, rd = 1 keys 8 + 4 hf + [0, 4), the order of pk.
        const char *vb = wl + (SL::SLOTS + slot) * SL::VBUF;
        const int gq = lane >> 4, e = (lane >> 2) & 3, jj = lane & 3;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int row = 16 * ks + 4 * (gq >> 1) + e;
                const char *ad = vb + row * SL::ROW_BYTES + (32 * db + 16 * (gq & 1) + 4 * jj) * 2;
                const sk_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((sk_lds_i16x4 *)ad);
                const sk_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((sk_lds_i16x4 *)(ad + 8 * SL::ROW_BYTES));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                   __builtin_bit_cast(bf16x8, pk[ks]), oacc[db], 0, 0,
                                                                   0);
            }
        // The slot read here is refilled with step t + 2: its reads must land first.
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        if (t + 2 < nsteps) {
            load_k(k0 + 2 * SK_STEP, slot);
            load_v(k0 + 2 * SK_STEP, slot);
        }
    };
    if (nsteps > 0) {
        load_k(wbeg, 0);
        load_v(wbeg, 0);
    }
    if (nsteps > 1) {
        load_k(wbeg + SK_STEP, 1);
        load_v(wbeg + SK_STEP, 1);
    }
    for (int t = 0; t < nsteps; ++t) step(t);

    // ---- merge the waves' (m, l, O) through LDS.  Each wave writes its
    // partial into its own staging region (its last step waited for its
    // reads of it), so one barrier suffices.
    const float lr = row_sum(l);
    {
        float *const po = reinterpret_cast<float *>(wl);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v4 = {oacc[db][4 * q], oacc[db][4 * q + 1], oacc[db][4 * q + 2], oacc[db][4 * q + 3]};
                *reinterpret_cast<f32x4 *>(po + l32 * D + 32 * db + 8 * q + 4 * hf) = v4;
            }
        if (hf == 0) {
            po[SK_ROWS * D + l32] = m;
            po[SK_ROWS * D + SK_ROWS + l32] = lr;
        }
    }
    __syncthreads();
    // Wave ww's partial: O at part(ww), m at part(ww) + 32 D, l after m.
    auto part = [&](int ww) { return reinterpret_cast<const float *>(lds + ww * SL::WAVE_BYTES); };
    // 32 rows x D/4 groups of 4 dims over the workgroup's threads.
    for (int item = tid; item < SK_ROWS * (D / 4); item += 64 * SK_WAVES) {
        const int r = item / (D / 4), c4 = item % (D / 4);
        const int64_t qrow = q0 + r;
        if (qrow >= Nq) continue;
        float mx = kNegInf;
#pragma unroll
        for (int ww = 0; ww < SK_WAVES; ++ww) mx = fmaxf(mx, part(ww)[SK_ROWS * D + r]);
        float den = 0.0f;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (mx != kNegInf) {
#pragma unroll
            for (int ww = 0; ww < SK_WAVES; ++ww) {
                const float *pw = part(ww);
                const float f = fast_exp2(pw[SK_ROWS * D + r] - mx);  // 0 for a wave that saw no key
                den += f * pw[SK_ROWS * D + SK_ROWS + r];
                const f32x4 o4 = *reinterpret_cast<const f32x4 *>(pw + r * D + 4 * c4);
                acc += f * o4;
            }
        }
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
        const int64_t row = ((int64_t)b * p.H + h) * Nq + qrow;
        uint16_t *O = static_cast<uint16_t *>(p.o) + row * D + 4 * c4;
        const u32x2 x = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        *reinterpret_cast<u32x2 *>(O) = x;
        if (c4 == 0 && p.lse) p.lse[row] = den > 0.0f ? (mx + __log2f(den)) * kLn2 : kNegInf;
    }
}

template <int D, bool EXPLICIT, bool CAP>
int launch(const FwdParams &p, hipStream_t stream) {
    const int n_qtiles = (int)((p.Nq + SK_ROWS - 1) / SK_ROWS);
    const int64_t blocks = p.B * p.H * (int64_t)n_qtiles;
    if (blocks <= 0) return FA_OK;
    if (blocks > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((fwd_bf16_splitk_kernel<D, EXPLICIT, CAP>), dim3((unsigned)blocks), dim3(64 * sk_waves<D>()), 0,
                       stream, p, n_qtiles);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int D>
int launch_d(const FwdParams &p, hipStream_t stream) {
    if (p.softcap > 0.0f) return launch<D, true, true>(p, stream);
    if (!(p.scale > 0.0f)) return launch<D, true, false>(p, stream);
    return launch<D, false, false>(p, stream);
}

}  // namespace

// Whether a bf16 unsplit launch is better served by 4 waves per 32 query
// rows with the keys split among them: the 128-row workgroups of the tiled
// kernel would leave CUs idle, and there are keys enough for four waves.
bool fwd_bf16_splitk_applies(const FwdParams &p, int d) {
    if (d != 32 && d != 64 && d != 128) return false;
    const int64_t tiles128 = p.B * p.H * ((p.Nq + 127) / 128);
    return tiles128 < 256 && p.Nk >= 4 * 64;
}

int launch_fwd_bf16_splitk(const FwdParams &p, int d, hipStream_t stream) {
    switch (d) {
        case 32: return launch_d<32>(p, stream);
        case 64: return launch_d<64>(p, stream);
        case 128: return launch_d<128>(p, stream);
        default: return FA_ERR_UNSUPPORTED;
    }
}

}  // namespace fa
