// fa_fwd_fp8.hip -- tiled forward attention with an online softmax on fp8
// (OCP E4M3) Q, K and V: both contractions on the gfx950 fp8 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, 64-deep k-steps), the softmax state (running
// maximum, normaliser, output) in fp32.
//
// The method is the one of the bf16 kernel (Transformers & Math, Module 16,
// sections 16.1 and 16.2); the low-precision variant follows the idea of
// running both products of the attention loop in a narrow format while the
// online-softmax state stays wider (HiFA4, abstract: 4-bit operands on
// Ascend; here the narrowest format gfx950 multiplies at full density for
// attention, 8-bit).
//
// What is rounded: the caller's Q, K, V are already e4m3 with one fp32
// descale factor per tensor.  Products of e4m3 values are exact; the fp8
// instruction adds them in groups of 8 in a fixed-point window about 13 bits
// below each group's largest product and adds the group sums in fp32, so a
// score is exact when its products lie within 2^6 of one another and off by
// at most 2^-10 of the sum of |products| otherwise (measured on MI355X).
// The weights p = 2^(t - m) of a tile are rounded to e4m3 for the
// P.V product after a shift by 2^P_SHIFT, which keeps weights down to
// 2^-(P_SHIFT + 6) of the reference maximum in e4m3's normal range (3
// mantissa bits, relative error <= 2^-4).  The row sum l is taken from the
// fp32 weights before rounding, so lse is accurate to fp32; O is the P.V sum
// divided by l.
//
// Tiling as in the bf16 kernel: 8 waves, 32 query rows each, 64-key tiles
// through LDS, S^T = K Q^T and O^T += V^T P^T so every lane owns one query
// row, ping-pong between a matrix phase and a vector phase on the two waves
// of each SIMD.  What changes for one-byte elements:
//   * an MFMA consumes 32 bytes of each operand per lane; for S^T a lane
//     reads 32 consecutive bytes of a K row (two ds_read_b128) and holds the
//     same 32 columns of its Q row;
//   * the two 32-key halves of a tile's score accumulator, rounded to e4m3,
//     are exactly one 64-key P^T operand (8 dwords): byte e of half hf is key
//     32*(e/16) + 8*((e%16)/4) + 4*hf + e%4; the V^T tile stores each row's
//     64 keys in that order, so a V^T operand is again two ds_read_b128;
//   * V^T is built with byte permutes: each loading wave owns D/4 columns of
//     V for all 64 keys, loads them (direct to LDS) into a region laid out
//     so that its transposing reads are conflict-free, and turns every 4x4
//     byte block (4 keys x 4 columns) into 4 V^T dwords with 8 v_perm_b32;
//   * the lazy-rescale threshold is small (TAU = 1.5): weights stay below
//     2^(TAU + P_SHIFT) = 2^8.5, inside e4m3's range (largest value 448);
//   * with half the matrix work of bf16 per tile, the vector phase (its
//     exps issue at a quarter of the VALU rate) is the longer one, so it
//     holds only the mask, the maximum and the exps: the fp32 weights are
//     summed and rounded to E4M3 in the next matrix phase, while the P.V
//     MFMAs run.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_tile.h"

namespace fa {

namespace {

// Selects the masked or the unmasked softmax of a step at compile time.
template <bool B>
struct MaskTag {
    static constexpr bool value = B;
};

constexpr int NW = 8;        // waves per workgroup (two per SIMD)
constexpr int BM = NW * 32;  // query rows per workgroup
constexpr int BN = 64;       // keys per tile
constexpr int NT = 64 * NW;  // threads per workgroup
constexpr int LOADERS = 4;   // waves that issue the tile loads
constexpr float TAU = 1.5f;  // lazy-rescale threshold, log2 units
constexpr float P_SHIFT = 7.0f;
static_assert(TAU + P_SHIFT <= 8.8f, "weights must stay below e4m3's largest value, 448 = 2^8.8");

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int D>
struct Lay8 {
    static constexpr int CPR = D / 16;                     // 16-byte chunks per K/V row
    static constexpr int TILE = BN * D;                    // bytes of a K, V or V^T tile
    static constexpr int CPW = CPR / LOADERS;              // V chunks (columns / 16) per loading wave
    static constexpr int LPW = TILE / 16 / 64 / LOADERS;   // 16-byte loads per lane per tile
    static_assert(LPW == CPW, "one load per owned V chunk");
    static constexpr int RPL_LOG2 = D == 128 ? 1 : 2;      // log2(K rows per 256-byte bank line)
    // K: row-major, chunk c of row r in slot c ^ ((r / rows-per-line) % CPR):
    // the 16 rows one 16-lane pass of a ds_read_b128 reads land on 16
    // distinct 16-byte bank groups.
    __device__ static int kslot(int r, int c) { return c ^ ((r >> RPL_LOG2) & (CPR - 1)); }
    // V^T: D rows of 64 permuted keys; four rows share a bank line, so the
    // chunk is xor-ed with bits 2..3 of the row.
    static constexpr int VT_ROW = BN;
    __device__ static int vtslot(int d, int c) { return c ^ ((d >> 2) & 3); }
};

// MFMAs that take R operand reads each: AHEAD MFMAs' worth of reads first,
// then one MFMA and the reads of a later one, alternating.
template <int NMFMA, int R, int AHEAD>
__device__ __forceinline__ void sched_reads_per_mfma() {
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * R, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < NMFMA - AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

__device__ __forceinline__ i32x8 join(u32x4 a, u32x4 b) {
    i32x8 r;
    r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
    r[4] = (int)b[0]; r[5] = (int)b[1]; r[6] = (int)b[2]; r[7] = (int)b[3];
    return r;
}

// fp8 x fp8 -> fp32 32x32x64 product, both operands E4M3 (format code 0),
// no block scaling.
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max16v(const f32x16 &s) {
    const float a = vmax3(s[0], s[1], s[2]), b = vmax3(s[3], s[4], s[5]), c = vmax3(s[6], s[7], s[8]);
    const float d = vmax3(s[9], s[10], s[11]), e = vmax3(s[12], s[13], s[14]);
    return vmax3(vmax3(a, b, c), vmax3(d, e, s[15]), a);
}

template <int D>
struct Wave8 {
    using L = Lay8<D>;
    static constexpr int NDS = D / 64;  // 64-deep k-steps of the score product
    i32x8 qf[NDS];                      // Q^T operand
    f32x16 oacc[D / 32];                // O^T accumulators
    float m;                            // lazy reference maximum (log2 units)
    float l;                            // this lane's half of the fp32 weight sum
    int lo_rel, hi_rel;                 // visible keys relative to the first tile
    int koff[NDS][2];                   // K operand read offsets (bytes)
    int vko[2];                         // V^T operand read offsets (bytes)
    int hf;
    float c_log2;

    // S^T = K Q^T for the 64 keys of a tile (two 32-key halves).
    __device__ __forceinline__ void scores(const uint8_t *kbuf, f32x16 (&sacc)[2]) const {
        const char *Kb = reinterpret_cast<const char *>(kbuf);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                const u32x4 a0 = *reinterpret_cast<const u32x4 *>(Kb + kb * 32 * D + koff[ds][0]);
                const u32x4 a1 = *reinterpret_cast<const u32x4 *>(Kb + kb * 32 * D + koff[ds][1]);
                sacc[kb] = mfma_fp8(join(a0, a1), qf[ds], sacc[kb]);
            }
        sched_reads_per_mfma<2 * NDS, 2, 2>();
    }

    // Online softmax of one tile: mask (if MASK), row maximum, lazy move of
    // the reference maximum (returns whether any row of the wave moved, and
    // the factor), fp32 weights 2^(t - m + P_SHIFT) summed into l and
    // rounded to e4m3 as the P^T operand.
    template <bool MASK>
    __device__ __forceinline__ bool softmax(f32x16 (&sacc)[2], int it, f32x16 (&pw)[2], float &alpha) {
        if (MASK) {
            // Key ko = c + 4*hf of the tile is visible iff lo <= ko < hi.
            const int lo = lo_rel - it * BN, hi = hi_rel - it * BN;
            const int base = lo - 4 * hf;
            const uint32_t span = (uint32_t)(hi - lo);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int c = kb * 32 + 8 * (j / 4) + (j % 4);
                    if (!((uint32_t)(c - base) < span)) sacc[kb][j] = kNegInf;
                }
        }
        const float x = vmax3(max16v(sacc[0]), max16v(sacc[1]), sacc[0][0]);
        const float mt = row_max(x * c_log2);
        const bool move = __builtin_amdgcn_ballot_w64(mt > m + TAU) != 0;
        const float m_new = move ? fmaxf(m, mt) : m;
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        alpha = fast_exp2(m - m_use);
        m = m_new;
        const float bias = P_SHIFT - m_use;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) pw[kb][j] = fast_exp2(fmaf(sacc[kb][j], c_log2, bias));
        // Their sum and E4M3 rounding are left to the next matrix phase (pv).
        l *= alpha;
        return move;
    }

    __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
    }

    // O^T += V^T P^T: row db*32 + lane%32 of V^T, permuted keys 32*hf + [0,
    // 32).  The weights pw (fp32) are rounded to E4M3 here (byte e of the
    // operand is element e % 16 of half e / 16), and their fp32 sum is added
    // to l while the MFMAs run.
    __device__ __forceinline__ void pv(const uint8_t *vt, const f32x16 (&pw)[2]) {
        const char *Vb = reinterpret_cast<const char *>(vt);
        i32x8 pf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int lo2 = __builtin_amdgcn_cvt_pk_fp8_f32(pw[kb][4 * q], pw[kb][4 * q + 1], 0, false);
                pf[4 * kb + q] = __builtin_amdgcn_cvt_pk_fp8_f32(pw[kb][4 * q + 2], pw[kb][4 * q + 3], lo2, true);
            }
        float rs[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            rs[i] = (pw[i / 4][4 * (i % 4)] + pw[i / 4][4 * (i % 4) + 1]) +
                    (pw[i / 4][4 * (i % 4) + 2] + pw[i / 4][4 * (i % 4) + 3]);
        l += ((rs[0] + rs[1]) + (rs[2] + rs[3])) + ((rs[4] + rs[5]) + (rs[6] + rs[7]));
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const u32x4 a0 = *reinterpret_cast<const u32x4 *>(Vb + db * 32 * L::VT_ROW + vko[0]);
            const u32x4 a1 = *reinterpret_cast<const u32x4 *>(Vb + db * 32 * L::VT_ROW + vko[1]);
            oacc[db] = mfma_fp8(join(a0, a1), pf, oacc[db]);
        }
        sched_reads_per_mfma<D / 32, 2, 2>();
    }
};

// c_log2: scale * q_descale * k_descale * log2(e), > 0 (the host folds a
// negative product into qflip, which flips the sign bit of every Q byte).
// out_scale: v_descale, applied with 1/l in the epilogue.
template <int D>
__global__ __launch_bounds__(NT, 1) void fwd_fp8_kernel(const FwdParams p, const int n_qtiles, const float c_log2,
                                                        const float out_scale, const uint32_t qflip) {
    using L = Lay8<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[L::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[L::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t vstage[L::TILE];  // V as loaded, one region per loader
    __shared__ __attribute__((aligned(1024))) uint8_t vt0[L::TILE];     // V^T, permuted keys
    __shared__ __attribute__((aligned(1024))) uint8_t vt1[L::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool leader = wave < LOADERS;
    const int l32 = lane & 31, hf = lane >> 5;
    const Work w = decode_block(p, n_qtiles);
    const int h = w.h, b = w.b;
    const int g = h / p.group;
    const int64_t Nq = p.Nq, Nk = p.Nk;
    const int64_t off = Nk - Nq;
    const int W = head_window_of(p, h);

    const int64_t q0 = (int64_t)w.qtile * BM;
    const int64_t qlast = (q0 + BM < Nq ? q0 + BM : Nq) - 1;
    int64_t kbeg, hi_first, lo_last, kend;
    key_bounds(q0 + off, Nk, p.causal, W, kbeg, hi_first);
    key_bounds(qlast + off, Nk, p.causal, W, lo_last, kend);
    const int64_t full_lo = lo_last, full_hi = hi_first;  // keys every row of the block sees

    const uint8_t *Q = static_cast<const uint8_t *>(p.q) + ((int64_t)b * p.H + h) * Nq * D;
    const uint8_t *K = static_cast<const uint8_t *>(p.k) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;
    const uint8_t *V = static_cast<const uint8_t *>(p.v) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;

    Wave8<D> st;
    st.hf = hf;
    st.c_log2 = c_log2;
    const int64_t qrow = q0 + wave * 32 + l32;
    {
        int64_t lo, hi;
        key_bounds(qrow + off, Nk, p.causal, W, lo, hi);
        lo -= kbeg;
        hi -= kbeg;
        if (hi < lo) hi = lo;  // empty interval: the mask's unsigned span stays 0
        st.lo_rel = (int)(lo < -1 ? -1 : (lo > 0x3fffffff ? 0x3fffffff : lo));
        st.hi_rel = (int)(hi < -1 ? -1 : (hi > 0x3fffffff ? 0x3fffffff : hi));
        // Q^T operand of k-step ds: bytes 64*ds + 32*hf + [0, 32) of this row.
#pragma unroll
        for (int ds = 0; ds < Wave8<D>::NDS; ++ds) {
            u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
            if (qrow < Nq) {
                x0 = *reinterpret_cast<const u32x4 *>(Q + qrow * D + 64 * ds + 32 * hf);
                x1 = *reinterpret_cast<const u32x4 *>(Q + qrow * D + 64 * ds + 32 * hf + 16);
            }
            st.qf[ds] = join(x0 ^ qflip, x1 ^ qflip);
        }
        st.m = kNegInf;
        st.l = 0.0f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) st.oacc[db][j] = 0.0f;
    }
    // K operand reads: row kb*32 + l32 (the swizzle is the same for both
    // halves), chunks 4*ds + 2*hf + t.
#pragma unroll
    for (int ds = 0; ds < Wave8<D>::NDS; ++ds)
#pragma unroll
        for (int t = 0; t < 2; ++t) st.koff[ds][t] = l32 * D + L::kslot(l32, 4 * ds + 2 * hf + t) * 16;
    // V^T operand reads: row db*32 + l32, chunks 2*hf + t.
#pragma unroll
    for (int t = 0; t < 2; ++t) st.vko[t] = l32 * L::VT_ROW + L::vtslot(l32, 2 * hf + t) * 16;

    // V staging: loading wave lw owns columns [16*CPW*lw, 16*CPW*(lw+1)) of
    // all 64 keys, in a region of 4*CPW bank lines: chunk cl of key row R
    // sits in line (R % 4)*CPW + cl, 16-byte group R / 4.  A transposing
    // read (fixed R % 4 and cl) then touches one line, 64 distinct banks.
    const int lw = leader ? wave : 0;
    int k_goff[L::LPW], v_goff[L::LPW];
#pragma unroll
    for (int u = 0; u < L::LPW; ++u) {
        const int pos = (lw * L::LPW + u) * 64 + lane;
        const int rr = pos / L::CPR, sl = pos % L::CPR;
        k_goff[u] = rr * D + L::kslot(rr, sl) * 16;
        const int line = 4 * u + (lane >> 4);
        const int R = 4 * (lane & 15) + line / L::CPW, cl = line % L::CPW;
        v_goff[u] = R * D + (lw * L::CPW + cl) * 16;
    }
    // Transposition: lane (kg = lane % 16, gi = lane / 16) takes, for each
    // owned chunk b, keys 4*kg + [0, 4) x columns 4*dg + [0, 4) with dg =
    // 4*(CPW*lw + b) + gi, and writes V^T rows 4*dg + (j ^ gi) (j = 0..3:
    // the rotation by gi spreads the four 16-lane groups of one write over
    // the four quarters of a bank line) at key group kg's dword, which is
    // ((kg % 2) << 3) | (kg / 2) in the permuted key order.
    const int kg = lane & 15, gi = lane >> 4;
    const int tr_src = lw * L::CPW * 1024 + kg * 16 + gi * 4;
    int tr_dst[L::CPW][4];
    {
        const int qd = ((kg & 1) << 3) | (kg >> 1);
#pragma unroll
        for (int bb = 0; bb < L::CPW; ++bb) {
            const int dg = 4 * (L::CPW * lw + bb) + gi;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rho = 4 * dg + (j ^ gi);
                tr_dst[bb][j] = rho * L::VT_ROW + L::vtslot(rho, qd >> 2) * 16 + (qd & 3) * 4;
            }
        }
    }
    // Byte selectors of the first permute stage: columns x = k ^ gi.
    const uint32_t c0 = 0 ^ gi, c1 = 1 ^ gi, c2 = 2 ^ gi, c3 = 3 ^ gi;
    const uint32_t sel_lo = c0 | ((4 + c0) << 8) | (c1 << 16) | ((4 + c1) << 24);
    const uint32_t sel_hi = c2 | ((4 + c2) << 8) | (c3 << 16) | ((4 + c3) << 24);

    const uint32_t head_bytes = (uint32_t)(Nk * D);
    const int ntiles = kend > kbeg ? (int)((kend - kbeg + BN - 1) / BN) : 0;
    const int kt0 = (int)kbeg;

    auto load_k = [&](int t, uint8_t *buf) {
        const uint32_t toff = (uint32_t)(kt0 + t * BN) * (uint32_t)D;
#pragma unroll
        for (int u = 0; u < L::LPW; ++u)
            buffer_load_lds16(K, head_bytes, (lds_void *)(buf + (lw * L::LPW + u) * 1024), k_goff[u], toff);
    };
    auto load_v = [&](int t) {
        const uint32_t toff = (uint32_t)(kt0 + t * BN) * (uint32_t)D;
#pragma unroll
        for (int u = 0; u < L::LPW; ++u)
            buffer_load_lds16(V, head_bytes, (lds_void *)(vstage + (lw * L::LPW + u) * 1024), v_goff[u], toff);
    };
    // This loading wave's region of the staged V tile -> V^T tile vt (only
    // its own loads are read, so its own wait suffices).
    auto transpose_v = [&](uint8_t *vt) {
        const char *src = reinterpret_cast<const char *>(vstage) + tr_src;
        char *dst = reinterpret_cast<char *>(vt);
#pragma unroll
        for (int bb = 0; bb < L::CPW; ++bb) {
            uint32_t r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = *reinterpret_cast<const uint32_t *>(src + (i * L::CPW + bb) * 256);
            const uint32_t t01l = __builtin_amdgcn_perm(r[1], r[0], sel_lo);
            const uint32_t t01h = __builtin_amdgcn_perm(r[1], r[0], sel_hi);
            const uint32_t t23l = __builtin_amdgcn_perm(r[3], r[2], sel_lo);
            const uint32_t t23h = __builtin_amdgcn_perm(r[3], r[2], sel_hi);
            *reinterpret_cast<uint32_t *>(dst + tr_dst[bb][0]) = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
            *reinterpret_cast<uint32_t *>(dst + tr_dst[bb][1]) = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
            *reinterpret_cast<uint32_t *>(dst + tr_dst[bb][2]) = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
            *reinterpret_cast<uint32_t *>(dst + tr_dst[bb][3]) = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
        }
    };

    f32x16 sacc[2];
    f32x16 pw[2];  // fp32 weights of the tile whose P.V is next
    // Step j: matrix phase (loads of K_{j+1} and V_j by the leaders, scores
    // of tile j, P.V of tile j-1 with the sum and rounding of its weights),
    // barrier, vector phase (mask, maximum and exps of tile j; the leaders
    // then wait for their loads and transpose their part of V_j), barrier.
    // Waves 4..7 run one phase behind waves 0..3.
    auto step = [&](auto mask, int j, const uint8_t *kcur, const uint8_t *vtprev, uint8_t *knext,
                    uint8_t *vtcur) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask)::value;
        if (leader) {
            if (j + 1 < ntiles) load_k(j + 1, knext);
            if (j < ntiles) load_v(j);
        }
        if (j < ntiles) st.scores(kcur, sacc);
        if (j >= 1) st.pv(vtprev, pw);
        lds_barrier();
        if (j < ntiles) {
            float alpha;
            const bool move = st.template softmax<MASK>(sacc, j, pw, alpha);
            if (move) st.rescale(alpha);
        }
        if (leader) {
            __builtin_amdgcn_s_waitcnt(0);
            if (j < ntiles) transpose_v(vtcur);
        }
        lds_barrier();
    };

    if (leader && ntiles > 0) load_k(0, kbuf0);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (!leader) lds_barrier();
    // Tiles [t_a, t_b) are seen in full by every row of the block (tile t
    // starts at key kbeg + 64 t); the others need the mask.  One loop per
    // kind keeps the masked/unmasked choice out of the loop body: a branch
    // there makes the two softmax variants merge their registers, which
    // costs about 50 VGPRs and copies.
    const int t_a = min(ntiles, (int)((full_lo - kbeg + BN - 1) / BN));
    const int t_b = max(t_a, min(ntiles, (int)((full_hi - kbeg) / BN)));
    // Steps j0 .. j1-1; tile j's K sits in kbuf[j % 2], its V^T in vt[j % 2].
    auto run = [&](auto mask, int j0, int j1) __attribute__((always_inline)) {
        int j = j0;
        if (j < j1 && (j & 1)) {
            step(mask, j, kbuf1, vt0, kbuf0, vt1);
            ++j;
        }
        for (; j + 1 < j1; j += 2) {
            step(mask, j, kbuf0, vt1, kbuf1, vt0);
            step(mask, j + 1, kbuf1, vt0, kbuf0, vt1);
        }
        if (j < j1) step(mask, j, kbuf0, vt1, kbuf1, vt0);
    };
    run(MaskTag<true>(), 0, t_a);
    run(MaskTag<false>(), t_a, t_b);
    run(MaskTag<true>(), t_b, ntiles);
    // last step: P.V of the last tile only
    if (ntiles & 1) step(MaskTag<false>(), ntiles, kbuf1, vt0, kbuf0, vt1);
    else step(MaskTag<false>(), ntiles, kbuf0, vt1, kbuf1, vt0);
    if (leader) lds_barrier();

    // ---- epilogue: O = v_descale * acc / l.  Lane holds dims db*32 +
    // 8*(j/4) + 4*hf + (j%4) of its query row.
    const float lr = row_sum(st.l);
    if (qrow >= Nq) return;
    const float inv = lr > 0.0f ? out_scale / lr : 0.0f;
    const int64_t row = ((int64_t)b * p.H + h) * Nq + qrow;
    uint16_t *O = static_cast<uint16_t *>(p.o) + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            u32x2 x = {pack_bf16x2(st.oacc[db][4 * gq] * inv, st.oacc[db][4 * gq + 1] * inv),
                       pack_bf16x2(st.oacc[db][4 * gq + 2] * inv, st.oacc[db][4 * gq + 3] * inv)};
            *reinterpret_cast<u32x2 *>(O + db * 32 + 8 * gq + 4 * hf) = x;
        }
    if (p.lse && hf == 0) p.lse[row] = lr > 0.0f ? (st.m + __log2f(lr) - P_SHIFT) * kLn2 : kNegInf;
}

template <int D>
int launch_d(const FwdParams &p, float c_log2, float out_scale, uint32_t qflip, hipStream_t stream) {
    const int n_qtiles = (int)((p.Nq + BM - 1) / BM);
    const int64_t blocks = p.B * p.H * (int64_t)n_qtiles;
    if (blocks <= 0) return FA_OK;
    if (blocks > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((fwd_fp8_kernel<D>), dim3((unsigned)blocks), dim3(NT), 0, stream, p, n_qtiles, c_log2,
                       out_scale, qflip);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

int launch_fwd_fp8(const FwdParams &p, int d, float c_log2, float out_scale, uint32_t qflip, hipStream_t stream) {
    switch (d) {
        case 64: return launch_d<64>(p, c_log2, out_scale, qflip, stream);
        case 128: return launch_d<128>(p, c_log2, out_scale, qflip, stream);
        default: return FA_ERR_UNSUPPORTED;
    }
}

}  // namespace fa
