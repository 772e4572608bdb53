// fa_fwd_bf16_wide.hip -- bf16 tiled forward attention, d = 128, with 64
// query rows per wave: every LDS operand read feeds two MFMAs.
//
// The method is the one of fa_fwd_bf16.hip (Transformers & Math, Module 16,
// section 16.1 flow and 16.2 merge rule): a block of query rows stays on
// chip, K and V stream through LDS in tiles, each row keeps a running
// maximum, normaliser and unnormalised output, and O is written once.
//
// What differs is the shape of a wave's work.  With 32 query rows per wave
// a 32x32x16 MFMA (32 cycles) needs its own 1 KiB operand read from LDS,
// about what one wave can draw from LDS in that time.  Here a wave owns 64
// rows (two 32-row blocks): each K or V^T operand read serves both blocks,
// so a wave reads 16 KiB per 32 MFMAs instead of 32 KiB.  The price is
// registers: the O^T accumulators (128), the Q^T operands (64) and one
// 32-key score block (32) leave room for two waves per SIMD only if a wave
// processes each 64-key tile as two halves of 32 keys, and keeps its
// lane-dependent LDS and load offsets out of registers (recomputed per use).
//
// A group is 4 waves on one block of 256 query rows of one (batch, head)
// with its own K and V tiles in LDS (64 KiB).  Each wave alternates a
// matrix phase (P.V of the previous 32-key half, then the scores of the
// next one; MFMA and LDS reads only) and a vector phase (masks, exp2, row
// sum, bf16 packing), with workgroup barriers between phases (see the tile
// step).  Two waves share each SIMD, in one of two workgroup forms
// (template parameter NG):
//   * NG = 1: a workgroup is one group, two workgroups per CU.  They run
//     independently; a workgroup that ends leaves the CU to the other one
//     while the next starts loading.  Used when every head sees the same
//     keys (no windows) and scores are not soft-capped.
//   * NG = 2: a workgroup is two groups (8 waves) taking two heads' blocks
//     with the same query tile; wave i of group 0 and wave i of group 1
//     share SIMD i and ping-pong (group 1 runs one phase behind), so the
//     roles swap at each workgroup barrier.  Faster where the vector phase
//     is long (soft-capped scores: a tanh per score) or where heads differ
//     in length (windows on some heads): the pairing puts heads of equal
//     length side by side.
// Unless scores are soft-capped, a wave raises its priority for its matrix
// phases: the vector work of the other wave on the SIMD then fills the
// gaps between MFMAs instead of delaying them (the older wave wins the
// issue arbitration otherwise).
// Within a group, K and V tiles go from HBM straight into LDS (direct
// loads by the group's 4 waves, 16 keys each), row-major
// with swizzles against bank conflicts (fa_bf16_tile.h); the V^T operand of
// P.V is read from the row-major V tile with transposing LDS reads, so V is
// never transposed or copied inside LDS.
//
// Layout of a wave's state (lane l, hf = l / 32, row block rb = 0, 1):
//   * S^T = K Q^T for a 32-key half: 32x32 accumulator per row block; lane
//     l holds query row 32 rb + l % 32 and keys 8 (i / 4) + 4 hf + i % 4,
//     i = 0..15 (the partner lane l ^ 32 holds the other 16 keys);
//   * O^T += V^T P^T: the accumulator elements 8 ks .. 8 ks + 7, rounded to
//     bf16, are the P^T operand of k-step ks, in the accumulator's own key
//     order (the transposing reads of V deliver the V^T operand in the same
//     order); lane l owns query row 32 rb + l % 32 of O^T and the dims 32 db
//     + 8 (i / 4) + 4 hf + i % 4.
#include "fa_bf16_tile.h"
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_tile.h"

#include <type_traits>

namespace fa {

namespace {

constexpr int D = 128;
constexpr int BN = kTileKeys;          // keys per LDS tile (64)
constexpr int HALF = 32;               // keys per compute step
constexpr int RW = 64;                 // query rows per wave
constexpr int BM = RW * kTileLoaders;  // query rows per group (256)
constexpr float TAU = 8.0f;            // lazy-rescale threshold, log2 units
constexpr float kFixedMaxCap = 60.0f;  // largest soft-cap with a fixed reference maximum
using L = BfTile<D>;

// LDS of one group, 16 KiB each: K tiles and V tiles, both double-buffered.
constexpr int GROUP_TILES = 4;
constexpr int TILE_BYTES = L::TILE * 2;
constexpr int KT0 = 0, VT0 = 2;

// The bf16 weights of a 32-key half are packed into the first 8 registers
// of that half's fp32 score accumulator (element 4 ks + e holds weights 8 ks
// + 2 e and 8 ks + 2 e + 1): scores and weights share one register block,
// which is what leaves room for operand reads in flight at 256 VGPRs.
__device__ __forceinline__ bf16x8 p_operand(const f32x16 &s, int ks) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(s[4 * ks + e]);
    return __builtin_bit_cast(bf16x8, w);
}

// Maximum of the 16 scores a lane holds for one row, with v_max3_f32 (the
// plain fmaxf chain adds a quieting max per input in IEEE mode).
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float max16(const f32x16 &s) {
    const float a = max3(s[0], s[1], s[2]), b = max3(s[3], s[4], s[5]), c = max3(s[6], s[7], s[8]);
    const float d = max3(s[9], s[10], s[11]), e = max3(s[12], s[13], s[14]);
    return max3(max3(a, b, c), max3(d, e, s[15]), a);
}

__device__ __forceinline__ void pack_weights(f32x16 &s) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * ks + e] = __uint_as_float(pack_bf16x2(s[8 * ks + 2 * e], s[8 * ks + 2 * e + 1]));
}

template <bool EXPLICIT, bool CAP, bool FIXED>
struct WideWave {
    bf16x8 qf[2][D / 16];       // Q^T operand per row block and 16-dim step
    f32x16 oacc[2][D / 32];     // O^T accumulators per row block and 32-dim block
    float m[2], l[2];           // reference maximum (log2 units); this lane's half of the normaliser
    float mu[2];                // the reference the weights are taken against (0 while m is -inf)
    float lx[2];                // FIXED: this lane's half of the sum of the fp32 weights (for lse)
    float c_log2, scale, softcap;
    float cap_c2, cap_kl, cap_nkl2;  // soft-cap constants (softcap_log2_pre)
    // Lane-dependent offsets and mask bounds are recomputed from the lane id
    // where they are used: only the accumulators, Q^T and the row state stay
    // in registers through the loop.

    // S^T of key half hh of the K tile at kt, both row blocks.  K row r =
    // 32 hh + l % 32, chunk c = 2 ds + hf sits at byte r * 256 + 16 * (c ^
    // (r % 16)); with r % 16 = l % 16 that is hh * 8192 + (ka ^ 32 ds), ka =
    // 256 (l % 32) + 16 (hf ^ (l % 16)).
    template <bool SCHED = true>
    __device__ __forceinline__ void scores(const char *kt, int hh, f32x16 (&s)[2]) const {
        const char *kb = kt + hh * (HALF * D * 2);
        int lane = lane_id();
        asm volatile("" : "+v"(lane));
        const uint32_t ka = (uint32_t)((lane & 31) * 256 + 16 * ((lane >> 5) ^ (lane & 15)));
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(kb + (ka ^ (uint32_t)(ds << 5)));
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const f32x16 acc = ds == 0 ? f32x16{} : s[rb];
                s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[rb][ds], acc, 0,
                                                                0, 0);
            }
        }
        if (SCHED) sched_read_mfma_pipeline<D / 16, 2, 2>();
    }

    // O^T += V^T P^T for key half hh of the V tile at vt (row-major, 256
    // bytes per key, chunk c of row r in slot c ^ 4 (r % 4)).  The V^T
    // operand of dim block db and k-step ks is two transposing reads
    // (ds_read_b64_tr_b16): in lane group g = l / 16, lane i = 4 e + jj
    // supplies the address of key row 16 ks + 8 rd + 4 (g / 2) + e, dims
    // 32 db + 16 (g % 2) + 4 jj .. +3, and receives dim 32 db + 16 (g % 2) +
    // i of the group's 4 keys: rd = 0 gives keys 4 hf + [0,4) of the k-step,
    // rd = 1 keys 8 + 4 hf + [0,4) -- the order in which the score
    // accumulator holds a lane's weights, so P needs no permutation.  With
    // the swizzle the byte address is row * 256 + 64 (db ^ e) + 32 (g % 2) +
    // 8 jj = (va ^ 64 db) + 256 (32 hh + 16 ks + 8 rd).
    template <bool SCHED = true>
    __device__ __forceinline__ void pv(const char *vt, int hh, const f32x16 (&p)[2]) {
        int lane = lane_id();
        asm volatile("" : "+v"(lane));
        const int g = lane >> 4, e = (lane >> 2) & 3, jj = lane & 3;
        const uint32_t va = (uint32_t)((4 * (g >> 1) + e) * 256 + 64 * e + 32 * (g & 1) + 8 * jj);
        const char *vb = vt + hh * (HALF * D * 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const char *ad = vb + (va ^ (uint32_t)(64 * db)) + ks * (16 * D * 2);
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)ad);
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(ad + 8 * D * 2));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    oacc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a), p_operand(p[rb], ks), oacc[rb][db], 0, 0, 0);
            }
        if (SCHED) sched_read_mfma_pipeline<D / 32 * 4, 1, 4>();
    }

    // A whole matrix phase in one scheduling region: P.V of the previous
    // half (weights in s) then the scores of the next half (into s).  16
    // transposing reads feeding one MFMA each, 8 issued ahead, then 8 K
    // reads feeding two, 4 ahead.
    __device__ __forceinline__ void pv_scores(const char *vt, int hh_pv, const char *kt, int hh_s, f32x16 (&s)[2]) {
        pv<false>(vt, hh_pv, s);
        scores<false>(kt, hh_s, s);
        sched_read_mfma_pipeline<D / 32 * 4, 1, 8>();
        sched_read_mfma_pipeline<D / 16, 2, 4>();
    }

    // FIXED: this lane's sum of its bf16 weights (dot2 with (1, 1)), which
    // normalises O; the partner lane's half is added in the epilogue.
    __device__ __forceinline__ void sum_bf16_weights(const f32x16 (&p)[2]) {
        const bf16x2 ones = as_bf16x2(0x3f803f80u);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float rs = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 w = __builtin_bit_cast(u32x4, p_operand(p[rb], ks));
                const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
                rs = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), ones, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), ones, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), ones, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), ones, rs, false);
            }
            l[rb] += rs;
        }
    }

    // Scores of one 32-key half whose first key is `key` (absolute) made
    // ready for the weights: scale and soft-cap (EXPLICIT), masks (if MASK;
    // the wave's rows start at query row `row0` of a head with window W).
    template <bool MASK>
    __device__ __forceinline__ void prepare(f32x16 (&s)[2], int64_t key, const FwdParams &pr, int64_t row0, int W) {
        int lane = lane_id();
        if (MASK) asm volatile("" : "+v"(lane));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            if (EXPLICIT) {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    s[rb][j] = CAP ? softcap_log2_pre(s[rb][j], cap_c2, cap_kl, cap_nkl2) : s[rb][j] * c_log2;
            }
            if (MASK) {
                // Key c + 4 hf of the half (c = 8 (j / 4) + j % 4) is visible
                // iff lo <= key + c + 4 hf < hi: one unsigned compare.
                int64_t lo, hi;
                key_bounds(row0 + 32 * rb + (lane & 31) + (pr.Nk - pr.Nq), pr.Nk, pr.causal, W, lo, hi);
                // Bounds relative to this lane's first key, clamped to [-1, 64]
                // (which keeps the comparisons for c in [0, 27]).
                int64_t r0 = lo - key - 4 * (lane >> 5), r1 = hi - key - 4 * (lane >> 5);
                r0 = r0 < -1 ? -1 : (r0 > 64 ? 64 : r0);
                r1 = r1 < -1 ? -1 : (r1 > 64 ? 64 : r1);
                const int base = (int)r0;
                const uint32_t span = (uint32_t)(r1 > r0 ? r1 - r0 : 0);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int c = 8 * (j / 4) + (j % 4);
                    if (!((uint32_t)(c - base) < span)) s[rb][j] = kNegInf;
                }
            }
        }
    }

    // Online softmax of one 32-key half: lazy move of the reference maximum
    // (wave-uniform; returns whether it moved and the factors), weights
    // rounded to bf16 as the P^T operands.  The reference moves only when a
    // weight against it would exceed 2^TAU, which each lane sees from the
    // maximum of its own 16 scores; only then is the row maximum taken across
    // the lane pair and the reference moved.  FIXED (soft-capped scores, |z|
    // <= softcap <= kFixedMaxCap): the reference maximum stays 0 and the
    // maximum, the move and the rescale are skipped.
    template <bool MASK>
    __device__ __forceinline__ bool softmax(f32x16 (&s)[2], int64_t key, const FwdParams &pr, int64_t row0, int W,
                                            float (&alpha)[2]) {
        prepare<MASK>(s, key, pr, row0, W);
        if (FIXED) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                alpha[rb] = 1.0f;
#pragma unroll
                for (int j = 0; j < 16; ++j) s[rb][j] = fast_exp2(s[rb][j]);
                float rs[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    rs[i] = (s[rb][4 * i] + s[rb][4 * i + 1]) + (s[rb][4 * i + 2] + s[rb][4 * i + 3]);
                lx[rb] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
                pack_weights(s[rb]);
            }
            return false;
        }
        float x[2];
        bool grow = false;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            x[rb] = max16(s[rb]);
            // NaN (a lane whose keys are all masked, reference still -inf) is no growth.
            const float over = EXPLICIT ? x[rb] - m[rb] : fmaf(x[rb], c_log2, -m[rb]);
            grow = grow || over > TAU;
        }
        const bool move = __builtin_amdgcn_ballot_w64(grow) != 0;
        if (move) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const float mt = row_max(EXPLICIT ? x[rb] : x[rb] * c_log2);
                const float m_new = fmaxf(m[rb], mt);
                const float m_use = m_new == kNegInf ? 0.0f : m_new;
                alpha[rb] = fast_exp2(m[rb] - m_use);  // 0 while m is -inf (O and l are still 0)
                m[rb] = m_new;
                mu[rb] = m_use;
            }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                s[rb][j] = EXPLICIT ? fast_exp2(s[rb][j] - mu[rb]) : fast_exp2(fmaf(s[rb][j], c_log2, -mu[rb]));
            // The normaliser sums the fp32 weights, before their rounding to
            // bf16 for P.V.
            float rs[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rs[i] = (s[rb][4 * i] + s[rb][4 * i + 1]) + (s[rb][4 * i + 2] + s[rb][4 * i + 3]);
            const float r = (rs[0] + rs[1]) + (rs[2] + rs[3]);
            l[rb] = move ? fmaf(l[rb], alpha[rb], r) : l[rb] + r;
            pack_weights(s[rb]);
        }
        return move;
    }

    __device__ __forceinline__ void rescale(const float (&alpha)[2]) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[rb][db][j] *= alpha[rb];
    }
};

// Workgroup -> the two groups' blocks.  A pair of head slots (K/V head,
// query head within its group) shares one query tile.  Heads are paired so
// that, where windows follow a pattern over h (such as every other head),
// both have the same window: inside a K/V head group of even size rep,
// head hg pairs with hg + rep/2; otherwise slots pair across K/V heads.
// With B*Hkv a multiple of 8 the pairs of one XCD (workgroups are dealt
// round-robin over 8) cover whole K/V heads; a causal grid takes an XCD's
// pairs a few at a time, longest query tile first across those pairs.
struct PairMap {
    int units;     // B * Hkv
    int rep;       // H / Hkv
    int n_qtiles;  // 256-row query tiles per head
    int xcd;       // units % 8 == 0
    int upx;       // units per XCD (xcd) or all units
    int npairs;    // pairs per XCD (xcd) or in total

    // Pair pi -> (unit, head in group) of its two blocks, units counted in
    // the XCD's list (xcd) or globally.  False when an odd number of head
    // slots leaves the last pair with one block.
    __device__ bool slots(int pi, int &ua, int &ha, int &ub, int &hb) const {
        if (rep % 2 == 0) {
            ua = ub = pi / (rep / 2);
            ha = pi % (rep / 2);
            hb = ha + rep / 2;
            return true;
        }
        if (upx % 2 == 0) {
            ua = pi / rep;
            ub = ua + upx / 2;
            ha = hb = pi % rep;
            return true;
        }
        const int sa = 2 * pi, sb = 2 * pi + 1;
        ua = sa / rep;
        ha = sa % rep;
        ub = sb / rep;
        hb = sb % rep;
        return sb < upx * rep;
    }

    __device__ bool decode(int bid, int causal, int &ua, int &ha, int &ub, int &hb, int &qtile) const {
        int pi, rank;
        bool has_b;
        if (xcd) {
            const int x = bid & 7, s = bid >> 3;
            if (causal) {
                const int C = min(npairs, max(1, (64 + n_qtiles - 1) / n_qtiles));
                const int c0 = (s / (C * n_qtiles)) * C;
                const int csz = min(C, npairs - c0);
                const int rem = s - c0 * n_qtiles;
                rank = rem / csz;
                pi = c0 + rem % csz;
            } else {
                pi = s / n_qtiles;
                rank = s % n_qtiles;
            }
            has_b = slots(pi, ua, ha, ub, hb);
            ua = ua * 8 + x;
            ub = ub * 8 + x;
        } else {
            rank = bid / npairs;
            pi = bid % npairs;
            has_b = slots(pi, ua, ha, ub, hb);
        }
        qtile = causal ? (n_qtiles - 1 - rank) : rank;
        return has_b;
    }
};

// Number of 64-key tiles a block of query rows [q0, qlast] of a head with
// window W streams, and the first key.
__device__ __forceinline__ int block_tiles(const FwdParams &p, int64_t q0, int64_t qlast, int W, int64_t &kbeg) {
    const int64_t off = p.Nk - p.Nq;
    int64_t lo_first, hi_first, lo_last, hi_last;
    key_bounds(q0 + off, p.Nk, p.causal, W, lo_first, hi_first);
    key_bounds(qlast + off, p.Nk, p.causal, W, lo_last, hi_last);
    kbeg = lo_first;
    return hi_last > lo_first ? (int)((hi_last - lo_first + BN - 1) / BN) : 0;
}

template <int NG, bool EXPLICIT, bool CAP, bool FIXED>
__global__ __launch_bounds__(NG * 256, 2 / NG) void fwd_bf16_wide_kernel(const FwdParams p, const PairMap pm) {
    __shared__ __attribute__((aligned(1024))) uint16_t lds[NG * GROUP_TILES * L::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wi = wave & 3;  // group; wave within the group (its loader index)
    const int l32 = lane & 31, hf = lane >> 5;

    int ua, ha, ub, hb, qtile;
    bool has_b = false;
    if (NG == 2) {
        has_b = pm.decode(blockIdx.x, p.causal, ua, ha, ub, hb, qtile);
    } else {
        // One block per workgroup, in the XCD-aware order of decode_block
        // (two workgroups per CU: clusters of at least 128 blocks; measured
        // on the causal workload 527.9 -> 523.6 us against 64).
        const Work wk = decode_block(p, pm.n_qtiles, 128);
        qtile = wk.qtile;
        ua = wk.b * (int)p.Hkv + wk.h / pm.rep;
        ha = wk.h % pm.rep;
    }
    const bool active = grp == 0 || has_b;
    const int unit = grp == 0 ? ua : ub;
    const int b = unit / (int)p.Hkv;
    const int g = unit % (int)p.Hkv;
    const int h = g * pm.rep + (grp == 0 ? ha : hb);

    const int64_t Nq = p.Nq, Nk = p.Nk;
    const int64_t off = Nk - Nq;
    const int64_t q0 = (int64_t)qtile * BM;
    const int64_t qlast = (q0 + BM < Nq ? q0 + BM : Nq) - 1;
    const int W = active ? head_window_of(p, h) : 0;
    int64_t kbeg;
    const int ntiles = active ? block_tiles(p, q0, qlast, W, kbeg) : 0;
    if (!active) kbeg = 0;
    // Both groups run the longer of the two tile loops (the barriers pair up).
    int nsteps = ntiles;
    if (NG == 2) {
        const int h_o = grp == 0 ? (ub % (int)p.Hkv) * pm.rep + hb : (ua % (int)p.Hkv) * pm.rep + ha;
        const bool act_o = grp == 1 || has_b;
        int64_t kb_o;
        const int nt_o = act_o ? block_tiles(p, q0, qlast, head_window_of(p, h_o), kb_o) : 0;
        nsteps = nt_o > nsteps ? nt_o : nsteps;
    }

    const uint16_t *Q = static_cast<const uint16_t *>(p.q) + ((int64_t)b * p.H + h) * Nq * D;
    const uint16_t *K = static_cast<const uint16_t *>(p.k) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;

    char *const glds = reinterpret_cast<char *>(lds) + grp * GROUP_TILES * TILE_BYTES;
    // LDS byte address of this group's tiles, for the direct loads.
    const uint32_t glds_at =
        (uint32_t)reinterpret_cast<uintptr_t>((lds_void *)lds) + (uint32_t)(grp * GROUP_TILES * TILE_BYTES);
    char *const kt0 = glds + KT0 * TILE_BYTES;   // K tile j in kt0 + (j % 2) * TILE_BYTES
    char *const vt0 = glds + VT0 * TILE_BYTES;   // V tile j in vt0 + (j % 2) * TILE_BYTES

    WideWave<EXPLICIT, CAP, FIXED> st;
    st.c_log2 = p.scale * kLog2e;
    st.scale = p.scale;
    st.softcap = p.softcap;
    st.cap_kl = p.softcap * kLog2e;
    st.cap_nkl2 = -2.0f * st.cap_kl;
    st.cap_c2 = CAP ? p.scale * (2.0f * kLog2e) / p.softcap : 0.0f;

    // This wave's rows: row0 + 32 rb + l32.
    const int64_t row0 = q0 + RW * wi;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int64_t qrow = row0 + 32 * rb + l32;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (active && qrow < Nq) x = *reinterpret_cast<const u32x4 *>(Q + qrow * D + ds * 16 + hf * 8);
            st.qf[rb][ds] = __builtin_bit_cast(bf16x8, x);
        }
        st.m[rb] = FIXED ? 0.0f : kNegInf;
        st.mu[rb] = 0.0f;
        st.l[rb] = 0.0f;
        st.lx[rb] = 0.0f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) st.oacc[rb][db][j] = 0.0f;
    }
    // Keys (relative to kbeg) seen by some valid row of the wave, [wlo,
    // whi), and by all of them, [wfl, wfh).  Wave-uniform.
    int wlo = 0, whi = 0, wfl = 0, wfh = 0;
    {
        const int64_t r_last = (row0 + RW < Nq ? row0 + RW : Nq) - 1;
        if (active && row0 <= r_last) {
            int64_t a0, a1, b0, b1;
            key_bounds(row0 + off, Nk, p.causal, W, a0, a1);
            key_bounds(r_last + off, Nk, p.causal, W, b0, b1);
            wlo = (int)(a0 - kbeg);
            whi = (int)(b1 - kbeg);
            wfl = (int)(b0 - kbeg);
            wfh = (int)(a1 - kbeg);
        }
    }

    // Matrix phases at raised priority (not with the tanh-heavy vector phase
    // of soft-capped scores).
    constexpr bool PRIO = !CAP;
    TileLoader128 ld;
    ld.lw = wi;
    const uint32_t head_bytes = (uint32_t)(Nk * D * 2);

    // Prologue: this group's first K and V tiles.
    if (ntiles > 0) {
        ld.load<false>(K, head_bytes, glds_at + KT0 * TILE_BYTES, kbeg);
        ld.load<true>(V, head_bytes, glds_at + VT0 * TILE_BYTES, kbeg);
    }
    __builtin_amdgcn_s_waitcnt(0);  // also the Q loads
    lds_barrier();
    if (NG == 2 && grp == 1) lds_barrier();  // group 1 runs one phase behind group 0

    f32x16 s[2];          // scores of a half, then (packed) its weights
    bool have_p = false;  // s holds weights of the previous half, not yet multiplied into O

    // Tile step j: four phases.
    //   M(2j):   loads of K_{j+1}; P.V of half (j-1, 1); scores of half (j, 0)
    //   V(2j):   softmax of (j, 0)
    //   M(2j+1): loads of V_{j+1}; P.V of (j, 0); scores of (j, 1)
    //   V(2j+1): softmax of (j, 1)
    // NG = 2 ends every phase with a workgroup barrier (the barriers pace
    // the ping-pong); V_j (loaded at M(2j-1)) is waited for in V(2j) and
    // K_{j+1} in V(2j+1).  NG = 1 needs a barrier only after each matrix
    // phase: a vector phase touches no LDS, so the barrier ending M(2j)
    // both frees the buffers read there (V_{j-1}, whose slot V_{j+1} then
    // fills) and publishes V_j, waited for just before it; likewise the
    // barrier ending M(2j+1) frees K_j and publishes K_{j+1}.  A wave then
    // goes from its vector phase straight into its next matrix phase.
    // Loads are waited for two or three phases after they are issued; the
    // wait for the older batch leaves the newer one (4 loads per wave) in
    // flight.  Tiles whose keys every valid row of the wave sees in full
    // run in a loop of their own without masks and with each matrix phase
    // in one scheduling region, between a masked loop before them (window
    // starts, and the first full tile, whose previous half may hold no
    // weights) and one after them (the causal diagonal).
    auto tile_step = [&](int j, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int64_t kt = kbeg + (int64_t)j * BN;
        const bool mine = j < ntiles, more = j + 1 < ntiles;
        const char *const kcur = kt0 + (j & 1) * TILE_BYTES;
        const char *const vcur = vt0 + (j & 1) * TILE_BYTES;
        const char *const vprev = vt0 + ((j + 1) & 1) * TILE_BYTES;
        const int key0 = j * BN;  // relative to kbeg
        // ---- M(2j)
        if (PRIO) __builtin_amdgcn_s_setprio(1);
        ld.load<false>(K, more ? head_bytes : 0u, glds_at + (KT0 + ((j + 1) & 1)) * TILE_BYTES, more ? kt + BN : 0);
        const bool live0 = mine && (!MASK || (key0 < whi && key0 + HALF > wlo));
        if (MASK) {
            if (have_p) st.pv(vprev, 1, s);
            if (live0) st.scores(kcur, 0, s);
        } else {
            st.pv_scores(vprev, 1, kcur, 0, s);
        }
        if (NG == 1 && mine) {
            if (more)
                __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4): V_j's loads, not K_{j+1}'s
            else
                __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        }
        lds_barrier();
        // ---- V(2j)
        if (PRIO) __builtin_amdgcn_s_setprio(0);
        have_p = live0;
        if (live0) {
            float alpha[2];
            if (st.template softmax<MASK>(s, kt, p, row0, W, alpha)) st.rescale(alpha);
            if (FIXED) st.sum_bf16_weights(s);
        }
        if (NG == 2) {
            if (mine) {
                if (more)
                    __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4): V_j's loads, not K_{j+1}'s
                else
                    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            }
            lds_barrier();
        }
        // ---- M(2j+1)
        if (PRIO) __builtin_amdgcn_s_setprio(1);
        ld.load<true>(V, more ? head_bytes : 0u, glds_at + (VT0 + ((j + 1) & 1)) * TILE_BYTES, more ? kt + BN : 0);
        const bool live1 = mine && (!MASK || (key0 + HALF < whi && key0 + BN > wlo));
        if (MASK) {
            if (have_p) st.pv(vcur, 0, s);
            if (live1) st.scores(kcur, 1, s);
        } else {
            st.pv_scores(vcur, 0, kcur, 1, s);
        }
        if (NG == 1 && more) __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4): K_{j+1}'s loads, not V_{j+1}'s
        lds_barrier();
        // ---- V(2j+1)
        if (PRIO) __builtin_amdgcn_s_setprio(0);
        have_p = live1;
        if (live1) {
            float alpha[2];
            if (st.template softmax<MASK>(s, kt + HALF, p, row0, W, alpha)) st.rescale(alpha);
            if (FIXED) st.sum_bf16_weights(s);
        }
        if (NG == 2) {
            if (more) __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4): K_{j+1}'s loads, not V_{j+1}'s
            lds_barrier();
        }
    };
    // Tiles [jf0, jf1) need no mask for this wave; the first of them runs
    // in the masked loop.
    int jf0 = (wfl + BN - 1) / BN, jf1 = wfh / BN;
    jf1 = jf1 > ntiles ? ntiles : jf1;
    int lo_full = jf0 + 1 > nsteps ? nsteps : jf0 + 1;
    int hi_full = jf1 < lo_full ? lo_full : jf1;
    int j = 0;
    for (; j < lo_full; ++j) tile_step(j, std::true_type{});
    for (; j < hi_full; ++j) tile_step(j, std::false_type{});
    for (; j < nsteps; ++j) tile_step(j, std::true_type{});
    // The last step's zero-size loads still write LDS: they must land
    // before the workgroup's LDS can go to another workgroup.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    // Last matrix phase: P.V of the final half.
    if (have_p) st.pv(vt0 + ((nsteps - 1) & 1) * TILE_BYTES, 1, s);
    lds_barrier();
    if (NG == 2 && grp == 0) lds_barrier();  // same barrier count for both groups

    if (!active) return;
    // ---- epilogue: O = acc / l, lse = (m + log2 l) ln 2.
    const int el = lane_id(), e32 = el & 31, ehf = el >> 5;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float lr = row_sum(st.l[rb]);
        const float ls = FIXED ? row_sum(st.lx[rb]) : lr;
        const int64_t qrow = row0 + 32 * rb + e32;
        if (qrow >= Nq) continue;
        const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
        const int64_t row = ((int64_t)b * p.H + h) * Nq + qrow;
        uint16_t *O = static_cast<uint16_t *>(p.o) + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 x = {pack_bf16x2(st.oacc[rb][db][4 * gq] * inv, st.oacc[rb][db][4 * gq + 1] * inv),
                           pack_bf16x2(st.oacc[rb][db][4 * gq + 2] * inv, st.oacc[rb][db][4 * gq + 3] * inv)};
                *reinterpret_cast<u32x2 *>(O + db * 32 + 8 * gq + 4 * ehf) = x;
            }
        if (p.lse && ehf == 0) p.lse[row] = ls > 0.0f ? (st.m[rb] + __log2f(ls)) * kLn2 : kNegInf;
    }
}

template <int NG, bool EXPLICIT, bool CAP, bool FIXED>
int launch(const FwdParams &p, hipStream_t stream) {
    PairMap pm;
    pm.units = (int)(p.B * p.Hkv);
    pm.rep = p.group;
    pm.n_qtiles = (int)((p.Nq + BM - 1) / BM);
    pm.xcd = pm.units % 8 == 0 ? 1 : 0;
    pm.upx = pm.xcd ? pm.units / 8 : pm.units;
    pm.npairs = (pm.upx * pm.rep + 1) / 2;
    const int64_t wgs = NG == 2 ? (int64_t)pm.npairs * pm.n_qtiles * (pm.xcd ? 8 : 1) : p.B * p.H * pm.n_qtiles;
    if (wgs <= 0) return FA_OK;
    if (wgs > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((fwd_bf16_wide_kernel<NG, EXPLICIT, CAP, FIXED>), dim3((unsigned)wgs), dim3(NG * 256), 0, stream,
                       p, pm);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

// Whether the wide kernel takes this unsplit bf16 launch: d = 128 and
// enough 256-row blocks for a workgroup (two blocks) on every CU.
bool fwd_bf16_wide_applies(const FwdParams &p, int d) {
    if (d != D) return false;
    const int64_t blocks = p.B * p.H * ((p.Nq + BM - 1) / BM);
    return blocks >= 512;
}

int launch_fwd_bf16_wide(const FwdParams &p, hipStream_t stream) {
    if (p.softcap > 0.0f) {
        if (p.softcap <= kFixedMaxCap) return launch<2, true, true, true>(p, stream);
        return launch<2, true, true, false>(p, stream);
    }
    bool windows = p.window > 0;
    for (int h = 0; h < p.H && p.has_head_window; ++h) windows = windows || p.head_window[h] > 0;
    if (windows) {
        if (!(p.scale > 0.0f)) return launch<2, true, false, false>(p, stream);
        return launch<2, false, false, false>(p, stream);
    }
    if (!(p.scale > 0.0f)) return launch<1, true, false, false>(p, stream);
    return launch<1, false, false, false>(p, stream);
}

}  // namespace fa
