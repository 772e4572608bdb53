// fa_fwd_bf16.hip -- bf16 tiled forward attention with an online softmax,
// MFMA (v_mfma_f32_32x32x16_bf16) for both contractions, gfx950.
//
// The method (Transformers & Math, Module 16, section 16.1 flow and 16.2
// merge rule): a workgroup loads one block of query rows, streams blocks of
// K and V through LDS, computes that block's scores, updates each row's
// running maximum and sum, adds the block's contribution to an output kept
// on chip, and writes the finished output once.  The score matrix never
// reaches HBM.
//
// Tiling on CDNA4: 8 waves per workgroup, two per SIMD, 32 query rows per
// wave (256 per workgroup), key tiles of 64 shared in LDS by all 8 waves.
// Grids of fewer than 256 such workgroups use 4-wave workgroups of 128 rows
// instead (two per CU, so the two waves sharing a SIMD come from different
// workgroups and interleave without the ping-pong's barriers): twice the
// parallelism where CUs would otherwise idle.
//   * scores are computed transposed, S^T = K Q^T (A = K from LDS, B = Q^T
//     kept in registers), so the 32x32 accumulator gives every lane ONE
//     query row and 16 of its keys; the partner lane (lane ^ 32) holds the
//     other 16.  Row max / row sum are in-lane reductions plus one
//     v_permlane32_swap.
//   * the output is accumulated transposed, O^T += V^T P^T: the score
//     accumulator registers, rounded to bf16, are exactly the B operand
//     (keys permuted consistently with the V^T read), and each lane again
//     owns one query row, so the rescale by exp(m_old - m_new) is a per-lane
//     multiply.
//   * ping-pong: the two waves that share a SIMD alternate between a matrix
//     phase (scores of tile j and P.V of tile j-1, all MFMA) and a vector
//     phase (softmax of tile j).  Waves 4..7 run one phase behind waves
//     0..3, enforced by workgroup barriers, so while one wave of a SIMD
//     issues MFMAs its partner runs the exp/max/sum work.
//   * K and V tiles go from HBM straight into LDS (buffer_load ... lds, 16 B
//     per lane, no register staging; the buffer range check zero-fills rows
//     past the last key), row-major with an XOR swizzle of the 16-byte
//     chunks so the K operand reads (ds_read_b128) are bank-conflict free.
//   * each V tile is transposed once per workgroup: every loading wave
//     turns the 16 keys it loaded into V^T rows with transposing reads
//     (ds_read_b64_tr_b16 hands a lane four keys of one column) and 8-byte
//     writes into a V^T tile whose keys are permuted within each group of 16
//     (bits 2 and 3 of the key index swapped), so the 8 keys a lane supplies
//     to one P.V k-step are contiguous and the V^T operand is a single
//     ds_read_b128 (the transposing read is several times slower per byte).
//   * all query tiles of one K/V head run on the same XCD (shared L2); a
//     causal grid takes an XCD's heads a few at a time, longest query tile
//     first across those heads (balanced tail, K and V of few heads live in
//     the L2 at once).
//
// Softmax bookkeeping per tile is kept small, since at d = 128 its vector
// work rivals the matrix work:
//   * tiles that every row of the block sees in full skip all masking;
//   * without a soft-cap the row maximum is taken on the raw scores and the
//     weight is exp2(fma(s, scale*log2 e, -m)): one FMA and one exp each;
//   * the running maximum is only moved when a tile's maximum exceeds it by
//     more than TAU (log2 units).  Any reference point gives the same exact
//     result (the merge rule rescales consistently); this one keeps the
//     weights <= 2^TAU and makes the rescale of the output, a multiply of
//     every accumulator, rare;
//   * the normaliser is the sum of the fp32 weights, taken before they are
//     rounded to bf16 for P.V, so lse keeps fp32 accuracy however few keys
//     a row sees.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_tile.h"

namespace fa {

namespace {

constexpr int RB = 1;             // 32-row blocks per wave
// Waves per workgroup NW is a kernel parameter: 8 (two per SIMD, 256 query
// rows) or 4 (one per SIMD, 128 rows, two workgroups per CU) for grids that
// would not give every CU a workgroup of 8.
constexpr int kSmallGrid = 256;   // fewer 8-wave workgroups than this: use 4-wave ones
constexpr int BN = 64;            // keys per tile
constexpr int LOADERS = 4;        // waves that issue the tile loads
constexpr float TAU = 8.0f;       // lazy-rescale threshold, log2 units
// Largest soft-cap for the fixed reference maximum: e^60 per weight leaves
// room for 2^31 keys below the fp32 maximum (3.4e38).
constexpr float kFixedMaxCap = 60.0f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
struct Smem {
    static constexpr int CPR = D / 8;              // 16-byte chunks per row
    static constexpr int TILE = BN * D;            // bf16 elements of one K or V tile
    static constexpr int LPW = BN * CPR / 64 / LOADERS;  // loads per loader wave per tile
    // Swizzled chunk slot of chunk c in row r; LDS has 64 banks of 4 bytes
    // (256 bytes per bank line, RPB = 16 / CPR rows per line).  K: c ^ (r %
    // CPR) puts the same chunk of 16 consecutive rows in distinct banks.  V
    // (as loaded): the 32 lanes of one transposing-read pass address rows
    // {0..3, 8..11} or {4..7, 12..15} of a 16-row group (see the row order of
    // the transposition below), two chunk halves each; xor-ing the chunk
    // index with twice (row bits below 2 that select no bank line part, then
    // row bit 3) gives those 8 rows distinct bank positions.
    static constexpr int RPB_LOG2 = CPR == 16 ? 0 : (CPR == 8 ? 1 : 2);
    __device__ static int kslot(int r, int c) { return c ^ (r % CPR); }
    __device__ static int vslot(int r, int c) {
        return c ^ (2 * (((r & 3) >> RPB_LOG2) | (((r >> 3) & 1) << (2 - RPB_LOG2))));
    }
    // V^T tile: D rows (one per column of V) of BN = 64 permuted keys, 128
    // bytes per row; 16-byte chunk c of row d sits in slot c ^ ((d/2) % 8),
    // which spreads 16 consecutive rows' same chunk over all banks.
    static constexpr int VT_ROW = BN * 2;  // bytes
    __device__ static int vtslot(int d, int c) { return c ^ ((d >> 1) & 7); }
};

__device__ __forceinline__ u32x4 ldg16(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

constexpr int PREFETCH = 4;

// Per-wave state and the pieces of one pipelined step.
template <int D, bool EXPLICIT, bool CAP, bool FIXED>
struct Wave {
    using L = Smem<D>;
    bf16x8 qf[RB][D / 16];      // Q^T operand, per row block
    f32x16 oacc[RB][D / 32];    // O^T accumulators
    float m[RB], l[RB];         // lazy reference max (log2 units); this lane's half of the normaliser
                                // (fp32 weights; FIXED: the bf16 weights P.V uses)
    float lx[RB];               // FIXED: this lane's half of the sum of the fp32 weights (for lse)
    float mtrue[RB];            // exact running max (log2 units)
    int lo_rel[RB], hi_rel[RB]; // visible keys relative to the first tile
    int koff[D / 16];           // K operand read offsets (bytes)
    int vko[4];                 // V^T operand read offsets per k-step (bytes)
    int hf;
    float c_log2, scale, softcap;

    // S^T = K Q^T for the 64 keys of a tile, both row blocks.
    template <bool SCHED = true>
    __device__ __forceinline__ void scores(const uint16_t *kbuf, f32x16 (&sacc)[RB][2]) const {
        const char *Ksb = reinterpret_cast<const char *>(kbuf);
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) sacc[r][kb][j] = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(Ksb + kb * 32 * L::CPR * 16 + koff[ds]);
#pragma unroll
                for (int r = 0; r < RB; ++r)
                    sacc[r][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                          qf[r][ds], sacc[r][kb], 0, 0, 0);
            }
        if (SCHED) sched_read_mfma_pipeline<2 * (D / 16), RB, PREFETCH>();
    }

    // Online softmax of one tile: masks (if MASK), row max, lazy move of the
    // reference maximum (branch-free; returns whether any row moved and the
    // factors), weights rounded to bf16 as the P^T operand.  FIXED (soft-
    // capped scores, |z| <= softcap <= kFixedMaxCap): the reference maximum
    // stays 0, every weight e^z lies in [e^-cap, e^cap], inside fp32 and
    // bf16 range, and the row maximum, the move and the rescale are skipped.
    template <bool MASK>
    __device__ __forceinline__ bool softmax(f32x16 (&sacc)[RB][2], int it, bf16x8 (&pf)[RB][4],
                                            float (&alpha)[RB]) {
        float mt[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (EXPLICIT) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        sacc[r][kb][j] = CAP ? softcap_log2(sacc[r][kb][j] * scale, softcap) : sacc[r][kb][j] * c_log2;
            }
            if (MASK) {
                // Key ko = c + 4*hf of the tile is visible iff lo <= ko < hi,
                // i.e. (unsigned)(c - base) < span: one compare per element.
                const int lo = lo_rel[r] - it * BN, hi = hi_rel[r] - it * BN;
                const int base = lo - 4 * hf;
                const uint32_t span = (uint32_t)(hi - lo);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int c = kb * 32 + 8 * (j / 4) + (j % 4);
                        if (!((uint32_t)(c - base) < span)) sacc[r][kb][j] = kNegInf;
                    }
            }
            if (FIXED) continue;
            float x = sacc[r][0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) x = fmaxf(x, sacc[r][kb][j]);
            mt[r] = EXPLICIT ? x : x * c_log2;
            mt[r] = row_max(mt[r]);
            mtrue[r] = fmaxf(mtrue[r], mt[r]);
        }
        if (FIXED) {
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                alpha[r] = 1.0f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) sacc[r][kb][j] = fast_exp2(sacc[r][kb][j]);
                // O is normalised by the sum of the same bf16 weights P.V uses
                // (pv), so it stays a convex combination of V rows; lse takes
                // the sum of the fp32 weights: with no running maximum no
                // weight is exactly 1, and the bf16 rounding of a dominant
                // weight would otherwise reach lse.
                float rs[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    rs[i] = (sacc[r][i / 4][4 * (i % 4)] + sacc[r][i / 4][4 * (i % 4) + 1]) +
                            (sacc[r][i / 4][4 * (i % 4) + 2] + sacc[r][i / 4][4 * (i % 4) + 3]);
                lx[r] += ((rs[0] + rs[1]) + (rs[2] + rs[3])) + ((rs[4] + rs[5]) + (rs[6] + rs[7]));
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int gp = 0; gp < 2; ++gp) {
                        u32x4 xq;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            xq[e] = pack_bf16x2(sacc[r][kb][8 * gp + 2 * e], sacc[r][kb][8 * gp + 2 * e + 1]);
                        pf[r][kb * 2 + gp] = __builtin_bit_cast(bf16x8, xq);
                    }
            }
            return false;
        }
        bool grow = false;
#pragma unroll
        for (int r = 0; r < RB; ++r) grow = grow || (mt[r] > m[r] + TAU);
        const bool move = __builtin_amdgcn_ballot_w64(grow) != 0;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const float m_new = move ? fmaxf(m[r], mt[r]) : m[r];
            const float m_use = m_new == kNegInf ? 0.0f : m_new;
            alpha[r] = fast_exp2(m[r] - m_use);
            m[r] = m_new;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    sacc[r][kb][j] = EXPLICIT ? fast_exp2(sacc[r][kb][j] - m_use)
                                              : fast_exp2(fmaf(sacc[r][kb][j], c_log2, -m_use));
            // The normaliser sums the fp32 weights, before their rounding to
            // bf16 for P.V: a dominant weight's rounding (up to 2^-8 of it)
            // would otherwise reach lse whole when a row sees few keys.
            {
                float rs[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    rs[i] = (sacc[r][i / 4][4 * (i % 4)] + sacc[r][i / 4][4 * (i % 4) + 1]) +
                            (sacc[r][i / 4][4 * (i % 4) + 2] + sacc[r][i / 4][4 * (i % 4) + 3]);
                l[r] = fmaf(l[r], alpha[r],
                            ((rs[0] + rs[1]) + (rs[2] + rs[3])) + ((rs[4] + rs[5]) + (rs[6] + rs[7])));
            }
            // k-step (kb, gp) covers keys kb*32 + 16*gp + [0, 16): this lane
            // half supplies keys +4*hf+[0,4) and +8+4*hf+[0,4), which are
            // exactly accumulator elements 8*gp .. 8*gp+7.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int gp = 0; gp < 2; ++gp) {
                    u32x4 xq;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        xq[e] = pack_bf16x2(sacc[r][kb][8 * gp + 2 * e], sacc[r][kb][8 * gp + 2 * e + 1]);
                    pf[r][kb * 2 + gp] = __builtin_bit_cast(bf16x8, xq);
                }
        }
        return move;
    }

    __device__ __forceinline__ void rescale(const float (&alpha)[RB]) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) oacc[r][db][j] *= alpha[r];
    }

    // O^T += V^T P^T.  For k-step ks the lane supplies keys ks*16 +
    // 4*hf + [0,4) and ks*16 + 8 + 4*hf + [0,4) of column db*32 + lane%32:
    // permuted positions ks*16 + 8*hf + [0,8) of that V^T row, one 16-byte read.
    template <bool SCHED = true>
    __device__ __forceinline__ void pv(const uint16_t *vt, const bf16x8 (&pf)[RB][4]) {
        const char *Vtb = reinterpret_cast<const char *>(vt);
        // FIXED: row sum of this lane's 32 bf16 weights (dot2 with (1, 1)),
        // which normalises O; the partner lane's half is added once, in the
        // epilogue.  The running-maximum path sums fp32 weights in softmax.
        const bf16x2 ones = as_bf16x2(0x3f803f80u);
#pragma unroll
        for (int r = 0; r < (FIXED ? RB : 0); ++r) {
            float rs = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u32x4 w = __builtin_bit_cast(u32x4, pf[r][k]);
                const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
                rs = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w0), ones, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w1), ones, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w2), ones, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w3), ones, rs, false);
            }
            l[r] += rs;
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(Vtb + db * 32 * L::VT_ROW + vko[ks]);
#pragma unroll
                for (int r = 0; r < RB; ++r)
                    oacc[r][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf[r][ks],
                                                                          oacc[r][db], 0, 0, 0);
            }
        if (SCHED) sched_read_mfma_pipeline<4 * (D / 32), RB, PREFETCH>();
    }
};

template <int D, bool SPLIT, bool EXPLICIT, bool CAP, bool FIXED, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_bf16_kernel(const FwdParams p, const int n_qtiles) {
    using L = Smem<D>;
    constexpr int BM = NW * 32 * RB;  // query rows per workgroup
    // Separate arrays per buffer so the compiler can tell the buffer being
    // filled from the buffers being read.
    __shared__ __attribute__((aligned(1024))) uint16_t kbuf0[L::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t kbuf1[L::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vstage[L::TILE];  // V as loaded (row-major)
    __shared__ __attribute__((aligned(1024))) uint16_t vt0[L::TILE];     // V^T, permuted keys
    __shared__ __attribute__((aligned(1024))) uint16_t vt1[L::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool leader = wave < LOADERS;  // waves 0..3 lead and load; with 8 waves, 4..7 trail
    const int l32 = lane & 31, hf = lane >> 5;
    const Work w = decode_block(p, n_qtiles);
    const int h = w.h, b = w.b;
    const int g = h / p.group;
    const int64_t Nq = p.Nq, Nk = p.Nk;
    const int64_t off = Nk - Nq;
    const int W = head_window_of(p, h);

    // Key range of this split (the whole key axis unless split-KV).
    int64_t r_lo = 0, r_hi = Nk;
    if (SPLIT) {
        r_lo = (int64_t)w.split * p.split_len;
        r_hi = r_lo + p.split_len < Nk ? r_lo + p.split_len : Nk;
        if (r_lo > Nk) r_lo = Nk;
    }

    const int64_t q0 = (int64_t)w.qtile * BM;
    const int64_t qlast = (q0 + BM < Nq ? q0 + BM : Nq) - 1;
    int64_t lo_first, hi_first, lo_last, hi_last;
    key_bounds(q0 + off, Nk, p.causal, W, lo_first, hi_first);
    key_bounds(qlast + off, Nk, p.causal, W, lo_last, hi_last);
    // Union of the rows' visible keys, and the part every row sees.
    const int64_t kbeg = lo_first > r_lo ? lo_first : r_lo;
    const int64_t kend = hi_last < r_hi ? hi_last : r_hi;
    const int64_t full_lo = lo_last > r_lo ? lo_last : r_lo;
    const int64_t full_hi = hi_first < r_hi ? hi_first : r_hi;

    const uint16_t *Q = static_cast<const uint16_t *>(p.q) + ((int64_t)b * p.H + h) * Nq * D;
    const uint16_t *K = static_cast<const uint16_t *>(p.k) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + ((int64_t)b * p.Hkv + g) * p.kv_rows * D;

    Wave<D, EXPLICIT, CAP, FIXED> st;
    st.hf = hf;
    st.c_log2 = p.scale * kLog2e;
    st.scale = p.scale;
    st.softcap = p.softcap;
    const int64_t qrow = q0 + wave * 32 + l32;
    {
        // This lane's query row and its visible interval, relative to kbeg.
        int64_t lo, hi;
        key_bounds(qrow + off, Nk, p.causal, W, lo, hi);
        lo = (lo > r_lo ? lo : r_lo) - kbeg;
        hi = (hi < r_hi ? hi : r_hi) - kbeg;
        // A row whose keys all lie outside this split has hi < lo here; an
        // empty interval keeps the mask's unsigned span at 0 (not 2^32 - 1).
        if (hi < lo) hi = lo;
        st.lo_rel[0] = (int)(lo < -1 ? -1 : (lo > 0x3fffffff ? 0x3fffffff : lo));
        st.hi_rel[0] = (int)(hi < -1 ? -1 : (hi > 0x3fffffff ? 0x3fffffff : hi));
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qrow < Nq) x = ldg16(Q + qrow * D + ds * 16 + hf * 8);
            st.qf[0][ds] = __builtin_bit_cast(bf16x8, x);
        }
        st.m[0] = FIXED ? 0.0f : kNegInf;
        st.mtrue[0] = kNegInf;
        st.l[0] = 0.0f;
        st.lx[0] = 0.0f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) st.oacc[0][db][j] = 0.0f;
    }
    // K operand reads: row kb*32 + l32, chunk 2*ds + hf.
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) st.koff[ds] = (l32 * L::CPR + L::kslot(l32, 2 * ds + hf)) * 16;
    // V^T operand reads: row d = db*32 + l32, chunk 2*ks + hf.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) st.vko[ks] = l32 * L::VT_ROW + L::vtslot(l32, 2 * ks + hf) * 16;
    // Transposition of the 16 keys 16*lw + [0,16) each loading wave loads:
    // transposing read t (t < D/16) covers columns 16t + [0,16); lane group
    // gq = lane/16 provides rows 16*lw + 4*a + e with a = swap2(gq) (the two
    // bits of gq exchanged; e = (lane%16)/4), columns 16t + 4j (j = lane%4),
    // and receives keys 16*lw + 4*a + [0,4) of column 16t + lane%16.  Their
    // permuted positions are 16*lw + 4*swap2(a) + [0,4) = 16*lw + 4*gq +
    // [0,4): chunk 2*lw + gq/2, half gq%2, so each 32-lane pass of the
    // 8-byte writes fills whole chunks.
    int tr_src = 0, tr_dst = 0, tr_e = 0, tr_jb = 0;
    {
        const int gq = lane >> 4, e = (lane & 15) >> 2, j = lane & 3, i = lane & 15;
        const int lw0 = wave < LOADERS ? wave : 0;
        const int a = ((gq & 1) << 1) | (gq >> 1);
        const int rr = 16 * lw0 + 4 * a + e;
        tr_src = rr * L::CPR * 16 + (j & 1) * 8;
        tr_e = rr;
        tr_jb = j >> 1;
        tr_dst = i * L::VT_ROW + L::vtslot(i, 2 * lw0 + (gq >> 1)) * 16 + 8 * (gq & 1);
    }

    // Direct loads (leader waves only): load u of loader wave lw fills LDS
    // chunk slots q*64 + lane (q = lw*LPW + u) of a tile, i.e. row rr, slot
    // sl, which holds chunk kslot(rr, sl) of K (vslot for V; xor is its own
    // inverse).
    const int lw = leader ? wave : 0;
    int k_goff[L::LPW], v_goff[L::LPW];
#pragma unroll
    for (int u = 0; u < L::LPW; ++u) {
        const int pos = (lw * L::LPW + u) * 64 + lane;
        const int rr = pos / L::CPR, sl = pos % L::CPR;
        k_goff[u] = (rr * D + L::kslot(rr, sl) * 8) * 2;
        v_goff[u] = (rr * D + L::vslot(rr, sl) * 8) * 2;
    }
    const uint32_t head_bytes = (uint32_t)(Nk * D * 2);
    const int ntiles = kend > kbeg ? (int)((kend - kbeg + BN - 1) / BN) : 0;
    const int kt0 = (int)kbeg;

    auto load_k = [&](int t, uint16_t *buf) {
        const uint32_t toff = (uint32_t)(kt0 + t * BN) * (uint32_t)(D * 2);
#pragma unroll
        for (int u = 0; u < L::LPW; ++u)
            buffer_load_lds16(K, head_bytes, (lds_void *)(buf + (lw * L::LPW + u) * 64 * 8), k_goff[u], toff);
    };
    auto load_v = [&](int t, uint16_t *buf) {  // buf: vstage
        const uint32_t toff = (uint32_t)(kt0 + t * BN) * (uint32_t)(D * 2);
#pragma unroll
        for (int u = 0; u < L::LPW; ++u)
            buffer_load_lds16(V, head_bytes, (lds_void *)(buf + (lw * L::LPW + u) * 64 * 8), v_goff[u], toff);
    };
    auto is_full = [&](int t) {
        const int64_t kt = kbeg + (int64_t)t * BN;
        return kt >= full_lo && kt + BN <= full_hi;
    };
    // This loading wave's 16 keys of the staged V tile -> V^T tile vt.  Only
    // this wave's own loads are read, so its own wait suffices.
    auto transpose_v = [&](uint16_t *vt) {
        const char *src = reinterpret_cast<const char *>(vstage);
        char *dst = reinterpret_cast<char *>(vt);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            const int c = L::vslot(tr_e, 2 * t + tr_jb);
            const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(src + tr_src - (tr_src % (L::CPR * 16)) + c * 16 + (tr_src % 16)));
            *reinterpret_cast<i16x4 *>(dst + tr_dst + 16 * t * L::VT_ROW) = x;
        }
    };

    f32x16 sacc[RB][2];
    bf16x8 pf[RB][4];
    // Step j: matrix phase (loads of K for tile j+1 and V for tile j by the
    // leaders, scores of tile j from kcur, P.V of tile j-1 from vtprev),
    // barrier, vector phase (softmax of tile j; the leaders then wait for
    // their loads and transpose their part of V_j into vtcur), barrier.
    auto step = [&](int j, const uint16_t *kcur, const uint16_t *vtprev, uint16_t *knext, uint16_t *vtcur) {
        if (leader) {
            if (j + 1 < ntiles) load_k(j + 1, knext);
            if (j < ntiles) load_v(j, vstage);
        }
        if (j < ntiles) st.scores(kcur, sacc);
        if (j >= 1) st.pv(vtprev, pf);
        lds_barrier();
        if (j < ntiles) {
            float alpha[RB];
            const bool move = is_full(j) ? st.template softmax<false>(sacc, j, pf, alpha)
                                         : st.template softmax<true>(sacc, j, pf, alpha);
            if (move) st.rescale(alpha);
        }
        if (leader) {
            __builtin_amdgcn_s_waitcnt(0);
            if (j < ntiles) transpose_v(vtcur);
        }
        lds_barrier();
    };

    if (leader && ntiles > 0) load_k(0, kbuf0);
    // Every wave: the Q fragments (so that no wait for them is left inside
    // the loop, where it would also wait for the tile loads) and the first K
    // tile.
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (!leader) lds_barrier();  // trail the leaders by one phase
    // Tile j's K sits in kbuf[j % 2], its V^T in vt[j % 2].
    for (int j = 0; j <= ntiles; j += 2) {
        step(j, kbuf0, vt1, kbuf1, vt0);
        if (j + 1 > ntiles) break;
        step(j + 1, kbuf1, vt0, kbuf0, vt1);
    }
    if (leader) lds_barrier();  // same barrier count for both groups

    // ---- epilogue: O = acc / l.  Lane holds dims db*32 + 8*(j/4) + 4*hf + (j%4).
    const float lr = row_sum(st.l[0]);  // both halves of the row
    const float ls = FIXED ? row_sum(st.lx[0]) : lr;  // the sum lse is taken from
    if (qrow >= Nq) return;
    const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
    const int64_t row = ((int64_t)b * p.H + h) * Nq + qrow;
    if (!SPLIT) {
        uint16_t *O = static_cast<uint16_t *>(p.o) + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 x = {pack_bf16x2(st.oacc[0][db][4 * gq] * inv, st.oacc[0][db][4 * gq + 1] * inv),
                           pack_bf16x2(st.oacc[0][db][4 * gq + 2] * inv, st.oacc[0][db][4 * gq + 3] * inv)};
                *reinterpret_cast<u32x2 *>(O + db * 32 + 8 * gq + 4 * hf) = x;
            }
        if (p.lse && hf == 0) p.lse[row] = ls > 0.0f ? (st.m[0] + __log2f(ls)) * kLn2 : kNegInf;
    } else {
        const int64_t prow = row * p.num_splits + w.split;
        float *Op = p.o_part + prow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                f32x4 x = {st.oacc[0][db][4 * gq] * inv, st.oacc[0][db][4 * gq + 1] * inv,
                           st.oacc[0][db][4 * gq + 2] * inv, st.oacc[0][db][4 * gq + 3] * inv};
                *reinterpret_cast<f32x4 *>(Op + db * 32 + 8 * gq + 4 * hf) = x;
            }
        if (hf == 0) {
            // Report the split's exact maximum, with l relative to it.
            p.m_part[prow] = lr > 0.0f ? st.mtrue[0] * kLn2 : kNegInf;
            p.l_part[prow] = lr > 0.0f ? lr * fast_exp2(st.m[0] - st.mtrue[0]) : 0.0f;
        }
    }
}

template <int D, bool SPLIT, bool EXPLICIT, bool CAP, bool FIXED, int NW>
int launch_nw(const FwdParams &p, hipStream_t stream) {
    constexpr int BM = NW * 32 * RB;
    const int n_qtiles = (int)((p.Nq + BM - 1) / BM);
    const int64_t blocks = p.B * p.H * (int64_t)n_qtiles * p.num_splits;
    if (blocks <= 0) return FA_OK;
    if (blocks > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, SPLIT, EXPLICIT, CAP, FIXED, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0,
                       stream, p, n_qtiles);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// 8-wave workgroups unless that grid would leave CUs idle: then 4-wave
// ones, twice as many (measured: 25.3 -> 20.9 us on B=1, H=8, 1024^2, d=64;
// slower than 8 waves once every CU has work).
template <int D, bool SPLIT, bool EXPLICIT, bool CAP, bool FIXED = false>
int launch_one(const FwdParams &p, hipStream_t stream) {
    const int64_t blocks8 = p.B * p.H * ((p.Nq + 255) / 256) * p.num_splits;
    if (blocks8 < kSmallGrid) return launch_nw<D, SPLIT, EXPLICIT, CAP, FIXED, 4>(p, stream);
    return launch_nw<D, SPLIT, EXPLICIT, CAP, FIXED, 8>(p, stream);
}

template <int D, bool SPLIT>
int launch_s(const FwdParams &p, hipStream_t stream) {
    if (p.softcap > 0.0f) {
        // Soft-capped scores are bounded by the cap: a fixed reference
        // maximum replaces the running one (split partials keep their exact
        // maxima, so only the unsplit pass uses it).
        if (!SPLIT && p.softcap <= kFixedMaxCap) return launch_one<D, false, true, true, true>(p, stream);
        return launch_one<D, SPLIT, true, true>(p, stream);
    }
    if (!(p.scale > 0.0f)) return launch_one<D, SPLIT, true, false>(p, stream);
    return launch_one<D, SPLIT, false, false>(p, stream);
}

template <int D>
int launch_d(const FwdParams &p, bool split, hipStream_t stream) {
    return split ? launch_s<D, true>(p, stream) : launch_s<D, false>(p, stream);
}

}  // namespace

int launch_fwd_bf16(const FwdParams &p, int d, bool split, hipStream_t stream) {
    switch (d) {
        case 32: return launch_d<32>(p, split, stream);
        case 64: return launch_d<64>(p, split, stream);
        case 128: return launch_d<128>(p, split, stream);
        default: return FA_ERR_UNSUPPORTED;
    }
}

}  // namespace fa
