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
//     chunks chosen so that the K operand reads (ds_read_b128) and the
//     transposing V reads (ds_read_b64_tr_b16, which hand each lane four
//     keys of one column: the V^T operand) are bank-conflict free.
//   * blocks are ordered so that all query tiles of one K/V head run back to
//     back on the same XCD (shared L2), the longest causal tiles first.
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
//     every accumulator, rare.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int RB = 1;             // 32-row blocks per wave
constexpr int NW = 8;             // waves per workgroup (two per SIMD)
constexpr int BM = NW * 32 * RB;  // query rows per workgroup
constexpr int BN = 64;            // keys per tile
constexpr int NT = 64 * NW;       // threads per workgroup
constexpr int LOADERS = 4;        // waves that issue the tile loads
constexpr float TAU = 8.0f;       // lazy-rescale threshold, log2 units

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
struct Smem {
    static constexpr int CPR = D / 8;              // 16-byte chunks per row
    static constexpr int TILE = BN * D;            // bf16 elements of one K or V tile
    static constexpr int LPW = BN * CPR / 64 / LOADERS;  // loads per loader wave per tile
    // Swizzled chunk slot of chunk c in row r.  K: c ^ (r % CPR) puts the
    // same chunk of 16 consecutive rows in distinct banks.  V: c ^ (4r % CPR)
    // moves each of the 4 rows a transposing read touches (4 consecutive
    // rows, 64 bytes each for 32 lanes) to its own 64-byte bank block.
    __device__ static int kslot(int r, int c) { return c ^ (r % CPR); }
    __device__ static int vslot(int r, int c) { return c ^ ((4 * r) % CPR); }
};

__device__ __forceinline__ u32x4 ldg16(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// 16 bytes per lane from base + voff + soff straight into LDS (dst + 16*lane).
// The buffer resource bounds the access to [base, base + nbytes): bytes past
// the end read as zero.  soff is wave-uniform.
__device__ __forceinline__ void buffer_load_lds16(const void *base, int nbytes, lds_void *dst, int voff, int soff) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, nbytes,
                                                                         0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// {own, partner} values of a lane and lane ^ 32, in either order.
__device__ __forceinline__ void halves(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float row_max(float x) {
    float a, b;
    halves(x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float row_sum(float x) {
    float a, b;
    halves(x, a, b);
    return a + b;
}

// Block index -> (query tile, head, batch, split).  The unit of locality is
// one (batch, K/V head): its query heads and tiles are consecutive in the
// dispatch order of one XCD (block ids are dealt round-robin over 8 XCDs).
struct Work {
    int qtile, h, b, split;
};

__device__ __forceinline__ Work decode_block(const FwdParams &p, int n_qtiles) {
    const int bid = blockIdx.x;
    const int rep = p.group, S = p.num_splits;
    const int units = (int)(p.B * p.Hkv);
    const int per_unit = rep * n_qtiles * S;
    int unit, r;
    if (units % 8 == 0) {
        const int x = bid & 7, s = bid >> 3;
        unit = (s / per_unit) * 8 + x;
        r = s % per_unit;
    } else {
        unit = bid % units;
        r = bid / units;
    }
    Work w;
    const int hg = r % rep;
    const int rest = r / rep;
    w.split = rest % S;
    const int rank = rest / S;
    w.qtile = p.causal ? (n_qtiles - 1 - rank) : rank;
    w.b = unit / (int)p.Hkv;
    w.h = (unit % (int)p.Hkv) * rep + hg;
    return w;
}

// Per-wave state and the pieces of one pipelined step.
template <int D, bool EXPLICIT, bool CAP>
struct Wave {
    using L = Smem<D>;
    bf16x8 qf[RB][D / 16];      // Q^T operand, per row block
    f32x16 oacc[RB][D / 32];    // O^T accumulators
    float m[RB], l[RB];         // lazy reference max (log2 units) and sum
    float mtrue[RB];            // exact running max (log2 units)
    int lo_rel[RB], hi_rel[RB]; // visible keys relative to the first tile
    int koff[D / 16];           // K operand read offsets (bytes)
    int voff[D / 32];           // V^T operand read offsets (bytes)
    int hf;
    float c_log2, scale, softcap;

    // S^T = K Q^T for the 64 keys of a tile, both row blocks.
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
    }

    // Online softmax of one tile: masks (if MASK), row max, lazy move of the
    // reference maximum (branch-free; returns whether any row moved and the
    // factors), weights rounded to bf16 as the P^T operand.
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
                const int lo = lo_rel[r] - it * BN, hi = hi_rel[r] - it * BN;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int ko = kb * 32 + 8 * (j / 4) + 4 * hf + (j % 4);
                        if (ko < lo || ko >= hi) sacc[r][kb][j] = kNegInf;
                    }
            }
            float x = sacc[r][0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) x = fmaxf(x, sacc[r][kb][j]);
            mt[r] = EXPLICIT ? x : x * c_log2;
            mt[r] = row_max(mt[r]);
            mtrue[r] = fmaxf(mtrue[r], mt[r]);
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
            float rs = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float pj = EXPLICIT ? fast_exp2(sacc[r][kb][j] - m_use)
                                              : fast_exp2(fmaf(sacc[r][kb][j], c_log2, -m_use));
                    sacc[r][kb][j] = pj;
                    rs += pj;
                }
            l[r] = l[r] * alpha[r] + row_sum(rs);
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

    // O^T += V^T P^T.  Two transposing reads give this lane the keys
    // +4*hf+[0,4) and +8+4*hf+[0,4) of k-step ks at its column db*32 + lane%32.
    __device__ __forceinline__ void pv(const uint16_t *vbuf, const bf16x8 (&pf)[RB][4]) {
        const char *Vsb = reinterpret_cast<const char *>(vbuf);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const char *base = Vsb + voff[db] + ks * 16 * L::CPR * 16;
                const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base));
                const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + 8 * L::CPR * 16));
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int r = 0; r < RB; ++r)
                    oacc[r][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[r][ks], oacc[r][db], 0, 0, 0);
            }
    }
};

template <int D, bool SPLIT, bool EXPLICIT, bool CAP>
__global__ __launch_bounds__(NT, 1) void fwd_bf16_kernel(const FwdParams p, const int n_qtiles) {
    using L = Smem<D>;
    // Separate arrays per buffer so the compiler can tell the buffer being
    // filled from the buffers being read.
    __shared__ __attribute__((aligned(1024))) uint16_t kbuf0[L::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t kbuf1[L::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vbuf0[L::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vbuf1[L::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool leader = wave < LOADERS;  // waves 0..3 lead and load; 4..7 trail
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
    const uint16_t *K = static_cast<const uint16_t *>(p.k) + ((int64_t)b * p.Hkv + g) * Nk * D;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + ((int64_t)b * p.Hkv + g) * Nk * D;

    Wave<D, EXPLICIT, CAP> st;
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
        st.lo_rel[0] = (int)(lo < -1 ? -1 : (lo > 0x3fffffff ? 0x3fffffff : lo));
        st.hi_rel[0] = (int)(hi < -1 ? -1 : (hi > 0x3fffffff ? 0x3fffffff : hi));
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qrow < Nq) x = ldg16(Q + qrow * D + ds * 16 + hf * 8);
            st.qf[0][ds] = __builtin_bit_cast(bf16x8, x);
        }
        st.m[0] = kNegInf;
        st.mtrue[0] = kNegInf;
        st.l[0] = 0.0f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) st.oacc[0][db][j] = 0.0f;
    }
    // K operand reads: row kb*32 + l32, chunk 2*ds + hf.
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) st.koff[ds] = (l32 * L::CPR + L::kslot(l32, 2 * ds + hf)) * 16;
    // V^T operand reads: lane in group gq = lane/16 provides row 4*(gq/2) + e
    // (e = (lane%16)/4; + 16*ks, + 8 for the second read) and column
    // db*32 + 16*(gq%2) + 4*j (j = lane%4).
    {
        const int gq = lane >> 4, e = (lane & 15) >> 2, j = lane & 3;
        const int row = 4 * (gq >> 1) + e;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int c = db * 4 + 2 * (gq & 1) + (j >> 1);
            st.voff[db] = (row * L::CPR + L::vslot(row, c)) * 16 + (j & 1) * 8;
        }
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
    const int head_bytes = (int)(Nk * D * 2);
    const int ntiles = kend > kbeg ? (int)((kend - kbeg + BN - 1) / BN) : 0;
    const int kt0 = (int)kbeg;

    auto load_k = [&](int t, uint16_t *buf) {
        const int toff = (kt0 + t * BN) * D * 2;
#pragma unroll
        for (int u = 0; u < L::LPW; ++u)
            buffer_load_lds16(K, head_bytes, (lds_void *)(buf + (lw * L::LPW + u) * 64 * 8), k_goff[u], toff);
    };
    auto load_v = [&](int t, uint16_t *buf) {
        const int toff = (kt0 + t * BN) * D * 2;
#pragma unroll
        for (int u = 0; u < L::LPW; ++u)
            buffer_load_lds16(V, head_bytes, (lds_void *)(buf + (lw * L::LPW + u) * 64 * 8), v_goff[u], toff);
    };
    auto is_full = [&](int t) {
        const int64_t kt = kbeg + (int64_t)t * BN;
        return kt >= full_lo && kt + BN <= full_hi;
    };

    f32x16 sacc[RB][2];
    bf16x8 pf[RB][4];
    // Step j: matrix phase (loads for tiles j+1 / j by the leaders, scores of
    // tile j from kcur, P.V of tile j-1 from vprev), barrier, vector phase
    // (softmax of tile j), barrier.  kload/vload receive K of tile j+1 and V
    // of tile j.
    auto step = [&](int j, const uint16_t *kcur, const uint16_t *vprev, uint16_t *kload, uint16_t *vload) {
        if (leader) {
            if (j + 1 < ntiles) load_k(j + 1, kload);
            if (j < ntiles) load_v(j, vload);
        }
        if (j < ntiles) st.scores(kcur, sacc);
        if (j >= 1) st.pv(vprev, pf);
        __syncthreads();
        if (j < ntiles) {
            float alpha[RB];
            const bool move = is_full(j) ? st.template softmax<false>(sacc, j, pf, alpha)
                                         : st.template softmax<true>(sacc, j, pf, alpha);
            if (move) st.rescale(alpha);
        }
        if (leader) __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (leader && ntiles > 0) {
        load_k(0, kbuf0);
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    if (!leader) __syncthreads();  // trail the leaders by one phase
    // Tile j's K sits in kbuf[j % 2], its V in vbuf[j % 2].
    for (int j = 0; j <= ntiles; j += 2) {
        step(j, kbuf0, vbuf1, kbuf1, vbuf0);
        if (j + 1 > ntiles) break;
        step(j + 1, kbuf1, vbuf0, kbuf0, vbuf1);
    }
    if (leader) __syncthreads();  // same barrier count for both groups

    // ---- epilogue: O = acc / l.  Lane holds dims db*32 + 8*(j/4) + 4*hf + (j%4).
    if (qrow >= Nq) return;
    const float lr = st.l[0];
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
        if (p.lse && hf == 0) p.lse[row] = lr > 0.0f ? (st.m[0] + __log2f(lr)) * kLn2 : kNegInf;
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

template <int D, bool SPLIT, bool EXPLICIT, bool CAP>
int launch_one(const FwdParams &p, hipStream_t stream) {
    const int n_qtiles = (int)((p.Nq + BM - 1) / BM);
    const int64_t blocks = p.B * p.H * (int64_t)n_qtiles * p.num_splits;
    if (blocks <= 0) return FA_OK;
    if (blocks > 0x7fffffff) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, SPLIT, EXPLICIT, CAP>), dim3((unsigned)blocks), dim3(NT), 0, stream, p,
                       n_qtiles);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <int D, bool SPLIT>
int launch_s(const FwdParams &p, hipStream_t stream) {
    if (p.softcap > 0.0f) return launch_one<D, SPLIT, true, true>(p, stream);
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
