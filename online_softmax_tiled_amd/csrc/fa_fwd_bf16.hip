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
// Tiling on CDNA4:
//   * workgroup = 4 waves = 128 query rows (32 per wave); key tiles of 64.
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
//   * K and V tiles go from HBM straight into LDS (global_load_lds, 16 B per
//     lane, no register staging), row-major with an XOR swizzle of the
//     16-byte chunks chosen so that the K operand reads (ds_read_b128) and
//     the transposing V reads (ds_read_b64_tr_b16, which hand each lane
//     four keys of one column: the V^T operand) are bank-conflict free.
//     Two LDS stages in separate arrays: the next tile's loads are in flight
//     while the current tile is computed.
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

constexpr int BM = 128;      // query rows per workgroup
constexpr int BN = 64;       // keys per tile
constexpr int NT = 256;      // threads per workgroup
constexpr float TAU = 8.0f;  // lazy-rescale threshold, log2 units

template <int D>
struct Smem {
    static constexpr int CPR = D / 8;              // 16-byte chunks per row
    static constexpr int TILE = BN * D;            // bf16 elements of one K or V tile
    static constexpr int LPW = BN * CPR / 64 / 4;  // wave load instructions per tile
    // Swizzled chunk slot of chunk c in row r.  K: c ^ (r % CPR) makes 16
    // consecutive rows' same chunk hit distinct banks; V: c ^ (2r % CPR)
    // does the same for the 4-row x 32-byte footprint of a transposing read.
    __device__ static int kslot(int r, int c) { return c ^ (r % CPR); }
    __device__ static int vslot(int r, int c) { return c ^ ((2 * r) % CPR); }
};

__device__ __forceinline__ u32x4 ldg16(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

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

// Online-softmax update for one 64-key tile and O^T += V^T P^T.
// sacc: raw scores q.k (S^T accumulator layout).  lo/hi: this lane's visible
// keys as offsets from the tile start, applied when `masked`.
// EXPLICIT: the transformed score t = cap(s*scale)*log2 e (or s*scale*log2 e
// for a non-positive scale) is formed per element; otherwise the row
// maximum is taken on raw scores (scale > 0) and t is folded into the FMA
// that feeds the exp.
template <int D, bool EXPLICIT, bool CAP>
__device__ __forceinline__ void tile_update(f32x16 (&sacc)[2], float &m, float &l, f32x16 (&oacc)[D / 32],
                                            const char *Vsb, const int (&voff)[D / 32], bool masked, int lo, int hi,
                                            int hf, float c_log2, float scale, float softcap) {
    using L = Smem<D>;
    if (EXPLICIT) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                sacc[kb][j] = CAP ? softcap_log2(sacc[kb][j] * scale, softcap) : sacc[kb][j] * c_log2;
    }
    if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int koff = kb * 32 + 8 * (j / 4) + 4 * hf + (j % 4);
                if (koff < lo || koff >= hi) sacc[kb][j] = kNegInf;
            }
    }
    float mt = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sacc[kb][j]);
    if (!EXPLICIT) mt *= c_log2;
    mt = row_max(mt);

    // Move the reference maximum only when it grew by more than TAU (any lane).
    if (__builtin_amdgcn_ballot_w64(mt > m + TAU) != 0) {
        const float m_new = fmaxf(m, mt);
        const float alpha = fast_exp2(m - (m_new == kNegInf ? 0.0f : m_new));
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        m = m_new;
    }
    const float m_use = m == kNegInf ? 0.0f : m;

    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float pj = EXPLICIT ? fast_exp2(sacc[kb][j] - m_use) : fast_exp2(fmaf(sacc[kb][j], c_log2, -m_use));
            sacc[kb][j] = pj;
            rs += pj;
        }
    l += row_sum(rs);

    // O^T += V^T P^T.  k-step (kb, gp) covers keys kb*32 + 16*gp + [0, 16):
    // this lane half supplies keys +4*hf+[0,4) and +8+4*hf+[0,4), which are
    // exactly accumulator elements 8*gp .. 8*gp+7.
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            u32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = pack_bf16x2(sacc[kb][8 * gp + 2 * e], sacc[kb][8 * gp + 2 * e + 1]);
            pf[kb * 2 + gp] = __builtin_bit_cast(bf16x8, x);
        }
    // V^T operand: two transposing reads give this lane the keys
    // +4*hf+[0,4) and +8+4*hf+[0,4) of k-step ks at its column db*32 + lane%32.
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const char *base = Vsb + voff[db] + ks * 16 * L::CPR * 16;
            const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base));
            const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + 8 * L::CPR * 16));
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], oacc[db], 0, 0, 0);
        }
    }
}

template <int D, bool SPLIT, bool EXPLICIT, bool CAP>
__global__ __launch_bounds__(NT, 2) void fwd_bf16_kernel(const FwdParams p, const int n_qtiles) {
    using L = Smem<D>;
    // Two stages, each K tile then V tile; separate arrays so the compiler
    // can tell the stage being filled from the stage being read.
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[2 * L::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[2 * L::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // This lane's query row and its own visible interval, relative to kbeg.
    const int64_t qrow = q0 + wave * 32 + l32;
    int lo_rel, hi_rel;
    {
        int64_t lo, hi;
        key_bounds(qrow + off, Nk, p.causal, W, lo, hi);
        lo = (lo > r_lo ? lo : r_lo) - kbeg;
        hi = (hi < r_hi ? hi : r_hi) - kbeg;
        lo_rel = (int)(lo < -1 ? -1 : (lo > 0x3fffffff ? 0x3fffffff : lo));
        hi_rel = (int)(hi < -1 ? -1 : (hi > 0x3fffffff ? 0x3fffffff : hi));
    }

    const uint16_t *Q = static_cast<const uint16_t *>(p.q) + ((int64_t)b * p.H + h) * Nq * D;
    const uint16_t *K = static_cast<const uint16_t *>(p.k) + ((int64_t)b * p.Hkv + g) * Nk * D;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + ((int64_t)b * p.Hkv + g) * Nk * D;

    // Q^T fragments (the B operand of S^T = K Q^T): row qrow, 8 dims per step.
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qrow < Nq) x = ldg16(Q + qrow * D + ds * 16 + hf * 8);
        qf[ds] = __builtin_bit_cast(bf16x8, x);
    }

    const float c_log2 = p.scale * kLog2e;

    float m = kNegInf, l = 0.0f;
    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;

    const int ntiles = kend > kbeg ? (int)((kend - kbeg + BN - 1) / BN) : 0;
    const int kmax_row = (int)Nk - 1;  // keys past the end are clamped (and masked)

    // Global side of the direct loads: load u of this wave fills LDS chunk
    // slots q*64 + lane (q = wave*LPW + u) of the tile, i.e. row rr, slot sl.
    int g_row[L::LPW], g_col[L::LPW];
#pragma unroll
    for (int u = 0; u < L::LPW; ++u) {
        const int pos = (wave * L::LPW + u) * 64 + lane;
        g_row[u] = pos / L::CPR;
        g_col[u] = (pos % L::CPR) * 8;  // slot; the chunk it holds is per K / V
    }
    // K operand reads: row kb*32 + l32, chunk 2*ds + hf (bytes from the stage).
    int koff[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) koff[ds] = (l32 * L::CPR + L::kslot(l32, 2 * ds + hf)) * 16;
    // V^T operand reads (see tile_update): row 4*(hf) + e (+ 16*ks, + 8),
    // column db*32 + 16*(gq%2) + 4*j.
    int voff[D / 32];
    {
        const int gq = lane >> 4, e = (lane & 15) >> 2, j = lane & 3;
        const int row = 4 * (gq >> 1) + e;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int c = db * 4 + 2 * (gq & 1) + (j >> 1);
            voff[db] = L::TILE * 2 + (row * L::CPR + L::vslot(row, c)) * 16 + (j & 1) * 8;
        }
    }

    auto issue_loads = [&](int kt, uint16_t *stage) {
        const bool clamp = kt + BN > (int)Nk;
#pragma unroll
        for (int u = 0; u < L::LPW; ++u) {
            int key = kt + g_row[u];
            if (clamp) key = min(key, kmax_row);
            const int rr = g_row[u];
            const int kc = L::kslot(rr, g_col[u] / 8) * 8;  // chunk held by this slot (xor is an involution)
            const int vc = L::vslot(rr, g_col[u] / 8) * 8;
            lds_void *kdst = (lds_void *)(stage + (wave * L::LPW + u) * 64 * 8);
            lds_void *vdst = (lds_void *)(stage + L::TILE + (wave * L::LPW + u) * 64 * 8);
            __builtin_amdgcn_global_load_lds((const void *)(K + key * D + kc), kdst, 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(V + key * D + vc), vdst, 16, 0, 0);
        }
    };

    auto compute_tile = [&](int it, const uint16_t *stage) {
        const int kt = (int)kbeg + it * BN;
        const char *Ksb = reinterpret_cast<const char *>(stage);
        // ---- S^T = K Q^T for the 64 keys of this tile (two 32-key blocks)
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.0f;
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(Ksb + kb * 32 * L::CPR * 16 + koff[ds]);
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ds],
                                                                   sacc[kb], 0, 0, 0);
            }
        }
        const bool full = (int64_t)kt >= full_lo && (int64_t)kt + BN <= full_hi;
        tile_update<D, EXPLICIT, CAP>(sacc, m, l, oacc, Ksb, voff, !full, lo_rel - it * BN, hi_rel - it * BN, hf,
                                      c_log2, p.scale, p.softcap);
    };

    if (ntiles > 0) {
        issue_loads((int)kbeg, lds0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    // Two tiles per trip so each half names its stages statically.
    for (int it = 0; it < ntiles; it += 2) {
        if (it + 1 < ntiles) issue_loads((int)kbeg + (it + 1) * BN, lds1);
        compute_tile(it, lds0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (it + 1 >= ntiles) break;
        if (it + 2 < ntiles) issue_loads((int)kbeg + (it + 2) * BN, lds0);
        compute_tile(it + 1, lds1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l.  Lane holds dims db*32 + 8*(j/4) + 4*hf + (j%4).
    if (qrow >= Nq) return;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int64_t row = ((int64_t)b * p.H + h) * Nq + qrow;
    if (!SPLIT) {
        uint16_t *O = static_cast<uint16_t *>(p.o) + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 x = {pack_bf16x2(oacc[db][4 * gq] * inv, oacc[db][4 * gq + 1] * inv),
                           pack_bf16x2(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv)};
                *reinterpret_cast<u32x2 *>(O + db * 32 + 8 * gq + 4 * hf) = x;
            }
        if (p.lse && hf == 0) p.lse[row] = l > 0.0f ? (m + __log2f(l)) * kLn2 : kNegInf;
    } else {
        const int64_t prow = row * p.num_splits + w.split;
        float *Op = p.o_part + prow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                f32x4 x = {oacc[db][4 * gq] * inv, oacc[db][4 * gq + 1] * inv, oacc[db][4 * gq + 2] * inv,
                           oacc[db][4 * gq + 3] * inv};
                *reinterpret_cast<f32x4 *>(Op + db * 32 + 8 * gq + 4 * hf) = x;
            }
        if (hf == 0) {
            p.m_part[prow] = l > 0.0f ? m * kLn2 : kNegInf;
            p.l_part[prow] = l;
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
