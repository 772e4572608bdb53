// fa_bf16_tile.h -- the LDS tile machinery of the bf16 MFMA forward kernels:
// K and V tiles of 64 keys streamed from HBM straight into LDS by a group of
// four loading waves (16 keys each), and each V tile transposed once into a
// V^T tile whose keys are permuted for the P.V operand.
#pragma once

#include "fa_device.h"
#include "fa_tile.h"

namespace fa {

constexpr int kTileKeys = 64;     // keys per K / V tile
constexpr int kTileLoaders = 4;   // waves that load (and transpose) one tile

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
struct BfTile {
    static constexpr int BN = kTileKeys;
    static constexpr int CPR = D / 8;              // 16-byte chunks per row
    static constexpr int TILE = BN * D;            // bf16 elements of one K or V tile
    static constexpr int LPW = BN * CPR / 64 / kTileLoaders;  // loads per loader wave per tile
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

__device__ __forceinline__ int lane_id() {
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Direct tile loads of one loading wave (lw = 0..3 within its group) for
// D = 128.  K and V tiles are stored row-major (one 256-byte row per key)
// with 16-byte chunks swizzled against bank conflicts:
//   K: chunk c of row r in slot c ^ (r % 16) -- the MFMA operand read of
//      32 consecutive rows, same chunk, touches distinct banks;
//   V: chunk c of row r in slot c ^ 4 (r % 4) -- a transposing read
//      (ds_read_b64_tr_b16) covers 4 consecutive rows x 64 bytes per 32
//      lanes, and the xor puts the 4 rows' chunk quads on distinct banks.
// The per-lane offsets are recomputed from the lane id at each use (a few
// vector instructions per tile) instead of being kept in registers through
// the attention loop.
struct TileLoader128 {
    static constexpr int D = 128;
    using L = BfTile<D>;
    static_assert(L::LPW == 4 && L::CPR == 16, "offsets below are derived for D = 128");
    int lw;

    // Load u fills LDS chunk slots q*64 + lane (q = 4 lw + u) of a tile:
    // row rr = 16 lw + 4 u + lane/16, slot sl = lane % 16, which holds
    // chunk sl ^ (rr % 16) = sl ^ (lane/16) ^ 4u of K, or sl ^ 4 (lane/16)
    // of V (xor is its own inverse).  Byte offset in the head: the tile's
    // offset (scalar), a per-lane base (xor-ed with 64 u for K) and 1024 u.
    // The four loads of a wave share one M0 value: the 1024 u steps go in
    // the instruction offset, which the hardware adds to both the global
    // and the LDS address.  head_bytes = 0 makes every load read zeros
    // without touching memory (used when there is no next tile, so that
    // the loads need no branch).
    template <bool IS_V>
    __device__ __forceinline__ void load(const void *base, uint32_t head_bytes, uint32_t tile, int64_t kt) const {
        int lane = lane_id();
        asm volatile("" : "+v"(lane));
        const int x = lane >> 4, sl = lane & 15;
        const uint32_t g0 = (uint32_t)((16 * lw + x) * 256 + 16 * (IS_V ? (sl ^ (4 * x)) : (sl ^ x)));
        const uint64_t a = reinterpret_cast<uint64_t>(base);
        u32x4 rsrc;
        rsrc[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
        rsrc[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);  // stride 0
        rsrc[2] = __builtin_amdgcn_readfirstlane(head_bytes);                     // num_records
        rsrc[3] = 0x00020000u;                                                    // raw buffer, dword data
        const uint32_t m = __builtin_amdgcn_readfirstlane(tile + (uint32_t)(4 * lw * 1024));
        const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)kt * (uint32_t)(D * 2));
        uint32_t saved;
        if (IS_V) {
            asm volatile(
                "s_mov_b32 %0, m0\n\t"
                "s_mov_b32 m0, %1\n\t"
                "s_nop 0\n\t"
                "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
                "buffer_load_dwordx4 %2, %3, %4 offen offset:1024 lds\n\t"
                "buffer_load_dwordx4 %2, %3, %4 offen offset:2048 lds\n\t"
                "buffer_load_dwordx4 %2, %3, %4 offen offset:3072 lds\n\t"
                "s_mov_b32 m0, %0"
                : "=&s"(saved)
                : "s"(m), "v"(g0), "s"(rsrc), "s"(so)
                : "memory");
        } else {
            asm volatile(
                "s_mov_b32 %0, m0\n\t"
                "s_mov_b32 m0, %1\n\t"
                "s_nop 0\n\t"
                "buffer_load_dwordx4 %2, %6, %7 offen lds\n\t"
                "buffer_load_dwordx4 %3, %6, %7 offen offset:1024 lds\n\t"
                "buffer_load_dwordx4 %4, %6, %7 offen offset:2048 lds\n\t"
                "buffer_load_dwordx4 %5, %6, %7 offen offset:3072 lds\n\t"
                "s_mov_b32 m0, %0"
                : "=&s"(saved)
                : "s"(m), "v"(g0), "v"(g0 ^ 64u), "v"(g0 ^ 128u), "v"(g0 ^ 192u), "s"(rsrc), "s"(so)
                : "memory");
        }
    }
};

}  // namespace fa
