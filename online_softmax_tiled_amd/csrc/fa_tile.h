// fa_tile.h -- pieces shared by the MFMA forward kernels (bf16 and fp8):
// direct HBM -> LDS tile loads, an LDS-only workgroup barrier, the
// read/MFMA interleave recipe, half-row reductions over the lane pair of a
// 32x32 accumulator, and the XCD-aware block order.
#pragma once

#include "fa_device.h"

namespace fa {

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from base + voff + soff straight into LDS (dst + 16*lane).
// The buffer resource bounds the access to [base, base + nbytes): bytes past
// the end read as zero.  base, nbytes, dst and soff are wave-uniform; nbytes
// and soff are unsigned 32-bit byte counts (a head of K or V is at most
// 2^31 - 1 elements, so up to 2^32 - 2 bytes in bf16).
//
// Written as inline assembly so that the compiler does not see an LDS write
// in flight: it would otherwise wait for every such load to land before the
// next LDS read of any buffer.  The kernels wait for these loads themselves
// (s_waitcnt vmcnt) before the barrier that hands the tile to other waves.
// The instruction has no result register; M0 (the LDS address) is saved and
// restored around it.
__device__ __forceinline__ void buffer_load_lds16(const void *base, uint32_t nbytes, lds_void *dst, int voff,
                                                  uint32_t soff) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 rsrc;
    rsrc[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    rsrc[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);  // stride 0
    rsrc[2] = __builtin_amdgcn_readfirstlane(nbytes);                         // num_records
    rsrc[3] = 0x00020000u;                                                    // raw buffer, dword data
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(dst));
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m), "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory");
}

// The same load with the LDS destination given as a wave-uniform LDS byte
// address (no generic-to-LDS pointer conversion at each call).
__device__ __forceinline__ void buffer_load_lds16_at(const void *base, uint32_t nbytes, uint32_t lds_addr, int voff,
                                                     uint32_t soff) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 rsrc;
    rsrc[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    rsrc[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);  // stride 0
    rsrc[2] = __builtin_amdgcn_readfirstlane(nbytes);                         // num_records
    rsrc[3] = 0x00020000u;                                                    // raw buffer, dword data
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m), "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory");
}

// Workgroup barrier for LDS traffic only: it waits for this wave's LDS
// reads and writes but not for its loads still streaming into LDS, which
// __syncthreads() also drains (its fence counts them as LDS writes).  A
// wave that filled LDS for others waits for its own loads explicitly before
// the barrier that publishes them.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Scheduling recipe for a run of NREAD operand reads from LDS, each feeding
// PER MFMAs: issue PF reads ahead, then alternate PER MFMAs with one read,
// then drain.  Without it the reads are issued just before their MFMAs and
// every MFMA waits the full LDS latency.
template <int NREAD, int PER, int PF>
__device__ __forceinline__ void sched_read_mfma_pipeline() {
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < NREAD - PF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PF * PER, 0);
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

__device__ __forceinline__ Work decode_block(const FwdParams &p, int n_qtiles, int cluster_blocks = 64) {
    const int bid = blockIdx.x;
    const int rep = p.group, S = p.num_splits;
    const int units = (int)(p.B * p.Hkv);
    const int per_unit = rep * n_qtiles * S;
    int unit, r;
    if (units % 8 == 0 && p.causal) {
        // Causal tiles differ in length.  Each XCD takes its units in
        // clusters of C; inside a cluster the blocks run longest query tile
        // first across the cluster's units, so short tiles fill in at the
        // end of each cluster (one unit at a time, longest first, left the
        // last unit's long tiles in the tail).  C is the fewest units whose
        // blocks reach cluster_blocks, about twice the workgroups an XCD
        // holds at once (64 for one workgroup per CU, 128 for two): enough
        // to balance, while only about C units' K and V are live in the
        // XCD's L2 at a time (ordering across all units at once multiplied
        // the HBM reads of K and V).
        const int x = bid & 7, s = bid >> 3;
        const int upx = units / 8;
        const int unit_blocks = per_unit;
        const int C = min(upx, max(1, (cluster_blocks + unit_blocks - 1) / unit_blocks));
        const int c0 = (s / (C * unit_blocks)) * C;
        const int csz = min(C, upx - c0);
        const int rem = s - c0 * unit_blocks;
        const int per_rank = csz * rep * S;
        const int rank = rem / per_rank, rr = rem % per_rank;
        unit = (c0 + rr / (rep * S)) * 8 + x;
        r = rank * (rep * S) + rr % (rep * S);
    } else if (units % 8 == 0) {
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

}  // namespace fa
