// Tile geometry shared by the bfloat16 chunk kernels (kda_chunk_pipe.hip and
// kda_chunk_ps.hip): 64-token chunks of four 16-token tiles, the layout of a
// stored 16x16 fp16 tile, and the numbering of the tiles of the lower block
// triangle ("Kimi K3 - Lesson 3 of 14 - Sequence axis": chunks sequential,
// 16-token tiles inside, keys rescaled by 1/Gamma within a tile).
#pragma once

#include "kda_device.h"

namespace kda {
namespace chunk {

constexpr int C = 64;             // tokens per chunk
constexpr int TILE = 16;          // tokens per tile
constexpr int NT = C / TILE;      // tiles per chunk
constexpr int LDT = TILE;         // row stride (elements) of a stored 16x16 tile
constexpr float LOG2E = 1.4426950408889634f;

// Element offset of the four-element group c (0..3) of row t of a stored
// 16x16 fp16 tile.  Rows are 32 bytes, so rows t and t + 8 fall in the same
// banks; rows 8..15 hold their groups in the order c ^ 2, so a half-wave
// writing rows 0..15 (groups 0,1 or 2,3) touches every bank once, and a
// transposed read (rows 4g + a, all four groups of each) still does.
__device__ __forceinline__ int tile_at(int t, int c) { return t * LDT + 4 * (c ^ ((t >> 2) & 2)); }
// The lane's address for a transposed read of such a tile (the offset
// h16::tr_offset gives for an unpermuted one, with the groups permuted).
__device__ __forceinline__ int tile_tr_offset(int lane) {
    return tile_at(4 * (lane >> 4) + ((lane & 15) >> 2), lane & 3);
}

// Tiles (m, n) of the lower block triangle, n <= m, and of the strict one, n < m.
__host__ __device__ constexpr int lower_index(int m, int n) { return m * (m + 1) / 2 + n; }
__host__ __device__ constexpr int strict_index(int m, int n) { return m * (m - 1) / 2 + n; }
template <int M> struct TileIndex { static constexpr int value = M; };
constexpr int NLOWER = NT * (NT + 1) / 2;
constexpr int NSTRICT = NT * (NT - 1) / 2;

// The q, k, g of one token row of one chunk, as raw storage bits.  A producer
// lane (g, r) holds token r of its tile, channels 16 blk + 4 g + (0..3).
template <int DK, typename GT>
struct RowIn {
    static constexpr int KT = DK / 16;
    Raw4<uint16_t> q[KT], k[KT];
    Raw4<GT> g[KT];
};

// A group of waves meets at an LDS counter: every wave adds one arrival and
// waits until `target` arrivals are counted, so LDS writes made before the
// meeting are visible to the group after it.  The wait is bounded: at most
// `spin_limit` sleeps between polls; the result is false when the bound
// expired first (the caller then marks its results as invalid).
__device__ __forceinline__ bool lds_meet(unsigned *arrivals, unsigned target, int lane, unsigned spin_limit) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    bool ok = false;
    for (unsigned it = 0;; ++it) {
        const unsigned seen = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(arrivals, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (seen >= target) { ok = true; break; }
        if (it >= spin_limit) break;
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    return ok;
}

}  // namespace chunk
}  // namespace kda
