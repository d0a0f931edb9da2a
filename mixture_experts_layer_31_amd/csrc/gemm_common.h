// Device helpers shared by the grouped GEMM kernels (gemm_bf16.hip, gemm_kmajor.hip).
#pragma once
#include <type_traits>

#include "common.h"

namespace moe {

constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;   // LDS row pitch in bf16 elements (144 bytes)

struct TileCoord {
  int group, row0, rows;
};

__device__ __forceinline__ TileCoord lookup_tile(const int32_t* tiles, int n_single, int BM,
                                                 int m_tile) {
  TileCoord c;
  if (tiles != nullptr) {
    const int4 t = reinterpret_cast<const int4*>(tiles)[m_tile];
    c.group = t.x; c.row0 = t.y; c.rows = t.z;
  } else {
    c.group = 0; c.row0 = m_tile * BM; c.rows = min(BM, n_single - c.row0);
  }
  return c;
}

// Launch index -> (m_tile, n_tile), XCD-contiguous (see the file comment):
// m fastest over a contiguous range of (n, m) pairs per XCD.
// L: the launch index (a multiple of 8 apart from blockIdx.x when a launch runs
// several copies of the tile grid, so the XCD is the same).
__device__ __forceinline__ void xcd_tile_at(int L, int n_logical, int max_tiles, int& m_tile,
                                            int& n_tile) {
  const int per = (n_logical + 7) >> 3;
  const int logical = (L & 7) * per + (L >> 3);
  if (logical >= n_logical) { m_tile = -1; n_tile = 0; return; }
  m_tile = logical % max_tiles;
  n_tile = logical / max_tiles;
}
__device__ __forceinline__ void xcd_tile(int n_logical, int max_tiles, int& m_tile, int& n_tile) {
  xcd_tile_at(blockIdx.x, n_logical, max_tiles, m_tile, n_tile);
}

// Launch index -> (m_tile, n_tile) with the n tiles of one m tile in a row on
// one XCD: m tile m runs on XCD m % 8, its n_tiles tiles consecutively, so the
// workgroups that share its token rows share an L2 and stream neighbouring
// panels of one weight matrix at the same time; the empty m tiles at the end of
// the table fall evenly on all XCDs. Grid: 8 * ceil(max_tiles / 8) * n_tiles.
__device__ __forceinline__ void xcd_tile_nfast_at(int L, int max_tiles, int n_tiles, int& m_tile,
                                                  int& n_tile) {
  const int j = L >> 3;
  m_tile = (j / n_tiles) * 8 + (L & 7);
  n_tile = j % n_tiles;
  if (m_tile >= max_tiles) m_tile = -1;
}
__device__ __forceinline__ void xcd_tile_nfast(int max_tiles, int n_tiles, int& m_tile,
                                               int& n_tile) {
  xcd_tile_nfast_at(blockIdx.x, max_tiles, n_tiles, m_tile, n_tile);
}

// Launch index -> (m_tile, n_tile) in blocks of m tiles: XCD x owns the n tiles
// [x * n_tiles / 8, (x + 1) * n_tiles / 8) and walks one block of m tiles over all
// of them (m fastest), then the next block. Each weight panel is then read by one
// XCD only, and the workgroups in flight on an XCD share their token rows (the
// block's m tiles) as well as their weight panels (a few n tiles) in its L2; in
// m-fastest order over all m tiles they would share only the weight panels and
// read every token row again for every n tile.
// With a tile table the blocks are the table's order blocks (tile_block_word):
// all tiles of a group of up to eight, so the workgroups in flight on an XCD work
// on one expert's weights at a time. Slot j of XCD x lies in the block of tile
// j / nn (nn: the XCD's n tiles), which spans slots [nn * start, nn * (start +
// tiles)), so the grid is the same as for fixed blocks and no slot is wasted.
// Measured on the gate/up product of the Mixtral shape at 4096 tokens (groups of
// four or five 256-row tiles): 1.98 -> 1.90 ms against fixed blocks of two m
// tiles, which straddle the experts (fixed blocks of five: 1.97 ms). Without a
// table (one dense group), fixed blocks of kTileBlockM m tiles.
// Grid: blocked_grid(max_tiles, n_tiles).
#ifndef MOE_TILE_BLOCK_M
#define MOE_TILE_BLOCK_M 2
#endif
constexpr int kTileBlockM = MOE_TILE_BLOCK_M;
__host__ __device__ constexpr bool tile_order_blocked(int BM, int n_tiles) {
  return BM == 256 && n_tiles >= 16;   // enough n tiles for every XCD
}
__host__ __device__ constexpr long long blocked_grid(int max_tiles, int n_tiles) {
  return 8LL * ((max_tiles + kTileBlockM - 1) / kTileBlockM) * kTileBlockM * ((n_tiles + 7) / 8);
}
__device__ __forceinline__ void xcd_tile_blocked(const int32_t* tiles, int max_tiles, int n_tiles,
                                                 int& m_tile, int& n_tile) {
  const int L = blockIdx.x, x = L & 7, j = L >> 3;
  const int n_lo = x * n_tiles / 8;
  const int nn = (x + 1) * n_tiles / 8 - n_lo;
  m_tile = -1;
  n_tile = 0;
  if (nn <= 0) return;
  if (tiles != nullptr) {
    const int t = j / nn;
    if (t >= max_tiles) return;
    const int4 e = reinterpret_cast<const int4*>(tiles)[t];
    if (e.z <= 0) return;   // past the last real tile
    const int s0 = e.w >> 8, c = e.w & 255;
    const int r = j - nn * s0;
    m_tile = s0 + r % c;
    n_tile = n_lo + r / c;
    return;
  }
  const int per = kTileBlockM * nn;   // workgroups of one block on this XCD
  const int b = j / per, r = j - b * per;
  const int m = b * kTileBlockM + r % kTileBlockM;
  if (m >= max_tiles) return;
  m_tile = m;
  n_tile = n_lo + r / kTileBlockM;
}

#if defined(__HIP_DEVICE_COMPILE__)
// s_waitcnt with vmcnt = n and the other counters not waited on (gfx9 encoding)
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
// 16 bytes per lane from global memory to LDS at lds_base + 16 * lane
#define MOE_LDS_DMA16(g, l) __builtin_amdgcn_global_load_lds((g), (l), 16, 0, 0)
// s_waitcnt vmcnt(n) for a wave-uniform n <= N (the count is an immediate)
template <int N>
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
  if constexpr (N == 0) {
    MOE_WAIT_VMCNT(0);
  } else {
    if (n >= N) MOE_WAIT_VMCNT(N);
    else wait_vmcnt_at_most<N - 1>(n);
  }
}
// keeps vector-memory instructions on their side of this point; every other
// instruction kind may still be scheduled across it
#define MOE_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0x78F)
// Workgroup barrier for pipelines with LDS-DMA loads of later stages still in
// flight. __syncthreads() carries a workgroup fence, for which the compiler
// waits for every outstanding vector-memory load (an LDS-DMA load counts as a
// pending LDS write), so it would drain those stages too. Here each wave has
// already waited (s_waitcnt vmcnt) for the loads of the stage it is about to
// publish; the barrier then waits only for the wave's own LDS accesses
// (lgkmcnt(0)), and the empty asm statements keep the compiler from moving any
// memory access across it.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Workgroup barrier that waits for no memory counter at all: for rings whose
// stages are published by each wave's own s_waitcnt vmcnt and whose slot reuse
// is ordered by the MFMAs that consumed the slot's fragments (those MFMAs waited
// for their LDS reads). The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
#else
#define MOE_SCHED_FENCE() ((void)0)
__device__ __forceinline__ void dma_barrier() {}
__device__ __forceinline__ void lds_barrier() {}
template <int N>
__device__ __forceinline__ void wait_vmcnt_at_most(int) {}
#define MOE_WAIT_VMCNT(n) ((void)0)
#define MOE_LDS_DMA16(g, l) ((void)(g), (void)(l))
#endif

constexpr int kRowBytes = 128;   // one LDS row holds 64 bf16 of K
constexpr size_t kMaxLdsBytes = 160 * 1024;   // LDS per workgroup on gfx950
constexpr int kNumCUs = 256;                    // MI355X

// The next stage's LDS-DMA loads are spread over this many points of the
// K-step instead of issued in one burst after the barrier: a burst of 1 KB
// loads from every wave fills the CU's vector-memory queue, and the waves
// then stall at their later loads instead of issuing MFMAs.
#ifndef MOE_DMA_SLICES
#define MOE_DMA_SLICES 2
#endif
constexpr int kDmaSlices = MOE_DMA_SLICES;
static_assert(kDmaSlices == 1 || kDmaSlices == 2 || kDmaSlices == 4, "1, 2 or 4 slices");
#ifndef MOE_DMA_SLICES3
#define MOE_DMA_SLICES3 4
#endif
constexpr int kDmaSlices3 = MOE_DMA_SLICES3;   // with three LDS stages
static_assert(kDmaSlices3 == 1 || kDmaSlices3 == 2 || kDmaSlices3 == 4, "1, 2 or 4 slices");

// f(integral_constant<int, min(n, N)>) for 0 <= n: a runtime count turned into
// a compile-time one, so each count gets its own fully unrolled code.
template <int N, class F>
__device__ __forceinline__ void with_count(int n, F&& f) {
  if constexpr (N == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (n >= N) f(std::integral_constant<int, N>{});
    else with_count<N - 1>(n, f);
  }
}

}  // namespace moe
