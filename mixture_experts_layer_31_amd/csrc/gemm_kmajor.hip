// Grouped GEMMs with K-major operands: the products of the layer's backward.
//
// The backward contracts over indices that the forward's operands do not keep
// contiguous: u = dY W2 and dX = dH [W1; W3] run over the first index of the
// expert weights as stored, and the weight gradients dW2 = dY_perm^T act,
// dW1 = dH1^T X_perm, dW3 = dH3^T X_perm run over the token rows (CMU 15-779
// Lecture 21 notes, §7). Rather than transposing those operands in memory,
// their tiles go into LDS as stored, one 512-byte LDS row per k, and become
// MFMA fragments through the gfx950 LDS transpose read (ds_read_b64_tr_b16):
// within each group of 16 lanes, lane i receives as its element j the element
// i % 4 of the 8 bytes addressed by lane 4 j + i / 4 (measured on the device).
// When lane s of a group addresses row kb + s / 4, columns nb + 4 (s % 4) .. +3
// of a [k][n] tile, lane i holds k = kb .. kb + 3 of column nb + i, and two
// such reads (kb and kb + 4) give the 8 consecutive k values of one operand of
// v_mfma_f32_32x32x16_bf16, in the same lane layout as a K-contiguous read.
//
// One kernel, two modes:
//  * data (u, dX): the token rows as in the forward's kernels (K-contiguous,
//    gathered through src, grouped by a tile table, ragged tails skipped), the
//    expert's weights [K][N] read K-major; K may run over two matrices, W1 then
//    W3, split at ksplit.
//  * grouped K (dW): out[g] = A^T B over group g's rows [off[g], off[g+1]) of
//    two row-major operands; no padding is needed (rows past the group's end
//    read as zeros). Each 64-row slab of the fp32 tile goes out through LDS so
//    that every store instruction writes one whole 1 KB output row.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kKmBM = 256, kKmBN = 256;         // output tile
constexpr int kKmRowBytes = 512;                 // a K-major LDS row: 256 bf16 of one k

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;

__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(p));
}

// The two transpose reads of one operand fragment (k and k + 4 of the lane's
// 8), at byte offset off of a K-major tile, joined into the MFMA operand.
__device__ __forceinline__ bf16x8 km_frag(const unsigned char* tile, int off) {
  const s16x4 lo = lds_read_tr16(tile + off);
  const s16x4 hi = lds_read_tr16(tile + off + 4 * kKmRowBytes);
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Byte offset, in a K-major tile, of this lane's first transpose read for the
// 32-column block starting at column col (a multiple of 32) and k step kk = 0.
// Row kr's 16-byte chunks are XOR-swizzled by 4 (kr % 4): the 4 rows x 4 chunks
// that a half-wave reads land on 16 distinct bank groups.
__device__ __forceinline__ int km_frag_off(int lane, int col) {
  const int g = lane >> 4, s = lane & 15;
  const int kr = 8 * (g >> 1) + (s >> 2);                 // kr % 4 == s / 4
  const int chunk = (col >> 3) + 2 * (g & 1) + ((s >> 1) & 1);
  return kr * kKmRowBytes + ((chunk ^ (4 * (s >> 2))) << 4) + 8 * (s & 1);
}

// Grouped K, long groups: launch index -> (m_tile, n_tile) in blocks of
// kGkBlockM x kGkBlockN tiles of one group, one block per XCD at a time (block b
// on XCD b % 8), so the 32 workgroups an XCD holds share their A and B K-slices in
// its L2 (4 A and 8 B slices per K-step) instead of 32 A slices and one B slice in
// m-fastest order. Workgroups past a partial block's edge return.
constexpr int kGkBlockM = 4, kGkBlockN = 8;   // kGkBlockM * kGkBlockN workgroups per XCD
__host__ __device__ constexpr long long gk_blocks(int G, int n_single, int n_tiles) {
  return static_cast<long long>(G) * ((n_single + kGkBlockM - 1) / kGkBlockM) *
         ((n_tiles + kGkBlockN - 1) / kGkBlockN);
}
__device__ __forceinline__ void gk_tile_blocked(int max_tiles, int n_single, int n_tiles,
                                                int& m_tile, int& n_tile) {
  const int L = blockIdx.x, j = L >> 3;
  constexpr int per = kGkBlockM * kGkBlockN;
  const int b = (j / per) * 8 + (L & 7), r = j % per;
  const int mb = (n_single + kGkBlockM - 1) / kGkBlockM;
  const int nb = (n_tiles + kGkBlockN - 1) / kGkBlockN;
  const int g = b / (mb * nb), q = b % (mb * nb);
  const int mi = (q % mb) * kGkBlockM + r % kGkBlockM;
  const int ni = (q / mb) * kGkBlockN + r / kGkBlockM;
  m_tile = -1;
  n_tile = 0;
  if (mi >= n_single || ni >= n_tiles || g * n_single >= max_tiles) return;
  m_tile = g * n_single + mi;
  n_tile = ni;
}

}  // namespace

// ---------------------------------------------------------------- the kernel
//
// Four waves of 128 x 128 each (one per SIMD) over 256 x 256 tiles, and every
// operand tile filled by LDS-DMA in a ring of ST
// stages of 32 k: a K-major stage is 32 LDS rows of 512 bytes (one k, 256
// columns), a K-contiguous token stage 256 rows of 64 bytes, as in the forward's
// gemm_bf16_w4_kernel, whose K loop this kernel follows (stage kt + LA loaded at
// step kt into the slot of stage kt - 2, one barrier per step, the second
// k-slice's fragments read before the barrier and multiplied after it).
//
// The loads are issued from inline assembly (kmajor_dma16): with the builtin the
// compiler cannot tell which LDS bytes an LDS-DMA load writes, and it makes every
// transpose read wait for all loads in flight (vmcnt(0)), which empties the ring
// at each read. The assembly has no register outputs; the kernel's own vmcnt
// waits (in-order completion) order the loads against the reads, as they do in
// the forward kernels. M0, the load's LDS base, is an input operand of the
// statement, so the compiler writes it (one wait state before the load).
//
// Grouped K: rows past the group's end load a 16-byte zero chunk (both
// operands), so a ragged last stage adds nothing.
constexpr int kKw4BK = 32;                           // k per stage
constexpr int kKw4Half = kKw4BK * kKmRowBytes;       // one operand's stage: 16 KB
constexpr int kKw4Stage = 2 * kKw4Half;
constexpr int kKw4XRow = 64;                         // K-contiguous token row bytes per stage
#ifndef MOE_KW4_STAGES
#define MOE_KW4_STAGES 5
#endif
constexpr int kKw4Stages = MOE_KW4_STAGES;
static_assert(kKw4Stages * kKw4Stage <= static_cast<int>(kMaxLdsBytes), "ring must fit");

__device__ __attribute__((aligned(64))) const uint16_t kKmZeroChunk[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// 16 bytes per lane from g to LDS at l + 16 * lane (l wave-uniform).
__device__ __forceinline__ void kmajor_dma16(const void* g, const unsigned char* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t la =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(l)));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(la));
#else
  (void)g;
  (void)l;
#endif
}

template <bool GK, bool NF, int ST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gemm_kmajor_w4_kernel(const int32_t* __restrict__ tiles, int max_tiles, int n_single,
                      int n_logical, const uint16_t* __restrict__ xa, int lda,
                      const int32_t* __restrict__ src, int a_row0,
                      const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb,
                      int ksplit, int ldw, long long w_stride, float* __restrict__ out,
                      int out_stride, int out_row0, int K, float* __restrict__ out2) {
  constexpr int BM = 256, BN = 256;
  constexpr int ND = 8;        // LDS-DMA loads per wave per stage (4 token / A, 4 weight / B)
  constexpr int LA = ST - 2;   // stages loaded ahead
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // data mode with out2: the grid holds the tile grid twice; the second copy runs
  // k in [ksplit, K) into out2, the first k in [0, ksplit) into out
  int L = blockIdx.x, kbase = 0;
  if (!GK && out2 != nullptr) {
    const int half = gridDim.x >> 1;
    if (L >= half) {
      L -= half;
      kbase = ksplit;
      out = out2;
    }
    K = kbase ? K - ksplit : ksplit;
  }
  int m_tile, n_tile;
  if constexpr (NF) xcd_tile_nfast_at(L, max_tiles, n_logical / max_tiles, m_tile, n_tile);
  else if constexpr (GK) gk_tile_blocked(max_tiles, n_single, n_logical / max_tiles, m_tile, n_tile);
  else xcd_tile_at(L, n_logical, max_tiles, m_tile, n_tile);
  if (m_tile < 0) return;
  const int n0 = n_tile * BN;

  TileCoord tc;
  int nk, nk_full, kbeg = 0, kend = 0, m0 = 0;   // nk_full: stages with no row past the group
  size_t obase = 0;
  if constexpr (GK) {
    const int g = m_tile / n_single;
    tc.group = g;
    tc.row0 = 0;
    tc.rows = BM;
    m0 = (m_tile % n_single) * BM;
    kbeg = tiles[g];
    kend = tiles[g + 1];
    nk = (kend - kbeg + kKw4BK - 1) / kKw4BK;
    nk_full = (kend - kbeg) / kKw4BK;
    obase = static_cast<size_t>(g) * static_cast<size_t>(w_stride) +
            static_cast<size_t>(m0) * out_stride;
  } else {
    tc = lookup_tile(tiles, n_single, BM, m_tile);
    if (tc.rows <= 0) return;
    nk = K / kKw4BK;
    nk_full = nk;
  }

  // K-major loads: load j of this wave fills LDS rows 8 j + 2 wave + h (h = lane /
  // 32) of its operand's half; lane l writes that row's physical chunk l % 32,
  // which holds logical chunk (l % 32) ^ 4 (row % 4), the swizzle km_frag_off reads
  const int h = lane >> 5;
  const int krow = 2 * wave + h;   // row of load 0; load j adds 8 j
  const int kchunk = (lane & 31) ^ (4 * (krow & 3));
  // GK: both operands K-major over the group's rows; data: B only
  const uint16_t* pb0;   // GK: B at k = krow of stage 0
  size_t boffs = 0;      // data: B element offset of k = krow in either matrix
  const uint16_t* pa0 = nullptr;
  const uint16_t* xg[4] = {nullptr, nullptr, nullptr, nullptr};
  int klim = 0;   // GK: k offsets (within the group) below this are in the group
  if constexpr (GK) {
    pa0 = xa + static_cast<size_t>(kbeg + krow) * lda + m0 + 8 * kchunk;
    pb0 = wa + static_cast<size_t>(kbeg + krow) * ldw + n0 + 8 * kchunk;
    klim = kend - kbeg - krow;
  } else {
    pb0 = nullptr;
    boffs = static_cast<size_t>(tc.group) * static_cast<size_t>(w_stride) +
            static_cast<size_t>(krow) * ldw + n0 + 8 * kchunk;
    // token rows as in gemm_bf16_w4_kernel: load j fills rows 16 (4 j + wave) +
    // lane / 4, physical chunk lane % 4 = logical chunk (lane % 4) ^ ((lane >> 3) & 3)
    const int lrow = lane >> 2;
    const int lchunk = (lane & 3) ^ ((lane >> 3) & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * (4 * j + wave) + lrow;
      int grow = tc.row0 + min(r, tc.rows - 1);
      if (src != nullptr) grow = src[grow];
      xg[j] = xa + (static_cast<size_t>(a_row0) + grow) * lda + lchunk * 8;
    }
  }
  auto dma = [&](int kt, int buf) {
    unsigned char* st = lds_raw + buf * kKw4Stage;
    const int kb = kbase + kt * kKw4BK;
    if constexpr (GK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = kb + 8 * j < klim;
        const size_t off = static_cast<size_t>(kb + 8 * j);
        const void* ga = ok ? static_cast<const void*>(pa0 + off * lda)
                            : static_cast<const void*>(kKmZeroChunk);
        const void* gb = ok ? static_cast<const void*>(pb0 + off * ldw)
                            : static_cast<const void*>(kKmZeroChunk);
        kmajor_dma16(ga, st + (8 * j + 2 * wave) * kKmRowBytes);
        kmajor_dma16(gb, st + kKw4Half + (8 * j + 2 * wave) * kKmRowBytes);
      }
    } else {
      // one weight matrix per stage (ksplit is a multiple of 32)
      const bool second = kb >= ksplit;
      const uint16_t* pb = (second ? wb : wa) + boffs +
                           static_cast<size_t>(second ? kb - ksplit : kb) * ldw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kmajor_dma16(xg[j] + kb, st + (4 * j + wave) * 16 * kKw4XRow);
        kmajor_dma16(pb + static_cast<size_t>(8 * j) * ldw,
                     st + kKw4Half + (8 * j + 2 * wave) * kKmRowBytes);
      }
    }
  };

  // fragments: B blocks b = columns (4 wn + b) * 32; A / token blocks a = rows
  // (2 a + wm) * 32
  const int frow = lane & 31, fhi = lane >> 5;
  int boff[4], aoff[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) boff[b] = kKw4Half + km_frag_off(lane, (4 * wn + b) * 32);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if constexpr (GK) aoff[a] = km_frag_off(lane, (2 * a + wm) * 32);
    else aoff[a] = (2 * a + wm) * 32 * kKw4XRow + frow * kKw4XRow;
  }
  const int fsw = (frow >> 1) & 3;
  const int xoff0 = ((0 + fhi) ^ fsw) << 4, xoff1 = ((2 + fhi) ^ fsw) << 4;

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  auto rfrag = [&](int buf, int kk, bf16x8 (&fa)[4], bf16x8 (&fb)[4], auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    const unsigned char* st = lds_raw + buf * kKw4Stage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = km_frag(st, boff[i] + kk * 16 * kKmRowBytes);
      if (i < NA) {
        if constexpr (GK) fb[i] = km_frag(st, aoff[i] + kk * 16 * kKmRowBytes);
        else fb[i] = *reinterpret_cast<const bf16x8*>(st + aoff[i] + (kk ? xoff1 : xoff0));
      }
    }
  };
  auto mfmas = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4], auto na_c) {
    constexpr int NA = decltype(na_c)::value;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b], fb[a], acc[a][b], 0, 0, 0);
  };

  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
  auto step = [&](int kt, auto na_c) {
    const int later = min(LA - 1, nk - 1 - kt);
    if (later == LA - 1) MOE_WAIT_VMCNT((LA - 1) * ND);
    else wait_vmcnt_at_most<(LA - 1) * ND>(later * ND);
    lds_barrier();   // publishes stage kt
    const int cur = kt % ST;
    if (kt + LA < nk) dma(kt + LA, (kt + LA) % ST);
    MOE_SCHED_FENCE();
    rfrag(cur, 0, fa0, fb0, na_c);
    if (kt > 0) mfmas(fa1, fb1, na_c);
    rfrag(cur, 1, fa1, fb1, na_c);
    mfmas(fa0, fb0, na_c);
  };
  // The steady-state step of a full tile, in sixteen bundles kept in order by
  // scheduling fences (the loads are inline assembly, which the scheduler's
  // instruction groups cannot place): bundle i of the first half issues two
  // MFMAs of the previous step's second k-slice and reads fragment i of this
  // step's first slice; bundle i of the second half issues two MFMAs of the first
  // slice, one load of stage kt + LA and fragment i of the second slice.
  // Fragments in the order the MFMAs (a = m / 4, b = m % 4) first use them:
  // A/token block 0, B blocks 0..3, A/token blocks 1..3.
  auto frag_one = [&](int buf, int kk, int f, bf16x8(&fa)[4], bf16x8(&fb)[4]) {
    const unsigned char* st = lds_raw + buf * kKw4Stage;
    if (f == 0 || f >= 5) {
      const int a = f == 0 ? 0 : f - 4;
      if constexpr (GK) fb[a] = km_frag(st, aoff[a] + kk * 16 * kKmRowBytes);
      else fb[a] = *reinterpret_cast<const bf16x8*>(st + aoff[a] + (kk ? xoff1 : xoff0));
    } else {
      fa[f - 1] = km_frag(st, boff[f - 1] + kk * 16 * kKmRowBytes);
    }
  };
  auto mfma_one = [&](const bf16x8(&fa)[4], const bf16x8(&fb)[4], int m) {
    acc[m >> 2][m & 3] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m & 3], fb[m >> 2], acc[m >> 2][m & 3], 0, 0, 0);
  };
  // load i of a full stage (no row checks): GK i < 4 A rows, else B rows; data
  // i < 4 token rows, else weight rows
  auto dma_one = [&](int kt, int buf, int i) {
    unsigned char* st = lds_raw + buf * kKw4Stage;
    const int kb = kbase + kt * kKw4BK;
    const int j = i & 3;
    if constexpr (GK) {
      const size_t off = static_cast<size_t>(kb + 8 * j);
      if (i < 4) kmajor_dma16(pa0 + off * lda, st + (8 * j + 2 * wave) * kKmRowBytes);
      else kmajor_dma16(pb0 + off * ldw, st + kKw4Half + (8 * j + 2 * wave) * kKmRowBytes);
    } else {
      if (i < 4) {
        kmajor_dma16(xg[j] + kb, st + (4 * j + wave) * 16 * kKw4XRow);
      } else {
        const bool second = kb >= ksplit;
        const uint16_t* pb = (second ? wb : wa) + boffs +
                             static_cast<size_t>((second ? kb - ksplit : kb) + 8 * j) * ldw;
        kmajor_dma16(pb, st + kKw4Half + (8 * j + 2 * wave) * kKmRowBytes);
      }
    }
  };
  auto main_step = [&](int kt, auto slot_c) {
    constexpr int S = decltype(slot_c)::value;
    constexpr int DS = (S + LA) % ST;
    MOE_WAIT_VMCNT((LA - 1) * ND);
    lds_barrier();
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_sched_barrier(0);
#endif
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mfma_one(fa1, fb1, 2 * i);
      mfma_one(fa1, fb1, 2 * i + 1);
      frag_one(S, 0, i, fa0, fb0);
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mfma_one(fa0, fb0, 2 * i);
      mfma_one(fa0, fb0, 2 * i + 1);
      dma_one(kt + LA, DS, i);
      frag_one(S, 1, i, fa1, fb1);
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
  };
  auto kloop = [&](auto na_c) {
    constexpr int NA = decltype(na_c)::value;
#pragma unroll
    for (int p = 0; p < LA; ++p)
      if (p < nk) dma(p, p);
    int kt = 0;
    if constexpr (NA == 4) {
      for (; kt < ST && kt < nk; ++kt) step(kt, na_c);
      for (; kt + ST - 1 + LA < nk_full; kt += ST) {
        main_step(kt, std::integral_constant<int, 0>{});
        main_step(kt + 1, std::integral_constant<int, 1>{});
        main_step(kt + 2, std::integral_constant<int, 2>{});
        main_step(kt + 3, std::integral_constant<int, 3>{});
        if constexpr (ST > 4) main_step(kt + 4, std::integral_constant<int, 4 % ST>{});
        if constexpr (ST > 5) main_step(kt + 5, std::integral_constant<int, 5 % ST>{});
      }
    }
    for (; kt < nk; ++kt) step(kt, na_c);
    if (nk > 0) mfmas(fa1, fb1, na_c);
  };

  if constexpr (GK) {
    kloop(std::integral_constant<int, 4>{});
    // staged epilogue: slab a holds token blocks 2 a and 2 a + 1 (64 rows); each
    // store instruction then writes one whole 1 KB output row
    constexpr int P = BN + 4;   // floats per staged row
    static_assert(64 * P * 4 <= ST * kKw4Stage, "staged slab fits the ring");
    float* stg = reinterpret_cast<float*>(lds_raw);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      __syncthreads();   // the K loop's / previous slab's reads are done
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[a][b][4 * rq + q];
          *reinterpret_cast<f32x4*>(stg + (wm * 32 + frow) * P + (4 * wn + b) * 32 + 8 * rq +
                                    4 * fhi) = v;
        }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int srow = wave * 16 + j;
        const int m = (2 * a + srow / 32) * 32 + (srow & 31);
        const f32x4 v = *reinterpret_cast<const f32x4*>(stg + srow * P + lane * 4);
        float* o = out + obase + static_cast<size_t>(m) * out_stride + n0 + lane * 4;
        if constexpr (NF) *reinterpret_cast<f32x4*>(o) = v;
        else __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(o));
      }
    }
  } else {
    const int nb = (min(tc.rows, BM) + 31) / 32;
    with_count<4>((nb - wm + 1) / 2, kloop);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int m = (2 * a + wm) * 32 + frow;
      if (m >= tc.rows) continue;
      const size_t orow = static_cast<size_t>(out_row0) + tc.row0 + m;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int n = n0 + (4 * wn + b) * 32 + 8 * rq + 4 * fhi;
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[a][b][4 * rq + q];
          *reinterpret_cast<f32x4*>(out + orow * out_stride + n) = v;
        }
    }
  }
}

hipError_t launch_gemm_kmajor_data(const GemmTileMap& map, const KmDataArgs& a, hipStream_t s) {
  if (a.K % kKw4BK || a.ksplit % kKw4BK || a.N % kKmBN || a.lda % 8 || a.ldw % 8)
    return hipErrorInvalidValue;
  if (a.y2 != nullptr && (a.ksplit <= 0 || a.ksplit >= a.K)) return hipErrorInvalidValue;
  // weight-streaming shapes (gemm_n_fast): the n tiles of each m tile together
  auto kern = map.n_fast ? gemm_kmajor_w4_kernel<false, true, kKw4Stages>
                         : gemm_kmajor_w4_kernel<false, false, kKw4Stages>;
  constexpr size_t lds = static_cast<size_t>(kKw4Stages) * kKw4Stage;
  const dim3 block(256);
  hipError_t e = allow_large_lds(reinterpret_cast<const void*>(kern), lds);
  if (e != hipSuccess) return e;
  const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + kKmBM - 1) / kKmBM;
  const long long n_logical = static_cast<long long>(m_tiles) * (a.N / kKmBN);
  if (n_logical == 0) return hipSuccess;
  const long long grid = (map.n_fast ? 8LL * ((m_tiles + 7) / 8) * (a.N / kKmBN)
                                     : ((n_logical + 7) / 8) * 8) *
                         (a.y2 != nullptr ? 2 : 1);
  kern<<<dim3(static_cast<unsigned>(grid)), block, lds, s>>>(
      map.tiles, m_tiles, map.n_single, static_cast<int>(n_logical), a.x, a.lda, a.src, a.x_row0,
      a.wa, a.wb, a.ksplit, a.ldw, a.w_stride, a.y, a.y_stride, a.y_row0, a.K, a.y2);
  return hipGetLastError();
}

// Short groups (DeepSeek shape: ~128 rows each) make the weight gradients a
// write stream of 256 KB per tile after two K-steps. Measured on a store-only
// probe of that pattern (15 GB): m-fastest with nontemporal stores 4.8 TB/s,
// n-fastest with plain stores 6.0 TB/s (neighbouring tiles complete whole
// output rows together); in the product, dW 3.6 -> 3.4 ms each. Long groups
// (Mixtral shape) keep m-fastest and nontemporal stores.
hipError_t launch_gemm_kmajor_groupk(const int32_t* offsets, int G, const uint16_t* A, int lda,
                                     int N1, const uint16_t* B, int ldb, int N2, float* out,
                                     bool rows_stream, hipStream_t s) {
  if (N1 % kKmBM || N2 % kKmBN || lda % 8 || ldb % 8) return hipErrorInvalidValue;
  auto kern = rows_stream ? gemm_kmajor_w4_kernel<true, true, kKw4Stages>
                          : gemm_kmajor_w4_kernel<true, false, kKw4Stages>;
  constexpr size_t lds = static_cast<size_t>(kKw4Stages) * kKw4Stage;
  const dim3 block(256);
  hipError_t e = allow_large_lds(reinterpret_cast<const void*>(kern), lds);
  if (e != hipSuccess) return e;
  const int n_single = N1 / kKmBM;
  const int m_tiles = G * n_single;
  const long long n_logical = static_cast<long long>(m_tiles) * (N2 / kKmBN);
  if (n_logical == 0) return hipSuccess;
  const long long grid = rows_stream
                             ? 8LL * ((m_tiles + 7) / 8) * (N2 / kKmBN)
                             : (gk_blocks(G, n_single, N2 / kKmBN) + 7) / 8 * 8 * kGkBlockM * kGkBlockN;
  kern<<<dim3(static_cast<unsigned>(grid)), block, lds, s>>>(
      offsets, m_tiles, n_single, static_cast<int>(n_logical), A, lda, nullptr, 0, B, nullptr, 0,
      ldb, static_cast<long long>(N1) * N2, out, N2, 0, 0, nullptr);
  return hipGetLastError();
}

}  // namespace moe
