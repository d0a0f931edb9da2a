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
// 256 x 256 output tiles, BK = 64, eight waves, two LDS stages of 64 KB filled
// through registers; two modes:
//  * data (u, dX): the token rows as in the forward's kernels (K-contiguous,
//    gathered through src, grouped by a tile table, ragged tails skipped), the
//    expert's weights [K][N] read K-major; K may run over two matrices, W1 then
//    W3, split at ksplit.
//  * grouped K (dW): out[g] = A^T B over group g's rows [off[g], off[g+1]) of
//    two row-major operands; rows past the group's end are zeroed in registers,
//    so no padding is needed. Each 64-row slab of the fp32 tile goes out through LDS
//    so that every store instruction writes one whole 1 KB output row.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kKmBM = 256, kKmBN = 256, kKmWM = 2, kKmWN = 4, kKmNW = kKmWM * kKmWN;
constexpr int kKmRowBytes = 512;                 // a K-major LDS row: 256 bf16 of one k
constexpr int kKmTile = kBK * kKmRowBytes;       // 32 KB per operand per stage
constexpr int kKmStage = 2 * kKmTile;
constexpr int kKmLds = 2 * kKmStage;             // two stages

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

}  // namespace

template <bool GK, bool NF = false>
__global__ __launch_bounds__(64 * kKmNW)
__attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kmajor_kernel(
    const int32_t* __restrict__ tiles, int max_tiles, int n_single, int n_logical,
    const uint16_t* __restrict__ xa, int lda, const int32_t* __restrict__ src, int a_row0,
    const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb, int ksplit, int ldw,
    long long w_stride, float* __restrict__ out, int out_stride, int out_row0, int K) {
  constexpr int BM = kKmBM, BN = kKmBN, WM = kKmWM, WN = kKmWN, NW = kKmNW;
  constexpr int MT = BM / WM / 32;   // 32-row token blocks per wave
  constexpr int NT = BN / WN / 32;   // 32-column output blocks per wave
  static_assert(64 * NW * 64 == kKmTile, "a stage's operand tile is 64 bytes per thread");

  extern __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[];

  int m_tile, n_tile;
  if constexpr (NF) xcd_tile_nfast(max_tiles, n_logical / max_tiles, m_tile, n_tile);
  else xcd_tile(n_logical, max_tiles, m_tile, n_tile);
  if (m_tile < 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int n0 = n_tile * BN;

  TileCoord tc;
  int nk, kbeg = 0, kend = 0, m0 = 0;
  size_t obase = 0;
  if constexpr (GK) {
    const int g = m_tile / n_single;
    tc.group = g;
    tc.row0 = 0;
    tc.rows = BM;
    m0 = (m_tile % n_single) * BM;
    kbeg = tiles[g];
    kend = tiles[g + 1];
    nk = (kend - kbeg + kBK - 1) / kBK;
    obase = static_cast<size_t>(g) * static_cast<size_t>(w_stride) + static_cast<size_t>(m0) * out_stride;
  } else {
    tc = lookup_tile(tiles, n_single, BM, m_tile);
    if (tc.rows <= 0) return;
    nk = K / kBK;
  }

  // Fill: each stage goes global -> registers -> LDS (16-byte loads, ds_write_b128),
  // loaded one K-step before it is written to LDS. LDS-DMA loads are not used:
  // while one is in flight the compiler holds every transpose read until it lands.
  // K-major tile: thread t loads row t / 8, logical chunks t % 8 + 8 q (q < 4);
  // row kr's chunk c sits at physical chunk c ^ 4 (kr % 4).
  const int skr = tid >> 3, sci = tid & 7;
  int km_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    km_off[q] = skr * kKmRowBytes + (((sci + 8 * q) ^ (4 * (skr & 3))) << 4);
  const int scol = 8 * sci;   // element column of chunk q: scol + 64 q
  // token tile (data mode): thread t loads row t / 2, chunks 4 (t % 2) + q, 128-byte
  // LDS rows with chunks XOR-swizzled by row as in the forward's kernel
  const int sxr = tid >> 1, sxh = tid & 1;
  int x_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) x_off[q] = sxr * kRowBytes + (((4 * sxh + q) ^ (sxr & 7)) << 4);
  const uint16_t* xrow = nullptr;
  bool xvalid = false;
  if constexpr (!GK) {
    xvalid = sxr < tc.rows;
    int grow = tc.row0 + min(sxr, tc.rows - 1);
    if (src != nullptr) grow = src[grow];
    xrow = xa + (static_cast<size_t>(a_row0) + grow) * lda + 32 * sxh;
  }
  const size_t wgroup = GK ? 0 : static_cast<size_t>(tc.group) * static_cast<size_t>(w_stride);
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  u32x4 rx[4], rw[4];
  bool rok = true;   // grouped K: the loaded row lies in the group (else written as zeros)
  auto gload = [&](int kt) {
    const int kglob = kt * kBK;
    if constexpr (GK) {
      // rows past the group's end load a valid row; swrite zeroes them
      const int r = kbeg + kglob + skr;
      rok = r < kend;
      const size_t rr = static_cast<size_t>(rok ? r : kbeg);
      const uint16_t* pa = xa + rr * lda + m0 + scol;
      const uint16_t* pb = wa + rr * ldw + n0 + scol;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rx[q] = *reinterpret_cast<const u32x4*>(pa + 64 * q);
        rw[q] = *reinterpret_cast<const u32x4*>(pb + 64 * q);
      }
    } else {
      // one weight matrix per 64-row step (ksplit is a multiple of 64)
      const uint16_t* wbase = kglob < ksplit ? wa + wgroup + static_cast<size_t>(kglob) * ldw
                                             : wb + wgroup + static_cast<size_t>(kglob - ksplit) * ldw;
      const uint16_t* pw = wbase + static_cast<size_t>(skr) * ldw + n0 + scol;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 vx = *reinterpret_cast<const u32x4*>(xrow + kglob + 8 * q);
        rx[q] = xvalid ? vx : zero4;
        rw[q] = *reinterpret_cast<const u32x4*>(pw + 64 * q);
      }
    }
  };
  auto swrite = [&](int buf) {
    unsigned char* xs = lds_raw + buf * kKmStage;
    unsigned char* ws = xs + kKmTile;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<u32x4*>(ws + km_off[q]) = rok ? rw[q] : zero4;
      *reinterpret_cast<u32x4*>(xs + (GK ? km_off[q] : x_off[q])) = rok ? rx[q] : zero4;
    }
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int frow = lane & 31, fhi = lane >> 5;
  int woff[NT], xoff[MT];
#pragma unroll
  for (int b = 0; b < NT; ++b) woff[b] = km_frag_off(lane, wn * (BN / WN) + b * 32);
#pragma unroll
  for (int a = 0; a < MT; ++a) xoff[a] = km_frag_off(lane, (a * WM + wm) * 32);
  int koff[4];   // K-contiguous token fragments (data mode)
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = frow * kRowBytes + (((2 * kk + fhi) ^ (frow & 7)) << 4);

  bf16x8 fa[4][NT], fb[4][MT];
  auto rfrag = [&](int buf, int kk, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    const unsigned char* xs = lds_raw + buf * kKmStage;
    const unsigned char* ws = xs + kKmTile;
#pragma unroll
    for (int b = 0; b < NT; ++b) fa[kk][b] = km_frag(ws, woff[b] + kk * 16 * kKmRowBytes);
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      if constexpr (GK)
        fb[kk][a] = km_frag(xs, xoff[a] + kk * 16 * kKmRowBytes);
      else
        fb[kk][a] = *reinterpret_cast<const bf16x8*>(xs + (a * WM + wm) * 32 * kRowBytes + koff[kk]);
    }
  };
  auto mfmas = [&](int kk, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int b = 0; b < NT; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][b], fb[kk][a], acc[a][b], 0, 0, 0);
  };

  // one barrier per K-step: it publishes the stage written at the end of the
  // previous step and retires this step's reads of the buffer the next write
  // fills; global loads run one step ahead of their LDS write
  auto kloop = [&](auto na_c) {
    if (nk > 0) {
      gload(0);
      swrite(0);
    }
    if (nk > 1) gload(1);
    __syncthreads();
    int cur = 0;
    for (int kt = 0; kt < nk; ++kt) {
      rfrag(cur, 0, na_c);
      rfrag(cur, 1, na_c);
      mfmas(0, na_c);
      rfrag(cur, 2, na_c);
      mfmas(1, na_c);
      rfrag(cur, 3, na_c);
      mfmas(2, na_c);
      mfmas(3, na_c);
      if (kt + 1 < nk) {
        swrite(cur ^ 1);
        if (kt + 2 < nk) gload(kt + 2);
      }
      __syncthreads();
      cur ^= 1;
    }
  };

  if constexpr (GK) {
    kloop(std::integral_constant<int, MT>{});
    // staged epilogue: slab a holds token blocks a*WM + 0 and a*WM + 1
    constexpr int P = BN + 4;   // floats per staged row
    static_assert(64 * P * 4 <= kKmLds, "staged slab fits the pipeline's LDS");
    float* stg = reinterpret_cast<float*>(lds_raw);
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      __syncthreads();   // the K loop's / previous slab's reads are done
#pragma unroll
      for (int b = 0; b < NT; ++b)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[a][b][4 * rq + q];
          *reinterpret_cast<f32x4*>(stg + (wm * 32 + frow) * P + wn * (BN / WN) + b * 32 + 8 * rq +
                                    4 * fhi) = v;
        }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int srow = wave * 8 + j;
        const int m = (a * WM + srow / 32) * 32 + (srow & 31);
        const f32x4 v = *reinterpret_cast<const f32x4*>(stg + srow * P + lane * 4);
        float* o = out + obase + static_cast<size_t>(m) * out_stride + n0 + lane * 4;
        if constexpr (NF) *reinterpret_cast<f32x4*>(o) = v;
        else __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(o));
      }
    }
  } else {
    const int nb = (min(tc.rows, BM) + 31) / 32;
    with_count<MT>((nb - wm + WM - 1) / WM, kloop);
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const int m = (a * WM + wm) * 32 + frow;
      if (m >= tc.rows) continue;
      const size_t orow = static_cast<size_t>(out_row0) + tc.row0 + m;
#pragma unroll
      for (int b = 0; b < NT; ++b)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int n = n0 + wn * (BN / WN) + b * 32 + 8 * rq + 4 * fhi;
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[a][b][4 * rq + q];
          *reinterpret_cast<f32x4*>(out + orow * out_stride + n) = v;
        }
    }
  }
}

hipError_t launch_gemm_kmajor_data(const GemmTileMap& map, const KmDataArgs& a, hipStream_t s) {
  if (a.K % kBK || a.ksplit % kBK || a.N % kKmBN || a.lda % 8 || a.ldw % 8)
    return hipErrorInvalidValue;
  // weight-streaming shapes (gemm_n_fast): the n tiles of each m tile together
  auto kern = map.n_fast ? gemm_kmajor_kernel<false, true> : gemm_kmajor_kernel<false>;
  hipError_t e = allow_large_lds(reinterpret_cast<const void*>(kern), kKmLds);
  if (e != hipSuccess) return e;
  const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + kKmBM - 1) / kKmBM;
  const long long n_logical = static_cast<long long>(m_tiles) * (a.N / kKmBN);
  if (n_logical == 0) return hipSuccess;
  const long long grid = map.n_fast ? 8LL * ((m_tiles + 7) / 8) * (a.N / kKmBN)
                                    : ((n_logical + 7) / 8) * 8;
  kern<<<dim3(static_cast<unsigned>(grid)), dim3(64 * kKmNW), kKmLds, s>>>(
      map.tiles, m_tiles, map.n_single, static_cast<int>(n_logical), a.x, a.lda, a.src, a.x_row0,
      a.wa, a.wb, a.ksplit, a.ldw, a.w_stride, a.y, a.y_stride, a.y_row0, a.K);
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
  auto kern = rows_stream ? gemm_kmajor_kernel<true, true> : gemm_kmajor_kernel<true>;
  hipError_t e = allow_large_lds(reinterpret_cast<const void*>(kern), kKmLds);
  if (e != hipSuccess) return e;
  const int n_single = N1 / kKmBM;
  const int m_tiles = G * n_single;
  const long long n_logical = static_cast<long long>(m_tiles) * (N2 / kKmBN);
  if (n_logical == 0) return hipSuccess;
  const long long grid = rows_stream ? 8LL * ((m_tiles + 7) / 8) * (N2 / kKmBN)
                                     : ((n_logical + 7) / 8) * 8;
  kern<<<dim3(static_cast<unsigned>(grid)), dim3(64 * kKmNW), kKmLds, s>>>(
      offsets, m_tiles, n_single, static_cast<int>(n_logical), A, lda, nullptr, 0, B, nullptr, 0,
      ldb, static_cast<long long>(N1) * N2, out, N2, 0, 0);
  return hipGetLastError();
}

}  // namespace moe
