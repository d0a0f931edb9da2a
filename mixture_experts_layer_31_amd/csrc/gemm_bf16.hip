// Grouped expert GEMMs in bf16 on the CDNA4 matrix cores.
//
// Z = GroupGemm(data, indptr, weights) (CMU 15-779 Lecture 21 notes, §3.3):
// rows [offsets[e], offsets[e+1]) of the permuted tokens multiply expert e's
// weights, for every expert in one launch and without padding a group beyond
// its last tile (§3.4's grouped-GEMM formulation). Two kernels per layer:
//   gate/up: act = silu(X W1_e^T) * (X W3_e^T), the SwiGLU hidden activation,
//            with X's rows gathered through src (the permute is fused) and
//            rounded to bf16 in the epilogue;
//   down:    y_perm = act W2_e^T in fp32.
//
// Design for gfx950:
// * v_mfma_f32_32x32x16_bf16 with the weight tile as the A operand and the
//   token tile as B, so each lane's accumulators hold 4 consecutive output
//   columns of one token row: the epilogue stores 8 (bf16) or 16 (fp32) bytes.
// * Large tiles (gemm_bf16_lds_kernel, 256 token rows): operands go
//   straight from global memory into LDS with the 16-byte global->LDS loads of
//   gfx950 (no staging registers, no LDS store instructions), double-buffered,
//   into 128-byte LDS rows whose 16-byte chunks are XOR-swizzled by row so the
//   MFMA fragment reads are free of bank conflicts. Eight waves per workgroup
//   (two per SIMD) let one wave's LDS waits overlap the other's MFMAs.
// * Small tiles (gemm_bf16_kernel, 32 token rows, decode-sized groups): the
//   operands are staged through registers into padded LDS rows.
// * A device-side tile table (one entry per BM-row tile of each group) lets
//   one launch cover every group with no host sync; grid slots past the last
//   real tile exit at once.
// * Workgroups are dispatched round-robin over the 8 XCDs; the launch index is
//   remapped so each XCD works on a contiguous range of (n-tile, m-tile) pairs
//   with m fastest, so the tiles that share a weight panel share an L2.
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

// H16: gate/up writes the activation as IEEE half; down takes half activation
// rows, widens its bf16 weights to half as they are staged, and multiplies on half
// MFMAs.
template <int BM, int BN, int WM, int WN, bool GATEUP, bool H16>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(
    const int32_t* __restrict__ tiles, int max_tiles, int n_single, int n_logical,
    const uint16_t* __restrict__ xa,      // A rows: x (gate/up) or act (down)
    const int32_t* __restrict__ src,      // gate/up only; nullable
    int a_stride, int a_row0,
    const uint16_t* __restrict__ w_a,     // W1 (gate/up) or W2 (down)
    const uint16_t* __restrict__ w_b,     // W3 (gate/up)
    long long w_stride, void* __restrict__ out, int out_stride, int out_row0, int K, int N) {
  constexpr int NTH = 64 * WM * WN;
  constexpr int WR = GATEUP ? 2 * BN : BN;          // weight rows per tile
  constexpr int XC = BM * 8 / NTH;                  // 16-byte chunks per thread
  constexpr int WC = WR * 8 / NTH;
  constexpr int MT = BM / WM / 32;                  // 32-row blocks per wave
  constexpr int NT = BN / WN / 32;                  // 32-col blocks per wave
  constexpr int NTW = GATEUP ? 2 * NT : NT;
  static_assert(XC * NTH == BM * 8 && WC * NTH == WR * 8, "tile/thread mismatch");

  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* Xs = lds;                               // [2][BM][kPitch]
  uint16_t* Ws = lds + 2 * BM * kPitch;             // [2][WR][kPitch]

  int m_tile, n_tile;
  xcd_tile(n_logical, max_tiles, m_tile, n_tile);
  if (m_tile < 0) return;
  const TileCoord tc = lookup_tile(tiles, n_single, BM, m_tile);
  if (tc.rows <= 0) return;
  const int n0 = n_tile * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // per-thread global source rows for the X and W chunks
  const uint16_t* xg[XC];
  int xoff[XC];
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int q = tid + NTH * i;
    const int r = q >> 3;
    const int rr = min(r, tc.rows - 1);
    int grow = tc.row0 + rr;
    if (src != nullptr) grow = src[grow];
    xg[i] = xa + (static_cast<size_t>(a_row0) + grow) * a_stride + (q & 7) * 8;
    xoff[i] = r * kPitch + (q & 7) * 8;
  }
  const uint16_t* wg[WC];
  int woff[WC];
  const size_t wbase = static_cast<size_t>(tc.group) * w_stride;
#pragma unroll
  for (int i = 0; i < WC; ++i) {
    const int q = tid + NTH * i;
    const int r = q >> 3;
    const uint16_t* wsrc = (!GATEUP || r < BN) ? w_a : w_b;
    const int n = n0 + ((GATEUP && r >= BN) ? r - BN : r);
    wg[i] = wsrc + wbase + static_cast<size_t>(n) * K + (q & 7) * 8;
    woff[i] = r * kPitch + (q & 7) * 8;
  }

  f32x16 acc[MT][NTW];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NTW; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  u32x4 xr[XC], wr[WC];
  auto gload = [&](int kt) {
    const int ko = kt * kBK;
#pragma unroll
    for (int i = 0; i < XC; ++i) xr[i] = *reinterpret_cast<const u32x4*>(xg[i] + ko);
#pragma unroll
    for (int i = 0; i < WC; ++i) wr[i] = *reinterpret_cast<const u32x4*>(wg[i] + ko);
  };
  auto lstore = [&](int buf) {
    uint16_t* xs = Xs + buf * BM * kPitch;
    uint16_t* ws = Ws + buf * WR * kPitch;
#pragma unroll
    for (int i = 0; i < XC; ++i) *reinterpret_cast<u32x4*>(xs + xoff[i]) = xr[i];
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      u32x4 w = wr[i];
      if constexpr (H16 && !GATEUP)
        w = __builtin_bit_cast(u32x4, bf16x8_to_f16(__builtin_bit_cast(bf16x8, w)));
      *reinterpret_cast<u32x4*>(ws + woff[i]) = w;
    }
  };

  const int nk = K / kBK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* xs = Xs + cur * BM * kPitch;
    const uint16_t* ws = Ws + cur * WR * kPitch;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 bfr[MT];
#pragma unroll
      for (int a = 0; a < MT; ++a)
        bfr[a] = *reinterpret_cast<const bf16x8*>(
            xs + (wm * (BM / WM) + a * 32 + lrow) * kPitch + kk * 16 + lk);
      bf16x8 afr[NTW];
#pragma unroll
      for (int b = 0; b < NTW; ++b) {
        const int wrow = (b < NT) ? wn * (BN / WN) + b * 32
                                  : BN + wn * (BN / WN) + (b - NT) * 32;
        afr[b] = *reinterpret_cast<const bf16x8*>(ws + (wrow + lrow) * kPitch + kk * 16 + lk);
      }
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < NTW; ++b)
          acc[a][b] = mfma32x16<H16 && !GATEUP>(afr[b], bfr[a], acc[a][b]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds row m = .. + lane%32, columns n = 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int a = 0; a < MT; ++a) {
    const int m = wm * (BM / WM) + a * 32 + lrow;
    if (m >= tc.rows) continue;
    const size_t orow = static_cast<size_t>(out_row0) + tc.row0 + m;
#pragma unroll
    for (int b = 0; b < NT; ++b) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int n = n0 + wn * (BN / WN) + b * 32 + 8 * rq + 4 * (lane >> 5);
        if (GATEUP) {
          float h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            h[q] = silu(acc[a][b][4 * rq + q]) * acc[a][NT + b][4 * rq + q];
          u32x2 pk;
          pk[0] = H16 ? pack_f16x2(h[0], h[1]) : pack_bf16x2(h[0], h[1]);
          pk[1] = H16 ? pack_f16x2(h[2], h[3]) : pack_bf16x2(h[2], h[3]);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow * out_stride + n) = pk;
        } else {
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[a][b][4 * rq + q];
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + orow * out_stride + n) = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- large tiles

// Real tiles of a launch: the tile table's prefix of entries with rows (one
// group: its tiles). Every thread of the workgroup gets the count.
template <int BM>
__device__ __forceinline__ int real_tiles(const int32_t* tiles, int max_tiles, int n_single,
                                          int* s_real) {
  if (tiles == nullptr) return (n_single + BM - 1) / BM;
  if (threadIdx.x == 0) *s_real = max_tiles;
  __syncthreads();
  for (int i = threadIdx.x; i < max_tiles; i += blockDim.x)
    if (tiles[4 * i + 2] <= 0) atomicMin(s_real, i);
  __syncthreads();
  return *s_real;
}

// HOUT (gate/up only): the epilogue also stores the pre-activations h1 = X W1^T
// and h3 = X W3^T in fp32 to h1o / h3o, at the activation's row index and stride
// (the backward's recompute).
// SK (stream-K, plain products): a persistent grid of P workgroups, one per CU,
// in which workgroup p takes an equal share [U p / P, U (p+1) / P) of the
// U = tiles x K-steps of the launch, tiles in the one-tile-per-workgroup order
// (m fastest); the launch index is remapped so each XCD holds a contiguous
// eighth. With shares of at least one tile's K-steps a tile is split at most
// once: its last part writes out, its first part writes the fp32 tile to
// sk_part slot p (the share's end), and streamk_fixup_kernel adds it after.
// LDS ring of a K loop: st stages of `stage` bytes, the token rows in the first
// xb bytes of each, loads issued in sl slices per K-step.
template <int ST_, int XB_, int STAGE_, int SL_>
struct LdsRing {
  static constexpr int st = ST_, xb = XB_, stage = STAGE_, sl = SL_;
};

// Stages of the short ring (xs token rows, wr weight rows): four when they fit
// in the LDS, else three.
constexpr int short_ring_stages(int xs, int wr) {
  return 4 * (xs + wr) * kRowBytes <= static_cast<int>(kMaxLdsBytes) ? 4 : 3;
}

// H16: as gemm_bf16_kernel (half activations; down widens its weight fragments).
template <int BM, int BN, int WM, int WN, bool GATEUP, int ST, bool HOUT = false, bool SK = false,
          bool NF = false, int XS = 0, bool H16 = false>
__global__ __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void gemm_bf16_lds_kernel(
    const int32_t* __restrict__ tiles, int max_tiles, int n_single, int n_logical,
    const uint16_t* __restrict__ xa, const int32_t* __restrict__ src, int a_stride, int a_row0,
    const uint16_t* __restrict__ w_a, const uint16_t* __restrict__ w_b, long long w_stride,
    void* __restrict__ out, int out_stride, int out_row0, int K, int N,
    float* __restrict__ h1o, float* __restrict__ h3o, float* __restrict__ sk_part) {
  static_assert(!HOUT || GATEUP, "pre-activations come from the gate/up product");
  static_assert(!HOUT || !H16, "the backward's activation stays bf16");
  static_assert(!SK || !GATEUP, "stream-K splits plain fp32 products");
  constexpr bool WIDEN = H16 && !GATEUP;   // half activation rows x widened weights
  constexpr int NW = WM * WN;
  constexpr int WR = GATEUP ? 2 * BN : BN;     // weight rows per tile
  constexpr int XD = BM / 8 / NW;              // LDS-DMA instructions per wave per stage
  constexpr int WD = WR / 8 / NW;
  constexpr int MT = BM / WM / 32;             // 32-row blocks per wave
  constexpr int NT = BN / WN / 32;             // 32-col output blocks per wave
  constexpr int NTW = GATEUP ? 2 * NT : NT;
  constexpr int XBYTES = BM * kRowBytes;
  constexpr int STAGE = (BM + WR) * kRowBytes;
  static_assert(XD * 8 * NW == BM && WD * 8 * NW == WR, "tile/wave mismatch");
  static_assert(ST == 2 || ST == 3, "two or three LDS stages");
  // a stage's loads go out in SL slices over the K-step that precedes its use
  // by ST - 1 steps (with three stages every slice still has a full step of
  // latency to hide)
  constexpr int SL = ST == 3 ? kDmaSlices3 : kDmaSlices;
  // XS > 0: tiles of at most XS rows run a deeper ring (three or four stages)
  // whose stages hold only XS token rows, in the LDS of the full stages
  static_assert(XS == 0 || (XS % 32 == 0 && XS < BM && 3 * (XS + WR) * kRowBytes <= kMaxLdsBytes),
                "three short stages must fit");
  constexpr int XSR = XS > 0 ? XS : BM;
  constexpr int SRS = short_ring_stages(XSR, WR);
  using FullRing = LdsRing<ST, XBYTES, STAGE, SL>;
  using ShortRing = LdsRing<SRS, XSR * kRowBytes, (XSR + WR) * kRowBytes, kDmaSlices3>;

  extern __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int nk_all = K / kBK;

  // One output tile over K-steps [kt0, kt1). part != nullptr (stream-K): the
  // fp32 tile goes there (rows * BN, tile-local) instead of to out.
  auto run_tile = [&](int m_tile, int n_tile, int kt0, int kt1, float* part) {
    if constexpr (SK) __syncthreads();   // the previous tile's reads of the LDS stages are done
    const TileCoord tc = lookup_tile(tiles, n_single, BM, m_tile);
    if (tc.rows <= 0) return;
    const int nk = kt1 - kt0;
    const int n0 = n_tile * BN;

    // DMA instruction i of this wave fills LDS rows 8*(i*NW + wave) .. +7 (1 KB);
    // lane l writes row +l/8, physical chunk l%8, which holds logical K-chunk
    // (l%8) ^ (l/8): the row's chunks are XOR-swizzled by the row index.
    const int lrow8 = lane >> 3;
    const int lchunk = (lane & 7) ^ lrow8;
    const uint16_t* xg[XD];
#pragma unroll
    for (int i = 0; i < XD; ++i) {
      const int r = 8 * (i * NW + wave) + lrow8;
      int grow = tc.row0 + min(r, tc.rows - 1);
      if (src != nullptr) grow = src[grow];
      xg[i] = xa + (static_cast<size_t>(a_row0) + grow) * a_stride + lchunk * 8;
    }
    const uint16_t* wg[WD];
    const size_t wbase = static_cast<size_t>(tc.group) * w_stride;
#pragma unroll
    for (int i = 0; i < WD; ++i) {
      const int r = 8 * (i * NW + wave) + lrow8;
      const uint16_t* wsrc = (!GATEUP || r < BN) ? w_a : w_b;
      const int n = n0 + ((GATEUP && r >= BN) ? r - BN : r);
      wg[i] = wsrc + wbase + static_cast<size_t>(n) * K + lchunk * 8;
    }
    // the stage's XD + WD LDS-DMA instructions, issued in slices: instruction j
    // goes out in slice j * kDmaSlices / (XD + WD)
    constexpr int ND = XD + WD;
    auto dma_slice = [&](int kt, int buf, auto slice_c, auto ring) {
      using R = decltype(ring);
      constexpr int S = decltype(slice_c)::value;
      const int ko = (kt0 + kt) * kBK;
      unsigned char* xs = lds_raw + buf * R::stage;
      unsigned char* ws = xs + R::xb;
#pragma unroll
      for (int j = 0; j < ND; ++j) {
        if (j * R::sl / ND != S) continue;
        if (j < XD) {
          // token rows past the tile's last row are never stored: skip their loads
          if (8 * (j * NW + wave) < tc.rows) MOE_LDS_DMA16(xg[j] + ko, xs + (j * NW + wave) * 1024);
        } else {
          MOE_LDS_DMA16(wg[j - XD] + ko, ws + ((j - XD) * NW + wave) * 1024);
        }
      }
    };
    auto dma = [&](int kt, int buf, auto ring) {
      dma_slice(kt, buf, std::integral_constant<int, 0>{}, ring);
      dma_slice(kt, buf, std::integral_constant<int, 1>{}, ring);
      dma_slice(kt, buf, std::integral_constant<int, 2>{}, ring);
      dma_slice(kt, buf, std::integral_constant<int, 3>{}, ring);
    };

    f32x16 acc[MT][NTW];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
      for (int b = 0; b < NTW; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // fragment reads: row lane%32 of a 32-row block, logical K-chunk 2*kk + lane/32
    const int frow = lane & 31, fhi = lane >> 5;
    int koff[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) koff[kk] = frow * kRowBytes + (((2 * kk + fhi) ^ (frow & 7)) << 4);
    // token block a of wave row wm is the tile's 32-row block a*WM + wm: the
    // blocks of a short (ragged-tail) tile are shared by all wave rows
    bf16x8 fa[4][NTW], fb[4][MT];
    auto rfrag = [&](int buf, int kk, auto na_c, auto ring) {
      using R = decltype(ring);
      constexpr int NA = decltype(na_c)::value;
      const unsigned char* xs = lds_raw + buf * R::stage;
      const unsigned char* ws = xs + R::xb;
#pragma unroll
      for (int b = 0; b < NTW; ++b) {
        const int wrow = (b < NT) ? wn * (BN / WN) + b * 32 : BN + wn * (BN / WN) + (b - NT) * 32;
        fa[kk][b] = *reinterpret_cast<const bf16x8*>(ws + wrow * kRowBytes + koff[kk]);
        if constexpr (WIDEN) fa[kk][b] = bf16x8_to_f16(fa[kk][b]);
      }
#pragma unroll
      for (int a = 0; a < NA; ++a)
        fb[kk][a] = *reinterpret_cast<const bf16x8*>(xs + (a * WM + wm) * 32 * kRowBytes + koff[kk]);
    };
    auto mfmas = [&](int kk, auto na_c) {
      constexpr int NA = decltype(na_c)::value;
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NTW; ++b)
          acc[a][b] = mfma32x16<WIDEN>(fa[kk][b], fb[kk][a], acc[a][b]);
    };

    // one barrier per K-step: it publishes stage kt (every thread waited for its
    // own LDS-DMA loads of that stage) and retires all reads of the buffer that
    // this step's loads fill, stage kt + ST - 1 (ST buffers in rotation).
    // The loop is specialised on the number of this wave's token blocks that
    // hold rows (NA): a full tile runs NA = MT, a ragged tail only the MFMAs of
    // its rows, so it costs about its share of a full tile.
    int nd_stage = WD;                 // LDS-DMA instructions this wave issues per stage
#pragma unroll
    for (int j = 0; j < XD; ++j) nd_stage += 8 * (j * NW + wave) < tc.rows ? 1 : 0;
    auto kloop = [&](auto na_c, auto ring) {
      using R = decltype(ring);
      constexpr int RS = R::st;
#pragma unroll
      for (int p = 0; p < RS - 1; ++p)
        if (p < nk) dma(p, p, ring);
      int cur = 0;
      for (int kt = 0; kt < nk; ++kt) {
        // loads complete in issue order: stage kt has landed once no more than
        // the later stages' loads (nd_stage each) are outstanding
        const int later = min(RS - 2, nk - 1 - kt);
        if (RS >= 3 && later > 0) wait_vmcnt_at_most<(RS >= 3 ? RS - 2 : 1) * ND>(later * nd_stage);
        else MOE_WAIT_VMCNT(0);
        // with three or more stages the later stages' loads stay in flight across it
        if constexpr (RS >= 3) dma_barrier();
        else __syncthreads();
        const int ahead = kt + RS - 1;
        const bool more = ahead < nk;
        const int nbuf = cur == 0 ? RS - 1 : cur - 1;   // (cur + RS - 1) % RS
        if (more) dma_slice(ahead, nbuf, std::integral_constant<int, 0>{}, ring);
        MOE_SCHED_FENCE();
        rfrag(cur, 0, na_c, ring);
        rfrag(cur, 1, na_c, ring);
        mfmas(0, na_c);
        if (more && R::sl > 1) dma_slice(ahead, nbuf, std::integral_constant<int, 1>{}, ring);
        MOE_SCHED_FENCE();
        rfrag(cur, 2, na_c, ring);
        mfmas(1, na_c);
        if (more && R::sl > 2) dma_slice(ahead, nbuf, std::integral_constant<int, 2>{}, ring);
        MOE_SCHED_FENCE();
        rfrag(cur, 3, na_c, ring);
        mfmas(2, na_c);
        if (more && R::sl > 3) dma_slice(ahead, nbuf, std::integral_constant<int, 3>{}, ring);
        MOE_SCHED_FENCE();
        mfmas(3, na_c);
        cur = cur + 1 == RS ? 0 : cur + 1;
      }
    };
    const int nb = (min(tc.rows, BM) + 31) / 32;
    const int na_count = (nb - wm + WM - 1) / WM;
    if (XS > 0 && tc.rows <= XS)
      with_count<MT>(na_count, [&](auto na_c) { kloop(na_c, ShortRing{}); });
    else
      with_count<MT>(na_count, [&](auto na_c) { kloop(na_c, FullRing{}); });

    if constexpr (SK) {
      if (part != nullptr) {
#pragma unroll
        for (int a = 0; a < MT; ++a) {
          const int m = (a * WM + wm) * 32 + frow;
          if (m >= tc.rows) continue;
#pragma unroll
          for (int b = 0; b < NT; ++b)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              f32x4 v;
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = acc[a][b][4 * rq + q];
              *reinterpret_cast<f32x4*>(part + static_cast<size_t>(m) * BN + wn * (BN / WN) +
                                        b * 32 + 8 * rq + 4 * fhi) = v;
            }
        }
        return;
      }
    }
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const int m = (a * WM + wm) * 32 + frow;
      if (m >= tc.rows) continue;
      const size_t orow = static_cast<size_t>(out_row0) + tc.row0 + m;
#pragma unroll
      for (int b = 0; b < NT; ++b) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int n = n0 + wn * (BN / WN) + b * 32 + 8 * rq + 4 * fhi;
          if (GATEUP) {
            float h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              h[q] = silu(acc[a][b][4 * rq + q]) * acc[a][NT + b][4 * rq + q];
            u32x2 pk;
            pk[0] = H16 ? pack_f16x2(h[0], h[1]) : pack_bf16x2(h[0], h[1]);
            pk[1] = H16 ? pack_f16x2(h[2], h[3]) : pack_bf16x2(h[2], h[3]);
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow * out_stride + n) = pk;
            if constexpr (HOUT) {
              f32x4 v1, v3;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                v1[q] = acc[a][b][4 * rq + q];
                v3[q] = acc[a][NT + b][4 * rq + q];
              }
              *reinterpret_cast<f32x4*>(h1o + orow * out_stride + n) = v1;
              *reinterpret_cast<f32x4*>(h3o + orow * out_stride + n) = v3;
            }
          } else {
            f32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = acc[a][b][4 * rq + q];
            *reinterpret_cast<f32x4*>(static_cast<float*>(out) + orow * out_stride + n) = v;
          }
        }
      }
    }
  };

  if constexpr (!SK) {
    int m_tile, n_tile;
    if constexpr (NF) xcd_tile_nfast(max_tiles, N / BN, m_tile, n_tile);
    else if (tile_order_blocked(BM, N / BN)) xcd_tile_blocked(tiles, max_tiles, N / BN, m_tile, n_tile);
    else xcd_tile(n_logical, max_tiles, m_tile, n_tile);
    if (m_tile < 0) return;
    run_tile(m_tile, n_tile, 0, nk_all, nullptr);
  } else {
    __shared__ int s_real;
    const int n_real = real_tiles<BM>(tiles, max_tiles, n_single, &s_real);
    const long long n_tiles = static_cast<long long>(n_real) * (N / BN);
    const long long U = n_tiles * nk_all;
    const int P = gridDim.x;   // a multiple of 8
    const int L = blockIdx.x;
    const int p = (L & 7) * (P >> 3) + (L >> 3);
    if (U < static_cast<long long>(P) * nk_all) {
      // under one tile per workgroup: whole tiles, no split
      for (long long t = p; t < n_tiles; t += P)
        run_tile(static_cast<int>(t % n_real), static_cast<int>(t / n_real), 0, nk_all, nullptr);
      return;
    }
    const long long u1 = U * (p + 1) / P;
    for (long long u = U * p / P; u < u1;) {
      const long long t = u / nk_all;
      const int kt0 = static_cast<int>(u - t * nk_all);
      const int kt1 = static_cast<int>(min(static_cast<long long>(nk_all), kt0 + (u1 - u)));
      // a segment that stops before its tile's end is that tile's first part
      float* part = kt1 < nk_all ? sk_part + static_cast<size_t>(p) * BM * BN : nullptr;
      run_tile(static_cast<int>(t % n_real), static_cast<int>(t / n_real), kt0, kt1, part);
      u += kt1 - kt0;
    }
  }
}


// out tile += the fp32 first part of each tile that a stream-K share boundary
// splits (its last part already wrote out): workgroups (p, q) take the boundary
// between shares p and p + 1, recomputed as in the GEMM, q the q-th quarter of
// the tile's rows. One fp32 addition per element, so the result does not depend
// on which part finished first.
template <int BM, int BN, int BK>
__global__ __launch_bounds__(256) void streamk_fixup_kernel(
    const int32_t* __restrict__ tiles, int max_tiles, int n_single, int K, int N, int P,
    const float* __restrict__ sk_part, float* __restrict__ out, int out_stride, int out_row0) {
  __shared__ int s_real;
  const int n_real = real_tiles<BM>(tiles, max_tiles, n_single, &s_real);
  const int nk_all = K / BK;   // the GEMM's K-steps
  const long long U = static_cast<long long>(n_real) * (N / BN) * nk_all;
  if (U < static_cast<long long>(P) * nk_all) return;   // nothing was split
  const int p = blockIdx.x;
  const long long ub = U * (p + 1) / P;
  const long long t = ub / nk_all;
  if (ub == t * nk_all) return;                          // the boundary falls between tiles
  const TileCoord tc = lookup_tile(tiles, n_single, BM, static_cast<int>(t % n_real));
  const int n0 = static_cast<int>(t / n_real) * BN;
  const float* part = sk_part + static_cast<size_t>(p) * BM * BN;
  constexpr int QR = BM / 4;   // rows per quarter
  const int m_lo = blockIdx.y * QR;
  const int m_hi = min(tc.rows, m_lo + QR);
  for (int i = m_lo * (BN / 4) + threadIdx.x; i < m_hi * (BN / 4); i += 256) {
    const int m = i / (BN / 4), c = (i % (BN / 4)) * 4;
    f32x4* y = reinterpret_cast<f32x4*>(out + (static_cast<size_t>(out_row0) + tc.row0 + m) *
                                                  out_stride + n0 + c);
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + static_cast<size_t>(m) * BN + c);
    *y = *y + v;
  }
}
// ---------------------------------------------------------------- large tiles, one wave per SIMD
//
// 256 x 256 tiles (256 token rows x 256 weight rows: gate/up 128 gate + 128 up
// columns, down 256 columns), four waves of 128 x 128 each (one per SIMD), so a
// wave reads 8 fragments per 16 MFMAs (two waves of 128 x 64 read 12 per 16).
// K-steps of 32: a stage is 256 token + 256 weight rows of 64 bytes (32 KB),
// filled by LDS-DMA (16 rows per instruction; the four 16-byte chunks of a row
// XOR-swizzled by (row >> 1) & 3, so the fragment reads of eight consecutive rows
// hit distinct banks) in a ring of ST slots. The load issued at step kt is stage
// kt + LA (LA = ST - 2 stages ahead), into the slot of stage kt - 2: every wave
// has consumed that stage's fragments before it reaches step kt - 1's MFMAs, so
// the step's barrier waits only for the wave's own loads of stage kt, not for
// LDS reads still in flight. One barrier per K-step; the fragments of a step's
// second k-slice are read before the next barrier and multiplied after it, so
// the matrix pipe stays busy across the barrier while the next step's first
// fragments are read.
constexpr int kW4BK = 32;          // K per step
constexpr int kW4Row = 64;         // LDS row bytes (32 bf16)
constexpr int kW4Stage = 512 * kW4Row;   // 256 token + 256 weight rows

// H16: as gemm_bf16_kernel (half activations; down widens its weight fragments).
template <bool GATEUP, int ST, bool NF, bool H16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gemm_bf16_w4_kernel(const int32_t* __restrict__ tiles, int max_tiles, int n_single,
                    int n_logical, const uint16_t* __restrict__ xa,
                    const int32_t* __restrict__ src, int a_stride, int a_row0,
                    const uint16_t* __restrict__ w_a, const uint16_t* __restrict__ w_b,
                    long long w_stride, void* __restrict__ out, int out_stride, int out_row0,
                    int K, int N) {
  static_assert(ST >= 4 && ST * kW4Stage <= static_cast<int>(kMaxLdsBytes), "ring must fit");
  constexpr int BM = 256, BN = GATEUP ? 128 : 256;
  constexpr int ND = 8;        // LDS-DMA instructions per wave per stage (4 token, 4 weight)
  constexpr int LA = ST - 2;   // stages loaded ahead
  constexpr bool WIDEN = H16 && !GATEUP;   // half activation rows x widened weights
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int nk_all = K / kW4BK;

  int m_tile, n_tile;
  if constexpr (NF) xcd_tile_nfast(max_tiles, N / BN, m_tile, n_tile);
  else if (tile_order_blocked(BM, N / BN)) xcd_tile_blocked(tiles, max_tiles, N / BN, m_tile, n_tile);
  else xcd_tile(n_logical, max_tiles, m_tile, n_tile);
  if (m_tile < 0) return;
  const TileCoord tc = lookup_tile(tiles, n_single, BM, m_tile);
  if (tc.rows <= 0) return;
  const int nk = nk_all;
  const int n0 = n_tile * BN;
  {

    // DMA instruction j of this wave fills rows 16 * (4 * (j % 4) + wave) .. + 15
    // of the token (j < 4) or weight (j >= 4) half of a stage; lane l writes row
    // + l / 4, physical chunk l % 4, which holds logical chunk (l % 4) ^ ((l >> 3) & 3)
    const int lrow = lane >> 2;
    const int lchunk = (lane & 3) ^ ((lane >> 3) & 3);
    const uint16_t* gp[ND];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * (4 * j + wave) + lrow;
      int grow = tc.row0 + min(r, tc.rows - 1);
      if (src != nullptr) grow = src[grow];
      gp[j] = xa + (static_cast<size_t>(a_row0) + grow) * a_stride + lchunk * 8;
    }
    const size_t wbase = static_cast<size_t>(tc.group) * w_stride;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * (4 * j + wave) + lrow;
      const uint16_t* wsrc = (!GATEUP || r < BN) ? w_a : w_b;
      const int n = n0 + ((GATEUP && r >= BN) ? r - BN : r);
      gp[4 + j] = wsrc + wbase + static_cast<size_t>(n) * K + lchunk * 8;
    }
    // the eight loads of stage kt into ring slot buf; every wave issues all eight
    // (rows past a ragged tile's end load its last row again and are never
    // stored), so the count of loads in flight is the same on every wave
    auto dma = [&](int kt, int buf) {
      unsigned char* st = lds_raw + buf * kW4Stage;
#pragma unroll
      for (int j = 0; j < ND; ++j) {
        unsigned char* dst = st + (j >= 4 ? BM * kW4Row : 0) + (4 * (j & 3) + wave) * 16 * kW4Row;
        MOE_LDS_DMA16(gp[j] + kt * kW4BK, dst);
      }
    };

    // fragment of a 32-row block at k-slice kk: row lane % 32, logical chunk
    // 2 kk + lane / 32
    const int frow = lane & 31;
    const int fsw = (frow >> 1) & 3;
    const int foff0 = frow * kW4Row + (((0 + (lane >> 5)) ^ fsw) << 4);
    const int foff1 = frow * kW4Row + (((2 + (lane >> 5)) ^ fsw) << 4);
    // this wave's weight blocks: gate/up the gate and up rows of its 64 columns
    int wblk[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      wblk[b] = GATEUP ? (b < 2 ? wn * 2 + b : 4 + wn * 2 + (b - 2)) : wn * 4 + b;

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // token block a of this wave is the tile's 32-row block 2 a + wm
    auto rfrag = [&](int buf, int kk, bf16x8 (&fa)[4], bf16x8 (&fb)[4], auto na_c) {
      constexpr int NA = decltype(na_c)::value;
      const unsigned char* st = lds_raw + buf * kW4Stage;
      const int fo = kk ? foff1 : foff0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        fa[b] = *reinterpret_cast<const bf16x8*>(st + BM * kW4Row + wblk[b] * 32 * kW4Row + fo);
        if constexpr (WIDEN) fa[b] = bf16x8_to_f16(fa[b]);
      }
#pragma unroll
      for (int a = 0; a < NA; ++a)
        fb[a] = *reinterpret_cast<const bf16x8*>(st + (2 * a + wm) * 32 * kW4Row + fo);
    };
    auto mfmas = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4], auto na_c) {
      constexpr int NA = decltype(na_c)::value;
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = mfma32x16<WIDEN>(fa[b], fb[a], acc[a][b]);
    };

    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    // One K-step (any step; conditions at run time): publish stage kt, load stage
    // kt + LA, read this stage's first k-slice while the previous step's second
    // slice is multiplied, then its second slice while the first is multiplied.
    auto step = [&](int kt, auto na_c) {
      const int later = min(LA - 1, nk - 1 - kt);   // stages after kt already issued
      if (later == LA - 1) MOE_WAIT_VMCNT((LA - 1) * ND);
      else wait_vmcnt_at_most<(LA - 1) * ND>(later * ND);
      dma_barrier();   // publishes stage kt
      const int cur = kt % ST;
      if (kt + LA < nk) dma(kt + LA, (kt + LA) % ST);
      MOE_SCHED_FENCE();
      rfrag(cur, 0, fa0, fb0, na_c);
      if (kt > 0) mfmas(fa1, fb1, na_c);       // second slice of the previous step
      rfrag(cur, 1, fa1, fb1, na_c);
      mfmas(fa0, fb0, na_c);
    };
    // The same step in the steady state of a full tile: ring slot S known at
    // compile time (LDS offsets and the DMA's M0 values become immediates), a
    // step before it and the load ahead of it always present, no branches. With
    // one wave per SIMD the wave issues in order, so every other instruction is
    // placed in the shadow of an MFMA (32 cycles each): the 16 MFMAs of the
    // previous step's second slice alternate with this step's first-slice reads
    // and its eight LDS-DMA loads, the first 8 MFMAs of its first slice with the
    // second-slice reads.
    auto main_step = [&](int kt, auto slot_c) {
      constexpr int S = decltype(slot_c)::value;
      constexpr int DS = (S + LA) % ST;
      using N4 = std::integral_constant<int, 4>;
      MOE_WAIT_VMCNT((LA - 1) * ND);
      lds_barrier();
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_sched_barrier(0);   // nothing crosses the barrier
#endif
      rfrag(S, 0, fa0, fb0, N4{});
      mfmas(fa1, fb1, N4{});
      dma(kt + LA, DS);
      rfrag(S, 1, fa1, fb1, N4{});
      mfmas(fa0, fb0, N4{});
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // LDS-DMA load
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
#endif
    };

    auto kloop = [&](auto na_c) {
      constexpr int NA = decltype(na_c)::value;
#pragma unroll
      for (int p = 0; p < LA; ++p)
        if (p < nk) dma(p, p);
      int kt = 0;
      if constexpr (NA == 4) {
        // the first ST steps, then whole turns of the ring while every load of the
        // turn is before the tile's end, then the rest
        for (; kt < ST && kt < nk; ++kt) step(kt, na_c);
        for (; kt + ST - 1 + LA < nk; kt += ST) {
          main_step(kt, std::integral_constant<int, 0>{});
          main_step(kt + 1, std::integral_constant<int, 1>{});
          main_step(kt + 2, std::integral_constant<int, 2>{});
          main_step(kt + 3, std::integral_constant<int, 3>{});
          if constexpr (ST > 4) main_step(kt + 4, std::integral_constant<int, 4 % ST>{});
          if constexpr (ST > 5) main_step(kt + 5, std::integral_constant<int, 5 % ST>{});
        }
      }
      for (; kt < nk; ++kt) step(kt, na_c);
      mfmas(fa1, fb1, na_c);
    };
    const int nb = (min(tc.rows, BM) + 31) / 32;
    const int na_count = (nb - wm + 1) / 2;
    with_count<4>(na_count, [&](auto na_c) { kloop(na_c); });

#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int m = (2 * a + wm) * 32 + frow;
      if (m >= tc.rows) continue;
      const size_t orow = static_cast<size_t>(out_row0) + tc.row0 + m;
      if constexpr (GATEUP) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int n = n0 + wn * 64 + b * 32 + 8 * rq + 4 * (lane >> 5);
            float h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              h[q] = silu(acc[a][b][4 * rq + q]) * acc[a][b + 2][4 * rq + q];
            u32x2 pk;
            pk[0] = H16 ? pack_f16x2(h[0], h[1]) : pack_bf16x2(h[0], h[1]);
            pk[1] = H16 ? pack_f16x2(h[2], h[3]) : pack_bf16x2(h[2], h[3]);
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow * out_stride + n) = pk;
          }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int n = n0 + wblk[b] * 32 + 8 * rq + 4 * (lane >> 5);
            f32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = acc[a][b][4 * rq + q];
            *reinterpret_cast<f32x4*>(static_cast<float*>(out) + orow * out_stride + n) = v;
          }
      }
    }
  }
}

// ---------------------------------------------------------------- decode tiles
//
// Groups of at most a few rows (decode): the time is reading the experts'
// weights, which are streamed exactly once. A work item is 16 weight rows
// (output columns) of one 16-row token tile; KS waves of a workgroup split
// its K range and their partial sums are added in LDS in a fixed order. Each
// wave walks its K range with v_mfma_f32_16x16x32_bf16: lane l loads 16 bytes
// of weight row l%16 and 16 bytes of token row l%16, both at K-chunk l/16 of
// the current 32-wide step, straight from global memory into registers (the
// token rows are tiny and stay in cache). Batches of U steps are double-
// buffered in registers, so the next batch's loads are in flight while the
// current batch is multiplied. The accumulators then hold token l%16 and four
// consecutive output columns 4*(l/16)..+3. Items with the same n-slice and
// consecutive token tiles run in the same workgroup (KS < 4) so they share the
// weight rows in cache.
//
// An optional second segment (seg.rows > 0) is one dense group with weights,
// widths and rows of its own (the shared expert of a decode step): its items
// follow the grouped ones in the same launch, so both weight streams fill the
// device together instead of one launch's ramp and tail after the other's.
struct StreamSeg {
  const uint16_t* xa = nullptr;   // row r reads xa[(a_row0 + r) * a_stride ...] (no src)
  const uint16_t* wa = nullptr;   // [N][K]
  const uint16_t* wb = nullptr;   // [N][K] (gate/up only)
  int a_row0 = 0, rows = 0, K = 0, N = 0, out_row0 = 0;
};

static __host__ __device__ long long stream_seg_items(const StreamSeg& seg) {
  return seg.rows > 0 ? static_cast<long long>((seg.rows + 15) >> 4) * (seg.N >> 4) : 0;
}

// One wave's share of a streamed item: K-steps [s_lo, s_hi) of 16 weight rows
// (wp; gate/up also wq) against 16 token rows (xp), lane l holding 16 bytes of
// row l % 16 at K-chunk l / 16 of each 32-wide step. Batches of U steps are
// double-buffered in registers: the next batch's loads are issued before the
// current batch is multiplied. WIDEN: the weights are bf16 and the token rows
// IEEE half (each weight fragment widened to half before its MFMA).
template <bool GATEUP, int U, bool WIDEN>
__device__ __forceinline__ void stream_wave(const uint16_t* wp, const uint16_t* wq,
                                            const uint16_t* xp, int s_lo, int s_hi, f32x4& acc,
                                            f32x4& acc2) {
  typedef __attribute__((ext_vector_type(8))) __bf16 bf8;
  auto wfrag = [](bf8 w) { if constexpr (WIDEN) return bf16x8_to_f16(w); else return w; };
  bf8 wv[2][U], xv[2][U], qv[2][U];
  auto load = [&](int s0, int b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s0 + u) << 5;
      wv[b][u] = *reinterpret_cast<const bf8*>(wp + k);
      if (GATEUP) qv[b][u] = *reinterpret_cast<const bf8*>(wq + k);
      xv[b][u] = *reinterpret_cast<const bf8*>(xp + k);
    }
  };
  auto comp = [&](int b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc = mfma16x32<WIDEN>(wfrag(wv[b][u]), xv[b][u], acc);
      if (GATEUP) acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv[b][u], xv[b][u], acc2, 0, 0, 0);
    }
  };
  const int nb = (s_hi - s_lo) / U;
  if (nb > 0) {
    load(s_lo, 0);
    int i = 0;
    for (; i + 2 <= nb; i += 2) {
      load(s_lo + (i + 1) * U, 1);
      comp(0);
      if (i + 2 < nb) load(s_lo + (i + 2) * U, 0);
      comp(1);
    }
    if (i < nb) comp(0);
  }
  for (int st = s_lo + nb * U; st < s_hi; ++st) {
    const int k = st << 5;
    const bf8 w1v = *reinterpret_cast<const bf8*>(wp + k);
    const bf8 x1v = *reinterpret_cast<const bf8*>(xp + k);
    acc = mfma16x32<WIDEN>(wfrag(w1v), x1v, acc);
    if (GATEUP) {
      const bf8 q1v = *reinterpret_cast<const bf8*>(wq + k);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q1v, x1v, acc2, 0, 0, 0);
    }
  }
}

// H16: as gemm_bf16_kernel (half activations; down widens its weight fragments).
template <bool GATEUP, int U, int KS, bool H16>
__global__ __launch_bounds__(256) void gemm_bf16_stream_kernel(
    const int32_t* __restrict__ tiles, int max_tiles, int n_single,
    const uint16_t* __restrict__ xa_g, const int32_t* __restrict__ src_g, int a_stride,
    int a_row0_g, const uint16_t* __restrict__ w_a_g, const uint16_t* __restrict__ w_b_g,
    long long w_stride, void* __restrict__ out, int out_stride, int out_row0_g, int K_g, int N,
    StreamSeg seg) {
  constexpr int IPB = 4 / KS;                  // items per workgroup
  constexpr bool WIDEN = H16 && !GATEUP;       // half activation rows x widened weights
  __shared__ f32x4 red[KS > 1 ? 3 : 1][GATEUP ? 2 : 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kpart = wave % KS;
  // The second segment's workgroups come first (all of their items are real, and
  // at 64 rows a shared expert's workgroups hold its whole K: started last, they
  // formed a tail; DeepSeek shape at 64 tokens, joint gate/up launch 2.47 ms).
  // Then workgroup L of the grouped rows: n-slice L % ncol of token tiles
  // (L / ncol) * IPB .. + IPB - 1 (one per item of the workgroup, so items of a
  // group's consecutive tiles share the weight rows in cache). n-slices run
  // fastest, so the empty tiles at the end of the table (the table holds an upper
  // bound of tiles) are the last workgroups of the grid. With token tiles fastest,
  // a table of 4 tiles of which 2 were empty made every other workgroup empty, and
  // that pattern of active workgroups kept half of the CUs' slots idle (2 tokens,
  // Mixtral shape: gate/up 92 -> 134 us).
  const int ncol = N >> 4;
  const long long wg_s = (stream_seg_items(seg) + IPB - 1) / IPB;
  const long long L0 = blockIdx.x;
  // this wave's item: a tile of the grouped rows or of the second segment
  const uint16_t* xa = xa_g;
  const int32_t* src = src_g;
  const uint16_t* w_a = w_a_g;
  const uint16_t* w_b = w_b_g;
  int a_row0 = a_row0_g, out_row0 = out_row0_g, K = K_g;
  bool live;
  int n0 = 0;
  TileCoord tc{0, 0, 0};
  if (L0 >= wg_s) {
    const long long L = L0 - wg_s;
    const int mt = static_cast<int>(L / ncol) * IPB + wave / KS;
    live = mt < max_tiles;
    n0 = static_cast<int>(L % ncol) * 16;
    if (live) tc = lookup_tile(tiles, n_single, 16, mt);
  } else {
    const long long j = L0 * IPB + wave / KS;
    live = j < stream_seg_items(seg);
    if (live) {
      const int seg_tiles = (seg.rows + 15) >> 4;
      const int mt = static_cast<int>(j % seg_tiles);
      n0 = static_cast<int>(j / seg_tiles) * 16;
      tc.row0 = mt * 16;
      tc.rows = min(16, seg.rows - mt * 16);
      xa = seg.xa;
      src = nullptr;
      w_a = seg.wa;
      w_b = seg.wb;
      a_row0 = seg.a_row0;
      out_row0 = seg.out_row0;
      K = seg.K;
    }
  }
  const bool active = live && tc.rows > 0;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
  const int r16 = lane & 15, ck = (lane >> 4) * 8;
  if (active) {
    int grow = tc.row0 + min(r16, tc.rows - 1);
    if (src != nullptr) grow = src[grow];
    const uint16_t* xp = xa + (static_cast<size_t>(a_row0) + grow) * a_stride + ck;
    const size_t wrow = static_cast<size_t>(tc.group) * w_stride + static_cast<size_t>(n0 + r16) * K + ck;
    const uint16_t* wp = w_a + wrow;
    const uint16_t* wq = GATEUP ? w_b + wrow : nullptr;
    // this wave's K range: whole 32-wide steps, split as evenly as possible
    const int steps = K >> 5;
    stream_wave<GATEUP, U, WIDEN>(wp, wq, xp, steps * kpart / KS, steps * (kpart + 1) / KS, acc,
                                  acc2);
  }
  if (KS > 1) {
    // partial sums of waves 1..KS-1 of this item, added by wave 0 in wave order
    const int slot = wave / KS;   // KS > 1 => IPB <= 2
    if (kpart > 0) {
      red[(kpart - 1) + slot * (KS - 1)][0][lane] = acc;
      if (GATEUP) red[(kpart - 1) + slot * (KS - 1)][GATEUP ? 1 : 0][lane] = acc2;
    }
    __syncthreads();
    if (kpart > 0) return;
#pragma unroll
    for (int p = 0; p < KS - 1; ++p) {
      const f32x4 v = red[p + slot * (KS - 1)][0][lane];
      acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
      if (GATEUP) {
        const f32x4 v2 = red[p + slot * (KS - 1)][GATEUP ? 1 : 0][lane];
        acc2[0] += v2[0]; acc2[1] += v2[1]; acc2[2] += v2[2]; acc2[3] += v2[3];
      }
    }
  }
  if (!active || r16 >= tc.rows) return;
  const size_t orow = static_cast<size_t>(out_row0) + tc.row0 + r16;
  const int n = n0 + (lane >> 4) * 4;
  if (GATEUP) {
    auto pack = [](float lo, float hi) { return H16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi); };
    u32x2 pk;
    pk[0] = pack(silu(acc[0]) * acc2[0], silu(acc[1]) * acc2[1]);
    pk[1] = pack(silu(acc[2]) * acc2[2], silu(acc[3]) * acc2[3]);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + orow * out_stride + n) = pk;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + orow * out_stride + n) = acc;
  }
}

// Down product and combine in one launch, for decode steps whose groups each fit
// one 16-row tile and whose tiles times the K split fit one workgroup (a layer of
// few experts per token at one or two tokens): workgroup j owns output columns
// 16 j .. 16 j + 15 of every tile, so it holds all k rows of each token's slice.
// Wave w streams tile w / KS over the K range of wave w % KS exactly as
// gemm_bf16_stream_kernel does, and the KS partial sums of a tile are added in the
// same wave order, so each y_perm value is the same bit for bit; the values stay
// in LDS (indexed by y_perm row). Then y[t][slice] is the gate-weighted sum of
// the token's kept rows as combine_kernel computes it: fused multiply-adds from
// zero in slot order. The layer output is the routed experts' weighted sum (no
// shared expert here).
constexpr int kCombineMaxK = 8;   // slots per token the fused combine holds in registers
template <int U, int KS, int NTL, bool H16>
__global__ __launch_bounds__(64 * KS * NTL) void gemm_down_combine_kernel(
    const int32_t* __restrict__ tiles, int max_tiles, const uint16_t* __restrict__ act,
    int a_stride, const uint16_t* __restrict__ w2, long long w_stride, int K, int N,
    const int32_t* __restrict__ dest, const float* __restrict__ gates, int T, int k,
    float* __restrict__ y) {
  __shared__ f32x4 red[NTL][KS > 1 ? KS - 1 : 1][64];
  __shared__ float yl[16 * NTL][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ti = wave / KS, kpart = wave % KS;
  const int n0 = blockIdx.x * 16;
  TileCoord tc{0, 0, 0};
  if (ti < max_tiles) tc = lookup_tile(tiles, 0, 16, ti);
  const bool active = tc.rows > 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
  const int r16 = lane & 15, ck = (lane >> 4) * 8;
  // this thread's combine item (token t, column c of the slice): its slots' rows
  // and gates are loaded now, so their latency passes while the weights stream
  const int t = threadIdx.x >> 4, c = threadIdx.x & 15;
  const bool has_item = t < T;
  int rj[kCombineMaxK];
  float gj[kCombineMaxK];
#pragma unroll
  for (int j = 0; j < kCombineMaxK; ++j) {
    rj[j] = has_item && j < k ? dest[t * k + j] : -1;
    gj[j] = has_item && j < k ? gates[t * k + j] : 0.f;
  }
  if (active) {
    const uint16_t* xp = act + static_cast<size_t>(tc.row0 + min(r16, tc.rows - 1)) * a_stride + ck;
    const uint16_t* wp = w2 + static_cast<size_t>(tc.group) * w_stride +
                         static_cast<size_t>(n0 + r16) * K + ck;
    const int steps = K >> 5;
    stream_wave<false, U, H16>(wp, nullptr, xp, steps * kpart / KS, steps * (kpart + 1) / KS, acc,
                               acc2);
  }
  if (KS > 1 && kpart > 0) red[ti][kpart - 1][lane] = acc;
  __syncthreads();
  if (kpart == 0 && active) {
#pragma unroll
    for (int p = 0; p < KS - 1; ++p) {
      const f32x4 v = red[ti][p][lane];
      acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
    }
    if (r16 < tc.rows) {
#pragma unroll
      for (int q = 0; q < 4; ++q) yl[tc.row0 + r16][(lane >> 4) * 4 + q] = acc[q];
    }
  }
  __syncthreads();
  if (has_item) {
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kCombineMaxK; ++j)
      if (rj[j] >= 0) sum = fmaf(gj[j], yl[rj[j]][c], sum);
    y[static_cast<size_t>(t) * N + n0 + c] = sum;
  }
}

// Decode launch shape, measured on MI355X from cold caches over the Mixtral,
// DeepSeek and Switch shapes at 1-32 tokens and a single group of 16-128 rows:
// K split over KS = 4 waves while the items are very few, or few and the groups
// hold at most 2 rows (more waves in flight per weight byte), fewer splits as
// either grows; batches of U = 8 steps,
// or 4 when a wave's K range is short (one batch) or, in the down product,
// very long (more waves per SIMD in place of deeper batches).
template <bool GATEUP, int U, int KS, bool H16>
static void launch_stream(const GemmTileMap& map, int m_tiles,
                          const uint16_t* xa, const int32_t* src, int a_stride, int a_row0,
                          const uint16_t* wa, const uint16_t* wb, long long w_stride, void* out,
                          int out_stride, int out_row0, int K, int N, const StreamSeg& seg,
                          hipStream_t s) {
  constexpr int IPB = 4 / KS;
  const long long wgs = static_cast<long long>((m_tiles + IPB - 1) / IPB) * (N >> 4) +
                        (stream_seg_items(seg) + IPB - 1) / IPB;
  gemm_bf16_stream_kernel<GATEUP, U, KS, H16>
      <<<dim3(static_cast<unsigned>(wgs)), dim3(256), 0, s>>>(
          map.tiles, m_tiles, map.n_single, xa, src, a_stride, a_row0, wa, wb, w_stride, out,
          out_stride, out_row0, K, N, seg);
}

// seg: an optional dense group launched with the grouped rows (its K may differ;
// the launch shape follows the grouped rows' K and the total item count)
static int stream_split_rule(long long items, int avg) {
  if (items < 1024 || (items < 8192 && avg <= 2)) return 4;
  // groups of up to 8 rows with few items (the down product of a Mixtral-shaped
  // decode step of 17-32 tokens: 3072 items) split too: down at 32 tokens 195 -> 179
  // us; the gate/up product of the same step (10752 items) ran 5 % slower split
  if ((items < 16384 && avg <= 4) || (items < 4096 && avg <= 8)) return 2;
  return 1;
}

static int stream_split(const GemmTileMap& map, int N, const StreamSeg& seg) {
  const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + 15) / 16;
  const long long items = static_cast<long long>(m_tiles) * (N / 16) + stream_seg_items(seg);
  return stream_split_rule(items, map.tiles ? map.avg_rows : map.n_single);
}

int stream_gateup_split(int max_tiles, int avg_rows, int N, int seg_rows, int seg_N) {
  StreamSeg seg;
  seg.rows = seg_rows;
  seg.N = seg_N;
  return stream_split_rule(static_cast<long long>(max_tiles) * (N / 16) + stream_seg_items(seg),
                           avg_rows);
}

// ks_force > 0: that K split instead of the rule's (4, 2 or 1)
template <bool GATEUP, bool H16>
static hipError_t run_stream(const GemmTileMap& map, const uint16_t* xa, const int32_t* src,
                             int a_stride, int a_row0, const uint16_t* wa, const uint16_t* wb,
                             long long w_stride, void* out, int out_stride, int out_row0, int K,
                             int N, hipStream_t s, const StreamSeg& seg = StreamSeg{},
                             int ks_force = 0) {
  const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + 15) / 16;
  const int KS = ks_force > 0 ? ks_force : stream_split(map, N, seg);
  if (KS != 1 && KS != 2 && KS != 4) return hipErrorInvalidValue;
  const int steps = K / 32 / KS;
  const bool u4 = steps < 16 || (!GATEUP && steps >= 100);
#define MOE_STREAM(U_, KS_)                                                                  \
  launch_stream<GATEUP, U_, KS_, H16>(map, m_tiles, xa, src, a_stride, a_row0, wa, wb,       \
                                 w_stride, out, out_stride, out_row0, K, N, seg, s)
  if (KS == 4) {
    if (u4) MOE_STREAM(4, 4); else MOE_STREAM(8, 4);
  } else if (KS == 2) {
    if (u4) MOE_STREAM(4, 2); else MOE_STREAM(8, 2);
  } else {
    if (u4) MOE_STREAM(4, 1); else MOE_STREAM(8, 1);
  }
#undef MOE_STREAM
  return hipGetLastError();
}

// ---------------------------------------------------------------- tile table

__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets,
                                                        int E, int BM, int max_tiles, int ep,
                                                        int4* __restrict__ tiles) {
  __shared__ int part[16];
  const int e = threadIdx.x;
  int lo = 0, n = 0, nt = 0;
  if (e < E) {
    lo = offsets[e];
    n = offsets[e + 1] - lo;
    nt = (n + BM - 1) / BM;
  }
  int total = 0;
  const int start = block_scan_1024(nt, part, &total) - nt;
  const int w = tile_group_weights(e, E, ep);
  for (int i = 0; i < nt && start + i < max_tiles; ++i)
    tiles[start + i] =
        make_int4(w, lo + i * BM, min(BM, n - i * BM), tile_block_word(start, nt, i));
  for (int i = total + e; i < max_tiles; i += 1024) tiles[i] = make_int4(0, 0, 0, 0);
}

int gemm_tile_rows(int dtype_bf16, int R_max, int groups, bool n256_ok) {
  if (!dtype_bf16) return 64;
  // average rows per non-empty group decides how tall a tile can be without
  // mostly computing padding
  const int g = groups < R_max ? groups : R_max;
  const int avg = g > 0 ? R_max / g : 0;
  if (avg <= 16) return 16;          // decode: stream the weights
  if (!n256_ok || avg < 96) return 32;
  // one 256-row tile covers a group of up to 256 rows, so each expert's weight
  // panel is read once; the MFMAs and loads of a tail's empty rows are skipped
  return 256;
}

// Measured on MI355X from cold caches (DeepSeek shape, 256 experts of ~128 rows:
// gate/up -9 %, down -10 % against the m-fastest order with stream-K; 64 experts:
// -2 % and -11 %); with 8 experts the m-fastest order stays ahead, also when
// their rows come as 64 groups (the expert-parallel layout of 8 ranks).
constexpr int kNFastMinExperts = 32;

bool gemm_n_fast(int BM, long long R_max, int experts) {
  return BM == 256 && experts >= kNFastMinExperts && R_max <= 256LL * experts;
}

int gemm_max_tiles(int BM, int R_max, int E) {
  // sum_e ceil(n_e / BM) <= sum_e floor(n_e / BM) + (non-empty groups)
  //                      <= floor(R / BM) + min(E, R)
  // (ceil(n / BM) <= floor(n / BM) + 1 for n > 0). Tight for a decode step of
  // one token: k groups of one row, k tiles, so its streaming launches hold no
  // empty tile rows.
  return R_max / BM + (E < R_max ? E : R_max);
}

hipError_t launch_tile_map(const int32_t* offsets, int E, int BM, int max_tiles, int ep,
                           int32_t* tiles, hipStream_t s) {
  tile_map_kernel<<<dim3(1), dim3(1024), 0, s>>>(offsets, E, BM, max_tiles, ep,
                                                 reinterpret_cast<int4*>(tiles));
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers

template <typename Kern, typename... Extra>
static hipError_t launch_tiled(Kern kern, bool n_fast, int BM, int BN, int threads, size_t lds,
                               const GemmTileMap& map, const uint16_t* xa, const int32_t* src,
                               int a_stride, int a_row0, const uint16_t* wa, const uint16_t* wb,
                               long long w_stride, void* out, int out_stride, int out_row0, int K,
                               int N, hipStream_t s, Extra... extra) {
  if (lds > 65536) {
    hipError_t e = allow_large_lds(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
  }
  const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + BM - 1) / BM;
  const long long n_logical = static_cast<long long>(m_tiles) * (N / BN);
  const long long grid = n_fast                               ? 8LL * ((m_tiles + 7) / 8) * (N / BN)
                         : tile_order_blocked(BM, N / BN) ? blocked_grid(m_tiles, N / BN)
                                                          : ((n_logical + 7) / 8) * 8;
  kern<<<dim3(static_cast<unsigned>(grid)), dim3(threads), lds, s>>>(
      map.tiles, m_tiles, map.n_single, static_cast<int>(n_logical), xa, src, a_stride, a_row0,
      wa, wb, w_stride, out, out_stride, out_row0, K, N, extra...);
  return hipGetLastError();
}

// register-staged small tiles
template <int BM, int BN, int WM, int WN, bool GATEUP, bool H16>
static hipError_t run_small(const GemmTileMap& map, const uint16_t* xa, const int32_t* src,
                            int a_stride, int a_row0, const uint16_t* wa, const uint16_t* wb,
                            long long w_stride, void* out, int out_stride, int out_row0, int K,
                            int N, hipStream_t s) {
  constexpr int WR = GATEUP ? 2 * BN : BN;
  const size_t lds = static_cast<size_t>(2) * (BM + WR) * kPitch * sizeof(uint16_t);
  return launch_tiled(gemm_bf16_kernel<BM, BN, WM, WN, GATEUP, H16>, false, BM, BN, 64 * WM * WN, lds, map,
                      xa, src, a_stride, a_row0, wa, wb, w_stride, out, out_stride, out_row0, K,
                      N, s);
}

// LDS-DMA large tiles
// Three LDS stages where they fit (256 x 128 down tiles: 3 x 48 KB), which
// keeps two stages of loads in flight per CU; those tiles serve short groups,
// where the weights stream from HBM and load latency matters most.
template <int BM, int BN, int WM, int WN, bool GATEUP, bool H16, bool HOUT = false,
          bool NF = false, int XS = 0>
static hipError_t run_lds(const GemmTileMap& map, const uint16_t* xa, const int32_t* src,
                          int a_stride, int a_row0, const uint16_t* wa, const uint16_t* wb,
                          long long w_stride, void* out, int out_stride, int out_row0, int K,
                          int N, hipStream_t s, float* h1o = nullptr, float* h3o = nullptr) {
  constexpr int WR = GATEUP ? 2 * BN : BN;
  constexpr size_t kStage = static_cast<size_t>(BM + WR) * kRowBytes;
  constexpr int ST = 3 * kStage <= kMaxLdsBytes ? 3 : 2;
  constexpr size_t kShort =
      XS > 0 ? short_ring_stages(XS, WR) * static_cast<size_t>(XS + WR) * kRowBytes : 0;
  const size_t lds = ST * kStage > kShort ? ST * kStage : kShort;
  return launch_tiled(gemm_bf16_lds_kernel<BM, BN, WM, WN, GATEUP, ST, HOUT, false, NF, XS, H16>, NF, BM, BN,
                      64 * WM * WN, lds, map, xa, src, a_stride, a_row0, wa, wb, w_stride, out,
                      out_stride, out_row0, K, N, s, h1o, h3o, static_cast<float*>(nullptr));
}

// Workgroups of a persistent launch: one per CU of the current device, a multiple
// of 8 (one share per XCD), at most `cap`; 0 if the count is unavailable.
int persistent_workgroups(int cap) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cus = cus < cap ? cus : cap;
  return cus / 8 * 8;
}

static int streamk_workgroups() { return persistent_workgroups(kStreamKMaxWorkgroups); }

// Plain 256 x 256 products as stream-K (see gemm_bf16_lds_kernel) when the
// launch has at least one tile per workgroup: the fix-up kernel follows.
// Returns hipErrorNotSupported when stream-K does not apply.
template <bool H16>
static hipError_t run_lds_streamk(const GemmTileMap& map, const uint16_t* xa, const int32_t* src,
                                  int a_stride, int a_row0, const uint16_t* wa, long long w_stride,
                                  float* out, int out_stride, int out_row0, int K, int N,
                                  float* sk_part, hipStream_t s) {
  constexpr int BM = 256, BN = 256;
  constexpr size_t lds = 2 * static_cast<size_t>(BM + BN) * kRowBytes;
  const int P = streamk_workgroups();
  const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + BM - 1) / BM;
  if (P < 8 || static_cast<long long>(m_tiles) * (N / BN) < P) return hipErrorNotSupported;
  auto kern = gemm_bf16_lds_kernel<BM, BN, 2, 4, false, 2, false, true, false, 0, H16>;
  hipError_t e = allow_large_lds(reinterpret_cast<const void*>(kern), lds);
  if (e != hipSuccess) return e;
  kern<<<dim3(P), dim3(512), lds, s>>>(map.tiles, m_tiles, map.n_single, 0, xa, src, a_stride,
                                       a_row0, wa, nullptr, w_stride, out, out_stride, out_row0,
                                       K, N, nullptr, nullptr, sk_part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  streamk_fixup_kernel<BM, BN, kBK><<<dim3(P - 1, 4), dim3(256), 0, s>>>(
      map.tiles, m_tiles, map.n_single, K, N, P, sk_part, out, out_stride, out_row0);
  return hipGetLastError();
}

// One wave per SIMD, 256 x 256 weight-row tiles, BK = 32 in an ST-stage ring.
#ifndef MOE_W4_STAGES
#define MOE_W4_STAGES 5
#endif
constexpr int kW4Stages = MOE_W4_STAGES;

template <bool GATEUP, bool NF, bool H16>
static hipError_t run_w4(const GemmTileMap& map, const uint16_t* xa, const int32_t* src,
                         int a_stride, int a_row0, const uint16_t* wa, const uint16_t* wb,
                         long long w_stride, void* out, int out_stride, int out_row0, int K,
                         int N, hipStream_t s) {
  constexpr int BN = GATEUP ? 128 : 256;
  constexpr size_t lds = static_cast<size_t>(kW4Stages) * kW4Stage;
  return launch_tiled(gemm_bf16_w4_kernel<GATEUP, kW4Stages, NF, H16>, NF, 256, BN, 256, lds,
                      map, xa, src, a_stride, a_row0, wa, wb, w_stride, out, out_stride,
                      out_row0, K, N, s);
}

// Token rows of the short three-stage ring of the 256 x 128 gate/up tiles:
// 3 x (160 + 256) x 128 B = 156 KB of LDS. Measured from cold caches: gate/up
// at the DeepSeek shape (4096 tokens) 3.22 -> 3.06 ms with the shared expert,
// Mixtral shape at 512 tokens 0.43 -> 0.39 ms; with full tiles (4096 tokens) the
// larger LDS allotment cost 1-3 %, hence the average-rows condition.
constexpr int kShortRingRows = 160;

// BM = 256 needs N % 256 == 0 (down) / N % 128 == 0 (gate/up); the
// caller picks BM with gemm_tile_rows(), which checks that.
// The forward's gate/up products write the activation as IEEE half (its down
// product reads it so); the backward's recompute (h1 set) keeps bf16.
hipError_t launch_gemm_gateup_bf16(const GemmTileMap& map, const GateUpArgs& a, int BM,
                                   hipStream_t s) {
  const auto* x = static_cast<const uint16_t*>(a.x);
  const auto* w1 = static_cast<const uint16_t*>(a.w1);
  const auto* w3 = static_cast<const uint16_t*>(a.w3);
  // groups of at most kShortRingRows rows on average: tiles that short take
  // three LDS stages of kShortRingRows token rows (gemm_bf16_lds_kernel, XS)
  const bool short_ring = map.tiles != nullptr && map.avg_rows > 0 && map.avg_rows <= kShortRingRows;
  if (a.h1 != nullptr) {   // pre-activations too: 256-row tiles only
    if (BM != 256 || a.h3 == nullptr) return hipErrorInvalidValue;
    if (map.n_fast)
      return run_lds<256, 128, 2, 4, true, false, true, true, kShortRingRows>(
          map, x, a.src, a.K, 0, w1, w3, a.w_stride, a.act, a.act_stride, a.out_row0, a.K, a.N, s,
          a.h1, a.h3);
    if (short_ring)
      return run_lds<256, 128, 2, 4, true, false, true, false, kShortRingRows>(
          map, x, a.src, a.K, 0, w1, w3, a.w_stride, a.act, a.act_stride, a.out_row0, a.K, a.N, s,
          a.h1, a.h3);
    return run_lds<256, 128, 2, 4, true, false, true>(map, x, a.src, a.K, 0, w1, w3, a.w_stride,
                                                      a.act, a.act_stride, a.out_row0, a.K, a.N,
                                                      s, a.h1, a.h3);
  }
  if (BM == 256 && map.n_fast)
    return run_lds<256, 128, 2, 4, true, true, false, true, kShortRingRows>(
        map, x, a.src, a.K, 0, w1, w3, a.w_stride, a.act, a.act_stride, a.out_row0, a.K, a.N, s);
  if (BM == 256 && short_ring)
    return run_lds<256, 128, 2, 4, true, true, false, false, kShortRingRows>(
        map, x, a.src, a.K, 0, w1, w3, a.w_stride, a.act, a.act_stride, a.out_row0, a.K, a.N, s);
  // full 256-row tiles: one wave per SIMD (gemm_bf16_w4_kernel)
  if (BM == 256)
    return run_w4<true, false, true>(map, x, a.src, a.K, 0, w1, w3, a.w_stride, a.act,
                                     a.act_stride, a.out_row0, a.K, a.N, s);
  if (BM == 16)
    return run_stream<true, true>(map, x, a.src, a.K, 0, w1, w3, a.w_stride, a.act, a.act_stride,
                                  a.out_row0, a.K, a.N, s, StreamSeg{}, a.stream_ks);
  return run_small<32, 64, 1, 2, true, true>(map, x, a.src, a.K, 0, w1, w3, a.w_stride, a.act,
                                             a.act_stride, a.out_row0, a.K, a.N, s);
}

hipError_t launch_gemm_gateup_bf16_with_shared(const GemmTileMap& map, const GateUpArgs& a,
                                               const GateUpArgs& sh, int sh_rows, hipStream_t s) {
  if (a.h1 != nullptr || sh.src != nullptr || a.act_stride != sh.act_stride)
    return hipErrorInvalidValue;
  StreamSeg seg;
  seg.xa = static_cast<const uint16_t*>(sh.x);
  seg.wa = static_cast<const uint16_t*>(sh.w1);
  seg.wb = static_cast<const uint16_t*>(sh.w3);
  seg.rows = sh_rows;
  seg.K = sh.K;
  seg.N = sh.N;
  seg.out_row0 = sh.out_row0;
  return run_stream<true, true>(map, static_cast<const uint16_t*>(a.x), a.src, a.K, 0,
                                static_cast<const uint16_t*>(a.w1),
                                static_cast<const uint16_t*>(a.w3), a.w_stride, a.act,
                                a.act_stride, a.out_row0, a.K, a.N, s, seg);
}

hipError_t launch_gemm_down_bf16_with_shared(const GemmTileMap& map, const DownArgs& a,
                                             const DownArgs& sh, int sh_rows, hipStream_t s) {
  const int ys = a.out_stride > 0 ? a.out_stride : a.N;
  if (sh.src != nullptr || sh.act_stride != a.act_stride || sh.N != a.N ||
      (sh.out_stride > 0 ? sh.out_stride : sh.N) != ys || sh.y != a.y ||
      sh.act_f16 != a.act_f16)
    return hipErrorInvalidValue;
  StreamSeg seg;
  seg.xa = static_cast<const uint16_t*>(sh.act);
  seg.wa = static_cast<const uint16_t*>(sh.w2);
  seg.a_row0 = sh.in_row0;
  seg.rows = sh_rows;
  seg.K = sh.K;
  seg.N = sh.N;
  seg.out_row0 = sh.out_row0;
  if (a.act_f16)
    return run_stream<false, true>(map, static_cast<const uint16_t*>(a.act), a.src, a.act_stride,
                                   a.in_row0, static_cast<const uint16_t*>(a.w2), nullptr,
                                   a.w_stride, a.y, ys, a.out_row0, a.K, a.N, s, seg);
  return run_stream<false, false>(map, static_cast<const uint16_t*>(a.act), a.src, a.act_stride,
                                  a.in_row0, static_cast<const uint16_t*>(a.w2), nullptr,
                                  a.w_stride, a.y, ys, a.out_row0, a.K, a.N, s, seg);
}

// The fused down product and combine (gemm_down_combine_kernel) where it applies:
// half activation rows in y_perm order (no src, no row offsets), at most 16 tokens
// (so each group is one tile), and the K split and batch depth that the streaming
// launch's own rule picks, with that split times the tile bound within one
// workgroup, and at most kCombineMaxK slots per token. Otherwise
// hipErrorNotSupported, and nothing is launched.
hipError_t launch_gemm_down_combine_bf16(const GemmTileMap& map, const DownArgs& a,
                                         const int32_t* dest, const float* gates, int T, int k,
                                         float* y, hipStream_t s) {
  if (map.tiles == nullptr || !a.act_f16 || a.src != nullptr || a.in_row0 != 0 ||
      T <= 0 || T > 16 || k <= 0 || k > kCombineMaxK || a.N % 16 != 0 || a.K % 32 != 0 ||
      map.max_tiles > 4)
    return hipErrorNotSupported;
  const int KS = stream_split(map, a.N, StreamSeg{});
  const int steps = a.K / 32 / KS;
  const bool u4 = steps < 16 || steps >= 100;   // as run_stream for the down product
  const auto* act = static_cast<const uint16_t*>(a.act);
  const auto* w2 = static_cast<const uint16_t*>(a.w2);
  const dim3 grid(a.N / 16);
#define MOE_DOWN_COMBINE(U_, KS_, NTL_)                                                        \
  gemm_down_combine_kernel<U_, KS_, NTL_, true><<<grid, dim3(64 * KS_ * NTL_), 0, s>>>(      \
      map.tiles, map.max_tiles, act, a.act_stride, w2, a.w_stride, a.K, a.N, dest, gates, T, \
      k, y)
  if (KS == 4 && u4 && map.max_tiles <= 2) MOE_DOWN_COMBINE(4, 4, 2);
  else if (KS == 4 && u4) MOE_DOWN_COMBINE(4, 4, 4);
  else if (KS == 4 && map.max_tiles <= 2) MOE_DOWN_COMBINE(8, 4, 2);
  else return hipErrorNotSupported;
#undef MOE_DOWN_COMBINE
  return hipGetLastError();
}

// Output tiles of 256 columns unless that leaves fewer than two tiles per CU
// (few, short groups, as in a prefill of a few hundred tokens): then 128
// columns, which doubles the tiles and, at 3 x 48 KB, runs three LDS stages.
static int gemm_down_cols(int BM, int m_tiles, int N) {
  if (BM != 256 || N % 256 != 0) return 256;
  return static_cast<long long>(m_tiles) * (N / 256) < 2 * kNumCUs ? 128 : 256;
}

template <bool H16>
static hipError_t launch_down(const GemmTileMap& map, const DownArgs& a, int BM, hipStream_t s) {
  const int ys = a.out_stride > 0 ? a.out_stride : a.N;
  const auto* act = static_cast<const uint16_t*>(a.act);
  const auto* w2 = static_cast<const uint16_t*>(a.w2);
  // weight-streaming shapes, n-fastest order: 256 x 256 tiles whose groups of at
  // most kShortRingRows rows run three stages of that many token rows and 256
  // weight rows (3 x 52 KB), so two stages of 32 KB of weights are in flight per
  // CU. Measured at the DeepSeek shape (4096 tokens, ~128 rows per expert): 2.22
  // -> 2.00 ms against 256 x 128 tiles with three full stages (16 KB of weights
  // per stage); Switch shape even. (A four-stage ring of 160-row stages at 128
  // columns, 4 x 36 KB, measured no faster than the three full stages.)
  if (BM == 256 && map.n_fast && a.N % 256 == 0)
    return run_lds<256, 256, 2, 4, false, H16, false, true, kShortRingRows>(
        map, act, a.src, a.act_stride, a.in_row0, w2, nullptr, a.w_stride, a.y, ys, a.out_row0,
        a.K, a.N, s);
  if (BM == 256 && map.n_fast && a.N % 128 == 0)
    return run_lds<256, 128, 2, 4, false, H16, false, true>(
        map, act, a.src, a.act_stride, a.in_row0, w2, nullptr, a.w_stride, a.y, ys, a.out_row0,
        a.K, a.N, s);
  if (BM == 256) {
    const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + BM - 1) / BM;
    if (gemm_down_cols(BM, m_tiles, a.N) == 128)
      return run_lds<256, 128, 2, 4, false, H16>(map, act, a.src, a.act_stride, a.in_row0, w2,
                                                 nullptr, a.w_stride, a.y, ys, a.out_row0, a.K,
                                                 a.N, s);
    if (a.sk_part != nullptr) {
      const hipError_t e = run_lds_streamk<H16>(map, act, a.src, a.act_stride, a.in_row0, w2,
                                                a.w_stride, a.y, ys, a.out_row0, a.K, a.N,
                                                a.sk_part, s);
      if (e != hipErrorNotSupported) return e;
    }
    return run_lds<256, 256, 2, 4, false, H16>(map, act, a.src, a.act_stride, a.in_row0, w2,
                                               nullptr, a.w_stride, a.y, ys, a.out_row0, a.K,
                                               a.N, s);
  }
  if (BM == 16)
    return run_stream<false, H16>(map, act, a.src, a.act_stride, a.in_row0, w2, nullptr,
                                  a.w_stride, a.y, ys, a.out_row0, a.K, a.N, s);
  return run_small<32, 64, 1, 2, false, H16>(map, act, a.src, a.act_stride, a.in_row0, w2,
                                             nullptr, a.w_stride, a.y, ys, a.out_row0, a.K,
                                             a.N, s);
}

hipError_t launch_gemm_down_bf16(const GemmTileMap& map, const DownArgs& a, int BM,
                                 hipStream_t s) {
  return a.act_f16 ? launch_down<true>(map, a, BM, s) : launch_down<false>(map, a, BM, s);
}

}  // namespace moe
