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
// * BK = 64 tiles of both operands double-buffered in LDS with a 16-byte row
//   pad (no bank conflicts for the 16-byte fragment reads); global loads of
//   tile k+1 are in flight while tile k is multiplied.
// * A device-side tile table (one entry per 128-row tile of each group) lets
//   one launch cover every group with no host sync; grid slots past the last
//   real tile exit at once.
// * Workgroups are dispatched round-robin over the 8 XCDs; the launch index is
//   remapped so each XCD works on a contiguous range of (n-tile, m-tile) pairs
//   with m fastest, so the tiles that share a weight panel share an L2.
#include "common.h"
#include "kernels.h"

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

// Launch index -> (m_tile, n_tile), XCD-contiguous (see the file comment).
__device__ __forceinline__ void xcd_tile(int n_logical, int max_tiles, int& m_tile, int& n_tile) {
  const int L = blockIdx.x;
  const int per = (n_logical + 7) >> 3;
  const int logical = (L & 7) * per + (L >> 3);
  if (logical >= n_logical) { m_tile = -1; n_tile = 0; return; }
  m_tile = logical % max_tiles;
  n_tile = logical / max_tiles;
}

template <int BM, int BN, int WM, int WN, bool GATEUP>
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
    for (int i = 0; i < WC; ++i) *reinterpret_cast<u32x4*>(ws + woff[i]) = wr[i];
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
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[b], bfr[a], acc[a][b], 0, 0, 0);
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
          pk[0] = pack_bf16x2(h[0], h[1]);
          pk[1] = pack_bf16x2(h[2], h[3]);
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

// ---------------------------------------------------------------- tile table

__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets,
                                                        int E, int BM, int max_tiles,
                                                        int4* __restrict__ tiles) {
  __shared__ int part[1024];
  const int e = threadIdx.x;
  int lo = 0, n = 0, nt = 0;
  if (e < E) {
    lo = offsets[e];
    n = offsets[e + 1] - lo;
    nt = (n + BM - 1) / BM;
  }
  part[e] = nt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = e >= off ? part[e - off] : 0;
    __syncthreads();
    part[e] += v;
    __syncthreads();
  }
  const int start = part[e] - nt;
  const int total = part[1023];
  for (int i = 0; i < nt; ++i) tiles[start + i] = make_int4(e, lo + i * BM, min(BM, n - i * BM), 0);
  for (int i = total + e; i < max_tiles; i += 1024) tiles[i] = make_int4(0, 0, 0, 0);
}

int gemm_tile_rows(int dtype_bf16, int R_max, bool n128_ok) {
  if (!dtype_bf16) return 64;
  return (R_max >= 2048 && n128_ok) ? 128 : 32;
}

int gemm_max_tiles(int BM, int R_max, int E) {
  // sum_e ceil(n_e / BM) <= ceil(R / BM) + (number of non-empty groups)
  return (R_max + BM - 1) / BM + (E < R_max ? E : R_max);
}

hipError_t launch_tile_map(const int32_t* offsets, int E, int BM, int max_tiles, int32_t* tiles,
                           hipStream_t s) {
  tile_map_kernel<<<dim3(1), dim3(1024), 0, s>>>(offsets, E, BM, max_tiles,
                                                 reinterpret_cast<int4*>(tiles));
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers

template <int BM, int BN, int WM, int WN, bool GATEUP>
static hipError_t run_bf16(const GemmTileMap& map, const uint16_t* xa, const int32_t* src,
                           int a_stride, int a_row0, const uint16_t* wa, const uint16_t* wb,
                           long long w_stride, void* out, int out_stride, int out_row0, int K,
                           int N, hipStream_t s) {
  constexpr int WR = GATEUP ? 2 * BN : BN;
  const size_t lds = static_cast<size_t>(2) * (BM + WR) * kPitch * sizeof(uint16_t);
  auto kern = gemm_bf16_kernel<BM, BN, WM, WN, GATEUP>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + BM - 1) / BM;
  const long long n_logical = static_cast<long long>(m_tiles) * (N / BN);
  const long long grid = ((n_logical + 7) / 8) * 8;
  kern<<<dim3(static_cast<unsigned>(grid)), dim3(64 * WM * WN), lds, s>>>(
      map.tiles, m_tiles, map.n_single, static_cast<int>(n_logical), xa, src, a_stride, a_row0,
      wa, wb, w_stride, out, out_stride, out_row0, K, N);
  return hipGetLastError();
}

hipError_t launch_gemm_gateup_bf16(const GemmTileMap& map, const GateUpArgs& a, int BM,
                                   hipStream_t s) {
  const auto* x = static_cast<const uint16_t*>(a.x);
  const auto* w1 = static_cast<const uint16_t*>(a.w1);
  const auto* w3 = static_cast<const uint16_t*>(a.w3);
  if (BM == 128)
    return run_bf16<128, 128, 2, 2, true>(map, x, a.src, a.K, 0, w1, w3, a.w_stride, a.act,
                                          a.act_stride, a.out_row0, a.K, a.N, s);
  return run_bf16<32, 64, 1, 2, true>(map, x, a.src, a.K, 0, w1, w3, a.w_stride, a.act,
                                      a.act_stride, a.out_row0, a.K, a.N, s);
}

hipError_t launch_gemm_down_bf16(const GemmTileMap& map, const DownArgs& a, int BM,
                                 hipStream_t s) {
  const auto* act = static_cast<const uint16_t*>(a.act);
  const auto* w2 = static_cast<const uint16_t*>(a.w2);
  if (BM == 128)
    return run_bf16<128, 128, 2, 2, false>(map, act, nullptr, a.act_stride, a.in_row0, w2,
                                           nullptr, a.w_stride, a.y, a.N, a.out_row0, a.K, a.N,
                                           s);
  return run_bf16<32, 64, 1, 2, false>(map, act, nullptr, a.act_stride, a.in_row0, w2, nullptr,
                                       a.w_stride, a.y, a.N, a.out_row0, a.K, a.N, s);
}

}  // namespace moe
