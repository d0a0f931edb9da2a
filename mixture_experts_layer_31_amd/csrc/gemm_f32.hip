// Grouped expert GEMMs in true fp32 arithmetic (fp32 inputs and weights).
//
// Same grouped formulation and tile table as the bf16 kernels (CMU 15-779
// Lecture 21 notes, §3.3), computed with fp32 FMAs: 64x64 output tiles, 16-deep
// K slices staged transposed in LDS, a 4x4 register micro-tile per thread. The
// gate/up kernel keeps a gate and an up accumulator per output and applies the
// SwiGLU epilogue act = silu(g) * u; the hidden activation stays fp32.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kFBM = 64, kFBN = 64, kFBK = 16;

template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const int32_t* __restrict__ tiles, int max_tiles, int n_single, const float* __restrict__ xa,
    const int32_t* __restrict__ src, int a_stride, int a_row0, const float* __restrict__ w_a,
    const float* __restrict__ w_b, long long w_stride, float* __restrict__ out, int out_stride,
    int out_row0, int K, int N) {
  constexpr int WR = GATEUP ? 2 * kFBN : kFBN;
  __shared__ float Xs[kFBK][kFBM + 4];
  __shared__ float Ws[kFBK][WR + 4];

  const int m_tile = blockIdx.x % max_tiles;
  const int n_tile = blockIdx.x / max_tiles;
  int group, row0, rows;
  if (tiles != nullptr) {
    const int4 t = reinterpret_cast<const int4*>(tiles)[m_tile];
    group = t.x; row0 = t.y; rows = t.z;
  } else {
    group = 0; row0 = m_tile * kFBM; rows = min(kFBM, n_single - row0);
  }
  if (rows <= 0) return;
  const int n0 = n_tile * kFBN;
  const int tid = threadIdx.x;

  // loader: X tile row tid/4, k quad (tid%4)*4
  const int xr = tid >> 2, xq = (tid & 3) * 4;
  int grow = row0 + min(xr, rows - 1);
  if (src != nullptr) grow = src[grow];
  const float* xg = xa + (static_cast<size_t>(a_row0) + grow) * a_stride + xq;
  const size_t wbase = static_cast<size_t>(group) * w_stride;
  const float* wg[WR / 64];
#pragma unroll
  for (int i = 0; i < WR / 64; ++i) {
    const int r = xr + 64 * i;
    const float* wsrc = (!GATEUP || r < kFBN) ? w_a : w_b;
    const int n = n0 + ((GATEUP && r >= kFBN) ? r - kFBN : r);
    wg[i] = wsrc + wbase + static_cast<size_t>(n) * K + xq;
  }

  const int tm = tid >> 4, tn = tid & 15;
  float ag[4][4], au[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) { ag[i][j] = 0.f; au[i][j] = 0.f; }

  for (int k0 = 0; k0 < K; k0 += kFBK) {
    const f32x4 xv = *reinterpret_cast<const f32x4*>(xg + k0);
#pragma unroll
    for (int q = 0; q < 4; ++q) Xs[xq + q][xr] = xv[q];
#pragma unroll
    for (int i = 0; i < WR / 64; ++i) {
      const f32x4 wv = *reinterpret_cast<const f32x4*>(wg[i] + k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) Ws[xq + q][xr + 64 * i] = wv[q];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFBK; ++kk) {
      float a[4], bg[4], bu[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = Xs[kk][tm * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bg[j] = Ws[kk][tn * 4 + j];
      if (GATEUP) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bu[j] = Ws[kk][kFBN + tn * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ag[i][j] = fmaf(a[i], bg[j], ag[i][j]);
          if (GATEUP) au[i][j] = fmaf(a[i], bu[j], au[i][j]);
        }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = tm * 4 + i;
    if (m >= rows) continue;
    float* o = out + (static_cast<size_t>(out_row0) + row0 + m) * out_stride + n0 + tn * 4;
    f32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (GATEUP) {
        const float g = ag[i][j];
        v[j] = g / (1.0f + expf(-g)) * au[i][j];
      } else {
        v[j] = ag[i][j];
      }
    }
    *reinterpret_cast<f32x4*>(o) = v;
  }
}

hipError_t launch_gemm_gateup_f32(const GemmTileMap& map, const GateUpArgs& a, hipStream_t s) {
  const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + kFBM - 1) / kFBM;
  const long long grid = static_cast<long long>(m_tiles) * (a.N / kFBN);
  gemm_f32_kernel<true><<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, s>>>(
      map.tiles, m_tiles, map.n_single, static_cast<const float*>(a.x), a.src, a.K, 0,
      static_cast<const float*>(a.w1), static_cast<const float*>(a.w3), a.w_stride,
      static_cast<float*>(a.act), a.act_stride, a.out_row0, a.K, a.N);
  return hipGetLastError();
}

hipError_t launch_gemm_down_f32(const GemmTileMap& map, const DownArgs& a, hipStream_t s) {
  const int m_tiles = map.tiles ? map.max_tiles : (map.n_single + kFBM - 1) / kFBM;
  const long long grid = static_cast<long long>(m_tiles) * (a.N / kFBN);
  gemm_f32_kernel<false><<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, s>>>(
      map.tiles, m_tiles, map.n_single, static_cast<const float*>(a.act), nullptr, a.act_stride,
      a.in_row0, static_cast<const float*>(a.w2), nullptr, a.w_stride, a.y, a.N, a.out_row0, a.K,
      a.N);
  return hipGetLastError();
}

}  // namespace moe
