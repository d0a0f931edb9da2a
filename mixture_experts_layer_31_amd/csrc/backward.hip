// Backward of the MoE layer: the elementwise, reduction and layout kernels.
//
// Gradients of L = sum_t <dy_t, y_t> (+ L_aux) for y_t = sum_j g_{t,j} f_{e_j}(x_t)
// (+ shared), f(x) = W2 (silu(W1 x) * (W3 x)). The top-k selection and the
// capacity drops pass no gradient; the router learns through the gates of the
// selected experts ("Week 2 Day 2: Mixture of Experts", §1.3), and the balance
// loss adds (alpha E / T) p_i (f_i - sum_j p_j f_j) to the logits' gradient
// (same notes, §3.2). The expert products are the transposed GEMMs of the
// forward ones (CMU 15-779 Lecture 21 notes, §7: dW2 = H^T dY and so on); the
// GEMMs themselves run in gemm_bf16.hip. Every reduction here sums in a fixed
// order, so the gradients are reproducible bit for bit.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPadRows = 64;   // per-group row padding of the transposed operands

// poff[g] = sum over g' < g of roundup(count_g', 64); poff[G] = padded total.
// One 1024-thread workgroup (G <= 1024).
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets,
                                                           int G, int32_t* __restrict__ poff) {
  __shared__ int part[1024];
  const int g = threadIdx.x;
  int pc = 0;
  if (g < G) {
    const int c = offsets[g + 1] - offsets[g];
    pc = (c + kPadRows - 1) / kPadRows * kPadRows;
  }
  part[g] = pc;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = g >= o ? part[g - o] : 0;
    __syncthreads();
    part[g] += v;
    __syncthreads();
  }
  if (g < G) poff[g + 1] = part[g];
  if (g == 0) poff[0] = 0;
}

// out[c][poff[g] + (r - offsets[g])] = in[row(r)][c] for every row r of group g,
// row(r) = src[r] (gather) or in_row0 + r; the padding columns of each group
// are zeros. grid.x: 64-column chunks of the padded row space (groups start at
// multiples of 64, so a chunk lies in one group; chunks past poff[G] exit),
// grid.y: 64-wide chunks of C.
__global__ __launch_bounds__(256) void transpose_rows_kernel(
    const uint16_t* __restrict__ in, int in_stride, const int32_t* __restrict__ src, int in_row0,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ poff, int G, int C,
    uint16_t* __restrict__ out, int out_stride) {
  __shared__ uint16_t tile[64][64 + 2];
  const int p0 = blockIdx.x * 64;
  if (p0 >= poff[G]) return;
  int lo = 0, hi = G;                       // largest g with poff[g] <= p0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (poff[mid] <= p0) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int r0 = offsets[g] + (p0 - poff[g]);
  const int nrows = min(64, max(0, offsets[g + 1] - r0));
  const int c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  {
    const int rr = tid >> 2, cc = (tid & 3) * 16;   // row rr, 16 columns from cc
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (rr < nrows) {
      const int r = r0 + rr;
      const size_t row = src != nullptr ? static_cast<size_t>(src[r]) : static_cast<size_t>(in_row0) + r;
      const u32x4* p = reinterpret_cast<const u32x4*>(in + row * in_stride + c0 + cc);
      a = p[0];
      b = p[1];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[rr][cc + 2 * q] = static_cast<uint16_t>(a[q] & 0xFFFFu);
      tile[rr][cc + 2 * q + 1] = static_cast<uint16_t>(a[q] >> 16);
      tile[rr][cc + 8 + 2 * q] = static_cast<uint16_t>(b[q] & 0xFFFFu);
      tile[rr][cc + 8 + 2 * q + 1] = static_cast<uint16_t>(b[q] >> 16);
    }
  }
  __syncthreads();
  {
    const int cc = tid >> 2, pp = (tid & 3) * 16;   // output row c0 + cc, 16 columns
    u32x4 a, b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = static_cast<uint32_t>(tile[pp + 2 * q][cc]) |
             (static_cast<uint32_t>(tile[pp + 2 * q + 1][cc]) << 16);
      b[q] = static_cast<uint32_t>(tile[pp + 8 + 2 * q][cc]) |
             (static_cast<uint32_t>(tile[pp + 8 + 2 * q + 1][cc]) << 16);
    }
    u32x4* o = reinterpret_cast<u32x4*>(out + static_cast<size_t>(c0 + cc) * out_stride + p0 + pp);
    o[0] = a;
    o[1] = b;
  }
}

// out[b][n][col0 + m] = in[b][m][n] for in [B][M][N]; M, N multiples of 64.
// grid (N/64, M/64, B).
__global__ __launch_bounds__(256) void transpose_mat_kernel(const uint16_t* __restrict__ in, int M,
                                                            int N, uint16_t* __restrict__ out,
                                                            int out_stride, int col0,
                                                            long long out_batch) {
  __shared__ uint16_t tile[64][64 + 2];
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  const uint16_t* ib = in + static_cast<size_t>(blockIdx.z) * M * N;
  uint16_t* ob = out + static_cast<size_t>(blockIdx.z) * out_batch;
  const int tid = threadIdx.x;
  {
    const int rr = tid >> 2, cc = (tid & 3) * 16;
    const u32x4* p = reinterpret_cast<const u32x4*>(ib + static_cast<size_t>(m0 + rr) * N + n0 + cc);
    const u32x4 a = p[0], b = p[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[rr][cc + 2 * q] = static_cast<uint16_t>(a[q] & 0xFFFFu);
      tile[rr][cc + 2 * q + 1] = static_cast<uint16_t>(a[q] >> 16);
      tile[rr][cc + 8 + 2 * q] = static_cast<uint16_t>(b[q] & 0xFFFFu);
      tile[rr][cc + 8 + 2 * q + 1] = static_cast<uint16_t>(b[q] >> 16);
    }
  }
  __syncthreads();
  {
    const int cc = tid >> 2, pp = (tid & 3) * 16;
    u32x4 a, b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = static_cast<uint32_t>(tile[pp + 2 * q][cc]) |
             (static_cast<uint32_t>(tile[pp + 2 * q + 1][cc]) << 16);
      b[q] = static_cast<uint32_t>(tile[pp + 8 + 2 * q][cc]) |
             (static_cast<uint32_t>(tile[pp + 8 + 2 * q + 1][cc]) << 16);
    }
    u32x4* o = reinterpret_cast<u32x4*>(ob + static_cast<size_t>(n0 + cc) * out_stride + col0 + m0 + pp);
    o[0] = a;
    o[1] = b;
  }
}

// act = silu(h1) * h3 rounded to bf16, rows [row0, row0 + rows), n columns.
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const float* __restrict__ h1,
                                                         const float* __restrict__ h3,
                                                         int stride, int row0, int rows, int n,
                                                         uint16_t* __restrict__ act) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long long>(rows) * n) return;
  const size_t o = static_cast<size_t>(row0 + i / n) * stride + i % n;
  act[o] = f32_to_bf16(silu(h1[o]) * h3[o]);
}

// dh1 = da * h3 * silu'(h1), dh3 = da * silu(h1), silu'(u) = s (1 + u (1 - s)),
// s = 1 / (1 + e^-u); written as bf16 into dH[row][0..n) and dH[row][n..2n)
// (dH row stride 2 * stride).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ da,
                                                         const float* __restrict__ h1,
                                                         const float* __restrict__ h3,
                                                         int stride, int row0, int rows, int n,
                                                         uint16_t* __restrict__ dH) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long long>(rows) * n) return;
  const size_t r = static_cast<size_t>(row0 + i / n);
  const int f = static_cast<int>(i % n);
  const size_t o = r * stride + f;
  const float u = h1[o];
  const float s = 1.0f / (1.0f + __expf(-u));
  const float g = da[o];
  dH[r * 2 * stride + f] = f32_to_bf16(g * h3[o] * s * (1.0f + u * (1.0f - s)));
  dH[r * 2 * stride + n + f] = f32_to_bf16(g * u * s);
}

// One workgroup per token: dg[t,j] = <dy_t, yp[dest[t,j]]> (0 for a dropped
// slot), dyp[dest[t,j]] = g[t,j] dy_t in bf16; with a shared expert its rows
// dyp[shared_row0 + t] = dy_t. The dot products sum per thread in index order,
// then over threads in a fixed tree.
__global__ __launch_bounds__(256) void combine_bwd_kernel(const float* __restrict__ dy,
                                                          const float* __restrict__ yp,
                                                          const int32_t* __restrict__ dest,
                                                          const float* __restrict__ gates,
                                                          int k, int d, int shared_row0,
                                                          float* __restrict__ dg,
                                                          uint16_t* __restrict__ dyp) {
  __shared__ float red[256];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* dyt = dy + static_cast<size_t>(t) * d;
  for (int j = 0; j < k; ++j) {
    const int r = dest[static_cast<size_t>(t) * k + j];
    if (r < 0) {
      if (tid == 0) dg[static_cast<size_t>(t) * k + j] = 0.f;
      continue;
    }
    const float g = gates[static_cast<size_t>(t) * k + j];
    const float* ypr = yp + static_cast<size_t>(r) * d;
    uint16_t* dr = dyp + static_cast<size_t>(r) * d;
    float acc = 0.f;
    for (int i = tid * 4; i < d; i += 1024) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(dyt + i);
      const f32x4 b = *reinterpret_cast<const f32x4*>(ypr + i);
      acc = fmaf(a[0], b[0], acc);
      acc = fmaf(a[1], b[1], acc);
      acc = fmaf(a[2], b[2], acc);
      acc = fmaf(a[3], b[3], acc);
      u32x2 pk;
      pk[0] = pack_bf16x2(g * a[0], g * a[1]);
      pk[1] = pack_bf16x2(g * a[2], g * a[3]);
      *reinterpret_cast<u32x2*>(dr + i) = pk;
    }
    red[tid] = acc;
    __syncthreads();
    for (int h = 128; h >= 1; h >>= 1) {
      if (tid < h) red[tid] += red[tid + h];
      __syncthreads();
    }
    if (tid == 0) dg[static_cast<size_t>(t) * k + j] = red[0];
    __syncthreads();
  }
  if (shared_row0 >= 0) {
    uint16_t* dr = dyp + static_cast<size_t>(shared_row0 + t) * d;
    for (int i = tid * 4; i < d; i += 1024) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(dyt + i);
      u32x2 pk;
      pk[0] = pack_bf16x2(a[0], a[1]);
      pk[1] = pack_bf16x2(a[2], a[3]);
      *reinterpret_cast<u32x2*>(dr + i) = pk;
    }
  }
}

// One wave per token: the logits' gradient dz[t, :] from the gates' gradient.
// SELECTED: g = softmax of the selected logits, dz_e = g_j (dg_j - sum_l g_l dg_l)
// for e = idx_j, 0 elsewhere. ALL: g_j = p_{idx_j}, dz = p (dp - sum p dp) with
// dp_e the dg of the slots that chose e. alpha > 0 adds the balance-loss term
// (alpha E / T) p_e (f_e - sum p f), f_e = counts_e / T.
__global__ __launch_bounds__(256) void gate_bwd_kernel(const float* __restrict__ z,
                                                       const int32_t* __restrict__ idx,
                                                       const float* __restrict__ gates,
                                                       const float* __restrict__ dg,
                                                       const int32_t* __restrict__ counts, int T,
                                                       int E, int k, int gate_all, float alpha,
                                                       float* __restrict__ dz) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* zt = z + static_cast<size_t>(t) * E;
  float* dzt = dz + static_cast<size_t>(t) * E;
  // slot j < k lives in lane j
  const int my_e = lane < k ? idx[static_cast<size_t>(t) * k + lane] : -1;
  const float my_g = lane < k ? gates[static_cast<size_t>(t) * k + lane] : 0.f;
  const float my_dg = lane < k ? dg[static_cast<size_t>(t) * k + lane] : 0.f;
  const bool need_p = gate_all || alpha > 0.f;
  float m = -INFINITY, se = 0.f;
  if (need_p) {
    for (int e = lane; e < E; e += 64) m = fmaxf(m, zt[e]);
    m = wave_allmax(m);
    for (int e = lane; e < E; e += 64) se += __expf(zt[e] - m);
    se = wave_allsum(se);
  }
  const float inv = need_p ? 1.0f / se : 0.f;
  const float invT = 1.0f / static_cast<float>(T);
  // wave-wide scalars: sum g dg (SELECTED), sum p dp (ALL), sum p f (balance)
  const float sgdg = wave_allsum(my_g * my_dg);
  float spdp = 0.f, spf = 0.f;
  if (need_p) {
    float a = 0.f, b = 0.f;
    for (int e = lane; e < E; e += 64) {
      const float p = __expf(zt[e] - m) * inv;
      float dp = 0.f;
      for (int j = 0; j < k; ++j) {
        const int ej = __shfl(my_e, j, 64);
        const float dgj = __shfl(my_dg, j, 64);
        if (ej == e) dp += dgj;
      }
      a += p * dp;
      b += p * static_cast<float>(counts[e]) * invT;
    }
    spdp = wave_allsum(a);
    spf = wave_allsum(b);
  }
  const float c_aux = alpha * static_cast<float>(E) * invT;
  for (int e = lane; e < E; e += 64) {
    float v = 0.f;
    float dp = 0.f, gj = 0.f, dgj_sel = 0.f;
    bool sel = false;
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(my_e, j, 64);
      const float dgj = __shfl(my_dg, j, 64);
      const float g = __shfl(my_g, j, 64);
      if (ej == e) { dp += dgj; gj = g; dgj_sel = dgj; sel = true; }
    }
    float p = 0.f;
    if (need_p) p = __expf(zt[e] - m) * inv;
    if (gate_all) v = p * (dp - spdp);
    else if (sel) v = gj * (dgj_sel - sgdg);
    if (alpha > 0.f) v += c_aux * p * (static_cast<float>(counts[e]) * invT - spf);
    dzt[e] = v;
  }
}

// One workgroup per token: dx_t = sum_j dXp[dest[t,j]] (slot order)
// + dXp[shared_row0 + t] + sum_e dz[t,e] W_r[e] (expert order), fp32.
template <typename Tw>
__global__ __launch_bounds__(256) void unpermute_dx_kernel(const float* __restrict__ dxp,
                                                           const int32_t* __restrict__ dest,
                                                           const float* __restrict__ dz,
                                                           const Tw* __restrict__ wr, int k,
                                                           int E, int d, int shared_row0,
                                                           float* __restrict__ dx) {
  const int t = blockIdx.x;
  const int32_t* dt = dest + static_cast<size_t>(t) * k;
  const float* dzt = dz + static_cast<size_t>(t) * E;
  for (int i = threadIdx.x; i < d; i += 256) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = dt[j];
      if (r >= 0) acc += dxp[static_cast<size_t>(r) * d + i];
    }
    if (shared_row0 >= 0) acc += dxp[static_cast<size_t>(shared_row0 + t) * d + i];
    float ra = 0.f;
    for (int e = 0; e < E; ++e) ra = fmaf(dzt[e], Elt<Tw>::load1(wr + static_cast<size_t>(e) * d + i), ra);
    dx[static_cast<size_t>(t) * d + i] = acc + ra;
  }
}

// dW_r[e][i] = sum_t dz[t][e] x[t][i], tokens in order.
template <typename Tx>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float* __restrict__ dz,
                                                           const Tx* __restrict__ x, int T,
                                                           int E, int d,
                                                           float* __restrict__ dwr) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (i >= d) return;
  float acc = 0.f;
  for (int t = 0; t < T; ++t)
    acc = fmaf(dz[static_cast<size_t>(t) * E + e], Elt<Tx>::load1(x + static_cast<size_t>(t) * d + i), acc);
  dwr[static_cast<size_t>(e) * d + i] = acc;
}

__global__ void single_group_offsets_kernel(int rows, int32_t* __restrict__ off) {
  if (threadIdx.x == 0) { off[0] = 0; off[1] = rows; }
}

// ---------------------------------------------------------------- launchers

static unsigned blocks_for(long long n) { return static_cast<unsigned>((n + 255) / 256); }

hipError_t launch_pad_offsets(const int32_t* offsets, int G, int32_t* poff, hipStream_t s) {
  pad_offsets_kernel<<<dim3(1), dim3(1024), 0, s>>>(offsets, G, poff);
  return hipGetLastError();
}

hipError_t launch_single_group_offsets(int rows, int32_t* off, hipStream_t s) {
  single_group_offsets_kernel<<<dim3(1), dim3(64), 0, s>>>(rows, off);
  return hipGetLastError();
}

hipError_t launch_transpose_rows(const uint16_t* in, int in_stride, const int32_t* src,
                                 int in_row0, const int32_t* offsets, const int32_t* poff, int G,
                                 int max_rows, int C, uint16_t* out, int out_stride,
                                 hipStream_t s) {
  const int chunks = (max_rows + kPadRows * G + 63) / 64;
  transpose_rows_kernel<<<dim3(chunks, C / 64), dim3(256), 0, s>>>(
      in, in_stride, src, in_row0, offsets, poff, G, C, out, out_stride);
  return hipGetLastError();
}

hipError_t launch_transpose_mat(const uint16_t* in, int B, int M, int N, uint16_t* out,
                                int out_stride, int col0, long long out_batch, hipStream_t s) {
  transpose_mat_kernel<<<dim3(N / 64, M / 64, B), dim3(256), 0, s>>>(in, M, N, out, out_stride,
                                                                     col0, out_batch);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const float* h1, const float* h3, int stride, int row0, int rows,
                             int n, uint16_t* act, hipStream_t s) {
  const long long cnt = static_cast<long long>(rows) * n;
  if (cnt == 0) return hipSuccess;
  swiglu_fwd_kernel<<<dim3(blocks_for(cnt)), dim3(256), 0, s>>>(h1, h3, stride, row0, rows, n, act);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* da, const float* h1, const float* h3, int stride,
                             int row0, int rows, int n, uint16_t* dH, hipStream_t s) {
  const long long cnt = static_cast<long long>(rows) * n;
  if (cnt == 0) return hipSuccess;
  swiglu_bwd_kernel<<<dim3(blocks_for(cnt)), dim3(256), 0, s>>>(da, h1, h3, stride, row0, rows,
                                                                n, dH);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const float* dy, const float* yp, const int32_t* dest,
                              const float* gates, int T, int k, int d, int shared_row0, float* dg,
                              uint16_t* dyp, hipStream_t s) {
  combine_bwd_kernel<<<dim3(T), dim3(256), 0, s>>>(dy, yp, dest, gates, k, d, shared_row0, dg,
                                                   dyp);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const float* z, const int32_t* idx, const float* gates, const float* dg,
                           const int32_t* counts, int T, int E, int k, int gate_all, float alpha,
                           float* dz, hipStream_t s) {
  gate_bwd_kernel<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(z, idx, gates, dg, counts, T, E, k,
                                                          gate_all, alpha, dz);
  return hipGetLastError();
}

hipError_t launch_unpermute_dx(int dtype_bf16, const float* dxp, const int32_t* dest,
                               const float* dz, const void* wr, int T, int k, int E, int d,
                               int shared_row0, float* dx, hipStream_t s) {
  if (dtype_bf16)
    unpermute_dx_kernel<uint16_t><<<dim3(T), dim3(256), 0, s>>>(
        dxp, dest, dz, static_cast<const uint16_t*>(wr), k, E, d, shared_row0, dx);
  else
    unpermute_dx_kernel<float><<<dim3(T), dim3(256), 0, s>>>(
        dxp, dest, dz, static_cast<const float*>(wr), k, E, d, shared_row0, dx);
  return hipGetLastError();
}

hipError_t launch_router_wgrad(int dtype_bf16, const float* dz, const void* x, int T, int E, int d,
                               float* dwr, hipStream_t s) {
  const dim3 grid((d + 255) / 256, E);
  if (dtype_bf16)
    router_wgrad_kernel<uint16_t><<<grid, dim3(256), 0, s>>>(dz, static_cast<const uint16_t*>(x),
                                                              T, E, d, dwr);
  else
    router_wgrad_kernel<float><<<grid, dim3(256), 0, s>>>(dz, static_cast<const float*>(x), T, E,
                                                           d, dwr);
  return hipGetLastError();
}

}  // namespace moe
