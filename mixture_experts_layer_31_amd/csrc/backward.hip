// Backward of the MoE layer: the elementwise, reduction and layout kernels.
//
// Gradients of L = sum_t <dy_t, y_t> (+ L_aux) for y_t = sum_j g_{t,j} f_{e_j}(x_t)
// (+ shared), f(x) = W2 (silu(W1 x) * (W3 x)). The top-k selection and the
// capacity drops pass no gradient; the router learns through the gates of the
// selected experts ("Week 2 Day 2: Mixture of Experts", §1.3), and the balance
// loss adds (alpha E / T) p_i (f_i - sum_j p_j f_j) to the logits' gradient
// (same notes, §3.2). The expert products are the transposed GEMMs of the
// forward ones (CMU 15-779 Lecture 21 notes, §7: dW2 = H^T dY and so on); the
// GEMMs themselves run in gemm_bf16.hip and gemm_kmajor.hip. Every reduction here sums in a fixed
// order, so the gradients are reproducible bit for bit.
#include "common.h"
#include "kernels.h"

namespace moe {

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

// Row-wise SwiGLU backward, one workgroup per row r in [row0, row0 + rows):
// da = g_r u_r (g_r = row_gate[r]; 1 when row_gate is null), dh1 = da h3 silu'(h1),
// dh3 = da silu(h1), silu'(v) = s (1 + v (1 - s)), s = 1 / (1 + e^-v); written as
// bf16 into dH[r][0..n) and dH[r][n..2n) (row stride 2 stride). u_r = dy_t W2 is the
// ungated gradient of the row's expert output, so with dg_row the gate's gradient
// <dy_t, y_perm[r]> = <act_r, u_r> comes out here too (act as stored, bf16): per
// thread in column order, then a fixed tree.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ u,
                                                         const float* __restrict__ h1,
                                                         const float* __restrict__ h3,
                                                         const uint16_t* __restrict__ act,
                                                         const float* __restrict__ row_gate,
                                                         int stride, int row0, int n,
                                                         uint16_t* __restrict__ dH,
                                                         float* __restrict__ dg_row) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const size_t r = static_cast<size_t>(row0) + blockIdx.x;
  const float g = row_gate != nullptr ? row_gate[r] : 1.0f;
  float acc = 0.f;
  for (int f = tid * 4; f < n; f += 1024) {
    const size_t o = r * stride + f;
    const f32x4 uu = *reinterpret_cast<const f32x4*>(u + o);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(h1 + o);
    const f32x4 v3 = *reinterpret_cast<const f32x4*>(h3 + o);
    float d1[4], d3[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float da = g * uu[q];
      const float sg = 1.0f / (1.0f + __expf(-v1[q]));
      d1[q] = da * v3[q] * sg * (1.0f + v1[q] * (1.0f - sg));
      d3[q] = da * v1[q] * sg;
    }
    if (dg_row != nullptr) {
      float av[4];
      Elt<uint16_t>::load4(act + o, av);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = fmaf(av[q], uu[q], acc);
    }
    uint16_t* dr = dH + r * 2 * stride + f;
    u32x2 p1, p3;
    p1[0] = pack_bf16x2(d1[0], d1[1]);
    p1[1] = pack_bf16x2(d1[2], d1[3]);
    p3[0] = pack_bf16x2(d3[0], d3[1]);
    p3[1] = pack_bf16x2(d3[2], d3[3]);
    *reinterpret_cast<u32x2*>(dr) = p1;
    *reinterpret_cast<u32x2*>(dr + n) = p3;
  }
  if (dg_row != nullptr) {
    red[tid] = acc;
    __syncthreads();
    for (int h = 128; h >= 1; h >>= 1) {
      if (tid < h) red[tid] += red[tid + h];
      __syncthreads();
    }
    if (tid == 0) dg_row[r] = red[0];
  }
}

// One workgroup per token: dyb[t] = bf16(dy_t), the operand of the activation
// gradient's GEMM; for every kept slot j, dyp[dest[t,j]] = bf16(g[t,j] dy_t), the
// operand of dW2, and row_gate[dest[t,j]] = g[t,j].
__global__ __launch_bounds__(256) void dy_rows_kernel(const float* __restrict__ dy,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ gates, int k,
                                                      int d, uint16_t* __restrict__ dyb,
                                                      uint16_t* __restrict__ dyp,
                                                      float* __restrict__ row_gate) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* dyt = dy + static_cast<size_t>(t) * d;
  const int32_t* dt = dest + static_cast<size_t>(t) * k;
  const float* gt = gates + static_cast<size_t>(t) * k;
  for (int i = tid * 4; i < d; i += 1024) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(dyt + i);
    u32x2 pk;
    pk[0] = pack_bf16x2(a[0], a[1]);
    pk[1] = pack_bf16x2(a[2], a[3]);
    *reinterpret_cast<u32x2*>(dyb + static_cast<size_t>(t) * d + i) = pk;
    for (int j = 0; j < k; ++j) {
      const int r = dt[j];
      if (r < 0) continue;
      const float g = gt[j];
      pk[0] = pack_bf16x2(g * a[0], g * a[1]);
      pk[1] = pack_bf16x2(g * a[2], g * a[3]);
      *reinterpret_cast<u32x2*>(dyp + static_cast<size_t>(r) * d + i) = pk;
    }
  }
  if (tid < k) {
    const int r = dt[tid];
    if (r >= 0) row_gate[r] = gt[tid];
  }
}

// One wave per token: the logits' gradient dz[t, :] from the gates' gradient
// dg[t,j] = dg_row[dest[t,j]] (0 for a dropped slot).
// SELECTED: g = softmax of the selected logits, dz_e = g_j (dg_j - sum_l g_l dg_l)
// for e = idx_j, 0 elsewhere. ALL: g_j = p_{idx_j}, dz = p (dp - sum p dp) with
// dp_e the dg of the slots that chose e. alpha > 0 adds the balance-loss term
// (alpha E / T) p_e (f_e - sum p f), f_e = counts_e / T.
__global__ __launch_bounds__(256) void gate_bwd_kernel(const float* __restrict__ z,
                                                       const int32_t* __restrict__ idx,
                                                       const float* __restrict__ gates,
                                                       const int32_t* __restrict__ dest,
                                                       const float* __restrict__ dg_row,
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
  const int my_r = lane < k ? dest[static_cast<size_t>(t) * k + lane] : -1;
  const float my_dg = my_r >= 0 ? dg_row[my_r] : 0.f;   // a dropped slot passes nothing
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

// dx_t = sum_j dXp[dest[t,j]] (slot order) + dXp[shared_row0 + t]
// + sum_e dz[t,e] W_r[e] (expert order), fp32. With dXp2 set, a routed row's
// dXp is the sum of two halves, dXp[r] + dXp2[r] (the W1 and W3 parts). With W_r
// null, dx holds dz W_r on entry (an MFMA product) and is read as that term. A workgroup takes TT tokens and
// 1024 columns (4 per thread), so each W_r row segment is loaded once for TT
// tokens; the TT tokens' dz rows sit in LDS. grid (d / 1024, ceil(T / TT)).
template <typename Tw, int TT>
__global__ __launch_bounds__(256) void unpermute_dx_kernel(const float* __restrict__ dxp,
                                                           const float* __restrict__ dxp2,
                                                           const int32_t* __restrict__ dest,
                                                           const float* __restrict__ dz,
                                                           const Tw* __restrict__ wr, int T,
                                                           int k, int E, int d, int shared_row0,
                                                           float* __restrict__ dx) {
  extern __shared__ float sdz[];   // [TT][E]
  const int t0 = blockIdx.y * TT;
  const int nt = min(TT, T - t0);
  if (wr != nullptr)
    for (int q = threadIdx.x; q < nt * E; q += 256) sdz[q] = dz[static_cast<size_t>(t0) * E + q];
  __syncthreads();
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= d) return;
  float acc[TT][4], ra[TT][4];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[tt][q] = ra[tt][q] = 0.f;
    if (tt < nt) {
      const int t = t0 + tt;
      for (int j = 0; j < k; ++j) {
        const int r = dest[static_cast<size_t>(t) * k + j];
        if (r < 0) continue;
        f32x4 v = *reinterpret_cast<const f32x4*>(dxp + static_cast<size_t>(r) * d + i);
        if (dxp2 != nullptr)
          v = v + *reinterpret_cast<const f32x4*>(dxp2 + static_cast<size_t>(r) * d + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[tt][q] += v[q];
      }
      if (shared_row0 >= 0) {
        const f32x4 v =
            *reinterpret_cast<const f32x4*>(dxp + static_cast<size_t>(shared_row0 + t) * d + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[tt][q] += v[q];
      }
    }
  }
  if (wr == nullptr) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (tt < nt) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(dx + static_cast<size_t>(t0 + tt) * d + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) ra[tt][q] = v[q];
      }
    }
  }
  for (int e = 0; wr != nullptr && e < E; ++e) {
    float w[4];
    Elt<Tw>::load4(wr + static_cast<size_t>(e) * d + i, w);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const float z = sdz[(tt < nt ? tt : 0) * E + e];
#pragma unroll
      for (int q = 0; q < 4; ++q) ra[tt][q] = fmaf(z, w[q], ra[tt][q]);
    }
  }
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    if (tt < nt) {
      f32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = acc[tt][q] + ra[tt][q];
      *reinterpret_cast<f32x4*>(dx + static_cast<size_t>(t0 + tt) * d + i) = o;
    }
  }
}

// dW_r[e][i] = sum_t dz[t][e] x[t][i] in two fixed-order passes. Pass 1: token
// chunks of tc tokens, part[c][e][i] = sum over the chunk's tokens in order; a
// workgroup takes 512 columns (2 per thread) and EB experts, the chunk's dz
// columns in LDS, so each x row segment is read once per EB experts.
// grid (ceil(d / 512), ceil(E / EB), chunks). Pass 2 sums the chunks in order.
template <typename Tx, int EB>
__global__ __launch_bounds__(256) void router_wgrad_part_kernel(const float* __restrict__ dz,
                                                                const Tx* __restrict__ x, int T,
                                                                int E, int d, int tc,
                                                                float* __restrict__ part) {
  extern __shared__ float sdz[];   // [tc][EB]
  const int c = blockIdx.z, e0 = blockIdx.y * EB;
  const int t0 = c * tc;
  const int nt = min(tc, T - t0);
  for (int q = threadIdx.x; q < nt * EB; q += 256) {
    const int tt = q / EB, ee = q - tt * EB;
    sdz[q] = e0 + ee < E ? dz[static_cast<size_t>(t0 + tt) * E + e0 + ee] : 0.f;
  }
  __syncthreads();
  const int i = (blockIdx.x * 256 + threadIdx.x) * 2;
  if (i >= d) return;
  float a0[EB], a1[EB];
#pragma unroll
  for (int ee = 0; ee < EB; ++ee) a0[ee] = a1[ee] = 0.f;
  for (int tt = 0; tt < nt; ++tt) {
    float xv[2];
    Elt<Tx>::load2(x + static_cast<size_t>(t0 + tt) * d + i, xv);
    const float* zr = sdz + tt * EB;
#pragma unroll
    for (int ee = 0; ee < EB; ++ee) {
      a0[ee] = fmaf(zr[ee], xv[0], a0[ee]);
      a1[ee] = fmaf(zr[ee], xv[1], a1[ee]);
    }
  }
#pragma unroll
  for (int ee = 0; ee < EB; ++ee) {
    if (e0 + ee < E) {
      float* pp = part + (static_cast<size_t>(c) * E + e0 + ee) * d + i;
      u32x2 v;
      v[0] = __float_as_uint(a0[ee]);
      v[1] = __float_as_uint(a1[ee]);
      *reinterpret_cast<u32x2*>(pp) = v;
    }
  }
}

__global__ __launch_bounds__(256) void router_wgrad_sum_kernel(const float* __restrict__ part,
                                                               int chunks, long long n,
                                                               float* __restrict__ dwr) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int c = 0; c < chunks; ++c) acc += part[static_cast<size_t>(c) * n + i];
  dwr[i] = acc;
}

// The router's gradients as MFMA products (wide routers, E a multiple of 128):
// dz (fp32 [T][E]) in two bf16 halves, dzs[t][e] = hi = bf16(dz) and
// dzs[t][E + e] = lo = bf16(dz - hi) (dz - hi is exact in fp32), so hi + lo is
// dz to within 2^-18 of |dz|; then dz W_r = [hi | lo] [W_r; W_r] and
// dz^T x = hi^T x + lo^T x with bf16 operands and fp32 sums. The same launch
// writes the token chunks of dW_r, chunk_off[c] = c T / C for c = 0..C.
__global__ __launch_bounds__(256) void dz_split_kernel(const float* __restrict__ dz, int T, int E,
                                                       int C, uint16_t* __restrict__ dzs,
                                                       int32_t* __restrict__ chunk_off) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i <= C) chunk_off[i] = static_cast<int32_t>(static_cast<long long>(i) * T / C);
  if (i >= static_cast<long long>(T) * E) return;
  const long long t = i / E, e = i - t * E;
  const float v = dz[i];
  const uint16_t hi = f32_to_bf16(v);
  dzs[t * 2 * E + e] = hi;
  dzs[t * 2 * E + E + e] = f32_to_bf16(v - bf16_to_f32(hi));
}

// dW_r[e][i] = sum over the chunks c in order of part[c][e][i] + part[c][E + e][i]
// (the hi and lo products of chunk c; part is [C][2E][d]).
__global__ __launch_bounds__(256) void router_wgrad_pairs_kernel(const float* __restrict__ part,
                                                                 int C, int E, int d,
                                                                 float* __restrict__ dwr) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const long long n = static_cast<long long>(E) * d;
  if (i >= n) return;
  float acc = 0.f;
  for (int c = 0; c < C; ++c) {
    const float* pc = part + static_cast<size_t>(c) * 2 * n;
    acc += pc[i] + pc[n + i];
  }
  dwr[i] = acc;
}

__global__ void single_group_offsets_kernel(int rows, int32_t* __restrict__ off) {
  if (threadIdx.x == 0) { off[0] = 0; off[1] = rows; }
}

// ---------------------------------------------------------------- launchers

static unsigned blocks_for(long long n) { return static_cast<unsigned>((n + 255) / 256); }

hipError_t launch_dz_split(const float* dz, int T, int E, int C, uint16_t* dzs, int32_t* chunk_off,
                           hipStream_t s) {
  const long long n = static_cast<long long>(T) * E;
  dz_split_kernel<<<dim3(blocks_for(n > C ? n : C + 1)), dim3(256), 0, s>>>(dz, T, E, C, dzs,
                                                                          chunk_off);
  return hipGetLastError();
}

hipError_t launch_router_wgrad_pairs(const float* part, int C, int E, int d, float* dwr,
                                     hipStream_t s) {
  const long long n = static_cast<long long>(E) * d;
  router_wgrad_pairs_kernel<<<dim3(blocks_for(n)), dim3(256), 0, s>>>(part, C, E, d, dwr);
  return hipGetLastError();
}

hipError_t launch_single_group_offsets(int rows, int32_t* off, hipStream_t s) {
  single_group_offsets_kernel<<<dim3(1), dim3(64), 0, s>>>(rows, off);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const float* h1, const float* h3, int stride, int row0, int rows,
                             int n, uint16_t* act, hipStream_t s) {
  const long long cnt = static_cast<long long>(rows) * n;
  if (cnt == 0) return hipSuccess;
  swiglu_fwd_kernel<<<dim3(blocks_for(cnt)), dim3(256), 0, s>>>(h1, h3, stride, row0, rows, n, act);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* u, const float* h1, const float* h3,
                             const uint16_t* act, const float* row_gate, int stride, int row0,
                             int rows, int n, uint16_t* dH, float* dg_row, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (n % 4 || stride % 4) return hipErrorInvalidValue;
  swiglu_bwd_kernel<<<dim3(rows), dim3(256), 0, s>>>(u, h1, h3, act, row_gate, stride, row0, n,
                                                     dH, dg_row);
  return hipGetLastError();
}

hipError_t launch_dy_rows(const float* dy, const int32_t* dest, const float* gates, int T, int k,
                          int d, uint16_t* dyb, uint16_t* dyp, float* row_gate, hipStream_t s) {
  if (d % 4) return hipErrorInvalidValue;
  dy_rows_kernel<<<dim3(T), dim3(256), 0, s>>>(dy, dest, gates, k, d, dyb, dyp, row_gate);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const float* z, const int32_t* idx, const float* gates,
                           const int32_t* dest, const float* dg_row, const int32_t* counts, int T,
                           int E, int k, int gate_all, float alpha, float* dz, hipStream_t s) {
  gate_bwd_kernel<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(z, idx, gates, dest, dg_row, counts, T,
                                                          E, k, gate_all, alpha, dz);
  return hipGetLastError();
}

template <typename Tw, int TT>
static void unpermute_dx_as(const float* dxp, const float* dxp2, const int32_t* dest,
                            const float* dz, const void* wr, int T, int k, int E, int d,
                            int shared_row0, float* dx, hipStream_t s) {
  const dim3 grid(d / 1024 + (d % 1024 ? 1 : 0), (T + TT - 1) / TT);
  unpermute_dx_kernel<Tw, TT><<<grid, dim3(256), TT * E * sizeof(float), s>>>(
      dxp, dxp2, dest, dz, static_cast<const Tw*>(wr), T, k, E, d, shared_row0, dx);
}

hipError_t launch_unpermute_dx(int dtype_bf16, const float* dxp, const float* dxp2,
                               const int32_t* dest, const float* dz, const void* wr, int T, int k,
                               int E, int d, int shared_row0, float* dx, hipStream_t s) {
  if (d % 4) return hipErrorInvalidValue;
  const bool wide = E > 32;   // more W_r rows per token: share each load among more tokens
  if (dtype_bf16) {
    if (wide) unpermute_dx_as<uint16_t, 16>(dxp, dxp2, dest, dz, wr, T, k, E, d, shared_row0, dx, s);
    else unpermute_dx_as<uint16_t, 8>(dxp, dxp2, dest, dz, wr, T, k, E, d, shared_row0, dx, s);
  } else {
    if (wide) unpermute_dx_as<float, 16>(dxp, dxp2, dest, dz, wr, T, k, E, d, shared_row0, dx, s);
    else unpermute_dx_as<float, 8>(dxp, dxp2, dest, dz, wr, T, k, E, d, shared_row0, dx, s);
  }
  return hipGetLastError();
}

RouterWgradPlan router_wgrad_plan(int T, int E, int d) {
  RouterWgradPlan p;
  p.eb = E <= 8 ? 8 : (E <= 16 ? 16 : 32);
  const int xy = ((d + 511) / 512) * ((E + p.eb - 1) / p.eb);
  const int want = (2048 + xy - 1) / xy;                        // about 2048 workgroups
  int tc = (T + want - 1) / want;
  tc = (tc + 15) / 16 * 16;
  p.tc = tc < 16 ? 16 : (tc > 256 ? 256 : tc);
  p.chunks = T > 0 ? (T + p.tc - 1) / p.tc : 0;
  return p;
}

template <typename Tx, int EB>
static void router_wgrad_as(const float* dz, const void* x, int T, int E, int d,
                            const RouterWgradPlan& p, float* part, hipStream_t s) {
  const dim3 grid((d + 511) / 512, (E + EB - 1) / EB, p.chunks);
  router_wgrad_part_kernel<Tx, EB><<<grid, dim3(256), p.tc * EB * sizeof(float), s>>>(
      dz, static_cast<const Tx*>(x), T, E, d, p.tc, part);
}

hipError_t launch_router_wgrad(int dtype_bf16, const float* dz, const void* x, int T, int E, int d,
                               float* part, float* dwr, hipStream_t s) {
  if (d % 2) return hipErrorInvalidValue;
  const RouterWgradPlan p = router_wgrad_plan(T, E, d);
  if (p.chunks == 0) return hipSuccess;
  if (dtype_bf16) {
    if (p.eb == 8) router_wgrad_as<uint16_t, 8>(dz, x, T, E, d, p, part, s);
    else if (p.eb == 16) router_wgrad_as<uint16_t, 16>(dz, x, T, E, d, p, part, s);
    else router_wgrad_as<uint16_t, 32>(dz, x, T, E, d, p, part, s);
  } else {
    if (p.eb == 8) router_wgrad_as<float, 8>(dz, x, T, E, d, p, part, s);
    else if (p.eb == 16) router_wgrad_as<float, 16>(dz, x, T, E, d, p, part, s);
    else router_wgrad_as<float, 32>(dz, x, T, E, d, p, part, s);
  }
  const long long n = static_cast<long long>(E) * d;
  router_wgrad_sum_kernel<<<dim3(blocks_for(n)), dim3(256), 0, s>>>(part, p.chunks, n, dwr);
  return hipGetLastError();
}

}  // namespace moe
