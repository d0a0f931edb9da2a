// Row movement: the permute gather and the unpermute/combine.
//
// The CMU 15-779 Lecture 21 notes, §3.2: after routing, tokens are permuted so
// each expert's rows are contiguous (step 2) and, after the expert compute, put
// back in token order and mixed with the gate weights (step 4):
// y_t = sum_i g_i f_i(x_t) ("Week 2 Day 2: Mixture of Experts", §1.3).
// Both kernels are HBM-bound streams of whole rows with 16-byte accesses.
#include "common.h"
#include "kernels.h"

namespace moe {

// x_perm[r] = x[src[r]] for r < offsets[E]; one workgroup per row, 16 B per lane.
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4* __restrict__ x,
                                                          const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ offsets,
                                                          int E, int row_vecs,
                                                          u32x4* __restrict__ xp) {
  const int r = blockIdx.x;
  if (r >= offsets[E]) return;
  const size_t s = static_cast<size_t>(src[r]);
  for (int v = threadIdx.x; v < row_vecs; v += 256)
    xp[static_cast<size_t>(r) * row_vecs + v] = x[s * row_vecs + v];
}

// y[t] = sum_{j: dest[t,j] >= 0} gates[t,j] * y_perm[dest[t,j]] (+ y_perm[shared_row0 + t]),
// summed in slot order. Workgroup (t, c) covers 1024 columns of token t, 4 per lane.
// KM > 0 (k <= KM): every slot's index and gate, then every slot's row, are loaded
// before the first sum, so a lane waits for two memory round trips instead of two
// per slot; the sums are the same fused multiply-adds in the same order.
template <int KM>
__global__ __launch_bounds__(256) void combine_kernel(const f32x4* __restrict__ yp,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ gates, int k,
                                                      int row_vecs, int shared_row0,
                                                      f32x4* __restrict__ y) {
  const int t = blockIdx.x;
  const int v = blockIdx.y * 256 + threadIdx.x;
  if (v >= row_vecs) return;
  const int32_t* dt = dest + static_cast<size_t>(t) * k;
  const float* gt = gates + static_cast<size_t>(t) * k;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto fma4 = [&](float g, const f32x4& a) {
    acc[0] = fmaf(g, a[0], acc[0]);
    acc[1] = fmaf(g, a[1], acc[1]);
    acc[2] = fmaf(g, a[2], acc[2]);
    acc[3] = fmaf(g, a[3], acc[3]);
  };
  f32x4 sh = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KM > 0) {
    int r[KM];
    float g[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      r[j] = j < k ? dt[j] : -1;
      g[j] = j < k ? gt[j] : 0.f;
    }
    f32x4 a[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (r[j] >= 0) a[j] = yp[static_cast<size_t>(r[j]) * row_vecs + v];
    if (shared_row0 >= 0) sh = yp[static_cast<size_t>(shared_row0 + t) * row_vecs + v];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (r[j] >= 0) fma4(g[j], a[j]);
  } else {
    for (int j = 0; j < k; ++j) {
      const int r = dt[j];
      if (r >= 0) fma4(gt[j], yp[static_cast<size_t>(r) * row_vecs + v]);
    }
    if (shared_row0 >= 0) sh = yp[static_cast<size_t>(shared_row0 + t) * row_vecs + v];
  }
  if (shared_row0 >= 0) {
    acc[0] += sh[0]; acc[1] += sh[1]; acc[2] += sh[2]; acc[3] += sh[3];
  }
  y[static_cast<size_t>(t) * row_vecs + v] = acc;
}

hipError_t launch_gather_rows(int elt_bytes, const void* x, const int32_t* src,
                              const int32_t* offsets, int E, int R_max, int d, void* x_perm,
                              hipStream_t s) {
  const int row_vecs = d * elt_bytes / 16;
  gather_rows_kernel<<<dim3(R_max), dim3(256), 0, s>>>(static_cast<const u32x4*>(x), src,
                                                       offsets, E, row_vecs,
                                                       static_cast<u32x4*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_perm, const int32_t* dest, const float* gates, int T,
                          int k, int d, int shared_row0, float* y, hipStream_t s) {
  const int row_vecs = d / 4;
  const dim3 grid(T, (row_vecs + 255) / 256);
  const f32x4* yp = reinterpret_cast<const f32x4*>(y_perm);
  f32x4* yo = reinterpret_cast<f32x4*>(y);
#define MOE_COMBINE(KM_) \
  combine_kernel<KM_><<<grid, dim3(256), 0, s>>>(yp, dest, gates, k, row_vecs, shared_row0, yo)
  if (k <= 1) MOE_COMBINE(1);
  else if (k <= 2) MOE_COMBINE(2);
  else if (k <= 4) MOE_COMBINE(4);
  else if (k <= 8) MOE_COMBINE(8);
  else MOE_COMBINE(0);
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
