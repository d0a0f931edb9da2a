// Router scores, top-k selection and gates.
//
// z = W_r^T x ("Week 2 Day 2: Mixture of Experts", §1.3), accumulated in fp32
// (the CMU 15-779 Lecture 21 notes, §7.1: only the router function runs in
// float32). Selection is a greedy top-k on z + b, highest first, ties to the
// lower expert index; the gates use the unbiased z (CME295 notes §4.2;
// "Mixture-of-Experts models" step 1).
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------- scores
//
// One wave computes z for TT tokens x EC experts. Lanes split d into chunks of 8
// consecutive elements (chunk c handled by lane c % 64), so the loads of one
// row are coalesced across the wave; each lane accumulates its chunks in order
// and a fixed butterfly sums the 64 lane partials. The tree keeps the fp32
// rounding error of z near log2(64) roundings of the total instead of d/8.
template <typename Tin, int TT, int EC>
__global__ __launch_bounds__(256) void router_scores_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ w, int T, int d, int E,
    float* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_ec = (E + EC - 1) / EC;
  const int n_tg = (T + TT - 1) / TT;
  if (wave >= n_ec * n_tg) return;
  const int tg = wave / n_ec, ec = wave % n_ec;
  const int t0 = tg * TT, e0 = ec * EC;

  const Tin* xr[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) xr[i] = x + static_cast<size_t>(min(t0 + i, T - 1)) * d;
  const Tin* wr[EC];
#pragma unroll
  for (int j = 0; j < EC; ++j) wr[j] = w + static_cast<size_t>(min(e0 + j, E - 1)) * d;

  float acc[TT][EC];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < EC; ++j) acc[i][j] = 0.f;

  const int nchunk = d >> 3;
  for (int c = lane; c < nchunk; c += 64) {
    float xv[TT][8];
#pragma unroll
    for (int i = 0; i < TT; ++i) Elt<Tin>::load8(xr[i] + c * 8, xv[i]);
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      float wv[8];
      Elt<Tin>::load8(wr[j] + c * 8, wv);
#pragma unroll
      for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][j] = fmaf(xv[i][q], wv[q], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const float s = wave_allsum(acc[i][j]);
      const int p = i * EC + j;
      if ((p & 63) == lane && t0 + i < T && e0 + j < E)
        z[static_cast<size_t>(t0 + i) * E + e0 + j] = s;
    }
}

// ---------------------------------------------------------------- selection
//
// One wave per token at a time; lane l owns experts l, l+64, ... (NE per lane).
// Top-k is k rounds of a wave argmax on (score desc, index asc). The full
// softmax (for the ALL gate and for P_i) is computed on every token. Per-wave
// sums of p_{t,e} and of the selection counts run in token order and are then
// combined across the block's waves in wave order, so the partial sums written
// per block are deterministic.
template <int NE>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ z, const float* __restrict__ bias, int T, int E, int k,
    int gate_all, int tokens_per_block, int32_t* __restrict__ idx,
    float* __restrict__ gates, float* __restrict__ p_part, int32_t* __restrict__ c_part) {
  extern __shared__ unsigned char smem_raw[];
  float* sp = reinterpret_cast<float*>(smem_raw);             // [4][E]
  int32_t* sc = reinterpret_cast<int32_t*>(sp + 4 * E);        // [4][E]
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int tb0 = blockIdx.x * tokens_per_block;
  const int tb1 = min(T, tb0 + tokens_per_block);

  float b[NE], pacc[NE];
  int cacc[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + 64 * i;
    b[i] = (bias != nullptr && e < E) ? bias[e] : 0.f;
    pacc[i] = 0.f;
    cacc[i] = 0;
  }

  for (int t = tb0 + wv; t < tb1; t += 4) {
    const float* zr = z + static_cast<size_t>(t) * E;
    float zl[NE], sl[NE];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = lane + 64 * i;
      zl[i] = e < E ? zr[e] : -INFINITY;
      sl[i] = e < E ? zl[i] + b[i] : -INFINITY;
      m = fmaxf(m, zl[i]);
    }
    m = wave_allmax(m);
    float ex[NE];
    float se = 0.f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      ex[i] = (lane + 64 * i < E) ? expf(zl[i] - m) : 0.f;
      se += ex[i];
    }
    se = wave_allsum(se);
    const float inv = 1.0f / se;
#pragma unroll
    for (int i = 0; i < NE; ++i) pacc[i] += ex[i] * inv;

    // k rounds of argmax; lane r keeps the round-r winner and its unbiased logit
    int my_e = 0;
    float my_z = -INFINITY;
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const int e = lane + 64 * i;
        if (e < E && (sl[i] > bv || (sl[i] == bv && e < be))) { bv = sl[i]; be = e; }
      }
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) {
        const float ov = __shfl_xor(bv, msk, 64);
        const int oe = __shfl_xor(be, msk, 64);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      const int owner = be & 63, slot = be >> 6;
      float zsel = 0.f;
#pragma unroll
      for (int i = 0; i < NE; ++i)
        if (i == slot) zsel = zl[i];
      zsel = __shfl(zsel, owner, 64);
      // the winner cannot win again: its score becomes -inf while at least
      // E - r - 1 >= 1 unselected experts keep finite scores
      if (lane == owner) {
#pragma unroll
        for (int i = 0; i < NE; ++i)
          if (i == slot) { sl[i] = -INFINITY; cacc[i] += 1; }
      }
      if (lane == r) { my_e = be; my_z = zsel; }
    }
    // gates from the unbiased logits
    float g;
    if (gate_all) {
      g = expf(my_z - m) / se;
    } else {
      const float ms = wave_allmax(lane < k ? my_z : -INFINITY);
      const float num = lane < k ? expf(my_z - ms) : 0.f;
      g = num / wave_allsum(num);
    }
    if (lane < k) {
      idx[static_cast<size_t>(t) * k + lane] = my_e;
      gates[static_cast<size_t>(t) * k + lane] = g;
    }
  }

  if (p_part == nullptr) return;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + 64 * i;
    if (e < E) { sp[wv * E + e] = pacc[i]; sc[wv * E + e] = cacc[i]; }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float p = sp[e];
    int c = sc[e];
    for (int w2 = 1; w2 < 4; ++w2) { p += sp[w2 * E + e]; c += sc[w2 * E + e]; }
    p_part[static_cast<size_t>(blockIdx.x) * E + e] = p;
    c_part[static_cast<size_t>(blockIdx.x) * E + e] = c;
  }
}

// Sum the per-block partials in block order and form f, P and the balance loss
// L_aux = alpha * E * sum_i f_i P_i (CME295 notes §3.2).
__global__ __launch_bounds__(256) void router_stats_kernel(
    const float* __restrict__ p_part, const int32_t* __restrict__ c_part, int nblocks,
    int T, int E, float alpha, float* __restrict__ f_out, float* __restrict__ P_out,
    float* __restrict__ aux_out) {
  __shared__ float red[256];
  float local = 0.f;
  const float invT = 1.0f / static_cast<float>(T);
  for (int e = threadIdx.x; e < E; e += 256) {
    float p = 0.f;
    int c = 0;
    for (int b = 0; b < nblocks; ++b) {
      p += p_part[static_cast<size_t>(b) * E + e];
      c += c_part[static_cast<size_t>(b) * E + e];
    }
    const float P = p * invT, f = static_cast<float>(c) * invT;
    if (P_out) P_out[e] = P;
    if (f_out) f_out[e] = f;
    local += f * P;
  }
  red[threadIdx.x] = local;
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0 && aux_out) aux_out[0] = alpha * static_cast<float>(E) * red[0];
}

// ---------------------------------------------------------------- launchers

template <typename Tin>
static hipError_t launch_scores_t(const void* x, const void* w, int T, int d, int E, float* z,
                                  hipStream_t s) {
  const Tin* xp = static_cast<const Tin*>(x);
  const Tin* wp = static_cast<const Tin*>(w);
  if (T >= 8) {
    constexpr int TT = 8, EC = 8;
    const long items = static_cast<long>((T + TT - 1) / TT) * ((E + EC - 1) / EC);
    router_scores_kernel<Tin, TT, EC><<<dim3((items + 3) / 4), dim3(256), 0, s>>>(xp, wp, T, d, E, z);
  } else {
    // few tokens: one wave per (token, expert) so the router rows stream in parallel
    constexpr int TT = 1, EC = 1;
    const long items = static_cast<long>(T) * ((E + EC - 1) / EC);
    router_scores_kernel<Tin, TT, EC><<<dim3((items + 3) / 4), dim3(256), 0, s>>>(xp, wp, T, d, E, z);
  }
  return hipGetLastError();
}

hipError_t launch_router_scores(int dtype_bf16, const void* x, const void* w, int T, int d, int E,
                                float* z, hipStream_t s) {
  return dtype_bf16 ? launch_scores_t<uint16_t>(x, w, T, d, E, z, s)
                    : launch_scores_t<float>(x, w, T, d, E, z, s);
}

int router_select_blocks(int T) { return (T + kSelectTokensPerBlock - 1) / kSelectTokensPerBlock; }

hipError_t launch_router_select(const float* z, const float* bias, int T, int E, int k,
                                int gate_all, int32_t* idx, float* gates, float* p_part,
                                int32_t* c_part, hipStream_t s) {
  const int nb = router_select_blocks(T);
  const size_t lds = static_cast<size_t>(8) * E * sizeof(float);
  const int ne = (E + 63) / 64;
#define MOE_SEL(NE_)                                                                       \
  router_select_kernel<NE_><<<dim3(nb), dim3(256), lds, s>>>(z, bias, T, E, k, gate_all,   \
                                                             kSelectTokensPerBlock, idx,   \
                                                             gates, p_part, c_part)
  if (ne <= 1) MOE_SEL(1);
  else if (ne <= 2) MOE_SEL(2);
  else if (ne <= 4) MOE_SEL(4);
  else MOE_SEL(16);
#undef MOE_SEL
  return hipGetLastError();
}

hipError_t launch_router_stats(const float* p_part, const int32_t* c_part, int nblocks, int T,
                               int E, float alpha, float* f, float* P, float* aux,
                               hipStream_t s) {
  router_stats_kernel<<<dim3(1), dim3(256), 0, s>>>(p_part, c_part, nblocks, T, E, alpha, f, P,
                                                   aux);
  return hipGetLastError();
}

}  // namespace moe
