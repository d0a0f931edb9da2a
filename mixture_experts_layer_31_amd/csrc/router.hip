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
// Reduce-scatter over a wave: at mask M a lane keeps the upper half of its N
// remaining values if lane & M, else the lower half, and adds its partner's
// copy of that half; once one value is left the remaining masks are plain
// butterfly sums. Lane l ends with the wave's sum of value l / (64 / N0).
template <int M, int N, int NV>
__device__ __forceinline__ void reduce_scatter(float (&v)[NV], int lane) {
  if constexpr (M >= 1) {
    if constexpr (N > 1) {
      constexpr int H = N / 2;
      const bool up = (lane & M) != 0;
#pragma unroll
      for (int q = 0; q < H; ++q) {
        const float send = up ? v[q] : v[q + H];
        const float keep = up ? v[q + H] : v[q];
        v[q] = keep + __shfl_xor(send, M, 64);
      }
      reduce_scatter<M / 2, H>(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], M, 64);
      reduce_scatter<M / 2, 1>(v, lane);
    }
  }
}

//
// A workgroup computes z for TT tokens x EC experts (TT * EC = NV values). Its
// 256 threads split d into chunks of 8 consecutive elements (chunk c handled by
// thread c % 256), so every load of a row is coalesced across the workgroup and
// the grid holds ceil(T / TT) * ceil(E / EC) workgroups. Each thread accumulates
// its chunks in order; a reduce-scatter butterfly then leaves every lane of a
// wave with the wave's sum of one value (log2(64) shuffle steps in all instead
// of NV full reductions), and the four waves' sums are added in wave order.
// Every summation order is fixed, so z is bitwise reproducible.
template <typename Tin, int TT, int EC>
__global__ __launch_bounds__(256) void router_scores_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ w, int T, int d, int E,
    float* __restrict__ z) {
  constexpr int NV = TT * EC;
  static_assert(NV >= 1 && NV <= 64 && (NV & (NV - 1)) == 0, "NV must be a power of 2 <= 64");
  constexpr int REP = 64 / NV;                 // lanes that end up holding the same value
  __shared__ float part[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_ec = (E + EC - 1) / EC;
  const int tg = blockIdx.x / n_ec, ec = blockIdx.x % n_ec;
  const int t0 = tg * TT, e0 = ec * EC;

  const Tin* xr[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) xr[i] = x + static_cast<size_t>(min(t0 + i, T - 1)) * d;
  const Tin* wr[EC];
#pragma unroll
  for (int j = 0; j < EC; ++j) wr[j] = w + static_cast<size_t>(min(e0 + j, E - 1)) * d;

  float v[NV];
#pragma unroll
  for (int q = 0; q < NV; ++q) v[q] = 0.f;
  const int nchunk = d >> 3;
  for (int c = tid; c < nchunk; c += 256) {
    float xv[TT][8];
#pragma unroll
    for (int i = 0; i < TT; ++i) Elt<Tin>::load8(xr[i] + c * 8, xv[i]);
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      float wv8[8];
      Elt<Tin>::load8(wr[j] + c * 8, wv8);
#pragma unroll
      for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) v[i * EC + j] = fmaf(xv[i][q], wv8[q], v[i * EC + j]);
    }
  }

  reduce_scatter<32, NV>(v, lane);
  part[wv][lane] = v[0];
  __syncthreads();
  if (wv == 0 && lane % REP == 0) {
    const int p = lane / REP, i = p / EC, j = p % EC;
    if (t0 + i < T && e0 + j < E)
      z[static_cast<size_t>(t0 + i) * E + e0 + j] =
          ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
  }
}

// bf16 inputs: z on the matrix cores. A workgroup covers 16 tokens x 16
// experts with v_mfma_f32_16x16x32_bf16 (A = 16 token rows, B = 16 router
// rows, both 32 elements of d per step); wave w takes the K-steps w, w+4, ...
// in order, and the four waves' 16x16 partial sums are added in wave order,
// so z is bitwise reproducible. Lane l loads 16 bytes of token row l%16 and of
// router row l%16 at K-offset 8*(l/16) of the step and ends holding expert
// l%16 of tokens 4*(l/16) .. +3. Products of bf16 values are exact in fp32;
// sums are fp32. Out-of-range tokens and experts read a clamped row and are
// not written.
constexpr int kScoreWaves = 16;
__global__ __launch_bounds__(64 * kScoreWaves) void router_scores_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int d, int E,
    float* __restrict__ z) {
  __shared__ f32x4 part[kScoreWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n_ec = (E + 15) / 16;
  const int t0 = (blockIdx.x / n_ec) * 16, e0 = (blockIdx.x % n_ec) * 16;
  const int r = lane & 15, q = lane >> 4;
  const uint16_t* xp = x + static_cast<size_t>(min(t0 + r, T - 1)) * d + q * 8;
  const uint16_t* wp = w + static_cast<size_t>(min(e0 + r, E - 1)) * d + q * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = d / 32;
  // wave w takes the step pairs (2j, 2j + 1) for j = w, w + NW, ... (a pair
  // covers 128 bytes of each row); U steps are loaded per batch, steps past the
  // end read as zeros, which add nothing
  constexpr int U = 8, NW = kScoreWaves;
  const bf16x8 zero = {};
  for (int base = 2 * wv; base < nsteps; base += NW * U) {
    bf16x8 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int stp = base + 2 * NW * (u >> 1) + (u & 1);
      const bool ok = stp < nsteps;
      a[u] = ok ? *reinterpret_cast<const bf16x8*>(xp + stp * 32) : zero;
      b[u] = ok ? *reinterpret_cast<const bf16x8*>(wp + stp * 32) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u], acc, 0, 0, 0);
  }
  part[wv][lane] = acc;
  __syncthreads();
  if (wv != 0) return;
  f32x4 tot = part[0][lane];
#pragma unroll
  for (int w2 = 1; w2 < kScoreWaves; ++w2) {
    const f32x4 o = part[w2][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] += o[i];
  }
  const int e = e0 + r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * q + i;
    if (t < T && e < E) z[static_cast<size_t>(t) * E + e] = tot[i];
  }
}

// ---------------------------------------------------------------- selection
//
// One wave per token at a time; lane l owns experts l, l+64, ... (NE per lane).
// A workgroup covers router_select_tokens(T) consecutive tokens (4 waves).
// Top-k is k rounds of a wave argmax on (score desc, index asc). The full
// softmax (for the ALL gate and for P_i) is computed on every token. Per-wave
// sums of p_{t,e} and of the selection counts run in token order and are then
// combined across the block's waves in wave order, so the partial sums written
// per block are deterministic.
template <int NE>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ z, const float* __restrict__ bias, int T, int E, int k,
    int gate_all, int tokens_per_block, int32_t* __restrict__ idx,
    float* __restrict__ gates, float* __restrict__ p_part, int32_t* __restrict__ c_part,
    float* __restrict__ q_part) {
  extern __shared__ unsigned char smem_raw[];
  __shared__ float sq[4][kScaleStats];
  float* sp = reinterpret_cast<float*>(smem_raw);             // [4][E]
  int32_t* sc = reinterpret_cast<int32_t*>(sp + 4 * E);        // [4][E]
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int tb0 = blockIdx.x * tokens_per_block;
  const int tb1 = min(T, tb0 + tokens_per_block);

  float b[NE], pacc[NE];
  int cacc[NE];
  float qacc[kScaleStats] = {0.f, 0.f, 0.f, 0.f};
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
    if (q_part != nullptr) {
      // scale statistics of p_t = softmax(z_t): with m the max logit and
      // se = sum e^{z-m}, log sum e^z = m + ln se, max p = 1/se,
      // entropy = ln se - sum e^{z-m} (z-m) / se, and the top-2 gap is
      // (1 - e^{z_(2) - m}) / se with z_(2) the second largest logit
      float zm = 0.f, t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        if (lane + 64 * i < E) {
          zm += ex[i] * (zl[i] - m);
          if (zl[i] > t1) { t2 = t1; t1 = zl[i]; }
          else if (zl[i] > t2) { t2 = zl[i]; }
        }
      }
      zm = wave_allsum(zm);
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) {
        const float o1 = __shfl_xor(t1, msk, 64), o2 = __shfl_xor(t2, msk, 64);
        const float n2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
        t1 = fmaxf(t1, o1);
        t2 = n2;
      }
      const float lse = m + logf(se);
      qacc[0] += lse * lse;
      qacc[1] += logf(se) - zm * inv;
      qacc[2] += inv;
      qacc[3] += (1.0f - expf(t2 - m)) * inv;
    }

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
  if (q_part != nullptr && lane == 0) {
#pragma unroll
    for (int q = 0; q < kScaleStats; ++q) sq[wv][q] = qacc[q];
  }
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
  if (q_part != nullptr && threadIdx.x < kScaleStats) {
    const int q = threadIdx.x;
    q_part[static_cast<size_t>(blockIdx.x) * kScaleStats + q] =
        ((sq[0][q] + sq[1][q]) + sq[2][q]) + sq[3][q];
  }
}

// f_i and P_i (CME295 notes §3.2): workgroup e sums column e of the per-block
// partials, thread j taking blocks j, j + 256, ... in order and a fixed tree
// adding the 256 thread sums, so the result does not depend on scheduling.
// fp[e] = f_e * P_e feeds the balance loss.
__global__ __launch_bounds__(256) void router_stats_kernel(
    const float* __restrict__ p_part, const int32_t* __restrict__ c_part, int nblocks,
    int T, int E, float* __restrict__ f_out, float* __restrict__ P_out,
    float* __restrict__ fp) {
  __shared__ float rp[256];
  __shared__ int rc[256];
  const int e = blockIdx.x;
  float p = 0.f;
  int c = 0;
  for (int b = threadIdx.x; b < nblocks; b += 256) {
    p += p_part[static_cast<size_t>(b) * E + e];
    c += c_part[static_cast<size_t>(b) * E + e];
  }
  rp[threadIdx.x] = p;
  rc[threadIdx.x] = c;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (threadIdx.x < h) {
      rp[threadIdx.x] += rp[threadIdx.x + h];
      rc[threadIdx.x] += rc[threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float invT = 1.0f / static_cast<float>(T);
    const float P = rp[0] * invT, f = static_cast<float>(rc[0]) * invT;
    if (P_out) P_out[e] = P;
    if (f_out) f_out[e] = f;
    fp[e] = f * P;
  }
}

// L_aux = alpha * E * sum_i f_i P_i (CME295 notes §3.2) and the token means of
// the scale statistics (z-loss, entropy, top probability, top-2 gap) from the
// per-block partials; every sum in a fixed order.
__device__ __forceinline__ float block_sum_fixed(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void router_aux_kernel(
    const float* __restrict__ fp, int E, float alpha, float* __restrict__ aux,
    const float* __restrict__ q_part, int nblocks, int T, float* __restrict__ z_loss,
    float* __restrict__ entropy, float* __restrict__ max_prob, float* __restrict__ top_gap) {
  __shared__ float red[256];
  float local = 0.f;
  for (int e = threadIdx.x; e < E; e += 256) local += fp[e];
  const float s = block_sum_fixed(local, red);
  if (threadIdx.x == 0 && aux) aux[0] = alpha * static_cast<float>(E) * s;
  if (q_part == nullptr) return;
  float* outs[kScaleStats] = {z_loss, entropy, max_prob, top_gap};
  const float invT = 1.0f / static_cast<float>(T);
  for (int q = 0; q < kScaleStats; ++q) {
    float acc = 0.f;
    for (int b = threadIdx.x; b < nblocks; b += 256) acc += q_part[static_cast<size_t>(b) * kScaleStats + q];
    const float tot = block_sum_fixed(acc, red);
    if (threadIdx.x == 0 && outs[q]) outs[q][0] = tot * invT;
  }
}

// Auxiliary-loss-free balancing (CME295 notes §4.2; CMU 15-779 notes §2.4):
// bias[e] moves by -gamma above the mean load T*k/E, +gamma below, 0 at it.
// With ep > 1 simulated expert-parallel ranks the counts are per row group
// (r*ep + s)*El + l; expert e = r*El + l sums its ep groups, in source order.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                          long long Tk, int E, int ep,
                                                          float gamma,
                                                          float* __restrict__ bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  long long ce = counts[e];
  if (ep > 1) {
    const int El = E / ep, r = e / El, l = e % El;
    ce = 0;
    for (int src = 0; src < ep; ++src) ce += counts[(r * ep + src) * El + l];
  }
  const long long c = ce * E;
  if (c > Tk) bias[e] -= gamma;
  else if (c < Tk) bias[e] += gamma;
}

// ---------------------------------------------------------------- launchers

template <typename Tin>
static hipError_t launch_scores_t(const void* x, const void* w, int T, int d, int E, float* z,
                                  hipStream_t s) {
  const Tin* xp = static_cast<const Tin*>(x);
  const Tin* wp = static_cast<const Tin*>(w);
  constexpr int EC = 8;
  const long n_ec = (E + EC - 1) / EC;
  if (T >= 8) {
    constexpr int TT = 8;
    const long blocks = static_cast<long>((T + TT - 1) / TT) * n_ec;
    router_scores_kernel<Tin, TT, EC><<<dim3(blocks), dim3(256), 0, s>>>(xp, wp, T, d, E, z);
  } else {
    const long blocks = static_cast<long>(T) * n_ec;
    router_scores_kernel<Tin, 1, EC><<<dim3(blocks), dim3(256), 0, s>>>(xp, wp, T, d, E, z);
  }
  return hipGetLastError();
}

hipError_t launch_router_scores(int dtype_bf16, const void* x, const void* w, int T, int d, int E,
                                float* z, hipStream_t s) {
  if (dtype_bf16) {
    const long blocks = static_cast<long>((T + 15) / 16) * ((E + 15) / 16);
    router_scores_mfma_kernel<<<dim3(blocks), dim3(64 * kScoreWaves), 0, s>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), T, d, E, z);
    return hipGetLastError();
  }
  return launch_scores_t<float>(x, w, T, d, E, z, s);
}

// 4 tokens per workgroup (one per wave) while that keeps the grid at <= 1024
// workgroups, else a multiple of 4 that does
int router_select_tokens(int T) {
  const int per_wave = (((T + 3) / 4) + kSelectMaxBlocks - 1) / kSelectMaxBlocks;
  return 4 * (per_wave > 1 ? per_wave : 1);
}

int router_select_blocks(int T) {
  const int tpb = router_select_tokens(T);
  return (T + tpb - 1) / tpb;
}

hipError_t launch_router_select(const float* z, const float* bias, int T, int E, int k,
                                int gate_all, int32_t* idx, float* gates, float* p_part,
                                int32_t* c_part, float* q_part, hipStream_t s) {
  const int nb = router_select_blocks(T);
  const int tpb = router_select_tokens(T);
  const size_t lds = static_cast<size_t>(8) * E * sizeof(float);
  const int ne = (E + 63) / 64;
#define MOE_SEL(NE_)                                                                       \
  router_select_kernel<NE_><<<dim3(nb), dim3(256), lds, s>>>(z, bias, T, E, k, gate_all,   \
                                                             tpb, idx,                     \
                                                             gates, p_part, c_part, q_part)
  if (ne <= 1) MOE_SEL(1);
  else if (ne <= 2) MOE_SEL(2);
  else if (ne <= 4) MOE_SEL(4);
  else MOE_SEL(16);
#undef MOE_SEL
  return hipGetLastError();
}

hipError_t launch_router_stats(const float* p_part, const int32_t* c_part, const float* q_part,
                               int nblocks, int T, int E, float alpha, float* f, float* P,
                               float* aux, float* fp, float* z_loss, float* entropy,
                               float* max_prob, float* top_gap, hipStream_t s) {
  router_stats_kernel<<<dim3(E), dim3(256), 0, s>>>(p_part, c_part, nblocks, T, E, f, P, fp);
  router_aux_kernel<<<dim3(1), dim3(256), 0, s>>>(fp, E, alpha, aux, q_part, nblocks, T, z_loss,
                                                  entropy, max_prob, top_gap);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, int T, int k, int E, int ep, float gamma,
                              float* bias, hipStream_t s) {
  bias_update_kernel<<<dim3((E + 255) / 256), dim3(256), 0, s>>>(
      counts, static_cast<long long>(T) * k, E, ep, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe
