// Router scores, top-k selection and gates.
//
// z = W_r^T x ("Week 2 Day 2: Mixture of Experts", §1.3), accumulated in fp32
// (the CMU 15-779 Lecture 21 notes, §7.1: only the router function runs in
// float32). Selection is a greedy top-k on z + b, highest first, ties to the
// lower expert index; the gates use the unbiased z (CME295 notes §4.2;
// "Mixture-of-Experts models" step 1).
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"
#include "select.h"

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

// bf16 inputs: z on the matrix cores, tiled through LDS. A workgroup of four
// waves covers BT = 32 * WT tokens x BE = 32 * WE experts (WT * WE = 4); wave
// (i, j) computes one 32 x 32 block with v_mfma_f32_32x32x16_bf16 (A = token
// rows, B = router rows, 16 elements of d per instruction). d runs in steps of
// 64 elements (128 bytes of a row) through kScoreStages LDS buffers filled by
// LDS-DMA: the loads of step s + kScoreStages - 1 are in flight while step s
// feeds the MFMAs. DMA instruction j of wave w fills the 8 LDS rows
// 8 (4 j + w) .. +7 (token rows first, then router rows); lane l writes row
// + l / 8 at physical 16-byte chunk l % 8, which holds the row's logical chunk
// (l % 8) ^ (l / 8), so the fragment reads are free of bank conflicts. An
// instruction whose 8 rows all lie past T (or E) is not issued; a partly valid
// one reads the last valid row again. Either way a row past T or E only feeds
// outputs that are not written.
//
// Split s of S takes the K-steps [s * nk / S, (s + 1) * nk / S) of nk = d / 64:
// S > 1 writes its partial sums to part[s][T][E] and router_scores_reduce_kernel
// adds the splits up in a fixed order; S = 1 writes z. Either way z is bitwise
// reproducible. Products of bf16 values are exact in fp32; sums are fp32.
//
// Launch index L maps to logical = (L % 8) * ceil(n / 8) + L / 8 (n = tiles * S),
// so consecutive logical indices run on one XCD (one L2), and logical runs over
// expert tiles fastest, then splits, then token tiles: the workgroups that read
// the same token rows over the same K range share an L2.
constexpr int kScoreStages = 3;

template <int WT, int WE>
__global__ __launch_bounds__(256) void router_scores_tiled_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int d, int E,
    int n_et, int S, float* __restrict__ z, float* __restrict__ part) {
  static_assert(WT * WE == 4, "four waves");
  constexpr int BT = 32 * WT, BE = 32 * WE, ROWS = BT + BE;
  constexpr int NI = ROWS / 32;                 // DMA instructions per wave per step
  constexpr int NS = kScoreStages;
  constexpr int STAGE = ROWS * 128;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NS * STAGE];

  const int n_tt = (T + BT - 1) / BT;
  const int n = n_tt * n_et * S;
  const int per = (n + 7) >> 3;
  const int logical = static_cast<int>(blockIdx.x & 7) * per + static_cast<int>(blockIdx.x >> 3);
  if (logical >= n) return;
  const int et = logical % n_et, rest = logical / n_et;
  const int sp = rest % S, tt = rest / S;
  const int t0 = tt * BT, e0 = et * BE;
  const int nk = d >> 6;
  const int k0 = static_cast<int>(static_cast<long long>(sp) * nk / S);
  const int k1 = static_cast<int>(static_cast<long long>(sp + 1) * nk / S);
  const int nsteps = k1 - k0;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;

  const int lrow8 = lane >> 3, lchunk = (lane & 7) ^ lrow8;
  const uint16_t* g[NI];
  bool live[NI];
  int nd = 0;                                  // instructions this wave issues per step
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int r0 = 8 * (4 * j + wv), r = r0 + lrow8;
    if (r0 < BT) {
      live[j] = t0 + r0 < T;
      g[j] = x + static_cast<size_t>(min(t0 + r, T - 1)) * d + lchunk * 8;
    } else {
      live[j] = e0 + r0 - BT < E;
      g[j] = w + static_cast<size_t>(min(e0 + r - BT, E - 1)) * d + lchunk * 8;
    }
    nd += live[j] ? 1 : 0;
  }
  auto dma = [&](int step, int buf) {
    const int ko = (k0 + step) * 64;
    unsigned char* base = lds + buf * STAGE;
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if (live[j]) MOE_LDS_DMA16(g[j] + ko, base + (4 * j + wv) * 1024);
  };

  // lane l of wave (wi, wj) reads row l % 32 of its token and router blocks,
  // elements 8 (l / 32) .. +7 of each 16-element sub-step kk (chunk 2 kk + l / 32)
  const int wi = wv / WE, wj = wv % WE;
  const int fr = lane & 31, fh = lane >> 5;
  const int arow = wi * 32 + fr, brow = BT + wj * 32 + fr;
  int aoff[4], boff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    aoff[kk] = arow * 128 + (((2 * kk + fh) ^ (arow & 7)) << 4);
    boff[kk] = brow * 128 + (((2 * kk + fh) ^ (brow & 7)) << 4);
  }

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < nsteps) dma(p, p);
  int cur = 0;
  for (int i = 0; i < nsteps; ++i) {
    // loads complete in issue order: step i has landed once no more than the
    // later steps' loads (at most NS - 2 steps of nd each) are outstanding
    const int later = min(NS - 2, nsteps - 1 - i);
    wait_vmcnt_at_most<(NS - 2) * NI>(later * nd);
    dma_barrier();   // step i visible to all waves; buffer (i - 1) % NS no longer read
    if (i + NS - 1 < nsteps) dma(i + NS - 1, cur == 0 ? NS - 1 : cur - 1);
    const unsigned char* base = lds + cur * STAGE;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + aoff[kk]);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(base + boff[kk]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    cur = cur + 1 == NS ? 0 : cur + 1;
  }

  // lane l holds expert e0 + 32 wj + l % 32 of the tokens
  // t0 + 32 wi + 8 (i / 4) + 4 (l / 32) + i % 4, i = 0 .. 15
  float* out = S == 1 ? z : part + static_cast<size_t>(sp) * T * E;
  const int e = e0 + wj * 32 + fr;
  if (e < E) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + wi * 32 + 8 * (i >> 2) + 4 * fh + (i & 3);
      if (t < T) out[static_cast<size_t>(t) * E + e] = acc[i];
    }
  }
}

// bf16 inputs, at most 16 experts: z on the matrix cores with one workgroup of
// kNarrowWaves waves per 16 tokens, so every token row is read once and no split
// of d is left to add up. v_mfma_f32_16x16x32_bf16 takes A = 16 token rows and
// B = the 16 router rows, 32 elements of d per step; wave w takes the step pairs
// (2j, 2j + 1) for j = w, w + kNarrowWaves, ... in order (U steps loaded per
// batch, steps past the end read as zeros), and the waves' 16 x 16 partial sums
// are then added in wave order, so z is bitwise reproducible. Lane l loads 16
// bytes of token row l % 16 and of router row l % 16 at K-offset 8 (l / 16) of a
// step and ends holding expert l % 16 of tokens 4 (l / 16) .. +3. Token and
// expert rows past T or E read a clamped row and are not written.
constexpr int kNarrowWaves = 16;
__global__ __launch_bounds__(64 * kNarrowWaves) void router_scores_narrow_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int d, int E,
    float* __restrict__ z) {
  __shared__ f32x4 part[kNarrowWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16;
  const int r = lane & 15, q = lane >> 4;
  const uint16_t* xp = x + static_cast<size_t>(min(t0 + r, T - 1)) * d + q * 8;
  const uint16_t* wp = w + static_cast<size_t>(min(r, E - 1)) * d + q * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = d / 32;
  constexpr int U = 8, NW = kNarrowWaves;
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
  for (int w2 = 1; w2 < NW; ++w2) {
    const f32x4 o = part[w2][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] += o[i];
  }
  if (r < E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * q + i;
      if (t < T) z[static_cast<size_t>(t) * E + r] = tot[i];
    }
  }
}

// bf16 inputs, a few tokens (decode): z as dot products on the vector units, one
// workgroup per expert and group of up to TT tokens, so the router matrix is
// read by E workgroups at once with no split of d to add up afterwards. The 256
// threads split d into 16-byte chunks (chunk c to thread c % 256, at most J per
// thread, every load issued before the first product); each thread accumulates
// its chunks in order, then a wave butterfly and the four waves in order give
// the sum, so z is bitwise reproducible. Rows past T read the last token again
// and are not written.
template <int TT, int J>
__global__ __launch_bounds__(256) void router_scores_gemv_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int d, int E,
    float* __restrict__ z) {
  __shared__ float red[4][TT];
  const int e = blockIdx.x, t0 = blockIdx.y * TT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nchunk = d >> 3;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  u32x4 wc[J], xc[TT][J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = tid + 256 * j;
    wc[j] = c < nchunk ? *reinterpret_cast<const u32x4*>(w + static_cast<size_t>(e) * d + c * 8)
                       : zero4;
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const size_t t = static_cast<size_t>(min(t0 + i, T - 1));
      xc[i][j] = c < nchunk ? *reinterpret_cast<const u32x4*>(x + t * d + c * 8) : zero4;
    }
  }
  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float w0 = __uint_as_float(wc[j][q] << 16), w1 = __uint_as_float(wc[j][q] & 0xFFFF0000u);
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        acc[i] = fmaf(__uint_as_float(xc[i][j][q] << 16), w0, acc[i]);
        acc[i] = fmaf(__uint_as_float(xc[i][j][q] & 0xFFFF0000u), w1, acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = wave_allsum(acc[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < TT; ++i) red[wv][i] = acc[i];
  }
  __syncthreads();
  if (tid < TT && t0 + tid < T)
    z[static_cast<size_t>(t0 + tid) * E + e] =
        ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// z[i] = the sum of part[s][i] over the S splits (n = T * E values per split).
// A workgroup covers 256 / G outputs with G lanes each: lane j adds the splits
// j, j + G, j + 2G, ... in increasing order (four loads in flight at a time),
// and the G lane sums are then added in lane order, so the order is fixed.
template <int G>
__global__ __launch_bounds__(256) void router_scores_reduce_kernel(const float* __restrict__ part,
                                                                   int S, size_t n,
                                                                   float* __restrict__ z) {
  constexpr int NO = 256 / G;
  __shared__ float red[G][NO];
  const int io = threadIdx.x % NO, j = threadIdx.x / NO;
  const size_t i = static_cast<size_t>(blockIdx.x) * NO + io;
  float acc = 0.f;
  if (i < n) {
    int s = j;
    for (; s + 3 * G < S; s += 4 * G) {
      const float a0 = part[static_cast<size_t>(s) * n + i];
      const float a1 = part[static_cast<size_t>(s + G) * n + i];
      const float a2 = part[static_cast<size_t>(s + 2 * G) * n + i];
      const float a3 = part[static_cast<size_t>(s + 3 * G) * n + i];
      acc = (((acc + a0) + a1) + a2) + a3;
    }
    for (; s < S; s += G) acc += part[static_cast<size_t>(s) * n + i];
  }
  if constexpr (G == 1) {
    if (i < n) z[i] = acc;
  } else {
    red[j][io] = acc;
    __syncthreads();
    if (j == 0 && i < n) {
      float t = red[0][io];
#pragma unroll
      for (int q = 1; q < G; ++q) t += red[q][io];
      z[i] = t;
    }
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
    float* __restrict__ q_part, float* __restrict__ margin) {
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
    TokenSelect<NE> ts;
    select_token<NE>(z + static_cast<size_t>(t) * E, b, E, k, gate_all, lane, ts);
    if (margin != nullptr) {
      const float mg = select_margin<NE>(ts, E, k);
      if (lane == 0) margin[t] = mg;
    }
    const float m = ts.m, se = ts.se;
    const float inv = 1.0f / se;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      pacc[i] += ts.ex[i] * inv;
      cacc[i] += ts.chosen[i];
    }
    if (q_part != nullptr) {
      // scale statistics of p_t = softmax(z_t): with m the max logit and
      // se = sum e^{z-m}, log sum e^z = m + ln se, max p = 1/se,
      // entropy = ln se - sum e^{z-m} (z-m) / se, and the top-2 gap is
      // (1 - e^{z_(2) - m}) / se with z_(2) the second largest logit
      float zm = 0.f, t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        if (lane + 64 * i < E) {
          zm += ts.ex[i] * (ts.zl[i] - m);
          if (ts.zl[i] > t1) { t2 = t1; t1 = ts.zl[i]; }
          else if (ts.zl[i] > t2) { t2 = ts.zl[i]; }
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
    const int my_e = ts.e;
    const float g = ts.g;
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

// Kernel choice for bf16 scores (measured on MI355X from cold caches):
// * up to kScoreGemvTokens tokens (decode), the vector-unit kernel: one
//   launch, one workgroup per (expert, token), every load in flight at once;
// * up to 16 experts, the narrow MFMA kernel: each token row read once, one
//   launch;
// * else the MFMA tiles: 32 x 128 for T <= 32 (one token block, four expert
//   blocks), 128 x 32 for E <= 32, else 64 x 64. S splits K so that about
//   kScoreTargetGroups workgroups run, with at least two K-steps per split,
//   while the partial sums (S T E floats, written and read once more) stay
//   under half the bytes the product reads.
constexpr int kScoreGemvTokens = 8;
constexpr int kScoreGemvMaxD = 8192;
constexpr int kScoreTargetGroups = 512;

RouterScorePlan router_score_plan(int T, int d, int E) {
  RouterScorePlan p;
  if (T <= 0) return p;
  if (T <= kScoreGemvTokens && d <= kScoreGemvMaxD) {
    p.gemv = true;
    p.groups = static_cast<long long>(T) * E;
    return p;
  }
  if (E <= 16) {
    p.narrow = true;
    p.groups = (T + 15) / 16;
    return p;
  }
  p.wt = T <= 32 ? 1 : (E <= 32 ? 4 : 2);
  p.we = 4 / p.wt;
  p.n_et = (E + 32 * p.we - 1) / (32 * p.we);
  const long long tiles = static_cast<long long>((T + 32 * p.wt - 1) / (32 * p.wt)) * p.n_et;
  const long long nk = d / 64;
  long long S = (kScoreTargetGroups + tiles - 1) / tiles;
  const double in_bytes = 2.0 * (static_cast<double>(T) + E) * d;
  const long long cap = static_cast<long long>(0.5 * in_bytes / (4.0 * T * E));
  if (S > cap) S = cap;
  if (S > nk / 2) S = nk / 2;
  if (S < 1) S = 1;
  p.S = static_cast<int>(S);
  p.groups = tiles * p.S;
  return p;
}

size_t router_scores_part_floats(int dtype_bf16, int T, int d, int E) {
  if (!dtype_bf16) return 0;
  const RouterScorePlan p = router_score_plan(T, d, E);
  return p.S > 1 ? static_cast<size_t>(p.S) * T * E : 0;
}

hipError_t launch_router_scores(int dtype_bf16, const void* x, const void* w, int T, int d, int E,
                                float* z, float* part, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (!dtype_bf16) return launch_scores_t<float>(x, w, T, d, E, z, s);
  const RouterScorePlan p = router_score_plan(T, d, E);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* wp = static_cast<const uint16_t*>(w);
  if (p.gemv) {
    const dim3 grid(E, T);
    const int nchunk = d / 8;
    if (nchunk <= 256) router_scores_gemv_kernel<1, 1><<<grid, dim3(256), 0, s>>>(xp, wp, T, d, E, z);
    else if (nchunk <= 512) router_scores_gemv_kernel<1, 2><<<grid, dim3(256), 0, s>>>(xp, wp, T, d, E, z);
    else router_scores_gemv_kernel<1, 4><<<grid, dim3(256), 0, s>>>(xp, wp, T, d, E, z);
    return hipGetLastError();
  }
  if (p.narrow) {
    router_scores_narrow_kernel<<<dim3(static_cast<unsigned>(p.groups)), dim3(64 * kNarrowWaves), 0,
                                  s>>>(xp, wp, T, d, E, z);
    return hipGetLastError();
  }
  if (p.S > 1 && part == nullptr) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((p.groups + 7) / 8 * 8));
  if (p.wt == 1)
    router_scores_tiled_kernel<1, 4><<<grid, dim3(256), 0, s>>>(xp, wp, T, d, E, p.n_et, p.S, z, part);
  else if (p.wt == 4)
    router_scores_tiled_kernel<4, 1><<<grid, dim3(256), 0, s>>>(xp, wp, T, d, E, p.n_et, p.S, z, part);
  else
    router_scores_tiled_kernel<2, 2><<<grid, dim3(256), 0, s>>>(xp, wp, T, d, E, p.n_et, p.S, z, part);
  if (p.S > 1) {
    const size_t n = static_cast<size_t>(T) * E;
    auto blocks = [&](int no) { return dim3(static_cast<unsigned>((n + no - 1) / no)); };
    if (p.S <= 4) router_scores_reduce_kernel<1><<<blocks(256), dim3(256), 0, s>>>(part, p.S, n, z);
    else if (p.S <= 32) router_scores_reduce_kernel<8><<<blocks(32), dim3(256), 0, s>>>(part, p.S, n, z);
    else router_scores_reduce_kernel<32><<<blocks(8), dim3(256), 0, s>>>(part, p.S, n, z);
  }
  return hipGetLastError();
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
                                int32_t* c_part, float* q_part, float* margin, hipStream_t s) {
  const int nb = router_select_blocks(T);
  const int tpb = router_select_tokens(T);
  const size_t lds = static_cast<size_t>(8) * E * sizeof(float);
  const int ne = (E + 63) / 64;
#define MOE_SEL(NE_)                                                                       \
  router_select_kernel<NE_><<<dim3(nb), dim3(256), lds, s>>>(z, bias, T, E, k, gate_all,   \
                                                             tpb, idx,                     \
                                                             gates, p_part, c_part, q_part, \
                                                             margin)
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
