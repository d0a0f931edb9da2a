// One token's top-k selection and gates by one wave, shared by the selection
// kernel and the single-workgroup route + index kernel of small batches.
//
// Selection is a greedy top-k on z + b, highest first, ties to the lower expert
// index; the gates use the unbiased z ("Week 2 Day 2: Mixture of Experts",
// §1.3 and §4.2; "Mixture-of-Experts models" step 1): a softmax over the k
// selected logits, or (gate_all) the full softmax's probability of each chosen
// expert.
#pragma once
#include "common.h"

namespace moe {

// Lane l of the wave holds experts l, l + 64, ... (NE per lane).
template <int NE>
struct TokenSelect {
  float zl[NE];    // logits, -inf past E
  float ex[NE];    // e^{z - m}, 0 past E
  float m, se;     // the largest logit and the wave's sum of e^{z - m}
  int chosen[NE];  // 1 where this lane's expert was chosen
  float sl[NE];    // selection scores z + b, -inf where chosen or past E
  float kth;       // the k-th largest selection score (the last one chosen)
  int e;           // lane r < k: the r-th choice
  float g;         // lane r < k: its gate
};

// zr: the token's E logits; b: this lane's selection biases (0 when none).
// Call with all 64 lanes active; every summation order is fixed.
template <int NE>
__device__ __forceinline__ void select_token(const float* __restrict__ zr, const float (&b)[NE],
                                             int E, int k, int gate_all, int lane,
                                             TokenSelect<NE>& o) {
  float* sl = o.sl;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + 64 * i;
    o.zl[i] = e < E ? zr[e] : -INFINITY;
    sl[i] = e < E ? o.zl[i] + b[i] : -INFINITY;
    m = fmaxf(m, o.zl[i]);
    o.chosen[i] = 0;
  }
  m = wave_allmax(m);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    o.ex[i] = (lane + 64 * i < E) ? expf(o.zl[i] - m) : 0.f;
    se += o.ex[i];
  }
  se = wave_allsum(se);
  o.m = m;
  o.se = se;

  // k rounds of argmax over the keys of (z + b, e); lane r keeps the round-r
  // winner and its unbiased logit. The starting key, (-inf, INT_MAX), is what
  // every lane holds before its first candidate.
  uint64_t key[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? select_key(sl[i], e) : 0ull;
  }
  const uint64_t floor_key = select_key(-INFINITY, 0x7fffffff);
  int my_e = 0;
  float my_z = -INFINITY;
  for (int r = 0; r < k; ++r) {
    uint64_t best = floor_key;
#pragma unroll
    for (int i = 0; i < NE; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_key(best);
    const int be = static_cast<int>(~static_cast<uint32_t>(best));
    const int owner = be & 63, slot = be >> 6;
    float zsel = 0.f, ssel = 0.f;
#pragma unroll
    for (int i = 0; i < NE; ++i)
      if (i == slot) { zsel = o.zl[i]; ssel = sl[i]; }
    zsel = readlane_f(zsel, owner);
    o.kth = best == floor_key ? -INFINITY : readlane_f(ssel, owner);
    // the winner cannot win again: its score becomes -inf while at least
    // E - r - 1 >= 1 unselected experts keep finite scores
    if (lane == owner) {
#pragma unroll
      for (int i = 0; i < NE; ++i)
        if (i == slot) {
          sl[i] = -INFINITY;
          o.chosen[i] = 1;
          key[i] = select_key(-INFINITY, be);
        }
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
  o.e = my_e;
  o.g = g;
}

// The selection's margin s_(k) - s_(k+1) over the scores s = z + b (+inf when
// k = E: nothing was left out), the distance of the k-th choice from the first
// expert left out: a small margin marks a token whose choice rounding can flip.
// Call after select_token on the same TokenSelect, with all 64 lanes active.
template <int NE>
__device__ __forceinline__ float select_margin(const TokenSelect<NE>& o, int E, int k) {
  float v = -INFINITY;
#pragma unroll
  for (int i = 0; i < NE; ++i) v = fmaxf(v, o.sl[i]);
  v = wave_allmax(v);
  return k < E ? o.kth - v : INFINITY;
}

}  // namespace moe
