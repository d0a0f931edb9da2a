// Device-side helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// bf16 is carried as raw uint16 bit patterns in memory.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// Two fp32 -> IEEE half (round to nearest even; v_cvt_pk_f16_f32), lo in bits 0-15.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// Eight bf16 -> eight IEEE half, in place of a fragment. Exact for |v| >= 2^-17
// (bf16's 8-bit significand fits half's 11 bits down to half's subnormals of step
// 2^-24); smaller magnitudes round to that step (error <= 2^-25); |v| > 65504
// overflows (not a weight or activation magnitude this layer meets).
__device__ __forceinline__ bf16x8 bf16x8_to_f16(bf16x8 v) {
  const u32x4 u = __builtin_bit_cast(u32x4, v);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack_f16x2(__uint_as_float(u[i] << 16), __uint_as_float(u[i] & 0xFFFF0000u));
  return __builtin_bit_cast(bf16x8, r);
}

// v_mfma_f32_32x32x16 on bf16 operands, or (H16) on half operands held in the
// same 16-byte registers
template <bool H16>
__device__ __forceinline__ f32x16 mfma32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (H16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <bool H16>
__device__ __forceinline__ f32x4 mfma16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (H16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Element loaders: 8 consecutive elements widened to fp32.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static void load8(const float* p, float* out) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
    out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void load2(const float* p, float* out) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    out[0] = __uint_as_float(v[0]); out[1] = __uint_as_float(v[1]);
  }
  __device__ __forceinline__ static void load4(const float* p, float* out) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
  }
};
template <> struct Elt<uint16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static void load8(const uint16_t* p, float* out) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static float load1(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void load2(const uint16_t* p, float* out) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    out[0] = __uint_as_float(v << 16); out[1] = __uint_as_float(v & 0xFFFF0000u);
  }
  __device__ __forceinline__ static void load4(const uint16_t* p, float* out) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    out[0] = __uint_as_float(v[0] << 16); out[1] = __uint_as_float(v[0] & 0xFFFF0000u);
    out[2] = __uint_as_float(v[1] << 16); out[3] = __uint_as_float(v[1] & 0xFFFF0000u);
  }
};


// DPP lane moves within rows of 16 lanes (gfx9 encodings): the value of the
// lane the control names, with no trip through the LDS unit.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor4 = 0x124;   // rotate the 16-lane row by 4
constexpr int kDppRowRor8 = 0x128;   // rotate the 16-lane row by 8
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Wave-wide max (all 64 lanes active): within each 16-lane row by DPP (after xor 1, xor 2 and the
// row rotations by 4 and 8 every lane holds its row's max), then the four row
// maxima through scalar registers. Max is exact, so every lane ends with the
// same value whatever the pairing order.
__device__ __forceinline__ float wave_allmax(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppRowRor4>(v));
  v = fmaxf(v, dpp_f<kDppRowRor8>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
               fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// Wave-wide sum in a fixed order: each 16-lane row is summed by DPP steps
// (lane 0 of row r ends with that row's sum in one fixed association), and the
// four row sums are added in row order in scalar registers, so every lane gets
// the same, deterministic total. Call with all 64 lanes active.
__device__ __forceinline__ float wave_allsum(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppRowRor4>(v);
  v += dpp_f<kDppRowRor8>(v);
  return ((readlane_f(v, 0) + readlane_f(v, 16)) + readlane_f(v, 32)) + readlane_f(v, 48);
}

// Key of a selection candidate (score s, expert e) whose unsigned order is the
// selection order: a higher score first, equal scores (-0 equal to +0) to the
// lower expert. The high word is s's sign-magnitude bits made monotonic, the low
// word ~e; a NaN score gets key 0, below every candidate.
__device__ __forceinline__ uint64_t select_key(float s, int e) {
  if (!(s == s)) return 0ull;
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_max_key(uint64_t key) {
  const int lo = static_cast<int>(static_cast<uint32_t>(key));
  const int hi = static_cast<int>(static_cast<uint32_t>(key >> 32));
  const uint32_t olo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false));
  const uint32_t ohi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false));
  const uint64_t o = (static_cast<uint64_t>(ohi) << 32) | olo;
  return o > key ? o : key;
}

// Wave-wide maximum of a 64-bit key (all 64 lanes active), without branches:
// DPP steps give every lane its 16-lane row's maximum, row_bcast:15 (into rows 1
// and 3) and row_bcast:31 (into rows 2 and 3) carry the rows' maxima up to lane
// 63, whose key every lane gets.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t key) {
  key = dpp_max_key<kDppQuadXor1, 0xF>(key);
  key = dpp_max_key<kDppQuadXor2, 0xF>(key);
  key = dpp_max_key<kDppRowRor4, 0xF>(key);
  key = dpp_max_key<kDppRowRor8, 0xF>(key);
  key = dpp_max_key<0x142, 0xA>(key);   // row_bcast:15
  key = dpp_max_key<0x143, 0xC>(key);   // row_bcast:31
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(key)), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(key >> 32)), 63));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Inclusive prefix sum of an int over the wave's 64 lanes (all active): DPP
// row shifts by 1, 2, 4 and 8 scan each 16-lane row (a lane with no source in
// its row adds 0), then each row adds the totals of the rows before it, read
// from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Inclusive prefix sum over a workgroup of 1024 threads, in thread order: a
// wave scan, then each wave adds the totals of the waves before it (wtot: 16
// ints of LDS). *total receives the sum over all threads. Every thread of the
// workgroup must call it; it holds two barriers.
__device__ __forceinline__ int block_scan_1024(int v, int* wtot, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_inclusive_scan(v, lane);
  if (lane == 63) wtot[wv] = v;
  __syncthreads();
  int add = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int t = wtot[w];
    add += w < wv ? t : 0;
    all += t;
  }
  __syncthreads();   // wtot is free for the next call
  *total = all;
  return v + add;
}

// Largest v over a 1024-thread workgroup, returned to every thread; wtot holds
// 16 ints of LDS and is free again on return.
__device__ __forceinline__ int block_max_1024(int v, int* wtot) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, kWave));
  if (lane == 0) wtot[wv] = v;
  __syncthreads();
  int all = wtot[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) all = max(all, wtot[w]);
  __syncthreads();
  return all;
}

__device__ __forceinline__ int wave_allsum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// silu(v) = v / (1 + e^-v), the quotient through the hardware reciprocal (v_rcp_f32,
// within 1 ulp) instead of an IEEE division (about ten instructions more per
// element in the GEMM epilogues); the result is rounded to half or bf16 next, or
// carries fp32 accumulation error of the same order. Limits: v -> -inf gives -0
// (e^-v = inf, rcp(inf) = 0), v -> +inf gives v.
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

}  // namespace moe
