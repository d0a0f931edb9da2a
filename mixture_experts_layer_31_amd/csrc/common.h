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

// Wave-wide butterfly sum: every lane ends with the total; the pairing order is
// fixed, so the result is deterministic.
__device__ __forceinline__ float wave_allsum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_allmax(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ int wave_allsum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// silu(v) = v / (1 + e^-v)
__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

}  // namespace moe
