// Ceilings of the device, measured beside the nominal peaks the benchmark uses:
// a dense MFMA loop (the matrix cores' rate at the clock the device actually
// holds under that load) and a streaming read (HBM bandwidth a plain kernel
// reaches). Built as a separate library; nothing on the layer's path uses it.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kChains = 4;   // independent accumulators per wave: covers the MFMA latency

// iters x kChains v_mfma_f32_32x32x16_bf16 per wave (32 x 32 x 16 x 2 flop each),
// operands from registers holding pseudo-random bf16 values (random data draws the
// power, and so the clock, of real operands).
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ out) {
  uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 12345u;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h = h * 1664525u + 1013904223u;
    a[i] = static_cast<__bf16>(static_cast<float>((h >> 8) & 0xFFFF) / 65536.0f - 0.5f);
    h = h * 1664525u + 1013904223u;
    b[i] = static_cast<__bf16>(static_cast<float>((h >> 8) & 0xFFFF) / 65536.0f - 0.5f);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Grid-stride 16-byte reads of n16 16-byte words; one sum per thread is written so
// the loads are kept.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                   uint32_t* __restrict__ out) {
  uint32_t s = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = buf[i];
    s += v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Flop count of one moe_calib_mfma launch.
double moe_calib_mfma_flops(int blocks, int iters) {
  return static_cast<double>(blocks) * 4 * kChains * iters * (32.0 * 32.0 * 16.0 * 2.0);
}

// blocks workgroups of 4 waves; out: blocks * 256 floats (device). Returns a hipError_t.
int moe_calib_mfma(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return static_cast<int>(hipErrorInvalidValue);
  mfma_loop_kernel<<<dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return static_cast<int>(hipGetLastError());
}

// Reads bytes (a multiple of 16) from buf; out: blocks * 256 words (device).
int moe_calib_read(const void* buf, size_t bytes, int blocks, uint32_t* out, void* stream) {
  if (buf == nullptr || out == nullptr || bytes % 16 || blocks <= 0)
    return static_cast<int>(hipErrorInvalidValue);
  read_kernel<<<dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(buf), bytes / 16, out);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
