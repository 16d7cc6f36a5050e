// Attainable matrix-core rate on this GPU: a reference measurement, not part
// of the layer.  Every wave issues back-to-back independent
// v_mfma_f32_32x32x16_bf16 instructions on operands held in registers (no
// memory traffic), eight waves per CU as in the grouped GEMM.  What it
// reaches is the MFMA issue rate at the clock the chip sustains under that
// load, an upper bound for any kernel that also moves data.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kAcc = 8;   // independent accumulators per wave

__global__ __launch_bounds__(512) void mfma_ref_kernel(int iters, float* out) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  // operands: bit patterns that vary per lane (finite bf16 values)
  bf16x8 a[2], b[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = (tid * 2654435761u) ^ (uint32_t)(k * 8 + e) * 40503u;
      a[k][e] = __builtin_bit_cast(__bf16, (uint16_t)(0x3c00u | (h & 0x7fu)));
      b[k][e] = __builtin_bit_cast(__bf16, (uint16_t)(0x3c00u | ((h >> 8) & 0x7fu)));
    }
  f32x16 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 1], b[(j >> 1) & 1], acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  out[tid] = s;
}

// The same instruction stream on operands drawn like a layer's: token
// values N(0,1) and weight values N(0,0.02), rounded to bf16, in four
// register sets used in rotation, so consecutive instructions multiply new
// data.  The matrix cores' power depends on the operand bits, and the chip
// holds a lower clock on such data than on the operands above.
__device__ __forceinline__ uint32_t ref_mix(uint32_t h) {
  h ^= h >> 16;
  h *= 0x7feb352du;
  h ^= h >> 15;
  h *= 0x846ca68bu;
  h ^= h >> 16;
  return h;
}
// approximately standard normal: a sum of four uniforms, rescaled
__device__ __forceinline__ float ref_normal(uint32_t& s) {
  float x = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = ref_mix(s + 0x9e3779b9u);
    x += (float)(s >> 8) * (1.0f / 16777216.0f);
  }
  return (x - 2.0f) * 1.7320508f;
}
__device__ __forceinline__ __bf16 ref_bf16(float f) {
  uint32_t x = __builtin_bit_cast(uint32_t, f);
  x += 0x7fffu + ((x >> 16) & 1u);
  return __builtin_bit_cast(__bf16, (uint16_t)(x >> 16));
}
constexpr int kSets = 4;

__global__ __launch_bounds__(512) void mfma_ref_data_kernel(int iters, float* out) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t s = tid * 2654435761u + 12345u;
  bf16x8 a[kSets], b[kSets];
#pragma unroll
  for (int q = 0; q < kSets; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[q][e] = ref_bf16(ref_normal(s));
      b[q][e] = ref_bf16(0.02f * ref_normal(s));
    }
  f32x16 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
  for (int it = 0; it < iters; it += kSets) {
#pragma unroll
    for (int r = 0; r < kSets; ++r)
#pragma unroll
      for (int j = 0; j < kAcc; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + j) % kSets], b[(r + 3 * j) % kSets], acc[j],
                                                         0, 0, 0);
  }
  float t = 0.0f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) t += acc[j][v];
  out[tid] = t;
}

}  // namespace

// As moe_ref_mfma, on operands drawn like a layer's (see above); iters is
// rounded up to a multiple of 4.
extern "C" int moe_ref_mfma_data(int blocks, int iters, float* out, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_ref_data_kernel, dim3(blocks), dim3(512), 0, stream, (iters + kSets - 1) / kSets * kSets,
                     out);
  return (int)hipGetLastError();
}

// Launch `blocks` blocks of 512 threads, each wave issuing iters * 8
// matrix instructions (32768 flops each); out holds blocks * 512 floats.
// Returns the HIP error code of the launch.
extern "C" int moe_ref_mfma(int blocks, int iters, float* out, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_ref_kernel, dim3(blocks), dim3(512), 0, stream, iters, out);
  return (int)hipGetLastError();
}
