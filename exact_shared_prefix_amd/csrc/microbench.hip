// Hardware micro-benchmarks that put the attention kernels' numbers in
// context: the sustained bf16 MFMA rate (32x32x16, register operands), and a
// plain copy kernel of known size used to scale the HBM byte counters. Not part
// of the attention path; built into a separate library
// (libdualkv_microbench.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Four independent accumulator chains per wave so MFMA issue, not the
// dependency latency, sets the rate. Operands come from registers.
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* out, int iters, float seed) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(threadIdx.x + e));
    b[e] = (__bf16)(seed * (float)(e - (int)threadIdx.x));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Eight independent chains per wave (four waves per CU).
__global__ __launch_bounds__(256) void mfma_rate8_kernel(float* out, int iters, float seed) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(threadIdx.x + e));
    b[e] = (__bf16)(seed * (float)(e - (int)threadIdx.x));
  }
  f32x16 c[8] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[u], 0, 0, 0);
  }
  float s = 0.f;
  for (int u = 0; u < 8; ++u)
    for (int r = 0; r < 16; ++r) s += c[u][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Plain copy of n16 16-byte words, grid-stride; each byte read once and
// written once. Used to scale the HBM byte counters (FETCH_SIZE, WRITE_SIZE).
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, long n16) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

extern "C" {

// Each launches `blocks` workgroups of 256 threads on `stream`; returns the
// hipError_t of the launch. FLOPs = blocks * 4 waves * iters * 4 * 32768
// (dkv_mb_mfma, four chains per wave) or * 8 * 32768 (dkv_mb_mfma8).
int dkv_mb_mfma(int blocks, int iters, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters,
                     1e-3f);
  return (int)hipGetLastError();
}

int dkv_mb_mfma8(int blocks, int iters, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_rate8_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters,
                     1e-3f);
  return (int)hipGetLastError();
}

// Copies n16 16-byte words from src to dst (device pointers, no overlap).
int dkv_mb_copy(const void* src, void* dst, long n16, void* stream) {
  hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                     (uint4*)dst, n16);
  return (int)hipGetLastError();
}

}  // extern "C"
