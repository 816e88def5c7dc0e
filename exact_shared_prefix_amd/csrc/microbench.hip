// Hardware micro-benchmarks used to put the attention kernels' numbers in
// context: sustained bf16 MFMA rate (32x32x16), and LDS read bandwidth for
// 16-byte reads and for 8-byte transpose reads. Not part of the attention
// path; built into a separate library (libdualkv_microbench.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

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

// 16-byte LDS reads, conflict-free (consecutive lanes, consecutive 16 B).
__global__ __launch_bounds__(256) void lds_b128_kernel(uint32_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint4 buf[4096];  // 64 KB
  for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  uint32_t acc = 0;
  int idx = threadIdx.x;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 v = buf[(idx + u * 256) & 4095];
      acc ^= v.x + v.y + v.z + v.w;
    }
    idx = (idx + 64) & 4095;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// 16-byte LDS reads with 16 independent reads in flight per lane and a 32 KB
// buffer, so four workgroups (16 waves) fit on a CU.
__global__ __launch_bounds__(256) void lds_b128_deep_kernel(uint32_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint4 buf[2048];  // 32 KB
  for (int i = threadIdx.x; i < 2048; i += 256) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  uint32_t acc = 0;
  int idx = threadIdx.x;
  for (int i = 0; i < iters / 2; ++i) {
    uint4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = buf[(idx + u * 128) & 2047];
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    idx = (idx + 64) & 2047;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// 8-byte transpose reads (ds_read_b64_tr_b16) over 4-row x 16-column tiles of
// a row-major array with a 72-dword row pitch.
__global__ __launch_bounds__(256) void lds_tr_kernel(uint32_t* out, int iters) {
  constexpr int PITCH = 144;  // bf16 elements per row
  __shared__ __attribute__((aligned(16))) short buf[128 * PITCH];
  for (int i = threadIdx.x; i < 128 * PITCH; i += 256) buf[i] = (short)i;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  uint32_t acc = 0;
  int row0 = 4 * g + 16 * w;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = (row0 + (j >> 2) + 8 * u) & 127;
      const int col = 16 * (u & 7) + 4 * (j & 3);
      v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(buf + row * PITCH + col));
      acc ^= (uint32_t)(v[0] + v[1] + v[2] + v[3]);
    }
    row0 = (row0 + 4) & 127;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// Same addresses as lds_tr_kernel but plain 8-byte reads (no transpose).
__global__ __launch_bounds__(256) void lds_b64_kernel(uint32_t* out, int iters) {
  constexpr int PITCH = 144;
  __shared__ __attribute__((aligned(16))) short buf[128 * PITCH];
  for (int i = threadIdx.x; i < 128 * PITCH; i += 256) buf[i] = (short)i;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  uint32_t acc = 0;
  int row0 = 4 * g + 16 * w;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = (row0 + (j >> 2) + 8 * u) & 127;
      const int col = 16 * (u & 7) + 4 * (j & 3);
      const uint2 v = *reinterpret_cast<const uint2*>(buf + row * PITCH + col);
      acc ^= v.x + v.y;
    }
    row0 = (row0 + 4) & 127;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// Eight independent chains, 1 wave per SIMD (launch 1 block of 256 per CU).
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

// fp32 atomic-add throughput: each wave adds 1.0 to 2 rows x 32 consecutive
// floats per instruction (the pattern of an accumulator tile in accumulator
// layout), 16 instructions per iteration, rows spread over `rows` rows of a
// 128-float pitch. Every address stays below rows * 128.
__global__ __launch_bounds__(256) void atomic_kernel(float* buf, int rows, int iters) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned r0 = (unsigned)(blockIdx.x * 4 + w) * 97u;
  for (int it = 0; it < iters; ++it) {
    const unsigned row = (r0 + (unsigned)it * 8u) % (unsigned)(rows - 32);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const unsigned rr = row + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
      unsafeAtomicAdd(buf + (size_t)rr * 128 + (lane & 31), 1.0f);
    }
  }
}

// VALU issue rate: 8 independent chains per lane of one operation, `iters`
// rounds. op 0: v_exp_f32 (transcendental unit), 1: v_fma_f32, 2: v_cvt_pk_bf16_f32.
template <int OP>
__global__ __launch_bounds__(256) void valu_rate_kernel(float* out, int iters, float seed) {
  float x[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) x[u] = seed * (float)(threadIdx.x + u) - 0.5f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (OP == 0) x[u] = __builtin_amdgcn_exp2f(-x[u]);
      else if (OP == 1) x[u] = fmaf(x[u], 0.999f, seed);
      else {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        f32x2 f = {x[u], x[(u + 1) & 7]};
        x[u] = __builtin_bit_cast(float, __builtin_convertvector(f, bf16x2));
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += x[u];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// MFMA and exp in one wave: per round four independent 32x32x16 MFMAs (if MF)
// and NEXP independent exp2 per lane (8 chains).
template <bool MF, int NEXP>
__global__ __launch_bounds__(256) void mix_kernel(float* out, int iters, float seed) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(threadIdx.x + e));
    b[e] = (__bf16)(seed * (float)(e - (int)threadIdx.x));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) x[u] = seed * (float)(threadIdx.x + u) + 0.25f;
  for (int i = 0; i < iters; ++i) {
    if (MF) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NEXP; j += 8)
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = __builtin_amdgcn_exp2f(-x[u]);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
#pragma unroll
  for (int u = 0; u < 8; ++u) s += x[u];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Dependent MFMA chains: CH independent accumulators per wave, each MFMA
// accumulating onto the previous one of its chain (as in a k-loop).
template <int CH>
__global__ __launch_bounds__(256) void mfma_chain_kernel(float* out, int iters, float seed) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(threadIdx.x + e));
    b[e] = (__bf16)(seed * (float)(e - (int)threadIdx.x));
  }
  f32x16 c[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) c[u] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 8 / CH; ++r)
#pragma unroll
      for (int u = 0; u < CH; ++u) c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[u], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < CH; ++u)
    for (int r = 0; r < 16; ++r) s += c[u][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

extern "C" {

// blocks x 256 threads x iters x 8 MFMAs in `chains` dependent chains (1, 2, 4, 8).
int dkv_mb_mfma_chain(int chains, int blocks, int iters, float* out, void* stream) {
  const dim3 g(blocks), b(256);
  hipStream_t st = (hipStream_t)stream;
  if (chains == 1) hipLaunchKernelGGL(mfma_chain_kernel<1>, g, b, 0, st, out, iters, 1e-3f);
  else if (chains == 2) hipLaunchKernelGGL(mfma_chain_kernel<2>, g, b, 0, st, out, iters, 1e-3f);
  else if (chains == 4) hipLaunchKernelGGL(mfma_chain_kernel<4>, g, b, 0, st, out, iters, 1e-3f);
  else if (chains == 8) hipLaunchKernelGGL(mfma_chain_kernel<8>, g, b, 0, st, out, iters, 1e-3f);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// VALU rate: blocks x 256 threads x iters x 8 operations of kind op (0 exp2,
// 1 fma, 2 cvt_pk_bf16).
int dkv_mb_valu(int op, int blocks, int iters, float* out, void* stream) {
  if (op == 0)
    hipLaunchKernelGGL(valu_rate_kernel<0>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 1e-3f);
  else if (op == 1)
    hipLaunchKernelGGL(valu_rate_kernel<1>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 1e-3f);
  else if (op == 2)
    hipLaunchKernelGGL(valu_rate_kernel<2>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 1e-3f);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// MFMA / exp overlap: see mix_kernel. (do_mfma, nexp): (1, 0), or nexp in {16, 32, 64}.
int dkv_mb_mix(int blocks, int iters, int do_mfma, int nexp, float* out, void* stream) {
  const dim3 g(blocks), b(256);
  hipStream_t st = (hipStream_t)stream;
#define DKV_MIX(MF, NE) \
  if (do_mfma == MF && nexp == NE) { hipLaunchKernelGGL((mix_kernel<MF, NE>), g, b, 0, st, out, iters, 1e-3f); return (int)hipGetLastError(); }
  DKV_MIX(1, 0) DKV_MIX(0, 16) DKV_MIX(1, 16) DKV_MIX(0, 32) DKV_MIX(1, 32) DKV_MIX(0, 64) DKV_MIX(1, 64)
#undef DKV_MIX
  return (int)hipErrorInvalidValue;
}

// blocks x 256 threads x iters x 16 atomic lanes into buf[rows * 128] (rows >= 64).
int dkv_mb_atomic(int blocks, int iters, float* buf, int rows, void* stream) {
  if (rows < 64) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(atomic_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, buf, rows, iters);
  return (int)hipGetLastError();
}

// Copies n16 16-byte words from src to dst (device pointers, no overlap).
int dkv_mb_copy(const void* src, void* dst, long n16, void* stream) {
  hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                     (uint4*)dst, n16);
  return (int)hipGetLastError();
}

int dkv_mb_lds_b64(int blocks, int iters, uint32_t* out, void* stream) {
  hipLaunchKernelGGL(lds_b64_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

int dkv_mb_mfma8(int blocks, int iters, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_rate8_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters,
                     1e-3f);
  return (int)hipGetLastError();
}

// Each launches `blocks` workgroups of 256 threads on `stream`; returns the
// hipError_t of the launch. FLOPs = blocks * 4 waves * iters * 4 * 32768;
// LDS bytes = blocks * 256 * iters * 8 * (16 or 8).
int dkv_mb_mfma(int blocks, int iters, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters,
                     1e-3f);
  return (int)hipGetLastError();
}

// iters / 2 rounds of 16 reads: the same byte count as dkv_mb_lds_b128.
int dkv_mb_lds_b128_deep(int blocks, int iters, uint32_t* out, void* stream) {
  hipLaunchKernelGGL(lds_b128_deep_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

int dkv_mb_lds_b128(int blocks, int iters, uint32_t* out, void* stream) {
  hipLaunchKernelGGL(lds_b128_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

int dkv_mb_lds_tr(int blocks, int iters, uint32_t* out, void* stream) {
  hipLaunchKernelGGL(lds_tr_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
