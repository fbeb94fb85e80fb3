// Ceilings of the GPU the library runs on, measured by bench.py next to the published peaks:
// a streaming read of device memory (16-byte loads, several in flight per lane), a streaming
// copy (the same loads, each word stored to a second buffer) and loops of
// independent bf16 MFMA products (v_mfma_f32_16x16x32_bf16, the instruction of the attention
// and linear kernels, and v_mfma_f32_32x32x16_bf16). Built as libsala_peaks.so, separate from libsala; not part of its ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// grid-stride read of n16 16-byte words; each lane keeps 4 loads in flight. The xor of the
// words is written once per thread (it keeps the loads live; the values are not used).
__global__ void __launch_bounds__(256) read_kernel(const uint4* __restrict__ src, long n16, uint32_t* __restrict__ sink) {
  const long stride = (long)gridDim.x * 256;
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(long)blockIdx.x * 256 + threadIdx.x] = acc;
}

// grid-stride copy of n16 16-byte words, 4 loads in flight per lane before their stores
__global__ void __launch_bounds__(256) copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, long n16) {
  const long stride = (long)gridDim.x * 256;
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// 8 independent accumulators per wave, `iters` rounds of 8 products each
__global__ void __launch_bounds__(256) mfma_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (lane + e));
    b[e] = (__bf16)(0.002f * (lane - e));
  }
  f32x4 c[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) c[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int x = 0; x < 8; ++x) c[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[x], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x) s += c[x][0] + c[x][1] + c[x][2] + c[x][3];
  sink[(long)blockIdx.x * 256 + threadIdx.x] = s;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// the same with v_mfma_f32_32x32x16_bf16 (32,768 flops each): 4 independent accumulators of 16
// floats per wave
__global__ void __launch_bounds__(256) mfma32_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (lane + e));
    b[e] = (__bf16)(0.002f * (lane - e));
  }
  f32x16 c[4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[x][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int x = 0; x < 4; ++x) c[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[x], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[x][e];
  sink[(long)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Stream `bytes` (a multiple of 16, 16-byte aligned) from src; sink holds wgs * 256 uint32.
int sala_peak_read(const void* src, size_t bytes, void* sink, int wgs, void* stream) {
  if (!src || !sink || wgs < 1 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15)) return 2;
  hipLaunchKernelGGL(read_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, (long)(bytes / 16),
                     (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Copy `bytes` (a multiple of 16; both buffers 16-byte aligned, not overlapping) from src to dst.
int sala_peak_copy(const void* src, void* dst, size_t bytes, int wgs, void* stream) {
  if (!src || !dst || wgs < 1 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (reinterpret_cast<uintptr_t>(dst) & 15))
    return 2;
  hipLaunchKernelGGL(copy_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, (uint4*)dst,
                     (long)(bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// wgs workgroups of 4 waves, each wave 8 * iters MFMA 16x16x32 bf16 products (16,384 flops
// each); sink holds wgs * 256 floats.
int sala_peak_mfma(void* sink, int iters, int wgs, void* stream) {
  if (!sink || wgs < 1 || iters < 1) return 2;
  hipLaunchKernelGGL(mfma_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream, (float*)sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// wgs workgroups of 4 waves, each wave 4 * iters MFMA 32x32x16 bf16 products (32,768 flops
// each); sink holds wgs * 256 floats.
int sala_peak_mfma32(void* sink, int iters, int wgs, void* stream) {
  if (!sink || wgs < 1 || iters < 1) return 2;
  hipLaunchKernelGGL(mfma32_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream, (float*)sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
