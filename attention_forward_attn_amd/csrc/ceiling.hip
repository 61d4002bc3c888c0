// Achievable-ceiling diagnostics for the benchmark (not part of the attention
// path): an MFMA-only loop that measures what the 32x32x16 bf16 matrix cores
// sustain on this device, and a plain streaming copy that measures what HBM
// sustains. bench.py reports each attention kernel against the published peak
// and, as context, against these measured ceilings.
//
// Built into its own library (libattn_ceiling.so) so that the attention
// library's boundary stays the one declared in include/attn_fwd.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 waves per workgroup (two per SIMD); every wave runs `iters` rounds of
// 8 MFMAs over four independent accumulators. The result is written so the
// work cannot be removed.
__global__ void __launch_bounds__(512) mfma_loop(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16_t)(1e-3f * (float)(lane + i));
    b[i] = (bf16_t)(1e-3f * (float)(lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 512 + threadIdx.x] = r;
}

// Grid-stride copy, 16 bytes per lane per access, four independent loads in
// flight per lane, non-temporal (streaming) loads and stores.
__global__ void __launch_bounds__(256) copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i), b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride), d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Timer self-test: one wave spins until the constant 100 MHz real-time
// counter has advanced by `ticks`, so the kernel's duration is known
// independently of the event timer being checked. The wait always ends.
__global__ void __launch_bounds__(64) spin(unsigned long long ticks, unsigned long long* out) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long t = t0;
  while (t - t0 < ticks) {
    __builtin_amdgcn_s_sleep(1);
    t = __builtin_amdgcn_s_memrealtime();
  }
  if (threadIdx.x == 0) out[0] = t - t0;
}

}  // namespace

extern "C" {

// Device facts: compute units and the maximum shader clock (kHz) of the
// current device. Returns 0 or a hipError_t.
int attn_ceiling_device_info(int* cus, int* clock_khz) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev);
  return (int)e;
}

// One launch of the MFMA loop: `blocks` workgroups of 8 waves, `iters`
// rounds each (8 MFMAs of 32x32x16 bf16 = 262144 flops per wave per round).
// `out` must hold blocks * 512 floats. Asynchronous on `stream`.
int attn_ceiling_mfma(float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(512), 0, reinterpret_cast<hipStream_t>(stream), out, iters);
  return (int)hipGetLastError();
}

// One launch of the copy: `bytes` (a multiple of 16) from src to dst, both
// 16-byte aligned device buffers. Asynchronous on `stream`.
int attn_ceiling_copy(const void* src, void* dst, int64_t bytes, int blocks, void* stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy16, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return (int)hipGetLastError();
}

// Launches the timer self-test kernel for `us` microseconds (measured on the
// device's 100 MHz real-time counter); `out` (one uint64, device memory)
// receives the ticks that actually elapsed. Asynchronous on `stream`.
int attn_ceiling_spin(int us, unsigned long long* out, void* stream) {
  if (out == nullptr || us <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(spin, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), (unsigned long long)us * 100ull,
                     out);
  return (int)hipGetLastError();
}

}  // extern "C"
