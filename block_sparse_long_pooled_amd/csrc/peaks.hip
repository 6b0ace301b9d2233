// Measured peaks of the MI355X the benchmark runs on, for the roofline fractions
// bench.py reports next to the datasheet figures.  Not part of the FlashPrefill
// ABI: built into its own small library (libfppeaks.so) by build.py.
//
//   fpk_mfma_loop   every SIMD runs one wave of back-to-back independent matrix-core
//                   products (bf16: v_mfma_f32_32x32x16_bf16, fp8:
//                   v_mfma_scale_f32_32x32x64_f8f6f4) on register operands: the
//                   instruction-issue ceiling of the matrix cores;
//   fpk_stream_read 16-byte non-temporal loads over a buffer much larger than the
//                   caches, summed so the loads cannot be dropped: the streaming HBM
//                   read ceiling;
//   fpk_read_passes ordinary 16-byte loads over the same working set several times in
//                   one launch: with a few MB per XCD it measures L2 bandwidth, with
//                   64-256 MB the Infinity Cache, beyond that HBM.
// Both enqueue on the caller's stream and allocate nothing; the caller times them.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

template <int DT>
__global__ __launch_bounds__(256, 1) void mfma_loop_kernel(float* sink, int iters, float seed) {
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
  if (DT == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(seed * (float)(threadIdx.x + e));
      b[e] = (__bf16)(seed - (float)e);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  } else {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x38383838 ^ (int)(threadIdx.x + e);
      b[e] = 0x30303030 + e;
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_passes_kernel(const u32x4* __restrict__ src, int64_t n16, int passes,
                                                          unsigned* __restrict__ sink) {
  unsigned acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int p = 0; p < passes; ++p)
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
      const u32x4 x = src[i];
      acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
    }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; practically never stores
}

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          unsigned* __restrict__ sink) {
  unsigned acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4 x = __builtin_nontemporal_load(src + i);
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; practically never stores
}

}  // namespace

extern "C" {

// Flops of one fpk_mfma_loop call (all workgroups, all iterations).
double fpk_mfma_loop_flops(int dtype, int workgroups, int iters) {
  const double per_product = dtype == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  return per_product * 4.0 /* products per iteration */ * iters * 4.0 /* waves */ * workgroups;
}

// dtype 0 bf16, 1 fp8; one 4-wave workgroup per CU (workgroups = the CU count);
// sink: device buffer of workgroups * 256 floats.
int fpk_mfma_loop(int dtype, int workgroups, int iters, float* sink, void* stream) {
  if ((dtype != 0 && dtype != 1) || workgroups < 1 || iters < 1 || sink == nullptr) return 1;
  if (dtype == 0)
    hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, sink, iters, 1.0f);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, sink, iters, 1.0f);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Reads `bytes` (a multiple of 16) from src; sink: one device word.
int fpk_stream_read(const void* src, int64_t bytes, int workgroups, unsigned* sink, void* stream) {
  if (src == nullptr || sink == nullptr || bytes <= 0 || (bytes & 15) || ((uintptr_t)src & 15) || workgroups < 1)
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Reads `bytes` (a multiple of 16) from src `passes` times in one launch; sink: one
// device word.
int fpk_read_passes(const void* src, int64_t bytes, int passes, int workgroups, unsigned* sink, void* stream) {
  if (src == nullptr || sink == nullptr || bytes <= 0 || (bytes & 15) || ((uintptr_t)src & 15) || workgroups < 1 ||
      passes < 1)
    return 1;
  hipLaunchKernelGGL(read_passes_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, passes, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
