// Device-side helpers shared by the gfx950 kernels: vector types, sequence
// bookkeeping for packed batches, and small lane utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "fp_internal.h"

namespace fp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uniform64(int64_t x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(uint64_t)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Where one sequence of a packed batch starts: its first token, its first
// packed block id and the start of its lists in the triangular-packed idx.
struct SeqPos {
  int64_t tok0;
  int len;
  int64_t blk0;
  int64_t tri0;
};

// Every wave of the workgroup computes the same prefix sums over the
// sequences before s (lanes stride the sequences, then a butterfly sum), so
// no LDS or barrier is needed.  Lengths are clamped to the declared token
// extent so malformed metadata cannot push addresses past the buffers.
__device__ inline SeqPos seq_pos(const SeqDesc& sd, int s) {
  SeqPos p;
  if (sd.cu_seqlens == nullptr) {
    p.tok0 = 0; p.len = sd.L; p.blk0 = 0; p.tri0 = 0;
    return p;
  }
  const int lane = threadIdx.x & 63;
  int64_t b = 0, t = 0;
  for (int r = lane; r < s; r += 64) {
    int n = sd.cu_seqlens[r + 1] - sd.cu_seqlens[r];
    n = n < 0 ? 0 : n;
    const int64_t nb = (n + kBlock - 1) / kBlock;
    b += nb;
    t += nb * (nb + 1) / 2;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    b += __shfl_xor(b, off);
    t += __shfl_xor(t, off);
  }
  // the butterfly leaves every lane with the same sums: make that visible to the
  // compiler so everything derived from them lives in scalar registers
  b = uniform64(b);
  t = uniform64(t);
  int64_t t0 = sd.cu_seqlens[s];
  int64_t t1 = sd.cu_seqlens[s + 1];
  t0 = t0 < 0 ? 0 : (t0 > sd.total_tokens ? sd.total_tokens : t0);
  t1 = t1 < t0 ? t0 : (t1 > sd.total_tokens ? sd.total_tokens : t1);
  p.tok0 = uniform64(t0);
  p.len = uniform((int)(t1 - t0));
  p.blk0 = b;
  p.tri0 = t;
  return p;
}

// Value of the partner lane l ^ 32 (v_permlane32_swap returns the pair
// {own, partner} in an order that depends on the half, so callers only use
// symmetric combinations of the two).
__device__ inline float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace fp
