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

// Where one sequence of a packed batch sits: its key tokens and key blocks, its
// query tokens, the absolute position of its first query, its query blocks (first
// absolute block, count, first packed block) and the start of its lists.  Query
// block I of a sequence has a list row of I + 1 slots, so a sequence whose query
// blocks are I0 .. I0+nq-1 takes nq(I0+1) + nq(nq-1)/2 slots.
struct SeqPos {
  int64_t tok0;   // keys
  int len;
  int64_t blk0;
  int64_t qtok0;  // queries
  int qlen;
  int qoff;       // absolute position of query 0
  int I0;         // absolute block of query 0
  int nq;         // query blocks
  int64_t qblk0;
  int64_t tri0;   // list base
};

__device__ inline int64_t tri_slots(int I0, int nq) { return (int64_t)nq * (I0 + 1) + (int64_t)nq * (nq - 1) / 2; }

// Every wave of the workgroup computes the same prefix sums over the
// sequences before s (lanes stride the sequences, then a butterfly sum), so
// no LDS or barrier is needed.  Lengths are clamped to the declared token
// extents (and query lengths to the key lengths) so malformed metadata cannot
// push addresses past the buffers.
__device__ inline SeqPos seq_pos(const SeqDesc& sd, int s) {
  SeqPos p;
  if (sd.cu_seqlens == nullptr) {
    p.tok0 = 0; p.len = sd.L; p.blk0 = 0;
    p.qtok0 = 0; p.qlen = sd.L; p.qoff = 0; p.I0 = 0; p.nq = (sd.L + kBlock - 1) / kBlock; p.qblk0 = 0;
    p.tri0 = 0;
    return p;
  }
  const bool chunked = sd.cu_seqlens_q != nullptr;
  auto lens = [&](int r, int& nk, int& nqt) {
    nk = sd.cu_seqlens[r + 1] - sd.cu_seqlens[r];
    nk = nk < 0 ? 0 : nk;
    nqt = chunked ? sd.cu_seqlens_q[r + 1] - sd.cu_seqlens_q[r] : nk;
    nqt = nqt < 0 ? 0 : (nqt > nk ? nk : nqt);
  };
  auto qblocks = [](int nk, int nqt, int& I0, int& nq) {
    const int off = nk - nqt;
    I0 = off / kBlock;
    nq = nqt > 0 ? (off + nqt - 1) / kBlock - I0 + 1 : 0;
  };
  const int lane = threadIdx.x & 63;
  int64_t b = 0, qb = 0, t = 0;
  for (int r = lane; r < s; r += 64) {
    int nk, nqt, I0, nq;
    lens(r, nk, nqt);
    qblocks(nk, nqt, I0, nq);
    b += (nk + kBlock - 1) / kBlock;
    qb += nq;
    t += tri_slots(I0, nq);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    b += __shfl_xor(b, off);
    qb += __shfl_xor(qb, off);
    t += __shfl_xor(t, off);
  }
  // the butterfly leaves every lane with the same sums: make that visible to the
  // compiler so everything derived from them lives in scalar registers
  p.blk0 = uniform64(b);
  p.qblk0 = uniform64(qb);
  p.tri0 = uniform64(t);
  int64_t t0 = sd.cu_seqlens[s];
  int64_t t1 = sd.cu_seqlens[s + 1];
  t0 = t0 < 0 ? 0 : (t0 > sd.total_tokens ? sd.total_tokens : t0);
  t1 = t1 < t0 ? t0 : (t1 > sd.total_tokens ? sd.total_tokens : t1);
  p.tok0 = uniform64(t0);
  p.len = uniform((int)(t1 - t0));
  if (!chunked) {
    p.qtok0 = p.tok0; p.qlen = p.len; p.qoff = 0; p.I0 = 0; p.nq = (p.len + kBlock - 1) / kBlock;
    return p;
  }
  int64_t u0 = sd.cu_seqlens_q[s];
  int64_t u1 = sd.cu_seqlens_q[s + 1];
  u0 = u0 < 0 ? 0 : (u0 > sd.total_qtokens ? sd.total_qtokens : u0);
  u1 = u1 < u0 ? u0 : (u1 > sd.total_qtokens ? sd.total_qtokens : u1);
  int qlen = (int)(u1 - u0);
  qlen = qlen > p.len ? p.len : qlen;
  p.qtok0 = uniform64(u0);
  p.qlen = uniform(qlen);
  p.qoff = uniform(p.len - p.qlen);
  int I0, nq;
  qblocks(p.len, p.qlen, I0, nq);
  p.I0 = uniform(I0);
  p.nq = uniform(nq);
  return p;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate (gfx9 layout) that waits until at most n vector-memory
// operations are outstanding and leaves the other counters unconstrained.
constexpr int vmcnt_le(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Buffer resource over [base, base + nbytes): loads at byte offsets past nbytes
// return zero, which zero-fills rows past a sequence end without branches.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

// Workgroup barrier that does not drain the direct-to-LDS loads in flight: only
// this wave's LDS reads/writes must be complete (lgkmcnt), the asm statements keep
// the compiler from moving memory operations across it.
__device__ inline void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(vmcnt_le(63) & ~(15 << 8));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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
