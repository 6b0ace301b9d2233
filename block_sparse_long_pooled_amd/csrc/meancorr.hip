// V2 mean correction, as a switchable assumption.  FlashPrefill V2 (abstract)
// names "a mean correction term that suppresses the approximation error" but does
// not define it.  Reading implemented here: every causal key block that the list of
// (h, i) prunes still enters the softmax, as n_j = 128 copies of its mean key kbar_j
// carrying its mean value vbar_j.  The pass runs after the sparse attention and
// folds the pruned blocks into its result:
//
//   O' = (Z O + sum_j n_j e^{s_j} vbar_j) / (Z + sum_j n_j e^{s_j}),
//   s_j = scale * q . kbar_j,  Z = e^{LSE},  LSE' = log(Z + sum_j n_j e^{s_j}).
//
// One workgroup per (query head, query block), 256 threads: two threads per query
// row, each owning 64 of the 128 dimensions.  Pruned blocks (j < i and not listed;
// the diagonal is always listed) are visited in chunks of 32 ids whose pooled
// means are staged in LDS as fp32; the running reference starts at the sparse LSE
// and is raised when a pruned block outweighs it (online softmax).
#include "fp_device.h"

namespace fp {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct MCK {
  MeanCorrLaunch a;
  int nb;
};

__global__ __launch_bounds__(kThreads) void meancorr_kernel(MCK p) {
  const MeanCorrLaunch& a = p.a;
  const int id = blockIdx.x;
  const int h = id % a.hq;
  const int i = p.nb - 1 - id / a.hq;  // longest rows first
  if (i <= 0) return;                  // block 0 has nothing below the diagonal
  const int g = h / (a.hq / a.hkv);
  const int tid = threadIdx.x;
  const int ql = tid >> 1;             // query row within the block
  const int half = tid & 1;            // dimensions 64*half .. +63
  const int64_t t = (int64_t)i * kBlock + ql;
  const bool valid = t < a.L;

  typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
  int cnt = ((cint_ptr)a.counts)[(int64_t)h * p.nb + i];
  cnt = uniform(cnt < 0 ? 0 : (cnt > i + 1 ? i + 1 : cnt));
  const cint_ptr list = (cint_ptr)(a.idx + (int64_t)h * ((int64_t)p.nb * (p.nb + 1) / 2) + (int64_t)i * (i + 1) / 2);

  // this thread's half of q (fp8: code * per-head scale)
  float q[64];
  if (valid) {
    if (a.dtype == 0) {
      const unsigned short* src = (const unsigned short*)a.q + t * a.q_st + (int64_t)h * a.q_sh + 64 * half;
#pragma unroll
      for (int e = 0; e < 64; ++e) q[e] = __uint_as_float((unsigned)src[e] << 16);
    } else {
      const unsigned char* src = (const unsigned char*)a.q + t * a.q_st + (int64_t)h * a.q_sh + 64 * half;
      const float qs = a.q_scale[h];
#pragma unroll
      for (int e = 0; e < 64; e += 4) {
        const int w4 = *(const int*)(src + e);
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w4, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w4, true);
        q[e] = lo[0] * qs; q[e + 1] = lo[1] * qs; q[e + 2] = hi[0] * qs; q[e + 3] = hi[1] * qs;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 64; ++e) q[e] = 0.0f;
  }

  float m = valid ? a.lse[(int64_t)h * a.L + t] : 0.0f;  // reference (natural log)
  float zs = 1.0f;                                        // e^{LSE - m}
  float ys = 0.0f;                                        // pruned mass, e^{-m} units
  float c[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) c[e] = 0.0f;
  const float logn = 4.852030263919617f;  // log(128): pruned blocks lie below the diagonal, all full

  __shared__ float kb[kChunk][kHeadDim];
  __shared__ float vb[kChunk][kHeadDim];
  const double* kbar = a.pooled_k + (int64_t)g * p.nb * kHeadDim;
  const double* vbar = a.pooled_v + (int64_t)g * p.nb * kHeadDim;
  int pos = 0;  // next list entry (the list is ascending)
  for (int j0 = 0; j0 < i; j0 += kChunk) {
    // kept bits of blocks j0 .. j0+31 from the ascending list (wave-uniform)
    unsigned kept = 0;
    while (pos < cnt) {
      const int j = uniform(list[pos]);
      if (j >= j0 + kChunk) break;
      if (j >= j0) kept |= 1u << (j - j0);
      ++pos;
    }
    const int nblk = min(kChunk, i - j0);
    const unsigned pruned = (nblk == 32 ? 0xffffffffu : ((1u << nblk) - 1u)) & ~kept;
    if (pruned == 0u) continue;
    __syncthreads();  // every thread is done with the previous chunk
#pragma unroll
    for (int u = 0; u < (kChunk * kHeadDim) / kThreads; ++u) {
      const int e = tid + u * kThreads;
      const int b = e / kHeadDim, dd = e % kHeadDim;
      const bool use = (pruned >> b) & 1u;
      kb[b][dd] = use ? (float)kbar[(int64_t)(j0 + b) * kHeadDim + dd] : 0.0f;
      vb[b][dd] = use ? (float)vbar[(int64_t)(j0 + b) * kHeadDim + dd] : 0.0f;
    }
    __syncthreads();
    for (int b = 0; b < nblk; ++b) {
      if (((pruned >> b) & 1u) == 0u) continue;
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 64; ++e) dot = fmaf(q[e], kb[b][64 * half + e], dot);
      dot += __shfl_xor(dot, 1);
      const float sj = dot * a.softmax_scale + logn;
      if (sj > m) {
        const float al = __builtin_amdgcn_exp2f((m - sj) * kLog2e);
        zs *= al;
        ys *= al;
#pragma unroll
        for (int e = 0; e < 64; ++e) c[e] *= al;
        m = sj;
      }
      const float w = __builtin_amdgcn_exp2f((sj - m) * kLog2e);
      ys += w;
#pragma unroll
      for (int e = 0; e < 64; ++e) c[e] = fmaf(w, vb[b][64 * half + e], c[e]);
    }
  }
  if (!valid) return;
  const float den = zs + ys;
  unsigned short* orow = (unsigned short*)a.out + t * a.o_st + (int64_t)h * a.o_sh + 64 * half;
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    const float o = __uint_as_float((unsigned)orow[e] << 16);
    const __bf16 r = (__bf16)((o * zs + c[e]) / den);
    orow[e] = __builtin_bit_cast(unsigned short, r);
  }
  if (half == 0) a.lse[(int64_t)h * a.L + t] = m + __builtin_log2f(den) * kLn2;
}

}  // namespace

hipError_t launch_meancorr(const MeanCorrLaunch& a, hipStream_t st) {
  MCK p{a, (int)((a.L + kBlock - 1) / kBlock)};
  dim3 grid((unsigned)((int64_t)a.hq * p.nb));
  hipLaunchKernelGGL(meancorr_kernel, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace fp
