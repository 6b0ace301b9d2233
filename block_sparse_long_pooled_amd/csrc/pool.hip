// Block mean pooling of Q and K (FlashPrefill, Method 1 "Instantaneous
// Pattern Discovery": each block of B tokens is represented by its mean
// vector, so the block-score map moves (L/B)^2 data instead of L*L/B).
//
// HBM-streaming kernel.  One workgroup owns one (sequence, block, group of
// 4 heads).  For token-major data the 4 heads of one token are one
// contiguous 1 KB run (bf16), so each wave reads whole 1 KB rows with 16-byte
// loads; 4 rows are in flight per pass and the pass loop is unrolled.
// Accumulation is fp64: sums of up to 128 bf16 values (or e4m3 codes) are
// exact in fp64, so the result is the exact mean rounded once and does not
// depend on summation order.  fp8 sums the codes and multiplies by the
// per-head scale once (code sums and their product with an fp32 scale are
// exact in fp64).
#include "fp_device.h"

namespace fp {
namespace {

constexpr int kHeadsPerWG = 4;
constexpr int kThreads = 256;
constexpr int kRowsPerPass = kThreads / (16 * kHeadsPerWG);  // 4 token rows per pass

struct PoolK {
  PoolLaunch a;
  SeqDesc sd;
  PageDesc pd;
};

__device__ inline void add_bf16x8(double* acc, u32x4 v) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    acc[2 * w] += (double)__uint_as_float(v[w] << 16);
    acc[2 * w + 1] += (double)__uint_as_float(v[w] & 0xffff0000u);
  }
}

__device__ inline void add_fp8x8(double* acc, u32x2 v) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], true);
    acc[4 * w + 0] += (double)lo[0];
    acc[4 * w + 1] += (double)lo[1];
    acc[4 * w + 2] += (double)hi[0];
    acc[4 * w + 3] += (double)hi[1];
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void pool_kernel(PoolK p) {
  const PoolLaunch& a = p.a;
  const int i = blockIdx.x;   // block within the sequence
  const int s = blockIdx.y;   // sequence
  const int hg = blockIdx.z;  // head group
  const SeqPos sp = seq_pos(p.sd, s);
  // the view: key blocks 0..nb-1 of the key tokens, or the query blocks of the
  // query tokens (block i = absolute block I0 + i; its tokens are the positions
  // 128(I0+i) .. 128(I0+i)+127 that the query chunk holds)
  const bool qv = a.query_view;
  const int nb = qv ? sp.nq : (sp.len + kBlock - 1) / kBlock;
  const int64_t blk0 = qv ? sp.qblk0 : sp.blk0;
  const int64_t total_blocks = qv ? p.sd.total_qblocks : p.sd.total_blocks;
  if (i >= nb || blk0 + i >= total_blocks) return;
  const int vlen = qv ? sp.qlen : sp.len;
  const int voff = qv ? sp.qoff : 0;
  const int first = max(0, (qv ? sp.I0 + i : i) * kBlock - voff);  // first token of the block in the view
  const int n = min(vlen, (qv ? sp.I0 + i + 1 : i + 1) * kBlock - voff) - first;

  const int tid = threadIdx.x;
  const int chunk = tid & 15;                  // 8 consecutive elements of a head row
  const int hl = (tid >> 4) & (kHeadsPerWG - 1);
  const int r0 = tid >> 6;                     // token row lane 0..3
  const int h = hg * kHeadsPerWG + hl;

  bool bad_page = false;
  const char* base;
  constexpr int esize = DT == 0 ? 2 : 1;
  if (a.paged) {
    const int page = p.pd.table[(int64_t)s * p.pd.max_pages + i];
    bad_page = page < 0 || page >= p.pd.num_pages;
    base = (const char*)a.x + ((int64_t)(bad_page ? 0 : page) * a.st_page) * esize;
  } else {
    base = (const char*)a.x + (((qv ? sp.qtok0 : sp.tok0) + first) * a.st_tok) * esize;
  }
  base += ((int64_t)h * a.st_head + chunk * 8) * esize;
  const int64_t row_step = a.st_tok * esize;

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;

  if (h < a.H && !bad_page) {
    int t = r0;
    // full passes of 8 rows per thread in flight
    for (; t + 7 * kRowsPerPass < n; t += 8 * kRowsPerPass) {
      if (DT == 0) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = __builtin_nontemporal_load((const u32x4*)(base + (int64_t)(t + u * kRowsPerPass) * row_step));
#pragma unroll
        for (int u = 0; u < 8; ++u) add_bf16x8(acc, v[u]);
      } else {
        u32x2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = __builtin_nontemporal_load((const u32x2*)(base + (int64_t)(t + u * kRowsPerPass) * row_step));
#pragma unroll
        for (int u = 0; u < 8; ++u) add_fp8x8(acc, v[u]);
      }
    }
    for (; t < n; t += kRowsPerPass) {
      if (DT == 0) add_bf16x8(acc, *(const u32x4*)(base + (int64_t)t * row_step));
      else add_fp8x8(acc, *(const u32x2*)(base + (int64_t)t * row_step));
    }
  }

  __shared__ double red[kRowsPerPass][kHeadsPerWG * kHeadDim];
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][hl * kHeadDim + chunk * 8 + e] = acc[e];
  __syncthreads();

  // 512 outputs (4 heads x 128), two per thread, contiguous per head row.
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = tid + u * kThreads;
    const int ho = hg * kHeadsPerWG + o / kHeadDim;
    if (ho >= a.H) continue;
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < kRowsPerPass; ++r) sum += red[r][o];
    if (DT == 1) sum *= (double)a.scale[ho];
    double mean = sum / (double)n;
    if (bad_page) mean = __builtin_nan("");
    a.out[((int64_t)ho * total_blocks + blk0 + i) * kHeadDim + (o & (kHeadDim - 1))] = mean;
  }
}

}  // namespace

hipError_t launch_pool(const PoolLaunch& a, const SeqDesc& sd, const PageDesc& pd, hipStream_t st) {
  PoolK p{a, sd, pd};
  if (!a.paged) p.pd.table = nullptr;
  dim3 grid(a.query_view ? sd.max_nq : sd.max_nb, sd.n_seqs, (a.H + kHeadsPerWG - 1) / kHeadsPerWG);
  if (a.dtype == 0)
    hipLaunchKernelGGL(pool_kernel<0>, grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(pool_kernel<1>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace fp
