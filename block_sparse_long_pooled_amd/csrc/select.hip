// Pooled block scores, dynamic threshold and index compaction (FlashPrefill
// Method 1 pooled score map, Method 2 "Dynamic Threshold Pruning": keep a
// block when its score reaches alpha times the row maximum, always keep the
// attention sinks and the local window; Method 3 "Index Compaction": write
// the kept block ids of every row into a contiguous ascending list).
//
// One workgroup owns a tile of 64 query blocks of one (sequence, query head)
// and sweeps the causal key-block tiles 0..(its own) twice: pass 1 computes
// the fp64 scores and the row maxima, pass 2 recomputes them, tests
// s - max >= ln(alpha) (or sink / local), and compacts.  Scores are fp64 dot
// products of the fp64 pooled means, tiled 64x64 with a 16-wide d-chunk in
// LDS; each thread owns a 4x4 sub-tile.  Compaction: the 16 lanes that share
// a row hold 4 consecutive columns each, so a 16-lane exclusive prefix sum of
// the per-lane keep counts gives every kept id its slot, ascending by
// construction.  The logical-skip ablation asks for the same decisions as a
// bit-packed block mask instead of lists (32 blocks per word, bit j%32 of word
// j/32 of row i).
#include "fp_device.h"

namespace fp {
namespace {

constexpr int kTile = 64;
constexpr int kDK = 16;
constexpr int kThreads = 256;

struct SelK {
  SelectLaunch a;
  SeqDesc sd;
};

// acc[4][4] = Qtile(rows tr*4..) x Ktile(cols tc*4..)^T for one (row tile, col tile);
// rows past nq and columns past nk read as zero.
__device__ inline void tile_scores(const double* __restrict__ Qb, const double* __restrict__ Kb,
                                   int row0, int col0, int nq, int nk, double (*Qs)[kTile], double (*Ks)[kTile],
                                   double acc[4][4]) {
  const int tid = threadIdx.x;
  const int tr = tid >> 4, tc = tid & 15;
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.0;
  for (int dk0 = 0; dk0 < kHeadDim; dk0 += kDK) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + u * kThreads;  // 0..1023 = 64 rows x 16 d
      const int rr = e >> 4, dd = e & 15;
      const int qi = row0 + rr, kj = col0 + rr;
      Qs[dd][rr] = qi < nq ? Qb[(int64_t)qi * kHeadDim + dk0 + dd] : 0.0;
      Ks[dd][rr] = kj < nk ? Kb[(int64_t)kj * kHeadDim + dk0 + dd] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int dd = 0; dd < kDK; ++dd) {
      double qv[4], kv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) qv[x] = Qs[dd][tr * 4 + x];
#pragma unroll
      for (int y = 0; y < 4; ++y) kv[y] = Ks[dd][tc * 4 + y];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fma(qv[x], kv[y], acc[x][y]);
    }
  }
}

template <bool MASK>
__global__ __launch_bounds__(kThreads) void select_kernel(SelK p) {
  const SelectLaunch& a = p.a;
  const int it = blockIdx.x;
  const int s = blockIdx.y;
  const int h = blockIdx.z;
  const SeqPos sp = seq_pos(p.sd, s);
  // rows: the sequence's query blocks r = 0..nq-1, absolute block I = I0 + r;
  // columns: its key blocks j = 0..I
  const int nq = sp.nq;
  const int nk = (sp.len + kBlock - 1) / kBlock;
  const int I0 = sp.I0;
  const int row0 = it * kTile;
  if (row0 >= nq) return;
  const int jt_last = (I0 + min(row0 + kTile, nq) - 1) / kTile;  // last key tile any row of this tile needs
  const int g = h / (a.hq / a.hkv);
  const double* Qb = a.pq + ((int64_t)h * p.sd.total_qblocks + sp.qblk0) * kHeadDim;
  const double* Kb = a.pk + ((int64_t)g * p.sd.total_blocks + sp.blk0) * kHeadDim;

  __shared__ double Qs[kDK][kTile];
  __shared__ double Ks[kDK][kTile];

  const int tid = threadIdx.x;
  const int tr = tid >> 4, tc = tid & 15;
  const double NEG_INF = -__builtin_huge_val();

  // pass 1: row maxima over the causal blocks j <= i
  double rmax[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
  double acc[4][4];
  for (int jt = 0; jt <= jt_last; ++jt) {
    tile_scores(Qb, Kb, row0, jt * kTile, nq, nk, Qs, Ks, acc);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int r = row0 + tr * 4 + x;
      const int i = I0 + r;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int j = jt * kTile + tc * 4 + y;
        if (j <= i && r < nq) rmax[x] = fmax(rmax[x], acc[x][y] * a.scale);
      }
    }
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) rmax[x] = fmax(rmax[x], __shfl_xor(rmax[x], off, 16));

  // pass 2: threshold + compaction
  int cnt[4] = {0, 0, 0, 0};
  int32_t* idx_h = a.idx + (int64_t)h * p.sd.total_tri + sp.tri0;
  const int64_t tri_cap = p.sd.total_tri - sp.tri0;
  for (int jt = 0; jt <= jt_last; ++jt) {
    tile_scores(Qb, Kb, row0, jt * kTile, nq, nk, Qs, Ks, acc);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int r = row0 + tr * 4 + x;
      const int i = I0 + r;
      unsigned bits = 0;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int j = jt * kTile + tc * 4 + y;
        const double sc = acc[x][y] * a.scale;
        const bool keep = (j <= i) && (r < nq) &&
                          ((sc - rmax[x] >= a.log_alpha) || (j < a.n_sink) || (j > i - a.n_local));
        bits |= (keep ? 1u : 0u) << y;
      }
      if (MASK) {
        // the 8 lanes tc&~7 .. tc|7 hold the 32 columns of one word of row i
        unsigned word = bits << (4 * (tc & 7));
        word |= __shfl_xor(word, 1, 16);
        word |= __shfl_xor(word, 2, 16);
        word |= __shfl_xor(word, 4, 16);
        const int wi = (jt * kTile + tc * 4) >> 5;
        if ((tc & 7) == 0 && r < nq && wi < a.mask_words) a.mask[((int64_t)h * nq + r) * a.mask_words + wi] = word;
        continue;
      }
      const int pc = __popc(bits);
      int incl = pc;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int v = __shfl_up(incl, off, 16);
        if (tc >= off) incl += v;
      }
      const int total = __shfl(incl, 15, 16);
      int pos = cnt[x] + incl - pc;
      const int64_t rbase = (int64_t)r * (I0 + 1) + (int64_t)r * (r - 1) / 2;  // rows I0 .. i-1 hold I0+1 .. i slots
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        if (bits & (1u << y)) {
          if (rbase + pos < tri_cap) idx_h[rbase + pos] = jt * kTile + tc * 4 + y;
          ++pos;
        }
      }
      cnt[x] += total;
    }
  }
  if (!MASK && tc == 0) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int r = row0 + tr * 4 + x;
      if (r < nq && sp.qblk0 + r < p.sd.total_qblocks)
        a.counts[(int64_t)h * p.sd.total_qblocks + sp.qblk0 + r] = cnt[x];
    }
  }
}

}  // namespace

hipError_t launch_select(const SelectLaunch& a, const SeqDesc& sd, hipStream_t st) {
  SelK p{a, sd};
  dim3 grid((sd.max_nq + kTile - 1) / kTile, sd.n_seqs, a.hq);
  if (a.mask != nullptr) hipLaunchKernelGGL(select_kernel<true>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(select_kernel<false>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace fp
