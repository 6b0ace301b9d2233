// Pooled block scores, dynamic threshold and index compaction (FlashPrefill
// Method 1 pooled score map, Method 2 "Dynamic Threshold Pruning": keep a
// block when its score reaches alpha times the row maximum, always keep the
// attention sinks and the local window; Method 3 "Index Compaction": write
// the kept block ids of every row into a contiguous ascending list).
//
// One workgroup owns a tile of 64 query blocks of one (sequence, query head)
// and sweeps the key-block tiles its rows need twice: pass 1 computes the fp64
// scores and the row maxima, pass 2 recomputes them, tests s - max >= ln(alpha)
// (or sink / local), and compacts.  Scores are fp64 dot products of the fp64
// pooled means in 64x64 tiles: the query tile stays in LDS for both passes, key
// tiles stream through LDS with the next one already in registers, and each
// thread owns a 4x4 sub-tile.  Row tiles with the longest rows start first.  Compaction: the 16 lanes that share
// a row hold 4 consecutive columns each, so a 16-lane exclusive prefix sum of
// the per-lane keep counts gives every kept id its slot, ascending by
// construction.  The logical-skip ablation asks for the same decisions as a
// bit-packed block mask instead of lists (32 blocks per word, bit j%32 of word
// j/32 of row i).
#include "fp_device.h"

namespace fp {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;

struct SelK {
  SelectLaunch a;
  SeqDesc sd;
};

template <bool MASK>
__global__ __launch_bounds__(kThreads, 1) void select_kernel(SelK p) {
  const SelectLaunch& a = p.a;
  const int it = gridDim.x - 1 - blockIdx.x;  // row tiles with the longest rows first
  const int s = blockIdx.y;
  const int h = blockIdx.z;
  const SeqPos sp = seq_pos(p.sd, s);
  // rows: the sequence's query blocks r = 0..nq-1, absolute block I = I0 + r;
  // columns: its key blocks j = 0..I
  // (clamped to the declared extents so inconsistent metadata cannot read past them)
  const int nq = (int)min((int64_t)sp.nq, max((int64_t)0, p.sd.total_qblocks - sp.qblk0));
  const int nk = (int)min((int64_t)(sp.len + kBlock - 1) / kBlock, max((int64_t)0, p.sd.total_blocks - sp.blk0));
  const int I0 = sp.I0;
  const int row0 = it * kTile;
  if (row0 >= nq) return;
  const int nt = (I0 + min(row0 + kTile, nq) - 1) / kTile + 1;  // key tiles any row of this tile needs
  const int g = h / (a.hq / a.hkv);
  const double* Qb = a.pq + ((int64_t)h * p.sd.total_qblocks + sp.qblk0) * kHeadDim;
  const double* Kb = a.pk + ((int64_t)g * p.sd.total_blocks + sp.blk0) * kHeadDim;

  // The query tile stays in LDS for both passes; key tiles stream through LDS and
  // the next one is in registers while the current one is used.  d-major layout:
  // a thread reads 4 consecutive rows (or columns) of one d as two 16-byte reads.
  __shared__ __attribute__((aligned(16))) double Qs[kHeadDim][kTile];
  __shared__ __attribute__((aligned(16))) double Ks[kHeadDim][kTile];

  const int tid = threadIdx.x;
  const int tr = tid >> 4, tc = tid & 15;
  const double NEG_INF = -__builtin_huge_val();

  // staging: thread t moves row t/4, d = 32(t%4) .. +31 of a 64-row tile
  typedef __attribute__((ext_vector_type(2))) double f64x2;
  f64x2 reg[16];
  auto load_rows = [&](const double* base, int first, int nrows) {
    const int rr = tid >> 2, d0 = (tid & 3) * 32;
    const bool ok = first + rr < nrows;
    const f64x2* src = (const f64x2*)(base + (int64_t)(first + rr) * kHeadDim + d0);
#pragma unroll
    for (int u = 0; u < 16; ++u) reg[u] = ok ? src[u] : f64x2{0.0, 0.0};
  };
  auto store_rows = [&](double (*S)[kTile]) {
    const int rr = tid >> 2, d0 = (tid & 3) * 32;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      S[d0 + 2 * u][rr] = reg[u][0];
      S[d0 + 2 * u + 1][rr] = reg[u][1];
    }
  };

  double acc[4][4];
  auto tile_scores = [&]() {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = 0.0;
#pragma unroll 8
    for (int dd = 0; dd < kHeadDim; ++dd) {
      const f64x2 q01 = *(const f64x2*)&Qs[dd][tr * 4], q23 = *(const f64x2*)&Qs[dd][tr * 4 + 2];
      const f64x2 k01 = *(const f64x2*)&Ks[dd][tc * 4], k23 = *(const f64x2*)&Ks[dd][tc * 4 + 2];
      const double qv[4] = {q01[0], q01[1], q23[0], q23[1]};
      const double kv[4] = {k01[0], k01[1], k23[0], k23[1]};
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fma(qv[x], kv[y], acc[x][y]);
    }
  };

  load_rows(Qb, row0, nq);
  store_rows(Qs);
  load_rows(Kb, 0, nk);

  double rmax[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
  int cnt[4] = {0, 0, 0, 0};
  int32_t* idx_h = a.idx + (int64_t)h * p.sd.total_tri + sp.tri0;
  const int64_t tri_cap = p.sd.total_tri - sp.tri0;
  // pass 1 (q < nt): row maxima over the causal blocks j <= I; pass 2: threshold +
  // compaction, recomputing the same scores
  for (int q = 0; q < 2 * nt; ++q) {
    const int jt = q < nt ? q : q - nt;
    __syncthreads();  // every thread is done with the previous key tile
    store_rows(Ks);
    __syncthreads();
    if (q + 1 < 2 * nt) load_rows(Kb, ((q + 1) % nt) * kTile, nk);
    tile_scores();
    if (q < nt) {
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
      if (q == nt - 1) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) rmax[x] = fmax(rmax[x], __shfl_xor(rmax[x], off, 16));
      }
      continue;
    }
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
