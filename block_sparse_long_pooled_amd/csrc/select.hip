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
// pooled means in 64x64 tiles on the fp64 matrix core: the query tile stays in
// LDS for both passes and key tiles stream through LDS with the next one
// already in registers.  Row tiles with the longest rows start first.
// Compaction: the 16 lanes that share a row hold one column of each 16-column
// slice, so a ballot per slice and a popcount of the lower lanes give every
// kept id its slot, ascending by construction.  The logical-skip ablation asks
// for the same decisions as a bit-packed block mask instead of lists (32 blocks
// per word, bit j%32 of word j/32 of row i).
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
__global__ __launch_bounds__(kThreads, 2) void select_kernel(SelK p) {
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

  // Key tiles stream through LDS (d-major, [d][column]) and the next one is in
  // registers while the current one is used.  The query tile passes through the
  // same LDS buffer once, at the start, into each lane's A operands, which then stay
  // in registers for both passes; with 64 KB of LDS two workgroups share a CU.
  __shared__ __attribute__((aligned(16))) double Ks[kHeadDim][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int lg = lane >> 4;   // 16-lane group
  const int lc = lane & 15;   // lane within the group
  const double NEG_INF = -__builtin_huge_val();

  // staging: thread t moves row t/4, d = 32(t%4) .. +31 of a 64-row tile
  typedef __attribute__((ext_vector_type(2))) double f64x2;
  typedef __attribute__((ext_vector_type(4))) double f64x4;
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

  // Scores on the fp64 matrix core (v_mfma_f64_16x16x4_f64: A lane = row l%16 at
  // k = l/16, B lane = column l%16 at k = l/16, C element v of lane l = row
  // l/16 + 4v, column l%16).  Wave w owns tile rows 16w .. 16w+15 and all 64
  // columns as four 16x16 products, so a row's 64 scores live in one 16-lane
  // group: lane lc of group lg holds rows 16w + lg + 4v (v = 0..3) at columns
  // 16t + lc (t = 0..3) in acc[t][v].
  f64x4 acc[4];
  double qa[kHeadDim / 4];  // A operand of step ks: row 16w + lc, d = 4ks + lg
  auto tile_scores = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 4; ++ks) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[ks], Ks[4 * ks + lg][16 * t + lc], acc[t], 0, 0, 0);
    }
  };

  load_rows(Qb, row0, nq);
  store_rows(Ks);
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 4; ++ks) qa[ks] = Ks[4 * ks + lg][16 * w + lc];
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
      for (int v = 0; v < 4; ++v) {
        const int r = row0 + 16 * w + lg + 4 * v;
        const int i = I0 + r;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int j = jt * kTile + 16 * t + lc;
          if (j <= i && r < nq) {
            rmax[v] = fmax(rmax[v], acc[t][v] * a.scale);
            if (a.scores != nullptr) a.scores[((int64_t)h * nq + r) * nk + j] = acc[t][v] * a.scale;
          }
        }
      }
      if (q == nt - 1) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) rmax[v] = fmax(rmax[v], __shfl_xor(rmax[v], off, 16));
      }
      continue;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = row0 + 16 * w + lg + 4 * v;
      const int i = I0 + r;
      const int64_t rbase = (int64_t)r * (I0 + 1) + (int64_t)r * (r - 1) / 2;  // rows I0 .. i-1 hold I0+1 .. i slots
      unsigned gb[4];  // keep bits of the 16 columns 16t .. 16t+15 of this lane's row
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = jt * kTile + 16 * t + lc;
        const double sc = acc[t][v] * a.scale;
        const bool keep = (j <= i) && (r < nq) &&
                          ((sc - rmax[v] >= a.log_alpha) || (j < a.n_sink) || (j > i - a.n_local));
        gb[t] = (unsigned)(__ballot(keep) >> (16 * lg)) & 0xffffu;
      }
      if (MASK) {
        // words 2jt and 2jt+1 of the row: columns 0..31 and 32..63 of this tile
        if (lc < 2 && r < nq) {
          const int wi = 2 * jt + lc;
          if (wi < a.mask_words)
            a.mask[((int64_t)h * nq + r) * a.mask_words + wi] = gb[2 * lc] | (gb[2 * lc + 1] << 16);
        }
        continue;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (gb[t] & (1u << lc)) {
          const int64_t pos = cnt[v] + __popc(gb[t] & ((1u << lc) - 1u));
          if (rbase + pos < tri_cap) idx_h[rbase + pos] = jt * kTile + 16 * t + lc;
        }
        cnt[v] += __popc(gb[t]);
      }
    }
  }
  if (!MASK && lc == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = row0 + 16 * w + lg + 4 * v;
      if (r < nq && sp.qblk0 + r < p.sd.total_qblocks)
        a.counts[(int64_t)h * p.sd.total_qblocks + sp.qblk0 + r] = cnt[v];
    }
  }
}

// Group-shared lists: one wave per (query block i, KV group g) ORs the group's
// per-head mask words covering j <= i and writes the set bits in ascending order
// (a wave prefix sum of the per-word popcounts gives each word its first slot).
__global__ __launch_bounds__(64) void union_kernel(UnionLaunch a) {
  const int i = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x;
  const int G = a.hq / a.hkv;
  const int nwords = (i >> 5) + 1;
  int32_t* out = a.idx + (int64_t)g * ((int64_t)a.nb * (a.nb + 1) / 2) + (int64_t)i * (i + 1) / 2;
  int base = 0;
  for (int w0 = 0; w0 < nwords; w0 += 64) {
    const int wi = w0 + lane;
    unsigned word = 0;
    if (wi < nwords && wi < a.mask_words) {
      for (int hh = 0; hh < G; ++hh) word |= a.mask[((int64_t)(g * G + hh) * a.nb + i) * a.mask_words + wi];
      if (wi == nwords - 1 && (i & 31) != 31) word &= (2u << (i & 31)) - 1u;  // only j <= i
    }
    const int pc = __popc(word);
    int incl = pc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    int pos = base + incl - pc;
    while (word != 0u) {
      const int b = __ffs(word) - 1;
      out[pos++] = wi * 32 + b;
      word &= word - 1u;
    }
    base += __shfl(incl, 63);
  }
  if (lane == 0) a.counts[(int64_t)g * a.nb + i] = base;
}

}  // namespace

hipError_t launch_union(const UnionLaunch& a, hipStream_t st) {
  dim3 grid(a.nb, a.hkv);
  hipLaunchKernelGGL(union_kernel, grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectLaunch& a, const SeqDesc& sd, hipStream_t st) {
  SelK p{a, sd};
  dim3 grid((sd.max_nq + kTile - 1) / kTile, sd.n_seqs, a.hq);
  if (a.mask != nullptr) hipLaunchKernelGGL(select_kernel<true>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(select_kernel<false>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace fp
