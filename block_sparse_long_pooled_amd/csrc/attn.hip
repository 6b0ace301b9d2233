// Causal GQA block-sparse flash attention over compacted block lists
// (FlashPrefill Method 3 "Index Compaction -> Physical Jumps": the inner loop
// walks only the listed key blocks; FlashPrefill V2 abstract: bf16 and FP8,
// paged KV cache, continuous batching).
//
// CDNA4 design (not the H20 one on the pages):
//   * one workgroup = one (query head, query block of 128 tokens), 4 waves,
//     each wave owns 32 query rows; two workgroups share a CU (64 KB LDS each);
//   * the transposed products S^T = K Q^T and O^T = V^T P^T on
//     v_mfma_f32_32x32x16_bf16 (fp8: v_mfma_f32_32x32x64_f8f6f4), so every
//     lane owns ONE query column of S^T and of O^T: the softmax row max and sum
//     are in-lane plus one v_permlane32_swap, and the O rescale is in-lane;
//   * the S^T accumulator (keys 8i+4h+j of the lane's query) is the P^T
//     operand of the PV product as it stands: the contraction over keys only
//     needs V^T to list keys in the same slot order;
//   * K (and bf16 V) go HBM -> LDS with 16-byte direct loads into rows whose
//     16-byte chunks are XOR-swizzled by row, so the MFMA operand reads are
//     free of bank conflicts; bf16 V^T operands come straight from the
//     row-major tile through ds_read_b64_tr_b16 (transposing LDS reads);
//   * split-phase pipelining with one K and one V buffer: the loads of tile
//     n+1's K start as soon as every wave has finished Q K^T of tile n, and
//     those of its V as soon as P V of tile n is done, so both overlap compute;
//   * lists are ascending with the diagonal last: only the last visited block
//     needs the causal mask;
//   * fp32 online softmax in exp2 units with a lazy rescale: O and the row sum
//     are rescaled only when the running maximum grows by more than TAU, so P
//     stays <= 2^TAU; the row sum adds the ROUNDED probabilities, i.e. exactly
//     the weights that enter P V, so output rows are true convex combinations;
//   * fp8: e4m3 Q K^T and P V (P rounded to e4m3 after a 2^4 range shift), V
//     staged through registers into the operand-slot order with an 8x8 byte
//     transpose.
#include "fp_device.h"

namespace fp {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnK {
  AttnLaunch a;
  SeqDesc sd;
  PageDesc pd;
  int group;
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// s_waitcnt immediate (gfx9 layout) that waits until at most n vector-memory
// operations are outstanding and leaves the other counters unconstrained.
constexpr int vmcnt_le(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ inline u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// One 16-byte direct HBM -> LDS load per lane; the wave writes 1 KB contiguous
// at lds_base (wave-uniform) + 16 * lane.
__device__ inline void dma16(const unsigned char* g, unsigned char* lds_base) {
  __builtin_amdgcn_global_load_lds((const void*)g, (lds_void_t*)lds_base, 16, 0, 0);
}

// 8x8 transpose of bytes: in[e] holds 8 consecutive d (bytes) of key e;
// out[r] holds key 0..7 of d = r.
__device__ inline void transpose8x8_b8(const u32x2 in[8], u32x2 out[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int w = r >> 2, b = r & 3;
    const unsigned s_lo = (unsigned)b | ((unsigned)(b + 4) << 8) | 0x0c0c0000u;
    const unsigned s_hi = 0x00000c0cu | ((unsigned)b << 16) | ((unsigned)(b + 4) << 24);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const unsigned lo = __builtin_amdgcn_perm(in[4 * q + 1][w], in[4 * q + 0][w], s_lo);
      const unsigned hi = __builtin_amdgcn_perm(in[4 * q + 3][w], in[4 * q + 2][w], s_hi);
      out[r][q] = lo | hi;
    }
  }
}

__device__ inline float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// LDS operand reads.  The restrict-qualified parameter gives each inlined read
// alias-scope information, which lets the compiler's wait-count pass see that a
// read of one tile buffer does not depend on the direct loads still filling the
// other one (otherwise it drains every outstanding load before any LDS read).
__device__ __attribute__((always_inline)) inline u32x4 lds16(const unsigned char* __restrict__ base, unsigned off) {
  return *(const u32x4*)(base + off);
}
__device__ __attribute__((always_inline)) inline s16x4 lds_tr16(const unsigned char* __restrict__ base, unsigned off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + off));
}

// Workgroup barrier that does not drain the in-flight HBM -> LDS loads: only
// this wave's LDS reads/writes must be complete (lgkmcnt), the asm statements
// keep the compiler from moving memory operations across it.
__device__ inline void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(vmcnt_le(63) & ~(15 << 8));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int DT, bool PAGED, bool DENSE, bool LSE>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnK p) {
  constexpr int ES = DT == 0 ? 2 : 1;             // element size in bytes
  constexpr int KROW = kHeadDim * ES;             // bytes per K (and bf16 V) row
  constexpr int TILE = kBlock * KROW;             // 32 KB bf16, 16 KB fp8
  constexpr float TAU = DT == 0 ? 8.0f : 4.0f;    // lazy-rescale slack (log2 units)
  constexpr float SHIFT = DT == 0 ? 0.0f : 4.0f;  // fp8: P in (0, 2^(TAU+SHIFT)] = (0, 256]
  constexpr int KLOADS = DT == 0 ? 8 : 4;         // K-tile loads per wave
  constexpr int VLOADS = 8;                       // V-tile loads per wave
  __shared__ __attribute__((aligned(1024))) unsigned char Ks[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs[TILE];

  const AttnLaunch& a = p.a;
  // Work decode: query heads fastest so that consecutive workgroups share the
  // same query block; with hq % 8 == 0 each XCD (workgroup id % 8) receives a
  // contiguous run of heads, i.e. heads of one KV group, for L2 reuse of K/V.
  const int id = blockIdx.x;
  int h;
  if ((a.hq & 7) == 0) {
    const int per = a.hq >> 3;
    h = (id & 7) * per + ((id >> 3) % per);
  } else {
    h = id % a.hq;
  }
  const int rest = id / a.hq;
  const int s = rest % p.sd.n_seqs;
  const int i = p.sd.max_nb - 1 - rest / p.sd.n_seqs;  // heaviest query blocks first
  const SeqPos sp = seq_pos(p.sd, s);
  const int nb = (sp.len + kBlock - 1) / kBlock;
  if (i < 0 || i >= nb || sp.blk0 + i >= p.sd.total_blocks) return;
  const int g = h / p.group;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int ql = lane & 31;
  const int hh = lane >> 5;
  const int qq = 32 * w + ql;  // query row within the block
  const int tq = i * kBlock + qq;
  const bool qvalid = tq < sp.len;

  // ---- Q fragments (B operand of S^T = K Q^T): lane = query column, 8 (bf16) or
  //      32 (fp8) consecutive d per MFMA step, half hh takes the upper part.
  const unsigned char* qrow = (const unsigned char*)a.q + ((sp.tok0 + tq) * a.q_st + (int64_t)h * a.q_sh) * ES;
  u32x4 qf[DT == 0 ? 8 : 4];
  if (DT == 0) {
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = qvalid ? *(const u32x4*)(qrow + (16 * st + 8 * hh) * 2) : zero4();
  } else {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      qf[2 * st] = qvalid ? *(const u32x4*)(qrow + 64 * st + 32 * hh) : zero4();
      qf[2 * st + 1] = qvalid ? *(const u32x4*)(qrow + 64 * st + 32 * hh + 16) : zero4();
    }
  }

  float c = a.softmax_scale * kLog2e;  // logits -> log2 units
  if (DT == 1) c *= a.q_scale[h] * a.k_scale[g];

  // list entries are wave-uniform: read them through the constant address space
  // so they become scalar loads (they must not share the vector-memory counter
  // with the in-flight tile loads).
  typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
  int cnt;
  cint_ptr list = nullptr;
  if (DENSE) {
    cnt = i + 1;
  } else {
    cnt = ((cint_ptr)a.counts)[(int64_t)h * p.sd.total_blocks + sp.blk0 + i];
    cnt = uniform(cnt < 0 ? 0 : (cnt > i + 1 ? i + 1 : cnt));
    list = (cint_ptr)(a.idx + (int64_t)h * p.sd.total_tri + sp.tri0 + (int64_t)i * (i + 1) / 2);
  }
  bool bad = cnt == 0;

  const unsigned kst = (unsigned)(a.k_st * ES), vst = (unsigned)(a.v_st * ES);  // token strides, bytes
  // K/V base of list entry n (wave-uniform); an invalid block id or page is
  // replaced by an in-bounds block (the output of this query block becomes NaN).
  auto tile = [&](int n, const unsigned char*& kb, const unsigned char*& vb, int& j, int& rows) {
    j = DENSE ? n : uniform(list[n]);
    if (j < 0 || j > i) { bad = true; j = 0; }
    if (PAGED) {
      int page = uniform(((cint_ptr)p.pd.table)[(int64_t)s * p.pd.max_pages + j]);
      if (page < 0 || page >= p.pd.num_pages) { bad = true; page = 0; }
      kb = (const unsigned char*)a.k + ((int64_t)page * a.k_sp + (int64_t)g * a.k_sh) * ES;
      vb = (const unsigned char*)a.v + ((int64_t)page * a.v_sp + (int64_t)g * a.v_sh) * ES;
    } else {
      kb = (const unsigned char*)a.k + ((sp.tok0 + (int64_t)j * kBlock) * a.k_st + (int64_t)g * a.k_sh) * ES;
      vb = (const unsigned char*)a.v + ((sp.tok0 + (int64_t)j * kBlock) * a.v_st + (int64_t)g * a.v_sh) * ES;
    }
    rows = min(kBlock, sp.len - j * kBlock);
  };

  // ---- per-lane byte offsets (the rest of every address is wave-uniform or an
  //      immediate).  K tile: row R's logical 16-byte chunk c sits at physical
  //      chunk c ^ (R & 7); bf16 V tile: at c ^ (2 * (R & 3)).
  // DMA sources: bf16 K needs two variants (R & 7 alternates with the load index).
  unsigned k_src[2], v_src = 0, k8_src = 0;
  if (DT == 0) {
    const int r = lane >> 4, pc = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) k_src[e] = r * kst + ((pc ^ ((r + 4 * e) & 7)) << 4);
    v_src = r * vst + ((pc ^ (2 * (r & 3))) << 4);
  } else {
    const int r = lane >> 3, pc = lane & 7;
    k8_src = r * kst + ((pc ^ (r & 7)) << 4);
    k_src[0] = k_src[1] = 0;
  }
  // Q K^T operand reads: logical chunk 2st+hh (bf16) of row 32kt+ql; st >= 4 is +128 B.
  unsigned k_rd[4];
  if (DT == 0) {
#pragma unroll
    for (int st = 0; st < 4; ++st) k_rd[st] = ql * KROW + ((((2 * st + hh)) ^ (ql & 7)) << 4);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) k_rd[q] = ql * KROW + (((4 * (q >> 1) + 2 * hh + (q & 1)) ^ (ql & 7)) << 4);
  }
  // bf16 V^T transposing reads: source lane sl points at key row 16cc + 8c + 4hh + sl/4,
  // d = 32dt + 16(G&1) + 4(sl&3); the (dt & 1) bit of the chunk meets the swizzle.
  unsigned v_rd[2];
  {
    const int G = lane >> 4, sl = lane & 15, z = 2 * (sl >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      v_rd[e] = (4 * hh + (sl >> 2)) * KROW + (((4 * e + 2 * (G & 1) + ((sl & 3) >> 1)) ^ z) << 4) + 8 * (sl & 1);
  }
  // fp8 V: thread (c2, h2, r4, dc) gathers 8 keys x 8 d of its operand slot group.
  const int v8_c2 = tid >> 7, v8_h2 = (tid >> 6) & 1, v8_r4 = (tid >> 4) & 3, v8_dc = tid & 15;
  const unsigned v8_st = (((v8_c2 * 2 + v8_h2) * kHeadDim) + 8 * v8_dc) * 32 + 8 * v8_r4;
  const unsigned v8_rd = (hh * kHeadDim + ql) * 32;

  auto issue_k = [&](const unsigned char* kb, int rows) {
    if (rows == kBlock) {
      if (DT == 0) {
#pragma unroll
        for (int u = 0; u < KLOADS; ++u) {
          const int R0 = 32 * w + 4 * u;
          dma16(kb + R0 * kst + k_src[u & 1], Ks + R0 * KROW);
        }
      } else {
#pragma unroll
        for (int u = 0; u < KLOADS; ++u) {
          const int R0 = 32 * w + 8 * u;
          dma16(kb + R0 * kst + k8_src, Ks + R0 * KROW);
        }
      }
    } else {  // partial last block: rows past the end re-read row 0 (finite, masked)
      const int per = DT == 0 ? 16 : 8;
#pragma unroll
      for (int u = 0; u < KLOADS; ++u) {
        const int R0 = 32 * w + (DT == 0 ? 4 : 8) * u, R = R0 + lane / per;
        const int lc = (lane % per) ^ (R & 7);
        dma16(kb + (R < rows ? R : 0) * kst + (lc << 4), Ks + R0 * KROW);
      }
    }
  };
  auto issue_v16 = [&](const unsigned char* vb, int rows) {
    if (rows == kBlock) {
#pragma unroll
      for (int u = 0; u < VLOADS; ++u) {
        const int R0 = 32 * w + 4 * u;
        dma16(vb + R0 * vst + v_src, Vs + R0 * KROW);
      }
    } else {
#pragma unroll
      for (int u = 0; u < VLOADS; ++u) {
        const int R0 = 32 * w + 4 * u, R = R0 + (lane >> 4);
        const int lc = (lane & 15) ^ (2 * (R & 3));
        dma16(vb + (R < rows ? R : 0) * vst + (lc << 4), Vs + R0 * KROW);
      }
    }
  };
  u32x2 vreg[8];
  auto load_v8 = [&](const unsigned char* vb, int rows) {  // rows past the end are zero
#pragma unroll
    for (int u = 0; u < VLOADS; ++u) {
      const int e = 8 * v8_r4 + u;
      const int key = 32 * (2 * v8_c2 + (e >> 4)) + 8 * ((e & 15) >> 2) + 4 * v8_h2 + (e & 3);
      vreg[u] = key < rows ? *(const u32x2*)(vb + key * vst + v8_dc * 8) : u32x2{0u, 0u};
    }
  };
  auto store_v8 = [&]() {
    u32x2 vt[8];
    transpose8x8_b8(vreg, vt);
#pragma unroll
    for (int r = 0; r < 8; ++r) *(u32x2*)(Vs + v8_st + r * 32) = vt[r];
  };

  float m = -__builtin_huge_valf();  // running reference maximum (log2 units)
  float l = 0.0f;                    // this lane's half of the row sum (rounded P)
  float lx = 0.0f;                   // fp8 with LSE: the same sum over unrounded P
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.0f;

  // Q has landed before the tile pipeline starts counting vector-memory ops.
  __builtin_amdgcn_s_waitcnt(vmcnt_le(0));

  const unsigned char *kb = nullptr, *vb = nullptr;
  int j = 0, rows = 0;
  if (cnt > 0) {
    tile(0, kb, vb, j, rows);
    issue_k(kb, rows);
    if (DT == 0) issue_v16(vb, rows); else load_v8(vb, rows);
  }

  for (int n = 0; n < cnt; ++n) {
    const int jn = j;
    // K_n has landed once only tile n's V loads can still be outstanding.
    __builtin_amdgcn_s_waitcnt(vmcnt_le(VLOADS));
    wg_barrier();

    // ---- S^T = K Q^T : 4 tiles of 32 keys x 32 queries per wave
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kt][v] = 0.0f;
    if (DT == 0) {
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        u32x4 af[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) af[kt] = lds16(Ks, k_rd[st & 3] + (st >> 2) * 128 + kt * 32 * KROW);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[kt]),
                                                             __builtin_bit_cast(bf16x8, qf[st]), sacc[kt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 b0 = qf[2 * st], b1 = qf[2 * st + 1];
        const i32x8 bf = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const u32x4 a0 = lds16(Ks, k_rd[2 * st] + kt * 32 * KROW);
          const u32x4 a1 = lds16(Ks, k_rd[2 * st + 1] + kt * 32 * KROW);
          const i32x8 af = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          sacc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, sacc[kt], 0, 0, 0, 0, 0, 0);
        }
      }
    }
    wg_barrier();  // every wave is done with K_n: its buffer takes K_{n+1}

    const bool more = n + 1 < cnt;
    if (more) {
      tile(n + 1, kb, vb, j, rows);
      issue_k(kb, rows);
    }
    if (DT == 1) store_v8();  // V_n: registers -> LDS (the buffer is free since P V of n-1)

    // ---- causal mask on the diagonal block (the last list entry)
    if (jn == i) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 32 * kt + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (kk > qq) sacc[kt][v] = -__builtin_huge_valf();
        }
    }

    // ---- online softmax with lazy rescale
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 16; v += 2) mx = max3(mx, sacc[kt][v], sacc[kt][v + 1]);
    mx = half_swap_max(mx) * c;
    const bool grow = mx > m + TAU;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = grow ? mx : m;
      const float al = __builtin_amdgcn_exp2f(m - mnew);
      l *= al;
      if (DT == 1 && LSE) lx *= al;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= al;
      m = mnew;
    }
    const float moff = m - SHIFT;

    // V_n has landed once only tile n+1's K loads can still be outstanding.
    if (DT == 0) {
      if (more) __builtin_amdgcn_s_waitcnt(vmcnt_le(KLOADS));
      else __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    }
    wg_barrier();

    // ---- O^T += V^T P^T, with P formed step by step right before its products.
    //      The row sum adds exactly the rounded values that enter the product.
    if (DT == 0) {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int kt = cc >> 1, t8 = (cc & 1) * 8;
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][t8 + e], c, -moff));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][t8 + e + 1], c, -moff));
          const bf16x2 pr = {(__bf16)p0, (__bf16)p1};
          pf[e] = pr[0];
          pf[e + 1] = pr[1];
          l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const unsigned off = v_rd[dt & 1] + (dt >> 1) * 128 + cc * 16 * KROW;
          const s16x4 t0 = lds_tr16(Vs, off);
          const s16x4 t1 = lds_tr16(Vs, off + 8 * KROW);
          const s16x8 af = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af), pf, o[dt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        i32x8 pf;
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) {
          const int kt = 2 * c2 + (q4 >> 2), v0 = (q4 & 3) * 4;
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kt][v0 + e], c, -moff));
          if (LSE) lx += (pv[0] + pv[1]) + (pv[2] + pv[3]);
          int wv = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
          wv = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], wv, true);
          pf[q4] = wv;
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(wv, false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(wv, true);
          l += (lo[0] + lo[1]) + (hi[0] + hi[1]);
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const unsigned off = v8_rd + c2 * 2 * kHeadDim * 32 + dt * 32 * 32;
          const u32x4 a0 = lds16(Vs, off);
          const u32x4 a1 = lds16(Vs, off + 16);
          const i32x8 af = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          o[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, pf, o[dt], 0, 0, 0, 0, 0, 0);
        }
      }
    }
    wg_barrier();  // every wave is done with V_n: its buffer takes V_{n+1}
    if (more) {
      if (DT == 0) issue_v16(vb, rows); else load_v8(vb, rows);
    }
  }

  // ---- epilogue: O = O^T / l, bf16 rows of 128 d per query
  const float lt = half_swap_sum(l);
  // LSE of the exact (unrounded) probabilities; fp8 P is rounded to e4m3 for the
  // product, so its normaliser lt differs from the exact sum by a few percent.
  const float lsum = (DT == 1 && LSE) ? half_swap_sum(lx) : lt;
  float inv = 1.0f / lt;
  if (DT == 1) inv *= a.v_scale[g];
  if (bad) inv = __builtin_nanf("");
  if (qvalid) {
    unsigned char* orow = (unsigned char*)a.out + ((sp.tok0 + tq) * a.o_st + (int64_t)h * a.o_sh) * 2;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        __attribute__((ext_vector_type(4))) __bf16 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(o[dt][4 * r + e] * inv);
        *(u32x2*)(orow + (32 * dt + 8 * r + 4 * hh) * 2) = __builtin_bit_cast(u32x2, ov);
      }
    if (LSE && hh == 0) {
      const float lse = bad ? __builtin_nanf("") : (m - SHIFT + __builtin_log2f(lsum)) * kLn2;
      a.lse[(int64_t)h * p.sd.total_tokens + sp.tok0 + tq] = lse;
    }
  }
}

template <int DT, bool PAGED, bool DENSE>
void launch_l(const AttnK& p, dim3 grid, hipStream_t st) {
  if (p.a.lse != nullptr)
    hipLaunchKernelGGL((attn_kernel<DT, PAGED, DENSE, true>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((attn_kernel<DT, PAGED, DENSE, false>), grid, dim3(kThreads), 0, st, p);
}

template <int DT, bool PAGED>
hipError_t launch_t(const AttnK& p, dim3 grid, hipStream_t st) {
  if (p.a.idx == nullptr) launch_l<DT, PAGED, true>(p, grid, st);
  else launch_l<DT, PAGED, false>(p, grid, st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnLaunch& a, const SeqDesc& sd, const PageDesc& pd, hipStream_t st) {
  AttnK p{a, sd, pd, a.hq / a.hkv};
  const int64_t n_wg = (int64_t)a.hq * sd.max_nb * sd.n_seqs;
  dim3 grid((unsigned)n_wg);
  const bool paged = pd.table != nullptr;
  if (a.dtype == 0) return paged ? launch_t<0, true>(p, grid, st) : launch_t<0, false>(p, grid, st);
  return paged ? launch_t<1, true>(p, grid, st) : launch_t<1, false>(p, grid, st);
}

}  // namespace fp
