// Causal GQA block-sparse flash attention over compacted block lists
// (FlashPrefill Method 3 "Index Compaction -> Physical Jumps": the inner loop
// walks only the listed key blocks; FlashPrefill V2 abstract: bf16 and FP8,
// paged KV cache, continuous batching).
//
// CDNA4 design (not the H20 one on the pages):
//   * one workgroup = one (query head, query block of 128 tokens), 4 waves of 32
//     query rows, two workgroups per CU (they take turns on the matrix cores the
//     way ping-pong warpgroups do on Hopper);
//   * the transposed products S^T = K Q^T and O^T = V^T P^T on
//     v_mfma_f32_32x32x16_bf16 (fp8: v_mfma_f32_32x32x64_f8f6f4), so every
//     lane owns ONE query column of S^T and of O^T: the softmax row max and sum
//     are in-lane plus one v_permlane32_swap, and the O rescale is in-lane;
//   * the S^T accumulator (keys 8i+4h+j of the lane's query) is the P^T
//     operand of the PV product as it stands: the contraction over keys only
//     needs V^T to list keys in the same slot order;
//   * each key block is handled as two halves of 64 keys.  A half (64 K rows and
//     64 V rows) goes HBM -> LDS with range-checked direct-to-LDS buffer loads (no
//     staging registers; rows past a sequence end read as zero) into one of two
//     LDS buffers that alternate, so the next half streams in while the current
//     one is computed; one wait and one barrier per half;
//   * LDS rows are unpadded; the 16-byte chunks of each row are permuted by an XOR
//     of the row index, chosen so the K operand reads (ds_read_b128) and the V^T
//     operand reads (ds_read_b64_tr_b16, fp8: ds_read_b64_tr_b8) touch every bank
//     at most once per cycle;
//   * lists are ascending with the diagonal last: only block i itself needs the
//     causal mask, and a list that does not end with i gives NaN rows;
//   * fp32 online softmax in exp2 units with a lazy rescale: O and the row sum
//     are rescaled only when the running maximum grows by more than TAU, so P
//     stays <= 2^TAU; the row sum adds the ROUNDED probabilities, i.e. exactly
//     the weights that enter P V, so output rows are true convex combinations;
//   * fp8: e4m3 Q K^T and P V (P rounded to e4m3 after a 2^4 range shift); the
//     row sum of the rounded P is one more matrix-core product (all-ones operand)
//     instead of VALU decodes and adds, and three workgroups share a CU.
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

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) int i32x2;

__device__ inline u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ inline float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// voff is per lane, soff wave-uniform (the instruction's scalar offset).
__device__ inline u32x4 bload16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff = 0) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ inline u32x2 bload8(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff = 0) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

// LDS operand reads (plain, transposing 16-bit, transposing 8-bit).
__device__ __attribute__((always_inline)) inline u32x4 lds16(const unsigned char* __restrict__ base, unsigned off) {
  return *(const u32x4*)(base + off);
}
__device__ __attribute__((always_inline)) inline s16x4 lds_tr16(const unsigned char* __restrict__ base, unsigned off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + off));
}
__device__ __attribute__((always_inline)) inline i32x2 lds_tr8(const unsigned char* __restrict__ base, unsigned off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(base + off));
}

// Modes (separate instances, so each workload has its own kernel):
//   kPrefill  per-head lists, one sequence, queries = keys;
//   kVarlen   the same over a packed batch of sequences (cu_seqlens), K/V packed
//             or paged;
//   kMasked   the logical-skip ablation (FlashPrefill Method 3 contrasts it with
//             physical jumps): the loop visits every causal block j <= i, tests
//             bit j of the row's block mask and branches past unselected blocks.
//             It cannot start the next selected block's loads before it has found
//             that block, so each selected block waits for its first half tile;
//   kGrouped  one list per KV group, read by every query head of the group;
//   kChunked  chunked / prefix-cached prefill: queries are the last positions of
//             each sequence, query blocks follow absolute positions.
enum { kPrefill = 0, kMasked = 1, kGrouped = 2, kChunked = 3, kVarlen = 4 };

// bf16: two workgroups per CU (<= 256 VGPRs); fp8: three (<= 168 VGPRs), which the
// fp8 loop needs to keep its matrix cores fed -- except with the LSE output, whose
// second (unrounded) row sum would not fit without spilling.
template <int DT, bool PAGED, bool DENSE, bool LSE, int MODE>
__global__ __launch_bounds__(kThreads, (DT == 0 || LSE) ? 2 : 3) void attn_kernel(AttnK p) {
  constexpr bool MASKED = MODE == kMasked;
  constexpr int ES = DT == 0 ? 2 : 1;             // element size in bytes
  constexpr int ROW = kHeadDim * ES;              // bytes of one K/V row: 256 (bf16), 128 (fp8)
  constexpr int CPR = ROW / 16;                   // 16-byte chunks per row
  constexpr int HT = 64 * ROW;                    // half tile (64 keys) of K or V: 16 KB / 8 KB
  constexpr int RPK = 1024 / ROW;                 // rows per 1 KB direct load of one wave
  constexpr int NI = HT / (1024 * 4);             // direct loads per wave per half tile: 4 / 2
  constexpr float TAU = DT == 0 ? 8.0f : 4.0f;    // lazy-rescale slack (log2 units)
  constexpr float SHIFT = DT == 0 ? 0.0f : 4.0f;  // fp8: P in (0, 2^(TAU+SHIFT)] = (0, 256]
  // Two (K, V) half-tile buffers.  They are separate LDS variables so that the
  // compiler can tell the direct loads filling one from the operand reads of the other.
  __shared__ __attribute__((aligned(1024))) unsigned char bufA[2 * HT];
  __shared__ __attribute__((aligned(1024))) unsigned char bufB[2 * HT];

  const AttnLaunch& a = p.a;
  // Work decode: query heads fastest so that consecutive workgroups share the
  // same query block, heaviest query blocks first.  Workgroup id % 8 is the XCD
  // (each with its own L2), so the heads an XCD receives should share K/V: with
  // hq % 8 == 0 each XCD takes a contiguous run of hq/8 heads (heads of one KV
  // group); otherwise, when the KV heads divide 8, each group goes to 8/hkv XCDs
  // that split its rows (else heads are dealt round robin).
  const int id = blockIdx.x;
  const int rows = p.sd.max_nq * p.sd.n_seqs;  // workgroups per query head
  int h, rest;
  if ((a.hq & 7) == 0) {
    const int per = a.hq >> 3;
    h = (id & 7) * per + ((id >> 3) % per);
    rest = id / a.hq;
  } else if (8 % a.hkv == 0 && rows % (8 / a.hkv) == 0) {
    const int xg = 8 / a.hkv, x = id & 7, k = id >> 3;
    h = (x / xg) * p.group + k % p.group;
    rest = (k / p.group) * xg + x % xg;
  } else {
    h = id % a.hq;
    rest = id / a.hq;
  }
  const int s = rest % p.sd.n_seqs;
  const int r = p.sd.max_nq - 1 - rest / p.sd.n_seqs;  // heaviest query blocks first
  SeqPos sp = seq_pos(p.sd, s);
  if (MODE != kChunked) {  // queries = keys: let the compiler drop the offset arithmetic
    sp.qtok0 = sp.tok0; sp.qlen = sp.len; sp.qoff = 0; sp.I0 = 0; sp.qblk0 = sp.blk0;
  }
  if (r < 0 || r >= sp.nq || sp.qblk0 + r >= p.sd.total_qblocks) return;
  // query block r of the sequence is absolute block i: its rows are positions
  // 128i .. 128i+127, of which the query chunk holds [qoff, qoff + qlen)
  const int i = sp.I0 + r;
  const int g = h / p.group;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int ql = lane & 31;
  const int hh = lane >> 5;
  const int qq = 32 * w + ql;  // query row within the block (= position - 128i)
  const int tq = i * kBlock + qq - sp.qoff;  // index of the row in the query chunk
  const bool qvalid = tq >= 0 && tq < sp.qlen;

  // ---- Q fragments (B operand of S^T = K Q^T): lane = query column, 8 (bf16) or
  //      32 (fp8) consecutive d per MFMA step, half hh takes the upper part.
  // The resource starts at the block's first row the chunk holds (row qs0 of the
  // block); rows before it (negative offsets wrap) and past the chunk end are out
  // of range and read as zero.
  const int qs0 = max(0, sp.qoff - i * kBlock);
  const int qrows = min(kBlock, sp.qoff + sp.qlen - i * kBlock) - qs0;
  const unsigned qst = (unsigned)(a.q_st * ES);
  const __amdgpu_buffer_rsrc_t qr =
      rsrc((const unsigned char*)a.q + ((sp.qtok0 + (int64_t)i * kBlock + qs0 - sp.qoff) * a.q_st +
                                        (int64_t)h * a.q_sh) * ES, qrows * qst);
  const unsigned qro = (unsigned)(qq - qs0) * qst;
  u32x4 qf[DT == 0 ? 8 : 4];
  if (DT == 0) {
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = bload16(qr, qro + (16 * st + 8 * hh) * 2);
  } else {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      qf[2 * st] = bload16(qr, qro + 64 * st + 32 * hh);
      qf[2 * st + 1] = bload16(qr, qro + 64 * st + 32 * hh + 16);
    }
  }

  float c = a.softmax_scale * kLog2e;  // logits -> log2 units
  if (DT == 1) c *= a.q_scale[h] * a.k_scale[g];

  // list entries are wave-uniform: read them through the constant address space
  // so they become scalar loads.
  typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
  int cnt;
  cint_ptr list = nullptr;
  if (DENSE || MASKED) {
    cnt = i + 1;
  } else {
    const int hl = MODE == kGrouped ? h / a.list_div : h;  // the list this head reads
    cnt = ((cint_ptr)a.counts)[(int64_t)hl * p.sd.total_qblocks + sp.qblk0 + r];
    cnt = uniform(cnt < 0 ? 0 : (cnt > i + 1 ? i + 1 : cnt));
    // rows I0 .. i-1 of the sequence hold I0+1 .. i slots
    list = (cint_ptr)(a.idx + (int64_t)hl * p.sd.total_tri + sp.tri0 + (int64_t)r * (sp.I0 + 1) +
                      (int64_t)r * (r - 1) / 2);
  }
  bool bad = cnt == 0;

  // ---- LDS half tiles: 64 K rows then 64 V rows of ROW bytes, unpadded, with the
  //      16-byte chunks of every row permuted by an XOR of the row index (swz_k /
  //      swz_v) so that each operand read below touches every LDS bank at most once
  //      per cycle.
  auto swz_k = [](int r) -> int { return DT == 0 ? (r & 15) : ((r >> 1) & 7); };
  auto swz_v = [](int r) -> int { return DT == 0 ? 4 * (r & 3) : 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1); };

  // ---- direct HBM -> LDS loads of a half tile.  Load u of wave w fills the 1 KB
  //      at (4u + w) KB of the half: rows RPK*(4u + w) + lane/CPR, physical chunk
  //      lane%CPR, which holds logical chunk (lane%CPR) ^ swz(row).  The swizzles only
  //      depend on the lane and on w, so each lane's offset within the 1 KB is the
  //      same for every u and both halves.  Rows past the sequence end read as zero
  //      (range check of the buffer resource).
  const unsigned kst = (unsigned)(a.k_st * ES), vst = (unsigned)(a.v_st * ES);  // token strides, bytes
  unsigned k_off, v_off;
  {
    const int r0 = RPK * w + lane / CPR;  // row of load u = 0; load u adds 4*RPK rows
    k_off = (lane / CPR) * kst + (((lane % CPR) ^ swz_k(r0)) * 16);
    v_off = (lane / CPR) * vst + (((lane % CPR) ^ swz_v(r0)) * 16);
  }
  auto entry = [&](int n) -> int { return DENSE ? n : uniform(list[n]); };
  auto load_half = [&](int j, int hf, unsigned char* buf) {
    if (j < 0 || j > i) { bad = true; j = 0; }
    const unsigned char *kb, *vb;
    if (PAGED) {
      int page = uniform(((cint_ptr)p.pd.table)[(int64_t)s * p.pd.max_pages + j]);
      if (page < 0 || page >= p.pd.num_pages) { bad = true; page = 0; }
      kb = (const unsigned char*)a.k + ((int64_t)page * a.k_sp + (int64_t)g * a.k_sh) * ES;
      vb = (const unsigned char*)a.v + ((int64_t)page * a.v_sp + (int64_t)g * a.v_sh) * ES;
    } else {
      kb = (const unsigned char*)a.k + ((sp.tok0 + (int64_t)j * kBlock) * a.k_st + (int64_t)g * a.k_sh) * ES;
      vb = (const unsigned char*)a.v + ((sp.tok0 + (int64_t)j * kBlock) * a.v_st + (int64_t)g * a.v_sh) * ES;
    }
    const int rows = min(kBlock, sp.len - j * kBlock);
    const __amdgpu_buffer_rsrc_t rk = rsrc(kb, rows * kst);
    const __amdgpu_buffer_rsrc_t rv = rsrc(vb, rows * vst);
#pragma unroll
    for (int u = 0; u < NI; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(buf + (4 * u + w) * 1024), 16, k_off,
                                              uniform((64 * hf + RPK * (4 * u + w)) * kst), 0, 0);
#pragma unroll
    for (int u = 0; u < NI; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(buf + HT + (4 * u + w) * 1024), 16, v_off,
                                              uniform((64 * hf + RPK * (4 * u + w)) * vst), 0, 0);
  };

  // ---- operand read offsets (per lane, loop invariant; rows that differ by a
  //      multiple of 16 share a swizzle, so row-block steps are immediates)
  // K operand of step st (bf16: 8 steps of 16 d, fp8: 2 steps of 64 d as 2 x 16 B)
  unsigned k_rd[DT == 0 ? 8 : 4];
  {
    const int r = ql;
    if (DT == 0) {
#pragma unroll
      for (int st = 0; st < 8; ++st) k_rd[st] = r * ROW + (((2 * st + hh) ^ swz_k(r)) * 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) k_rd[e] = r * ROW + (((4 * (e >> 1) + 2 * hh + (e & 1)) ^ swz_k(r)) * 16);
    }
  }
  // V^T operands: bf16 through ds_read_b64_tr_b16 (per 16-lane group G: rows
  // 4hh + sl/4, 8 bytes at d = 32dt + 16(G&1) + 4(sl&3)); fp8 through
  // ds_read_b64_tr_b8: within a 16-lane group, lane i receives byte i&7 of source
  // lanes 2r + i/8 (r = 0..7); source lanes 2r and 2r+1 point at the same key row, at
  // d0 and d0 + 8, so lane i gets d0 + i for 8 keys.  Byte slot e = 8q + r of half
  // hh holds key 16q + 8(r/4) + 4hh + r%4 (the P^T operand order), i.e. source lane
  // s reads key row 16q + 8(s/8) + 4hh + (s/2)%4.
  unsigned v_rd[4];
  {
    const int G = lane >> 4, sl = lane & 15;
    if (DT == 0) {
      const int r = 4 * hh + (sl >> 2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        v_rd[dt] = HT + r * ROW + (((4 * dt + 2 * (G & 1) + ((sl & 3) >> 1)) ^ swz_v(r)) * 16) + 8 * (sl & 1);
    } else {
      const int r = 8 * (sl >> 3) + 4 * hh + ((sl >> 1) & 3);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        v_rd[dt] = HT + r * ROW + (((2 * dt + (G & 1)) ^ swz_v(r)) * 16) + 8 * (sl & 1);
    }
  }

  // S^T = K Q^T for the 64 keys of the half tile: 2 tiles of 32 keys x 32
  // queries.  The K operands of step st+2 are read while step st's products run, so
  // every MFMA finds its LDS operand already in registers.
  auto qk = [&](f32x16 (&sacc)[2], const unsigned char* buf) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[t][v] = 0.0f;
    if (DT == 0) {
      u32x4 af[3][2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t) af[st][t] = lds16(buf, k_rd[st] + t * 32 * ROW);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st + 2 < 8) {
#pragma unroll
          for (int t = 0; t < 2; ++t) af[(st + 2) % 3][t] = lds16(buf, k_rd[st + 2] + t * 32 * ROW);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[st % 3][t]),
                                                            __builtin_bit_cast(bf16x8, qf[st]), sacc[t], 0, 0, 0);
      }
      // keep the operand reads two steps ahead of their products: 4 reads, then
      // alternate product / read (the scheduler would otherwise sink each read to
      // its product and wait out the full LDS latency every time)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k < 12; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    } else {
      u32x4 a0[2][2], a1[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          a0[st][t] = lds16(buf, k_rd[2 * st] + t * 32 * ROW);
          a1[st][t] = lds16(buf, k_rd[2 * st + 1] + t * 32 * ROW);
        }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 b0 = qf[2 * st], b1 = qf[2 * st + 1];
        const i32x8 bf = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 x0 = a0[st][t], x1 = a1[st][t];
          const i32x8 af = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
          sacc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, sacc[t], 0, 0, 0, 0, 0, 0);
        }
      }
    }
  };

  float m = -__builtin_huge_valf();  // running reference maximum (log2 units)
  float l = 0.0f;                    // this lane's half of the row sum (rounded P)
  float lx = 0.0f;                   // fp8 with LSE: the same sum over unrounded P
  // fp8: the row sum of the rounded P runs on the matrix core, as an all-ones A
  // operand against the P^T operand: every row of this accumulator is the sum over
  // keys for the lane's query column (replaces a decode and four adds per 4 keys).
  f32x16 lacc;
#pragma unroll
  for (int v = 0; v < 16; ++v) lacc[v] = 0.0f;
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.0f;

  // online softmax of this wave's 64 keys of S^T (masked if the tile is the
  // diagonal block) and O^T += V^T P^T with the V tile in LDS; P is formed step by
  // step right before its products and the row sum adds exactly the rounded values
  // that enter the product.
  auto softmax_pv = [&](f32x16 (&sacc)[2], int half, bool diag, const unsigned char* buf) {
    if (diag) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 32 * (2 * half + t) + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (kk > qq) sacc[t][v] = -__builtin_huge_valf();
        }
    }
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; v += 2) mx = max3(mx, sacc[t][v], sacc[t][v + 1]);
    mx = half_swap_max(mx) * c;
    const bool grow = mx > m + TAU;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = grow ? mx : m;
      const float al = __builtin_amdgcn_exp2f(m - mnew);
      l *= al;
      if (DT == 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) lacc[v] *= al;
      }
      if (DT == 1 && LSE) lx *= al;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= al;
      m = mnew;
    }
    const float moff = m - SHIFT;
    if (DT == 0) {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      // V^T operands of step c4+1 are read while step c4's products run
      s16x4 vt[2][4][2];
      auto vread = [&](int vb, int cc) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const unsigned off = v_rd[dt] + cc * 16 * ROW;
          vt[vb][dt][0] = lds_tr16(buf, off);
          vt[vb][dt][1] = lds_tr16(buf, off + 8 * ROW);
        }
      };
      vread(0, 0);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int t = c4 >> 1, t8 = (c4 & 1) * 8;
        if (c4 + 1 < 4) vread((c4 + 1) & 1, c4 + 1);
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[t][t8 + e], c, -moff));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[t][t8 + e + 1], c, -moff));
          const bf16x2 pr = {(__bf16)p0, (__bf16)p1};
          pf[e] = pr[0];
          pf[e + 1] = pr[1];
          l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 t0 = vt[c4 & 1][dt][0], t1 = vt[c4 & 1][dt][1];
          const s16x8 af = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af), pf, o[dt], 0, 0, 0);
        }
      }
    } else {
      // one 64-key P^T operand: byte e of half hh <-> key 64*half + 32*(e/16) + 8*((e%16)/4) + 4*hh + e%4
      i32x8 pf;
#pragma unroll
      for (int q4 = 0; q4 < 8; ++q4) {
        const int t = q4 >> 2, v0 = (q4 & 3) * 4;
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[t][v0 + e], c, -moff));
        if (LSE) lx += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        // the first conversion writes the low half of pv[0]'s own register (dead
        // afterwards), so no register has to be cleared first
        int wv = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], __float_as_int(pv[0]), false);
        wv = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], wv, true);
        pf[q4] = wv;
      }
      {
        const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                            0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0
        lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        i32x8 af;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x2 t = lds_tr8(buf, v_rd[dt] + 16 * q * ROW);
          af[2 * q] = t[0];
          af[2 * q + 1] = t[1];
        }
        o[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, pf, o[dt], 0, 0, 0, 0, 0, 0);
      }
    }
  };

  // ---- pipeline over half tiles.  Half tile (n, 0) sits in buffer A, (n, 1) in
  //      buffer B.  Each half step waits for its own direct loads, meets the other
  //      waves at the barrier (past it the half tile is complete and every wave has
  //      finished the previous half step, i.e. released the other buffer), starts
  //      the direct loads of the next half tile into the other buffer and computes
  //      while they fly.  The block id of the next entry is fetched a tile early, so
  //      the scalar load's latency never sits in front of the tile loads.
  f32x16 s0[2];
  if (MASKED) {
    typedef const __attribute__((address_space(4))) uint32_t* cu32_ptr;
    const cu32_ptr mrow = (cu32_ptr)(a.mask + ((int64_t)h * sp.nq + r) * a.mask_words);
    unsigned word = 0;
    int visited = 0;
    for (int j = 0; j <= i; ++j) {
      if ((j & 31) == 0) word = uniform(mrow[j >> 5]);
      if (((word >> (j & 31)) & 1u) == 0) continue;  // logical skip
      ++visited;
      load_half(j, 0, bufA);
      __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
      wg_barrier();  // half 0 in; every wave is done with the previous block's half 1
      load_half(j, 1, bufB);
      qk(s0, bufA);
      softmax_pv(s0, 0, j == i, bufA);
      __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
      wg_barrier();  // half 1 in; every wave is done with half 0
      qk(s0, bufB);
      softmax_pv(s0, 1, j == i, bufB);
    }
    bad = visited == 0;
  } else if (cnt > 0) {
    int jc = entry(0);
    int jn = entry(min(1, cnt - 1));
    load_half(jc, 0, bufA);
    for (int n = 0; n < cnt; ++n) {
      // the causal mask belongs to block i itself; a list must end with it, so a
      // last entry other than i makes the row NaN instead of mis-masking it
      const bool diag = jc == i;
      if (n + 1 == cnt && !diag) bad = true;
      __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
      wg_barrier();
      load_half(jc, 1, bufB);
      qk(s0, bufA);
      softmax_pv(s0, 0, diag, bufA);
      __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
      wg_barrier();
      if (n + 1 < cnt) load_half(jn, 0, bufA);
      jc = jn;
      jn = entry(min(n + 2, cnt - 1));
      qk(s0, bufB);
      softmax_pv(s0, 1, diag, bufB);
    }
  }

  // ---- epilogue: O = O^T / l, bf16 rows of 128 d per query
  const float lt = DT == 1 ? lacc[0] : half_swap_sum(l);
  // LSE of the exact (unrounded) probabilities; fp8 P is rounded to e4m3 for the
  // product, so its normaliser lt differs from the exact sum by a few percent.
  const float lsum = (DT == 1 && LSE) ? half_swap_sum(lx) : lt;
  float inv = 1.0f / lt;
  if (DT == 1) inv *= a.v_scale[g];
  if (bad) inv = __builtin_nanf("");
  if (qvalid) {
    unsigned char* orow = (unsigned char*)a.out + ((sp.qtok0 + tq) * a.o_st + (int64_t)h * a.o_sh) * 2;
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
      a.lse[(int64_t)h * p.sd.total_qtokens + sp.qtok0 + tq] = lse;
    }
  }
}

template <int DT, bool PAGED, bool DENSE, int MODE>
void launch_l(const AttnK& p, dim3 grid, hipStream_t st) {
  if (p.a.lse != nullptr)
    hipLaunchKernelGGL((attn_kernel<DT, PAGED, DENSE, true, MODE>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((attn_kernel<DT, PAGED, DENSE, false, MODE>), grid, dim3(kThreads), 0, st, p);
}

template <int DT, bool PAGED, int MODE>
void launch_t(const AttnK& p, dim3 grid, hipStream_t st) {
  if (p.a.idx == nullptr) launch_l<DT, PAGED, true, MODE>(p, grid, st);
  else launch_l<DT, PAGED, false, MODE>(p, grid, st);
}

template <int DT>
void launch_dt(const AttnK& p, const PageDesc& pd, dim3 grid, hipStream_t st) {
  const bool paged = pd.table != nullptr;
  if (p.a.mask != nullptr) launch_l<DT, false, false, kMasked>(p, grid, st);
  else if (p.a.list_div > 1) launch_l<DT, false, false, kGrouped>(p, grid, st);
  else if (p.sd.cu_seqlens_q != nullptr) {
    if (paged) launch_t<DT, true, kChunked>(p, grid, st);
    else launch_t<DT, false, kChunked>(p, grid, st);
  } else if (p.sd.cu_seqlens != nullptr) {
    if (paged) launch_t<DT, true, kVarlen>(p, grid, st);
    else launch_t<DT, false, kVarlen>(p, grid, st);
  } else {
    launch_t<DT, false, kPrefill>(p, grid, st);
  }
}

}  // namespace

hipError_t launch_attn(const AttnLaunch& a, const SeqDesc& sd, const PageDesc& pd, hipStream_t st) {
  AttnK p{a, sd, pd, a.hq / a.hkv};
  const int64_t n_wg = (int64_t)a.hq * sd.max_nq * sd.n_seqs;
  dim3 grid((unsigned)n_wg);
  if (a.dtype == 0) launch_dt<0>(p, pd, grid, st);
  else launch_dt<1>(p, pd, grid, st);
  return hipGetLastError();
}

}  // namespace fp
