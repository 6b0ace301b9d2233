// Causal GQA block-sparse flash attention over compacted block lists
// (FlashPrefill Method 3 "Index Compaction -> Physical Jumps": the inner loop
// walks only the listed key blocks; FlashPrefill V2 abstract: bf16 and FP8,
// paged KV cache, continuous batching).
//
// CDNA4 design (not the H20 one on the pages):
//   * one workgroup = one (query head, query block of 128 tokens), 4 waves,
//     each wave owns 32 query rows; two workgroups share a CU;
//   * the transposed products S^T = K Q^T and O^T = V^T P^T on
//     v_mfma_f32_32x32x16_bf16 (fp8 Q K^T: v_mfma_f32_32x32x64_f8f6f4), so every
//     lane owns ONE query column of S^T and of O^T: the softmax row max/sum
//     is in-lane plus one v_permlane32_swap, and the O rescale is in-lane;
//   * the S^T accumulator (keys 8i+4h+j of the lane's query) feeds the P^T
//     operand of the PV product directly: the contraction over keys only
//     needs V^T to list keys in the same slot order, so V is staged into LDS
//     already permuted and transposed (an 8x8 register transpose per thread),
//     and K is staged row-major with a 16-byte row pad;
//   * lists are ascending with the diagonal last, so only the last visited
//     block needs the causal mask;
//   * fp32 online softmax in exp2 units, P rounded to bf16 for the PV product on
//     both paths.  The fp8 path keeps Q K^T on the e4m3 MFMA and widens V from
//     e4m3 to bf16 while staging (exact); rounding P itself to e4m3 (3 mantissa
//     bits) puts up to 6% error on single weights, which breaks the fp8 error
//     bound on rows that attend to only a few keys.
#include "fp_device.h"

namespace fp {
namespace {

constexpr int kThreads = 256;
constexpr int kKPitch16 = 272;  // bf16 K row in LDS: 256 B + 16 B pad
constexpr int kKPitch8 = 144;   // fp8 K row in LDS: 128 B + 16 B pad
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnK {
  AttnLaunch a;
  SeqDesc sd;
  PageDesc pd;
  int group;
};

__device__ inline u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// 8x8 transpose of 16-bit elements: in[e] holds 8 consecutive d of key e;
// out[r] holds key 0..7 of d = r.
__device__ inline void transpose8x8_b16(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const unsigned sel = (r & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[r][q] = __builtin_amdgcn_perm(in[2 * q + 1][r >> 1], in[2 * q][r >> 1], sel);
  }
}

// 8 e4m3fn codes -> 8 bf16 (exact): decode to fp32 in hardware, keep the top halves.
__device__ inline u32x4 fp8x8_to_bf16x8(u32x2 v) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], true);
    r[2 * w] = __builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]), 0x07060302u);
    r[2 * w + 1] = __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]), 0x07060302u);
  }
  return r;
}

template <int DT, bool PAGED, bool DENSE>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnK p) {
  constexpr int KP = DT == 0 ? kKPitch16 : kKPitch8;
  constexpr int K_BYTES = kBlock * KP;
  constexpr int V_BYTES = kBlock * kHeadDim * 2;  // V is bf16 in LDS on both paths
  __shared__ __attribute__((aligned(16))) unsigned char smem[K_BYTES + V_BYTES];
  unsigned char* Ks = smem;
  unsigned char* Vs = smem + K_BYTES;
  constexpr int ES = DT == 0 ? 2 : 1;  // element size in bytes

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
  const int w = tid >> 6;
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

  float m = -__builtin_huge_valf();
  float l = 0.0f;
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.0f;

  int cnt;
  const int32_t* list = nullptr;
  if (DENSE) {
    cnt = i + 1;
  } else {
    cnt = a.counts[(int64_t)h * p.sd.total_blocks + sp.blk0 + i];
    cnt = cnt < 0 ? 0 : (cnt > i + 1 ? i + 1 : cnt);
    list = a.idx + (int64_t)h * p.sd.total_tri + sp.tri0 + (int64_t)i * (i + 1) / 2;
  }
  bool bad = cnt == 0;

  for (int n = 0; n < cnt; ++n) {
    const int j = DENSE ? n : list[n];
    if (j < 0 || j > i) { bad = true; continue; }
    const unsigned char* kb;
    const unsigned char* vb;
    if (PAGED) {
      const int page = p.pd.table[(int64_t)s * p.pd.max_pages + j];
      if (page < 0 || page >= p.pd.num_pages) { bad = true; continue; }
      kb = (const unsigned char*)a.k + ((int64_t)page * a.k_sp + (int64_t)g * a.k_sh) * ES;
      vb = (const unsigned char*)a.v + ((int64_t)page * a.v_sp + (int64_t)g * a.v_sh) * ES;
    } else {
      kb = (const unsigned char*)a.k + ((sp.tok0 + (int64_t)j * kBlock) * a.k_st + (int64_t)g * a.k_sh) * ES;
      vb = (const unsigned char*)a.v + ((sp.tok0 + (int64_t)j * kBlock) * a.v_st + (int64_t)g * a.v_sh) * ES;
    }
    const int rows = min(kBlock, sp.len - j * kBlock);  // valid key rows of block j

    __syncthreads();  // every wave is done reading the previous K/V tile
    if (DT == 0) {
      // K: row-major, 16 lanes per 256-byte row, 8 rows per thread
      u32x4 kr[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int row = (tid >> 4) + 16 * r;
        kr[r] = row < rows ? *(const u32x4*)(kb + (int64_t)row * a.k_st * 2 + (tid & 15) * 16) : zero4();
      }
      // V: thread (c, half, d-chunk) gathers the 8 keys of its operand slot group
      const int cc = tid >> 5, h2 = (tid >> 4) & 1, dc = tid & 15;
      u32x4 vr[8], vt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * cc + 8 * (e >> 2) + 4 * h2 + (e & 3);
        vr[e] = key < rows ? *(const u32x4*)(vb + (int64_t)key * a.v_st * 2 + dc * 16) : zero4();
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) *(u32x4*)(Ks + ((tid >> 4) + 16 * r) * KP + (tid & 15) * 16) = kr[r];
      transpose8x8_b16(vr, vt);
#pragma unroll
      for (int r = 0; r < 8; ++r) *(u32x4*)(Vs + (((cc * 2 + h2) * kHeadDim) + 8 * dc + r) * 16) = vt[r];
    } else {
      u32x4 kr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = (tid >> 3) + 32 * r;
        kr[r] = row < rows ? *(const u32x4*)(kb + (int64_t)row * a.k_st + (tid & 7) * 16) : zero4();
      }
      // V: same operand-slot gather as the bf16 path; e4m3 -> bf16 is exact (an e4m3
      // value has at most 4 significant bits, so the top half of its fp32 is it).
      const int cc = tid >> 5, h2 = (tid >> 4) & 1, dc = tid & 15;
      u32x2 vr8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * cc + 8 * (e >> 2) + 4 * h2 + (e & 3);
        vr8[e] = key < rows ? *(const u32x2*)(vb + (int64_t)key * a.v_st + dc * 8) : u32x2{0u, 0u};
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) *(u32x4*)(Ks + ((tid >> 3) + 32 * r) * KP + (tid & 7) * 16) = kr[r];
      u32x4 vr[8], vt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vr[e] = fp8x8_to_bf16x8(vr8[e]);
      transpose8x8_b16(vr, vt);
#pragma unroll
      for (int r = 0; r < 8; ++r) *(u32x4*)(Vs + (((cc * 2 + h2) * kHeadDim) + 8 * dc + r) * 16) = vt[r];
    }
    __syncthreads();

    // ---- S^T = K Q^T : 4 tiles of 32 keys x 32 queries per wave
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kt][v] = 0.0f;
      const unsigned char* kp = Ks + (32 * kt + ql) * KP;
      if (DT == 0) {
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const u32x4 af = *(const u32x4*)(kp + 32 * st + 16 * hh);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af),
                                                             __builtin_bit_cast(bf16x8, qf[st]), sacc[kt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 a0 = *(const u32x4*)(kp + 64 * st + 32 * hh);
          const u32x4 a1 = *(const u32x4*)(kp + 64 * st + 32 * hh + 16);
          const i32x8 af = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          const u32x4 b0 = qf[2 * st], b1 = qf[2 * st + 1];
          const i32x8 bf = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
          sacc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, sacc[kt], 0, 0, 0, 0, 0, 0);
        }
      }
    }

    // ---- causal mask on the diagonal block (the last list entry)
    if (j == i) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 32 * kt + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (kk > qq) sacc[kt][v] = -__builtin_huge_valf();
        }
    }

    // ---- online softmax (log2 units); each lane holds 64 of its query's 128 keys
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kt][v]);
    mx = half_swap_max(mx);
    const float mnew = fmaxf(m, mx * c);
    const float alpha = exp2f(m - mnew);
    const float moff = mnew;
    float rs = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = exp2f(fmaf(sacc[kt][v], c, -moff));
        sacc[kt][v] = pv;
        rs += pv;
      }
    l = l * alpha + rs;
    m = mnew;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;

    // ---- O^T += V^T P^T (bf16 P and V on both paths)
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int kt = cc >> 1, t8 = (cc & 1) * 8;
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (__bf16)sacc[kt][t8 + e];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const u32x4 af = *(const u32x4*)(Vs + (((cc * 2 + hh) * kHeadDim) + 32 * dt + ql) * 16);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af), pf, o[dt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = O^T / l, bf16 rows of 128 d per query
  const float lt = half_swap_sum(l);
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
    if (a.lse != nullptr && hh == 0) {
      const float lse = bad ? __builtin_nanf("") : (m + log2f(lt)) * kLn2;
      a.lse[(int64_t)h * p.sd.total_tokens + sp.tok0 + tq] = lse;
    }
  }
}

template <int DT, bool PAGED>
hipError_t launch_t(const AttnK& p, dim3 grid, hipStream_t st) {
  if (p.a.idx == nullptr)
    hipLaunchKernelGGL((attn_kernel<DT, PAGED, true>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((attn_kernel<DT, PAGED, false>), grid, dim3(kThreads), 0, st, p);
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
