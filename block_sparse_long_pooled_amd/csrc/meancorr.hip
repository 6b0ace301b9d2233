// V2 mean correction, as a switchable assumption.  The FlashPrefill V2 abstract
// mentions a mean-based correction that reduces the error of the sparse
// approximation, without a formula.  Reading implemented here: every causal key
// block that the list of (h, i) prunes still enters the softmax, as n_j = 128
// copies of its mean key kbar_j carrying its mean value vbar_j.  The pass runs
// after the sparse attention and folds the pruned blocks into its result:
//
//   O' = (Z O + sum_j n_j e^{s_j} vbar_j) / (Z + sum_j n_j e^{s_j}),
//   s_j = scale * q . kbar_j,  Z = e^{LSE},  LSE' = log(Z + sum_j n_j e^{s_j}).
//
// This is an attention of the block's 128 queries over the pooled keys j < i with
// a per-row key mask (pruned = not listed) and a log(128) bias, started from the
// sparse result: the online-softmax state begins at reference m = LSE, mass 1 and
// accumulator O.  Two kernels:
//   - meanprep_kernel converts the fp64 means once per (KV head, tile of 32 pooled
//     keys) into a 24 KB tile image in the caller's workspace: Kbar as two bf16
//     terms (hi = bf16(kbar), lo = bf16(kbar - hi), so logits carry ~2^-17 relative
//     error, like fp32 dot products of the fp64 means; a single bf16 term would put
//     ~2^-9 on logits of magnitude ~20) in rows with their 16-byte chunks permuted
//     by an XOR of the row, and Vbar in bf16 transposed to [dim][key] with the keys
//     of each 16-key step in the order of the S^T accumulator.  The image is the
//     LDS layout byte for byte, so it moves with direct-to-LDS loads and every
//     operand is one conflict-free 16-byte LDS read;
//   - meancorr_kernel: one workgroup per (query head, query block), 4 waves x 32
//     query rows, on v_mfma_f32_32x32x16_bf16.  The list of (h, i) becomes a bit mask
//     in LDS (bit j of word j/32), so a tile is one mask word and tiles with nothing
//     pruned are skipped; the next pruned tile streams into the other LDS buffer while
//     the current one is computed.  S^T = (Kbar_hi + Kbar_lo) Q^T, O^T += Vbar^T P^T
//     with P rounded to bf16 (the correction term carries ~2^-8 relative error); the
//     row mass adds the unrounded P.
#include <mutex>

#include "fp_device.h"

namespace fp {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;                       // pooled keys per tile = one mask word
constexpr int kTileBytes = 3 * kTile * 256;     // hi, lo (32 rows x 256 B), V^T (128 rows x 64 B)
constexpr int kMaxBlocks = 65536;               // mask of one row: 8 KB of LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2n = 7.0f;                  // log2(128): every pruned block lies below the diagonal and is full

typedef __attribute__((ext_vector_type(2))) double f64x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;

__device__ inline unsigned short bf16_bits(float x) { return __builtin_bit_cast(unsigned short, (__bf16)x); }

// Slot of a key inside a 16-key step of the V^T image.  The P^T operand of step kst
// takes accumulator elements v = 8 kst + e, which hold key 8(v/4) + 4hh + v%4 of the
// 32-key tile, so slot 8hh + e of step kst must hold key 16 kst + 8(e/4) + 4hh + e%4;
// inverted for k16 = key % 16: slot = 8((k16/4)%2) + 4(k16/8) + k16%4.
__device__ inline int vt_slot(int k16) { return 8 * ((k16 >> 2) & 1) + 4 * (k16 >> 3) + (k16 & 3); }

// Byte offsets inside a tile image.
__device__ inline unsigned k_pos(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) * 16); }
__device__ inline unsigned vt_pos(int d, int chunk) { return 2 * kTile * 256 + d * 64 + ((chunk ^ ((d >> 2) & 3)) * 16); }

// First tile image of sequence s: sum over the sequences before it of ceil(nb / 32)
// (every lane strides the sequences, then a butterfly sum, as seq_pos does).
__device__ inline int64_t tile_base(const SeqDesc& sd, int s) {
  if (sd.cu_seqlens == nullptr) return 0;
  int64_t acc = 0;
  for (int r = (int)(threadIdx.x & 63); r < s; r += 64) {
    int n = sd.cu_seqlens[r + 1] - sd.cu_seqlens[r];
    n = n < 0 ? 0 : n;
    const int nb = (n + kBlock - 1) / kBlock;
    acc += (nb + kTile - 1) / kTile;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  return uniform64(acc);
}

__global__ __launch_bounds__(kThreads) void meanprep_kernel(MeanCorrLaunch a) {
  const int J = blockIdx.x, s = blockIdx.y, g = blockIdx.z;
  const int tid = threadIdx.x;
  const SeqPos sp = seq_pos(a.sd, s);
  const int nb = (sp.len + kBlock - 1) / kBlock;
  if (kTile * J >= nb) return;
  const int nk = min(kTile, nb - kTile * J);
  unsigned char* img = (unsigned char*)a.workspace + ((int64_t)g * a.total_tiles + tile_base(a.sd, s) + J) * kTileBytes;
  const double* kbar = a.pooled_k + ((int64_t)g * a.sd.total_blocks + sp.blk0 + kTile * J) * kHeadDim;
  const double* vbar = a.pooled_v + ((int64_t)g * a.sd.total_blocks + sp.blk0 + kTile * J) * kHeadDim;
  {  // Kbar row kr, dims 16dc .. +15 -> hi/lo (rows past nb are zero)
    const int kr = tid >> 3, dc = tid & 7;
    const f64x2* src = (const f64x2*)(kbar + kr * kHeadDim + 16 * dc);
    unsigned hw[8], lw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f64x2 x = kr < nk ? src[u] : f64x2{0.0, 0.0};
      unsigned short hs[2], ls[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const __bf16 hi = (__bf16)(float)x[e];
        hs[e] = __builtin_bit_cast(unsigned short, hi);
        ls[e] = bf16_bits((float)(x[e] - (double)(float)hi));
      }
      hw[u] = hs[0] | ((unsigned)hs[1] << 16);
      lw[u] = ls[0] | ((unsigned)ls[1] << 16);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const unsigned off = k_pos(kr, 2 * dc + c);
      *(u32x4*)(img + off) = u32x4{hw[4 * c], hw[4 * c + 1], hw[4 * c + 2], hw[4 * c + 3]};
      *(u32x4*)(img + kTile * 256 + off) = u32x4{lw[4 * c], lw[4 * c + 1], lw[4 * c + 2], lw[4 * c + 3]};
    }
  }
  {  // Vbar keys 2kp, 2kp+1 (adjacent slots), dims 8dg .. +7 -> bf16 V^T
    const int kp = tid & 15, dg = tid >> 4;
    const int k0 = 2 * kp;
    const f64x2* s0 = (const f64x2*)(vbar + k0 * kHeadDim + 8 * dg);
    const f64x2* s1 = (const f64x2*)(vbar + (k0 + 1) * kHeadDim + 8 * dg);
    const int sl = vt_slot(k0 & 15);
    const int chunk = 2 * (k0 >> 4) + (sl >> 3);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f64x2 x0 = k0 < nk ? s0[u] : f64x2{0.0, 0.0};
      const f64x2 x1 = k0 + 1 < nk ? s1[u] : f64x2{0.0, 0.0};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int d = 8 * dg + 2 * u + e;
        *(unsigned*)(img + vt_pos(d, chunk) + (sl & 7) * 2) =
            bf16_bits((float)x0[e]) | ((unsigned)bf16_bits((float)x1[e]) << 16);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void meancorr_kernel(MeanCorrLaunch a) {
  const int id = blockIdx.x;
  const int h = id % a.hq;
  const int rest = id / a.hq;
  const int s = rest % a.sd.n_seqs;
  const int i = a.sd.max_nb - 1 - rest / a.sd.n_seqs;  // longest rows first
  if (i <= 0) return;                                  // block 0 has nothing below the diagonal
  const SeqPos sp = seq_pos(a.sd, s);
  if (i * kBlock >= sp.len) return;
  const int g = h / (a.hq / a.hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ql = lane & 31, hh = lane >> 5;
  const int64_t tl = (int64_t)i * kBlock + 32 * w + ql;  // this lane's query within the sequence
  const bool valid = tl < sp.len;
  const int64_t t = sp.tok0 + tl;                          // ... and in the packed batch
  const int nw = (i + kTile - 1) / kTile;  // tiles of keys j < i

  extern __shared__ unsigned listed[];  // nw words
  __shared__ __attribute__((aligned(1024))) unsigned char bufA[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char bufB[kTileBytes];

  // ---- listed blocks of (h, i) as a bit mask
  for (int u = tid; u < nw; u += kThreads) listed[u] = 0u;
  __syncthreads();
  int cnt = ((cint_ptr)a.counts)[(int64_t)h * a.sd.total_blocks + sp.blk0 + i];
  cnt = cnt < 0 ? 0 : (cnt > i + 1 ? i + 1 : cnt);
  const int32_t* list = a.idx + (int64_t)h * a.sd.total_tri + sp.tri0 + (int64_t)i * (i + 1) / 2;
  for (int e = tid; e < cnt; e += kThreads) {
    const int j = list[e];
    if (j >= 0 && j < i) atomicOr(&listed[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  auto pruned_of = [&](int J) -> unsigned {
    const int nk = min(kTile, i - kTile * J);
    const unsigned inrange = nk == kTile ? 0xffffffffu : ((1u << nk) - 1u);
    return (unsigned)uniform((int)(~listed[J] & inrange));
  };
  auto next_tile = [&](int J) -> int {  // first tile after J with a pruned key, or -1
    for (++J; J < nw; ++J)
      if (pruned_of(J) != 0u) return J;
    return -1;
  };
  const int first = next_tile(-1);
  if (first < 0) return;  // nothing pruned: output and LSE stay bit-identical

  // ---- direct loads of a tile image: load u of wave w fills KB 4u + w
  const int ntiles = ((sp.len + kBlock - 1) / kBlock + kTile - 1) / kTile;  // this sequence's tile images
  const __amdgpu_buffer_rsrc_t rws =
      rsrc((const unsigned char*)a.workspace + ((int64_t)g * a.total_tiles + tile_base(a.sd, s)) * kTileBytes,
           (unsigned)(ntiles * kTileBytes));
  auto load_tile = [&](int J, unsigned char* buf) {
#pragma unroll
    for (int u = 0; u < kTileBytes / 4096; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rws, (lds_void_t*)(buf + (4 * u + w) * 1024), 16, lane * 16,
                                              uniform(J * kTileBytes + (4 * u + w) * 1024), 0, 0);
  };
  load_tile(first, bufA);

  // ---- Q^T operand of this lane (bf16; fp8 codes are exact in bf16, the
  //      per-head scale goes into the logit scale)
  u32x4 qf[8];
  if (valid) {
    if (a.dtype == 0) {
      const unsigned char* src = (const unsigned char*)a.q + (t * a.q_st + (int64_t)h * a.q_sh) * 2;
#pragma unroll
      for (int st = 0; st < 8; ++st) qf[st] = *(const u32x4*)(src + (16 * st + 8 * hh) * 2);
    } else {
      const unsigned char* src = (const unsigned char*)a.q + t * a.q_st + (int64_t)h * a.q_sh;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x2 c8 = *(const u32x2*)(src + 16 * st + 8 * hh);
        unsigned wds[4];
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c8[hw], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c8[hw], true);
          wds[2 * hw] = bf16_bits(lo[0]) | ((unsigned)bf16_bits(lo[1]) << 16);
          wds[2 * hw + 1] = bf16_bits(hi[0]) | ((unsigned)bf16_bits(hi[1]) << 16);
        }
        qf[st] = u32x4{wds[0], wds[1], wds[2], wds[3]};
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = u32x4{0u, 0u, 0u, 0u};
  }
  const float c2 = a.softmax_scale * (a.dtype == 1 ? a.q_scale[h] : 1.0f) * kLog2e;

  // ---- state of the sparse result: reference m = LSE (log2 units), mass 1 (held by
  //      the hh = 0 lane of the pair), accumulator = O.  Lane (ql, hh) holds
  //      O^T[d][q] at d = 32dt + 8(v/4) + 4hh + v%4, the layout of the products.
  float m = 0.0f, l = hh == 0 ? 1.0f : 0.0f;
  f32x16 o[4];
  unsigned char* orow = (unsigned char*)a.out + (t * a.o_st + (int64_t)h * a.o_sh) * 2;
  if (valid) {
    m = a.lse[(int64_t)h * a.sd.total_tokens + t] * kLog2e;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bf16x4 ov = __builtin_bit_cast(bf16x4, *(const u32x2*)(orow + (32 * dt + 8 * r + 4 * hh) * 2));
#pragma unroll
        for (int e = 0; e < 4; ++e) o[dt][4 * r + e] = (float)ov[e];
      }
  } else {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[dt][v] = 0.0f;
  }

  auto compute = [&](int J, const unsigned char* buf) {
    const unsigned pruned = pruned_of(J);
    // S^T = (Kbar_hi + Kbar_lo) Q^T: 32 keys x 32 queries
    f32x16 s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = 0.0f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const unsigned off = k_pos(ql, 2 * st + hh);
      const bf16x8 b = __builtin_bit_cast(bf16x8, qf[st]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, *(const u32x4*)(buf + off)), b, s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, *(const u32x4*)(buf + kTile * 256 + off)), b, s, 0, 0, 0);
    }
    // logits in log2 units with the log2(128) copies; listed keys and keys >= i drop out
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = 8 * (v >> 2) + 4 * hh + (v & 3);
      s[v] = ((pruned >> key) & 1u) ? fmaf(s[v], c2, kLog2n) : -__builtin_huge_valf();
      mx = fmaxf(mx, s[v]);
    }
    mx = half_swap_max(mx);
    if (mx > m) {
      const float al = __builtin_amdgcn_exp2f(m - mx);
      l *= al;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= al;
      m = mx;
    }
    // O^T += Vbar^T P^T, two 16-key steps
#pragma unroll
    for (int kst = 0; kst < 2; ++kst) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = __builtin_amdgcn_exp2f(s[8 * kst + e] - m);
        l += pv;
        pf[e] = (__bf16)pv;
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const u32x4 av = *(const u32x4*)(buf + vt_pos(32 * dt + ql, 2 * kst + hh));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pf, o[dt], 0, 0, 0);
      }
    }
  };

  // ---- pipeline: tile jc sits in buffer A, the next pruned tile streams into B
  //      while jc is computed, and the roles swap.  Each step waits for its own
  //      direct loads and meets the other waves at the barrier (past it the tile is
  //      complete and every wave is done with the other buffer).
  int jc = first;
  while (true) {
    const int jn = next_tile(jc);
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    wg_barrier();
    if (jn >= 0) load_tile(jn, bufB);
    compute(jc, bufA);
    if (jn < 0) break;
    const int jn2 = next_tile(jn);
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    wg_barrier();
    if (jn2 >= 0) load_tile(jn2, bufA);
    compute(jn, bufB);
    if (jn2 < 0) break;
    jc = jn2;
  }
  if (!valid) return;

  const float lt = half_swap_sum(l);
  const float inv = 1.0f / lt;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bf16x4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(o[dt][4 * r + e] * inv);
      *(u32x2*)(orow + (32 * dt + 8 * r + 4 * hh) * 2) = __builtin_bit_cast(u32x2, ov);
    }
  if (hh == 0) a.lse[(int64_t)h * a.sd.total_tokens + t] = (m + __builtin_log2f(lt)) * kLn2;
}

}  // namespace

// Scratch of the no-allocation entry point (fp_mean_correct_noalloc): room for the
// tile images of hkv * ceil(nb / 32) <= 341 tiles, e.g. 4 KV heads up to 348K tokens.
// Every GPU the library runs on holds its own copy until the process ends.  The
// array's name is only a host-side stand-in: kernels get the device address taken
// below, once per device.
constexpr int64_t kScratchBytes = (int64_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int64_t meancorr_scratch_bytes() { return kScratchBytes; }

hipError_t meancorr_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int meancorr_max_blocks() { return kMaxBlocks; }

int64_t meancorr_tile_bytes() { return kTileBytes; }

int64_t meancorr_tiles(int L) {
  const int64_t nb = ((int64_t)L + kBlock - 1) / kBlock;
  return (nb + kTile - 1) / kTile;
}

// sum_s ceil(nb_s / 32) <= ceil(total_blocks / 32) + n_seqs
int64_t meancorr_tiles_varlen(int64_t total_blocks, int n_seqs) { return (total_blocks + kTile - 1) / kTile + n_seqs; }

int64_t meancorr_workspace_bytes(int L, int hkv) { return (int64_t)hkv * meancorr_tiles(L) * kTileBytes; }

hipError_t launch_meancorr(const MeanCorrLaunch& a, hipStream_t st) {
  const int max_tiles = (a.sd.max_nb + kTile - 1) / kTile;
  if (max_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(meanprep_kernel, dim3(max_tiles, a.sd.n_seqs, a.hkv), dim3(kThreads), 0, st, a);
  const size_t mask_bytes = (size_t)max_tiles * 4;
  hipLaunchKernelGGL(meancorr_kernel, dim3((unsigned)((int64_t)a.hq * a.sd.max_nb * a.sd.n_seqs)), dim3(kThreads),
                     mask_bytes, st, a);
  return hipGetLastError();
}

}  // namespace fp
