// C ABI of libflashprefill (include/flashprefill.h): host-side validation,
// launch descriptors, status codes.  Nothing here allocates, frees or
// synchronises; every call only enqueues kernels on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstdint>
#include <string>

#include "../../include/flashprefill.h"
#include "fp_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return FP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) { return dtype == FP_BF16 ? 2 : 1; }

// Common shape checks.  Returns FP_OK or an error code (message set).
int check_shape(int dtype, int hq, int hkv, int d, int block) {
  if (dtype != FP_BF16 && dtype != FP_FP8_E4M3) return fail(FP_EUNSUPPORTED, "unknown dtype %d", dtype);
  if (d != fp::kHeadDim) return fail(FP_EUNSUPPORTED, "head dim %d unsupported (needs 128)", d);
  if (block != fp::kBlock) return fail(FP_EUNSUPPORTED, "block size %d unsupported (needs 128)", block);
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return fail(FP_EINVAL, "bad head counts hq=%d hkv=%d", hq, hkv);
  if (hq > 4096) return fail(FP_EINVAL, "hq=%d too large", hq);
  return FP_OK;
}

// A strided [rows, heads, 128] operand: pointer alignment and strides that
// keep every head row 16-byte aligned and non-negative.
int check_tensor(const char* name, const void* ptr, int dtype, int64_t st_a, int64_t st_b) {
  if (ptr == nullptr) return fail(FP_EINVAL, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(FP_EINVAL, "%s is not 16-byte aligned", name);
  const int64_t unit = 16 / elem_size(dtype);
  if (st_a < 0 || st_b < 0) return fail(FP_EINVAL, "%s has a negative stride", name);
  if (st_a % unit || st_b % unit) return fail(FP_EINVAL, "%s strides (%lld, %lld) break 16-byte row alignment", name,
                                              (long long)st_a, (long long)st_b);
  return FP_OK;
}

int check_scales(int dtype, const float* a, const float* b, const float* c) {
  if (dtype != FP_FP8_E4M3) return FP_OK;
  if (a == nullptr || b == nullptr || c == nullptr) return fail(FP_EINVAL, "fp8 needs per-head scale arrays");
  return FP_OK;
}

int launch_status(hipError_t e) {
  if (e != hipSuccess) return fail(FP_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int64_t nblocks(int64_t L) { return (L + fp::kBlock - 1) / fp::kBlock; }

fp::SeqDesc single_seq(int L) {
  fp::SeqDesc sd{};
  sd.cu_seqlens = nullptr;
  sd.n_seqs = 1;
  sd.L = L;
  sd.max_nb = (int)nblocks(L);
  sd.total_tokens = L;
  sd.total_blocks = sd.max_nb;
  sd.total_tri = (int64_t)sd.max_nb * (sd.max_nb + 1) / 2;
  sd.cu_seqlens_q = nullptr;
  sd.max_nq = sd.max_nb;
  sd.total_qtokens = sd.total_tokens;
  sd.total_qblocks = sd.total_blocks;
  return sd;
}

int check_varlen(const int32_t* cu, int n_seqs, int max_seqlen, int64_t total_tokens, int64_t total_blocks,
                 int64_t total_tri, int hq, fp::SeqDesc* sd) {
  if (cu == nullptr) return fail(FP_EINVAL, "cu_seqlens is NULL");
  if (n_seqs < 1 || n_seqs > 65535) return fail(FP_EINVAL, "n_seqs=%d out of range [1, 65535]", n_seqs);
  if (max_seqlen < 0) return fail(FP_EINVAL, "max_seqlen < 0");
  if (total_tokens < 0 || total_blocks < 0 || total_tri < 0) return fail(FP_EINVAL, "negative extent");
  const int64_t mnb = nblocks(max_seqlen);
  if ((int64_t)hq * mnb * n_seqs >= (int64_t)1 << 31) return fail(FP_EINVAL, "grid too large");
  sd->cu_seqlens = cu;
  sd->n_seqs = n_seqs;
  sd->L = 0;
  sd->max_nb = (int)mnb;
  sd->total_tokens = total_tokens;
  sd->total_blocks = total_blocks;
  sd->total_tri = total_tri;
  sd->cu_seqlens_q = nullptr;
  sd->max_nq = sd->max_nb;
  sd->total_qtokens = total_tokens;
  sd->total_qblocks = total_blocks;
  return FP_OK;
}

// Chunked prefill: key (sequence) lengths in cu_k, query lengths in cu_q (each at
// most the key length; the queries are the last positions of the sequence).
int check_chunked(const int32_t* cu_q, const int32_t* cu_k, int n_seqs, int max_seqlen_q, int max_seqlen_k,
                  int64_t total_q, int64_t total_k, int64_t total_qblocks, int64_t total_kblocks, int64_t total_tri,
                  int hq, fp::SeqDesc* sd) {
  int r;
  if (cu_q == nullptr) return fail(FP_EINVAL, "cu_seqlens_q is NULL");
  if ((r = check_varlen(cu_k, n_seqs, max_seqlen_k, total_k, total_kblocks, total_tri, hq, sd))) return r;
  if (max_seqlen_q < 0) return fail(FP_EINVAL, "max_seqlen_q < 0");
  if (total_q < 0 || total_qblocks < 0) return fail(FP_EINVAL, "negative extent");
  // a chunk of n queries starting mid-block spans at most ceil(n/128) + 1 blocks
  const int64_t mnq = std::min(nblocks(max_seqlen_q) + (max_seqlen_q > 0 ? 1 : 0), nblocks(max_seqlen_k));
  if ((int64_t)hq * mnq * n_seqs >= (int64_t)1 << 31) return fail(FP_EINVAL, "grid too large");
  sd->cu_seqlens_q = cu_q;
  sd->max_nq = (int)mnq;
  sd->total_qtokens = total_q;
  sd->total_qblocks = total_qblocks;
  return FP_OK;
}

}  // namespace

extern "C" {

const char* fp_status_string(int status) {
  switch (status) {
    case FP_OK: return "FP_OK";
    case FP_EINVAL: return "FP_EINVAL";
    case FP_EUNSUPPORTED: return "FP_EUNSUPPORTED";
    case FP_EHIP: return "FP_EHIP";
    default: return "FP_UNKNOWN";
  }
}

const char* fp_last_error(void) { return g_last_error.c_str(); }

int fp_abi_version(void) { return 4; }

int64_t fp_num_blocks(int64_t L, int block) { return block > 0 && L >= 0 ? (L + block - 1) / block : -1; }

int64_t fp_idx_capacity(int hq, int64_t nb) { return hq > 0 && nb >= 0 ? (int64_t)hq * nb * (nb + 1) / 2 : -1; }

// ------------------------------------------------------------------ discovery
static int discover_common(const void* q, const void* k, int dtype, const float* q_scale, const float* k_scale,
                           const fp::SeqDesc& sd, const fp::PageDesc& pd, int hq, int hkv,
                           int64_t q_st, int64_t q_sh, int64_t k_sp, int64_t k_st, int64_t k_sh,
                           double* pooled_q, double* pooled_k, void* stream) {
  if (pooled_q == nullptr || pooled_k == nullptr) return fail(FP_EINVAL, "pooled output is NULL");
  if (!aligned16(pooled_q) || !aligned16(pooled_k)) return fail(FP_EINVAL, "pooled output not 16-byte aligned");
  if (sd.max_nb == 0 || sd.total_blocks == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  fp::PoolLaunch a{};
  a.dtype = dtype;
  a.query_view = true;
  a.x = q; a.scale = q_scale; a.H = hq; a.st_page = 0; a.st_tok = q_st; a.st_head = q_sh; a.paged = false;
  a.out = pooled_q;
  if (sd.max_nq > 0 && sd.total_qblocks > 0) {
    hipError_t e = fp::launch_pool(a, sd, pd, st);
    if (e != hipSuccess) return launch_status(e);
  }
  a.query_view = false;
  a.x = k; a.scale = k_scale; a.H = hkv; a.st_page = k_sp; a.st_tok = k_st; a.st_head = k_sh;
  a.paged = pd.table != nullptr;
  a.out = pooled_k;
  return launch_status(fp::launch_pool(a, sd, pd, st));
}

int fp_discover(const void* q, const void* k, int dtype, const float* q_scale, const float* k_scale,
                int L, int hq, int hkv, int d, int block,
                int64_t q_stride_tok, int64_t q_stride_head, int64_t k_stride_tok, int64_t k_stride_head,
                double* pooled_q, double* pooled_k, void* stream) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  if (L < 0) return fail(FP_EINVAL, "L < 0");
  if (L == 0) return ok();
  if ((r = check_tensor("q", q, dtype, q_stride_tok, q_stride_head))) return r;
  if ((r = check_tensor("k", k, dtype, k_stride_tok, k_stride_head))) return r;
  if (dtype == FP_FP8_E4M3 && (q_scale == nullptr || k_scale == nullptr)) return fail(FP_EINVAL, "fp8 needs q/k scales");
  fp::PageDesc pd{nullptr, 0, 0};
  return discover_common(q, k, dtype, q_scale, k_scale, single_seq(L), pd, hq, hkv, q_stride_tok, q_stride_head,
                         0, k_stride_tok, k_stride_head, pooled_q, pooled_k, stream);
}

int fp_discover_paged(const void* q, const void* k, int dtype, const float* q_scale, const float* k_scale,
                      const int32_t* cu_seqlens, int n_seqs, int max_seqlen, int64_t total_tokens,
                      int64_t total_blocks, const int32_t* page_table, int max_pages, int num_pages,
                      int hq, int hkv, int d, int block,
                      int64_t q_stride_tok, int64_t q_stride_head,
                      int64_t k_stride_page, int64_t k_stride_tok, int64_t k_stride_head,
                      double* pooled_q, double* pooled_k, void* stream) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  fp::SeqDesc sd{};
  if ((r = check_varlen(cu_seqlens, n_seqs, max_seqlen, total_tokens, total_blocks, 0, hq, &sd))) return r;
  if (total_tokens == 0 || sd.max_nb == 0) return ok();
  if ((r = check_tensor("q", q, dtype, q_stride_tok, q_stride_head))) return r;
  if ((r = check_tensor("k", k, dtype, k_stride_tok, k_stride_head))) return r;
  fp::PageDesc pd{page_table, max_pages, num_pages};
  if (page_table != nullptr) {
    if ((r = check_tensor("k", k, dtype, k_stride_page, 0))) return r;
    if (max_pages < sd.max_nb) return fail(FP_EINVAL, "max_pages=%d < ceil(max_seqlen/128)=%d", max_pages, sd.max_nb);
    if (num_pages < 1) return fail(FP_EINVAL, "num_pages < 1");
  }
  if (dtype == FP_FP8_E4M3 && (q_scale == nullptr || k_scale == nullptr)) return fail(FP_EINVAL, "fp8 needs q/k scales");
  return discover_common(q, k, dtype, q_scale, k_scale, sd, pd, hq, hkv, q_stride_tok, q_stride_head,
                         k_stride_page, k_stride_tok, k_stride_head, pooled_q, pooled_k, stream);
}

// ------------------------------------------------------- threshold + compact
static int select_common(const double* pq, const double* pk, const fp::SeqDesc& sd, int hq, int hkv,
                         double softmax_scale, double alpha, int n_sink, int n_local, int32_t* idx, int32_t* counts,
                         void* stream, uint32_t* mask = nullptr, double* scores = nullptr) {
  if (pq == nullptr || pk == nullptr) return fail(FP_EINVAL, "pooled input is NULL");
  if (mask == nullptr && (idx == nullptr || counts == nullptr)) return fail(FP_EINVAL, "idx/counts is NULL");
  if (!std::isfinite(alpha) || alpha < 0.0) return fail(FP_EINVAL, "alpha must be finite and >= 0 (got %g)", alpha);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.0) return fail(FP_EINVAL, "softmax_scale must be > 0");
  if (n_sink < 0) return fail(FP_EINVAL, "n_sink < 0");
  if (n_local < 1) return fail(FP_EINVAL, "n_local < 1");
  if (sd.max_nb == 0 || sd.total_blocks == 0) return ok();
  fp::SelectLaunch a{};
  a.pq = pq; a.pk = pk; a.hq = hq; a.hkv = hkv;
  a.scale = softmax_scale;
  a.log_alpha = alpha == 0.0 ? -HUGE_VAL : std::log(alpha);
  a.n_sink = n_sink; a.n_local = n_local; a.idx = idx; a.counts = counts;
  a.mask = mask; a.mask_words = (int)((sd.max_nb + 31) / 32);
  a.scores = scores;
  return launch_status(fp::launch_select(a, sd, (hipStream_t)stream));
}

int fp_mask_words(int64_t nb) { return nb <= 0 ? 0 : (int)((nb + 31) / 32); }

int fp_threshold_mask(const double* pooled_q, const double* pooled_k, int nb, int hq, int hkv, int d,
                      double softmax_scale, double alpha, int n_sink, int n_local, uint32_t* mask, void* stream) {
  int r;
  if ((r = check_shape(FP_BF16, hq, hkv, d, fp::kBlock))) return r;
  if (nb < 0 || nb > (1 << 24)) return fail(FP_EINVAL, "nb=%d out of range", nb);
  if (nb == 0) return ok();
  if (mask == nullptr) return fail(FP_EINVAL, "mask is NULL");
  if ((uintptr_t)mask & 3u) return fail(FP_EINVAL, "mask not 4-byte aligned");
  fp::SeqDesc sd = single_seq(nb * fp::kBlock);
  return select_common(pooled_q, pooled_k, sd, hq, hkv, softmax_scale, alpha, n_sink, n_local, nullptr, nullptr,
                       stream, mask);
}

int fp_threshold_compact(const double* pooled_q, const double* pooled_k, int nb, int hq, int hkv, int d,
                         double softmax_scale, double alpha, int n_sink, int n_local,
                         int32_t* idx, int32_t* counts, double* scores, void* stream) {
  int r;
  if ((r = check_shape(FP_BF16, hq, hkv, d, fp::kBlock))) return r;
  if (nb < 0 || nb > (1 << 24)) return fail(FP_EINVAL, "nb=%d out of range", nb);
  if (nb == 0) return ok();
  if (scores != nullptr && ((uintptr_t)scores & 7u)) return fail(FP_EINVAL, "scores not 8-byte aligned");
  fp::SeqDesc sd = single_seq(nb * fp::kBlock);
  return select_common(pooled_q, pooled_k, sd, hq, hkv, softmax_scale, alpha, n_sink, n_local, idx, counts, stream,
                       nullptr, scores);
}

int fp_threshold_compact_varlen(const double* pooled_q, const double* pooled_k, const int32_t* cu_seqlens,
                                int n_seqs, int max_seqlen, int64_t total_blocks, int64_t total_tri,
                                int hq, int hkv, int d, double softmax_scale, double alpha, int n_sink, int n_local,
                                int32_t* idx, int32_t* counts, void* stream) {
  int r;
  if ((r = check_shape(FP_BF16, hq, hkv, d, fp::kBlock))) return r;
  fp::SeqDesc sd{};
  if ((r = check_varlen(cu_seqlens, n_seqs, max_seqlen, 0, total_blocks, total_tri, hq, &sd))) return r;
  sd.total_tokens = (int64_t)1 << 62;  // lengths only; no token buffer is touched here
  return select_common(pooled_q, pooled_k, sd, hq, hkv, softmax_scale, alpha, n_sink, n_local, idx, counts, stream);
}

// ------------------------------------------------------------------ attention
static int attn_common(const void* q, const void* k, const void* v, int dtype, const float* q_scale,
                       const float* k_scale, const float* v_scale, const fp::SeqDesc& sd, const fp::PageDesc& pd,
                       int hq, int hkv, int64_t q_st, int64_t q_sh, int64_t k_sp, int64_t k_st, int64_t k_sh,
                       int64_t v_sp, int64_t v_st, int64_t v_sh, int64_t o_st, int64_t o_sh,
                       const int32_t* idx, const int32_t* counts, float softmax_scale, void* out, float* lse,
                       void* stream, const uint32_t* mask = nullptr, int list_div = 1) {
  int r;
  if ((r = check_tensor("q", q, dtype, q_st, q_sh))) return r;
  if ((r = check_tensor("k", k, dtype, k_st, k_sh))) return r;
  if ((r = check_tensor("v", v, dtype, v_st, v_sh))) return r;
  if (pd.table != nullptr) {
    if ((r = check_tensor("k", k, dtype, k_sp, 0))) return r;
    if ((r = check_tensor("v", v, dtype, v_sp, 0))) return r;
  }
  if ((r = check_tensor("out", out, FP_BF16, o_st, o_sh))) return r;
  if ((r = check_scales(dtype, q_scale, k_scale, v_scale))) return r;
  // a 128-token tile is addressed with 32-bit byte offsets from its first row
  if (q_st * elem_size(dtype) * fp::kBlock > INT32_MAX || k_st * elem_size(dtype) * fp::kBlock > INT32_MAX ||
      v_st * elem_size(dtype) * fp::kBlock > INT32_MAX)
    return fail(FP_EINVAL, "Q/K/V token stride too large for 32-bit tile offsets");
  if ((idx == nullptr) != (counts == nullptr)) return fail(FP_EINVAL, "idx and counts must both be set or both NULL");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.0f) return fail(FP_EINVAL, "softmax_scale must be > 0");
  if (lse != nullptr && ((uintptr_t)lse & 3u)) return fail(FP_EINVAL, "lse not 4-byte aligned");
  if (sd.max_nb == 0 || sd.total_tokens == 0 || sd.max_nq == 0 || sd.total_qtokens == 0) return ok();
  fp::AttnLaunch a{};
  a.q = q; a.k = k; a.v = v; a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.dtype = dtype; a.hq = hq; a.hkv = hkv;
  a.q_st = q_st; a.q_sh = q_sh; a.k_sp = k_sp; a.k_st = k_st; a.k_sh = k_sh;
  a.v_sp = v_sp; a.v_st = v_st; a.v_sh = v_sh; a.o_st = o_st; a.o_sh = o_sh;
  a.idx = idx; a.counts = counts; a.softmax_scale = softmax_scale; a.out = out; a.lse = lse;
  a.mask = mask; a.mask_words = (int)((sd.max_nb + 31) / 32);
  a.list_div = list_div;
  return launch_status(fp::launch_attn(a, sd, pd, (hipStream_t)stream));
}

int fp_pool(const void* x, int dtype, const float* scale, int L, int H, int d, int block,
            int64_t stride_tok, int64_t stride_head, double* pooled, void* stream) {
  int r;
  if ((r = check_shape(dtype, H, H, d, block))) return r;
  if (L < 0) return fail(FP_EINVAL, "L < 0");
  if (L == 0) return ok();
  if ((r = check_tensor("x", x, dtype, stride_tok, stride_head))) return r;
  if (pooled == nullptr) return fail(FP_EINVAL, "pooled output is NULL");
  if (!aligned16(pooled)) return fail(FP_EINVAL, "pooled output not 16-byte aligned");
  if (dtype == FP_FP8_E4M3 && scale == nullptr) return fail(FP_EINVAL, "fp8 needs a per-head scale");
  fp::SeqDesc sd = single_seq(L);
  fp::PageDesc pd{nullptr, 0, 0};
  fp::PoolLaunch a{};
  a.query_view = false;
  a.dtype = dtype;
  a.x = x; a.scale = scale; a.H = H; a.st_page = 0; a.st_tok = stride_tok; a.st_head = stride_head; a.paged = false;
  a.out = pooled;
  return launch_status(fp::launch_pool(a, sd, pd, (hipStream_t)stream));
}

int64_t fp_mean_correct_workspace_bytes(int L, int hkv) {
  if (L < 0 || hkv < 1) return -1;
  return fp::meancorr_workspace_bytes(L, hkv);
}

// Argument checks shared by both mean-correction entry points (workspace aside).
static int meancorr_check(const void* q, int dtype, const float* q_scale, const double* pooled_k,
                          const double* pooled_v, int L, int hq, int hkv, int d, int block,
                          int64_t q_stride_tok, int64_t q_stride_head, int64_t o_stride_tok, int64_t o_stride_head,
                          const int32_t* idx, const int32_t* counts, float softmax_scale, void* out, float* lse) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  if (L < 0) return fail(FP_EINVAL, "L < 0");
  if (L == 0) return FP_OK;
  if ((r = check_tensor("q", q, dtype, q_stride_tok, q_stride_head))) return r;
  if ((r = check_tensor("out", out, FP_BF16, o_stride_tok, o_stride_head))) return r;
  if (pooled_k == nullptr || pooled_v == nullptr) return fail(FP_EINVAL, "pooled K/V is NULL");
  if (!aligned16(pooled_k) || !aligned16(pooled_v)) return fail(FP_EINVAL, "pooled K/V not 16-byte aligned");
  if (idx == nullptr || counts == nullptr) return fail(FP_EINVAL, "idx/counts is NULL");
  if (lse == nullptr) return fail(FP_EINVAL, "lse is NULL (the correction needs the sparse LSE)");
  if (nblocks(L) > fp::meancorr_max_blocks())
    return fail(FP_EUNSUPPORTED, "L=%d exceeds the mean correction's %d blocks", L, fp::meancorr_max_blocks());
  if ((uintptr_t)lse & 3u) return fail(FP_EINVAL, "lse not 4-byte aligned");
  if (dtype == FP_FP8_E4M3 && q_scale == nullptr) return fail(FP_EINVAL, "fp8 needs q_scale");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.0f) return fail(FP_EINVAL, "softmax_scale must be > 0");
  if ((int64_t)hq * nblocks(L) >= (int64_t)1 << 31) return fail(FP_EINVAL, "grid too large");
  return FP_OK;
}

int fp_mean_correct(const void* q, int dtype, const float* q_scale,
                    const double* pooled_k, const double* pooled_v,
                    int L, int hq, int hkv, int d, int block,
                    int64_t q_stride_tok, int64_t q_stride_head, int64_t o_stride_tok, int64_t o_stride_head,
                    const int32_t* idx, const int32_t* counts, float softmax_scale,
                    void* out, float* lse, void* workspace, int64_t workspace_bytes, void* stream) {
  int r;
  if ((r = meancorr_check(q, dtype, q_scale, pooled_k, pooled_v, L, hq, hkv, d, block, q_stride_tok, q_stride_head,
                          o_stride_tok, o_stride_head, idx, counts, softmax_scale, out, lse)))
    return r;
  if (L == 0) return ok();
  if (workspace == nullptr || !aligned16(workspace)) return fail(FP_EINVAL, "workspace is NULL or not 16-byte aligned");
  if (workspace_bytes < fp::meancorr_workspace_bytes(L, hkv))
    return fail(FP_EINVAL, "workspace of %lld bytes < fp_mean_correct_workspace_bytes = %lld",
                (long long)workspace_bytes, (long long)fp::meancorr_workspace_bytes(L, hkv));
  fp::MeanCorrLaunch a{q, q_scale, dtype, single_seq(L), fp::meancorr_tiles(L), hq, hkv, q_stride_tok, q_stride_head,
                       o_stride_tok, o_stride_head, pooled_k, pooled_v, idx, counts, softmax_scale, out, lse, workspace};
  return launch_status(fp::launch_meancorr(a, (hipStream_t)stream));
}

int fp_mean_correct_noalloc(const void* q, int dtype, const float* q_scale,
                            const double* pooled_k, const double* pooled_v,
                            int L, int hq, int hkv, int d, int block,
                            int64_t q_stride_tok, int64_t q_stride_head, int64_t o_stride_tok, int64_t o_stride_head,
                            const int32_t* idx, const int32_t* counts, float softmax_scale,
                            void* out, float* lse, void* stream) {
  int r;
  if ((r = meancorr_check(q, dtype, q_scale, pooled_k, pooled_v, L, hq, hkv, d, block, q_stride_tok, q_stride_head,
                          o_stride_tok, o_stride_head, idx, counts, softmax_scale, out, lse)))
    return r;
  if (L == 0) return ok();
  const int64_t need = fp::meancorr_workspace_bytes(L, hkv);
  if (need > fp::meancorr_scratch_bytes())
    return fail(FP_EUNSUPPORTED, "L=%d with hkv=%d needs %lld bytes of scratch; the library's static scratch holds "
                "%lld (use fp_mean_correct with a caller workspace)", L, hkv, (long long)need,
                (long long)fp::meancorr_scratch_bytes());
  void* ws = nullptr;
  hipError_t e = fp::meancorr_scratch(&ws);
  if (e != hipSuccess) return fail(FP_EHIP, "static scratch address: %s", hipGetErrorString(e));
  fp::MeanCorrLaunch a{q, q_scale, dtype, single_seq(L), fp::meancorr_tiles(L), hq, hkv, q_stride_tok, q_stride_head,
                       o_stride_tok, o_stride_head, pooled_k, pooled_v, idx, counts, softmax_scale, out, lse, ws};
  return launch_status(fp::launch_meancorr(a, (hipStream_t)stream));
}

int64_t fp_mean_correct_varlen_workspace_bytes(int64_t total_blocks, int n_seqs, int hkv) {
  if (total_blocks < 0 || n_seqs < 1 || hkv < 1) return -1;
  return (int64_t)hkv * fp::meancorr_tiles_varlen(total_blocks, n_seqs) * fp::meancorr_tile_bytes();
}

int fp_mean_correct_varlen(const void* q, int dtype, const float* q_scale,
                           const double* pooled_k, const double* pooled_v,
                           const int32_t* cu_seqlens, int n_seqs, int max_seqlen,
                           int64_t total_tokens, int64_t total_blocks, int64_t total_tri,
                           int hq, int hkv, int d, int block,
                           int64_t q_stride_tok, int64_t q_stride_head, int64_t o_stride_tok, int64_t o_stride_head,
                           const int32_t* idx, const int32_t* counts, float softmax_scale,
                           void* out, float* lse, void* workspace, int64_t workspace_bytes, void* stream) {
  int r;
  fp::SeqDesc sd{};
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  if ((r = check_varlen(cu_seqlens, n_seqs, max_seqlen, total_tokens, total_blocks, total_tri, hq, &sd))) return r;
  // the per-sequence checks of the single-sequence call, with the longest sequence
  if ((r = meancorr_check(q, dtype, q_scale, pooled_k, pooled_v, max_seqlen, hq, hkv, d, block, q_stride_tok,
                          q_stride_head, o_stride_tok, o_stride_head, idx, counts, softmax_scale, out, lse)))
    return r;
  if (total_tokens == 0 || sd.max_nb == 0) return ok();
  const int64_t need = (int64_t)hkv * fp::meancorr_tiles_varlen(total_blocks, n_seqs) * fp::meancorr_tile_bytes();
  if (workspace == nullptr || !aligned16(workspace)) return fail(FP_EINVAL, "workspace is NULL or not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(FP_EINVAL, "workspace of %lld bytes < fp_mean_correct_varlen_workspace_bytes = %lld",
                (long long)workspace_bytes, (long long)need);
  fp::MeanCorrLaunch a{q, q_scale, dtype, sd, fp::meancorr_tiles_varlen(total_blocks, n_seqs), hq, hkv,
                       q_stride_tok, q_stride_head, o_stride_tok, o_stride_head, pooled_k, pooled_v, idx, counts,
                       softmax_scale, out, lse, workspace};
  return launch_status(fp::launch_meancorr(a, (hipStream_t)stream));
}

int fp_pool_varlen(const void* x, int dtype, const float* scale, const int32_t* cu_seqlens, int n_seqs,
                   int max_seqlen, int64_t total_tokens, int64_t total_blocks,
                   const int32_t* page_table, int max_pages, int num_pages, int H, int d, int block,
                   int64_t stride_page, int64_t stride_tok, int64_t stride_head, double* pooled, void* stream) {
  int r;
  if ((r = check_shape(dtype, H, H, d, block))) return r;
  fp::SeqDesc sd{};
  if ((r = check_varlen(cu_seqlens, n_seqs, max_seqlen, total_tokens, total_blocks, 0, H, &sd))) return r;
  if (total_tokens == 0 || sd.max_nb == 0) return ok();
  if ((r = check_tensor("x", x, dtype, stride_tok, stride_head))) return r;
  fp::PageDesc pd{page_table, max_pages, num_pages};
  if (page_table != nullptr) {
    if ((r = check_tensor("x", x, dtype, stride_page, 0))) return r;
    if (max_pages < sd.max_nb) return fail(FP_EINVAL, "max_pages=%d < ceil(max_seqlen/128)=%d", max_pages, sd.max_nb);
    if (num_pages < 1) return fail(FP_EINVAL, "num_pages < 1");
  }
  if (pooled == nullptr || !aligned16(pooled)) return fail(FP_EINVAL, "pooled output is NULL or not 16-byte aligned");
  if (dtype == FP_FP8_E4M3 && scale == nullptr) return fail(FP_EINVAL, "fp8 needs a per-head scale");
  fp::PoolLaunch a{};
  a.query_view = false;
  a.dtype = dtype;
  a.x = x; a.scale = scale; a.H = H; a.st_page = stride_page; a.st_tok = stride_tok; a.st_head = stride_head;
  a.paged = page_table != nullptr;
  a.out = pooled;
  return launch_status(fp::launch_pool(a, sd, pd, (hipStream_t)stream));
}

int fp_union_compact(const uint32_t* mask, int nb, int hq, int hkv, int32_t* idx, int32_t* counts, void* stream) {
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return fail(FP_EINVAL, "hq=%d must be a positive multiple of hkv=%d", hq, hkv);
  if (nb < 0 || nb > (1 << 24)) return fail(FP_EINVAL, "nb=%d out of range", nb);
  if (nb == 0) return ok();
  if (mask == nullptr || idx == nullptr || counts == nullptr) return fail(FP_EINVAL, "mask/idx/counts is NULL");
  if ((uintptr_t)mask & 3u) return fail(FP_EINVAL, "mask not 4-byte aligned");
  fp::UnionLaunch a{mask, hq, hkv, nb, (int)((nb + 31) / 32), idx, counts};
  return launch_status(fp::launch_union(a, (hipStream_t)stream));
}

int fp_sparse_attn_grouped(const void* q, const void* k, const void* v, int dtype,
                           const float* q_scale, const float* k_scale, const float* v_scale,
                           int L, int hq, int hkv, int d, int block,
                           int64_t q_stride_tok, int64_t q_stride_head, int64_t k_stride_tok, int64_t k_stride_head,
                           int64_t v_stride_tok, int64_t v_stride_head, int64_t o_stride_tok, int64_t o_stride_head,
                           const int32_t* idx, const int32_t* counts, float softmax_scale,
                           void* out, float* lse, void* stream) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  if (L < 0) return fail(FP_EINVAL, "L < 0");
  if (L == 0) return ok();
  if (idx == nullptr || counts == nullptr) return fail(FP_EINVAL, "idx/counts is NULL");
  if ((int64_t)hq * nblocks(L) >= (int64_t)1 << 31) return fail(FP_EINVAL, "grid too large");
  fp::PageDesc pd{nullptr, 0, 0};
  return attn_common(q, k, v, dtype, q_scale, k_scale, v_scale, single_seq(L), pd, hq, hkv,
                     q_stride_tok, q_stride_head, 0, k_stride_tok, k_stride_head, 0, v_stride_tok, v_stride_head,
                     o_stride_tok, o_stride_head, idx, counts, softmax_scale, out, lse, stream, nullptr, hq / hkv);
}

int fp_sparse_attn_masked(const void* q, const void* k, const void* v, int dtype,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          int L, int hq, int hkv, int d, int block,
                          int64_t q_stride_tok, int64_t q_stride_head, int64_t k_stride_tok, int64_t k_stride_head,
                          int64_t v_stride_tok, int64_t v_stride_head, int64_t o_stride_tok, int64_t o_stride_head,
                          const uint32_t* mask, float softmax_scale, void* out, float* lse, void* stream) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  if (L < 0) return fail(FP_EINVAL, "L < 0");
  if (L == 0) return ok();
  if (mask == nullptr) return fail(FP_EINVAL, "mask is NULL");
  if ((uintptr_t)mask & 3u) return fail(FP_EINVAL, "mask not 4-byte aligned");
  if ((int64_t)hq * nblocks(L) >= (int64_t)1 << 31) return fail(FP_EINVAL, "grid too large");
  fp::PageDesc pd{nullptr, 0, 0};
  return attn_common(q, k, v, dtype, q_scale, k_scale, v_scale, single_seq(L), pd, hq, hkv,
                     q_stride_tok, q_stride_head, 0, k_stride_tok, k_stride_head, 0, v_stride_tok, v_stride_head,
                     o_stride_tok, o_stride_head, nullptr, nullptr, softmax_scale, out, lse, stream, mask);
}

int fp_sparse_attn(const void* q, const void* k, const void* v, int dtype,
                   const float* q_scale, const float* k_scale, const float* v_scale,
                   int L, int hq, int hkv, int d, int block,
                   int64_t q_stride_tok, int64_t q_stride_head, int64_t k_stride_tok, int64_t k_stride_head,
                   int64_t v_stride_tok, int64_t v_stride_head, int64_t o_stride_tok, int64_t o_stride_head,
                   const int32_t* idx, const int32_t* counts, float softmax_scale,
                   void* out, float* lse, void* stream) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  if (L < 0) return fail(FP_EINVAL, "L < 0");
  if (L == 0) return ok();
  if (idx == nullptr || counts == nullptr) return fail(FP_EINVAL, "idx/counts is NULL (use fp_dense_attn)");
  if ((int64_t)hq * nblocks(L) >= (int64_t)1 << 31) return fail(FP_EINVAL, "grid too large");
  fp::PageDesc pd{nullptr, 0, 0};
  return attn_common(q, k, v, dtype, q_scale, k_scale, v_scale, single_seq(L), pd, hq, hkv,
                     q_stride_tok, q_stride_head, 0, k_stride_tok, k_stride_head, 0, v_stride_tok, v_stride_head,
                     o_stride_tok, o_stride_head, idx, counts, softmax_scale, out, lse, stream);
}

int fp_dense_attn(const void* q, const void* k, const void* v, int dtype,
                  const float* q_scale, const float* k_scale, const float* v_scale,
                  int L, int hq, int hkv, int d, int block,
                  int64_t q_stride_tok, int64_t q_stride_head, int64_t k_stride_tok, int64_t k_stride_head,
                  int64_t v_stride_tok, int64_t v_stride_head, int64_t o_stride_tok, int64_t o_stride_head,
                  float softmax_scale, void* out, float* lse, void* stream) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  if (L < 0) return fail(FP_EINVAL, "L < 0");
  if (L == 0) return ok();
  if ((int64_t)hq * nblocks(L) >= (int64_t)1 << 31) return fail(FP_EINVAL, "grid too large");
  fp::PageDesc pd{nullptr, 0, 0};
  return attn_common(q, k, v, dtype, q_scale, k_scale, v_scale, single_seq(L), pd, hq, hkv,
                     q_stride_tok, q_stride_head, 0, k_stride_tok, k_stride_head, 0, v_stride_tok, v_stride_head,
                     o_stride_tok, o_stride_head, nullptr, nullptr, softmax_scale, out, lse, stream);
}

int fp_sparse_attn_paged(const void* q, const void* k, const void* v, int dtype,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         const int32_t* cu_seqlens, int n_seqs, int max_seqlen,
                         int64_t total_tokens, int64_t total_blocks, int64_t total_tri,
                         const int32_t* page_table, int max_pages, int num_pages,
                         int hq, int hkv, int d, int block,
                         int64_t q_stride_tok, int64_t q_stride_head,
                         int64_t k_stride_page, int64_t k_stride_tok, int64_t k_stride_head,
                         int64_t v_stride_page, int64_t v_stride_tok, int64_t v_stride_head,
                         int64_t o_stride_tok, int64_t o_stride_head,
                         const int32_t* idx, const int32_t* counts, float softmax_scale,
                         void* out, float* lse, void* stream) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  fp::SeqDesc sd{};
  if ((r = check_varlen(cu_seqlens, n_seqs, max_seqlen, total_tokens, total_blocks, total_tri, hq, &sd))) return r;
  if (total_tokens == 0 || sd.max_nb == 0) return ok();
  fp::PageDesc pd{page_table, max_pages, num_pages};
  if (page_table != nullptr) {
    if (max_pages < sd.max_nb) return fail(FP_EINVAL, "max_pages=%d < ceil(max_seqlen/128)=%d", max_pages, sd.max_nb);
    if (num_pages < 1) return fail(FP_EINVAL, "num_pages < 1");
  }
  return attn_common(q, k, v, dtype, q_scale, k_scale, v_scale, sd, pd, hq, hkv,
                     q_stride_tok, q_stride_head, k_stride_page, k_stride_tok, k_stride_head,
                     v_stride_page, v_stride_tok, v_stride_head, o_stride_tok, o_stride_head,
                     idx, counts, softmax_scale, out, lse, stream);
}

// ------------------------------------------------------------ chunked prefill
int fp_discover_chunked(const void* q, const void* k, int dtype, const float* q_scale, const float* k_scale,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seqs,
                        int max_seqlen_q, int max_seqlen_k, int64_t total_q, int64_t total_k,
                        int64_t total_qblocks, int64_t total_kblocks,
                        const int32_t* page_table, int max_pages, int num_pages,
                        int hq, int hkv, int d, int block,
                        int64_t q_stride_tok, int64_t q_stride_head,
                        int64_t k_stride_page, int64_t k_stride_tok, int64_t k_stride_head,
                        double* pooled_q, double* pooled_k, void* stream) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  fp::SeqDesc sd{};
  if ((r = check_chunked(cu_seqlens_q, cu_seqlens_k, n_seqs, max_seqlen_q, max_seqlen_k, total_q, total_k,
                         total_qblocks, total_kblocks, 0, hq, &sd))) return r;
  if (total_k == 0 || sd.max_nb == 0) return ok();
  if ((r = check_tensor("q", q, dtype, q_stride_tok, q_stride_head))) return r;
  if ((r = check_tensor("k", k, dtype, k_stride_tok, k_stride_head))) return r;
  fp::PageDesc pd{page_table, max_pages, num_pages};
  if (page_table != nullptr) {
    if ((r = check_tensor("k", k, dtype, k_stride_page, 0))) return r;
    if (max_pages < sd.max_nb) return fail(FP_EINVAL, "max_pages=%d < ceil(max_seqlen_k/128)=%d", max_pages, sd.max_nb);
    if (num_pages < 1) return fail(FP_EINVAL, "num_pages < 1");
  }
  if (dtype == FP_FP8_E4M3 && (q_scale == nullptr || k_scale == nullptr)) return fail(FP_EINVAL, "fp8 needs q/k scales");
  return discover_common(q, k, dtype, q_scale, k_scale, sd, pd, hq, hkv, q_stride_tok, q_stride_head,
                         k_stride_page, k_stride_tok, k_stride_head, pooled_q, pooled_k, stream);
}

int fp_threshold_compact_chunked(const double* pooled_q, const double* pooled_k,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seqs,
                                 int max_seqlen_q, int max_seqlen_k, int64_t total_qblocks, int64_t total_kblocks,
                                 int64_t total_tri, int hq, int hkv, int d,
                                 double softmax_scale, double alpha, int n_sink, int n_local,
                                 int32_t* idx, int32_t* counts, void* stream) {
  int r;
  if ((r = check_shape(FP_BF16, hq, hkv, d, fp::kBlock))) return r;
  fp::SeqDesc sd{};
  if ((r = check_chunked(cu_seqlens_q, cu_seqlens_k, n_seqs, max_seqlen_q, max_seqlen_k, 0, 0, total_qblocks,
                         total_kblocks, total_tri, hq, &sd))) return r;
  // lengths only; no token buffer is touched here
  sd.total_tokens = (int64_t)1 << 62;
  sd.total_qtokens = (int64_t)1 << 62;
  if (sd.max_nq == 0 || total_qblocks == 0) return ok();
  return select_common(pooled_q, pooled_k, sd, hq, hkv, softmax_scale, alpha, n_sink, n_local, idx, counts, stream);
}

int fp_sparse_attn_chunked(const void* q, const void* k, const void* v, int dtype,
                           const float* q_scale, const float* k_scale, const float* v_scale,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seqs,
                           int max_seqlen_q, int max_seqlen_k, int64_t total_q, int64_t total_k,
                           int64_t total_qblocks, int64_t total_kblocks, int64_t total_tri,
                           const int32_t* page_table, int max_pages, int num_pages,
                           int hq, int hkv, int d, int block,
                           int64_t q_stride_tok, int64_t q_stride_head,
                           int64_t k_stride_page, int64_t k_stride_tok, int64_t k_stride_head,
                           int64_t v_stride_page, int64_t v_stride_tok, int64_t v_stride_head,
                           int64_t o_stride_tok, int64_t o_stride_head,
                           const int32_t* idx, const int32_t* counts, float softmax_scale,
                           void* out, float* lse, void* stream) {
  int r;
  if ((r = check_shape(dtype, hq, hkv, d, block))) return r;
  fp::SeqDesc sd{};
  if ((r = check_chunked(cu_seqlens_q, cu_seqlens_k, n_seqs, max_seqlen_q, max_seqlen_k, total_q, total_k,
                         total_qblocks, total_kblocks, total_tri, hq, &sd))) return r;
  if (total_q == 0 || total_k == 0 || sd.max_nq == 0) return ok();
  fp::PageDesc pd{page_table, max_pages, num_pages};
  if (page_table != nullptr) {
    if (max_pages < sd.max_nb) return fail(FP_EINVAL, "max_pages=%d < ceil(max_seqlen_k/128)=%d", max_pages, sd.max_nb);
    if (num_pages < 1) return fail(FP_EINVAL, "num_pages < 1");
  }
  return attn_common(q, k, v, dtype, q_scale, k_scale, v_scale, sd, pd, hq, hkv,
                     q_stride_tok, q_stride_head, k_stride_page, k_stride_tok, k_stride_head,
                     v_stride_page, v_stride_tok, v_stride_head, o_stride_tok, o_stride_head,
                     idx, counts, softmax_scale, out, lse, stream);
}

}  // extern "C"
