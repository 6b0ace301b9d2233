// Internal interface between the C-ABI layer (api.hip) and the kernels.
// Not installed; the public contract is include/flashprefill.h.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fp {

constexpr int kBlock = 128;   // tokens per block (= page size)
constexpr int kHeadDim = 128; // head dimension

// Sequence layout of a (possibly single-sequence) batch.
// Keys: sequence s owns key tokens cu_seqlens[s] .. cu_seqlens[s+1]-1.  Queries:
// in prefill the same tokens; in chunked prefill (cu_seqlens_q set) the last
// len_q = cu_seqlens_q[s+1] - cu_seqlens_q[s] positions of the sequence, so query t
// sits at absolute position len_k - len_q + t.  Query blocks are numbered by
// absolute position: block I covers positions 128I .. 128I+127 (the first and
// last can be partial); list row I holds key blocks 0..I.
struct SeqDesc {
  const int32_t* cu_seqlens;  // device [n_seqs+1] key (sequence) lengths; nullptr: one sequence of length L
  const int32_t* cu_seqlens_q;  // device [n_seqs+1] query lengths, or nullptr: queries = keys
  int n_seqs;
  int L;                      // the single sequence's length when cu_seqlens == nullptr
  int max_nb;                 // grid extent over key blocks
  int max_nq;                 // grid extent over query blocks
  int64_t total_tokens;       // declared extents of the packed key-side buffers
  int64_t total_blocks;
  int64_t total_qtokens;      // ... and of the query-side ones (= the key side in prefill)
  int64_t total_qblocks;
  int64_t total_tri;          // list capacity per head
};

// Paged KV addressing (table == nullptr: packed like Q).
struct PageDesc {
  const int32_t* table;       // device [n_seqs, max_pages]
  int max_pages;
  int num_pages;
};

struct PoolLaunch {
  bool query_view;            // pool the query blocks of each sequence (else the key blocks)
  const void* x;              // [tokens, H, d] or pages [P, 128, H, d]
  const float* scale;         // fp8 per-head scale or nullptr
  int dtype;                  // 0 bf16, 1 fp8
  int H;
  int64_t st_page, st_tok, st_head;
  bool paged;
  double* out;                // [H, total_blocks, d]
};

struct SelectLaunch {
  const double* pq;           // [hq, total_blocks, d]
  const double* pk;           // [hkv, total_blocks, d]
  int hq, hkv;
  double scale;               // softmax scale applied to the pooled dot product
  double log_alpha;           // ln(alpha), -inf for alpha == 0
  int n_sink, n_local;
  int32_t* idx;               // [hq, total_tri]
  int32_t* counts;            // [hq, total_blocks]
  uint32_t* mask;             // bit-packed keep mask [hq, nb, mask_words] instead of lists, or nullptr
  int mask_words;             // ceil(nb / 32)
  double* scores;             // single sequence only: scaled pooled scores [hq, nb, nb] (j <= i written), or nullptr
};

struct AttnLaunch {
  const void* q; const void* k; const void* v;
  const float* q_scale; const float* k_scale; const float* v_scale;
  int dtype;
  int hq, hkv;
  int64_t q_st, q_sh;
  int64_t k_sp, k_st, k_sh;
  int64_t v_sp, v_st, v_sh;
  int64_t o_st, o_sh;
  const int32_t* idx;         // nullptr: dense (implicit list 0..i)
  const int32_t* counts;
  float softmax_scale;
  void* out;
  float* lse;                 // [hq, total_tokens] or nullptr
  const uint32_t* mask;       // logical-skip mode: bit-packed keep mask [hq, nb, mask_words], or nullptr
  int mask_words;
  int list_div;               // query head h reads list h / list_div (1: per head; hq/hkv: per KV group)
};

// Union of the per-head block masks of every KV group, compacted to ascending
// lists (group-shared lists).
struct UnionLaunch {
  const uint32_t* mask;       // [hq, nb, mask_words]
  int hq, hkv, nb, mask_words;
  int32_t* idx;               // [hkv, nb(nb+1)/2]
  int32_t* counts;            // [hkv, nb]
};
hipError_t launch_union(const UnionLaunch& a, hipStream_t st);

// V2 mean correction (an assumption): fold the pruned blocks' pooled means into a
// sparse attention result, in place.
struct MeanCorrLaunch {
  const void* q;
  const float* q_scale;
  int dtype;
  SeqDesc sd;                 // one sequence (cu_seqlens == nullptr) or a packed batch
  int64_t total_tiles;        // tile images per KV head in the workspace (its stride)
  int hq, hkv;
  int64_t q_st, q_sh, o_st, o_sh;
  const double* pooled_k;     // [hkv, total_blocks, d]
  const double* pooled_v;     // [hkv, total_blocks, d]
  const int32_t* idx;         // per-head lists of the sparse call
  const int32_t* counts;
  float softmax_scale;
  void* out;                  // bf16 [L, hq, d], in and out
  float* lse;                 // [hq, L], in and out
  void* workspace;            // hkv * total_tiles tile images, 16-byte aligned
};
hipError_t launch_meancorr(const MeanCorrLaunch& a, hipStream_t st);
int meancorr_max_blocks();  // longest row the mean correction handles (blocks)
int64_t meancorr_scratch_bytes();          // size of the library's static scratch
hipError_t meancorr_scratch(void** ptr);   // its address on the current device
int64_t meancorr_workspace_bytes(int L, int hkv);
int64_t meancorr_tiles(int L);                                   // tile images per KV head, one sequence
int64_t meancorr_tiles_varlen(int64_t total_blocks, int n_seqs);  // upper bound for a packed batch
int64_t meancorr_tile_bytes();

hipError_t launch_pool(const PoolLaunch& a, const SeqDesc& sd, const PageDesc& pd, hipStream_t st);
hipError_t launch_select(const SelectLaunch& a, const SeqDesc& sd, hipStream_t st);
hipError_t launch_attn(const AttnLaunch& a, const SeqDesc& sd, const PageDesc& pd, hipStream_t st);

}  // namespace fp
