// Stand-alone consumer of libflashprefill through its C ABI only (no Python, no
// torch): random bf16 Q/K/V with a per-block mean (so lists are sparse), then
// fp_discover -> fp_threshold_compact -> fp_sparse_attn on a stream of its own.
// Checks what holds for any input: every list is strictly ascending, inside
// [0, i] and ends with i, counts are in [1, i + 1], outputs are finite; with
// alpha = 0 every list is 0..i and the sparse output equals fp_dense_attn bit for
// bit; a bad argument returns FP_EINVAL with a message and launches nothing.
// Prints one line per check and exits non-zero on the first failure.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "flashprefill.h"

#define HIP_OK(x)                                                               \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      std::printf("FAIL hip %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                 \
    }                                                                           \
  } while (0)
#define FP_OK_(x)                                                                       \
  do {                                                                                  \
    int s_ = (x);                                                                       \
    if (s_ != FP_OK) {                                                                  \
      std::printf("FAIL %s: %s (%s)\n", #x, fp_status_string(s_), fp_last_error());    \
      return 1;                                                                         \
    }                                                                                   \
  } while (0)
#define CHECK(c, ...)                 \
  do {                                \
    if (!(c)) {                       \
      std::printf("FAIL ");           \
      std::printf(__VA_ARGS__);       \
      std::printf("\n");              \
      return 1;                       \
    }                                 \
  } while (0)

static uint16_t to_bf16(float x) {  // round to nearest even (finite inputs)
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

int main() {
  const int L = 128 * 37 + 45, hq = 8, hkv = 2, d = 128, B = 128;
  const int nb = (int)fp_num_blocks(L, B);
  const double scale = 1.0 / std::sqrt((double)d);
  std::mt19937 rng(1234);
  std::normal_distribution<float> nrm(0.0f, 1.0f);
  auto fill = [&](std::vector<uint16_t>& x, int H) {
    x.resize((size_t)L * H * d);
    std::vector<float> mu((size_t)nb * H * d);
    for (auto& m : mu) m = nrm(rng);
    for (int t = 0; t < L; ++t)
      for (int h = 0; h < H; ++h)
        for (int c = 0; c < d; ++c)
          x[((size_t)t * H + h) * d + c] = to_bf16(mu[((size_t)(t / B) * H + h) * d + c] + 0.3f * nrm(rng));
  };
  std::vector<uint16_t> hq_(0), hk(0), hv(0);
  fill(hq_, hq);
  fill(hk, hkv);
  fill(hv, hkv);

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  void *q, *k, *v, *out, *out_dense;
  double *pq, *pk;
  int32_t *idx, *counts;
  const int64_t cap = fp_idx_capacity(hq, nb);
  HIP_OK(hipMalloc(&q, hq_.size() * 2));
  HIP_OK(hipMalloc(&k, hk.size() * 2));
  HIP_OK(hipMalloc(&v, hv.size() * 2));
  HIP_OK(hipMalloc(&out, hq_.size() * 2));
  HIP_OK(hipMalloc(&out_dense, hq_.size() * 2));
  HIP_OK(hipMalloc((void**)&pq, (size_t)hq * nb * d * 8));
  HIP_OK(hipMalloc((void**)&pk, (size_t)hkv * nb * d * 8));
  HIP_OK(hipMalloc((void**)&idx, (size_t)cap * 4));
  HIP_OK(hipMalloc((void**)&counts, (size_t)hq * nb * 4));
  HIP_OK(hipMemcpy(q, hq_.data(), hq_.size() * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk.data(), hk.size() * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv.data(), hv.size() * 2, hipMemcpyHostToDevice));
  std::printf("abi %d, L=%d hq=%d hkv=%d nb=%d\n", fp_abi_version(), L, hq, hkv, nb);

  for (double alpha : {0.1, 0.0}) {
    FP_OK_(fp_discover(q, k, FP_BF16, nullptr, nullptr, L, hq, hkv, d, B, hq * d, d, hkv * d, d, pq, pk, st));
    FP_OK_(fp_threshold_compact(pq, pk, nb, hq, hkv, d, scale, alpha, 1, 3, idx, counts, nullptr, st));
    FP_OK_(fp_sparse_attn(q, k, v, FP_BF16, nullptr, nullptr, nullptr, L, hq, hkv, d, B, hq * d, d, hkv * d, d,
                          hkv * d, d, hq * d, d, idx, counts, (float)scale, out, nullptr, st));
    HIP_OK(hipStreamSynchronize(st));
    std::vector<int32_t> hidx(cap), hcnt((size_t)hq * nb);
    std::vector<uint16_t> ho(hq_.size());
    HIP_OK(hipMemcpy(hidx.data(), idx, (size_t)cap * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hcnt.data(), counts, hcnt.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ho.data(), out, ho.size() * 2, hipMemcpyDeviceToHost));
    int64_t kept = 0;
    for (int h = 0; h < hq; ++h)
      for (int i = 0; i < nb; ++i) {
        const int c = hcnt[(size_t)h * nb + i];
        CHECK(c >= 1 && c <= i + 1, "count(%d,%d)=%d", h, i, c);
        const int32_t* row = &hidx[(size_t)h * nb * (nb + 1) / 2 + (size_t)i * (i + 1) / 2];
        for (int e = 0; e < c; ++e) CHECK(row[e] >= 0 && row[e] <= i && (e == 0 || row[e] > row[e - 1]),
                                          "list(%d,%d) entry %d = %d", h, i, e, row[e]);
        CHECK(row[c - 1] == i, "list(%d,%d) does not end with the diagonal", h, i);
        if (alpha == 0.0) CHECK(c == i + 1, "alpha=0 count(%d,%d)=%d", h, i, c);
        kept += c;
      }
    for (uint16_t b : ho) CHECK(std::isfinite(from_bf16(b)), "non-finite output");
    std::printf("ok alpha=%.2f: lists valid, density %.3f, outputs finite\n", alpha,
                (double)kept / ((double)hq * nb * (nb + 1) / 2));
    if (alpha == 0.0) {
      FP_OK_(fp_dense_attn(q, k, v, FP_BF16, nullptr, nullptr, nullptr, L, hq, hkv, d, B, hq * d, d, hkv * d, d,
                           hkv * d, d, hq * d, d, (float)scale, out_dense, nullptr, st));
      HIP_OK(hipStreamSynchronize(st));
      std::vector<uint16_t> hd(hq_.size());
      HIP_OK(hipMemcpy(hd.data(), out_dense, hd.size() * 2, hipMemcpyDeviceToHost));
      CHECK(std::memcmp(hd.data(), ho.data(), hd.size() * 2) == 0, "alpha=0 sparse != dense");
      std::printf("ok alpha=0 sparse == dense bit for bit\n");
    }
  }
  // a rejected call: negative alpha
  const int s = fp_threshold_compact(pq, pk, nb, hq, hkv, d, scale, -1.0, 1, 3, idx, counts, nullptr, st);
  CHECK(s == FP_EINVAL && std::strlen(fp_last_error()) > 0, "negative alpha not rejected");
  std::printf("ok reject: %s (%s)\n", fp_status_string(s), fp_last_error());
  HIP_OK(hipFree(q)); HIP_OK(hipFree(k)); HIP_OK(hipFree(v)); HIP_OK(hipFree(out)); HIP_OK(hipFree(out_dense));
  HIP_OK(hipFree(pq)); HIP_OK(hipFree(pk)); HIP_OK(hipFree(idx)); HIP_OK(hipFree(counts));
  HIP_OK(hipStreamDestroy(st));
  std::printf("capi_check passed\n");
  return 0;
}
