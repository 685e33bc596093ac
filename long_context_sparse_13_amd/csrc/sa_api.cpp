// C ABI of libsa: argument validation, kernel selection and launch on the caller's
// stream.  Validation runs entirely on the host before any HIP call, so an invalid
// request never touches the GPU.  See include/sa.h for the contract of each entry point.
#include "../../include/sa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "sa_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, ...)                                 \
  do {                                                     \
    if (!(cond)) return fail(SA_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)
#define REQUIRE_PTR(p)                                                        \
  do {                                                                        \
    if (!(p)) return fail(SA_ERR_INVALID_ARG, "%s is NULL", #p);              \
    if (!aligned16(p)) return fail(SA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)
#define SUPPORT(cond, ...)                                 \
  do {                                                     \
    if (!(cond)) return fail(SA_ERR_UNSUPPORTED, __VA_ARGS__); \
  } while (0)

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int64_t kMaxElems = (int64_t)1 << 46;  // sanity bound on tensor sizes

// SA_VALIDATE set to anything but "" or "0" turns on the debug checks (read on every call).
bool validate_mode() {
  const char* e = std::getenv("SA_VALIDATE");
  return e && e[0] && std::strcmp(e, "0") != 0;
}

// The index contract: no position counted twice in a row (debug mode; synchronises).
int check_idx_unique(const char* fn, const int32_t* idx, int B, int T, int topk, int window,
                     int row_begin, int row_end, hipStream_t st) {
  long long bad = -1;
  const hipError_t e = sa::validate_idx_unique(idx, B, T, topk, window, row_begin, row_end,
                                               &bad, st);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "%s: SA_VALIDATE index check: %s", fn,
                                   hipGetErrorString(e));
  if (bad >= 0)
    return fail(SA_ERR_INVALID_ARG,
                "%s: SA_VALIDATE: idx row (b=%lld, t=%lld) lists a position in [0, t - window] "
                "more than once", fn, bad / T, bad % T);
  return SA_OK;
}

}  // namespace

extern "C" {

int sa_version(void) { return SA_VERSION; }

const char* sa_status_str(int status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARG: return "SA_ERR_INVALID_ARG";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
    case SA_ERR_INTERNAL: return "SA_ERR_INTERNAL";
    default: return "SA_ERR_UNKNOWN";
  }
}

const char* sa_last_error(void) { return g_err; }

int sa_indexer_scores(const void* qi, const void* ki, const float* w, int B, int T, int H_I,
                      int D_I, int dtype, int row_begin, int row_end, float* scores, int64_t ld,
                      void* stream) {
  try {
    REQUIRE_PTR(qi);
    REQUIRE_PTR(ki);
    REQUIRE_PTR(w);
    REQUIRE_PTR(scores);
    REQUIRE(B >= 1 && T >= 1, "B and T must be >= 1 (B=%d T=%d)", B, T);
    REQUIRE(H_I >= 1 && H_I <= 64, "H_I must be in [1, 64] (got %d)", H_I);
    REQUIRE(D_I >= 8 && D_I <= 256 && D_I % 8 == 0, "D_I must be a multiple of 8 in [8, 256] (got %d)", D_I);
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d",
            dtype);
    REQUIRE(0 <= row_begin && row_begin < row_end && row_end <= T,
            "need 0 <= row_begin < row_end <= T (got %d, %d, T=%d)", row_begin, row_end, T);
    REQUIRE(ld >= row_end && ld % 4 == 0, "ld must be >= row_end and a multiple of 4 (got %lld)",
            (long long)ld);
    REQUIRE((int64_t)B * (row_end - row_begin) * ld <= kMaxElems, "scores buffer too large");
    REQUIRE(B <= 65535, "B must be <= 65535 (got %d)", B);
    SUPPORT(H_I * D_I <= 4096, "H_I * D_I must be <= 4096 (got %d)", H_I * D_I);
    SUPPORT(dtype != SA_FP8_E4M3 || sa::indexer_has_mfma(dtype, H_I, D_I),
            "E4M3 inputs need H_I in {1,2,4} and D_I in {32,64,128} (H_I=%d D_I=%d)", H_I, D_I);
    return hip_status(sa::launch_indexer_scores(qi, ki, w, B, T, H_I, D_I, dtype,
                                                row_begin, row_end, scores, ld, as_stream(stream)),
                      "sa_indexer_scores launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_indexer_scores: unexpected exception");
  }
}

int sa_topk_select(const float* scores, int64_t ld, int B, int T, int row_begin, int row_end,
                   int k, int32_t* idx, void* stream) {
  try {
    REQUIRE_PTR(scores);
    REQUIRE_PTR(idx);
    REQUIRE(B >= 1 && T >= 1, "B and T must be >= 1 (B=%d T=%d)", B, T);
    REQUIRE(0 <= row_begin && row_begin < row_end && row_end <= T,
            "need 0 <= row_begin < row_end <= T (got %d, %d, T=%d)", row_begin, row_end, T);
    REQUIRE(ld >= row_end && ld % 4 == 0, "ld must be >= row_end and a multiple of 4 (got %lld)",
            (long long)ld);
    REQUIRE(k >= 1 && k <= 4096, "k must be in [1, 4096] (got %d)", k);
    REQUIRE((int64_t)B * (row_end - row_begin) <= 0x7fffffff, "too many rows in one call");
    SUPPORT(row_end <= 262144, "rows longer than 262144 are not supported (row_end=%d)", row_end);
    return hip_status(sa::launch_topk_select(scores, ld, B, T, row_begin, row_end, k, idx,
                                             as_stream(stream)),
                      "sa_topk_select launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_topk_select: unexpected exception");
  }
}

static bool indexer_topk_sizes_ok(int B, int T, int H_I, int D_I, int row_begin, int row_end,
                                  int k) {
  return B >= 1 && B <= 65535 && T >= 1 && T <= 262144 && 0 <= row_begin &&
         row_begin < row_end && row_end <= T && k >= 1 && k <= 4096 && H_I >= 1 && D_I >= 1 &&
         (int64_t)B * (row_end - row_begin) <= 0x7fffffff;
}

size_t sa_indexer_topk_workspace(int B, int T, int H_I, int D_I, int row_begin, int row_end,
                                 int k) {
  if (!indexer_topk_sizes_ok(B, T, H_I, D_I, row_begin, row_end, k)) return 0;
  return sa::indexer_topk_workspace_bytes(B, row_begin, row_end, k);
}

int sa_indexer_topk(const void* qi, const void* ki, const float* w, int B, int T, int H_I,
                    int D_I, int dtype, int row_begin, int row_end, int k, int32_t* idx,
                    void* workspace, size_t ws_bytes, void* stream) {
  try {
    REQUIRE_PTR(qi);
    REQUIRE_PTR(ki);
    REQUIRE_PTR(w);
    REQUIRE_PTR(idx);
    REQUIRE(B >= 1 && T >= 1, "B and T must be >= 1 (B=%d T=%d)", B, T);
    REQUIRE(B <= 65535, "B must be <= 65535 (got %d)", B);
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d",
            dtype);
    REQUIRE(0 <= row_begin && row_begin < row_end && row_end <= T,
            "need 0 <= row_begin < row_end <= T (got %d, %d, T=%d)", row_begin, row_end, T);
    REQUIRE(k >= 1 && k <= 4096, "k must be in [1, 4096] (got %d)", k);
    REQUIRE(H_I >= 1 && D_I >= 1, "H_I and D_I must be >= 1 (H_I=%d D_I=%d)", H_I, D_I);
    REQUIRE((int64_t)B * (row_end - row_begin) <= 0x7fffffff, "too many rows in one call");
    SUPPORT(T <= 262144, "T > 262144 is not supported (T=%d)", T);
    SUPPORT(sa::indexer_has_mfma(dtype, H_I, D_I),
            "the fused path needs bf16 or E4M3, H_I in {1,2,4} and D_I in {32,64,128} "
            "(dtype=%d H_I=%d D_I=%d)", dtype, H_I, D_I);
    const size_t need = sa::indexer_topk_workspace_bytes(B, row_begin, row_end, k);
    if (!workspace || ws_bytes < need)
      return fail(SA_ERR_WORKSPACE, "sa_indexer_topk: workspace of %zu bytes needed (got %zu)",
                  need, workspace ? ws_bytes : (size_t)0);
    REQUIRE(aligned16(workspace), "workspace is not 16-byte aligned");
    return hip_status(sa::launch_indexer_topk(qi, ki, w, B, T, H_I, D_I, dtype == SA_FP8_E4M3,
                                              row_begin, row_end, k, idx, workspace,
                                              as_stream(stream)),
                      "sa_indexer_topk launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_indexer_topk: unexpected exception");
  }
}

int sa_sparse_attn_fwd_rows(const void* q, const void* k, const void* v, const int32_t* idx,
                            int B, int T, int Hq, int Hkv, int D, int topk, int window,
                            float scale, int dtype, int row_begin, int row_end, void* out,
                            float* lse, void* stream) {
  try {
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(out);
    REQUIRE(B >= 1 && T >= 1, "B and T must be >= 1 (B=%d T=%d)", B, T);
    REQUIRE(0 <= row_begin && row_begin <= row_end && row_end <= T,
            "need 0 <= row_begin <= row_end <= T (got %d, %d, T=%d)", row_begin, row_end, T);
    REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv (Hq=%d Hkv=%d)", Hq, Hkv);
    REQUIRE(topk >= 0 && window >= 0 && topk + window >= 1,
            "need topk >= 0, window >= 0 and topk + window >= 1 (topk=%d window=%d)", topk, window);
    REQUIRE(topk == 0 || idx, "idx is NULL with topk=%d", topk);
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d",
            dtype);
    SUPPORT(dtype != SA_FP8_E4M3, "E4M3 inputs are taken by the indexer entry points only");
    REQUIRE((int64_t)B * T * Hq * D <= kMaxElems, "tensors too large");
    REQUIRE(((int64_t)B * T * Hkv + 7) / 8 * 8 <= 0x7fffffffLL, "too many (token, KV head) items");
    SUPPORT(D == 64 || D == 128, "head dim D=%d is not supported (64, 128)", D);
    const int G = Hq / Hkv;
    SUPPORT(G <= 64 && G * D <= 4096, "Hq/Hkv=%d with D=%d is not supported", G, D);
    if (lse) REQUIRE(aligned16(lse), "lse is not 16-byte aligned");
    if (idx) REQUIRE(aligned16(idx), "idx is not 16-byte aligned");
    if (topk > 0 && validate_mode()) {
      const int rc = check_idx_unique("sa_sparse_attn_fwd", idx, B, T, topk, window, row_begin,
                                      row_end, as_stream(stream));
      if (rc != SA_OK) return rc;
    }
    return hip_status(sa::launch_sparse_attn_fwd(q, k, v, idx, B, T, Hq, Hkv, D, topk, window,
                                                 scale, dtype == SA_BF16, out, lse, row_begin,
                                                 row_end, as_stream(stream)),
                      "sa_sparse_attn_fwd launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_sparse_attn_fwd: unexpected exception");
  }
}

int sa_sparse_attn_fwd(const void* q, const void* k, const void* v, const int32_t* idx, int B,
                       int T, int Hq, int Hkv, int D, int topk, int window, float scale,
                       int dtype, void* out, float* lse, void* stream) {
  return sa_sparse_attn_fwd_rows(q, k, v, idx, B, T, Hq, Hkv, D, topk, window, scale, dtype, 0,
                                 T > 0 ? T : 0, out, lse, stream);
}

int sa_graph_attn_fwd(const void* cq, const void* ck, const void* v, const float* bias,
                      float tau, int B, int T, int H, int D, int local, int n_pow2, int dtype,
                      void* out, float* lse, void* stream) {
  try {
    REQUIRE(cq && ck, "cq/ck is NULL");
    REQUIRE_PTR(v);
    REQUIRE(bias, "bias is NULL");
    REQUIRE_PTR(out);
    REQUIRE(B >= 1 && T >= 1 && H >= 1, "B, T and H must be >= 1 (B=%d T=%d H=%d)", B, T, H);
    REQUIRE(D >= 8 && D % 8 == 0, "D must be a positive multiple of 8 (got %d)", D);
    REQUIRE(local >= 0 && local <= 64, "local must be in [0, 64] (got %d)", local);
    REQUIRE(n_pow2 >= 0 && n_pow2 <= 30, "n_pow2 must be in [0, 30] (got %d)", n_pow2);
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d",
            dtype);
    SUPPORT(dtype != SA_FP8_E4M3, "E4M3 inputs are taken by the indexer entry points only");
    REQUIRE((int64_t)B * T * H * D <= kMaxElems, "tensors too large");
    SUPPORT(H * D <= 4096, "H * D must be <= 4096 (got %d)", H * D);
    REQUIRE(((int64_t)B * T * ((H * D / 8 + 63) / 64) + 7) / 8 * 8 <= 0x7fffffffLL, "too many tokens");
    return hip_status(sa::launch_graph_attn_fwd(cq, ck, v, bias, tau, B, T, H, D, local, n_pow2,
                                                dtype == SA_BF16, out, lse, as_stream(stream)),
                      "sa_graph_attn_fwd launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_graph_attn_fwd: unexpected exception");
  }
}

int sa_block_meanpool(const void* kcache, const int32_t* lens, int B, int Lmax, int Hkv, int D,
                      int block, int dtype, float* kbar, void* stream) {
  try {
    REQUIRE_PTR(kcache);
    REQUIRE(lens, "lens is NULL");
    REQUIRE_PTR(kbar);
    REQUIRE(B >= 1 && Lmax >= 1 && Hkv >= 1, "B, Lmax and Hkv must be >= 1");
    REQUIRE(D >= 4 && D % 4 == 0, "D must be a positive multiple of 4 (got %d)", D);
    REQUIRE(block == 16 || block == 32 || block == 64 || block == 128,
            "block must be 16, 32, 64 or 128 (got %d)", block);
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d",
            dtype);
    SUPPORT(dtype != SA_FP8_E4M3, "E4M3 inputs are taken by the indexer entry points only");
    REQUIRE((int64_t)B * Lmax * Hkv * D <= kMaxElems, "cache too large");
    return hip_status(sa::launch_block_meanpool(kcache, lens, B, Lmax, Hkv, D, block,
                                                dtype == SA_BF16, kbar, false, as_stream(stream)),
                      "sa_block_meanpool launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_block_meanpool: unexpected exception");
  }
}

int sa_block_meanpool_bf16(const void* kcache, const int32_t* lens, int B, int Lmax, int Hkv,
                           int D, int block, int dtype, void* kbar, void* stream) {
  try {
    REQUIRE_PTR(kcache);
    REQUIRE(lens, "lens is NULL");
    REQUIRE_PTR(kbar);
    REQUIRE(B >= 1 && Lmax >= 1 && Hkv >= 1, "B, Lmax and Hkv must be >= 1");
    REQUIRE(D >= 4 && D % 4 == 0, "D must be a positive multiple of 4 (got %d)", D);
    REQUIRE(block == 16 || block == 32 || block == 64 || block == 128,
            "block must be 16, 32, 64 or 128 (got %d)", block);
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d",
            dtype);
    SUPPORT(dtype != SA_FP8_E4M3, "E4M3 inputs are taken by the indexer entry points only");
    REQUIRE((int64_t)B * Lmax * Hkv * D <= kMaxElems, "cache too large");
    return hip_status(sa::launch_block_meanpool(kcache, lens, B, Lmax, Hkv, D, block,
                                                dtype == SA_BF16, kbar, true, as_stream(stream)),
                      "sa_block_meanpool_bf16 launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_block_meanpool_bf16: unexpected exception");
  }
}

int sa_sparse_attn_bwd(const void* q, const void* k, const void* v, const int32_t* idx, int B,
                       int T, int Hq, int Hkv, int D, int topk, int window, float scale,
                       int dtype, const void* out, const float* lse, const void* dout, float* dq,
                       float* dk, float* dv, void* workspace, size_t ws_bytes, void* stream) {
  try {
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(out);
    REQUIRE_PTR(lse);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(dq);
    REQUIRE_PTR(dk);
    REQUIRE_PTR(dv);
    REQUIRE(B >= 1 && T >= 1, "B and T must be >= 1 (B=%d T=%d)", B, T);
    REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv (Hq=%d Hkv=%d)", Hq, Hkv);
    REQUIRE(topk >= 0 && window >= 0 && topk + window >= 1,
            "need topk >= 0, window >= 0 and topk + window >= 1 (topk=%d window=%d)", topk, window);
    REQUIRE(topk == 0 || idx != nullptr, "idx is NULL with topk=%d", topk);
    REQUIRE(std::isfinite(scale), "scale must be finite");
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d", dtype);
    REQUIRE((int64_t)B * T * Hq * D <= kMaxElems, "tensors too large");
    SUPPORT(dtype == SA_BF16, "the backward takes bf16 tensors (dtype=%d)", dtype);
    SUPPORT(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
    SUPPORT(Hq / Hkv <= 16, "at most 16 query heads per KV head (got %d)", Hq / Hkv);
    if (workspace) {
      SUPPORT(sa::sparse_attn_bwd_partial_ok(B, T, topk, window),
              "the workspace path needs T <= 2^20 and B*T*(topk+window) < 2^31");
      REQUIRE(aligned16(workspace), "workspace is not 16-byte aligned");
      const int C = sa::sparse_attn_bwd_chunk_rows(B, T, Hkv, D, topk, window, ws_bytes);
      if (C < 1)
        return fail(SA_ERR_WORKSPACE,
                    "sa_sparse_attn_bwd: workspace of at least %zu bytes needed (got %zu)",
                    sa::sparse_attn_bwd_workspace_bytes(B, T, Hkv, D, topk, window, 1), ws_bytes);
    }
    if (topk > 0 && validate_mode()) {
      const int rc = check_idx_unique("sa_sparse_attn_bwd", idx, B, T, topk, window, 0, T,
                                      as_stream(stream));
      if (rc != SA_OK) return rc;
    }
    return hip_status(sa::launch_sparse_attn_bwd(q, k, v, idx, B, T, Hq, Hkv, D, topk, window,
                                                 scale, out, lse, dout, dq, dk, dv, workspace,
                                                 ws_bytes, as_stream(stream)),
                      "sa_sparse_attn_bwd launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_sparse_attn_bwd: unexpected exception");
  }
}

size_t sa_sparse_attn_bwd_workspace(int B, int T, int Hkv, int D, int topk, int window,
                                    int rows) {
  if (B < 1 || T < 1 || Hkv < 1 || (D != 64 && D != 128) || topk < 0 || window < 0 ||
      topk + window < 1 || !sa::sparse_attn_bwd_partial_ok(B, T, topk, window))
    return 0;
  return sa::sparse_attn_bwd_workspace_bytes(B, T, Hkv, D, topk, window, rows);
}

// ---------------------------------------------------------------- NSA branches (prefill)
static bool nsa_block_ok(int block) { return block == 16 || block == 32 || block == 64 || block == 128; }

size_t sa_cmp_attn_workspace(int B, int T, int Hkv, int D, int block) {
  if (B < 1 || T < 1 || Hkv < 1 || D < 1 || !nsa_block_ok(block)) return 0;
  return sa::cmp_attn_workspace_bytes(B, T, Hkv, D, block);
}

int sa_cmp_attn_fwd(const void* q, const float* kbar, const float* vbar, int B, int T, int Hq,
                    int Hkv, int D, int block, float scale, int dtype, void* out, float* lse,
                    void* workspace, size_t ws_bytes, void* stream) {
  try {
    REQUIRE_PTR(q);
    REQUIRE_PTR(kbar);
    REQUIRE_PTR(vbar);
    REQUIRE_PTR(out);
    REQUIRE(B >= 1 && T >= 1, "B and T must be >= 1 (B=%d T=%d)", B, T);
    REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv (Hq=%d Hkv=%d)", Hq, Hkv);
    REQUIRE(nsa_block_ok(block), "block must be 16, 32, 64 or 128 (got %d)", block);
    REQUIRE(std::isfinite(scale), "scale must be finite");
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d", dtype);
    REQUIRE((int64_t)B * T * Hq * D <= kMaxElems, "tensors too large");
    REQUIRE(lse == nullptr || aligned16(lse), "lse is not 16-byte aligned");
    SUPPORT(dtype == SA_BF16, "the compressed branch takes bf16 queries (dtype=%d)", dtype);
    SUPPORT(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
    SUPPORT(Hq / Hkv <= 16, "at most 16 query heads per KV head (got %d)", Hq / Hkv);
    const size_t need = sa::cmp_attn_workspace_bytes(B, T, Hkv, D, block);
    if (!workspace || ws_bytes < need)
      return fail(SA_ERR_WORKSPACE, "sa_cmp_attn_fwd: workspace of %zu bytes needed (got %zu)",
                  need, workspace ? ws_bytes : (size_t)0);
    REQUIRE(aligned16(workspace), "workspace is not 16-byte aligned");
    return hip_status(sa::launch_cmp_attn(q, kbar, vbar, B, T, Hq, Hkv, D, block, scale, out, lse,
                                          workspace, as_stream(stream)),
                      "sa_cmp_attn_fwd launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_cmp_attn_fwd: unexpected exception");
  }
}

size_t sa_block_select_workspace(int B, int T, int Hkv, int D, int block, int row_begin,
                                 int row_end) {
  if (B < 1 || T < 1 || Hkv < 1 || D < 1 || !nsa_block_ok(block) || row_begin < 0 ||
      row_begin >= row_end || row_end > T)
    return 0;
  return sa::block_select_workspace_bytes(B, T, Hkv, D, block, row_begin, row_end);
}

int sa_block_select(const void* q, const float* kbar, int B, int T, int Hq, int Hkv, int D,
                    int block, int top_blocks, int dtype, int row_begin, int row_end,
                    int32_t* idx, void* workspace, size_t ws_bytes, void* stream) {
  try {
    REQUIRE_PTR(q);
    REQUIRE_PTR(kbar);
    REQUIRE_PTR(idx);
    REQUIRE(B >= 1 && T >= 1, "B and T must be >= 1 (B=%d T=%d)", B, T);
    REQUIRE(B <= 65535, "B must be <= 65535 (got %d)", B);
    REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv (Hq=%d Hkv=%d)", Hq, Hkv);
    REQUIRE(D >= 4 && D % 4 == 0, "D must be a positive multiple of 4 (got %d)", D);
    REQUIRE(nsa_block_ok(block), "block must be 16, 32, 64 or 128 (got %d)", block);
    REQUIRE(top_blocks >= 1 && top_blocks <= 64, "top_blocks must be in [1, 64] (got %d)", top_blocks);
    REQUIRE(0 <= row_begin && row_begin < row_end && row_end <= T,
            "need 0 <= row_begin < row_end <= T (got %d, %d, T=%d)", row_begin, row_end, T);
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d", dtype);
    REQUIRE((int64_t)B * T * top_blocks * block <= kMaxElems, "index buffer too large");
    SUPPORT(dtype != SA_FP8_E4M3, "E4M3 inputs are taken by the indexer entry points only");
    SUPPORT(T / block <= 4096, "at most 4096 blocks per row (T=%d block=%d)", T, block);
    const size_t need = sa::block_select_workspace_bytes(B, T, Hkv, D, block, row_begin, row_end);
    if (!workspace || ws_bytes < need)
      return fail(SA_ERR_WORKSPACE, "sa_block_select: workspace of %zu bytes needed (got %zu)",
                  need, workspace ? ws_bytes : (size_t)0);
    REQUIRE(aligned16(workspace), "workspace is not 16-byte aligned");
    return hip_status(sa::launch_block_select(q, kbar, B, T, Hq, Hkv, D, dtype == SA_BF16, block,
                                              top_blocks, row_begin, row_end, idx, workspace,
                                              as_stream(stream)),
                      "sa_block_select launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_block_select: unexpected exception");
  }
}

int sa_nsa_decode_branch(const void* q, const void* keys, const void* vals,
                         const int32_t* lens, int B, int Lrows, int Hq, int Hkv, int D, int kind,
                         int block, int window, float scale, int dtype, void* out, float* lse,
                         int n_splits, void* workspace, size_t ws_bytes, void* stream) {
  try {
    REQUIRE_PTR(q);
    REQUIRE_PTR(keys);
    REQUIRE_PTR(vals);
    REQUIRE(lens, "lens is NULL");
    REQUIRE_PTR(out);
    REQUIRE(B >= 1 && Lrows >= 1, "B and Lrows must be >= 1 (B=%d Lrows=%d)", B, Lrows);
    REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv (Hq=%d Hkv=%d)", Hq, Hkv);
    REQUIRE(kind == 0 || kind == 1, "kind must be 0 (window) or 1 (compressed) (got %d)", kind);
    REQUIRE(nsa_block_ok(block), "block must be 16, 32, 64 or 128 (got %d)", block);
    REQUIRE(window >= 0, "window must be >= 0 (got %d)", window);
    REQUIRE(std::isfinite(scale), "scale must be finite");
    REQUIRE((int64_t)B * Hkv <= 0x7fffffff, "too many (sequence, KV head) pairs");
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d", dtype);
    REQUIRE((int64_t)B * Lrows * Hkv * D <= kMaxElems, "cache too large");
    SUPPORT(dtype == SA_BF16, "the decode branches take bf16 tensors (dtype=%d)", dtype);
    SUPPORT(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
    SUPPORT(Hq / Hkv <= 16, "at most 16 query heads per KV head (got %d)", Hq / Hkv);
    REQUIRE(n_splits >= 1 && n_splits <= 64, "n_splits must be in [1, 64] (got %d)", n_splits);
    if (n_splits > 1) {
      const size_t need = sa::nsa_decode_workspace_bytes(B, Hq, Hkv, D, n_splits);
      if (!workspace || ws_bytes < need)
        return fail(SA_ERR_WORKSPACE,
                    "sa_nsa_decode_branch: workspace of %zu bytes needed for %d splits (got %zu)",
                    need, n_splits, workspace ? ws_bytes : (size_t)0);
      REQUIRE(aligned16(workspace), "workspace is not 16-byte aligned");
    }
    return hip_status(sa::launch_nsa_decode_range(q, keys, vals, lens, B, Lrows, Hq, Hkv, D, kind,
                                                  block, window, scale, out, lse, n_splits,
                                                  workspace, as_stream(stream)),
                      "sa_nsa_decode_branch launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_nsa_decode_branch: unexpected exception");
  }
}

static size_t cmp_win_ws(int B, int Hq, int Hkv, int D, int ns_cmp, int ns_win) {
  return (ns_cmp > 1 ? sa::nsa_decode_workspace_bytes(B, Hq, Hkv, D, ns_cmp) : 0) +
         (ns_win > 1 ? sa::nsa_decode_workspace_bytes(B, Hq, Hkv, D, ns_win) : 0);
}

int sa_nsa_decode_cmp_win(const void* q, const void* kbar16, const void* vbar16,
                          const void* kcache, const void* vcache, const int32_t* lens, int B,
                          int Lmax, int Hq, int Hkv, int D, int block, int window, float scale,
                          int dtype, void* out_cmp, float* lse_cmp, void* out_win, float* lse_win,
                          int n_splits_cmp, int n_splits_win, void* workspace, size_t ws_bytes,
                          void* stream) {
  try {
    REQUIRE_PTR(q);
    REQUIRE_PTR(kbar16);
    REQUIRE_PTR(vbar16);
    REQUIRE_PTR(kcache);
    REQUIRE_PTR(vcache);
    REQUIRE(lens, "lens is NULL");
    REQUIRE_PTR(out_cmp);
    REQUIRE_PTR(out_win);
    REQUIRE(B >= 1 && Lmax >= 1, "B and Lmax must be >= 1 (B=%d Lmax=%d)", B, Lmax);
    REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv (Hq=%d Hkv=%d)", Hq, Hkv);
    REQUIRE(nsa_block_ok(block), "block must be 16, 32, 64 or 128 (got %d)", block);
    REQUIRE(Lmax >= block, "Lmax must hold at least one block (Lmax=%d block=%d)", Lmax, block);
    REQUIRE(window >= 0, "window must be >= 0 (got %d)", window);
    REQUIRE(std::isfinite(scale), "scale must be finite");
    REQUIRE((int64_t)B * Hkv <= 0x7fffffff, "too many (sequence, KV head) pairs");
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d", dtype);
    REQUIRE((int64_t)B * Lmax * Hkv * D <= kMaxElems, "cache too large");
    SUPPORT(dtype == SA_BF16, "the decode branches take bf16 tensors (dtype=%d)", dtype);
    SUPPORT(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
    SUPPORT(Hq / Hkv <= 16, "at most 16 query heads per KV head (got %d)", Hq / Hkv);
    REQUIRE(n_splits_cmp >= 1 && n_splits_cmp <= 64 && n_splits_win >= 1 && n_splits_win <= 64,
            "n_splits_cmp and n_splits_win must be in [1, 64] (got %d, %d)", n_splits_cmp,
            n_splits_win);
    const size_t need = cmp_win_ws(B, Hq, Hkv, D, n_splits_cmp, n_splits_win);
    if (need > 0) {
      if (!workspace || ws_bytes < need)
        return fail(SA_ERR_WORKSPACE,
                    "sa_nsa_decode_cmp_win: workspace of %zu bytes needed for %d + %d splits "
                    "(got %zu)", need, n_splits_cmp, n_splits_win, workspace ? ws_bytes : (size_t)0);
      REQUIRE(aligned16(workspace), "workspace is not 16-byte aligned");
    }
    return hip_status(sa::launch_nsa_decode_cmp_win(q, kbar16, vbar16, kcache, vcache, lens, B,
                                                    Lmax, Hq, Hkv, D, block, window, scale,
                                                    out_cmp, lse_cmp, out_win, lse_win,
                                                    n_splits_cmp, n_splits_win, workspace,
                                                    as_stream(stream)),
                      "sa_nsa_decode_cmp_win launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_nsa_decode_cmp_win: unexpected exception");
  }
}

size_t sa_nsa_decode_cmp_win_workspace(int B, int Hq, int Hkv, int D, int n_splits_cmp,
                                       int n_splits_win) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || (D != 64 && D != 128) || n_splits_cmp < 1 ||
      n_splits_cmp > 64 || n_splits_win < 1 || n_splits_win > 64)
    return 0;
  return cmp_win_ws(B, Hq, Hkv, D, n_splits_cmp, n_splits_win);
}

size_t sa_nsa_decode_branch_workspace(int B, int Hq, int Hkv, int D, int n_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || (D != 64 && D != 128) || n_splits < 1 ||
      n_splits > 64)
    return 0;
  return sa::nsa_decode_workspace_bytes(B, Hq, Hkv, D, n_splits);
}

int sa_nsa_combine(const void* o_cmp, const void* o_slc, const void* o_win, const float* gates,
                   int B, int T, int Hq, int D, int dtype, void* out, void* stream) {
  try {
    REQUIRE_PTR(o_cmp);
    REQUIRE_PTR(o_slc);
    REQUIRE_PTR(o_win);
    REQUIRE_PTR(gates);
    REQUIRE_PTR(out);
    REQUIRE(B >= 1 && T >= 1 && Hq >= 1, "B, T and Hq must be >= 1");
    REQUIRE(D >= 8 && D % 8 == 0, "D must be a positive multiple of 8 (got %d)", D);
    REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d", dtype);
    REQUIRE((int64_t)B * T * Hq * D <= kMaxElems, "tensors too large");
    SUPPORT(dtype == SA_BF16, "the combine takes bf16 branch outputs (dtype=%d)", dtype);
    return hip_status(sa::launch_nsa_combine(o_cmp, o_slc, o_win, gates, B, T, Hq, D, out,
                                             as_stream(stream)),
                      "sa_nsa_combine launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_nsa_combine: unexpected exception");
  }
}

static int decode_check_sizes(int B, int Lmax, int Hq, int Hkv, int D, int block, int top_blocks,
                              int window, int n_splits) {
  REQUIRE(B >= 1 && Lmax >= 1, "B and Lmax must be >= 1 (B=%d Lmax=%d)", B, Lmax);
  REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq must be a positive multiple of Hkv (Hq=%d Hkv=%d)", Hq, Hkv);
  REQUIRE(block == 16 || block == 32 || block == 64 || block == 128,
          "block must be 16, 32, 64 or 128 (got %d)", block);
  REQUIRE(top_blocks >= 1 && top_blocks <= 64, "top_blocks must be in [1, 64] (got %d)", top_blocks);
  REQUIRE(window >= 0, "window must be >= 0 (got %d)", window);
  REQUIRE(n_splits >= 0 && n_splits <= 64, "n_splits must be in [0, 64] (got %d)", n_splits);
  REQUIRE((int64_t)B * Hkv <= 65535, "B * Hkv must be <= 65535");
  SUPPORT(D == 64 || D == 128, "head dim D=%d is not supported (64, 128)", D);
  SUPPORT(Hq / Hkv <= 16, "Hq/Hkv=%d is not supported by the decode kernel (<= 16)", Hq / Hkv);
  SUPPORT(Lmax / block <= 262144, "too many blocks per sequence");
  SUPPORT((int64_t)(Lmax / block) * Hkv * D * 4 < ((int64_t)1 << 31),
          "the block means of one sequence must span less than 2 GiB");
  return SA_OK;
}

size_t sa_sparse_decode_workspace(int B, int Lmax, int Hq, int Hkv, int D, int block,
                                  int top_blocks, int window, int n_splits) {
  if (decode_check_sizes(B, Lmax, Hq, Hkv, D, block, top_blocks, window, n_splits) != SA_OK)
    return 0;
  const int ns = n_splits ? n_splits : sa::decode_auto_splits(B, Lmax, Hkv, block, top_blocks, window);
  return sa::decode_workspace_bytes(B, Lmax, Hq, Hkv, D, block, top_blocks, ns);
}

int sa_sparse_decode_auto_splits(int B, int Lmax, int Hkv, int block, int top_blocks, int window) {
  if (B < 1 || Lmax < 1 || Hkv < 1 || block < 1 || top_blocks < 1 || window < 0) return 0;
  return sa::decode_auto_splits(B, Lmax, Hkv, block, top_blocks, window);
}

// Arguments shared by both decode entry points; *ns = the split count used.
static int decode_args(const void* q, const void* kcache, const void* vcache, const float* kbar,
                       const int32_t* lens, int B, int Lmax, int Hq, int Hkv, int D, int block,
                       int top_blocks, int window, int n_splits, int dtype, const void* out,
                       int* ns) {
  REQUIRE_PTR(q);
  REQUIRE_PTR(kcache);
  REQUIRE_PTR(vcache);
  REQUIRE_PTR(kbar);
  REQUIRE(lens, "lens is NULL");
  REQUIRE_PTR(out);
  REQUIRE(dtype == SA_F32 || dtype == SA_BF16 || dtype == SA_FP8_E4M3, "unknown dtype %d",
          dtype);
  SUPPORT(dtype != SA_FP8_E4M3, "E4M3 inputs are taken by the indexer entry points only");
  const int rc = decode_check_sizes(B, Lmax, Hq, Hkv, D, block, top_blocks, window, n_splits);
  if (rc != SA_OK) return rc;
  SUPPORT(dtype == SA_BF16, "the decode supports bf16 only");
  REQUIRE((int64_t)B * Lmax * Hkv * D <= kMaxElems, "cache too large");
  *ns = n_splits ? n_splits : sa::decode_auto_splits(B, Lmax, Hkv, block, top_blocks, window);
  return SA_OK;
}

int sa_sparse_decode(const void* q, const void* kcache, const void* vcache, const float* kbar,
                     const int32_t* lens, int B, int Lmax, int Hq, int Hkv, int D, int block,
                     int top_blocks, int window, int n_splits, float scale, int dtype, void* out,
                     float* lse, int32_t* sel_blocks, void* workspace, size_t ws_bytes,
                     void* stream) {
  try {
    int ns = 0;
    const int rc = decode_args(q, kcache, vcache, kbar, lens, B, Lmax, Hq, Hkv, D, block,
                               top_blocks, window, n_splits, dtype, out, &ns);
    if (rc != SA_OK) return rc;
    const size_t need = sa::decode_workspace_bytes(B, Lmax, Hq, Hkv, D, block, top_blocks, ns);
    if (!workspace || !aligned16(workspace))
      return fail(SA_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
    if (ws_bytes < need)
      return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
    const sa::DecodeWs ws = sa::decode_workspace_carve(workspace, B, Lmax, Hq, Hkv, D, block, top_blocks, ns);
    return hip_status(sa::launch_sparse_decode(q, kcache, vcache, kbar, lens, B, Lmax, Hq, Hkv, D,
                                               block, top_blocks, window, ns, scale, out, lse,
                                               sel_blocks, ws, as_stream(stream)),
                      "sa_sparse_decode launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_sparse_decode: unexpected exception");
  }
}

int sa_sparse_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                             const float* kbar, const int32_t* lens, int B, int Lmax, int Hq,
                             int Hkv, int D, int block, int top_blocks, int window, int n_splits,
                             float scale, int dtype, void* out, float* lse, int32_t* sel_blocks,
                             void* stream) {
  try {
    int ns = 0;
    const int rc = decode_args(q, kcache, vcache, kbar, lens, B, Lmax, Hq, Hkv, D, block,
                               top_blocks, window, n_splits, dtype, out, &ns);
    if (rc != SA_OK) return rc;
    const size_t need = sa::decode_workspace_bytes(B, Lmax, Hq, Hkv, D, block, top_blocks, ns);
    if (need > sa::decode_scratch_bytes())
      return fail(SA_ERR_UNSUPPORTED,
                  "sa_sparse_decode_noalloc: these sizes need %zu bytes of scratch, more than the "
                  "%zu it holds (use sa_sparse_decode with a workspace)",
                  need, sa::decode_scratch_bytes());
    void* scratch = nullptr;
    const hipError_t e = sa::decode_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e, "sa_sparse_decode_noalloc: scratch address");
    const sa::DecodeWs ws = sa::decode_workspace_carve(scratch, B, Lmax, Hq, Hkv, D, block,
                                                       top_blocks, ns);
    return hip_status(sa::launch_sparse_decode(q, kcache, vcache, kbar, lens, B, Lmax, Hq, Hkv, D,
                                               block, top_blocks, window, ns, scale, out, lse,
                                               sel_blocks, ws, as_stream(stream)),
                      "sa_sparse_decode_noalloc launch");
  } catch (...) {
    return fail(SA_ERR_INTERNAL, "sa_sparse_decode_noalloc: unexpected exception");
  }
}

size_t sa_sparse_decode_noalloc_max_scratch(void) { return sa::decode_scratch_bytes(); }

}  // extern "C"
