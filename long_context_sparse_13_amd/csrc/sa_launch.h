// Internal launchers: host functions in the kernel translation units, called by the
// C ABI layer (sa_api.cpp) after it has validated every argument.  Each returns the
// hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

// Stored element types (the values of the public dtype codes).
enum Elem { kF32 = 0, kBF16 = 1, kE4M3 = 2 };

hipError_t launch_indexer_scores(const void* qi, const void* ki, const float* w, int B, int T,
                                 int H_I, int D_I, int elem, int row_begin, int row_end,
                                 float* scores, int64_t ld, hipStream_t st);

// MFMA indexer over key slots j at positions j << sshift (sshift = 0: plain scores), slots
// cut into chunks of `chunk` (a multiple of 64) spread over the workgroups of a strip.
// f8: qi and ki hold E4M3 codes (else bf16).
bool indexer_has_mfma(int elem, int H_I, int D_I);
hipError_t launch_indexer_mfma(const void* qi, const void* ki, const float* w, int B, int T,
                               int H_I, int D_I, bool f8, int row_begin, int row_end, int sshift,
                               int chunk, float* scores, int64_t ld, hipStream_t st);

hipError_t launch_topk_select(const float* scores, int64_t ld, int B, int T, int row_begin,
                              int row_end, int k, int32_t* idx, hipStream_t st);

// Fused indexer -> top-k (MFMA indexer configurations only).
size_t indexer_topk_workspace_bytes(int B, int row_begin, int row_end, int k);
hipError_t launch_indexer_topk(const void* qi, const void* ki, const float* w, int B, int T,
                               int H_I, int D_I, bool f8, int row_begin, int row_end, int k,
                               int32_t* idx, void* workspace, hipStream_t st);

hipError_t launch_sparse_attn_fwd(const void* q, const void* k, const void* v, const int32_t* idx,
                                  int B, int T, int Hq, int Hkv, int D, int topk, int window,
                                  float scale, bool bf16, void* out, float* lse, int row_begin,
                                  int row_end, hipStream_t st);

// SA_VALIDATE: the first row (b * T + t) of [row_begin, row_end) that lists a position
// 0 <= s <= t - window more than once, or -1; synchronises the stream.
hipError_t validate_idx_unique(const int32_t* idx, int B, int T, int topk, int window,
                               int row_begin, int row_end, long long* bad_row, hipStream_t st);

hipError_t launch_sparse_attn_bwd(const void* q, const void* k, const void* v, const int32_t* idx,
                                  int B, int T, int Hq, int Hkv, int D, int topk, int window,
                                  float scale, const void* out, const float* lse,
                                  const void* dout, float* dq, float* dk, float* dv,
                                  void* workspace, size_t ws_bytes, hipStream_t st);
// The workspace path: its size for chunks of `rows` query rows (rows <= 0: all T), the
// chunk that a workspace of ws_bytes holds (0 if none), and the shapes it handles.
size_t sparse_attn_bwd_workspace_bytes(int B, int T, int Hkv, int D, int topk, int window,
                                       int rows);
int sparse_attn_bwd_chunk_rows(int B, int T, int Hkv, int D, int topk, int window,
                               size_t ws_bytes);
bool sparse_attn_bwd_partial_ok(int B, int T, int topk, int window);

hipError_t launch_graph_attn_fwd(const void* cq, const void* ck, const void* v, const float* bias,
                                 float tau, int B, int T, int H, int D, int local, int n_pow2,
                                 bool bf16, void* out, float* lse, hipStream_t st);

hipError_t launch_block_meanpool(const void* kcache, const int32_t* lens, int B, int Lmax, int Hkv,
                                 int D, int block, bool bf16, void* kbar, bool out16,
                                 hipStream_t st);

struct DecodeWs {
  uint32_t* cand;        // [B, Hkv, scoring workgroups, 16] packed (order key, block)
  float* partials;       // [B, Hkv, n_splits, G, D + 4]  (o[D], m, l, pad)
  uint32_t* counters;    // [B * Hkv] merge counters
};
size_t decode_workspace_bytes(int B, int Lmax, int Hq, int Hkv, int D, int block, int top_blocks,
                              int n_splits);
int decode_auto_splits(int B, int Lmax, int Hkv, int block, int top_blocks, int window);
DecodeWs decode_workspace_carve(void* ws, int B, int Lmax, int Hq, int Hkv, int D, int block,
                                int top_blocks, int n_splits);

hipError_t launch_sparse_decode(const void* q, const void* kcache, const void* vcache,
                                const float* kbar, const int32_t* lens, int B, int Lmax, int Hq,
                                int Hkv, int D, int block, int top_blocks, int window,
                                int n_splits, float scale, void* out, float* lse,
                                int32_t* sel_out, const DecodeWs& ws, hipStream_t st);
// The no-alloc decode's scratch: its size, and its device address on the current device
// (looked up once per device).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);

// NSA branches (prefill) and the gated combine.
size_t cmp_attn_workspace_bytes(int B, int T, int Hkv, int D, int block);
// Sliding-window attention with no listed keys (bf16, D in {64, 128}, up to 16 query
// heads per KV head, window >= 1): the 8 tokens of a workgroup share each K/V tile
// through LDS (band_attn_tile in k_nsa.hip).
hipError_t launch_window_attn(const void* q, const void* k, const void* v, int B, int T, int Hq,
                              int Hkv, int D, int window, float scale, void* out, float* lse,
                              int row_begin, int row_end, hipStream_t st);
hipError_t launch_cmp_attn(const void* q, const float* kbar, const float* vbar, int B, int T,
                           int Hq, int Hkv, int D, int block, float scale, void* out, float* lse,
                           void* workspace, hipStream_t st);
size_t block_select_workspace_bytes(int B, int T, int Hkv, int D, int block, int row_begin,
                                    int row_end);
hipError_t launch_block_select(const void* q, const float* kbar, int B, int T, int Hq, int Hkv,
                               int D, bool bf16, int block, int top_blocks, int row_begin,
                               int row_end, int32_t* idx, void* workspace, hipStream_t st);
// Decode attention of each sequence's query over one contiguous row range of a bf16
// cache: kind 0 = the window [max(0, L - window), L) of the token cache, kind 1 = the
// complete blocks [0, L / block) of the pooled cache.
hipError_t launch_nsa_decode_range(const void* q, const void* keys, const void* vals,
                                   const int32_t* lens, int B, int Lrows, int Hq, int Hkv, int D,
                                   int kind, int block, int window, float scale, void* out,
                                   float* lse, int n_splits, void* workspace, hipStream_t st);
size_t nsa_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int n_splits);
// The compressed (kind 1, over the pooled bf16 rows) and the window (kind 0) branch in one
// launch; the workspace holds the compressed side's partials and counters, then the window
// side's (each nsa_decode_workspace_bytes, present when that side has more than one split).
hipError_t launch_nsa_decode_cmp_win(const void* q, const void* kbar16, const void* vbar16,
                                     const void* kcache, const void* vcache, const int32_t* lens,
                                     int B, int Lmax, int Hq, int Hkv, int D, int block,
                                     int window, float scale, void* out_cmp, float* lse_cmp,
                                     void* out_win, float* lse_win, int ns_cmp, int ns_win,
                                     void* workspace, hipStream_t st);
hipError_t launch_nsa_combine(const void* oc, const void* os, const void* ow, const float* gates,
                              int B, int T, int Hq, int D, void* out, hipStream_t st);

}  // namespace sa
