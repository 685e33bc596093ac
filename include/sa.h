/*
 * sa.h — C ABI of libsa, causal sparse attention for AMD Instinct MI355X (gfx950).
 *
 * Every entry point is asynchronous on the HIP stream it is given (``stream`` is a
 * hipStream_t passed as void*; NULL means the default stream).  The library never
 * allocates or frees memory and never synchronises the host: all tensors, including
 * the decode workspace, belong to the caller, who keeps them alive until the stream
 * has executed the call.  All tensor pointers are DEVICE pointers to contiguous,
 * 16-byte-aligned buffers in the layouts documented below (row-major, last index
 * fastest).  Scalars and sizes are plain host values.
 *
 * Error behaviour: every call validates its arguments before touching the GPU and
 * returns SA_OK or an SA_ERR_* status.  On error nothing is launched and
 * sa_last_error() (per host thread) describes the problem.  A failed kernel launch
 * returns SA_ERR_HIP with the HIP error text; faults inside a kernel surface at the
 * caller's next synchronisation.  No C++ exception crosses this boundary.
 *
 * Debug mode: with the environment variable SA_VALIDATE set (to anything but "" or "0",
 * read on every call), sa_sparse_attn_fwd, sa_sparse_attn_fwd_rows and sa_sparse_attn_bwd
 * also check the index contract on the device before they launch: no row may list a
 * position 0 <= s <= t - window more than once.  A violation returns SA_ERR_INVALID_ARG
 * naming the first such row (b, t), and nothing is launched.  This check synchronises
 * the stream (it hands its result to the host); without SA_VALIDATE nothing synchronises.
 *
 * Notation: B batch, T tokens, Hq query heads, Hkv key/value heads (Hq % Hkv == 0,
 * query head h reads KV head h / (Hq / Hkv)), D head dimension.  "bf16" tensors are
 * stored as bfloat16 and accumulated in float32; "f32" tensors are float32.
 *
 * Sources (web pages, cited by title and section):
 *   [IC]   "IndexCache ... inferencia 82% más rápida" (larebelion.com, from VentureBeat), body
 *   [HS2]  "Xiaomi presenta HySparse2 ..." (diariobitcoin.com), sections "Dos niveles para
 *          compartir la caché" and "Más precisión con menos memoria"
 *   [SLM]  "SpatialLM-Mini aceleró el entrenamiento con un contexto de 16K en 2,47 veces en
 *          una RTX 3050" (news.hamidun.com), section "Cómo eligen los tokens a quién escuchar"
 *   [NSA]  "Native Sparse Attention: Revolucionando el Procesamiento de Contexto Extenso ..."
 *          (ctol-es.com), sections "Puntos Clave" and "Análisis Profundo"
 *   [STAR] "NVIDIA AI Research presenta Star Attention ..." (7minutos.es), body paragraph 3
 */
#ifndef LIBSA_SA_H
#define LIBSA_SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_VERSION 100 /* 1.0.0 */

/* Element types of the input/output tensors.  SA_FP8_E4M3: 8-bit floats as the OCP 8-bit
 * floating point specification defines E4M3 ("fn": bias 7, subnormals, no infinities,
 * 0x7F/0xFF NaN), one byte per element, no scale factor; accepted by the indexer entry
 * points only (sa_indexer_scores, sa_indexer_topk), SA_ERR_UNSUPPORTED elsewhere. */
typedef enum { SA_F32 = 0, SA_BF16 = 1, SA_FP8_E4M3 = 2 } sa_dtype;

/* Status codes. */
enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, inconsistent shapes */
  SA_ERR_UNSUPPORTED = 2, /* valid request the library has no kernel for (dtype, D, ...) */
  SA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace query */
  SA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  SA_ERR_INTERNAL = 5     /* unexpected internal error */
};

/*
 * Indexer scores.  [IC] body paragraphs 2-3: a lightweight indexer scores every
 * earlier token of every query.
 *
 *   scores[b, r, s] = sum_{h < H_I} w[h] * max(0, qi[b, t, h, :] . ki[b, s, :])
 *   for t = row_begin + r and every s <= t.
 *
 * qi     [B, T, H_I, D_I]  dtype
 * ki     [B, T, D_I]       dtype   (one indexer key per token, shared by the heads)
 * w      [H_I]             float32 (one weight per indexer head; no scale factor)
 * scores [B, row_end - row_begin, ld] float32, written for s <= t only; entries with
 *        s > t are left untouched.  Rows may be computed in chunks by calling with
 *        consecutive [row_begin, row_end) ranges.
 * Requires 0 <= row_begin < row_end <= T, ld >= row_end, ld % 4 == 0, 1 <= H_I <= 64,
 * D_I % 8 == 0 and D_I <= 256.  bf16 with H_I in {1,2,4} and D_I % 32 == 0 runs on MFMA.
 * SA_FP8_E4M3 (qi and ki as E4M3 codes) requires H_I in {1,2,4} and D_I in {32,64,128}
 * (else SA_ERR_UNSUPPORTED); the codes are widened exactly to bf16 inside the kernel and
 * contracted on the bf16 MFMA, so the scores are those of the decoded values with the
 * same float32 accumulation as bf16 inputs.  A positive per-tensor or per-query scale
 * leaves every row's top-k unchanged; fold it into w if the scores themselves matter.
 */
int sa_indexer_scores(const void* qi, const void* ki, const float* w, int B, int T, int H_I,
                      int D_I, int dtype, int row_begin, int row_end, float* scores,
                      int64_t ld, void* stream);

/*
 * Top-k selection.  [IC] body paragraph 2 (select a small subset) and [HS2] "Más
 * precisión con menos memoria" (individual tokens).
 *
 * For each row t in [row_begin, row_end): the min(k, t+1) positions s <= t with the
 * largest scores[b, t - row_begin, s]; ties go to the lower s; -0.0 counts as +0.0.
 * Written ascending to idx[b, t, 0:k] and padded with -1.  Scores must be finite.
 *
 * scores [B, row_end - row_begin, ld] float32 (as written by sa_indexer_scores)
 * idx    [B, T, k] int32; only rows [row_begin, row_end) are written.
 * Requires 1 <= k <= 4096, ld >= row_end and ld % 4 == 0.
 */
int sa_topk_select(const float* scores, int64_t ld, int B, int T, int row_begin, int row_end,
                   int k, int32_t* idx, void* stream);

/*
 * Fused indexer scores + top-k selection.  [IC] body paragraphs 2-3 (the indexer scores
 * every earlier token; only the selected subset is used afterwards).
 *
 * Writes to idx[b, t, 0:k], for t in [row_begin, row_end), exactly what
 * sa_indexer_scores followed by sa_topk_select write (bit for bit), without
 * materialising the score matrix: a strided sample of each row's scores gives a
 * threshold, only scores above it are kept (per 256-key chunk, in position order), and
 * the exact selection runs over those (in registers up to 4096 kept scores, else by
 * passes over the kept lists).  A row whose kept set turns out smaller than k is
 * recomputed in full inside the call; the result never depends on the inputs'
 * distribution, only the time does.
 *
 * qi [B, T, H_I, D_I] and ki [B, T, D_I] bf16 or E4M3 (dtype); w [H_I] float32;
 * idx [B, T, k] int32.
 * workspace: device memory of at least sa_indexer_topk_workspace(...) bytes, no
 * initialisation needed; it holds per-row samples, thresholds and candidate lists (up to
 * 64 lists of 324 entries of 8 bytes per row: about 162 KB per row once row_end exceeds
 * 16,384) and up to 256 MB of slots for rows recomputed in full.
 * Once the call has run, the first 4 bytes of the workspace hold, as a uint32, the
 * number of rows that were recomputed in full (a diagnostic; 0 in the usual case).  The
 * kept set is about 1.3-1.6 k entries; beyond k of about 3000 most rows are selected by
 * list passes, which is slower (the two-step path may be faster there).
 * Requires bf16 or E4M3, H_I in {1, 2, 4}, D_I in {32, 64, 128} (else SA_ERR_UNSUPPORTED:
 * use the two-step path), 1 <= k <= 4096, 0 <= row_begin < row_end <= T <= 262144.
 */
int sa_indexer_topk(const void* qi, const void* ki, const float* w, int B, int T, int H_I,
                    int D_I, int dtype, int row_begin, int row_end, int k, int32_t* idx,
                    void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes sa_indexer_topk needs for these sizes (0 on invalid sizes). */
size_t sa_indexer_topk_workspace(int B, int T, int H_I, int D_I, int row_begin, int row_end,
                                 int k);

/*
 * Sparse attention forward over the selected set.  [IC] body paragraph 2 (attend only
 * to the selected subset), [HS2] "Dos niveles ..." (the most recent tokens are forced
 * into the set), [NSA] "Análisis Profundo" (one selection and one K/V fetch shared by
 * the query heads of a KV group).
 *
 *   S_t = { s in idx[b, t, :] : 0 <= s <= t }  U  { max(0, t-window+1), ..., t }
 *   out[b, t, h, :] = sum_{s in S_t} softmax_s(scale * q[b,t,h,:] . k[b,s,g,:]) v[b,s,g,:]
 *   lse[b, h, t]    = log sum_{s in S_t} exp(scale * q . k)       (natural log)
 *
 * Each key counts once: listed positions inside the window, -1 and any value outside
 * [0, t] are ignored.  Listed positions must be distinct (duplicates are a caller
 * error: they are counted twice, or rejected with SA_ERR_INVALID_ARG under SA_VALIDATE).
 * An empty S_t gives out = 0 and lse = -inf.
 *
 * q   [B, T, Hq, D]  dtype        k, v [B, T, Hkv, D] dtype
 * idx [B, T, topk]   int32        (topk may be 0 with idx == NULL)
 * out [B, T, Hq, D]  dtype        lse  [B, Hq, T] float32, may be NULL
 * Requires D in {64, 128}, window >= 0, topk >= 0, topk + window >= 1.
 * bf16 with Hq/Hkv <= 16 runs the grouped-head MFMA kernel; other cases a VALU kernel.
 */
int sa_sparse_attn_fwd(const void* q, const void* k, const void* v, const int32_t* idx, int B,
                       int T, int Hq, int Hkv, int D, int topk, int window, float scale,
                       int dtype, void* out, float* lse, void* stream);
/*
 * The same for the query rows [row_begin, row_end) only (0 <= row_begin <= row_end <= T):
 * out and lse rows outside the range are not touched, and only idx rows inside it are read,
 * so the attention of a row chunk can run as soon as that chunk's indices exist (on
 * another stream while the next chunk's indices are built).  sa_sparse_attn_fwd is the
 * range [0, T).
 */
int sa_sparse_attn_fwd_rows(const void* q, const void* k, const void* v, const int32_t* idx,
                            int B, int T, int Hq, int Hkv, int D, int topk, int window,
                            float scale, int dtype, int row_begin, int row_end, void* out,
                            float* lse, void* stream);

/*
 * Sparse attention backward.  [NSA] "Puntos Clave" (the backward pass of sparse attention,
 * reported beside the forward).  For the forward of sa_sparse_attn_fwd on the same
 * q, k, v, idx, window and scale, with its out and lse, and the upstream gradient dout:
 *
 *   P[t,h,s] = exp(scale q[t,h].k[s,g] - lse[h,t]) on S_t (0 elsewhere)
 *   dS[t,h,s] = P (dout[t,h].v[s,g] - dout[t,h].out[t,h])
 *   dq[t,h]   = scale sum_s dS[t,h,s] k[s,g]
 *   dk[s,g]   = scale sum_{t, h in g} dS[t,h,s] q[t,h]
 *   dv[s,g]   = sum_{t, h in g} P[t,h,s] dout[t,h]
 *
 * q, k, v, out, dout bf16 in the forward's layouts; idx as for the forward (NULL with
 * topk = 0), in any order; lse [B, Hq, T] float32 from the forward (required).
 * dq [B, T, Hq, D], dk, dv [B, T, Hkv, D] float32: every entry is written.
 *
 * workspace NULL: dk and dv are cleared, then accumulated with float atomics (one per
 * (query, key, feature)); no extra memory, but the atomics bound the call.
 * workspace non-NULL (ws_bytes of device memory, any contents, 16-byte aligned): each
 * (query, key) pair's dK and dV contributions are written as a bf16 row into the
 * workspace, then summed per key in float32 (the query rows go in chunks of as many rows
 * as the workspace holds; sa_sparse_attn_bwd_workspace gives the size for a chunk of
 * `rows` rows, rows <= 0 meaning all T: about B*Hkv*rows*(topk+window)*4*D bytes).  The
 * contributions are rounded to bf16 before the sum (2^-9 relative each).  Needs T <= 2^20
 * and B*T*(topk+window) < 2^31; a workspace too small for one row gives SA_ERR_WORKSPACE.
 * Both ways add in an order that varies from run to run, so the low bits of dk and dv do.
 * Requires bf16, D in {64, 128}, Hq/Hkv <= 16.
 */
int sa_sparse_attn_bwd(const void* q, const void* k, const void* v, const int32_t* idx, int B,
                       int T, int Hq, int Hkv, int D, int topk, int window, float scale,
                       int dtype, const void* out, const float* lse, const void* dout, float* dq,
                       float* dk, float* dv, void* workspace, size_t ws_bytes, void* stream);
size_t sa_sparse_attn_bwd_workspace(int B, int T, int Hkv, int D, int topk, int window,
                                    int rows);

/*
 * Fixed-graph distance attention.  [SLM] "Cómo eligen los tokens a quién escuchar": a
 * fixed list of allowed positions (the token itself, its near predecessors and
 * positions at distances 1, 2, 4, 8, ...), never future ones; the weight grows as the
 * distance between learned 3-D query and key coordinates shrinks, shifted by a learned
 * per-head parameter.
 *
 *   N(t) = { t - o : o in {0, 1, ..., local} U {2^j : 0 <= j < n_pow2}, o <= t }
 *   logit(t, s, h) = -tau * ||cq[b,t,h,:] - ck[b,s,h,:]||^2 + bias[h]
 *   out[b, t, h, :] = sum_{s in N(t)} softmax_s(logit) v[b, s, h, :]
 *
 * Positions that would be negative are dropped.  Distances and softmax run in float32.
 * cq, ck [B, T, H, 3] dtype     v, out [B, T, H, D] dtype     bias [H] float32
 * lse    [B, H, T] float32, may be NULL
 * Requires 0 <= local <= 64, 0 <= n_pow2 <= 30, D % 8 == 0, H * D <= 4096.
 */
int sa_graph_attn_fwd(const void* cq, const void* ck, const void* v, const float* bias,
                      float tau, int B, int T, int H, int D, int local, int n_pow2, int dtype,
                      void* out, float* lse, void* stream);

/*
 * Block mean-pooling of a key cache.  [NSA] "Puntos Clave" (coarse compression).
 *
 *   kbar[b, j, g, :] = (1/block) sum_{i < block} kcache[b, block*j + i, g, :]
 *   for complete blocks j < lens[b] / block (integer division); other rows untouched.
 *
 * kcache [B, Lmax, Hkv, D] dtype; lens [B] int32 on the device (1 <= lens[b] <= Lmax);
 * kbar   [B, Lmax / block, Hkv, D] float32.  Meant to run once per cache, not per step.
 * Requires block in {16, 32, 64, 128}, D % 4 == 0.
 */
int sa_block_meanpool(const void* kcache, const int32_t* lens, int B, int Lmax, int Hkv, int D,
                      int block, int dtype, float* kbar, void* stream);

/*
 * One block-selected decode step.  [NSA] "Puntos Clave" (blockwise selection plus a
 * sliding window), [STAR] paragraph 3 (partial attentions merged by a distributed
 * softmax: here the split-K partials are merged by their log-sum-exp).
 *
 * For each sequence b and KV head g, with L = lens[b]:
 *   score_j = sum_{h in group g} q[b,h,:] . kbar[b,j,g,:]    for complete blocks j < L/block
 *   sel     = the top_blocks best j (ties to the lower j), ascending, padded with -1
 *   U       = { s in block j : j in sel, s < L - window }  U  [max(0, L-window), L)
 *   out[b,h,:] = sum_{s in U} softmax_s(scale * q[b,h,:] . kcache[b,s,g,:]) vcache[b,s,g,:]
 * computed as n_splits partial softmaxes (m, l, o) over slices of U merged with
 * M = max m_i, out = sum e^(m_i-M) o_i / sum e^(m_i-M) l_i, lse = M + log sum e^(m_i-M) l_i.
 *
 * q [B, Hq, D] dtype; kcache, vcache [B, Lmax, Hkv, D] dtype; kbar from sa_block_meanpool;
 * lens [B] int32 on the device; out [B, Hq, D] dtype; lse [B, Hq] float32 or NULL;
 * sel_blocks [B, Hkv, top_blocks] int32 or NULL.
 * n_splits: 0 = automatic, else 1..64.  workspace: device memory of at least
 * sa_sparse_decode_workspace(...) bytes, any contents (the call clears what it needs).
 * Calls that share a workspace must be ordered on one stream.
 * Requires D in {64, 128}, bf16, Hq/Hkv <= 16, block in {16, 32, 64, 128},
 * 1 <= top_blocks <= 64, window >= 0.
 */
int sa_sparse_decode(const void* q, const void* kcache, const void* vcache, const float* kbar,
                     const int32_t* lens, int B, int Lmax, int Hq, int Hkv, int D, int block,
                     int top_blocks, int window, int n_splits, float scale, int dtype, void* out,
                     float* lse, int32_t* sel_blocks, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * sa_sparse_decode without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * sa_sparse_decode (the same kernels run); the workspace is instead a scratch array inside
 * the library, one per GPU, of sa_sparse_decode_noalloc_max_scratch() bytes (16 MiB),
 * held from the first call on that GPU until the process ends.  Sizes whose
 * sa_sparse_decode_workspace(...) exceeds it return SA_ERR_UNSUPPORTED (nothing launched).
 * The stream must belong to the current device.  Every call on one GPU shares that GPU's
 * scratch: calls that overlap in time on one GPU (other streams, other host threads) race
 * and must be serialised by the caller; calls ordered on one stream are safe.
 */
int sa_sparse_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                             const float* kbar, const int32_t* lens, int B, int Lmax, int Hq,
                             int Hkv, int D, int block, int top_blocks, int window, int n_splits,
                             float scale, int dtype, void* out, float* lse, int32_t* sel_blocks,
                             void* stream);

/* Bytes of scratch sa_sparse_decode_noalloc holds per GPU (its size limit). */
size_t sa_sparse_decode_noalloc_max_scratch(void);

/* Workspace bytes sa_sparse_decode needs for these sizes (0 on invalid sizes). */
size_t sa_sparse_decode_workspace(int B, int Lmax, int Hq, int Hkv, int D, int block,
                                  int top_blocks, int window, int n_splits);

/* The n_splits value sa_sparse_decode uses for n_splits == 0 (0 on invalid sizes). */
int sa_sparse_decode_auto_splits(int B, int Lmax, int Hkv, int block, int top_blocks,
                                 int window);

/*
 * NSA compressed branch (prefill).  [NSA] "Puntos Clave": coarse token compression keeps
 * the global context with fewer tokens.  The compressed tokens are the block means of K
 * and V (sa_block_meanpool of each, lens = T), and a query attends to the blocks that are
 * complete at or before it:
 *
 *   out[b, t, h, :] = sum_{j < (t+1)/block} softmax_j(scale * q[b,t,h,:] . kbar[b,j,g,:])
 *                                            * vbar[b,j,g,:],   g = h / (Hq/Hkv)
 *   lse[b, h, t]    = log sum_j exp(scale * q . kbar)   (natural log; -inf, out = 0 when
 *                                                         no block is complete)
 *
 * q, out [B, T, Hq, D] bf16; kbar, vbar [B, T/block, Hkv, D] float32 (rounded to bf16 once
 * per call into the workspace); lse [B, Hq, T] float32 or NULL.
 * workspace: at least sa_cmp_attn_workspace(B, T, Hkv, D, block) bytes, any contents.
 * Requires bf16, D in {64, 128}, Hq/Hkv <= 16, block in {16, 32, 64, 128}.
 */
int sa_cmp_attn_fwd(const void* q, const float* kbar, const float* vbar, int B, int T, int Hq,
                    int Hkv, int D, int block, float scale, int dtype, void* out, float* lse,
                    void* workspace, size_t ws_bytes, void* stream);
size_t sa_cmp_attn_workspace(int B, int T, int Hkv, int D, int block);

/*
 * NSA block selection (prefill).  [NSA] "Puntos Clave": fine-grained selection in blocks
 * ("Utiliza la selección de tokens por bloques").  For each row t in [row_begin, row_end):
 *
 *   score_j = sum_h q[b,t,h,:] . kbar[b,j,g(h),:]   (float32; every query head)
 *
 * over the complete blocks j < (t+1)/block; the top_blocks best (ties to the lower j; all
 * of them when fewer are complete), j_0 < j_1 < ..., are written as their tokens, the
 * blocks interleaved: idx[b, t, e*top_blocks + i] = j_i*block + e (e < block), -1 where
 * block i does not exist, so idx [B, T, top_blocks*block] int32 feeds sa_sparse_attn_fwd
 * (window 0) as the selected branch; each 32-entry step of the attention then reads rows
 * of many blocks instead of one run of consecutive rows.  One selection per query row,
 * shared by all heads, as for the token-level top-k.
 * q [B, T, Hq, D] bf16 or float32; kbar as for sa_cmp_attn_fwd.
 * workspace: at least sa_block_select_workspace(...) bytes (scores and summed queries).
 * Requires 1 <= top_blocks <= 64, block in {16, 32, 64, 128}, T/block <= 4096.
 */
int sa_block_select(const void* q, const float* kbar, int B, int T, int Hq, int Hkv, int D,
                    int block, int top_blocks, int dtype, int row_begin, int row_end,
                    int32_t* idx, void* workspace, size_t ws_bytes, void* stream);
size_t sa_block_select_workspace(int B, int T, int Hkv, int D, int block, int row_begin,
                                 int row_end);

/*
 * Block means rounded to bf16: the same means as sa_block_meanpool (float32 sums of the
 * block's rows divided by block), written as bf16 (nearest even) for the attention kernels
 * that read pooled rows as MFMA operands (the compressed branch of decode).
 * kbar [B, Lmax/block, Hkv, D] bf16, complete blocks only (other rows untouched).
 */
int sa_block_meanpool_bf16(const void* kcache, const int32_t* lens, int B, int Lmax, int Hkv,
                           int D, int block, int dtype, void* kbar, void* stream);

/*
 * NSA decode branches over one contiguous row range.  [NSA] "Puntos Clave" (compression,
 * sliding window).  For each sequence b with L = lens[b]:
 *   kind 0 (window):     rows [max(0, L - window), L) of keys/vals = the K/V caches
 *                        [B, Lrows = Lmax, Hkv, D];
 *   kind 1 (compressed): rows [0, L / block) of keys/vals = the bf16 block means
 *                        (sa_block_meanpool_bf16 of K and of V) [B, Lrows = Lmax/block, Hkv, D];
 *   out[b, h, :] = sum_{s in range} softmax_s(scale * q[b,h,:] . keys[b,s,g,:]) vals[b,s,g,:]
 *   lse[b, h]    = log sum exp (natural log; -inf and out = 0 for an empty range)
 * The selected branch is sa_sparse_decode with window 0 (all tokens of the chosen blocks).
 * q, out [B, Hq, D] bf16; lens [B] int32 on the device, 0 <= lens[b] <= Lmax (values
 * outside are clamped to [0, Lrows] for kind 0 and [0, Lrows * block] for kind 1);
 * lse [B, Hq] float32 or NULL.
 * n_splits (1..64) workgroups share each (sequence, KV head)'s range, their partial softmaxes
 * merged by log-sum-exp [STAR paragraph 3]; with n_splits > 1, workspace holds at least
 * sa_nsa_decode_branch_workspace(B, Hq, Hkv, D, n_splits) bytes, ZERO-FILLED before its first
 * use (every call leaves its counters at zero again; calls sharing a workspace must be
 * ordered on one stream).  workspace may be NULL with n_splits = 1.
 * Requires bf16, D in {64, 128}, Hq/Hkv <= 16, block in {16, 32, 64, 128}.
 */
int sa_nsa_decode_branch(const void* q, const void* keys, const void* vals,
                         const int32_t* lens, int B, int Lrows, int Hq, int Hkv, int D, int kind,
                         int block, int window, float scale, int dtype, void* out, float* lse,
                         int n_splits, void* workspace, size_t ws_bytes, void* stream);
size_t sa_nsa_decode_branch_workspace(int B, int Hq, int Hkv, int D, int n_splits);

/*
 * NSA decode: the compressed and the window branch of sa_nsa_decode_branch (kinds 1 and 0)
 * in one launch.  [NSA] "Puntos Clave": the branches are independent; here they share the
 * launch's fixed costs and run side by side.  Results equal those of the two
 * sa_nsa_decode_branch calls bit for bit (each branch's workgroups run that call's code).
 * kbar16, vbar16 [B, Lmax/block, Hkv, D] bf16 (sa_block_meanpool_bf16 of K and of V);
 * kcache, vcache [B, Lmax, Hkv, D] bf16; q, out_cmp, out_win [B, Hq, D] bf16; lens [B]
 * int32 on the device (clamped as for sa_nsa_decode_branch); lse_cmp, lse_win [B, Hq]
 * float32 or NULL.  n_splits_cmp, n_splits_win in 1..64; workspace: at least
 * sa_nsa_decode_cmp_win_workspace(...) bytes (the compressed side's area, then the window
 * side's), ZERO-FILLED before its first use and left that way by every call (calls sharing
 * a workspace must be ordered on one stream); may be NULL when both split counts are 1.
 * Requires bf16, D in {64, 128}, Hq/Hkv <= 16, block in {16, 32, 64, 128}, Lmax >= block.
 */
int sa_nsa_decode_cmp_win(const void* q, const void* kbar16, const void* vbar16,
                          const void* kcache, const void* vcache, const int32_t* lens, int B,
                          int Lmax, int Hq, int Hkv, int D, int block, int window, float scale,
                          int dtype, void* out_cmp, float* lse_cmp, void* out_win, float* lse_win,
                          int n_splits_cmp, int n_splits_win, void* workspace, size_t ws_bytes,
                          void* stream);
size_t sa_nsa_decode_cmp_win_workspace(int B, int Hq, int Hkv, int D, int n_splits_cmp,
                                       int n_splits_win);

/*
 * NSA gated combine.  [NSA] "Puntos Clave" (three branches) -- the page does not say how
 * they are joined; NSA gates them per head with weights it learns from the query, which
 * are an input here:
 *   out = gates[..., 0] * o_cmp + gates[..., 1] * o_slc + gates[..., 2] * o_win
 * o_cmp, o_slc, o_win, out [B, T, Hq, D] bf16 (out may alias an input); gates
 * [B, T, Hq, 3] float32.  Requires D % 8 == 0.
 */
int sa_nsa_combine(const void* o_cmp, const void* o_slc, const void* o_win, const float* gates,
                   int B, int T, int Hq, int D, int dtype, void* out, void* stream);

/* Human-readable name of a status code (static storage). */
const char* sa_status_str(int status);

/* Detail of the last error on the calling host thread ("" if none). */
const char* sa_last_error(void);

/* SA_VERSION of the built library. */
int sa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSA_SA_H */
