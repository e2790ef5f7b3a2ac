/*
 * wf.h — exact attention forward on AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operation is exact scaled-dot-product attention,
 *     out = softmax(scale * Q K^T + mask) V,
 * as specified by the pages this library implements:
 *   [CORE]  WorldFoundry API reference, page "Core 注意力" (core attention):
 *           section "选择最窄的入口" (choose the narrowest entry point): the PyTorch SDPA
 *           contract, GQA expansion, exact matmul path; the sentence after the CPU/GPU
 *           example: a bool mask marks the scores that are kept, a float mask is added
 *           to the score matrix, dropout must be passed as 0 at inference; section
 *           "Block KV cache 的调用顺序" (block KV cache call order): chunk protocol and
 *           the sink + window rule.
 *   [MLA]   Huawei Ascend CANN ATB page "MLA Prefill": the definition of
 *           AtbMLAPreFillGetWorkspaceSize / AtbMLAPreFill and its parameter table.
 *
 * Conventions for every entry point:
 *   - All tensor data, sequence-length arrays and workspaces are caller-owned DEVICE
 *     memory. The library never allocates or frees device memory and never synchronises
 *     the stream; kernels are enqueued on `stream` (a hipStream_t, NULL = default stream).
 *   - Arguments are validated completely before anything is enqueued. A call that returns
 *     an error has enqueued nothing and changed no state. wf_last_error() gives the
 *     reason (thread-local). Faults inside kernels surface at the caller's next
 *     synchronisation, as for any asynchronous HIP work.
 *   - Tensor descriptors hold strides in ELEMENTS. The innermost (head-dim) stride must
 *     be 1; row/head/batch strides and base pointers must keep every row 16-byte
 *     aligned (a multiple of 8 elements for 16-bit data, 4 for fp32).
 *   - Results are deterministic: the same inputs give bit-identical outputs on every run
 *     (no atomics in any reduction; fixed split and combine order).
 *   - A call enqueues kernel launches only (no memset, copy, allocation or host wait), so a
 *     sequence of calls may be captured into a HIP graph and replayed; the kernel arguments
 *     are fixed at capture, and so are the host-side cache state changes a captured block
 *     KV cache call makes (a replay repeats the captured chunks).
 */
#ifndef WF_H_
#define WF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WF_F32 = 0,   /* float32                                   */
  WF_F16 = 1,   /* IEEE binary16                             */
  WF_BF16 = 2,  /* bfloat16                                  */
  WF_BOOL = 3,  /* one byte per element, nonzero = keep      */
  WF_I32 = 4
} wf_dtype;

typedef enum {
  WF_OK = 0,
  WF_ERR_NULL = 1,         /* a required pointer or descriptor is NULL                 */
  WF_ERR_SHAPE = 2,        /* shapes disagree with each other or with the operation    */
  WF_ERR_DTYPE = 3,        /* unsupported or mismatched element type                   */
  WF_ERR_LAYOUT = 4,       /* inner stride != 1, misaligned pointer or stride          */
  WF_ERR_UNSUPPORTED = 5,  /* dropout_p != 0, head dim not built, mask with causal ... */
  WF_ERR_CHUNK_ORDER = 6,  /* block KV cache: chunk index skipped or went backwards    */
  WF_ERR_CACHE_CONFIG = 7, /* block KV cache: sink/window/chunk sizes break the rule   */
  WF_ERR_WORKSPACE = 8,    /* workspace NULL, misaligned or smaller than required      */
  WF_ERR_HIP = 9           /* a HIP launch reported an error                           */
} wf_status;

/* A strided view of caller-owned device memory. Only the first `ndim` entries of shape
 * and stride are read. A stride of 0 broadcasts that dimension (masks only). */
typedef struct {
  void* data;
  int32_t dtype;      /* wf_dtype */
  int32_t ndim;       /* 1..4     */
  int64_t shape[4];
  int64_t stride[4];  /* in elements */
} wf_tensor;

/* ---------------------------------------------------------------------------------------
 * wf_sdpa_fwd — split-head scaled-dot-product attention forward ([CORE] "选择最窄的入口":
 * PyTorch SDPA contract with GQA expansion; mask sentence after the CPU/GPU example).
 *
 *   q    [B, Hq,  Lq, Dqk]   f32 | f16 | bf16
 *   k    [B, Hkv, Lk, Dqk]   same dtype as q
 *   v    [B, Hkv, Lk, Dv ]   same dtype as q
 *   mask NULL, or 4-d broadcastable to [B, Hq, Lq, Lk] (stride 0 on broadcast dims, key
 *        stride 1): WF_BOOL = keep where nonzero; a float dtype (q's dtype or WF_F32) is
 *        added to the scaled score (-inf drops the key).
 *   is_causal  nonzero: key j is kept for query i iff j <= i (top-left alignment).
 *              Not accepted together with a mask (WF_ERR_UNSUPPORTED).
 *   dropout_p  must be 0 (inference); anything else is WF_ERR_UNSUPPORTED.
 *   scale      multiplies Q K^T; NaN selects 1/sqrt(Dqk). Must be finite and > 0.
 *   out  [B, Hq, Lq, Dv]     same dtype as q (written; rounding to nearest even)
 *   lse  NULL, or device float32 [B*Hq*Lq] contiguous: natural-log sum of exp of the
 *        scaled, masked scores per query (-inf for a query that keeps no key).
 * GQA: query head h reads KV head h / (Hq / Hkv); Hq must be a multiple of Hkv.
 * A query that keeps no key gets out = 0.
 * Built head dims: 16-bit q: (Dqk, Dv) in {(64,64), (64,96), (128,128), (128,64)}; fp32:
 * Dqk in {64,128}, Dv in {64, 96, 128}. Others return WF_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------------------- */
int wf_sdpa_fwd(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v,
                const wf_tensor* mask, int is_causal, float dropout_p, float scale,
                wf_tensor* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------------------
 * wf_sdpa_rope_fwd — wf_sdpa_fwd with rotary position embedding applied to q and k first
 * ([CORE] opening paragraph: applying RoPE is one of the core's jobs; no convention is given).
 * The first rot_dim dims of every q and k head turn pairwise: pair i of a row at position p
 * by cos[p * rot_dim/2 + i], sin[...] (caller-tabulated, so any frequency schedule works):
 *   (x_a, x_b) -> (x_a cos - x_b sin, x_b cos + x_a sin),
 * pairs (i, i + rot_dim/2) for style 0 (rotate-half) or (2i, 2i + 1) for style 1
 * (interleaved). Query row r sits at position q_pos0 + r, key row j at k_pos0 + j; v is not
 * rotated. One launch writes a rotated contiguous copy of k, and of q, into `workspace`, then
 * the attention of wf_sdpa_fwd runs on them (same masks, causal rule, lse, dtypes, head dims).
 * When the call takes the persistent kernel (16-bit, no mask) with style 0 over the whole
 * head or with style 1, q is instead turned inside that kernel as it is read (fp32, rounded
 * once), and only k is copied; the workspace size does not depend on which happens.
 *   rope->cos, rope->sin  device fp32 [max_pos, rot_dim/2], contiguous, 16-byte aligned;
 *   rot_dim 0 (no rotation) or a multiple of 16 up to the head dim; positions must lie in the
 *   table. workspace: at least wf_sdpa_rope_workspace_size(q, k) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------------------- */
typedef struct {
  const float* cos;
  const float* sin;
  int64_t max_pos;
  int rot_dim;
  int style;
  int64_t q_pos0, k_pos0;
} wf_rope;

size_t wf_sdpa_rope_workspace_size(const wf_tensor* q, const wf_tensor* k);
int wf_sdpa_rope_fwd(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v,
                     const wf_tensor* mask, int is_causal, float scale, const wf_rope* rope,
                     wf_tensor* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ---------------------------------------------------------------------------------------
 * wf_sdpa_decode — the same attention as wf_sdpa_fwd for few queries against a long K/V
 * (decode, and speculative decoding with several new tokens: [MLA] maskType SPEC / calcType
 * SPEC, q lengths above 1). The key range is split across work groups, each writing an fp32
 * partial output and log-sum-exp into `workspace`, and a combine kernel merges the splits.
 *   q [B, Hq, Lq, D], k [B, Hkv, Lk, D], v [B, Hkv, Lk, D], out [B, Hq, Lq, D]; f16 | bf16;
 *   D in {64, 128}; Hq a multiple of Hkv (GQA as in wf_sdpa_fwd). No mask.
 *   is_causal: the Lq queries are the last Lq positions of the key sequence (bottom-right:
 *     query i keeps key j iff j <= i + Lk - Lq) — unlike wf_sdpa_fwd's top-left rule.
 *   scale as in wf_sdpa_fwd. lse: NULL, or device fp32 [B, Hq, Lq] (natural log).
 *   workspace: device memory of at least wf_sdpa_decode_workspace_size(q, k, v, is_causal)
 *     bytes (0 = unsupported shape), 256-byte aligned; its size depends on the shapes only.
 * Rows that keep no key are 0 (lse -inf). Errors as for wf_sdpa_fwd, plus WF_ERR_WORKSPACE.
 * ------------------------------------------------------------------------------------- */
size_t wf_sdpa_decode_workspace_size(const wf_tensor* q, const wf_tensor* k,
                                     const wf_tensor* v, int is_causal);
int wf_sdpa_decode(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v, int is_causal,
                   float scale, wf_tensor* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * MLA prefill over a packed variable-length batch ([MLA] definition and parameter table).
 *
 *   q       [nTq, Hq,  Dv]  f16 | bf16 (the value-width "nope" part of the query)
 *   q_rope  [nTq, Hq,  64]  rotary part of the query (same dtype)
 *   k       [nTk, Hkv, Dv]  k_rope [nTk, Hkv, 64]   v [nTk, Hkv, Dv]   (packed), or
 *           [batch, max_seq, Hkv, Dv] / [batch, max_seq, Hkv, 64] / [batch, max_seq, Hkv, Dv]
 *           (padded: the page's [batch, max_seq, kv_head*d] viewed with the head split
 *           out). All three take the same form; a 4-d k means padded.
 *           A concatenated cache (k_rope stored right after k in each token row) is the
 *           same call with k_rope->data = k->data + Dv and matching strides, in either form.
 *   q_seqlen, kv_seqlen  device int32 [batch]; sequence i owns query tokens
 *           [sum_{t<i} q_seqlen[t], ... + q_seqlen[i]) and likewise for packed keys/values;
 *           with padded keys/values it owns rows [0, kv_seqlen[i]) of batch entry i.
 *   head_num, kv_head_num  Hq, Hkv (Hq a multiple of Hkv; q head h reads kv head
 *           h / (Hq/Hkv)).
 *   qk_scale  multiplies (q . k + q_rope . k_rope); finite and > 0.
 *   mask_type 0 = none (UNDEFINED: an all-zero mask), 1 = causal, aligned bottom-right:
 *           query i of a sequence keeps key j iff j <= i + kv_len - q_len. This also serves
 *           as the page's MASK_TYPE_SPEC (new tokens at the end of a longer cached sequence,
 *           q lengths above 1); the page gives that enum no number.
 *   out     [nTq, Hq, Dv], dtype of q. Rows of queries that keep no key are 0.
 *   workspace  device memory of at least
 *           wf_varlen_mla_prefill_workspace_size(batch, nTq, head_num) bytes, 256-byte
 *           aligned; it holds the tile schedule built on the device from the lengths.
 * Score width is Dv + 64, Dv in {128, 64} (the built instantiations). The query heads of a
 * KV head share each K/V tile, four (or two) to a work group when Hq / Hkv allows.
 * If the device lengths are negative, sum past nTq (or, packed, nTk) or, padded, exceed
 * max_seq, no attention is computed (out is left as it was) and word 2 of the workspace
 * (int32) is set to 1; it is 0 after a good call. A mix of packed and padded k / k_rope / v
 * is WF_ERR_LAYOUT.
 * Where this differs from the two-phase interface the page defines: the workspace size is a
 * function of (batch, nTq) rather than of the largest query length (the schedule is built
 * on the device from the lengths, so the host never reads them and the bound must come from
 * the token count; head_num is accepted and unused), the call itself takes no max_q_len for
 * the same reason, and `stream` is a hipStream_t passed as void*.
 * ------------------------------------------------------------------------------------- */
size_t wf_varlen_mla_prefill_workspace_size(int batch, int64_t total_q_tokens, int head_num);
int wf_varlen_mla_prefill(const wf_tensor* q, const wf_tensor* q_rope, const wf_tensor* k,
                          const wf_tensor* k_rope, const wf_tensor* v,
                          const int32_t* q_seqlen, const int32_t* kv_seqlen, int batch,
                          int head_num, int kv_head_num, float qk_scale, int mask_type,
                          wf_tensor* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* wf_varlen_mla_prefill without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, layouts and results as wf_varlen_mla_prefill; the workspace
 * is a fixed 1 MiB device array inside the library (one per device, held until the process
 * ends). It serves any call whose wf_varlen_mla_prefill_workspace_size(batch, nTq, head_num)
 * is at most 1 MiB: 8 bytes per work item (nTq / 64 + batch items) plus two (batch + 1)-entry
 * offset tables, e.g. 1024 sequences with 8 million query tokens in all. A call that needs
 * more returns WF_ERR_WORKSPACE and enqueues nothing. The call allocates nothing. All calls on one device share the array:
 * calls that overlap on a device (two streams, or two threads) race and must be serialised
 * by the caller; each call's schedule kernel rewrites everything the attention kernel reads,
 * so consecutive calls need nothing cleared. Bad device lengths compute nothing, as above;
 * the error word is then in the internal array and not visible to the caller. */
int wf_varlen_mla_prefill_noalloc(const wf_tensor* q, const wf_tensor* q_rope, const wf_tensor* k,
                                  const wf_tensor* k_rope, const wf_tensor* v,
                                  const int32_t* q_seqlen, const int32_t* kv_seqlen, int batch,
                                  int head_num, int kv_head_num, float qk_scale, int mask_type,
                                  wf_tensor* out, void* stream);

/* ---------------------------------------------------------------------------------------
 * Rolling block KV cache ([CORE] "Block KV cache 的调用顺序").
 *
 * The cache is two caller-owned device tensors k_cache [B, Hkv, cache_len, Dk] and
 * v_cache [B, Hkv, cache_len, Dv] plus this caller-owned host state. The first `sink`
 * tokens are never evicted; the next `window` slots form a ring that holds the newest
 * tokens. Token t lives in slot t if t < sink, else sink + (t - sink) mod window.
 * Rules: sink + window == cache_len; cache_len % chunk == 0; window >= chunk.
 * A snapshot of the cache is a copy of the state and the two tensors.
 * ------------------------------------------------------------------------------------- */
typedef struct {
  int64_t cache_len, sink, window, chunk;
  int64_t last_chunk; /* -1 while empty */
} wf_block_kv_state;

int wf_block_kv_init(wf_block_kv_state* st, int64_t cache_len, int64_t sink, int64_t window,
                     int64_t chunk);

/* before_update(chunk_idx) + update(k_new, v_new) + after_update(chunk_idx) in one call:
 * chunk_idx must equal last_chunk (overwrite the same logical chunk) or last_chunk + 1
 * (append / roll); anything else is WF_ERR_CHUNK_ORDER with nothing changed.
 *   k_new [B, Hkv, chunk, Dk], v_new [B, Hkv, chunk, Dv], same dtype as the caches
 *   (f32 | f16 | bf16). The copy is enqueued on `stream`; st->last_chunk is updated on
 *   success. */
int wf_block_kv_cache_update(wf_block_kv_state* st, int64_t chunk_idx,
                             const wf_tensor* k_new, const wf_tensor* v_new,
                             wf_tensor* k_cache, wf_tensor* v_cache, void* stream);

/* Number of visible tokens (sink prefix plus the window, including the newest chunk) and,
 * if phys_index is not NULL, the cache slot of each visible token in chronological order
 * (host array of n_visible entries). Host-only; enqueues nothing. */
int wf_block_kv_visible(const wf_block_kv_state* st, int64_t* n_visible,
                        int64_t* phys_index);

/* Writes the visible tokens of `cache` [B, H, cache_len, D] in chronological order into
 * logical_out [B, H, n_visible, D] (same dtype), using the same slot map as the attend
 * kernel. A test aid for checking the cache bit-exactly. */
int wf_block_kv_gather(const wf_block_kv_state* st, const wf_tensor* cache,
                       wf_tensor* logical_out, void* stream);

/* Attention of the current chunk's queries over every visible cached token (including
 * the chunk itself). The kernel reads the keys in chronological order (the sink prefix,
 * then the window from its oldest token) through the slot map of wf_block_kv_visible.
 *   q [B, Hq, Lq, Dk] (Hq a multiple of Hkv), out [B, Hq, Lq, Dv]; 16-bit dtypes with
 *   (Dk, Dv) in {(64,64), (128,128)}. scale as in wf_sdpa_fwd.
 *   is_causal 0: every query sees every visible token (the page's attend). 1 (an addition
 *     to the page's protocol): the Lq queries are the last Lq visible tokens (bottom-right:
 *     query i keeps visible token j iff j <= i + n_vis - Lq).
 *   workspace: at least wf_block_kv_attend_workspace_size(...) bytes, 256-byte aligned;
 *   it holds per-split partial results (fp32) that a combine kernel merges. */
size_t wf_block_kv_attend_workspace_size(const wf_block_kv_state* st, int B, int Hq, int Lq,
                                         int Dv);
int wf_block_kv_attend(const wf_block_kv_state* st, const wf_tensor* q,
                       const wf_tensor* k_cache, const wf_tensor* v_cache, int is_causal,
                       float scale, wf_tensor* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* wf_block_kv_cache_update(st, chunk_idx, k_new, v_new, k_cache, v_cache) followed by
 * wf_block_kv_attend(st, q, ...) in one attention launch (plus the combine): the attend's
 * work groups also copy the chunk into its ring slots, and read the chunk's own rows from
 * k_new / v_new (the slots they overwrite are not visible any more, so the launch never reads
 * a slot it writes). Same arguments, checks, results and cache contents as the two calls;
 * the workspace is the attend's. All checks of both calls run before anything is enqueued;
 * on any error neither the state nor the caches change. Rows or strides that are not
 * multiples of 16 bytes take the two calls one by one. */
int wf_block_kv_update_attend(wf_block_kv_state* st, int64_t chunk_idx, const wf_tensor* k_new,
                              const wf_tensor* v_new, wf_tensor* k_cache, wf_tensor* v_cache,
                              const wf_tensor* q, int is_causal, float scale, wf_tensor* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable status name, and the thread-local detail of the last failed call. */
const char* wf_status_string(int status);
const char* wf_last_error(void);

/* Hex sha256 of the sources, headers and compile flags this library was built from (static
 * string). The Python package compares it with the tree it sits in and refuses a stale build. */
const char* wf_build_id(void);

/* Kernel-selection overrides, for tests that must reach every kernel shape and for tuning
 * (not part of the pages' operation; every setting computes the same attention).
 * Process-wide values, initialised once from the environment variables WF_TUNE_<NAME>
 * (upper-case name) on first use, then changed only here; -1 restores the automatic choice.
 * Names: "hpw" (query heads per work group), "persist" (0: no persistent 32-query kernel),
 * "q64" (1: the persistent 64-query-wave kernel where it applies; off by default),
 * "qpw" (32 | 64: queries per wave of the one-item-per-group kernels), "nw" (4: waves per
 * group of the 32-query kernel), "decode_pack" (0: no (head, position) row packing in wf_sdpa_decode), "decode_groups",
 * "decode_min_tiles" (split plan of wf_sdpa_decode), "mla_xcd" (0: no per-XCD split of the
 * MLA prefill), "attend_groups", "attend_nw" (4 | 8: waves per group when each KV head
 * has one query head), "attend_min_tiles" (split plan of wf_block_kv_attend and
 * wf_block_kv_update_attend), "mask_pre" (0: masked calls without the lse keep Q as given and scale
 * every score in fp32). Changing a value while
 * another thread launches work races with that launch's choice (never with its result's
 * correctness). Returns WF_ERR_UNSUPPORTED for an unknown name, WF_ERR_NULL for a NULL
 * value pointer. */
int wf_tune_set(const char* name, int value);
int wf_tune_get(const char* name, int* value);

#ifdef __cplusplus
}
#endif
#endif /* WF_H_ */
