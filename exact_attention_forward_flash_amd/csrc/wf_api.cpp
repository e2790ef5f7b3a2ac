// C-ABI entry points (include/wf.h): argument validation, kernel selection from the compiled
// instantiation tables, launch geometry and the block KV cache state machine.
// Validation completes before anything is enqueued; a failing call changes nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cctype>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "wf.h"
#include "wf_internal.hpp"

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
  return WF_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(WF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int esize(int dt) {
  switch (dt) {
    case WF_F32: return 4;
    case WF_F16: return 2;
    case WF_BF16: return 2;
    case WF_BOOL: return 1;
    case WF_I32: return 4;
    default: return 0;
  }
}

bool is_float_dt(int dt) { return dt == WF_F32 || dt == WF_F16 || dt == WF_BF16; }

int64_t numel(const wf_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// Checks a data tensor: rank, non-negative shape, inner stride 1, every row start
// 16-byte aligned (base pointer and all outer strides).
int check_data(const wf_tensor* t, const char* name, int ndim) {
  if (t == nullptr) return fail(WF_ERR_NULL, "%s is NULL", name);
  if (t->ndim != ndim) return fail(WF_ERR_SHAPE, "%s must be %d-d, got %d-d", name, ndim, t->ndim);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(WF_ERR_SHAPE, "%s has a negative dimension", name);
  if (!is_float_dt(t->dtype)) return fail(WF_ERR_DTYPE, "%s must be f32, f16 or bf16", name);
  if (numel(t) == 0) return WF_OK;
  if (t->data == nullptr) return fail(WF_ERR_NULL, "%s->data is NULL", name);
  if (t->stride[ndim - 1] != 1 && t->shape[ndim - 1] != 1)
    return fail(WF_ERR_LAYOUT, "%s: innermost stride must be 1", name);
  const int es = esize(t->dtype);
  const int64_t al = 16 / es;
  if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
    return fail(WF_ERR_LAYOUT, "%s: data pointer must be 16-byte aligned", name);
  for (int i = 0; i < ndim - 1; ++i)
    if (t->shape[i] > 1 && t->stride[i] % al != 0)
      return fail(WF_ERR_LAYOUT, "%s: stride[%d] = %lld is not a multiple of %lld elements", name,
                  i, (long long)t->stride[i], (long long)al);
  if ((t->shape[ndim - 1] * es) % 16 != 0)
    return fail(WF_ERR_LAYOUT, "%s: rows must be a multiple of 16 bytes", name);
  return WF_OK;
}

int64_t st(const wf_tensor* t, int i) { return t->shape[i] == 1 ? 0 : t->stride[i]; }

// Cache copies accept any row width: only the inner stride and element alignment matter.
// *unit16 is cleared when a tensor does not allow 16-byte copies.
int check_cache_data(const wf_tensor* t, const char* name, bool* unit16) {
  if (t == nullptr) return fail(WF_ERR_NULL, "%s is NULL", name);
  if (t->ndim != 4) return fail(WF_ERR_SHAPE, "%s must be 4-d [B,H,S,D]", name);
  for (int i = 0; i < 4; ++i)
    if (t->shape[i] < 0) return fail(WF_ERR_SHAPE, "%s has a negative dimension", name);
  if (!is_float_dt(t->dtype)) return fail(WF_ERR_DTYPE, "%s must be f32, f16 or bf16", name);
  if (numel(t) == 0) return WF_OK;
  if (t->data == nullptr) return fail(WF_ERR_NULL, "%s->data is NULL", name);
  if (t->stride[3] != 1 && t->shape[3] != 1)
    return fail(WF_ERR_LAYOUT, "%s: innermost stride must be 1", name);
  const int es = esize(t->dtype);
  if (reinterpret_cast<uintptr_t>(t->data) % es != 0)
    return fail(WF_ERR_LAYOUT, "%s: data pointer is not aligned to its element size", name);
  if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0 || (t->shape[3] * es) % 16 != 0) *unit16 = false;
  for (int i = 0; i < 3; ++i)
    if ((t->stride[i] * es) % 16 != 0) *unit16 = false;
  return WF_OK;
}

// Kernel-selection overrides for tests and tuning: WF_TUNE_<NAME> from the environment, read
// once on first use, then changed only through wf_tune_set. -1 = automatic choice.
enum TuneKey { T_HPW, T_PERSIST, T_Q64, T_QPW, T_NW, T_DECODE_PACK, T_DECODE_GROUPS,
               T_DECODE_MIN_TILES, T_MLA_XCD, T_ATTEND_GROUPS, T_ATTEND_NW, T_ATTEND_MIN_TILES,
               T_MASK_PRE, T_COUNT };
const char* const kTuneNames[T_COUNT] = {"hpw", "persist", "q64", "qpw", "nw", "decode_pack",
                                         "decode_groups", "decode_min_tiles", "mla_xcd",
                                         "attend_groups", "attend_nw", "attend_min_tiles",
                                         "mask_pre"};
std::atomic<int>* tune_table() {
  static std::atomic<int> t[T_COUNT];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int i = 0; i < T_COUNT; ++i) {
      std::string env = "WF_TUNE_";
      for (const char* c = kTuneNames[i]; *c; ++c) env += (char)std::toupper((unsigned char)*c);
      const char* v = getenv(env.c_str());
      t[i].store(v ? atoi(v) : -1, std::memory_order_relaxed);
    }
  });
  return t;
}
int tune(TuneKey k) { return tune_table()[k].load(std::memory_order_relaxed); }
int tune_key(const char* name) {
  if (name == nullptr) return -1;
  for (int i = 0; i < T_COUNT; ++i)
    if (std::strcmp(name, kTuneNames[i]) == 0) return i;
  return -1;
}
// HPW override: a set value that divides G and does not exceed the automatic choice.
int tuned_hpw(int hpw, int G) {
  const int h = tune(T_HPW);
  return (h >= 1 && h <= hpw && G % h == 0) ? h : hpw;
}

// qpw: queries per wave (32 or 64), 0 = any. nw, hpw: 0 = any.
const wf::AttnEntry* find_attn(int dtype, int dqk, int dqk1, int dv, int nw, int hpw, int mask,
                               int causal, int mode, int qpw = 32) {
  typedef const wf::AttnEntry* (*TableFn)(int*);
  static const TableFn tables[] = {wf::attn_table_sdpa_bf16_d64, wf::attn_table_sdpa_bf16_d128,
                                   wf::attn_table_sdpa_f16_d64,  wf::attn_table_sdpa_f16_d128,
                                   wf::attn_table_sdpa_bf16_dmix, wf::attn_table_sdpa_f16_dmix,
                                   wf::attn_table_mla,           wf::attn_table_mla_v64,
                                   wf::attn_table_split_bf16,
                                   wf::attn_table_split_f16,     wf::attn_table_splitp_bf16,
                                   wf::attn_table_splitp_f16,    wf::attn_table_splitu_bf16,
                                   wf::attn_table_splitu_f16,
                                   wf::attn_table_w_bf16_d64,    wf::attn_table_w_bf16_d128,
                                   wf::attn_table_w_f16_d64,     wf::attn_table_w_f16_d128,
                                   wf::attn_table_p_bf16_d64,    wf::attn_table_p_bf16_d128,
                                   wf::attn_table_p_f16_d64,     wf::attn_table_p_f16_d128,
                                   wf::attn_table_p_rope_bf16,   wf::attn_table_p_rope_f16,
                                   wf::attn_table_p_ropei_bf16,  wf::attn_table_p_ropei_f16,
                                   wf::attn_table_q_bf16_d128,   wf::attn_table_q_f16_d128};
  for (TableFn f : tables) {
    int n = 0;
    const wf::AttnEntry* t = f(&n);
    for (int i = 0; i < n; ++i) {
      const wf::AttnEntry& e = t[i];
      if (e.dtype == dtype && e.dqk == dqk && e.dqk1 == dqk1 && e.dv == dv &&
          (nw == 0 || e.nw == nw) && (hpw == 0 || e.hpw == hpw) && e.mask == mask &&
          e.causal == causal && e.mode == mode && (qpw == 0 || e.qpw == qpw))
        return &e;
    }
  }
  return nullptr;
}

const wf::F32Entry* find_f32(int dqk, int dv, int mask, int causal, bool ks = false) {
  int n = 0;
  const wf::F32Entry* t = ks ? wf::attn_table_f32_ks(&n) : wf::attn_table_f32(&n);
  for (int i = 0; i < n; ++i)
    if (t[i].dqk == dqk && t[i].dv == dv && t[i].mask == mask && t[i].causal == causal) return &t[i];
  return nullptr;
}

int kernel_dtype(int dt) { return dt == WF_BF16 ? wf::DT_BF16 : dt == WF_F16 ? wf::DT_F16 : wf::DT_F32; }

// Compute units of the current device (0 if the query fails), cached per device.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch(const void* fn, dim3 grid, dim3 block, wf::FwdArgs& a, hipStream_t s) {
  void* args[] = {&a};
  return hipLaunchKernel(fn, grid, block, args, 0, s);
}

int resolve_scale(float scale, int64_t dqk, float* out) {
  if (std::isnan(scale)) {
    *out = (float)(1.0 / std::sqrt((double)dqk));
    return WF_OK;
  }
  if (!std::isfinite(scale) || scale <= 0.f)
    return fail(WF_ERR_UNSUPPORTED, "scale must be finite and > 0 (or NaN for 1/sqrt(d))");
  *out = scale;
  return WF_OK;
}

// Persistent form of the 32-query kernel (one work group per CU walking a list of work
// items): calls without a mask whose Q/K/V copy offsets fit in 32 bits and, when causal, whose
// work groups cover one 64-key tile of query positions (HPW = 4). Returns the table entry and
// sets the query-tile count and the grid, or returns nullptr when the call takes the
// one-item-per-group kernels. rope: 0, or the variant that turns Q by a rotary table
// (1 rotate-half over the whole head, 2 interleaved). WF_TUNE_PERSIST=0 turns it off.
static const wf::AttnEntry* persist_plan(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v,
                                         int mask_kind, int causal, bool has_lse, int64_t Lk,
                                         int rope, int* n_qtiles, int64_t* grid) {
  const int dt = kernel_dtype(q->dtype);
  if (dt == wf::DT_F32 || mask_kind != wf::MASK_NONE || Lk <= 0) return nullptr;
  const int B = (int)q->shape[0], Hq = (int)q->shape[1], Lq = (int)q->shape[2];
  const int Dqk = (int)q->shape[3], Hkv = (int)k->shape[1], Dv = (int)v->shape[3];
  const int G = Hq / Hkv;
  const int hpw = tuned_hpw((G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1, G);
  const int64_t max_sm = std::max(k->stride[2], v->stride[2]);
  const bool kv_ok = max_sm >= 0 && max_sm * 2 * 64 < ((int64_t)1 << 31);
  const bool q_ok = q->stride[2] >= 0 && q->stride[2] * 2 * 32 < ((int64_t)1 << 31);
  const bool persist = kv_ok && q_ok && (!causal || hpw == 4) && tune(T_PERSIST) != 0;
  if (!persist) return nullptr;
  // Without the lse the row sums are taken over the 16-bit weights (exactly the weights
  // that multiply V; their sum keeps the 16-bit rounding, which the lse would show).
  const int pmode = rope == 1   ? (has_lse ? wf::MODE_DENSE_PR : wf::MODE_DENSE_PR16)
                    : rope == 2 ? (has_lse ? wf::MODE_DENSE_PI : wf::MODE_DENSE_PI16)
                                : (has_lse ? wf::MODE_DENSE_P : wf::MODE_DENSE_P16);
  const wf::AttnEntry* pe = find_attn(dt, Dqk, Dqk, Dv, 8, hpw, wf::MASK_NONE, causal, pmode);
  const int ncu = cu_count();
  if (pe == nullptr || ncu <= 0) return nullptr;
  *n_qtiles = (Lq + pe->bmp - 1) / pe->bmp;
  const int64_t items = (int64_t)*n_qtiles * B * Hkv * (G / hpw);
  const int64_t P = std::min<int64_t>(ncu, items);
  if (P <= 0 || (items + P - 1) / P > wf::kPersistMaxItems) return nullptr;
  *grid = P;
  return pe;
}

// Persistent 64-query-wave kernel (attn_fwd_q.hpp): 16-bit calls without a mask or a rotary
// Q, head dims 128, whose K/V/Q copy offsets fit in 32 bits (64 rows of each span less than
// 2 GiB) and, when causal, whose work groups hold four query heads of one KV head. Returns the
// table entry and sets the query-tile count and the grid, or nullptr.
static const wf::AttnEntry* q64_plan(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v,
                                     int mask_kind, int causal, int64_t Lk, bool rope,
                                     int* n_qtiles, int64_t* grid) {
  const int dt = kernel_dtype(q->dtype);
  if (dt == wf::DT_F32 || mask_kind != wf::MASK_NONE || rope || Lk <= 0) return nullptr;
  // Opt-in: on the 4k causal GQA shape it measured 7% slower than the persistent 32-query
  // kernel (0.540 against 0.504 ms), and 5% slower non-causal (0.978 against 0.932 ms).
  if (tune(T_Q64) != 1) return nullptr;
  const int B = (int)q->shape[0], Hq = (int)q->shape[1], Lq = (int)q->shape[2];
  const int Dqk = (int)q->shape[3], Hkv = (int)k->shape[1], Dv = (int)v->shape[3];
  if (Dqk != 128 || Dv != 128) return nullptr;
  const int G = Hq / Hkv;
  const int hpw = tuned_hpw((G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1, G);
  if (causal && hpw != 4) return nullptr;
  const int64_t max_sm = std::max(k->stride[2], v->stride[2]);
  if (max_sm < 0 || max_sm * 2 * 64 >= ((int64_t)1 << 31)) return nullptr;
  if (q->stride[2] < 0 || q->stride[2] * 2 * 64 >= ((int64_t)1 << 31)) return nullptr;
  const wf::AttnEntry* e = find_attn(dt, 128, 128, 128, 4, hpw, wf::MASK_NONE, causal,
                                     wf::MODE_DENSE_Q, 64);
  const int ncu = cu_count();
  if (e == nullptr || ncu <= 0) return nullptr;
  *n_qtiles = (Lq + e->bmp - 1) / e->bmp;
  const int64_t items = (int64_t)*n_qtiles * B * Hkv * (G / hpw);
  const int64_t P = std::min<int64_t>(ncu, items);
  if (P <= 0 || (items + P - 1) / P > wf::kQMaxItems) return nullptr;
  *grid = P;
  return e;
}

// Dense attention over already validated operands (shared by SDPA and the cache attend when
// a single split suffices). mask_kind: wf::MASK_*. rope_q: turn Q by this rotary table on
// its way into the persistent kernel (the caller has checked with persist_plan that the call
// takes it).
int run_dense(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v, const wf_tensor* mask,
              int mask_kind, bool mask_vec, bool mask_lds, int causal, float scale, wf_tensor* out, float* lse,
              int64_t Lk, hipStream_t stream, const wf_rope* rope_q = nullptr) {
  const int B = (int)q->shape[0], Hq = (int)q->shape[1], Lq = (int)q->shape[2];
  const int Dqk = (int)q->shape[3], Hkv = (int)k->shape[1], Dv = (int)v->shape[3];
  const int G = Hq / Hkv;
  wf::FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q->data; a.q2 = q->data; a.k = k->data; a.k2 = k->data; a.v = v->data;
  a.o = out->data; a.lse = lse; a.mask = mask ? mask->data : nullptr;
  a.q_sb = st(q, 0); a.q_sh = st(q, 1); a.q_sm = q->stride[2];
  a.q2_sb = a.q_sb; a.q2_sh = a.q_sh; a.q2_sm = a.q_sm;
  a.k_sb = st(k, 0); a.k_sh = st(k, 1); a.k_sm = k->stride[2];
  a.k2_sb = a.k_sb; a.k2_sh = a.k_sh; a.k2_sm = a.k_sm;
  a.v_sb = st(v, 0); a.v_sh = st(v, 1); a.v_sm = v->stride[2];
  a.o_sb = st(out, 0); a.o_sh = st(out, 1); a.o_sm = out->stride[2];
  if (mask) { a.mk_sb = st(mask, 0); a.mk_sh = st(mask, 1); a.mk_sm = st(mask, 2); }
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.Lq = Lq; a.Lk = (int)Lk;
  a.causal_shift = 0;
  a.mask_vec = mask_vec ? 1 : 0;
  a.mask_lds = mask_lds ? 1 : 0;
  a.scale_log2 = scale * wf::kLog2e;
  a.inv_scale = 1.0f / scale;
  const int dt = kernel_dtype(q->dtype);
  if (dt == wf::DT_F32) {
    // One 32-query tile per (batch, head) over more than one 32-key tile: the key-split form
    // (its four waves share the key tiles instead of three of them idling).
    const bool ks = Lq <= 32 && Lk > 32;
    const wf::F32Entry* e = find_f32(Dqk, Dv, mask_kind, causal, ks);
    if (!e) return fail(WF_ERR_UNSUPPORTED, "no fp32 kernel for Dqk=%d Dv=%d", Dqk, Dv);
    a.n_qtiles = (Lq + e->bm - 1) / e->bm;
    const int64_t blocks = (int64_t)a.n_qtiles * B * Hq;
    if (blocks > 0x7fffffff) return fail(WF_ERR_SHAPE, "problem too large for one launch");
    return hip_status(launch(e->fn, dim3((unsigned)blocks), dim3(256), a, stream), "attention launch");
  }
  int hpw = 1;
  if (mask_kind == wf::MASK_NONE) hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  hpw = tuned_hpw(hpw, G);
  // Kernel shape: 64-query waves (one per SIMD) for non-causal calls without the log-sum-exp
  // (their row sums are taken over the 16-bit weights: exact for the normalised output, but
  // the sum, and so the lse, keeps the 16-bit rounding; the 32-query kernel sums in fp32);
  // 32-query waves otherwise. The 64-query kernel keeps its K/V copy offsets in 32 bits, so
  // 64 rows of K and of V must span less than 2 GiB. WF_TUNE_QPW=32|64 overrides.
  const int64_t max_sm = std::max(k->stride[2], v->stride[2]);
  const bool w64_ok = max_sm >= 0 && max_sm * 2 * 64 < ((int64_t)1 << 31);
  {
    int nqt = 0;
    int64_t P = 0;
    const wf::AttnEntry* qe = q64_plan(q, k, v, mask_kind, causal, Lk, rope_q != nullptr, &nqt, &P);
    if (qe != nullptr) {
      a.n_qtiles = nqt;
      return hip_status(launch(qe->fn, dim3((unsigned)P), dim3(256), a, stream), "attention launch");
    }
    const int rk = rope_q == nullptr ? 0 : rope_q->style == 0 ? 1 : 2;
    const wf::AttnEntry* pe = persist_plan(q, k, v, mask_kind, causal, lse != nullptr, Lk, rk,
                                           &nqt, &P);
    if (pe != nullptr) {
      a.n_qtiles = nqt;
      if (rope_q != nullptr) {
        const int64_t row0 = rope_q->q_pos0 * (rope_q->rot_dim / 2);
        a.rq_cos = rope_q->cos + row0;
        a.rq_sin = rope_q->sin + row0;
        a.rq_rot = rope_q->rot_dim;
      }
      return hip_status(launch(pe->fn, dim3((unsigned)P), dim3(512), a, stream), "attention launch");
    }
    if (rope_q != nullptr) return fail(WF_ERR_UNSUPPORTED, "rotary Q needs the persistent kernel");
  }
  // Masked calls take the 32-query kernel, which copies bool / 16-bit mask tiles into LDS.
  int qpw = (lse == nullptr && !causal && w64_ok && !(mask_lds && mask_kind != wf::MASK_NONE)) ? 64 : 32;
  if (tune(T_QPW) == 32) qpw = 32;
  else if (tune(T_QPW) == 64 && w64_ok) qpw = 64;
  const wf::AttnEntry* e = nullptr;
  // Bool / 16-bit masked calls without the lse: the prescaled form (no per-score FMA); fp32
  // masks keep the exact form (the prescaled one spills registers with them).
  if (mask_kind != wf::MASK_NONE && lse == nullptr && !causal && tune(T_MASK_PRE) != 0)
    e = find_attn(dt, Dqk, Dqk, Dv, 8, hpw, mask_kind, 0, wf::MODE_DENSE_PM, 32);
  if (!e && qpw == 64) e = find_attn(dt, Dqk, Dqk, Dv, 4, hpw, mask_kind, causal, wf::MODE_DENSE, 64);
  if (!e) {
    int nw = 8;
    if (tune(T_NW) == 4 && mask_kind == wf::MASK_NONE) nw = 4;
    e = find_attn(dt, Dqk, Dqk, Dv, nw, hpw, mask_kind, causal, wf::MODE_DENSE, 32);
  }
  if (!e) return fail(WF_ERR_UNSUPPORTED, "no 16-bit kernel for Dqk=%d Dv=%d", Dqk, Dv);
  a.n_qtiles = (Lq + e->bmp - 1) / e->bmp;
  const int64_t blocks = (int64_t)a.n_qtiles * B * Hkv * (G / hpw);
  if (blocks > 0x7fffffff) return fail(WF_ERR_SHAPE, "problem too large for one launch");
  return hip_status(launch(e->fn, dim3((unsigned)blocks), dim3(e->nw * 64), a, stream),
                    "attention launch");
}

int check_cache_state(const wf_block_kv_state* s) {
  if (s == nullptr) return fail(WF_ERR_NULL, "state is NULL");
  if (s->chunk <= 0 || s->window <= 0 || s->sink < 0 || s->cache_len <= 0)
    return fail(WF_ERR_CACHE_CONFIG, "cache sizes must be positive (sink may be 0)");
  if (s->sink + s->window != s->cache_len)
    return fail(WF_ERR_CACHE_CONFIG, "sink + window (%lld) must equal the cache length (%lld)",
                (long long)(s->sink + s->window), (long long)s->cache_len);
  if (s->cache_len % s->chunk != 0)
    return fail(WF_ERR_CACHE_CONFIG, "sink + window must be divisible by chunk_size");
  if (s->window < s->chunk) return fail(WF_ERR_CACHE_CONFIG, "window must hold at least one chunk");
  if (s->last_chunk < -1) return fail(WF_ERR_CACHE_CONFIG, "corrupt state (last_chunk < -1)");
  return WF_OK;
}

void visible_range(const wf_block_kv_state* s, int64_t* T, int64_t* head, int64_t* start,
                   int64_t* n) {
  *T = (s->last_chunk + 1) * s->chunk;
  *head = *T < s->sink ? *T : s->sink;
  *start = (*T - s->window) > s->sink ? (*T - s->window) : s->sink;
  *n = *head + (*T > *start ? *T - *start : 0);
}

constexpr int kMaxSplits = 16;

// Split-KV plan for decode-shaped calls (few queries, long KV): the query heads of a KV group
// share each K/V tile (hpw heads per work group), and the key tiles are cut into splits so
// that about kDecodeGroups work groups stream K/V at once. It depends on shapes only, so the
// workspace size does not depend on the device.
constexpr int kMaxDecodeSplits = 256;
constexpr int64_t kDecodeMinGroups = 256;
constexpr int64_t kDecodeGroups = 512;
struct DecodePlan {
  const wf::AttnEntry* e = nullptr;
  int n_qt = 0, n_splits = 1, tps = 1;
  bool pack = false;   // (query head, position) rows packed: one item per KV head and row block
  int64_t base = 0;    // work items before the split
};
DecodePlan decode_plan(int dt, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                       int64_t D, int64_t Dv, bool causal) {
  DecodePlan p;
  if (Hkv <= 0 || Hq % Hkv != 0) return p;
  const int64_t G = Hq / Hkv;
  // More than 4 query heads per KV head: pack the G*Lq (head, position) rows of a KV head into
  // the tiles' query rows, so each K/V tile is read once per KV head (not once per 4 heads).
  p.pack = G > 4 && G * Lq <= 0x7fffffff;
  p.pack = p.pack && tune(T_DECODE_PACK) != 0;
  const int hpw = p.pack ? 1 : G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1;
  p.e = find_attn(dt, (int)D, (int)D, (int)Dv, 4, hpw, wf::MASK_NONE, causal ? 1 : 0,
                  p.pack ? wf::MODE_SPLITP : wf::MODE_SPLIT);
  if (p.e == nullptr) return p;
  const int64_t rows = p.pack ? G * Lq : Lq;
  p.n_qt = (int)((rows + p.e->bmp - 1) / p.e->bmp);
  p.base = (int64_t)p.n_qt * B * Hkv * (p.pack ? 1 : G / hpw);
  const int64_t base = std::max<int64_t>(1, p.base);
  const int64_t n_kt = (Lk + p.e->bn - 1) / p.e->bn;
  // About kDecodeGroups groups, but splits of at least min_tiles tiles unless that leaves
  // fewer than kDecodeMinGroups (measured: multi-query decode, 8 KV groups over 16k keys,
  // 0.056 ms with 64 splits of 4 tiles, 0.038 ms with 16 of 16; the per-split start-up and
  // the merge outweigh the extra parallelism on short per-group K/V).
  int64_t groups = kDecodeGroups, min_tiles = 16;
  if (tune(T_DECODE_GROUPS) > 0) groups = tune(T_DECODE_GROUPS);
  if (tune(T_DECODE_MIN_TILES) > 0) min_tiles = tune(T_DECODE_MIN_TILES);
  int64_t n = (groups + base - 1) / base;
  n = std::min<int64_t>(n, std::max<int64_t>(1, n_kt / min_tiles));
  n = std::max<int64_t>(n, std::min<int64_t>((kDecodeMinGroups + base - 1) / base, n_kt));
  n = std::min<int64_t>(n, kMaxDecodeSplits);
  p.tps = (int)std::max<int64_t>(1, (n_kt + n - 1) / n);
  p.n_splits = (int)std::max<int64_t>(1, (n_kt + p.tps - 1) / p.tps);
  return p;
}

}  // namespace

extern "C" {

const char* wf_status_string(int status) {
  switch (status) {
    case WF_OK: return "WF_OK";
    case WF_ERR_NULL: return "WF_ERR_NULL";
    case WF_ERR_SHAPE: return "WF_ERR_SHAPE";
    case WF_ERR_DTYPE: return "WF_ERR_DTYPE";
    case WF_ERR_LAYOUT: return "WF_ERR_LAYOUT";
    case WF_ERR_UNSUPPORTED: return "WF_ERR_UNSUPPORTED";
    case WF_ERR_CHUNK_ORDER: return "WF_ERR_CHUNK_ORDER";
    case WF_ERR_CACHE_CONFIG: return "WF_ERR_CACHE_CONFIG";
    case WF_ERR_WORKSPACE: return "WF_ERR_WORKSPACE";
    case WF_ERR_HIP: return "WF_ERR_HIP";
    default: return "WF_ERR_UNKNOWN";
  }
}

const char* wf_last_error(void) { return g_last_error.c_str(); }

int wf_tune_set(const char* name, int value) {
  const int k = tune_key(name);
  if (k < 0) return fail(WF_ERR_UNSUPPORTED, "unknown tuning key '%s'", name ? name : "(null)");
  tune_table()[k].store(value, std::memory_order_relaxed);
  return ok();
}

int wf_tune_get(const char* name, int* value) {
  const int k = tune_key(name);
  if (k < 0) return fail(WF_ERR_UNSUPPORTED, "unknown tuning key '%s'", name ? name : "(null)");
  if (value == nullptr) return fail(WF_ERR_NULL, "value is NULL");
  *value = tune_table()[k].load(std::memory_order_relaxed);
  return ok();
}

}  // extern "C"

namespace {
// The checks of wf_sdpa_fwd (nothing enqueued); on success *plan holds what run_dense needs.
struct SdpaPlan {
  int mask_kind = wf::MASK_NONE;
  bool mask_vec = false, mask_lds = false, empty = false;
  float scale = 0.f;
};
int sdpa_validate(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v,
                  const wf_tensor* mask, int is_causal, float dropout_p, float scale,
                  const wf_tensor* out, const float* lse, SdpaPlan* plan) {
  int rc;
  if ((rc = check_data(q, "q", 4)) || (rc = check_data(k, "k", 4)) ||
      (rc = check_data(v, "v", 4)) || (rc = check_data(out, "out", 4)))
    return rc;
  if (k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype)
    return fail(WF_ERR_DTYPE, "q, k, v and out must share one dtype");
  const int64_t B = q->shape[0], Hq = q->shape[1], Lq = q->shape[2], Dqk = q->shape[3];
  const int64_t Hkv = k->shape[1], Lk = k->shape[2], Dv = v->shape[3];
  if (k->shape[0] != B || v->shape[0] != B || k->shape[3] != Dqk || v->shape[1] != Hkv ||
      v->shape[2] != Lk)
    return fail(WF_ERR_SHAPE, "k must be [B,Hkv,Lk,Dqk] and v [B,Hkv,Lk,Dv] for q [B,Hq,Lq,Dqk]");
  if (out->shape[0] != B || out->shape[1] != Hq || out->shape[2] != Lq || out->shape[3] != Dv)
    return fail(WF_ERR_SHAPE, "out must be [B,Hq,Lq,Dv]");
  if (Hkv <= 0 || Hq % Hkv != 0)
    return fail(WF_ERR_SHAPE, "Hq (%lld) must be a positive multiple of Hkv (%lld)",
                (long long)Hq, (long long)Hkv);
  if (Lq > 0x7fffffff || Lk > 0x7fffffff || B > 0x7fffffff || Hq > 0x7fffffff)
    return fail(WF_ERR_SHAPE, "dimension exceeds 2^31");
  if (dropout_p != 0.f)
    return fail(WF_ERR_UNSUPPORTED, "dropout_p must be 0 (inference forward only)");
  if (mask && is_causal)
    return fail(WF_ERR_UNSUPPORTED, "a mask together with is_causal is not accepted");
  if ((rc = resolve_scale(scale, Dqk, &plan->scale))) return rc;
  const bool f32 = q->dtype == WF_F32;
  if (f32 ? !((Dqk == 64 || Dqk == 128) && (Dv == 64 || Dv == 96 || Dv == 128))
          : !((Dqk == 64 && (Dv == 64 || Dv == 96)) || (Dqk == 128 && (Dv == 128 || Dv == 64))))
    return fail(WF_ERR_UNSUPPORTED, "head dims Dqk=%lld Dv=%lld are not built for this dtype",
                (long long)Dqk, (long long)Dv);
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(WF_ERR_LAYOUT, "lse must be 4-byte aligned");
  int& mask_kind = plan->mask_kind;
  bool& mask_vec = plan->mask_vec;
  bool& mask_lds = plan->mask_lds;
  if (mask) {
    if (mask->ndim != 4) return fail(WF_ERR_SHAPE, "mask must be 4-d [B|1, Hq|1, Lq, Lk]");
    const int64_t want[4] = {B, Hq, Lq, Lk};
    for (int i = 0; i < 4; ++i)
      if (mask->shape[i] != want[i] && !(mask->shape[i] == 1 && i < 2))
        return fail(WF_ERR_SHAPE, "mask dim %d is %lld, expected %lld%s", i,
                    (long long)mask->shape[i], (long long)want[i], i < 2 ? " or 1" : "");
    if (mask->dtype == WF_BOOL) mask_kind = wf::MASK_BOOL;
    else if (mask->dtype == WF_F32) mask_kind = wf::MASK_F32;
    else if (mask->dtype == q->dtype && !f32) mask_kind = wf::MASK_HALF;
    else return fail(WF_ERR_DTYPE, "mask must be bool, f32 or the dtype of q");
    if (numel(mask) > 0) {
      if (mask->data == nullptr) return fail(WF_ERR_NULL, "mask->data is NULL");
      if (Lk > 1 && mask->stride[3] != 1) return fail(WF_ERR_LAYOUT, "mask key stride must be 1");
      const int ms = esize(mask->dtype);
      if (reinterpret_cast<uintptr_t>(mask->data) % ms != 0)
        return fail(WF_ERR_LAYOUT, "mask pointer is not aligned to its element size");
      mask_vec = reinterpret_cast<uintptr_t>(mask->data) % (4 * ms) == 0;
      for (int i = 0; i < 3; ++i)
        if (mask->shape[i] > 1 && mask->stride[i] % 4 != 0) mask_vec = false;
      // Bool / 16-bit mask tiles can be copied into LDS when every row starts 16-byte aligned,
      // 256 rows span less than 2 GiB (32-bit per-lane copy offsets) and a row's keys end on a
      // dword boundary: the copy's bounds check zeroes whole dwords, so a last row ending
      // inside a dword would lose its last valid keys (those masks read global memory).
      mask_lds = mask_kind != wf::MASK_F32 && reinterpret_cast<uintptr_t>(mask->data) % 16 == 0 &&
                 mask->stride[2] >= 0 && mask->stride[2] * ms * 256 < ((int64_t)1 << 31) &&
                 (Lk * ms) % 4 == 0;
      for (int i = 0; i < 3; ++i)
        if (mask->shape[i] > 1 && (mask->stride[i] * ms) % 16 != 0) mask_lds = false;
    }
  }
  plan->empty = B * Hq * Lq == 0 || Dv == 0;
  return WF_OK;
}
}  // namespace

extern "C" {

int wf_sdpa_fwd(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v,
                const wf_tensor* mask, int is_causal, float dropout_p, float scale,
                wf_tensor* out, float* lse, void* stream) {
  SdpaPlan p;
  int rc = sdpa_validate(q, k, v, mask, is_causal, dropout_p, scale, out, lse, &p);
  if (rc) return rc;
  if (p.empty) return ok();
  return run_dense(q, k, v, mask, p.mask_kind, p.mask_vec, p.mask_lds, is_causal ? 1 : 0, p.scale,
                   out, lse, k->shape[2], (hipStream_t)stream);
}

static int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

size_t wf_sdpa_rope_workspace_size(const wf_tensor* q, const wf_tensor* k) {
  if (q == nullptr || k == nullptr || q->ndim != 4 || k->ndim != 4) return 0;
  for (int i = 0; i < 4; ++i)
    if (q->shape[i] < 0 || k->shape[i] < 0) return 0;
  const int64_t es = esize(q->dtype);
  return (size_t)(align256(numel(q) * es) + align256(numel(k) * es) + 256);
}

int wf_sdpa_rope_fwd(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v,
                     const wf_tensor* mask, int is_causal, float scale, const wf_rope* rope,
                     wf_tensor* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream) {
  SdpaPlan p;
  int rc = sdpa_validate(q, k, v, mask, is_causal, 0.f, scale, out, lse, &p);
  if (rc) return rc;
  if (rope == nullptr) return fail(WF_ERR_NULL, "rope is NULL");
  const int64_t Lq = q->shape[2], Lk = k->shape[2], D = q->shape[3];
  const int rot = rope->rot_dim;
  if (rot < 0 || rot > D || rot % 16 != 0)
    return fail(WF_ERR_UNSUPPORTED, "rot_dim must be a multiple of 16 in [0, %lld]", (long long)D);
  if (rope->style != 0 && rope->style != 1)
    return fail(WF_ERR_UNSUPPORTED, "rope style must be 0 (rotate-half) or 1 (interleaved)");
  if (rot > 0) {
    if (rope->cos == nullptr || rope->sin == nullptr) return fail(WF_ERR_NULL, "rope tables are NULL");
    if (reinterpret_cast<uintptr_t>(rope->cos) % 16 != 0 || reinterpret_cast<uintptr_t>(rope->sin) % 16 != 0)
      return fail(WF_ERR_LAYOUT, "rope tables must be 16-byte aligned");
    if (rope->q_pos0 < 0 || rope->k_pos0 < 0 || rope->q_pos0 + Lq > rope->max_pos ||
        rope->k_pos0 + Lk > rope->max_pos)
      return fail(WF_ERR_SHAPE, "positions [%lld, %lld) and [%lld, %lld) must lie in the %lld table rows",
                  (long long)rope->q_pos0, (long long)(rope->q_pos0 + Lq), (long long)rope->k_pos0,
                  (long long)(rope->k_pos0 + Lk), (long long)rope->max_pos);
  }
  const size_t need = wf_sdpa_rope_workspace_size(q, k);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(WF_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(WF_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (p.empty) return ok();
  if (rot == 0)
    return run_dense(q, k, v, mask, p.mask_kind, p.mask_vec, p.mask_lds, is_causal ? 1 : 0, p.scale,
                     out, lse, Lk, (hipStream_t)stream);
  // rotated copies, contiguous [B, H, L, D], in the workspace
  const int64_t es = esize(q->dtype);
  wf_tensor qr = *q, kr = *k;
  qr.data = workspace;
  kr.data = (char*)workspace + align256(numel(q) * es);
  for (wf_tensor* t : {&qr, &kr}) {
    t->stride[3] = 1;
    t->stride[2] = t->shape[3];
    t->stride[1] = t->shape[2] * t->stride[2];
    t->stride[0] = t->shape[1] * t->stride[1];
  }
  auto desc = [&](const wf_tensor* t, const wf_tensor* o, int64_t pos0) {
    wf::RopeDesc d;
    d.x = t->data; d.sb = st(t, 0); d.sh = st(t, 1); d.sm = t->stride[2];
    d.y = o->data;
    d.B = (int)t->shape[0]; d.H = (int)t->shape[1]; d.L = (int)t->shape[2];
    d.pos0 = pos0;
    return d;
  };
  hipStream_t strm = (hipStream_t)stream;
  // When the call takes the persistent kernel (rotate-half over the whole head, or
  // interleaved), Q is turned in its registers as it is read and only K goes through the
  // rotation pass.
  int nqt = 0;
  int64_t P = 0;
  const bool fuse_q = (rope->style == 1 || rot == D) &&
                      persist_plan(q, k, v, p.mask_kind, is_causal ? 1 : 0, lse != nullptr, Lk,
                                   rope->style == 0 ? 1 : 2, &nqt, &P) != nullptr;
  wf::RopeDesc dq = desc(q, &qr, rope->q_pos0);
  if (fuse_q) dq.B = 0;   // no Q rows in the pass
  hipError_t he = wf::launch_rope(kernel_dtype(q->dtype), dq, desc(k, &kr, rope->k_pos0), (int)D,
                                  rot, rope->style, rope->cos, rope->sin, strm);
  if (he != hipSuccess) return hip_status(he, "rope launch");
  if (fuse_q)
    return run_dense(q, &kr, v, mask, p.mask_kind, p.mask_vec, p.mask_lds, is_causal ? 1 : 0,
                     p.scale, out, lse, Lk, strm, rope);
  return run_dense(&qr, &kr, v, mask, p.mask_kind, p.mask_vec, p.mask_lds, is_causal ? 1 : 0,
                   p.scale, out, lse, Lk, strm);
}

size_t wf_varlen_mla_prefill_workspace_size(int batch, int64_t total_q_tokens, int head_num) {
  (void)head_num;
  if (batch < 0 || total_q_tokens < 0) return 0;
  // query positions per work item of the smallest-tile MLA kernel (four query heads of a KV
  // head per work group: 64 rows); the call picks the kernel from kv_head_num, unknown here
  const int64_t bmp = 64;
  const int64_t max_items = total_q_tokens / bmp + batch;
  return (size_t)wf::VarlenWs::bytes(batch, max_items);
}

static int as3d(const wf_tensor* t, const char* name, int64_t heads, wf_tensor* o) {
  // Accepts [n, H, d] or the flat [n, H*d] form of the same bytes.
  if (t == nullptr) return fail(WF_ERR_NULL, "%s is NULL", name);
  *o = *t;
  if (t->ndim == 2) {
    if (heads <= 0 || t->shape[1] % heads != 0)
      return fail(WF_ERR_SHAPE, "%s: flat width %lld is not a multiple of the head count",
                  name, (long long)t->shape[1]);
    o->ndim = 3;
    o->shape[2] = t->shape[1] / heads;
    o->shape[1] = heads;
    o->stride[2] = t->stride[1];
    o->stride[1] = o->shape[2] * t->stride[1];
  }
  return check_data(o, name, 3);
}

// K, kRope and V are packed ([nTk, Hkv, d] or flat) or padded per sequence
// ([batch, max_seq, Hkv, d]: sequence i's keys are rows [0, kv_seqlen[i]) of entry i). The
// padded form comes back as a [max_seq, Hkv, d] view plus its batch stride (0 when packed).
static int kv_view(const wf_tensor* t, const char* name, int64_t heads, int batch, wf_tensor* o,
                   int64_t* sb) {
  *sb = 0;
  if (t == nullptr || t->ndim != 4) return as3d(t, name, heads, o);
  int rc = check_data(t, name, 4);
  if (rc) return rc;
  if (t->shape[0] != batch)
    return fail(WF_ERR_SHAPE, "%s: the padded form is [batch=%d, max_seq, H, d]", name, batch);
  *o = *t;
  o->ndim = 3;
  for (int i = 0; i < 3; ++i) {
    o->shape[i] = t->shape[i + 1];
    o->stride[i] = t->stride[i + 1];
  }
  *sb = t->stride[0];
  return check_data(o, name, 3);
}

int wf_varlen_mla_prefill(const wf_tensor* q_, const wf_tensor* q_rope_, const wf_tensor* k_,
                          const wf_tensor* k_rope_, const wf_tensor* v_,
                          const int32_t* q_seqlen, const int32_t* kv_seqlen, int batch,
                          int head_num, int kv_head_num, float qk_scale, int mask_type,
                          wf_tensor* out_, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int rc;
  wf_tensor q, qr, k, kr, v, out;
  int64_t k_sb, kr_sb, v_sb;
  if ((rc = as3d(q_, "q", head_num, &q)) || (rc = as3d(q_rope_, "q_rope", head_num, &qr)) ||
      (rc = kv_view(k_, "k", kv_head_num, batch, &k, &k_sb)) ||
      (rc = kv_view(k_rope_, "k_rope", kv_head_num, batch, &kr, &kr_sb)) ||
      (rc = kv_view(v_, "v", kv_head_num, batch, &v, &v_sb)) || (rc = as3d(out_, "out", head_num, &out)))
    return rc;
  const bool padded = k_->ndim == 4;
  if ((k_rope_->ndim == 4) != padded || (v_->ndim == 4) != padded)
    return fail(WF_ERR_LAYOUT, "k, k_rope and v must all be packed or all padded");
  if (q.dtype == WF_F32) return fail(WF_ERR_DTYPE, "MLA prefill takes f16 or bf16");
  if (qr.dtype != q.dtype || k.dtype != q.dtype || kr.dtype != q.dtype || v.dtype != q.dtype ||
      out.dtype != q.dtype)
    return fail(WF_ERR_DTYPE, "all MLA tensors must share one dtype");
  const int64_t nTq = q.shape[0], nTk = k.shape[0], Dv = q.shape[2];
  if (head_num <= 0 || kv_head_num <= 0 || head_num % kv_head_num != 0)
    return fail(WF_ERR_SHAPE, "headNum must be a positive multiple of kvHeadNum");
  if (q.shape[1] != head_num || qr.shape[1] != head_num || out.shape[1] != head_num ||
      k.shape[1] != kv_head_num || kr.shape[1] != kv_head_num || v.shape[1] != kv_head_num)
    return fail(WF_ERR_SHAPE, "head counts disagree with headNum / kvHeadNum");
  if (qr.shape[0] != nTq || out.shape[0] != nTq || kr.shape[0] != nTk || v.shape[0] != nTk)
    return fail(WF_ERR_SHAPE, "token counts disagree between q/q_rope/out or k/k_rope/v");
  if (qr.shape[2] != 64 || kr.shape[2] != 64)
    return fail(WF_ERR_SHAPE, "the rotary part must be 64 wide");
  if (k.shape[2] != Dv || v.shape[2] != Dv || out.shape[2] != Dv)
    return fail(WF_ERR_SHAPE, "q, k, v and out must share the value width");
  if (Dv != 128 && Dv != 64)
    return fail(WF_ERR_UNSUPPORTED, "value width %lld is not built (128, 64)", (long long)Dv);
  if (mask_type != 0 && mask_type != 1)
    return fail(WF_ERR_UNSUPPORTED, "mask_type must be 0 (none) or 1 (causal)");
  if (batch < 0) return fail(WF_ERR_SHAPE, "batch must be >= 0");
  if (nTq > 0x7fffffff || nTk > 0x7fffffff || (padded && (int64_t)batch * nTk > 0x7fffffff))
    return fail(WF_ERR_SHAPE, "token count exceeds 2^31");
  float sc;
  if ((rc = resolve_scale(qk_scale, Dv + 64, &sc))) return rc;
  if (batch > 0 && (q_seqlen == nullptr || kv_seqlen == nullptr))
    return fail(WF_ERR_NULL, "qSeqLen / kvSeqLen are NULL");
  const size_t need = wf_varlen_mla_prefill_workspace_size(batch, nTq, head_num);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(WF_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(WF_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  // The query heads of a KV head share each K/V tile (as in the dense kernels).
  const int G = head_num / kv_head_num;
  const int hpw = tuned_hpw(G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1, G);
  const wf::AttnEntry* e = find_attn(kernel_dtype(q.dtype), (int)Dv + 64, (int)Dv, (int)Dv, 8, hpw,
                                     wf::MASK_NONE, mask_type, wf::MODE_VARLEN);
  if (!e) return fail(WF_ERR_UNSUPPORTED, "MLA kernel not built for this dtype");
  if (batch == 0 || nTq == 0) return ok();
  if (e->bmp < 64) return fail(WF_ERR_UNSUPPORTED, "internal: MLA tile height below the workspace's");
  const int max_items = (int)(nTq / e->bmp + batch);
  int* ws = (int*)workspace;
  hipStream_t s = (hipStream_t)stream;
  hipError_t he = wf::launch_varlen_schedule(q_seqlen, kv_seqlen, batch, nTq, nTk,
                                             padded ? (int)nTk : -1, e->bmp, e->bn, mask_type,
                                             max_items, ws, s);
  if (he != hipSuccess) return hip_status(he, "schedule launch");
  wf::FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q.data; a.q2 = qr.data; a.k = k.data; a.k2 = kr.data; a.v = v.data; a.o = out.data;
  a.q_sm = q.stride[0]; a.q_sh = q.stride[1];
  a.q2_sm = qr.stride[0]; a.q2_sh = qr.stride[1];
  a.k_sm = k.stride[0]; a.k_sh = k.stride[1]; a.k_sb = k_sb;
  a.k2_sm = kr.stride[0]; a.k2_sh = kr.stride[1]; a.k2_sb = kr_sb;
  a.v_sm = v.stride[0]; a.v_sh = v.stride[1]; a.v_sb = v_sb;
  a.kv_padded = padded ? 1 : 0;
  a.o_sm = out.stride[0]; a.o_sh = out.stride[1];
  a.B = batch; a.Hq = head_num; a.Hkv = kv_head_num; a.G = head_num / kv_head_num;
  a.scale_log2 = sc * wf::kLog2e;
  a.inv_scale = 1.0f / sc;
  a.cu_q = (const int*)((char*)workspace + wf::VarlenWs::cu_q_off());
  a.cu_k = (const int*)((char*)workspace + wf::VarlenWs::cu_k_off(batch));
  a.items = (const int2*)((char*)workspace + wf::VarlenWs::items_off(batch));
  a.counter = ws;
  a.n_items = ws + 1;
  // The schedule counts (sequence, query tile) items on the device; the kernel expands each
  // over the head groups and takes work from the counter, so the persistent grid only
  // needs an upper bound on the work.
  const int64_t total_work = (int64_t)max_items * (head_num / e->hpw);
  const int cus = cu_count();
  if (cus <= 0) return fail(WF_ERR_HIP, "cannot query the device's compute units");
  int grid = (int)(total_work < cus ? total_work : cus);
  // Split the work over the 8 XCDs by KV head when the heads and the grid divide evenly (the
  // head groups of one KV head never straddle XCDs); WF_TUNE_MLA_XCD=0 turns it off.
  a.xcd_parts = kv_head_num % 8 == 0 && (head_num / kv_head_num) % e->hpw == 0 && cus % 8 == 0;
  a.xcd_parts = a.xcd_parts && tune(T_MLA_XCD) != 0;
  if (a.xcd_parts) grid = (grid + 7) / 8 * 8;
  return hip_status(launch(e->fn, dim3(grid), dim3(e->nw * 64), a, s), "MLA launch");
}

}  // extern "C"

// ---- scratch of wf_varlen_mla_prefill_noalloc ------------------------------------------
// A fixed device array holds the prefill's workspace (schedule header, prefix sums, item list)
// for callers that cannot allocate. Each device that runs the library has its own copy at its
// own address, looked up once per device with that device current; host code uses only that
// address (the array's name in host code is not a device address). Every call on a device
// shares the array: the schedule kernel rewrites all of it that the attention kernel reads
// (the counters, the item count and the error word included), so nothing needs clearing
// between calls, and calls that overlap on one device race.
static constexpr size_t kMlaScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) unsigned char scratch[kMlaScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(WF_ERR_UNSUPPORTED, "device %d: the static scratch covers devices 0..%d", dev,
                kMaxScratchDevices - 1);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
      if (p == nullptr) return fail(WF_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return WF_OK;
}
}  // namespace

extern "C" {

int wf_varlen_mla_prefill_noalloc(const wf_tensor* q, const wf_tensor* q_rope, const wf_tensor* k,
                                  const wf_tensor* k_rope, const wf_tensor* v,
                                  const int32_t* q_seqlen, const int32_t* kv_seqlen, int batch,
                                  int head_num, int kv_head_num, float qk_scale, int mask_type,
                                  wf_tensor* out, void* stream) {
  if (q == nullptr) return fail(WF_ERR_NULL, "q is NULL");
  // (a malformed q is rejected by the checks of wf_varlen_mla_prefill below)
  const bool q_shaped = (q->ndim == 2 || q->ndim == 3) && q->shape[0] >= 0;
  const size_t need = q_shaped ? wf_varlen_mla_prefill_workspace_size(batch, q->shape[0], head_num) : 0;
  if (need > kMlaScratchBytes)
    return fail(WF_ERR_WORKSPACE,
                "the call needs %zu bytes of scratch and the static scratch holds %zu (batch %d, "
                "%lld query tokens); use wf_varlen_mla_prefill with a workspace",
                need, kMlaScratchBytes, batch, (long long)q->shape[0]);
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc) return rc;
  return wf_varlen_mla_prefill(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, batch, head_num,
                               kv_head_num, qk_scale, mask_type, out, ws, kMlaScratchBytes, stream);
}

int wf_block_kv_init(wf_block_kv_state* s, int64_t cache_len, int64_t sink, int64_t window,
                     int64_t chunk) {
  if (s == nullptr) return fail(WF_ERR_NULL, "state is NULL");
  wf_block_kv_state t;
  t.cache_len = cache_len; t.sink = sink; t.window = window; t.chunk = chunk; t.last_chunk = -1;
  int rc = check_cache_state(&t);
  if (rc) return rc;
  *s = t;
  return ok();
}

}  // extern "C"

// Checks of wf_block_kv_cache_update (also taken by the fused update + attend); *u16 is
// cleared when rows or strides are not 16-byte multiples.
static int check_update(const wf_block_kv_state* s, int64_t chunk_idx, const wf_tensor* k_new,
                        const wf_tensor* v_new, const wf_tensor* k_cache, const wf_tensor* v_cache,
                        bool* u16_out) {
  int rc;
  if ((rc = check_cache_state(s))) return rc;
  if (chunk_idx != s->last_chunk && chunk_idx != s->last_chunk + 1)
    return fail(WF_ERR_CHUNK_ORDER, "chunk %lld after chunk %lld: only a repeat or the next index",
                (long long)chunk_idx, (long long)s->last_chunk);
  if (chunk_idx < 0) return fail(WF_ERR_CHUNK_ORDER, "the first chunk index is 0");
  bool u16 = true;
  if ((rc = check_cache_data(k_new, "k_new", &u16)) || (rc = check_cache_data(v_new, "v_new", &u16)) ||
      (rc = check_cache_data(k_cache, "k_cache", &u16)) ||
      (rc = check_cache_data(v_cache, "v_cache", &u16)))
    return rc;
  if (v_new->dtype != k_new->dtype || k_cache->dtype != k_new->dtype || v_cache->dtype != k_new->dtype)
    return fail(WF_ERR_DTYPE, "cache and update tensors must share one dtype");
  const int64_t B = k_cache->shape[0], H = k_cache->shape[1], Dk = k_cache->shape[3];
  const int64_t Dv = v_cache->shape[3];
  if (k_cache->shape[2] != s->cache_len || v_cache->shape[2] != s->cache_len ||
      v_cache->shape[0] != B || v_cache->shape[1] != H)
    return fail(WF_ERR_SHAPE, "caches must be [B,H,cache_len,D] with cache_len = %lld",
                (long long)s->cache_len);
  if (k_new->shape[0] != B || k_new->shape[1] != H || k_new->shape[2] != s->chunk ||
      k_new->shape[3] != Dk || v_new->shape[0] != B || v_new->shape[1] != H ||
      v_new->shape[2] != s->chunk || v_new->shape[3] != Dv)
    return fail(WF_ERR_SHAPE, "updates must be [B,H,chunk,D] with chunk = %lld", (long long)s->chunk);
  *u16_out = u16;
  return WF_OK;
}

extern "C" {

int wf_block_kv_cache_update(wf_block_kv_state* s, int64_t chunk_idx, const wf_tensor* k_new,
                             const wf_tensor* v_new, wf_tensor* k_cache, wf_tensor* v_cache,
                             void* stream) {
  int rc;
  bool u16 = true;
  if ((rc = check_update(s, chunk_idx, k_new, v_new, k_cache, v_cache, &u16))) return rc;
  const int64_t B = k_cache->shape[0], H = k_cache->shape[1], Dk = k_cache->shape[3];
  const int64_t Dv = v_cache->shape[3];
  if (B * H > 0 && (Dk > 0 || Dv > 0)) {
    const int64_t kn[3] = {k_new->stride[0], k_new->stride[1], k_new->stride[2]};
    const int64_t vn[3] = {v_new->stride[0], v_new->stride[1], v_new->stride[2]};
    const int64_t kc[3] = {k_cache->stride[0], k_cache->stride[1], k_cache->stride[2]};
    const int64_t vc[3] = {v_cache->stride[0], v_cache->stride[1], v_cache->stride[2]};
    hipError_t he = wf::launch_kv_update(u16 ? 16 : esize(k_new->dtype), esize(k_new->dtype), k_new->data, kn, v_new->data, vn,
                                         k_cache->data, kc, v_cache->data, vc, (int)B, (int)H,
                                         (int)s->chunk, (int)Dk, (int)Dv, chunk_idx * s->chunk,
                                         s->sink, s->window, (hipStream_t)stream);
    if (he != hipSuccess) return hip_status(he, "cache update launch");
  }
  s->last_chunk = chunk_idx;
  return ok();
}

int wf_block_kv_visible(const wf_block_kv_state* s, int64_t* n_visible, int64_t* phys_index) {
  int rc;
  if ((rc = check_cache_state(s))) return rc;
  if (n_visible == nullptr) return fail(WF_ERR_NULL, "n_visible is NULL");
  int64_t T, head, start, n;
  visible_range(s, &T, &head, &start, &n);
  *n_visible = n;
  if (phys_index) {
    for (int64_t p = 0; p < n; ++p) {
      const int64_t tok = p < head ? p : start + (p - head);
      phys_index[p] = tok < s->sink ? tok : s->sink + (tok - s->sink) % s->window;
    }
  }
  return ok();
}

int wf_block_kv_gather(const wf_block_kv_state* s, const wf_tensor* cache, wf_tensor* out,
                       void* stream) {
  int rc;
  if ((rc = check_cache_state(s))) return rc;
  bool u16 = true;
  if ((rc = check_cache_data(cache, "cache", &u16)) || (rc = check_cache_data(out, "logical_out", &u16)))
    return rc;
  if (out->dtype != cache->dtype) return fail(WF_ERR_DTYPE, "cache and output dtypes differ");
  int64_t T, head, start, n;
  visible_range(s, &T, &head, &start, &n);
  if (cache->shape[2] != s->cache_len) return fail(WF_ERR_SHAPE, "cache length mismatch");
  if (out->shape[0] != cache->shape[0] || out->shape[1] != cache->shape[1] ||
      out->shape[2] != n || out->shape[3] != cache->shape[3])
    return fail(WF_ERR_SHAPE, "logical_out must be [B,H,%lld,D]", (long long)n);
  const int64_t cs[3] = {cache->stride[0], cache->stride[1], cache->stride[2]};
  const int64_t os[3] = {out->stride[0], out->stride[1], out->stride[2]};
  return hip_status(wf::launch_kv_gather(u16 ? 16 : esize(cache->dtype), esize(cache->dtype),
                                         cache->data, cs, out->data, os,
                                         (int)cache->shape[0], (int)cache->shape[1], n,
                                         (int)cache->shape[3], T, s->sink, s->window,
                                         (hipStream_t)stream),
                    "gather launch");
}

size_t wf_block_kv_attend_workspace_size(const wf_block_kv_state* s, int B, int Hq, int Lq,
                                         int Dv) {
  if (s == nullptr || B < 0 || Hq < 0 || Lq < 0 || Dv < 0) return 0;
  const int64_t rows = (int64_t)B * Hq * Lq;
  return (size_t)(kMaxSplits * rows * ((int64_t)Dv + 1) * 4 + 256);
}

}  // extern "C"

// The chunk a fused update + attend writes: its rows and first token.
struct FusedUpdate {
  const wf_tensor* k_new;
  const wf_tensor* v_new;
  int64_t tok0;
};

// wf_block_kv_attend over state s; with fu, the same launch also writes the chunk fu names
// into the caches (s is then the state after that update) and reads its rows from fu's
// tensors. dry: validate only, enqueue nothing.
static int attend_impl(const wf_block_kv_state* s, const wf_tensor* q, const wf_tensor* k_cache,
                       const wf_tensor* v_cache, int is_causal, float scale, wf_tensor* out,
                       void* workspace, size_t workspace_bytes, void* stream,
                       const FusedUpdate* fu, bool dry) {
  int rc;
  if ((rc = check_cache_state(s))) return rc;
  if ((rc = check_data(q, "q", 4)) || (rc = check_data(k_cache, "k_cache", 4)) ||
      (rc = check_data(v_cache, "v_cache", 4)) || (rc = check_data(out, "out", 4)))
    return rc;
  if (k_cache->dtype != q->dtype || v_cache->dtype != q->dtype || out->dtype != q->dtype)
    return fail(WF_ERR_DTYPE, "q, caches and out must share one dtype");
  if (q->dtype == WF_F32) return fail(WF_ERR_DTYPE, "cache attend takes f16 or bf16");
  const int64_t B = q->shape[0], Hq = q->shape[1], Lq = q->shape[2], D = q->shape[3];
  const int64_t Hkv = k_cache->shape[1], Dv = v_cache->shape[3];
  if (k_cache->shape[0] != B || v_cache->shape[0] != B || v_cache->shape[1] != Hkv ||
      k_cache->shape[2] != s->cache_len || v_cache->shape[2] != s->cache_len || k_cache->shape[3] != D)
    return fail(WF_ERR_SHAPE, "caches must be [B,Hkv,cache_len,D]");
  if (out->shape[0] != B || out->shape[1] != Hq || out->shape[2] != Lq || out->shape[3] != Dv)
    return fail(WF_ERR_SHAPE, "out must be [B,Hq,Lq,Dv]");
  if (Hkv <= 0 || Hq % Hkv != 0) return fail(WF_ERR_SHAPE, "Hq must be a multiple of Hkv");
  if (!((D == 64 && Dv == 64) || (D == 128 && Dv == 128)))
    return fail(WF_ERR_UNSUPPORTED, "head dims (%lld, %lld) not built", (long long)D, (long long)Dv);
  float sc;
  if ((rc = resolve_scale(scale, D, &sc))) return rc;
  const size_t need = wf_block_kv_attend_workspace_size(s, (int)B, (int)Hq, (int)Lq, (int)Dv);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(WF_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(WF_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (s->cache_len > 0x7fffffff) return fail(WF_ERR_SHAPE, "cache_len exceeds 2^31");
  if (dry) return WF_OK;
  if (B * Hq * Lq == 0) return ok();
  int64_t T, head, start, n_vis;
  visible_range(s, &T, &head, &start, &n_vis);
  // The split kernel reads the visible tokens in chronological order through the slot map
  // (sink prefix, then the window from its oldest token, wrapping round the ring).
  const int dt = kernel_dtype(q->dtype);
  // The query heads of a KV head share each K/V tile (as in wf_sdpa_decode).
  const int64_t G = Hq / Hkv;
  const int hpw = G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1;
  const int causal = is_causal ? 1 : 0;
  const int cus = cu_count();
  if (cus <= 0) return fail(WF_ERR_HIP, "cannot query the device's compute units");
  // About 3/4 of a work group per CU: measured on the 256-query chunk over a 4k window (256
  // CUs), 4-wave groups: 192 run 20% faster than 512 (fewer fp32 partials to write and
  // merge) and ~4% faster than 256; 8-wave groups: 192 (8 splits) as fast as 240 (10 splits,
  // whose combine takes 1.4 us more), while 264 no longer fit in one round.
  int64_t target = std::max(1, cus * 3 / 4);
  if (tune(T_ATTEND_GROUPS) > 0) target = tune(T_ATTEND_GROUPS);
  const int64_t n_kt_all = (n_vis + 63) / 64;
  // One query head per KV head and more than 128 queries: 8-wave groups (256 query rows of
  // one head, two waves per SIMD) share each K/V tile. Measured on the 256-query chunk over a
  // 4k window (kernel trace of the 64-chunk stream): split kernel 24.8 us against 29.4 us
  // with 4-wave groups (one wave per SIMD), combine 6.1 against 4.5 us (8 splits instead
  // of 4). Fewer queries keep 4-wave groups (rows past Lq still run their MFMAs), and so do
  // short caches where the 8-wave plan would give each split a single key tile (the first
  // chunks of that stream: 18-19 us against 14 us).
  const int tnw = tune(T_ATTEND_NW);
  const int64_t groups8 = ((Lq + 255) / 256) * B * Hkv;
  const bool long8 = n_kt_all >= 2 * std::min<int64_t>(n_kt_all, (target + groups8 - 1) / groups8);
  const int nw = (hpw == 1 && (tnw == 8 || (tnw != 4 && Lq > 128 && long8))) ? 8 : 4;
  const wf::AttnEntry* e = find_attn(dt, (int)D, (int)D, (int)Dv, nw, hpw, wf::MASK_NONE, causal,
                                     fu != nullptr ? wf::MODE_SPLITU : wf::MODE_SPLIT);
  if (!e) return fail(WF_ERR_UNSUPPORTED, "split kernel not built");
  const int n_kt = (int)((n_vis + e->bn - 1) / e->bn);
  const int n_qt = (int)((Lq + e->bmp - 1) / e->bmp);
  const int64_t base_blocks = (int64_t)n_qt * B * Hkv * (G / hpw);
  int n_splits = (int)((target + base_blocks - 1) / base_blocks);
  if (n_splits > kMaxSplits) n_splits = kMaxSplits;
  if (n_splits > n_kt) n_splits = n_kt;
  {
    // each split keeps at least min_tiles key tiles: a split re-reads the queries and writes
    // an fp32 partial row per query, which short key ranges do not pay for
    const int min_tiles = tune(T_ATTEND_MIN_TILES) > 0 ? tune(T_ATTEND_MIN_TILES) : 1;
    const int cap = std::max(1, n_kt / min_tiles);
    if (n_splits > cap) n_splits = cap;
  }
  // One split suffices when the query tiles alone fill the GPU: a non-causal attend does
  // not depend on the order of the keys, so the dense kernels read slots [0, n_vis) in place.
  if (n_splits <= 1 && !causal && n_vis > 0 && fu == nullptr)
    return run_dense(q, k_cache, v_cache, nullptr, wf::MASK_NONE, false, false, 0, sc, out, nullptr,
                     n_vis, (hipStream_t)stream);
  if (n_splits < 1) n_splits = 1;
  const int tps = n_kt > 0 ? (n_kt + n_splits - 1) / n_splits : 1;
  n_splits = n_kt > 0 ? (n_kt + tps - 1) / tps : 1;
  wf::FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q->data; a.q2 = q->data; a.k = k_cache->data; a.k2 = k_cache->data; a.v = v_cache->data;
  a.o = out->data;
  a.q_sb = st(q, 0); a.q_sh = st(q, 1); a.q_sm = q->stride[2];
  a.q2_sb = a.q_sb; a.q2_sh = a.q_sh; a.q2_sm = a.q_sm;
  a.k_sb = st(k_cache, 0); a.k_sh = st(k_cache, 1); a.k_sm = k_cache->stride[2];
  a.k2_sb = a.k_sb; a.k2_sh = a.k_sh; a.k2_sm = a.k_sm;
  a.v_sb = st(v_cache, 0); a.v_sh = st(v_cache, 1); a.v_sm = v_cache->stride[2];
  a.B = (int)B; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.G = (int)(Hq / Hkv); a.Lq = (int)Lq;
  a.Lk = (int)n_vis;
  a.n_qtiles = n_qt;
  a.scale_log2 = sc * wf::kLog2e;
  a.inv_scale = 1.0f / sc;
  a.tiles_per_split = tps;
  // the chunk's queries are the last Lq visible tokens (bottom-right)
  a.causal_shift = causal ? (int)(n_vis - Lq) : 0;
  // key rows in chronological order: sink tokens, then the window from its oldest token
  a.kv_remap = 1;
  a.rm_head = (int)head;
  a.rm_sink = (int)s->sink;
  a.rm_off = (int)((start - s->sink) % s->window);
  a.rm_window = (int)s->window;
  if (fu != nullptr) {
    // the chunk is the newest `chunk` visible tokens
    a.new_lo = (int)(n_vis - s->chunk);
    a.upd_chunk = (int)s->chunk;
    a.upd_tok0 = fu->tok0;
    // window offset of the chunk's first token past the sink (negative while the chunk
    // still overlaps the sink: its rows past the sink then need no folding)
    a.upd_off = (int)(fu->tok0 >= s->sink ? (fu->tok0 - s->sink) % s->window : fu->tok0 - s->sink);
    a.knew = fu->k_new->data;
    a.vnew = fu->v_new->data;
    a.kn_sb = fu->k_new->stride[0]; a.kn_sh = fu->k_new->stride[1]; a.kn_sm = fu->k_new->stride[2];
    a.vn_sb = fu->v_new->stride[0]; a.vn_sh = fu->v_new->stride[1]; a.vn_sm = fu->v_new->stride[2];
  }
  const int64_t rows = B * Hq * Lq;
  a.part_o = (float*)workspace;
  a.part_lse = (float*)((char*)workspace + (size_t)kMaxSplits * rows * Dv * 4);
  hipStream_t strm = (hipStream_t)stream;
  hipError_t he = launch(e->fn, dim3((unsigned)base_blocks, n_splits),
                         dim3(e->nw * 64), a, strm);
  if (he != hipSuccess) return hip_status(he, "split attention launch");
  return hip_status(wf::launch_split_combine(dt, a.part_o, a.part_lse, n_splits, (int)B, (int)Hq,
                                             (int)Lq, (int)Dv, out->data, st(out, 0), st(out, 1),
                                             out->stride[2], nullptr, strm),
                    "combine launch");
}

extern "C" {

int wf_block_kv_attend(const wf_block_kv_state* s, const wf_tensor* q, const wf_tensor* k_cache,
                       const wf_tensor* v_cache, int is_causal, float scale, wf_tensor* out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return attend_impl(s, q, k_cache, v_cache, is_causal, scale, out, workspace, workspace_bytes,
                     stream, nullptr, false);
}

int wf_block_kv_update_attend(wf_block_kv_state* s, int64_t chunk_idx, const wf_tensor* k_new,
                              const wf_tensor* v_new, wf_tensor* k_cache, wf_tensor* v_cache,
                              const wf_tensor* q, int is_causal, float scale, wf_tensor* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  bool u16 = true;
  if ((rc = check_update(s, chunk_idx, k_new, v_new, k_cache, v_cache, &u16))) return rc;
  wf_block_kv_state after = *s;
  after.last_chunk = chunk_idx;
  if ((rc = attend_impl(&after, q, k_cache, v_cache, is_causal, scale, out, workspace,
                        workspace_bytes, stream, nullptr, true)))
    return rc;
  const bool empty = q->shape[0] * q->shape[1] * q->shape[2] == 0 || numel(k_new) == 0;
  if (!u16 || empty) {
    // rows that are not 16-byte multiples (or nothing to attend): the two calls one by one
    if ((rc = wf_block_kv_cache_update(s, chunk_idx, k_new, v_new, k_cache, v_cache, stream)))
      return rc;
    return wf_block_kv_attend(s, q, k_cache, v_cache, is_causal, scale, out, workspace,
                              workspace_bytes, stream);
  }
  const int64_t units = q->shape[0] * k_cache->shape[1] * s->chunk * (k_cache->shape[3] + v_cache->shape[3]) / 8;
  if (units >= ((int64_t)1 << 31)) {   // beyond the fused copy's 32-bit indexing: two calls
    if ((rc = wf_block_kv_cache_update(s, chunk_idx, k_new, v_new, k_cache, v_cache, stream)))
      return rc;
    return wf_block_kv_attend(s, q, k_cache, v_cache, is_causal, scale, out, workspace,
                              workspace_bytes, stream);
  }
  const FusedUpdate fu{k_new, v_new, chunk_idx * s->chunk};
  if ((rc = attend_impl(&after, q, k_cache, v_cache, is_causal, scale, out, workspace,
                        workspace_bytes, stream, &fu, false)))
    return rc;
  s->last_chunk = chunk_idx;
  return ok();
}

size_t wf_sdpa_decode_workspace_size(const wf_tensor* q, const wf_tensor* k,
                                     const wf_tensor* v, int is_causal) {
  if (q == nullptr || k == nullptr || v == nullptr || q->ndim != 4 || k->ndim != 4 || v->ndim != 4)
    return 0;
  const DecodePlan p = decode_plan(kernel_dtype(q->dtype), q->shape[0], q->shape[1], k->shape[1],
                                   q->shape[2], k->shape[2], q->shape[3], v->shape[3],
                                   is_causal != 0);
  if (p.e == nullptr) return 0;
  const int64_t rows = q->shape[0] * q->shape[1] * q->shape[2];
  return (size_t)((int64_t)p.n_splits * rows * (v->shape[3] + 1) * 4 + 256);
}

int wf_sdpa_decode(const wf_tensor* q, const wf_tensor* k, const wf_tensor* v, int is_causal,
                   float scale, wf_tensor* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_data(q, "q", 4)) || (rc = check_data(k, "k", 4)) ||
      (rc = check_data(v, "v", 4)) || (rc = check_data(out, "out", 4)))
    return rc;
  if (k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype)
    return fail(WF_ERR_DTYPE, "q, k, v and out must share one dtype");
  if (q->dtype == WF_F32) return fail(WF_ERR_DTYPE, "decode takes f16 or bf16");
  const int64_t B = q->shape[0], Hq = q->shape[1], Lq = q->shape[2], D = q->shape[3];
  const int64_t Hkv = k->shape[1], Lk = k->shape[2], Dv = v->shape[3];
  if (k->shape[0] != B || v->shape[0] != B || k->shape[3] != D || v->shape[1] != Hkv ||
      v->shape[2] != Lk)
    return fail(WF_ERR_SHAPE, "k must be [B,Hkv,Lk,D] and v [B,Hkv,Lk,Dv] for q [B,Hq,Lq,D]");
  if (out->shape[0] != B || out->shape[1] != Hq || out->shape[2] != Lq || out->shape[3] != Dv)
    return fail(WF_ERR_SHAPE, "out must be [B,Hq,Lq,Dv]");
  if (Hkv <= 0 || Hq % Hkv != 0) return fail(WF_ERR_SHAPE, "Hq must be a multiple of Hkv");
  if (!((D == 64 && Dv == 64) || (D == 128 && Dv == 128)))
    return fail(WF_ERR_UNSUPPORTED, "head dims (%lld, %lld) not built", (long long)D, (long long)Dv);
  if (Lq > 0x7fffffff || Lk > 0x7fffffff) return fail(WF_ERR_SHAPE, "sequence length exceeds 2^31");
  float sc;
  if ((rc = resolve_scale(scale, D, &sc))) return rc;
  const int dt = kernel_dtype(q->dtype);
  const DecodePlan p = decode_plan(dt, B, Hq, Hkv, Lq, Lk, D, Dv, is_causal != 0);
  if (p.e == nullptr) return fail(WF_ERR_UNSUPPORTED, "split kernel not built");
  const int64_t rows = B * Hq * Lq;
  const size_t need = (size_t)((int64_t)p.n_splits * rows * (Dv + 1) * 4 + 256);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(WF_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(WF_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (rows == 0 || Dv == 0) return ok();
  const int64_t G = Hq / Hkv;
  const int64_t base_blocks = p.base;
  if (base_blocks > 0x7fffffff) return fail(WF_ERR_SHAPE, "problem too large for one launch");
  wf::FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q->data; a.q2 = q->data; a.k = k->data; a.k2 = k->data; a.v = v->data;
  a.o = out->data;
  a.q_sb = st(q, 0); a.q_sh = st(q, 1); a.q_sm = q->stride[2];
  a.q2_sb = a.q_sb; a.q2_sh = a.q_sh; a.q2_sm = a.q_sm;
  a.k_sb = st(k, 0); a.k_sh = st(k, 1); a.k_sm = k->stride[2];
  a.k2_sb = a.k_sb; a.k2_sh = a.k_sh; a.k2_sm = a.k_sm;
  a.v_sb = st(v, 0); a.v_sh = st(v, 1); a.v_sm = v->stride[2];
  a.B = (int)B; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.G = (int)G; a.Lq = (int)Lq; a.Lk = (int)Lk;
  a.causal_shift = is_causal ? (int)(Lk - Lq) : 0;   // the queries are the last Lq positions
  a.n_qtiles = p.n_qt;
  a.scale_log2 = sc * wf::kLog2e;
  a.inv_scale = 1.0f / sc;
  a.tiles_per_split = p.tps;
  a.part_o = (float*)workspace;
  a.part_lse = (float*)((char*)workspace + (size_t)p.n_splits * rows * Dv * 4);
  hipStream_t strm = (hipStream_t)stream;
  hipError_t he = launch(p.e->fn, dim3((unsigned)base_blocks, p.n_splits), dim3(p.e->nw * 64), a, strm);
  if (he != hipSuccess) return hip_status(he, "split attention launch");
  return hip_status(wf::launch_split_combine(dt, a.part_o, a.part_lse, p.n_splits, (int)B, (int)Hq,
                                             (int)Lq, (int)Dv, out->data, st(out, 0), st(out, 1),
                                             out->stride[2], lse, strm),
                    "combine launch");
}

}  // extern "C"
