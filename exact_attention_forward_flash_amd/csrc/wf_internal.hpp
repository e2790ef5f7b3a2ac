// Internal interface between the C-ABI layer (wf_api.cpp) and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd.hpp"
#include "attn_fwd_w.hpp"
#include "attn_fwd_p.hpp"
#include "attn_fwd_q.hpp"

namespace wf {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// One compiled instantiation of attn_fwd_kernel (32 queries per wave) or attn_fwd_w_kernel
// (64 queries per wave).
struct AttnEntry {
  int dtype, dqk, dqk1, dv, nw, qpw, hpw, mask, causal, mode;
  const void* fn;   // __global__ void(FwdArgs)
  int bmp;          // query positions per work group
  int bn;           // keys per tile
};

// Tables exported by the kernel translation units.
const AttnEntry* attn_table_sdpa_bf16_d64(int* n);
const AttnEntry* attn_table_sdpa_bf16_d128(int* n);
const AttnEntry* attn_table_sdpa_f16_d64(int* n);
const AttnEntry* attn_table_sdpa_f16_d128(int* n);
const AttnEntry* attn_table_sdpa_bf16_dmix(int* n);
const AttnEntry* attn_table_sdpa_f16_dmix(int* n);
const AttnEntry* attn_table_mla(int* n);
const AttnEntry* attn_table_mla_v64(int* n);
const AttnEntry* attn_table_p_rope_bf16(int* n);
const AttnEntry* attn_table_p_rope_f16(int* n);
const AttnEntry* attn_table_p_ropei_bf16(int* n);
const AttnEntry* attn_table_p_ropei_f16(int* n);
const AttnEntry* attn_table_split_bf16(int* n);
const AttnEntry* attn_table_split_f16(int* n);
const AttnEntry* attn_table_splitp_bf16(int* n);
const AttnEntry* attn_table_splitp_f16(int* n);
const AttnEntry* attn_table_splitu_bf16(int* n);
const AttnEntry* attn_table_splitu_f16(int* n);
const AttnEntry* attn_table_w_bf16_d128(int* n);
const AttnEntry* attn_table_w_bf16_d64(int* n);
const AttnEntry* attn_table_w_f16_d128(int* n);
const AttnEntry* attn_table_w_f16_d64(int* n);
const AttnEntry* attn_table_p_bf16_d128(int* n);
const AttnEntry* attn_table_p_bf16_d64(int* n);
const AttnEntry* attn_table_p_f16_d128(int* n);
const AttnEntry* attn_table_p_f16_d64(int* n);
const AttnEntry* attn_table_q_bf16_d128(int* n);
const AttnEntry* attn_table_q_f16_d128(int* n);

#define WF_ATTN_ENTRY(T, DT, DQK, DQK1, DV, NW, HPW, MASK, CAUSAL, MODE)                     \
  {DT, DQK, DQK1, DV, NW, 32, HPW, MASK, CAUSAL, MODE,                                      \
   (const void*)&attn_fwd_kernel<T, DQK, DQK1, DV, NW, HPW, MASK, CAUSAL, MODE>,             \
   AttnFwd<T, DQK, DQK1, DV, NW, HPW, MASK, CAUSAL, MODE>::BMP, 64}

// Translation units holding 64-query-wave instantiations are compiled with the MFMA VGPR
// form forced for compiler-generated MFMAs (the S^T products), see attn_fwd_w.hpp.
#define WF_ATTN_W_ENTRY(T, DT, DQK, DQK1, DV, HPW, MASK, CAUSAL, MODE)                       \
  {DT, DQK, DQK1, DV, 4, 64, HPW, MASK, CAUSAL, MODE,                                       \
   (const void*)&attn_fwd_w_kernel<T, DQK, DQK1, DV, HPW, MASK, CAUSAL, MODE>,               \
   AttnFwdW<T, DQK, DQK1, DV, HPW, MASK, CAUSAL, MODE>::BMP, 64}

// Persistent dense kernel (32 queries per wave, 8 waves, no mask): one work group per CU
// walks its list of at most AttnFwdP<...>::MAX_ITEMS work items.
#define WF_ATTN_P_ENTRY(T, DT, D, HPW, CAUSAL, SUM16)                                        \
  {DT, D, D, D, 8, 32, HPW, MASK_NONE, CAUSAL, SUM16 ? MODE_DENSE_P16 : MODE_DENSE_P,      \
   (const void*)&attn_fwd_p_kernel<T, D, D, HPW, CAUSAL, SUM16>,                             \
   AttnFwdP<T, D, D, HPW, CAUSAL, SUM16>::BMP, 64}
// ROPE 1 (rotate-half) or 2 (interleaved): the persistent kernel that turns Q as it reads it.
#define WF_ATTN_PR_ENTRY(T, DT, D, HPW, CAUSAL, SUM16, ROPE)                                 \
  {DT, D, D, D, 8, 32, HPW, MASK_NONE, CAUSAL,                                              \
   ROPE == 1 ? (SUM16 ? MODE_DENSE_PR16 : MODE_DENSE_PR) : (SUM16 ? MODE_DENSE_PI16 : MODE_DENSE_PI), \
   (const void*)&attn_fwd_p_kernel<T, D, D, HPW, CAUSAL, SUM16, ROPE>,                       \
   AttnFwdP<T, D, D, HPW, CAUSAL, SUM16, ROPE>::BMP, 64}
constexpr int kPersistMaxItems = AttnFwdP<__bf16, 128, 128, 4, false, false>::MAX_ITEMS;
// Persistent 64-query-wave kernel (4 waves, one per SIMD, no mask, no lse), built in
// translation units that force the VGPR form of compiler-generated MFMAs.
#define WF_ATTN_Q_ENTRY(T, DT, D, HPW, CAUSAL)                                               \
  {DT, D, D, D, 4, 64, HPW, MASK_NONE, CAUSAL, MODE_DENSE_Q,                                \
   (const void*)&attn_fwd_q_kernel<T, D, HPW, CAUSAL>, AttnFwdQ<T, D, HPW, CAUSAL>::BMP, 64}
constexpr int kQMaxItems = AttnFwdQ<__bf16, 128, 4, false>::MAX_ITEMS;

// fp32 path (MFMA 32x32x2 f32).
struct F32Entry {
  int dqk, dv, mask, causal;
  const void* fn;
  int bm;  // queries per work group
};
const F32Entry* attn_table_f32(int* n);
// key-split form for one 32-query tile per (batch, head)
const F32Entry* attn_table_f32_ks(int* n);

// Rotary embedding pass (rope.hip): one tensor's input strides, contiguous output, shape and
// first position.
struct RopeDesc {
  const void* x;
  int64_t sb, sh, sm;
  void* y;
  int B, H, L;
  int64_t pos0;
};
hipError_t launch_rope(int dtype, const RopeDesc& q, const RopeDesc& k, int D, int rot, int style,
                       const float* cosb, const float* sinb, hipStream_t st);

// Auxiliary kernels.
hipError_t launch_varlen_schedule(const int32_t* q_seqlen, const int32_t* kv_seqlen, int batch,
                                  int64_t total_q, int64_t total_k, int max_kv, int bmp, int bn,
                                  int causal, int max_items, int* ws, hipStream_t s);
hipError_t launch_split_combine(int dtype, const float* part_o, const float* part_lse,
                                int n_splits, int B, int Hq, int Lq, int Dv, void* out,
                                int64_t o_sb, int64_t o_sh, int64_t o_sm, float* lse,
                                hipStream_t s);
hipError_t launch_kv_update(int unit, int esize, const void* k_new, const int64_t* kn_st,
                            const void* v_new, const int64_t* vn_st, void* k_cache,
                            const int64_t* kc_st, void* v_cache, const int64_t* vc_st, int B,
                            int H, int chunk, int Dk, int Dv, int64_t tok0, int64_t sink,
                            int64_t window, hipStream_t s);
hipError_t launch_kv_gather(int unit, int esize, const void* cache, const int64_t* c_st, void* out,
                            const int64_t* o_st, int B, int H, int64_t n_vis, int D,
                            int64_t T, int64_t sink, int64_t window, hipStream_t s);

// Varlen workspace layout (bytes from the workspace base).
struct VarlenWs {
  // [0] counter, [1] n_items, [2] error, [16 + 4x] the work counter of XCD x (x < 8)
  static constexpr int64_t kHeaderInts = 64;
  __host__ __device__ static int64_t cu_q_off() { return kHeaderInts * 4; }
  __host__ __device__ static int64_t cu_k_off(int batch) { return cu_q_off() + align(((int64_t)batch + 1) * 4); }
  __host__ __device__ static int64_t items_off(int batch) { return cu_k_off(batch) + align(((int64_t)batch + 1) * 4); }
  __host__ __device__ static int64_t bytes(int batch, int64_t max_items) { return items_off(batch) + align(max_items * 8); }
  __host__ __device__ static int64_t align(int64_t x) { return (x + 255) / 256 * 256; }
};

}  // namespace wf
