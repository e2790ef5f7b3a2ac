// Flash-style exact attention forward for gfx950, 16-bit inputs (bf16 / fp16).
//
// Computes out = softmax(scale * Q K^T [+ mask]) V exactly (online softmax, fp32 state)
// for the PyTorch-SDPA-style call (WorldFoundry "Core 注意力", "选择最窄的入口"), the
// packed varlen MLA prefill whose score is q.k + qRope.kRope (Ascend "MLA Prefill"
// parameter table) and the split-KV attend over a block KV cache ("Block KV cache 的调用顺序").
//
// Work decomposition
//   A work group holds HPW query heads of one KV head (GQA) times BMP query positions;
//   each of its NW waves owns 32 queries of one head. Keys stream through in tiles of
//   BN = 64, double-buffered in LDS and copied there by direct global->LDS loads.
//
// Transposed formulation
//   Each wave computes S^T = K Q^T (A = K tile from LDS, B = Q^T resident in VGPRs) and
//   O^T += V^T P^T (A = V^T read from the row-major V tile with ds_read_b64_tr_b16,
//   B = P^T taken straight from the S^T accumulator). In this layout lane l owns query
//   l % 32 and half of its keys, so the row max / row sum of the online softmax need no
//   shuffles inside a half-wave and a single permlane32 swap across halves; O^T is
//   rescaled by a per-lane factor.
//
// Online softmax (log2 domain, t = scale*log2(e)*s [+ log2(e)*mask]):
//   m is a per-query reference max; p = exp2(t - m); l = sum p; O = sum p v.
//   m is raised (and O, l rescaled by exp2(m_old - m_new)) only when some query's tile
//   max exceeds m by more than 8, so p <= 2^8; the result O / l is the same quantity.
//
// LDS layouts (16-byte chunks, XOR-swizzled so MFMA operand reads hit distinct banks)
//   K tile row r (a key), chunk c (8 head-dim elements) at chunk position c ^ (r % 8).
//   V tile row r, chunk c at position c ^ (2 * (r % 4)).
#pragma once
#include <type_traits>

#include "wf_device.hpp"

namespace wf {

enum { MASK_NONE = 0, MASK_BOOL = 1, MASK_HALF = 2, MASK_F32 = 3 };
// MODE_DENSE_P / MODE_DENSE_P16 tag the table rows of the persistent dense kernel
// (attn_fwd_p.hpp) with fp32 row sums and with row sums over the 16-bit weights.
// MODE_SPLITP: split-KV with the G*Lq (query head, position) rows of a KV head packed into
// the query rows of the tiles (row r = head r / Lq, position r % Lq), for few queries per head.
// MODE_DENSE_PR / MODE_DENSE_PR16: the persistent kernel that turns Q by a rotate-half table;
// MODE_DENSE_PI / MODE_DENSE_PI16: by an interleaved one.
// MODE_DENSE_Q: the persistent 64-query-wave kernel (attn_fwd_q.hpp), calls without the lse.
enum { MODE_DENSE = 0, MODE_VARLEN = 1, MODE_SPLIT = 2, MODE_DENSE_P = 3, MODE_DENSE_P16 = 4,
       MODE_SPLITP = 5, MODE_DENSE_PR = 6, MODE_DENSE_PR16 = 7, MODE_DENSE_PI = 8,
       MODE_DENSE_PI16 = 9, MODE_DENSE_Q = 10,
       MODE_SPLITU = 11,     // split-KV over the block KV cache with the fused chunk update
       MODE_DENSE_PM = 12 }; // dense with a mask, no lse: Q prescaled, scores from -m (see PRE)

struct FwdArgs {
  const void* q; const void* q2; const void* k; const void* k2; const void* v;
  void* o; float* lse; const void* mask;
  // strides in elements: batch, head, row (token)
  int64_t q_sb, q_sh, q_sm, q2_sb, q2_sh, q2_sm;
  int64_t k_sb, k_sh, k_sm, k2_sb, k2_sh, k2_sm;
  int64_t v_sb, v_sh, v_sm;
  int64_t o_sb, o_sh, o_sm;
  int64_t mk_sb, mk_sh, mk_sm;
  int B, Hq, Hkv, G, Lq, Lk;
  int causal_shift;   // key j kept for query i iff j <= i + shift
  int n_qtiles;       // query tiles per head group (dense / split)
  int mask_vec;       // mask rows allow 4-element vector loads
  int mask_lds;       // bool / 16-bit mask tiles may be copied into LDS (16-byte aligned rows)
  float scale_log2;   // scale * log2(e)
  float inv_scale;    // 1 / scale (float masks are added to raw scores as mask / scale)
  // varlen (persistent) mode
  const int* cu_q; const int* cu_k; const int2* items; int* counter; const int* n_items;
  int kv_padded;      // K/V rows of sequence i start at i * k_sb (padded), not at cu_k[i]
  int xcd_parts;      // work split over the 8 XCDs by KV head (counter[16 + 4x] for XCD x)
  // split-KV mode
  int tiles_per_split; float* part_o; float* part_lse;
  // rotary embedding of Q as it is read (persistent ROPE kernels): query row i turns pair d by
  // rq_cos[i][d], rq_sin[i][d] (rows of rq_rot / 2 floats, already offset to the first query's
  // position); rotate-half kernels take rq_rot = head dim
  const float* rq_cos; const float* rq_sin;
  int rq_rot;
  // block KV cache (split mode): key row t is the t-th visible token in chronological order,
  // held in slot t (t < rm_head: the sink) or rm_sink + (rm_off + t - rm_head) mod rm_window
  int kv_remap, rm_head, rm_sink, rm_off, rm_window;
  // fused cache update (MODE_SPLITU): the chunk's new K / V rows [B, Hkv, upd_chunk, d] are
  // read for key rows >= new_lo straight from knew / vnew, and the work groups also copy
  // them into their ring slots (tokens upd_tok0 ..) of the caches a.k / a.v
  int new_lo, upd_chunk, upd_off;
  const void* knew; const void* vnew;
  int64_t kn_sb, kn_sh, kn_sm, vn_sb, vn_sh, vn_sm;
  int64_t upd_tok0;
};

struct WorkItem {
  int b, hq0, pos0, Lq, Lk, shift, kt_lo, kt_hi, split;
  int64_t qtok0, ktok0;
};

// LDS swizzles (chunk position = chunk ^ swizzle(row)) for tiles of CH 16-byte chunks per
// row. They keep the MFMA operand reads conflict-free whether the LDS serves 128 or 256
// bytes per clock:
//  K (16-byte reads, lane -> row): any 8 and any 16 consecutive rows get distinct banks.
//  V (8-byte transpose reads over 4 consecutive rows x 2 or 4 chunks): the 4 rows of a
//    16-lane group and of a 32-lane group land on distinct banks.
template <int CH>
__device__ __forceinline__ int lds_kswz(int row) {
  return CH == 16 ? (row & 15) : ((row ^ ((row >> 3) & 3)) & 7);  // period 32 in row
}
template <int CH>
__device__ __forceinline__ int lds_vswz(int row) {
  // 12-chunk (96-wide) rows: the swizzle stays inside aligned groups of 4 chunks, and the
  // 4 rows of a transpose read (192 bytes apart) land on disjoint banks.
  return CH == 16 ? (((row & 1) * 6) ^ ((row & 2) * 5)) : CH == 12 ? 2 * ((row >> 1) & 1) : 2 * (row & 3);
}

template <typename T, int DQK, int DQK1, int DV, int NW, int HPW, int MASK, bool CAUSAL, int MODE>
struct AttnFwd {
  typedef T elem_t;
  static constexpr int kDQK = DQK, kDV = DV;
  static constexpr int BN = 64;
  static constexpr int kNW = NW;
  static constexpr int kHPW = HPW;
  static constexpr bool kPack = MODE == MODE_SPLITP;  // rows are packed (head, position) pairs
  static constexpr int KCH = DQK / 8;
  static constexpr int VCH = DV / 8;
  static constexpr int WPH = NW / HPW;
  static constexpr int BMP = WPH * 32;
  static constexpr int NT = NW * 64;
  static constexpr int KLOADS = BN * KCH / NT;
  // V copies: whole waves of 64 chunks; with 96-wide rows the last round covers only part of
  // the group (the waves past the tile skip it)
  static constexpr int VLOADS = (BN * VCH + NT - 1) / NT;
  static constexpr int KBYTES = BN * DQK * 2;
  static constexpr int VBYTES = BN * DV * 2;
  static constexpr int NS = DQK / 16;
  static constexpr int NDV = DV / 32;
  // Bool and 16-bit masks of one-head groups: the mask tile of the group's rows (BMP rows x BN
  // keys) is copied into LDS with the K tile (coalesced), instead of every lane reading its own
  // row from global memory (32 rows per load instruction).
  static constexpr int MSZ = MASK == MASK_BOOL ? 1 : MASK == MASK_HALF ? 2 : 4;
  static constexpr bool MLDS = (MASK == MASK_BOOL || MASK == MASK_HALF) && HPW == 1 &&
                               (MODE == MODE_DENSE || MODE == MODE_DENSE_PM);
  static constexpr int MROWB = BN * MSZ;                 // bytes of one row of a mask tile
  static constexpr int MCPR = MROWB / 16;                // its 16-byte chunks
  // chunk swizzle of mask tile rows in LDS (position = chunk ^ mswz(row))
  static __device__ __forceinline__ int mswz(int row) {
    return ((row >> 1) ^ (row >> 3)) & (MCPR - 1);
  }
  static constexpr int MBYTES = MLDS ? BMP * MROWB : 16;
  static constexpr int MLOADS = MLDS ? MBYTES / (NT * 16) : 0;
  static_assert(!MLDS || MBYTES % (NT * 16) == 0, "mask tile copies split evenly");
  // K and V tiles of 16 KiB carry the largest alignment, which places them first in LDS
  // (operand reads then address them with immediate offsets).
  static constexpr int KALIGN = (KBYTES == VBYTES && (KBYTES & (KBYTES - 1)) == 0) ? KBYTES : 1024;
  static_assert(sizeof(T) == 2, "16-bit inputs only");
  static_assert(NW % HPW == 0, "waves split evenly over heads");
  static_assert((BN * KCH) % NT == 0 && (BN * VCH) % 64 == 0, "tile copies split evenly");
  static_assert(KCH % 8 == 0 && (VCH % 8 == 0 || VCH == 12) && DQK1 % 16 == 0 && DV % 32 == 0,
                "tile shape");

  static __device__ __forceinline__ int kswz(int row) { return lds_kswz<KCH>(row); }
  static __device__ __forceinline__ int vswz(int row) { return lds_vswz<VCH>(row); }

  // Number of key tiles a work group covering positions [pos0, pos0 + BMP) must visit.
  static __device__ __forceinline__ int tile_end(int pos0, int Lk, int shift) {
    const int n_kt = (Lk + BN - 1) / BN;
    if (!CAUSAL) return n_kt;
    const int lim = pos0 + BMP - 1 + shift;  // last key any query of the group keeps
    if (lim < 0) return 0;
    const int e = lim / BN + 1;
    return e < n_kt ? e : n_kt;
  }

  static __device__ __forceinline__ void run(const FwdArgs& a, const WorkItem& it,
                                             WF_LDS char* sK0, WF_LDS char* sK1,
                                             WF_LDS char* sV0, WF_LDS char* sV1,
                                             WF_LDS char* sM0, WF_LDS char* sM1) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, hf = lane >> 5;
    const int hw = w / WPH;
    const int qw = (w % WPH) * 32;
    const int hq = it.hq0 + hw;
    const int g = it.hq0 / a.G;
    const float c = a.scale_log2;

    constexpr bool PACK = MODE == MODE_SPLITP;
    // PRE (masked dense calls without the lse): Q is multiplied by scale*log2(e) and rounded
    // back to the input type once, and the S^T accumulators start from -m_ref, so the MFMAs
    // give log2-domain scores relative to the reference max and the weights are exp2 of them
    // with no per-score FMA (the VALU work per score is what bounds masked calls at small head
    // dims). The rounding of the scaled Q changes every score of a row by a common factor of
    // order 1e-4, as in the persistent kernel without the lse; calls asking for the lse keep
    // the exact form.
    constexpr bool PRE = MODE == MODE_DENSE_PM;
    static_assert(!PACK || (HPW == 1 && MASK == MASK_NONE && DQK1 == DQK), "packed rows: plain split only");
    const T* qp = (const T*)a.q + it.b * a.q_sb + hq * a.q_sh + it.qtok0 * a.q_sm;
    const T* q2p = (const T*)a.q2 + it.b * a.q2_sb + hq * a.q2_sh + it.qtok0 * a.q2_sm;
    const T* kp = (const T*)a.k + it.b * a.k_sb + g * a.k_sh + it.ktok0 * a.k_sm;
    const T* k2p = (const T*)a.k2 + it.b * a.k2_sb + g * a.k2_sh + it.ktok0 * a.k2_sm;
    const T* vp = (const T*)a.v + it.b * a.v_sb + g * a.v_sh + it.ktok0 * a.v_sm;

    // ---- Q^T operand: lane (j, hf) holds query row j, head-dim elements 16s + 8hf.. ----
    const int qlo = it.pos0 + qw;
    const int qrow = qlo + j;
    const int qrow_c = qrow < it.Lq ? qrow : it.Lq - 1;
    // This lane's query: its head, its position (the causal rule) and whether it exists.
    // Packed rows: row qrow of the item is (head hq0 + qrow / Lq, position qrow % Lq); the
    // wave's positions then lie anywhere in [0, Lq), so tile ranges use that whole interval.
    const int prow_c = PACK ? (qrow < a.G * it.Lq ? qrow : a.G * it.Lq - 1) : 0;
    const int hq_l = PACK ? it.hq0 + prow_c / it.Lq : hq;
    const int qpos = PACK ? prow_c % it.Lq : qrow;
    const bool row_ok = PACK ? qrow < a.G * it.Lq : qrow < it.Lq;
    const int pos_lo = PACK ? 0 : qlo;                 // lowest position of the wave's rows
    const int pos_hi = PACK ? it.Lq - 1 : qlo + 31;    // highest
    u32x4 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int col = 16 * s + 8 * hf;
      const T* src;
      if constexpr (PACK)
        src = (const T*)a.q + it.b * a.q_sb + hq_l * a.q_sh + (it.qtok0 + qpos) * a.q_sm + col;
      else
        src = (16 * s < DQK1) ? qp + (int64_t)qrow_c * a.q_sm + col
                              : q2p + (int64_t)qrow_c * a.q2_sm + (col - DQK1);
      qf[s] = *reinterpret_cast<const u32x4*>(src);
      if constexpr (PRE) {
        typedef typename Mfma16<T>::v8 v8;
        v8 x = __builtin_bit_cast(v8, qf[s]);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (T)((float)x[e] * a.scale_log2);
        qf[s] = __builtin_bit_cast(u32x4, x);
      }
    }

    // ---- per-thread copy descriptors for the K and V tiles ---------------------------
    // Copy i of wave w fills tile chunks [(i*NW + w)*64, +64): lane -> chunk p, row p/KCH,
    // swizzled position p%KCH, which holds logical chunk (p%KCH) ^ swizzle(row).
    const T* ksrc[KLOADS];
    int64_t kstride[KLOADS];
    int krow[KLOADS], kcol[KLOADS];
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int p = (i * NW + w) * 64 + lane;
      const int r = p / KCH, pos = p % KCH;
      const int col = (pos ^ kswz(r)) * 8;
      krow[i] = r;
      kcol[i] = col;
      if (DQK1 == DQK || col < DQK1) { ksrc[i] = kp + col; kstride[i] = a.k_sm; }
      else { ksrc[i] = k2p + (col - DQK1); kstride[i] = a.k2_sm; }
    }
    const T* vsrc[VLOADS];
    int vrow[VLOADS], vcol[VLOADS];
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int p = (i * NW + w) * 64 + lane;
      const int pc = p < BN * VCH ? p : BN * VCH - 1;   // past the tile: never issued
      const int r = pc / VCH, pos = pc % VCH;
      vrow[i] = r;
      vcol[i] = (pos ^ vswz(r)) * 8;
      vsrc[i] = vp + vcol[i];
    }
    const int lk_last = it.Lk - 1;
    // Memory row of key row r: r itself, or (block KV cache) the slot of the r-th visible
    // token, so that key rows run in chronological order whatever the ring's rotation.
    constexpr bool kSplitMode = MODE == MODE_SPLIT || MODE == MODE_SPLITU;
    const int rm_on = kSplitMode ? a.kv_remap : 0, rm_head = kSplitMode ? a.rm_head : 0;
    const int rm_off = kSplitMode ? a.rm_off : 0, rm_window = kSplitMode ? a.rm_window : 1;
    const int rm_sink = kSplitMode ? a.rm_sink : 0;
    auto key_row = [&](int r) {
      if constexpr (!kSplitMode) return r;
      int x = rm_off + (r - rm_head);   // < 2 * rm_window when r >= rm_head
      x = x >= rm_window ? x - rm_window : x;
      return (rm_on && r >= rm_head) ? rm_sink + x : r;   // selects, no branch
    };
    // Rows past the last key are clamped onto it: their scores are masked to -inf, and
    // the duplicated V rows meet p = 0.
    // Fused cache update: rows of the new chunk come from its own tensors (same bits as the
    // slots the update writes, which this launch does not read).
    constexpr bool fresh = MODE == MODE_SPLITU;
    // uniform values of the fresh-row addressing, read once: a new row's element offset from
    // the cache head base is (new head base - cache head base) + (r - new_lo) * row stride
    const int new_lo = fresh ? a.new_lo : 0;
    const int64_t kn_sm = fresh ? a.kn_sm : 0, vn_sm = fresh ? a.vn_sm : 0;
    const int64_t kn_delta =
        fresh ? (int64_t)(((const T*)a.knew + it.b * a.kn_sb + g * a.kn_sh) - kp) : 0;
    const int64_t vn_delta =
        fresh ? (int64_t)(((const T*)a.vnew + it.b * a.vn_sb + g * a.vn_sh) - vp) : 0;
    const int64_t k_sm = a.k_sm, v_sm = a.v_sm;
    // With the fused update a lane's row comes from one of two uniform bases (cache or new
    // chunk) at its column: only the column offset is kept per copy.
    auto issue_k = [&](int kt, WF_LDS char* Kt) {
      const int k0 = kt * BN;
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) {
        int r = k0 + krow[i];
        r = r < lk_last ? r : lk_last;
        const T* src;
        if constexpr (fresh) {
          const int64_t off = r >= new_lo ? kn_delta + (int64_t)(r - new_lo) * kn_sm
                                          : (int64_t)key_row(r) * k_sm;
          src = kp + kcol[i] + off;
        } else {
          src = ksrc[i] + (int64_t)key_row(r) * kstride[i];
        }
        dma16(src, Kt + (i * NW + w) * 1024);
      }
    };
    auto issue_v = [&](int kt, WF_LDS char* Vt) {
      const int k0 = kt * BN;
#pragma unroll
      for (int i = 0; i < VLOADS; ++i) {
        if ((BN * VCH) % NT != 0 && (i * NW + w) * 64 >= BN * VCH) continue;  // wave-uniform
        int r = k0 + vrow[i];
        r = r < lk_last ? r : lk_last;
        const T* src;
        if constexpr (fresh) {
          const int64_t off = r >= new_lo ? vn_delta + (int64_t)(r - new_lo) * vn_sm
                                          : (int64_t)key_row(r) * v_sm;
          src = vp + vcol[i] + off;
        } else {
          src = vsrc[i] + (int64_t)key_row(r) * v_sm;
        }
        dma16(src, Vt + (i * NW + w) * 1024);
      }
    };

    // Mask tile copies (MLDS): buffer loads with a per-tile descriptor ending after the last
    // valid row's keys; copy i of wave w fills chunks [(i*NW + w)*64, +64) of the tile, lane
    // -> LDS chunk c: row c / MCPR, position c % MCPR, which holds the row's 16-byte chunk
    // (c % MCPR) ^ mswz(row). Every lane reads its own query row, so unswizzled rows (64 or
    // 128 bytes apart) would put 16 lanes of a read on one bank. With the swizzle, bool
    // masks (read as whole chunks) are conflict-free and 16-bit masks (8-byte reads) 2-way,
    // whether the LDS serves 128 or 256 bytes per clock.
    uint32_t mvo[MLOADS > 0 ? MLOADS : 1];
    const char* mtile0 = nullptr;
    int64_t mrows_bytes = 0;
    if constexpr (MLDS) {
      const int64_t rs = a.mk_sm * MSZ;
#pragma unroll
      for (int i = 0; i < MLOADS; ++i) {
        const int c = (i * NW + w) * 64 + lane;
        const int row = c / MCPR;
        mvo[i] = (uint32_t)row * (uint32_t)rs + (uint32_t)(16 * ((c % MCPR) ^ mswz(row)));
      }
      mtile0 = (const char*)a.mask + (it.b * a.mk_sb + it.hq0 * a.mk_sh + (int64_t)it.pos0 * a.mk_sm) * MSZ;
      const int rows = it.Lq - it.pos0 < BMP ? it.Lq - it.pos0 : BMP;
      mrows_bytes = (int64_t)(rows - 1) * rs;
    }
    auto issue_m = [&](int kt, WF_LDS char* Mt) {
      if constexpr (MLDS) {
        if (a.mask_lds) {
          const int k0 = kt * BN;
          const int64_t keys = it.Lk - k0 < BN ? it.Lk - k0 : BN;
          const int64_t bytes = mrows_bytes + keys * MSZ;
          const uint32_t nrec = bytes <= 0 ? 0u : bytes >= 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
          const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(mtile0 + (int64_t)k0 * MSZ), 0, (int)nrec, 0x00020000);
#pragma unroll
          for (int i = 0; i < MLOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (WF_LDS void*)(Mt + (i * NW + w) * 1024), 16,
                                                     (int)mvo[i], 0, 0, 0);
        }
      }
    };

    // ---- LDS operand offsets ----------------------------------------------------------
    // K operand (A of S^T): lane (j, hf) reads key row 32kb + j, chunk 2s + hf
    // (swizzle(32kb + j) == swizzle(j)).
    int koff[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = j * KCH * 16 + (((2 * s + hf) ^ kswz(j)) * 16);
    // V^T operand (A of O^T) through the transpose read: within each 16-lane group, lane
    // s names row kbase + s/4, head-dim columns dbase + 4*(s%4) .. +3, so lane t receives
    // head-dim dbase + t for the 4 keys kbase .. kbase+3. kbase = 16m + 4hf (+8 for the
    // second read), dbase = 32n + 16*((lane/16)%2).
    const int g16 = (lane >> 4) & 1, b2 = (lane & 3) >> 1;
    const int vrow0 = 4 * hf + ((lane & 15) >> 2);  // row within each 16-key step (+16m, +8)
    const int fv = vswz(vrow0);                      // rows 16m + vrow0 (+8) share it
    int voff[NDV];
#pragma unroll
    for (int n = 0; n < NDV; ++n)
      voff[n] = vrow0 * VCH * 16 + (((4 * n + 2 * g16 + b2) ^ fv) * 16) + 8 * (lane & 1);

    // ---- mask row ---------------------------------------------------------------------
    const char* mrow = nullptr;
    if constexpr (MASK != MASK_NONE) {
      constexpr int msz = MASK == MASK_BOOL ? 1 : MASK == MASK_HALF ? 2 : 4;
      mrow = (const char*)a.mask +
             (it.b * a.mk_sb + hq * a.mk_sh + (int64_t)qrow_c * a.mk_sm) * msz;
    }

    f32x16 oacc[NDV];
#pragma unroll
    for (int n = 0; n < NDV; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[n][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    // PRE: m_ref is the reference the pending tile's scores were computed against (m_run, or 0
    // while m_run is -inf).
    float m_ref = 0.f;

    // Tiles this wave computes: [kt_lo, kt_live). With causal masking a wave is done once a
    // tile starts past its last query; it still copies tiles and meets the barriers.
    int kt_live = it.kt_hi;
    if (CAUSAL) {
      const int lim = pos_hi + it.shift;
      const int e = lim < 0 ? 0 : lim / BN + 1;
      kt_live = e < kt_live ? e : kt_live;
    }
    // A wave whose rows all lie past the item's last query (the end of a sequence or of Lq)
    // computes nothing: no tile of it is live.
    if (!PACK && qlo >= it.Lq) kt_live = it.kt_lo;
    if (kt_live < it.kt_lo) kt_live = it.kt_lo;

    // ---- operand fragments from LDS ----------------------------------------------------
    auto kfrag = [&](const WF_LDS char* Kt, int s, int kb) {
      return lds_read16(Kt + koff[s] + kb * 32 * KCH * 16);
    };
    auto vfrag = [&](const WF_LDS char* Vt, int m, int n) {
      const WF_LDS char* base = Vt + voff[n] + 16 * m * VCH * 16;
      const u32x2 lo = lds_read_tr(base);
      const u32x2 hi = lds_read_tr(base + 8 * VCH * 16);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // ---- masking in the raw score domain ---------------------------------------------------
    // Element r of block kb is key k0 + 32kb + 8(r/4) + 4hf + r%4. Dropped keys become -inf;
    // a float mask m is added as m / scale so that scale*log2(e) times the stored value is
    // the log2-domain score plus log2(e) m.
    auto need_mask = [&](int kt) {
      const int k0 = kt * BN;
      return MASK != MASK_NONE || (k0 + BN > it.Lk) || (CAUSAL && k0 + BN - 1 > pos_lo + it.shift);
    };
    // LDS offsets of this lane's mask bytes in a tile (see mswz): 16-bit masks, the 8 bytes
    // of keys 32kb + 8q4 + 4hf .. +3; bool masks, the whole chunks 2kb + q4/2 (q4 even).
    int moff[2][4];
    if constexpr (MLDS) {
      const int r = qw + j;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int byte = MASK == MASK_BOOL ? 32 * kb + 16 * (q4 >> 1) : (32 * kb + 8 * q4 + 4 * hf) * MSZ;
          moff[kb][q4] = r * MROWB + (((byte >> 4) ^ mswz(r)) << 4) + (byte & 15);
        }
    }
    auto apply_mask = [&](int kt, f32x16* sc) {
      const int k0 = kt * BN;
      // Keys past Lk and, for causal calls, keys after the query: only tiles that reach
      // them need the checks.
      const bool bounds = (k0 + BN > it.Lk) || (CAUSAL && k0 + BN - 1 > pos_lo + it.shift);
      if constexpr (MASK != MASK_NONE) {
        if (MLDS && a.mask_lds) {
          // This lane's row of the tile (qw + j), keys 32kb + 8q4 + 4hf .. +3, from the LDS
          // copy (offsets moff, swizzled): every read is issued before the first use, so
          // the group waits once.
          const WF_LDS char* mt = ((kt - it.kt_lo) & 1) ? sM1 : sM0;
          if constexpr (MASK == MASK_BOOL) {
            // chunk 2kb + h holds keys 32kb + 16h .. +15; this lane's 4-key groups q4 = 2h,
            // 2h + 1 are its dwords hf and 2 + hf
            u32x4 ch[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int h = 0; h < 2; ++h) ch[kb][h] = lds_read16(mt + moff[kb][2 * h]);
            uint32_t bits[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const u32x4 v = ch[kb][q4 >> 1];
                bits[kb][q4] = (q4 & 1) ? (hf ? v[3] : v[2]) : (hf ? v[1] : v[0]);
              }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                sc[kb][r] = ((bits[kb][r >> 2] >> (8 * (r & 3))) & 0xffu) ? sc[kb][r] : -INFINITY;
          } else if constexpr (MASK == MASK_HALF) {
            typedef T t4 __attribute__((ext_vector_type(4)));
            t4 hv[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4)
                hv[kb][q4] = *reinterpret_cast<const WF_LDS t4*>(mt + moff[kb][q4]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                // convert, then an fp32 FMA: the fused mixed-precision FMA measured slower
                float mv = (float)hv[kb][r >> 2][r & 3];
                asm volatile("" : "+v"(mv));
                sc[kb][r] = fmaf(mv, PRE ? kLog2e : a.inv_scale, sc[kb][r]);
              }
          }
        } else {
          float mval[2][4][4];
          const bool vec = a.mask_vec && (k0 + BN <= it.Lk);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int key = k0 + 32 * kb + 8 * q4 + 4 * hf;
              if (vec) {
                if constexpr (MASK == MASK_BOOL) {
                  const uint32_t bits = *reinterpret_cast<const uint32_t*>(mrow + key);
#pragma unroll
                  for (int e = 0; e < 4; ++e)
                    mval[kb][q4][e] = ((bits >> (8 * e)) & 0xffu) ? 0.f : -INFINITY;
                } else if constexpr (MASK == MASK_HALF) {
                  typedef T t4 __attribute__((ext_vector_type(4)));
                  const t4 hv = *reinterpret_cast<const t4*>(mrow + 2 * key);
#pragma unroll
                  for (int e = 0; e < 4; ++e) mval[kb][q4][e] = (float)hv[e];
                } else {
                  const f32x4 f4 = *reinterpret_cast<const f32x4*>(mrow + 4 * key);
#pragma unroll
                  for (int e = 0; e < 4; ++e) mval[kb][q4][e] = f4[e];
                }
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int kk = key + e;
                  float mv = -INFINITY;
                  if (kk < it.Lk) {
                    if constexpr (MASK == MASK_BOOL) mv = mrow[kk] ? 0.f : -INFINITY;
                    else if constexpr (MASK == MASK_HALF) mv = (float)reinterpret_cast<const T*>(mrow)[kk];
                    else mv = reinterpret_cast<const float*>(mrow)[kk];
                  }
                  mval[kb][q4][e] = mv;
                }
              }
            }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              if constexpr (MASK == MASK_BOOL) sc[kb][r] += mval[kb][r >> 2][r & 3];
              else sc[kb][r] = fmaf(mval[kb][r >> 2][r & 3], PRE ? kLog2e : a.inv_scale, sc[kb][r]);
            }
        }
      }
      if (bounds) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            bool ok = key < it.Lk;
            if (CAUSAL) ok = ok && key <= qpos + it.shift;
            sc[kb][r] = ok ? sc[kb][r] : -INFINITY;
          }
      }
    };

    // ---- pipeline pieces -------------------------------------------------------------------
    // S^T = K Q^T for one tile, operand reads one step ahead (prologue only).
    auto s_tile = [&](const WF_LDS char* Kt, f32x16* sc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] = PRE ? -m_ref : 0.f;
      u32x4 k0f = kfrag(Kt, 0, 0), k1f = kfrag(Kt, 0, 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u32x4 n0 = k0f, n1 = k1f;
        if (s + 1 < NS) { n0 = kfrag(Kt, s + 1, 0); n1 = kfrag(Kt, s + 1, 1); }
        sc[0] = Mfma16<T>::run(k0f, qf[s], sc[0]);
        sc[1] = Mfma16<T>::run(k1f, qf[s], sc[1]);
        k0f = n0; k1f = n1;
      }
    };
    // Tile max of the (masked, raw) scores in log2 units, reduced over both half-waves.
    auto tile_max = [&](const f32x16* sc) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      return PRE ? xhalf_max(mx) : xhalf_max(mx) * c;
    };
    // Raise the reference max (rescaling O and l) only when a query's tile max passes it
    // by more than 8, so p = exp2(t - m) stays <= 2^8.
    // PRE: mt is relative to m_ref, and a moved reference shifts the pending tile onto it.
    auto rescale = [&](float mt, f32x16* cur) {
      if (PRE) mt += m_ref;
      if (wave_any(mt > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mt);
        const float m_new_ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_new_ref);
        l_run *= alpha;
#pragma unroll
        for (int n = 0; n < NDV; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[n][r] *= alpha;
        if constexpr (PRE) {
          const float d = m_new_ref - m_ref;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) cur[kb][r] -= d;
          m_ref = m_new_ref;
        }
        m_run = m_new;
      }
    };

    f32x16 sc[2], sn[2];  // scores of even / odd tiles (current and next alternate)
    u32x4 pk[4];          // P^T operands of the current tile
    float mt_cur = -INFINITY;

    // Phase A: p = exp2(scale*log2e*s - m) for the current tile (packed to 16 bits as the
    // P^T operand) while, if there is a next tile, its S^T MFMAs are issued in between.
    // A wave in phase A issues ahead of one in phase B (s_setprio), and the packed weights are
    // pinned at its end so that the exponentials stay among the S^T MFMAs (with the 192-wide
    // MLA score too: 2.6% faster there, no spills).
    auto phase_a = [&](const WF_LDS char* Kn, auto has_next_c, f32x16* cur, f32x16* nxt) {
      constexpr bool has_next = decltype(has_next_c)::value;
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      float psum = 0.f;
      __builtin_amdgcn_s_setprio(3);
      if constexpr (has_next) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) nxt[kb][r] = PRE ? -m_ref : 0.f;
        u32x4 k0f = kfrag(Kn, 0, 0), k1f = kfrag(Kn, 0, 1);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          u32x4 n0 = k0f, n1 = k1f;
          if (s + 1 < NS) { n0 = kfrag(Kn, s + 1, 0); n1 = kfrag(Kn, s + 1, 1); }
          nxt[0] = Mfma16<T>::run(k0f, qf[s], nxt[0]);
#pragma unroll
          for (int e = s * 32 / NS; e < (s + 1) * 32 / NS; ++e) {
            const float p = fast_exp2(PRE ? cur[e >> 4][e & 15] : fmaf(cur[e >> 4][e & 15], c, neg_m));
            cur[e >> 4][e & 15] = p;
            if (!PRE) psum += p;
          }
          nxt[1] = Mfma16<T>::run(k1f, qf[s], nxt[1]);
          k0f = n0; k1f = n1;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const float p = fast_exp2(PRE ? cur[e >> 4][e & 15] : fmaf(cur[e >> 4][e & 15], c, neg_m));
          cur[e >> 4][e & 15] = p;
          if (!PRE) psum += p;
        }
      }
      if (!PRE) l_run += psum;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        pk[m] = pack8<T>(cur[m >> 1], 8 * (m & 1));
        asm volatile("" ::"v"(pk[m]));
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // Phase B: O^T += V^T P^T for the current tile while, if there is a next tile, its row
    // max is folded in between the MFMAs.
    auto phase_b = [&](const WF_LDS char* Vc, auto has_next_c, const f32x16* nxt) {
      constexpr bool has_next = decltype(has_next_c)::value;
      u32x4 vf[NDV];
#pragma unroll
      for (int n = 0; n < NDV; ++n) vf[n] = vfrag(Vc, 0, n);
      float mx = -INFINITY;
      float lp[2] = {0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4 vn[NDV];
#pragma unroll
        for (int n = 0; n < NDV; ++n) vn[n] = m + 1 < 4 ? vfrag(Vc, m + 1, n) : vf[n];
#pragma unroll
        for (int n = 0; n < NDV; ++n) oacc[n] = Mfma16<T>::run(vf[n], pk[m], oacc[n]);
        // PRE: row sums over the packed 16-bit weights (exactly the weights that multiply V)
        if constexpr (PRE) lp[m & 1] = sum8_acc<T>(pk[m], lp[m & 1]);
        if constexpr (has_next) {
#pragma unroll
          for (int e = 8 * m; e < 8 * m + 8; ++e) mx = fmaxf(mx, nxt[e >> 4][e & 15]);
        }
#pragma unroll
        for (int n = 0; n < NDV; ++n) vf[n] = vn[n];
      }
      if constexpr (PRE) {
        // 3 wait states between the last v_dot2c write and an ordinary VALU read of it
        asm volatile("s_nop 2" : "+v"(lp[0]), "+v"(lp[1]));
        l_run += lp[0] + lp[1];
      }
      if constexpr (has_next) mt_cur = PRE ? xhalf_max(mx) : xhalf_max(mx) * c;
    };

    // ---- key-tile loop -----------------------------------------------------------------------
    // Tile u (counted from kt_lo) has K in buffer u%2 and V in buffer u%2. Iteration u reads
    // K_{u+1} (S^T of the next tile) and V_u, and copies K_{u+2} and V_{u+1} meanwhile.
    const int n_tiles = it.kt_hi - it.kt_lo;
    const int n_live = kt_live - it.kt_lo;
    if (n_tiles > 0) {
      issue_k(it.kt_lo, sK0);
      issue_m(it.kt_lo, sM0);
      issue_v(it.kt_lo, sV0);
      if (n_tiles > 1) {
        issue_k(it.kt_lo + 1, sK1);
        issue_m(it.kt_lo + 1, sM1);
      }
      wait_vmem();
      __syncthreads();
      if (n_live > 0) {
        s_tile(sK0, sc);
        if (need_mask(it.kt_lo)) apply_mask(it.kt_lo, sc);
        mt_cur = tile_max(sc);
      }
      __syncthreads();  // K_0's buffer is refilled by the first iteration
      auto iter = [&](int u, const WF_LDS char* Kn, WF_LDS char* Kfill, const WF_LDS char* Vc,
                      WF_LDS char* Vfill, f32x16* cur, f32x16* nxt) {
        if (u + 2 < n_tiles) {
          issue_k(it.kt_lo + u + 2, Kfill);
          issue_m(it.kt_lo + u + 2, (u & 1) ? sM1 : sM0);   // mask tile u+2 replaces tile u's
        }
        if (u + 1 < n_tiles) issue_v(it.kt_lo + u + 1, Vfill);
        if (u < n_live) {
          // The next tile's S^T and row max are always computed: on this wave's last live
          // tile they read a stale K buffer and the result is never used. This keeps both
          // phases branch-free for the scheduler.
          rescale(mt_cur, cur);
          phase_a(Kn, std::true_type(), cur, nxt);
          if (u + 1 < n_live && need_mask(it.kt_lo + u + 1)) apply_mask(it.kt_lo + u + 1, nxt);
          phase_b(Vc, std::true_type(), nxt);
        }
        wait_vmem();
        __syncthreads();
      };
      if constexpr (MODE != MODE_SPLIT && MODE != MODE_SPLITU && MODE != MODE_VARLEN) {
        for (int u = 0;;) {
          iter(u, sK1, sK0, sV0, sV1, sc, sn);  // even tiles: scores in sc, next in sn
          if (++u >= n_tiles) break;
          iter(u, sK0, sK1, sV1, sV0, sn, sc);  // odd tiles: roles swapped
          if (++u >= n_tiles) break;
        }
      } else {
        // Split-KV groups and the varlen items: an item's last tile computes no next S^T
        // (there is none); split groups end there without the wait and barrier, varlen groups
        // keep them for the next item. (The dense modes keep the uniform loop: this second
        // tail spills registers in some of their instantiations.)
        auto last = [&](const WF_LDS char* Vc, f32x16* cur, f32x16* nxt) {
          if (n_tiles - 1 < n_live) {
            rescale(mt_cur, cur);
            phase_a(sK0, std::false_type(), cur, nxt);
            phase_b(Vc, std::false_type(), nxt);
          }
          if constexpr (MODE == MODE_VARLEN) {
            // the group's next item refills the buffers: every wave must be done with them
            wait_vmem();
            __syncthreads();
          }
        };
        const int n_main = n_tiles - 1;
        for (int u = 0; u < n_main;) {
          iter(u, sK1, sK0, sV0, sV1, sc, sn);
          if (++u >= n_main) break;
          iter(u, sK0, sK1, sV1, sV0, sn, sc);
          if (++u >= n_main) break;
        }
        if (n_main & 1) last(sV1, sn, sc);
        else last(sV0, sc, sn);
      }
    }

    // ---- epilogue -----------------------------------------------------------------------
    const float l = xhalf_sum(l_run);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const float lse2 = l > 0.f ? (m_run == -INFINITY ? 0.f : m_run) + __builtin_log2f(l) : -INFINITY;
    if (row_ok) {
      if constexpr (MODE == MODE_SPLIT || MODE == MODE_SPLITP || MODE == MODE_SPLITU) {
        const int64_t row = (((int64_t)it.split * a.B + it.b) * a.Hq + hq_l) * a.Lq + qpos;
        float* dst = a.part_o + row * DV;
#pragma unroll
        for (int n = 0; n < NDV; ++n)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = oacc[n][4 * q4 + e] * inv;
            *reinterpret_cast<f32x4*>(dst + 32 * n + 8 * q4 + 4 * hf) = o4;
          }
        if (hf == 0) a.part_lse[row] = lse2 * kLn2;
      } else {
        T* dst = (T*)a.o + it.b * a.o_sb + hq * a.o_sh + (it.qtok0 + qrow) * a.o_sm;
        typedef T t4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int n = 0; n < NDV; ++n)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            t4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[n][4 * q4 + e] * inv);
            *reinterpret_cast<t4*>(dst + 32 * n + 8 * q4 + 4 * hf) = o4;
          }
        if (MODE == MODE_DENSE && a.lse != nullptr && hf == 0)
          a.lse[((int64_t)it.b * a.Hq + hq) * a.Lq + qrow] = lse2 * kLn2;
      }
    }
  }
};

// Work-group -> work-item decoding for the dense and split grids.
// Dense: longest-first for causal, and when B*Hkv is a multiple of 8 all work groups of one
// KV group run on one XCD (work groups are dealt to the 8 XCDs round-robin by block index),
// so their K/V tiles are served from that XCD's L2.
template <class K, bool CAUSAL>
__device__ __forceinline__ WorkItem decode_grid(const FwdArgs& a, int bid, int split) {
  // head groups per KV head (packed rows: one group holding all G heads)
  const int GH = K::kPack ? 1 : a.G / K::kHPW;
  const int nbg = a.B * a.Hkv;
  int hsub, bg, t_rank;
  if ((nbg & 7) == 0) {
    // XCD x owns KV groups x, x+8, ...; it finishes one group (all its query tiles and
    // head groups, longest first) before the next, so one group's K/V (Lk*d*4 bytes)
    // is the L2 working set.
    const int x = bid & 7;
    const int s = bid >> 3;
    const int per_group = a.n_qtiles * GH;
    bg = (s / per_group) * 8 + x;
    const int rem = s % per_group;
    t_rank = rem / GH;
    hsub = rem % GH;
  } else {
    hsub = bid % GH;
    const int s = bid / GH;
    bg = s % nbg;
    t_rank = s / nbg;
  }
  WorkItem it;
  const int t = CAUSAL ? a.n_qtiles - 1 - t_rank : t_rank;
  it.b = bg / a.Hkv;
  it.hq0 = (bg % a.Hkv) * a.G + hsub * K::kHPW;
  it.pos0 = t * K::BMP;
  it.Lq = a.Lq;
  it.Lk = a.Lk;
  it.shift = a.causal_shift;
  it.qtok0 = 0;
  it.ktok0 = 0;
  it.split = split;
  // packed rows hold positions anywhere in [0, Lq): tiles up to the last position's reach
  const int end = K::tile_end(K::kPack ? it.Lq - K::BMP : it.pos0, it.Lk, it.shift);
  if (split >= 0) {
    it.kt_lo = split * a.tiles_per_split;
    const int hi = it.kt_lo + a.tiles_per_split;
    it.kt_hi = hi < end ? hi : end;
  } else {
    it.kt_lo = 0;
    it.kt_hi = end;
  }
  return it;
}

// Work distribution shared by the kernel shapes: a persistent loop over the device-built
// schedule (varlen), or one work item per work group (dense, split). run_item(it) runs one
// work item with the kernel's LDS buffers.
// The fused cache update's copy: the grid's threads share the chunk's K and V rows (16-byte
// units), each written to the ring slot of its token (sink prefix, then the window). Index
// arithmetic in 32 bits (the host bounds rows * units below 2^31); a row's slot is
// rm_sink + (upd_off + row) folded once into the window, or the token itself in the sink.
template <class K>
__device__ __forceinline__ void kv_fused_update(const FwdArgs& a) {
  typedef typename K::elem_t T;
  constexpr int KU = K::kDQK / 8, VU = K::kDV / 8;   // 16-byte units per row
  const int rows = a.B * a.Hkv * a.upd_chunk;
  const int nk = rows * KU, n = nk + rows * VU;
  const int nthr = gridDim.x * gridDim.y * blockDim.x;
  for (int u = (blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; u < n; u += nthr) {
    const bool isv = u >= nk;
    const int x = isv ? u - nk : u;
    const int piece = isv ? x % VU : x % KU;
    const int rr = isv ? x / VU : x / KU;       // (b, h, row) flattened
    const int row = rr % a.upd_chunk;
    const int bh = rr / a.upd_chunk;
    const int h = bh % a.Hkv, b = bh / a.Hkv;
    int64_t slot;
    if (a.upd_tok0 + row < a.rm_sink) {
      slot = a.upd_tok0 + row;
    } else {
      int xo = a.upd_off + row;
      xo = xo >= a.rm_window ? xo - a.rm_window : xo;
      slot = a.rm_sink + xo;
    }
    const T* src = isv ? (const T*)a.vnew + b * a.vn_sb + h * a.vn_sh + row * a.vn_sm
                       : (const T*)a.knew + b * a.kn_sb + h * a.kn_sh + row * a.kn_sm;
    T* dst = isv ? (T*)a.v + b * a.v_sb + h * a.v_sh + slot * a.v_sm
                 : (T*)a.k + b * a.k_sb + h * a.k_sh + slot * a.k_sm;
    *reinterpret_cast<u32x4*>(dst + 8 * piece) = *reinterpret_cast<const u32x4*>(src + 8 * piece);
  }
}

template <class K, int MODE, bool CAUSAL, class RunItem>
__device__ __forceinline__ void attn_dispatch(const FwdArgs& a, const RunItem& run_item) {
  if constexpr (MODE == MODE_VARLEN) {
    __shared__ int s_item;
    const int NHG = a.Hq / K::kHPW;        // head groups per (sequence, query tile) item
    // With xcd_parts, work group p (on XCD p % 8: the hardware deals work groups to the XCDs
    // round-robin) takes only the head groups of KV heads g = p % 8 (mod 8), from that XCD's
    // own counter over the same longest-first list: a sequence's K/V for one KV head is then
    // read into one XCD's L2 instead of into all eight.
    const int part = a.xcd_parts ? (int)(blockIdx.x & 7) : 0;
    int* const ctr = a.xcd_parts ? a.counter + 16 + 4 * part : a.counter;
    const int per_kv = a.G / K::kHPW;      // head groups per KV head
    const int nhg = a.xcd_parts ? NHG / 8 : NHG;
    const int n_work = *a.n_items * nhg;
    for (;;) {
      if (threadIdx.x == 0) s_item = atomicAdd(ctr, 1);
      __syncthreads();
      const int idx = s_item;
      if (idx >= n_work) break;
      const int2 pr = a.items[idx / nhg];
      int hg = idx % nhg;
      if (a.xcd_parts) hg = (part + 8 * (hg / per_kv)) * per_kv + hg % per_kv;
      WorkItem it;
      it.b = pr.x;
      it.hq0 = hg * K::kHPW;
      it.pos0 = pr.y * K::BMP;
      const int cq0 = a.cu_q[it.b], ck0 = a.cu_k[it.b];
      it.Lq = a.cu_q[it.b + 1] - cq0;
      it.Lk = a.cu_k[it.b + 1] - ck0;
      it.qtok0 = cq0;
      it.ktok0 = a.kv_padded ? 0 : ck0;
      it.shift = CAUSAL ? it.Lk - it.Lq : 0;
      it.split = -1;
      it.kt_lo = 0;
      it.kt_hi = K::tile_end(it.pos0, it.Lk, it.shift);
      run_item(it);
      __syncthreads();
    }
  } else if constexpr (MODE == MODE_SPLIT || MODE == MODE_SPLITP || MODE == MODE_SPLITU) {
    if constexpr (MODE == MODE_SPLITU) kv_fused_update<K>(a);
    const WorkItem it = decode_grid<K, CAUSAL>(a, blockIdx.x, blockIdx.y);
    run_item(it);
  } else {
    const WorkItem it = decode_grid<K, CAUSAL>(a, blockIdx.x, -1);
    run_item(it);
  }
}

template <typename T, int DQK, int DQK1, int DV, int NW, int HPW, int MASK, bool CAUSAL, int MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdArgs a) {
  typedef AttnFwd<T, DQK, DQK1, DV, NW, HPW, MASK, CAUSAL, MODE> K;
  __shared__ __attribute__((aligned(K::KALIGN))) char sK0[K::KBYTES];
  __shared__ __attribute__((aligned(K::KALIGN))) char sK1[K::KBYTES];
  __shared__ __attribute__((aligned(K::KALIGN))) char sV0[K::VBYTES];
  __shared__ __attribute__((aligned(K::KALIGN))) char sV1[K::VBYTES];
  __shared__ __attribute__((aligned(1024))) char sM0[K::MBYTES];
  __shared__ __attribute__((aligned(1024))) char sM1[K::MBYTES];
  attn_dispatch<K, MODE, CAUSAL>(a, [&](const WorkItem& it) {
    K::run(a, it, (WF_LDS char*)sK0, (WF_LDS char*)sK1, (WF_LDS char*)sV0, (WF_LDS char*)sV1,
           (WF_LDS char*)sM0, (WF_LDS char*)sM1);
  });
}

}  // namespace wf
