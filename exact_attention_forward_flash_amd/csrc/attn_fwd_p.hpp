// Persistent form of the 32-query-wave attention kernel (attn_fwd.hpp) for dense calls
// without a mask: one work group per CU walks a fixed list of work items, and the key-tile
// pipeline runs on across item boundaries.
//
// Same arithmetic as attn_fwd.hpp (S^T = K Q^T, online softmax in the log2 domain with a
// lazy reference max, O^T += V^T P^T). What changes is what happens between work items:
// with one work group per CU, a work group that loads its Q, fills its first tiles and stores
// its output before and after its key loop leaves the CU idle for those phases (measured:
// about a sixth of a causal launch). Here the tiles of a group's items form one sequence:
//   * the K and V copies run two and one tiles ahead of the compute through that sequence,
//     so the first tiles of the next item are copied during the last tiles of this one;
//   * Q of the next item is loaded into registers one item ahead; in the last iteration of
//     an item the S^T of the next item's first tile is computed with it (that tile's
//     scores and max are ready when the item starts);
//   * an item's output is normalised and stored after the last iteration's barrier, and
//     those stores complete during the next iteration.
//
// Items (batch, KV head, HPW query heads, BMP query positions) are those of the one-item-
// per-group launch. Work group p of P (P a multiple of 8) takes the items of its XCD (the
// hardware deals work groups to the 8 XCDs round-robin by index and decode_grid keeps each
// KV group on one XCD) in rounds over the XCD's P/8 groups, alternating direction each round,
// which pairs long and short causal items on every CU.
//
// ROPE instantiations turn Q by a rotary table as it is read into registers (once per item):
// rotate-half over the whole head (1) or interleaved over the first rq_rot dims (2), so that
// such calls need a separate pass over K only.
//
// Every wave of a group must compute the same tiles, so for causal calls the group covers
// one 64-key tile's worth of positions (BMP == BN, HPW = 4 with 8 waves) and the causal
// alignment shift is 0; the host routes other calls to the one-item-per-group kernels.
#pragma once
#include "attn_fwd.hpp"

namespace wf {

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <typename T, int DQK, int DV, int HPW, bool CAUSAL, bool SUM16, int ROPE = 0>
struct AttnFwdP {
  static constexpr int NW = 8;
  static constexpr int BN = 64;
  static constexpr int kNW = NW;
  static constexpr int kHPW = HPW;
  static constexpr bool kPack = false;  // rows are packed (head, position) pairs
  static constexpr int KCH = DQK / 8;
  static constexpr int VCH = DV / 8;
  static constexpr int WPH = NW / HPW;
  static constexpr int BMP = WPH * 32;
  static constexpr int NT = NW * 64;
  static constexpr int KLOADS = BN * KCH / NT;
  static constexpr int VLOADS = BN * VCH / NT;
  static constexpr int KBYTES = BN * DQK * 2;
  static constexpr int VBYTES = BN * DV * 2;
  static constexpr int NS = DQK / 16;
  static constexpr int NDV = DV / 32;
  static constexpr int QBYTES = 32 * DQK * 2;   // staged Q rows of one wave
  static constexpr int QLOADS = 32 * KCH / 64;
  static_assert(sizeof(T) == 2, "16-bit inputs only");
  static_assert(NW % HPW == 0, "waves split evenly over heads");
  static_assert(KLOADS >= 1 && VLOADS >= 1 && (BN * KCH) % NT == 0 && (BN * VCH) % NT == 0,
                "tile copies split evenly");
  static_assert(!CAUSAL || BMP == BN, "causal: every wave of a group on the same key tiles");

  static __device__ __forceinline__ int kswz(int row) { return lds_kswz<KCH>(row); }
  static __device__ __forceinline__ int vswz(int row) { return lds_vswz<VCH>(row); }

  static __device__ __forceinline__ int tile_end(int pos0, int Lk, int shift) {
    const int n_kt = (Lk + BN - 1) / BN;
    if (!CAUSAL) return n_kt;
    const int lim = pos0 + BMP - 1 + shift;
    if (lim < 0) return 0;
    const int e = lim / BN + 1;
    return e < n_kt ? e : n_kt;
  }

  // Block index (in the one-item-per-group numbering of decode_grid) of the k-th item of
  // work group p of P, or -1 past the end of its list.
  static __device__ __forceinline__ int item_bid(const FwdArgs& a, int p, int P, int k) {
    const int nbg = a.B * a.Hkv;
    const int N = a.n_qtiles * (a.G / HPW) * nbg;
    if ((nbg & 7) == 0 && (P & 7) == 0) {
      const int Px = P >> 3, c = p >> 3;
      const int s = k * Px + ((k & 1) ? Px - 1 - c : c);
      return s < (N >> 3) ? s * 8 + (p & 7) : -1;
    }
    const int v = k * P + ((k & 1) ? P - 1 - p : p);
    return v < N ? v : -1;
  }

  // What the loop keeps of an item: batch, first query head, first query position and
  // key-tile count (0: past the end of the group's list).
  struct Item {
    int k, b, hq0, pos0, n;
  };
  // Items per work group the LDS list holds; the host sends larger problems to the
  // one-item-per-group kernel.
  static constexpr int MAX_ITEMS = 1024;

  // Decodes the group's items into LDS once (one thread per item), so that the loop reads
  // an item's fields instead of redoing the index arithmetic at every item boundary.
  static __device__ __forceinline__ void build_items(const FwdArgs& a, int p, int P, WF_LDS i32x4* list) {
    for (int k = threadIdx.x; k < MAX_ITEMS; k += NT) {
      const int bid = item_bid(a, p, P, k);
      i32x4 v = {0, 0, 0, 0};
      if (bid >= 0) {
        const WorkItem it = decode_grid<AttnFwdP, CAUSAL>(a, bid, -1);
        v = i32x4{it.b, it.hq0, it.pos0, it.kt_hi - it.kt_lo};
      }
      list[k] = v;
    }
  }
  static __device__ __forceinline__ Item item_at(const WF_LDS i32x4* list, int k) {
    Item r;
    r.k = k;
    const i32x4 v = list[k < MAX_ITEMS ? k : MAX_ITEMS - 1];
    const bool in = k < MAX_ITEMS;
    r.b = __builtin_amdgcn_readfirstlane(v[0]);
    r.hq0 = __builtin_amdgcn_readfirstlane(v[1]);
    r.pos0 = __builtin_amdgcn_readfirstlane(v[2]);
    r.n = in ? __builtin_amdgcn_readfirstlane(v[3]) : 0;
    return r;
  }

  static __device__ __forceinline__ void run(const FwdArgs& a, WF_LDS char* sK0, WF_LDS char* sK1,
                                             WF_LDS char* sV0, WF_LDS char* sV1, WF_LDS char* sQ,
                                             WF_LDS i32x4* list) {
    build_items(a, blockIdx.x, gridDim.x, list);
    __syncthreads();
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, hf = lane >> 5;
    const int hw = w / WPH;
    const int qw = (w % WPH) * 32;
    const float c = a.scale_log2;
    // PRESCALE (calls without the lse): Q carries c (see read_q) and scores come out in log2
    // units; otherwise they stay in raw units and the weight is exp2(c * (t - m_ref / c)).
    constexpr bool PRESCALE = SUM16;
    const float cs = PRESCALE ? 1.0f : c, inv_cs = PRESCALE ? 1.0f : 1.0f / c;

    // ---- copies into LDS: buffer loads with a descriptor whose size ends at the first row
    // that must not be read (those rows land as zeros) and a per-lane byte offset that is
    // the same for every tile. Lane -> chunk q of the copy, row q/CH, swizzled position q%CH,
    // which holds logical chunk (q%CH) ^ swizzle(row).
    //   K / V tiles: copy i of wave w fills chunks [(i*NW + w)*64, +64) of the tile; rows
    //     past key Lk are zero (their scores are masked to -inf, their V rows meet p = 0).
    //   Q: each wave stages its own 32 query rows (copy i fills chunks [64i, +64) of the
    //     wave's area) for the next item; rows past Lq are zero and never stored.
    auto rsrc = [](const void* base, int64_t bytes) {
      const uint32_t nrec = bytes <= 0 ? 0u : bytes >= 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
      return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)nrec, 0x00020000);
    };
    // The swizzles repeat every KPER rows (K, Q) / 4 rows (V), so copies that start a
    // multiple of that many rows apart share the per-lane offset; each gets a descriptor of
    // its own whose base is moved by those rows (and whose size shrinks with it: the range
    // check covers only the per-lane offset).
    constexpr int KPER = KCH == 16 ? 16 : 32;
    constexpr int KROWS = NT / KCH, VROWS = NT / VCH, QROWS = 64 / KCH;  // rows per copy
    constexpr int QV = KPER / QROWS < QLOADS ? KPER / QROWS : QLOADS;   // distinct Q offsets
    static_assert(KLOADS == 1 || KROWS % KPER == 0, "K copies share their offsets");
    static_assert(VLOADS == 1 || VROWS % 4 == 0, "V copies share their offsets");
    static_assert(QLOADS % QV == 0 && (QROWS * QV) % KPER == 0, "Q copies share their offsets");
    const uint32_t ksm2 = (uint32_t)(a.k_sm * 2), vsm2 = (uint32_t)(a.v_sm * 2), qsm2 = (uint32_t)(a.q_sm * 2);
    uint32_t kvo, vvo, qvo[QV];
    {
      const int q = w * 64 + lane;
      kvo = (uint32_t)(q / KCH) * ksm2 + (uint32_t)(((q % KCH) ^ kswz(q / KCH)) * 16);
      vvo = (uint32_t)(q / VCH) * vsm2 + (uint32_t)(((q % VCH) ^ vswz(q / VCH)) * 16);
    }
#pragma unroll
    for (int i = 0; i < QV; ++i) {
      const int q = i * 64 + lane;
      const int r = q / KCH, pos = q % KCH;
      qvo[i] = (uint32_t)r * qsm2 + (uint32_t)((pos ^ kswz(r)) * 16);
    }
    WF_LDS char* const sQw = sQ + w * QBYTES;
    auto stage_q = [&](const Item& it) {
      const int row0 = it.pos0 + qw;
      const T* base = (const T*)a.q + it.b * a.q_sb + (it.hq0 + hw) * a.q_sh + (int64_t)row0 * a.q_sm;
      const int64_t bytes = it.n > 0 ? (int64_t)(a.Lq - row0) * a.q_sm * 2 : 0;
#pragma unroll
      for (int i = 0; i < QLOADS; ++i) {
        const int64_t off = (int64_t)(i / QV) * QV * QROWS * qsm2;
        const auto rs = rsrc((const char*)base + off, bytes - off);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (WF_LDS void*)(sQw + i * 1024), 16, (int)qvo[i % QV], 0, 0, 0);
      }
    };
    // Q^T operand from the staging area: lane (j, hf) takes row j, head-dim 16s + 8hf .. +7.
    // With PRESCALE it is multiplied by c = scale*log2(e) in fp32 and rounded back to the
    // input type, so that the S^T MFMAs produce log2-domain scores and the weights need no
    // per-element scaling. That rounding (relative 2^-9 per element for bf16) does not
    // average out: for a fixed c it shifts all scores of a row by a common factor of order
    // 1e-4, which moves the log-sum-exp by a few 1e-4 (measured on N(0,1) inputs: output
    // error up to ~1e-3, as large as the output's own rounding). Calls that ask for the lse
    // therefore keep Q as it is and scale every score in fp32.
    //
    // ROPE (1: rotate-half over all DQK dims, 2: interleaved over the first rq_rot dims): Q is
    // turned first, in fp32, and rounded once. Both members of every pair sit in the lane's
    // own registers (rotate-half: chunk s pairs with chunk s + NS/2; interleaved: adjacent
    // elements of a chunk, and rq_rot % 16 == 0 turns whole chunks for both half-waves). The table rows are read from global memory (they stay in L2: one row per
    // query position, shared by every head and batch).
    u32x4 qf[NS];
    auto read_q = [&](const Item& it) {
      typedef typename Mfma16<T>::v8 v8;
      auto chunk = [&](int s) {
        return __builtin_bit_cast(v8, lds_read16(sQw + j * KCH * 16 + (((2 * s + hf) ^ kswz(j)) * 16)));
      };
      auto put = [&](int s, const float* y) {
        v8 r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (T)(PRESCALE ? y[e] * c : y[e]);
        qf[s] = __builtin_bit_cast(u32x4, r);
      };
      if constexpr (!ROPE) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const v8 x = chunk(s);
          v8 y;
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = PRESCALE ? (T)((float)x[e] * c) : x[e];
          qf[s] = __builtin_bit_cast(u32x4, y);
        }
      } else if constexpr (ROPE == 1) {   // rotate-half over all DQK dims: chunk s pairs with s + NS/2
        int p = it.pos0 + qw + j;
        p = p < a.Lq ? p : a.Lq - 1;   // rows past Lq are not stored; keep their reads in the table
        const float* cr = a.rq_cos + (int64_t)p * (DQK / 2);
        const float* sr = a.rq_sin + (int64_t)p * (DQK / 2);
#pragma unroll
        for (int s = 0; s < NS / 2; ++s) {
          const int i0 = 16 * s + 8 * hf;
          const f32x4 c0 = *(const f32x4*)(cr + i0), c1 = *(const f32x4*)(cr + i0 + 4);
          const f32x4 n0 = *(const f32x4*)(sr + i0), n1 = *(const f32x4*)(sr + i0 + 4);
          const v8 xa = chunk(s), xb = chunk(s + NS / 2);
          float ya[8], yb[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float cv = e < 4 ? c0[e] : c1[e - 4], sv = e < 4 ? n0[e] : n1[e - 4];
            const float fa = (float)xa[e], fb = (float)xb[e];
            ya[e] = fmaf(fa, cv, -fb * sv);
            yb[e] = fmaf(fb, cv, fa * sv);
          }
          put(s, ya);
          put(s + NS / 2, yb);
        }
      } else {   // interleaved over the first rq_rot dims: pairs (2i, 2i + 1) inside a chunk
        const int half = a.rq_rot >> 1, nrs = a.rq_rot >> 4;   // chunks s < nrs turn
        int p = it.pos0 + qw + j;
        p = p < a.Lq ? p : a.Lq - 1;
        const float* cr = a.rq_cos + (int64_t)p * half;
        const float* sr = a.rq_sin + (int64_t)p * half;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const v8 x = chunk(s);
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = (float)x[e];
          if (s < nrs) {
            const int i0 = 8 * s + 4 * hf;
            const f32x4 c4 = *(const f32x4*)(cr + i0), s4 = *(const f32x4*)(sr + i0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float fa = y[2 * i], fb = y[2 * i + 1];
              y[2 * i] = fmaf(fa, c4[i], -fb * s4[i]);
              y[2 * i + 1] = fmaf(fb, c4[i], fa * s4[i]);
            }
          }
          put(s, y);
        }
      }
    };

    // A copy cursor walks the tiles of the group's items for one tensor: the item, the tile
    // within it, the tile's address and the bytes left before key Lk.
    struct Cursor {
      int k, t, n;
      const char* base;
      int rows;   // rows of the tensor left from the tile's first row (key Lk - 64t)
    };
    const int64_t kstep = (int64_t)BN * a.k_sm * 2, vstep = (int64_t)BN * a.v_sm * 2;
    auto enter = [&](Cursor& cu, int k, bool is_v) {
      const Item it = item_at(list, k);
      cu.k = k;
      cu.t = 0;
      if (it.n == 0) {   // past the end: empty descriptors from now on
        cu.n = 0x7fffffff;
        cu.rows = 0;
        cu.base = (const char*)a.k;
        return;
      }
      cu.n = it.n;
      const int g = it.hq0 / a.G;
      cu.base = is_v ? (const char*)((const T*)a.v + it.b * a.v_sb + g * a.v_sh)
                     : (const char*)((const T*)a.k + it.b * a.k_sb + g * a.k_sh);
      cu.rows = a.Lk;
    };
    auto advance = [&](Cursor& cu, bool is_v) {
      if (++cu.t >= cu.n) {
        enter(cu, cu.k + 1, is_v);
      } else {
        cu.base += is_v ? vstep : kstep;
        cu.rows -= BN;
      }
    };
    Cursor ck, cv;  // the K copy runs two tiles ahead of the compute, the V copy one
    // Copy i of the tile the cursor points at: rows [i*ROWS, (i+1)*ROWS) of the tile, with a
    // descriptor that ends after the rows the tensor still has (32-bit arithmetic: a tile
    // spans less than 2 GiB).
    auto issue_one = [&](const Cursor& cu, bool is_v, WF_LDS char* dst, int i) {
      const int rows_per = is_v ? VROWS : KROWS;
      const uint32_t sm2 = is_v ? vsm2 : ksm2;
      int r = cu.rows - i * rows_per;
      // The clamp becomes a vector med3; read it back into a scalar register, or the
      // descriptor lands in vector registers and the load is wrapped in a per-lane loop.
      r = __builtin_amdgcn_readfirstlane(r < 0 ? 0 : r > rows_per ? rows_per : r);
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(cu.base + (int64_t)i * rows_per * sm2), 0, (int)((uint32_t)r * sm2), 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (WF_LDS void*)(dst + (i * NW + w) * 1024), 16,
                                               (int)(is_v ? vvo : kvo), 0, 0, 0);
    };
    auto issue = [&](const Cursor& cu, bool is_v, WF_LDS char* dst) {
#pragma unroll
      for (int i = 0; i < (is_v ? VLOADS : KLOADS); ++i) issue_one(cu, is_v, dst, i);
    };

    // ---- LDS operand offsets (as in attn_fwd.hpp) ----
    int koff[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = j * KCH * 16 + (((2 * s + hf) ^ kswz(j)) * 16);
    const int g16 = (lane >> 4) & 1, b2 = (lane & 3) >> 1;
    const int vrow0 = 4 * hf + ((lane & 15) >> 2);
    const int fv = vswz(vrow0);
    int voff[NDV];
#pragma unroll
    for (int n = 0; n < NDV; ++n)
      voff[n] = vrow0 * VCH * 16 + (((4 * n + 2 * g16 + b2) ^ fv) * 16) + 8 * (lane & 1);
    auto kfrag = [&](const WF_LDS char* Kt, int s, int kb) {
      return lds_read16(Kt + koff[s] + kb * 32 * KCH * 16);
    };
    auto vfrag = [&](const WF_LDS char* Vt, int m, int n) {
      const WF_LDS char* base = Vt + voff[n] + 16 * m * VCH * 16;
      const u32x2 lo = lds_read_tr(base);
      const u32x2 hi = lds_read_tr(base + 8 * VCH * 16);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // ---- masking of tile kt of an item whose queries start at pos0: keys past Lk and,
    // for causal calls, keys after the query. Element r of block kb is key
    // k0 + 32kb + 8(r/4) + 4hf + r%4. ----
    auto need_mask = [&](int kt, int pos0) {
      const int k0 = kt * BN;
      return (k0 + BN > a.Lk) || (CAUSAL && k0 + BN - 1 > pos0 + qw);
    };
    auto apply_mask = [&](int kt, int pos0, f32x16* sc) {
      const int k0 = kt * BN;
      const int qrow = pos0 + qw + j;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          bool ok = key < a.Lk;
          if (CAUSAL) ok = ok && key <= qrow;
          sc[kb][r] = ok ? sc[kb][r] : -INFINITY;
        }
    };

    f32x16 oacc[NDV];
#pragma unroll
    for (int n = 0; n < NDV; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[n][r] = 0.f;
    // Softmax state (per lane: its query row), in log2 units. m_run is the reference max
    // (-inf before the item's first tile), l_run the sum of the weights. The S^T accumulators
    // start from -m_ref (over c without PRESCALE) instead of 0, so a tile comes out relative
    // to m_ref and its weights need no subtraction; m_ref is the reference the pending tile
    // was computed against (m_run, or 0 while m_run is -inf). The start value is rebuilt for
    // every tile (16 moves) rather than kept in 16 registers.
    float m_run = -INFINITY, l_run = 0.f, m_ref = 0.f;
    auto acc_start = [&]() {
      float v = -m_ref * inv_cs;
      asm volatile("" : "+v"(v));  // not hoisted out of the loop
      f32x16 r16;
#pragma unroll
      for (int r = 0; r < 16; ++r) r16[r] = v;
      return r16;
    };

    auto s_tile = [&](const WF_LDS char* Kt, f32x16* sc) {
      const f32x16 mref16 = acc_start();
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 k0f = kfrag(Kt, s, 0), k1f = kfrag(Kt, s, 1);
        sc[0] = Mfma16<T>::run(k0f, qf[s], s == 0 ? mref16 : sc[0]);
        sc[1] = Mfma16<T>::run(k1f, qf[s], s == 0 ? mref16 : sc[1]);
      }
    };
    auto tile_max = [&](const f32x16* sc) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      return xhalf_max(mx) * cs;
    };
    // mt: max of the current tile relative to m_ref. The reference max moves (O and l
    // rescaled, the tile shifted onto the new reference) only when some query's tile max
    // passes it by more than 8, so p = exp2(t - m) stays <= 2^8.
    auto rescale = [&](float mt, f32x16* cur) {
      const float m_abs = m_ref + mt;
      if (wave_any(m_abs > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, m_abs);
        const float m_new_ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_new_ref);
        l_run *= alpha;
#pragma unroll
        for (int n = 0; n < NDV; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[n][r] *= alpha;
        const float d = m_new_ref - m_ref;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) cur[kb][r] -= d * inv_cs;
        m_run = m_new;
        m_ref = m_new_ref;
      }
    };

    f32x16 sc[2], sn[2];
    u32x4 pk[4];
    u32x4 vq[NDV];   // V^T operands of the next PV step
    float mt_cur = -INFINITY;

    // Phase A: the next tile's S^T MFMAs with the current tile's exponentials between them.
    // K operands run two steps ahead; near the end the V^T operands of the first PV step
    // are read (the V tile landed in the previous iteration).
    // A wave in this phase issues ahead of one in phase B (s_setprio): measured to keep the
    // MFMA pipe busier than equal priorities.
    auto phase_a = [&](const WF_LDS char* Kn, const WF_LDS char* Vc, f32x16* cur, f32x16* nxt,
                       WF_LDS char* Kfill) {
      __builtin_amdgcn_s_setprio(3);
      constexpr int EPS = 32 / NS;  // exponentials per step
      const f32x16 mref16 = acc_start();
      u32x4 kp[2][2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        kp[s][0] = kfrag(Kn, s, 0);
        kp[s][1] = kfrag(Kn, s, 1);
      }
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 a0 = kp[s & 1][0], a1 = kp[s & 1][1];
        if (s + 2 < NS) {
          kp[s & 1][0] = kfrag(Kn, s + 2, 0);
          kp[s & 1][1] = kfrag(Kn, s + 2, 1);
        }
        nxt[0] = Mfma16<T>::run(a0, qf[s], s == 0 ? mref16 : nxt[0]);
#pragma unroll
        for (int e = s * EPS; e < s * EPS + EPS / 2; ++e) {
          const float pe = fast_exp2(PRESCALE ? cur[e >> 4][e & 15] : cur[e >> 4][e & 15] * cs);
          cur[e >> 4][e & 15] = pe;
          if (!SUM16) ps[0] += pe;
        }
        nxt[1] = Mfma16<T>::run(a1, qf[s], s == 0 ? mref16 : nxt[1]);
#pragma unroll
        for (int e = s * EPS + EPS / 2; e < (s + 1) * EPS; ++e) {
          const float pe = fast_exp2(PRESCALE ? cur[e >> 4][e & 15] : cur[e >> 4][e & 15] * cs);
          cur[e >> 4][e & 15] = pe;
          if (!SUM16) ps[1] += pe;
        }
        if (s == NS - 2) {
#pragma unroll
          for (int n = 0; n < NDV; ++n) vq[n] = vfrag(Vc, 0, n);
        }
#pragma unroll
        for (int i = 0; i < KLOADS; ++i)
          if (s == (2 * i + 1) * NS / (2 * KLOADS)) issue_one(ck, false, Kfill, i);
      }
      if (!SUM16) l_run += ps[0] + ps[1];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        pk[m] = pack8<T>(cur[m >> 1], 8 * (m & 1));
        // keeps the exponentials here, among the S^T MFMAs, rather than sunk to their uses
        asm volatile("" ::"v"(pk[m]));
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // Phase B: O^T += V^T P^T for the current tile (V^T operands one step ahead), with the
    // next tile's row max in between.
    auto phase_b = [&](const WF_LDS char* Vc, const f32x16* nxt, WF_LDS char* Vfill) {
      float mx[2] = {-INFINITY, -INFINITY};
      float lp[2] = {0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4 va[NDV];
#pragma unroll
        for (int n = 0; n < NDV; ++n) {
          va[n] = vq[n];
          if (m + 1 < 4) vq[n] = vfrag(Vc, m + 1, n);
        }
#pragma unroll
        for (int n = 0; n < NDV; ++n) {
          oacc[n] = Mfma16<T>::run(va[n], pk[m], oacc[n]);
#pragma unroll
          for (int e = 8 * m + 2 * n; e < 8 * m + 2 * n + 2; ++e)
            mx[n & 1] = fmaxf(mx[n & 1], nxt[e >> 4][e & 15]);
        }
        if (SUM16) lp[m & 1] = sum8_acc<T>(pk[m], lp[m & 1]);
#pragma unroll
        for (int i = 0; i < VLOADS; ++i)
          if (m == i * 4 / VLOADS) issue_one(cv, true, Vfill, i);
      }
      if (SUM16) {
        // 3 wait states between the last v_dot2c write and an ordinary VALU read of it.
        asm volatile("s_nop 2" : "+v"(lp[0]), "+v"(lp[1]));
        l_run += lp[0] + lp[1];
      }
      mt_cur = xhalf_max(fmaxf(mx[0], mx[1])) * cs;
    };

    // Output of an item: O / l, rows past Lq dropped; the log-sum-exp when asked for.
    auto store_item = [&](const Item& it) {
      const float l = xhalf_sum(l_run);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const int hq = it.hq0 + hw;
      const int qrow = it.pos0 + qw + j;
      if (qrow < a.Lq) {
        T* dst = (T*)a.o + it.b * a.o_sb + hq * a.o_sh + (int64_t)qrow * a.o_sm;
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
        if (a.lse != nullptr && hf == 0) {
          const float lse2 = l > 0.f ? (m_run == -INFINITY ? 0.f : m_run) + __builtin_log2f(l) : -INFINITY;
          a.lse[((int64_t)it.b * a.Hq + hq) * a.Lq + qrow] = lse2 * kLn2;
        }
      }
    };

    // ---- start: the first item's Q and first tiles; then the second item's Q is staged ----
    Item cur_it = item_at(list, 0);
    if (cur_it.n == 0) return;
    Item nxt_it = item_at(list, 1);
    stage_q(cur_it);
    enter(ck, 0, false);
    enter(cv, 0, true);
    issue(ck, false, sK0);
    advance(ck, false);
    issue(cv, true, sV0);
    advance(cv, true);
    issue(ck, false, sK1);
    advance(ck, false);
    wait_vmem();
    __syncthreads();
    read_q(cur_it);
    s_tile(sK0, sc);
    if (need_mask(0, cur_it.pos0)) apply_mask(0, cur_it.pos0, sc);
    mt_cur = tile_max(sc);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // Q reads done before the area refills
    stage_q(nxt_it);
    __syncthreads();  // K_0's buffer is refilled by the first iteration

    // ---- tile loop over the group's items ----
    // Global tile g (counted over all items) has K in buffer g%2 and V in buffer g%2.
    // Iteration g reads K_{g+1} (S^T of the next tile) and V_g, and copies K_{g+2} and
    // V_{g+1} meanwhile. u is the current tile's index within its item. In an item's last
    // iteration the next tile is the next item's first: its Q^T is read from the staging
    // area (filled during the item), and the item after it is staged.
    int u = 0;
    bool done = false;
    auto iter = [&](const WF_LDS char* Kn, WF_LDS char* Kfill, const WF_LDS char* Vc,
                    WF_LDS char* Vfill, f32x16* cur, f32x16* nxt) {
      const bool last = u + 1 == cur_it.n;
      if (last) {
        read_q(nxt_it);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        stage_q(item_at(list, cur_it.k + 2));
      }
      rescale(mt_cur, cur);
      phase_a(Kn, Vc, cur, nxt, Kfill);   // copies K_{g+2} into Kfill on the way
      const int kt_n = last ? 0 : u + 1;
      const int pos_n = last ? nxt_it.pos0 : cur_it.pos0;
      if (need_mask(kt_n, pos_n)) apply_mask(kt_n, pos_n, nxt);
      phase_b(Vc, nxt, Vfill);            // copies V_{g+1} into Vfill on the way
      advance(ck, false);
      advance(cv, true);
      wait_vmem();
      __syncthreads();
      if (last) {
        store_item(cur_it);
#pragma unroll
        for (int n = 0; n < NDV; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[n][r] = 0.f;
        m_run = -INFINITY;   // m_ref stays: the next item's first tile was computed against it
        l_run = 0.f;
        cur_it = nxt_it;
        nxt_it = item_at(list, cur_it.k + 1);
        u = 0;
        done = cur_it.n == 0;
      } else {
        ++u;
      }
    };
    for (;;) {
      iter(sK1, sK0, sV0, sV1, sc, sn);  // even tiles: scores in sc, next in sn
      if (done) break;
      iter(sK0, sK1, sV1, sV0, sn, sc);  // odd tiles: roles swapped
      if (done) break;
    }
    wait_vmem();  // the last copies (empty) and stores
  }
};

template <typename T, int DQK, int DV, int HPW, bool CAUSAL, bool SUM16, int ROPE = 0>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_p_kernel(FwdArgs a) {
  typedef AttnFwdP<T, DQK, DV, HPW, CAUSAL, SUM16, ROPE> K;
  // Separate LDS arrays, so that the compiler can tell a tile copy into one buffer from the
  // operand reads of another and does not wait for the copy before them. The tile buffers
  // carry the largest alignment, which places them first: every operand read in the tile loop
  // then addresses them as a per-lane offset plus an immediate (< 64 KiB).
  __shared__ __attribute__((aligned(16384))) char sK0[K::KBYTES];
  __shared__ __attribute__((aligned(16384))) char sK1[K::KBYTES];
  __shared__ __attribute__((aligned(16384))) char sV0[K::VBYTES];
  __shared__ __attribute__((aligned(16384))) char sV1[K::VBYTES];
  __shared__ __attribute__((aligned(1024))) char sQ[K::NW * K::QBYTES];
  __shared__ __attribute__((aligned(16))) i32x4 list[K::MAX_ITEMS];
  K::run(a, (WF_LDS char*)sK0, (WF_LDS char*)sK1, (WF_LDS char*)sV0, (WF_LDS char*)sV1,
         (WF_LDS char*)sQ, (WF_LDS i32x4*)list);
}

}  // namespace wf
