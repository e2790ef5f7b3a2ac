// Exact attention forward for gfx950 with 64-query waves (one wave per SIMD), 16-bit inputs.
//
// Same arithmetic as attn_fwd.hpp (S^T = K Q^T, online softmax in the log2 domain with a lazy
// reference max, O^T += V^T P^T), laid out for the register file of a single wave per SIMD:
//
//   * each wave owns 64 queries of one head (two 32-query blocks), so every K / V operand
//     read from LDS feeds two MFMAs: the LDS read traffic per flop is half that of 32-query
//     waves, which on gfx950 is what bounds the narrower shape;
//   * O^T (2 x DV/32 accumulators of 32x32 fp32) and Q^T live in AGPRs, S^T and the P^T
//     operands in VGPRs. The O^T MFMAs are written out with an AGPR accumulator (the
//     compiler would otherwise place every accumulator, S^T included, in AGPRs and copy
//     them back for the softmax); the S^T MFMAs stay compiler builtins in VGPR form.
//   * the row sums of P are taken from the packed 16-bit P^T operands with 2-element dot
//     products against (1, 1), during the O^T MFMAs, so l is the sum of exactly the
//     weights that multiply V.
//
// Hazards of the hand-written MFMA (the compiler does not look inside inline asm):
//   VALU write of an operand -> MFMA read needs 2 wait states: the first MFMA that reads a
//   freshly packed P^T operand starts with s_nop 1 (V^T operands are LDS reads, checked in
//   the generated code to need no VALU moves; a rescale of the accumulators is followed by
//   more than 2 instructions before the next MFMA).
//   MFMA write of the accumulator -> VALU / memory read needs 12 wait states (8-pass
//   32x32x16): reads of O^T (rescale, epilogue) are preceded by 16 wait states issued after
//   all accumulator writes (o_settle, which takes the accumulators as operands so nothing
//   moves across it).
//   v_dot2c (row sums) write -> ordinary VALU read needs 3 wait states: one s_nop 2 that
//   takes the partial sums as operands precedes the adds that read them.
#pragma once
#include "attn_fwd.hpp"

namespace wf {

// NOP: start with s_nop 1 (2 wait states), for an MFMA that may follow a VALU write of one
// of its operands closely.
template <typename T, bool NOP>
__device__ __forceinline__ void mfma_acc_agpr(f32x16& c, u32x4 a, u32x4 b);
template <>
__device__ __forceinline__ void mfma_acc_agpr<__bf16, true>(f32x16& c, u32x4 a, u32x4 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
template <>
__device__ __forceinline__ void mfma_acc_agpr<__bf16, false>(f32x16& c, u32x4 a, u32x4 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
template <>
__device__ __forceinline__ void mfma_acc_agpr<_Float16, true>(f32x16& c, u32x4 a, u32x4 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
template <>
__device__ __forceinline__ void mfma_acc_agpr<_Float16, false>(f32x16& c, u32x4 a, u32x4 b) {
  asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// 16 wait states after the last accumulator write, before any VALU / memory read of them.
__device__ __forceinline__ void o_settle(f32x16 (&o)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]));
}
__device__ __forceinline__ void o_settle(f32x16 (&o)[2][4]) {
  asm volatile("s_nop 7\n\ts_nop 7"
               : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]),
                 "+a"(o[1][1]), "+a"(o[1][2]), "+a"(o[1][3]));
}

template <typename T, int DQK, int DQK1, int DV, int HPW, int MASK, bool CAUSAL, int MODE>
struct AttnFwdW {
  static constexpr int NW = 4;   // one wave per SIMD
  static constexpr int BN = 64;
  static constexpr int kNW = NW;
  static constexpr int kHPW = HPW;
  static constexpr bool kPack = false;  // rows are packed (head, position) pairs
  static constexpr int KCH = DQK / 8;
  static constexpr int VCH = DV / 8;
  static constexpr int WPH = NW / HPW;
  static constexpr int BMP = WPH * 64;
  static constexpr int NT = NW * 64;
  static constexpr int KLOADS = BN * KCH / NT;
  static constexpr int VLOADS = BN * VCH / NT;
  static constexpr int KBYTES = BN * DQK * 2;
  static constexpr int VBYTES = BN * DV * 2;
  static constexpr int NS = DQK / 16;
  static constexpr int NDV = DV / 32;
  static_assert(sizeof(T) == 2, "16-bit inputs only");
  static_assert(NW % HPW == 0, "waves split evenly over heads");
  static_assert((BN * KCH) % NT == 0 && (BN * VCH) % NT == 0, "tile copies split evenly");
  static_assert(KCH % 8 == 0 && VCH % 8 == 0 && DQK1 % 16 == 0 && DV % 32 == 0, "tile shape");
  static_assert(NDV == 2 || NDV == 4, "value width 64 or 128");
  static_assert(64 % NS == 0 || NS == 12, "softmax chunks");

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

  // sK[i] / sV[i]: three K / V tile buffers, distinct LDS arrays (so the compiler can tell
  // the copies into one from the operand reads of another).
  static __device__ __forceinline__ void run(const FwdArgs& a, const WorkItem& it,
                                             WF_LDS char* const (&sK)[3], WF_LDS char* const (&sV)[3]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, hf = lane >> 5;
    const int hw = w / WPH;
    const int qw = (w % WPH) * 64;
    const int hq = it.hq0 + hw;
    const int g = it.hq0 / a.G;
    const float c = a.scale_log2;

    const T* qp = (const T*)a.q + it.b * a.q_sb + hq * a.q_sh + it.qtok0 * a.q_sm;
    const T* q2p = (const T*)a.q2 + it.b * a.q2_sb + hq * a.q2_sh + it.qtok0 * a.q2_sm;
    const T* kp = (const T*)a.k + it.b * a.k_sb + g * a.k_sh + it.ktok0 * a.k_sm;
    const T* k2p = (const T*)a.k2 + it.b * a.k2_sb + g * a.k2_sh + it.ktok0 * a.k2_sm;
    const T* vp = (const T*)a.v + it.b * a.v_sb + g * a.v_sh + it.ktok0 * a.v_sm;

    // ---- Q^T operands (AGPRs): block qb, lane (j, hf): query qlo + 32qb + j, head-dim
    // elements 16s + 8hf .. +7 ----
    const int qlo = it.pos0 + qw;
    int qrow[2], qrow_c[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      qrow[qb] = qlo + 32 * qb + j;
      qrow_c[qb] = qrow[qb] < it.Lq ? qrow[qb] : it.Lq - 1;
    }
    u32x4 qf[2][NS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int col = 16 * s + 8 * hf;
        const T* src = (16 * s < DQK1) ? qp + (int64_t)qrow_c[qb] * a.q_sm + col
                                       : q2p + (int64_t)qrow_c[qb] * a.q2_sm + (col - DQK1);
        qf[qb][s] = *reinterpret_cast<const u32x4*>(src);
        asm volatile("" : "+a"(qf[qb][s]));
      }

    // ---- tile copies (global -> LDS) ----
    // Copy i of wave w fills tile chunks [(i*NW + w)*64, +64): lane -> chunk p, row p/CH,
    // swizzled position p%CH holding logical chunk (p%CH) ^ swizzle(row).
    // With one score tensor (DQK1 == DQK) the copies are buffer loads: a per-tile
    // descriptor (SGPRs) whose size ends at key Lk, and a per-lane byte offset that is the
    // same for every tile. Lanes past the last key read zeros (their scores are masked to
    // -inf, and their V rows meet p = 0). With a split score (MLA: two tensors for the two
    // parts) each lane keeps its own pointer and rows are clamped onto the last key.
    constexpr bool kBuf = DQK1 == DQK;
    uint32_t kvo[KLOADS], vvo[VLOADS];
    const T* ksrc[KLOADS];
    int64_t kstride[KLOADS];
    int krow[KLOADS];
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int p = (i * NW + w) * 64 + lane;
      const int r = p / KCH, pos = p % KCH;
      const int col = (pos ^ kswz(r)) * 8;
      krow[i] = r;
      kvo[i] = (uint32_t)r * (uint32_t)(a.k_sm * 2) + (uint32_t)col * 2;
      if (DQK1 == DQK || col < DQK1) { ksrc[i] = kp + col; kstride[i] = a.k_sm; }
      else { ksrc[i] = k2p + (col - DQK1); kstride[i] = a.k2_sm; }
    }
    const T* vsrc[VLOADS];
    int vrow[VLOADS];
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int p = (i * NW + w) * 64 + lane;
      const int r = p / VCH, pos = p % VCH;
      const int col = (pos ^ vswz(r)) * 8;
      vrow[i] = r;
      vsrc[i] = vp + col;
      vvo[i] = (uint32_t)r * (uint32_t)(a.v_sm * 2) + (uint32_t)col * 2;
    }
    const int lk_last = it.Lk - 1;
    // A copy stream walks the tiles of one tensor: base address of its next tile and the
    // bytes left before the first row it must not read (row min(Lk, kt_hi * BN)), both
    // stepped by one tile per iteration (scalar adds; the descriptor clamps to 32 bits).
    struct Stream { const char* base; int64_t rem, step; };
    const int rows_end = it.Lk < it.kt_hi * BN ? it.Lk : it.kt_hi * BN;
    auto make_stream = [&](const T* head, int64_t sm, int kt) {
      Stream st;
      st.step = (int64_t)BN * sm * 2;
      st.base = (const char*)head + (int64_t)kt * st.step;
      st.rem = (int64_t)(rows_end - kt * BN) * sm * 2;
      return st;
    };
    auto stream_rsrc = [&](const Stream& st) {
      const uint32_t nrec = st.rem <= 0 ? 0u : st.rem >= 0xffffffffLL ? 0xffffffffu : (uint32_t)st.rem;
      return __builtin_amdgcn_make_buffer_rsrc((void*)st.base, 0, (int)nrec, 0x00020000);
    };
    auto stream_next = [&](Stream& st) { st.base += st.step; st.rem -= st.step; };
    auto tile_rsrc = [&](const T* head, int64_t sm, int kt) { return stream_rsrc(make_stream(head, sm, kt)); };
    // One tile copy: K (is_v false) or V copy i of tile kt into Dst. With buffer loads rs is
    // the tile's descriptor.
    auto copy_one = [&](bool is_v, int i, int kt, const __amdgpu_buffer_rsrc_t& rs, WF_LDS char* Dst) {
      if constexpr (kBuf) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (WF_LDS void*)(Dst + (i * NW + w) * 1024), 16,
                                                 (int)(is_v ? vvo[i] : kvo[i]), 0, 0, 0);
      } else {
        int r = kt * BN + (is_v ? vrow[i] : krow[i]);
        r = r < lk_last ? r : lk_last;
        const T* src = is_v ? vsrc[i] + (int64_t)r * a.v_sm : ksrc[i] + (int64_t)r * kstride[i];
        dma16(src, Dst + (i * NW + w) * 1024);
      }
    };
    auto issue_k = [&](int kt, WF_LDS char* Kt) {
      const auto rs = tile_rsrc(kp, a.k_sm, kt);
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) copy_one(false, i, kt, rs, Kt);
    };
    auto issue_v = [&](int kt, WF_LDS char* Vt) {
      const auto rs = tile_rsrc(vp, a.v_sm, kt);
#pragma unroll
      for (int i = 0; i < VLOADS; ++i) copy_one(true, i, kt, rs, Vt);
    };
    // Copies of later tiles spread over the MFMA steps (K in phase A, V in phase B): one at a
    // time keeps the memory pipeline from stalling the wave. They are issued without
    // branches (which would cut the MFMA / softmax interleave): past the last tile a buffer
    // copy gets an empty descriptor (it writes zeros into the free buffer), a pointer copy
    // the last tile.
    struct Pending {
      int kt_k, kt_v;
      WF_LDS char* Kd; WF_LDS char* Vd;
      __amdgpu_buffer_rsrc_t rk, rv;
    };
    auto copy_step = [&](const Pending& pd, bool is_v, int step, int nsteps) {
      constexpr int NK = KLOADS, NV = VLOADS;
      if (!is_v) {
#pragma unroll
        for (int i = 0; i < NK; ++i)
          if (i * nsteps / NK == step) copy_one(false, i, pd.kt_k, pd.rk, pd.Kd);
      } else {
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (i * nsteps / NV == step) copy_one(true, i, pd.kt_v, pd.rv, pd.Vd);
      }
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

    const char* mrow[2] = {nullptr, nullptr};
    if constexpr (MASK != MASK_NONE) {
      constexpr int msz = MASK == MASK_BOOL ? 1 : MASK == MASK_HALF ? 2 : 4;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        mrow[qb] = (const char*)a.mask +
                   (it.b * a.mk_sb + hq * a.mk_sh + (int64_t)qrow_c[qb] * a.mk_sm) * msz;
    }

    f32x16 oacc[2][NDV];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int n = 0; n < NDV; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][n][r] = 0.f;
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    int kt_live = it.kt_hi;
    if (CAUSAL) {
      const int lim = qlo + 63 + it.shift;
      const int e = lim < 0 ? 0 : lim / BN + 1;
      kt_live = e < kt_live ? e : kt_live;
    }
    if (kt_live < it.kt_lo) kt_live = it.kt_lo;

    auto kfrag = [&](const WF_LDS char* Kt, int s, int kb) {
      return lds_read16(Kt + koff[s] + kb * 32 * KCH * 16);
    };
    auto vfrag = [&](const WF_LDS char* Vt, int m, int n) {
      const WF_LDS char* base = Vt + voff[n] + 16 * m * VCH * 16;
      const u32x2 lo = lds_read_tr(base);
      const u32x2 hi = lds_read_tr(base + 8 * VCH * 16);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // Scores: sc[kb][qb] element r = key k0 + 32kb + 8(r/4) + 4hf + r%4, query qrow[qb].
    auto need_mask = [&](int kt) {
      const int k0 = kt * BN;
      return MASK != MASK_NONE || (k0 + BN > it.Lk) || (CAUSAL && k0 + BN - 1 > qlo + it.shift);
    };
    auto apply_mask = [&](int kt, f32x16 (*sc)[2]) {
      const int k0 = kt * BN;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mval[2][4][4];
        if constexpr (MASK != MASK_NONE) {
          const char* mr = mrow[qb];
          const bool vec = a.mask_vec && (k0 + BN <= it.Lk);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int key = k0 + 32 * kb + 8 * q4 + 4 * hf;
              if (vec) {
                if constexpr (MASK == MASK_BOOL) {
                  const uint32_t bits = *reinterpret_cast<const uint32_t*>(mr + key);
#pragma unroll
                  for (int e = 0; e < 4; ++e)
                    mval[kb][q4][e] = ((bits >> (8 * e)) & 0xffu) ? 0.f : -INFINITY;
                } else if constexpr (MASK == MASK_HALF) {
                  typedef T t4 __attribute__((ext_vector_type(4)));
                  const t4 hv = *reinterpret_cast<const t4*>(mr + 2 * key);
#pragma unroll
                  for (int e = 0; e < 4; ++e) mval[kb][q4][e] = (float)hv[e];
                } else {
                  const f32x4 f4 = *reinterpret_cast<const f32x4*>(mr + 4 * key);
#pragma unroll
                  for (int e = 0; e < 4; ++e) mval[kb][q4][e] = f4[e];
                }
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int kk = key + e;
                  float mv = -INFINITY;
                  if (kk < it.Lk) {
                    if constexpr (MASK == MASK_BOOL) mv = mr[kk] ? 0.f : -INFINITY;
                    else if constexpr (MASK == MASK_HALF) mv = (float)reinterpret_cast<const T*>(mr)[kk];
                    else mv = reinterpret_cast<const float*>(mr)[kk];
                  }
                  mval[kb][q4][e] = mv;
                }
              }
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            bool ok = key < it.Lk;
            if (CAUSAL) ok = ok && key <= qrow[qb] + it.shift;
            float v = sc[kb][qb][r];
            if constexpr (MASK == MASK_BOOL) v += mval[kb][r >> 2][r & 3];
            else if constexpr (MASK != MASK_NONE) v += mval[kb][r >> 2][r & 3] * a.inv_scale;
            sc[kb][qb][r] = ok ? v : -INFINITY;
          }
      }
    };

    const f32x16 zero = {};
    auto s_tile = [&](const WF_LDS char* Kt, f32x16 (*sc)[2]) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 k0f = kfrag(Kt, s, 0), k1f = kfrag(Kt, s, 1);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          sc[0][qb] = Mfma16<T>::run(k0f, qf[qb][s], s == 0 ? zero : sc[0][qb]);
          sc[1][qb] = Mfma16<T>::run(k1f, qf[qb][s], s == 0 ? zero : sc[1][qb]);
        }
      }
    };
    float mt_cur[2] = {-INFINITY, -INFINITY};
    auto tile_max = [&](f32x16 (*sc)[2]) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][qb][r]);
        mt_cur[qb] = xhalf_max(mx) * c;
      }
    };
    // Raise a query's reference max (rescaling its O and l) only when its tile max passes
    // it by more than 8, so p = exp2(t - m) stays <= 2^8. The rescaled accumulators are
    // put back into AGPRs inside the branch, so both paths leave them there.
    auto rescale = [&]() {
      const bool need = mt_cur[0] > m_run[0] + 8.0f || mt_cur[1] > m_run[1] + 8.0f;
      if (wave_any(need)) {
        o_settle(oacc);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m_new = fmaxf(m_run[qb], mt_cur[qb]);
          const float alpha = fast_exp2(m_run[qb] - (m_new == -INFINITY ? 0.f : m_new));
          l_run[qb] *= alpha;
#pragma unroll
          for (int n = 0; n < NDV; ++n) {
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][n][r] *= alpha;
            asm volatile("" : "+a"(oacc[qb][n]));
          }
          m_run[qb] = m_new;
        }
      }
    };

    f32x16 sc[2][2], sn[2][2];  // scores of even / odd tiles (current and next alternate)
    u32x4 pk[4][2];             // P^T operands of the current tile, [PV step][query block]
    u32x4 kpre[2][2];           // K operands of the first two S^T steps, read ahead
    u32x4 vpre[2][NDV];         // V^T operands of the first two PV steps, read ahead

    // p = exp2(scale*log2e*s - m) of element e of the current tile (e = 32qb + 16kb + r).
    auto softmax_el = [&](f32x16 (*cur)[2], const float* neg_m, int e) {
      const int qb = e >> 5, kb = (e >> 4) & 1, r = e & 15;
      cur[kb][qb][r] = fast_exp2(fmaf(cur[kb][qb][r], c, neg_m[qb]));
    };
    // Order in which the current tile's elements are exponentiated: the key block kb = 0
    // (P^T operands of PV steps 0, 1) first, for both query blocks, then kb = 1.
    auto el_order = [](int i) { return ((i >> 4) & 1) * 32 + (i >> 5) * 16 + (i & 15); };
    constexpr int N_EXP_A = 48;   // exponentials issued among the S^T MFMAs of phase A

    // Phase A: the next tile's S^T MFMAs with the softmax of key block 0 and half of key
    // block 1 of the current tile in between, and the K copies of a later tile. K operands
    // run two steps ahead (the first two were read during the previous phase B); at the end
    // the first V^T operands of this tile's phase B are read.
    auto phase_a = [&](const WF_LDS char* Kn, const WF_LDS char* Vc, f32x16 (*cur)[2],
                       f32x16 (*nxt)[2], const float* neg_m, const Pending& pd) {
      constexpr int EPS = (N_EXP_A + NS - 1) / NS;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 a0 = kpre[s & 1][0], a1 = kpre[s & 1][1];
        if (s + 2 < NS) {
          kpre[s & 1][0] = kfrag(Kn, s + 2, 0);
          kpre[s & 1][1] = kfrag(Kn, s + 2, 1);
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          nxt[0][qb] = Mfma16<T>::run(a0, qf[qb][s], s == 0 ? zero : nxt[0][qb]);
          nxt[1][qb] = Mfma16<T>::run(a1, qf[qb][s], s == 0 ? zero : nxt[1][qb]);
        }
#pragma unroll
        for (int i = s * EPS; i < (s + 1) * EPS && i < N_EXP_A; ++i) softmax_el(cur, neg_m, el_order(i));
        copy_step(pd, false, s, NS);
        if (s == NS - 2) {
#pragma unroll
          for (int n = 0; n < NDV; ++n) vpre[0][n] = vfrag(Vc, 0, n);
        }
        if (s == NS - 1) {
#pragma unroll
          for (int n = 0; n < NDV; ++n) vpre[1][n] = vfrag(Vc, 1, n);
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          pk[m][qb] = pack8<T>(cur[0][qb], 8 * m);
          // keeps this work here, among the S^T MFMAs, rather than sunk next to its uses
          asm volatile("" ::"v"(pk[m][qb]));
        }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) asm volatile("" ::"v"(cur[1][qb]));
    };

    // Phase B: O^T += V^T P^T for the current tile (V^T operands two steps ahead), with the
    // V copies of a later tile. Steps 0, 1 carry the rest of the softmax of key block 1,
    // steps 2, 3 the next tile's row max. Row sums of P come from the packed operands
    // (independent partial sums). At the end the first K operands of the next phase A are
    // read (Kn2: the K tile that phase reads).
    auto phase_b = [&](const WF_LDS char* Vc, const WF_LDS char* Kn2, f32x16 (*cur)[2],
                       f32x16 (*nxt)[2], const float* neg_m, const Pending& pd) {
      float mx[2][4];
      float lp[2][4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4 va[NDV];
#pragma unroll
        for (int n = 0; n < NDV; ++n) {
          va[n] = vpre[m & 1][n];
          if (m + 2 < 4) vpre[m & 1][n] = vfrag(Vc, m + 2, n);
        }
        // The first MFMA of each P^T operand waits out a possible VALU write of it; V^T
        // operands come straight from LDS reads, accumulators from MFMAs (or from a rescale,
        // which ends long before).
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) mfma_acc_agpr<T, true>(oacc[qb][0], va[0], pk[m][qb]);
#pragma unroll
        for (int n = 1; n < NDV; ++n)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) mfma_acc_agpr<T, false>(oacc[qb][n], va[n], pk[m][qb]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) lp[qb][m] = sum8_acc<T>(pk[m][qb], 0.f);
        copy_step(pd, true, m, 4);
        if (m < 2) {
#pragma unroll
          for (int i = N_EXP_A + m * (64 - N_EXP_A) / 2; i < N_EXP_A + (m + 1) * (64 - N_EXP_A) / 2; ++i)
            softmax_el(cur, neg_m, el_order(i));
          if (m == 1) {
#pragma unroll
            for (int mm = 2; mm < 4; ++mm)
#pragma unroll
              for (int qb = 0; qb < 2; ++qb) pk[mm][qb] = pack8<T>(cur[1][qb], 8 * (mm & 1));
          }
        } else {
          // query block qb = m - 2: 32 scores in four independent max chains
          const int qb = m - 2;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float x = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int idx = 8 * g4 + e;
              x = fmaxf(x, nxt[idx >> 4][qb][idx & 15]);
            }
            mx[qb][g4] = x;
          }
        }
      }
      // 3 wait states between the last dot2c write and an ordinary VALU read of its result.
      asm volatile("s_nop 2"
                   : "+v"(lp[0][0]), "+v"(lp[0][1]), "+v"(lp[0][2]), "+v"(lp[0][3]), "+v"(lp[1][0]),
                     "+v"(lp[1][1]), "+v"(lp[1][2]), "+v"(lp[1][3]));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        l_run[qb] += (lp[qb][0] + lp[qb][1]) + (lp[qb][2] + lp[qb][3]);
        mt_cur[qb] = xhalf_max(fmaxf(fmaxf(mx[qb][0], mx[qb][1]), fmaxf(mx[qb][2], mx[qb][3]))) * c;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        kpre[0][kb] = kfrag(Kn2, 0, kb);
        kpre[1][kb] = kfrag(Kn2, 1, kb);
      }
    };

    // ---- key-tile loop: three K and three V buffers ----
    // Tile t lives in K buffer t%3 and V buffer t%3 (t counted from kt_lo). Iteration u:
    //   phase A  reads K_{u+1}, copies K_{u+3} (into the buffer of K_u), softmax of tile u;
    //   then it waits for all its copies but the four latest (those of K_{u+3}): K_{u+2}
    //   and V_{u+1} have landed; a barrier makes every wave's copies visible and ends every
    //   wave's reads of V_{u-1} and K_u;
    //   phase B  reads V_u, copies V_{u+2} (into the buffer of V_{u-1}), and reads ahead the
    //   first K operands of K_{u+2} for phase A of iteration u+1.
    const int n_tiles = it.kt_hi - it.kt_lo;
    const int n_live = kt_live - it.kt_lo;
    if (n_tiles > 0) {
      auto clamp_t = [&](int t) { return it.kt_lo + (t < n_tiles ? t : n_tiles - 1); };
      issue_k(clamp_t(0), sK[0]);
      issue_v(clamp_t(0), sV[0]);
      issue_k(clamp_t(1), sK[1]);
      issue_v(clamp_t(1), sV[1]);
      issue_k(clamp_t(2), sK[2]);
      wait_vmem();
      __syncthreads();
      if (n_live > 0) {
        s_tile(sK[0], sc);
        if (need_mask(it.kt_lo)) apply_mask(it.kt_lo, sc);
        tile_max(sc);
        // O and l are still zero: the first reference max is set without a rescale.
        m_run[0] = mt_cur[0];
        m_run[1] = mt_cur[1];
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        kpre[0][kb] = kfrag(sK[1], 0, kb);
        kpre[1][kb] = kfrag(sK[1], 1, kb);
      }
      __syncthreads();  // K_0's buffer is refilled in iteration 0
      // Buffer copies past the last tile get empty descriptors (see copy_step); the copies
      // of the prologue above use clamp_t only for the pointer form.
      Stream kst = make_stream(kp, a.k_sm, it.kt_lo + 3);  // copied during iteration 0
      Stream vst = make_stream(vp, a.v_sm, it.kt_lo + 2);
      // Iteration u with R = u % 6 known at compile time: buffers u%3, (u+1)%3, (u+2)%3 and
      // the score registers (even tiles in sc, odd in sn) are fixed per instance.
      auto iter = [&](int u, auto rc) {
        constexpr int R = decltype(rc)::value;
        constexpr int b0 = R % 3, b1 = (R + 1) % 3, b2 = (R + 2) % 3;
        f32x16 (*cur)[2] = R % 2 ? sn : sc;
        f32x16 (*nxt)[2] = R % 2 ? sc : sn;
        Pending pd;
        pd.kt_k = clamp_t(u + 3);
        pd.kt_v = clamp_t(u + 2);
        pd.Kd = sK[b0];  // K_{u+3} replaces K_u
        pd.Vd = sV[b2];  // V_{u+2} replaces V_{u-1}
        if constexpr (kBuf) {
          pd.rk = stream_rsrc(kst);
          pd.rv = stream_rsrc(vst);
          stream_next(kst);
          stream_next(vst);
        }
        const bool live = u < n_live;
        float neg_m[2] = {0.f, 0.f};
        if (live) {
          rescale();
          neg_m[0] = m_run[0] == -INFINITY ? 0.f : -m_run[0];
          neg_m[1] = m_run[1] == -INFINITY ? 0.f : -m_run[1];
          phase_a(sK[b1], sV[b0], cur, nxt, neg_m, pd);
          if (u + 1 < n_live && need_mask(it.kt_lo + u + 1)) apply_mask(it.kt_lo + u + 1, nxt);
        } else {  // past this wave's causal range: only the copies
#pragma unroll
          for (int st = 0; st < NS; ++st) copy_step(pd, false, st, NS);
        }
        wait_vmem_n<KLOADS>();
        asm volatile("s_barrier" ::: "memory");
        if (live) {
          phase_b(sV[b0], sK[b2], cur, nxt, neg_m, pd);
        } else {
#pragma unroll
          for (int st = 0; st < 4; ++st) copy_step(pd, true, st, 4);
        }
      };
      typedef std::integral_constant<int, 0> R0;
      typedef std::integral_constant<int, 1> R1;
      typedef std::integral_constant<int, 2> R2;
      typedef std::integral_constant<int, 3> R3;
      typedef std::integral_constant<int, 4> R4;
      typedef std::integral_constant<int, 5> R5;
      for (int u = 0;;) {
        iter(u, R0());
        if (++u >= n_tiles) break;
        iter(u, R1());
        if (++u >= n_tiles) break;
        iter(u, R2());
        if (++u >= n_tiles) break;
        iter(u, R3());
        if (++u >= n_tiles) break;
        iter(u, R4());
        if (++u >= n_tiles) break;
        iter(u, R5());
        if (++u >= n_tiles) break;
      }
      wait_vmem();  // nothing may still be landing in LDS when the work item ends
    }

    // ---- epilogue ----
    o_settle(oacc);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l = xhalf_sum(l_run[qb]);
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const float lse2 =
          l > 0.f ? (m_run[qb] == -INFINITY ? 0.f : m_run[qb]) + __builtin_log2f(l) : -INFINITY;
      if (qrow[qb] < it.Lq) {
        if constexpr (MODE == MODE_SPLIT) {
          const int64_t row = (((int64_t)it.split * a.B + it.b) * a.Hq + hq) * a.Lq + qrow[qb];
          float* dst = a.part_o + row * DV;
#pragma unroll
          for (int n = 0; n < NDV; ++n)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              f32x4 o4;
#pragma unroll
              for (int e = 0; e < 4; ++e) o4[e] = oacc[qb][n][4 * q4 + e] * inv;
              *reinterpret_cast<f32x4*>(dst + 32 * n + 8 * q4 + 4 * hf) = o4;
            }
          if (hf == 0) a.part_lse[row] = lse2 * kLn2;
        } else {
          T* dst = (T*)a.o + it.b * a.o_sb + hq * a.o_sh + (it.qtok0 + qrow[qb]) * a.o_sm;
          typedef T t4 __attribute__((ext_vector_type(4)));
#pragma unroll
          for (int n = 0; n < NDV; ++n)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              t4 o4;
#pragma unroll
              for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[qb][n][4 * q4 + e] * inv);
              *reinterpret_cast<t4*>(dst + 32 * n + 8 * q4 + 4 * hf) = o4;
            }
          if (MODE == MODE_DENSE && a.lse != nullptr && hf == 0)
            a.lse[((int64_t)it.b * a.Hq + hq) * a.Lq + qrow[qb]] = lse2 * kLn2;
        }
      }
    }
  }
};

template <typename T, int DQK, int DQK1, int DV, int HPW, int MASK, bool CAUSAL, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_w_kernel(FwdArgs a) {
  typedef AttnFwdW<T, DQK, DQK1, DV, HPW, MASK, CAUSAL, MODE> K;
  __shared__ __attribute__((aligned(1024))) char sK0[K::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[K::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sK2[K::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[K::VBYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[K::VBYTES];
  __shared__ __attribute__((aligned(1024))) char sV2[K::VBYTES];
  WF_LDS char* const kb[3] = {(WF_LDS char*)sK0, (WF_LDS char*)sK1, (WF_LDS char*)sK2};
  WF_LDS char* const vb[3] = {(WF_LDS char*)sV0, (WF_LDS char*)sV1, (WF_LDS char*)sV2};
  attn_dispatch<K, MODE, CAUSAL>(a, [&](const WorkItem& it) { K::run(a, it, kb, vb); });
}

}  // namespace wf
