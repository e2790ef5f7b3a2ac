// Persistent attention kernel with 64-query waves (one wave per SIMD) for dense 16-bit calls
// without a mask, head dim 128: out = softmax(scale Q K^T) V (and, when asked, the row
// log-sum-exp), the PyTorch SDPA contract of WorldFoundry "Core 注意力" ("选择最窄的入口"),
// with GQA head grouping and causal masking.
//
// Same arithmetic as attn_fwd_p.hpp with fp32 row sums (S^T = K Q^T, online softmax in the
// log2 domain with a lazy reference max, O^T += V^T P^T; each score is scaled by
// scale*log2(e) and shifted onto the reference max by one fp32 FMA). What differs is the
// shape of the work and the order of the instructions:
//
//   * Each wave owns 64 query rows (two blocks of 32), so every K and V^T operand read from
//     LDS feeds two MFMAs. With 32-query waves the operand reads alone are 1 KiB per MFMA,
//     which is the LDS bandwidth of a CU (about 128 B per clock) at the MFMA rate; here they
//     are half that.
//   * With one wave per SIMD nothing hides a stall, so the tile loop is written as a fixed
//     sequence of slots, one MFMA each (about 32 clocks), fenced so the compiler keeps the
//     order. Phase A (the next tile's 32 S^T MFMAs) carries two exponentials per slot and
//     the first P^T packs; phase B (the current tile's 32 O^T MFMAs) carries the next tile's
//     row max and its scaling and shift onto the reference max, the fp32 row sums and the
//     remaining packs. Measured on gfx950: up to three
//     exponentials or six plain VALU operations fit beside one MFMA without delaying it.
//   * Row sums are fp32 adds of the weights. A v_dot2 issued while MFMAs are in flight
//     waits for the matrix pipe (measured: one per MFMA slot turns 32 clocks into 50).
//   * K tiles rotate through three LDS buffers and V tiles through two, so that phase B can
//     read the first K operands of the next phase A (that tile landed an iteration earlier)
//     and the loop needs one barrier per tile.
//   * Each wave stages the Q rows of its next item in an LDS area of its own; the same area
//     turns a finished item's O around so that it is written to memory as whole rows (16
//     bytes per lane, consecutive lanes on consecutive bytes) rather than 8-byte pieces of
//     32 rows per instruction.
//
// Work items are those of the persistent 32-query kernel: (batch, KV head, HPW query heads,
// BMP query positions), dealt to the P = #CUs work groups XCD by XCD in alternating-direction
// rounds. A work group of four waves covers HPW heads x BMP positions = 256 rows; wave w
// takes head w / (4 / HPW), positions 64 (w % (4 / HPW)) .. +63. Every wave of a group must
// compute the same key tiles, so causal calls need HPW = 4 (BMP = 64, one key tile of
// positions); the host sends other causal calls to the other kernels.
//
// Hazards of the hand-written O^T MFMA (AGPR accumulator), as in attn_fwd_w.hpp: the first
// MFMA of each P^T operand starts with s_nop 1 (a VALU write of an operand needs 2 wait
// states before an MFMA reads it), and reads of the accumulators are preceded by o_settle.
#pragma once
#include "attn_fwd_w.hpp"

namespace wf {

typedef int i32x4q __attribute__((ext_vector_type(4)));

template <typename T, int D, int HPW, bool CAUSAL>
struct AttnFwdQ {
  static constexpr int NW = 4;
  static constexpr int BN = 64;
  static constexpr int kNW = NW;
  static constexpr int kHPW = HPW;
  static constexpr bool kPack = false;
  static constexpr int WPH = NW / HPW;      // waves per head
  static constexpr int BMP = WPH * 64;      // query positions per item
  static constexpr int NT = NW * 64;
  static constexpr int KCH = D / 8;         // 16-byte chunks per row
  static constexpr int KLOADS = BN * KCH / NT;
  static constexpr int VLOADS = BN * KCH / NT;
  static constexpr int TBYTES = BN * D * 2; // one K or V tile
  static constexpr int NS = D / 16;         // k-steps of the S^T MFMAs
  static constexpr int NDV = D / 32;        // 32-wide column blocks of O^T
  static constexpr int QBYTES = 64 * D * 2; // staged Q rows of one wave
  static constexpr int QLOADS = 64 * KCH / 64;
  static constexpr int MAX_ITEMS = 512;
  static_assert(sizeof(T) == 2, "16-bit inputs only");
  static_assert(D == 128, "the slot schedule is written for head dim 128");
  static_assert(NW % HPW == 0, "waves split evenly over heads");
  static_assert(!CAUSAL || BMP == BN, "causal: every wave of a group on the same key tiles");

  static __device__ __forceinline__ int kswz(int row) { return lds_kswz<KCH>(row); }
  static __device__ __forceinline__ int vswz(int row) { return lds_vswz<KCH>(row); }

  static __device__ __forceinline__ int tile_end(int pos0, int Lk, int shift) {
    const int n_kt = (Lk + BN - 1) / BN;
    if (!CAUSAL) return n_kt;
    const int lim = pos0 + BMP - 1 + shift;
    if (lim < 0) return 0;
    const int e = lim / BN + 1;
    return e < n_kt ? e : n_kt;
  }

  // Block index (one-item-per-group numbering of decode_grid) of the k-th item of work group
  // p of P, or -1 past the end of its list.
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

  struct Item {
    int k, b, hq0, pos0, n;   // n: key tiles (0 past the end of the list)
  };
  static __device__ __forceinline__ void build_items(const FwdArgs& a, int p, int P, WF_LDS i32x4q* list) {
    for (int k = threadIdx.x; k < MAX_ITEMS; k += NT) {
      const int bid = item_bid(a, p, P, k);
      i32x4q v = {0, 0, 0, 0};
      if (bid >= 0) {
        const WorkItem it = decode_grid<AttnFwdQ, CAUSAL>(a, bid, -1);
        v = i32x4q{it.b, it.hq0, it.pos0, it.kt_hi - it.kt_lo};
      }
      list[k] = v;
    }
  }
  static __device__ __forceinline__ Item item_at(const WF_LDS i32x4q* list, int k) {
    Item r;
    r.k = k;
    const i32x4q v = list[k < MAX_ITEMS ? k : MAX_ITEMS - 1];
    r.b = __builtin_amdgcn_readfirstlane(v[0]);
    r.hq0 = __builtin_amdgcn_readfirstlane(v[1]);
    r.pos0 = __builtin_amdgcn_readfirstlane(v[2]);
    r.n = k < MAX_ITEMS ? __builtin_amdgcn_readfirstlane(v[3]) : 0;
    return r;
  }

  typedef WF_LDS char* LP;

  static __device__ __forceinline__ void run(const FwdArgs& a, LP sK0, LP sK1, LP sK2, LP sV0,
                                             LP sV1, LP sQ, WF_LDS i32x4q* list) {
    build_items(a, blockIdx.x, gridDim.x, list);
    __syncthreads();
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, hf = lane >> 5;
    const int hw = w / WPH;
    const int qw = (w % WPH) * 64;
    const float c = a.scale_log2;

    // ---- copies into LDS (buffer loads; see attn_fwd_p.hpp): a descriptor whose size ends at
    // the first row that must not be read (those rows land as zeros) and a per-lane byte
    // offset shared by all tiles. Lane -> chunk q of the copy, row q / KCH, swizzled position
    // q % KCH, which holds logical chunk (q % KCH) ^ swizzle(row).
    //   K / V tiles: copy i of wave w fills chunks [(i*NW + w)*64, +64) = rows [16i, 16i + 16).
    //   Q: wave w stages its own 64 rows; copy i fills chunks [64i, +64) of its area.
    auto rsrc = [](const void* base, int64_t bytes) {
      const uint32_t nrec = bytes <= 0 ? 0u : bytes >= 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
      return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)nrec, 0x00020000);
    };
    constexpr int TROWS = NT / KCH;             // rows per tile copy (16)
    constexpr int QROWS = 64 / KCH;             // rows per Q copy (4)
    constexpr int QV = 16 / QROWS;              // distinct Q offsets (the swizzle repeats every 16 rows)
    static_assert(TROWS % 16 == 0 && QLOADS % QV == 0, "copies share their offsets");
    const uint32_t ksm2 = (uint32_t)(a.k_sm * 2), vsm2 = (uint32_t)(a.v_sm * 2), qsm2 = (uint32_t)(a.q_sm * 2);
    uint32_t kvo, vvo, qvo[QV];
    {
      const int q = w * 64 + lane;
      kvo = (uint32_t)(q / KCH) * ksm2 + (uint32_t)(((q % KCH) ^ kswz(q / KCH)) * 16);
      vvo = (uint32_t)(q / KCH) * vsm2 + (uint32_t)(((q % KCH) ^ vswz(q / KCH)) * 16);
    }
#pragma unroll
    for (int i = 0; i < QV; ++i) {
      const int q = i * 64 + lane;
      const int r = q / KCH, pos = q % KCH;
      qvo[i] = (uint32_t)r * qsm2 + (uint32_t)((pos ^ kswz(r)) * 16);
    }
    LP const sQw = sQ + w * QBYTES;
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
    // Q^T operands (AGPRs), as given: block qb, lane (j, hf): row 32qb + j, head-dim
    // 16s + 8hf .. +7.
    u32x4 qf[2][NS];
    auto read_q = [&]() {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          qf[qb][s] = lds_read16(sQw + (32 * qb + j) * KCH * 16 + (((2 * s + hf) ^ kswz(j)) * 16));
          asm volatile("" : "+a"(qf[qb][s]));
        }
    };

    // A copy cursor walks the tiles of the group's items for one tensor.
    struct Cursor {
      int k, t, n;
      const char* base;
      int rows;   // rows of the tensor left from the tile's first row
    };
    const int64_t kstep = (int64_t)BN * a.k_sm * 2, vstep = (int64_t)BN * a.v_sm * 2;
    auto enter = [&](Cursor& cu, int k, bool is_v) {
      const Item it = item_at(list, k);
      cu.k = k;
      cu.t = 0;
      if (it.n == 0) {
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
    Cursor ck, cv;   // K runs three tiles ahead of the compute, V one
    // The wave's part of a tile (w KiB past the copy's first KiB), re-derived every iteration
    // (laundered in iter) so that the compiler does not keep the LDS address of every copy of
    // every buffer in scalar registers.
    int wofs = w * 1024;
    auto issue_one = [&](const Cursor& cu, bool is_v, LP dst, int i) {
      const uint32_t sm2 = is_v ? vsm2 : ksm2;
      int r = cu.rows - i * TROWS;
      r = __builtin_amdgcn_readfirstlane(r < 0 ? 0 : r > TROWS ? TROWS : r);
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(cu.base + (int64_t)i * TROWS * sm2), 0, (int)((uint32_t)r * sm2), 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (WF_LDS void*)(dst + i * NW * 1024 + wofs), 16,
                                               (int)(is_v ? vvo : kvo), 0, 0, 0);
    };
    auto issue = [&](const Cursor& cu, bool is_v, LP dst) {
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) issue_one(cu, is_v, dst, i);
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
      voff[n] = vrow0 * KCH * 16 + (((4 * n + 2 * g16 + b2) ^ fv) * 16) + 8 * (lane & 1);
    // K fragment fi = 2s + kb (rows 32kb + j, chunk 2s + hf); V^T fragment fi = 4m + n.
    auto kfrag = [&](const WF_LDS char* Kt, int fi) {
      return lds_read16(Kt + koff[fi >> 1] + (fi & 1) * 32 * KCH * 16);
    };
    auto vfrag = [&](const WF_LDS char* Vt, int fi) {
      const WF_LDS char* base = Vt + voff[fi & 3] + 16 * (fi >> 2) * KCH * 16;
      const u32x2 lo = lds_read_tr(base);
      const u32x2 hi = lds_read_tr(base + 8 * KCH * 16);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // ---- masking: keys past Lk and, for causal calls, keys after the query. Element r of
    // block (kb, qb) is key k0 + 32kb + 8(r/4) + 4hf + r%4, query pos0 + qw + 32qb + j. ----
    auto need_mask = [&](int kt, int pos0) {
      const int k0 = kt * BN;
      return (k0 + BN > a.Lk) || (CAUSAL && k0 + BN - 1 > pos0 + qw);
    };
    auto apply_mask = [&](int kt, int pos0, f32x16 (*sc)[2]) {
      const int k0 = kt * BN;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qrow = pos0 + qw + 32 * qb + j;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            bool ok = key < a.Lk;
            if (CAUSAL) ok = ok && key <= qrow;
            sc[kb][qb][r] = ok ? sc[kb][qb][r] : -INFINITY;
          }
      }
    };

    f32x16 oacc[2][NDV];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int n = 0; n < NDV; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][n][r] = 0.f;
    // Softmax state per lane and query block, log2 units. A tile's scores are kept as
    // c*s - m_ref (c = scale*log2(e); m_ref the reference max when they are computed: phase B
    // applies the FMA as it takes their max), so a weight is one exp2 of the stored score;
    // m_ref moves only in rescale.
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f}, m_ref[2] = {0.f, 0.f};
    float mt[2] = {-INFINITY, -INFINITY};
    const f32x16 zero16 = {};

    // mt[qb]: max of the current tile relative to m_ref. The reference moves (O and l
    // rescaled, the tile shifted onto the new reference) only when some query's tile max
    // passes it by more than 8, so p = exp2(s - m) <= 2^8. At the first tile of an item O and
    // l are zero and only the reference moves.
    auto rescale = [&](f32x16 (*cur)[2]) {
      float m_abs[2];
      bool need = false;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        m_abs[qb] = m_ref[qb] + mt[qb];
        need = need || m_abs[qb] > m_run[qb] + 8.0f;
      }
      if (wave_any(need)) {
        const bool fresh = !wave_any(m_run[0] != -INFINITY || m_run[1] != -INFINITY);
        float alpha[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m_new = fmaxf(m_run[qb], m_abs[qb]);
          const float m_new_ref = m_new == -INFINITY ? 0.f : m_new;
          alpha[qb] = fast_exp2(m_run[qb] - m_new_ref);
          l_run[qb] *= alpha[qb];
          const float d = m_new_ref - m_ref[qb];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) cur[kb][qb][r] -= d;
          m_run[qb] = m_new;
          m_ref[qb] = m_new_ref;
        }
        if (!fresh) {
          o_settle(oacc);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int n = 0; n < NDV; ++n) {
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[qb][n][r] *= alpha[qb];
              asm volatile("" : "+a"(oacc[qb][n]));
            }
        }
      }
    };

    // S^T of one tile (prologue only), operands one step ahead.
    auto s_tile = [&](const WF_LDS char* Kt, f32x16 (*sc)[2]) {
      u32x4 k0f = kfrag(Kt, 0), k1f = kfrag(Kt, 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u32x4 n0 = k0f, n1 = k1f;
        if (s + 1 < NS) { n0 = kfrag(Kt, 2 * s + 2); n1 = kfrag(Kt, 2 * s + 3); }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          sc[0][qb] = Mfma16<T>::run(k0f, qf[qb][s], s == 0 ? zero16 : sc[0][qb]);
          sc[1][qb] = Mfma16<T>::run(k1f, qf[qb][s], s == 0 ? zero16 : sc[1][qb]);
        }
        k0f = n0; k1f = n1;
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[kb][qb][r] = fmaf(sc[kb][qb][r], c, -m_ref[qb]);
    };
    auto tile_max = [&](f32x16 (*sc)[2]) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][qb][r]);
        mt[qb] = fmaf(xhalf_max(mx), c, -m_ref[qb]);
      }
    };

    u32x4 kr[4];     // K fragment ring: fragment fi in kr[fi % 4], read three fragments ahead
    u32x4 vr[4];     // V^T fragment ring, likewise
    unsigned pk[4][2][4];   // P^T operands [PV step m][query block][dword]
    typedef typename Mfma16<T>::v8 v8;
    auto cvt2 = [](float x, float y) {
      typedef T t2 __attribute__((ext_vector_type(2)));
      t2 r;
      r[0] = (T)x;
      r[1] = (T)y;
      return __builtin_bit_cast(unsigned, r);
    };
    float ls[2][2];  // partial row sums of the current tile

    // Element e = 8 (m & 1) + i of group g = 2m + qb is element e of cur[m >> 1][qb]; group g
    // packs into pk[m][qb].
    // Phase A: slot a issues S^T MFMA (kb, qb) = ((a >> 1) & 1, a & 1) of k-step a >> 2 for
    // the next tile, two exponentials of group a >> 2 of the current tile, the packs of
    // groups 0 and 1 (slots 8-15) and the fp32 row sums of their weights (slots 16-31); the
    // copies of V_{g+1} go out at slots 2, 10, 18, 26 and those of K_{g+3} at 6, 14, 22, 30,
    // and the first three V^T fragments of phase B are read at slots 26, 28, 30.
    auto phase_a = [&](const WF_LDS char* Kn, const WF_LDS char* Vc, LP Kfill, LP Vfill,
                       f32x16 (*cur)[2], f32x16 (*nxt)[2]) {
#pragma unroll
      for (int q = 0; q < 2; ++q) ls[q][0] = ls[q][1] = 0.f;
#pragma unroll
      for (int sl = 0; sl < 32; ++sl) {
        const int s = sl >> 2, kb = (sl >> 1) & 1, qb = sl & 1, fi = sl >> 1;
        nxt[kb][qb] = Mfma16<T>::run(kr[fi & 3], qf[qb][s], s == 0 ? zero16 : nxt[kb][qb]);
        __builtin_amdgcn_sched_barrier(0);   // the slot's MFMA first, then its other work
        if ((sl & 1) == 0 && fi + 3 < 2 * NS) kr[(fi + 3) & 3] = kfrag(Kn, fi + 3);
        {
          const int g = sl >> 2, m = g >> 1, q = g & 1;
          const int e0 = 8 * (m & 1) + 2 * (sl & 3);
          cur[m >> 1][q][e0] = fast_exp2(cur[m >> 1][q][e0]);
          cur[m >> 1][q][e0 + 1] = fast_exp2(cur[m >> 1][q][e0 + 1]);
          // pinned here: otherwise the compiler sinks the exponentials to their uses in phase B
          asm volatile("" : "+v"(cur[m >> 1][q][e0]), "+v"(cur[m >> 1][q][e0 + 1]));
        }
        if (sl >= 8 && sl < 16) {
          const int g = (sl - 8) >> 2, q = g & 1, d = sl & 3;
          pk[0][q][d] = cvt2(cur[0][q][2 * d], cur[0][q][2 * d + 1]);
          asm volatile("" : "+v"(pk[0][q][d]));
        }
        if (sl >= 16) {
          const int i = sl - 16, q = i >> 3, e = i & 7;
          ls[q][e & 1] += cur[0][q][e];
          asm volatile("" : "+v"(ls[q][e & 1]));
        }
        if ((sl & 7) == 2) issue_one(cv, true, Vfill, sl >> 3);
        if ((sl & 7) == 6) issue_one(ck, false, Kfill, sl >> 3);
        if (sl >= 26 && (sl & 1) == 0) vr[(sl - 26) >> 1] = vfrag(Vc, (sl - 26) >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Phase B: slot b issues O^T MFMA (qb, n) = (b & 1, (b >> 1) & 3) of PV step b >> 3, two
    // elements of the next tile's row max, and for b < 24 the row sums and pack of two weights
    // of group 2 + (b >> 2); the first three K fragments of the next phase A (K_{g+2}, copied
    // during the previous iteration) are read at slots 26, 28, 30.
    auto phase_b = [&](const WF_LDS char* Vc, const WF_LDS char* Kpre, f32x16 (*cur)[2],
                       f32x16 (*nxt)[2]) {
      float mx[2][2] = {{-INFINITY, -INFINITY}, {-INFINITY, -INFINITY}};
#pragma unroll
      for (int sl = 0; sl < 32; ++sl) {
        const int m = sl >> 3, n = (sl >> 1) & 3, qb = sl & 1, fi = sl >> 1;
        {
          const u32x4 p = u32x4{pk[m][qb][0], pk[m][qb][1], pk[m][qb][2], pk[m][qb][3]};
          if (n == 0) mfma_acc_agpr<T, true>(oacc[qb][n], vr[fi & 3], p);
          else mfma_acc_agpr<T, false>(oacc[qb][n], vr[fi & 3], p);
        }
        __builtin_amdgcn_sched_barrier(0);   // the slot's MFMA first, then its other work
        // (this slot's pack is of a later PV step's operand: pk[1 + sl / 8])
        if (sl < 24) {
          const int g = 2 + (sl >> 2), mm = g >> 1, q = g & 1, d = sl & 3;
          const int e0 = 8 * (mm & 1) + 2 * d;
          const float x0 = cur[mm >> 1][q][e0], x1 = cur[mm >> 1][q][e0 + 1];
          ls[q][0] += x0;
          ls[q][1] += x1;
          pk[mm][q][d] = cvt2(x0, x1);
          asm volatile("" : "+v"(ls[q][0]), "+v"(ls[q][1]), "+v"(pk[mm][q][d]));
        }
        if ((sl & 1) == 0 && fi + 3 < 4 * NDV) vr[(fi + 3) & 3] = vfrag(Vc, fi + 3);
        {
          const int acc = sl >> 3, kb = acc >> 1, q = acc & 1, e0 = 2 * (sl & 7);
          mx[q][kb] = fmaxf(mx[q][kb], fmaxf(nxt[kb][q][e0], nxt[kb][q][e0 + 1]));
          nxt[kb][q][e0] = fmaf(nxt[kb][q][e0], c, -m_ref[q]);
          nxt[kb][q][e0 + 1] = fmaf(nxt[kb][q][e0 + 1], c, -m_ref[q]);
          asm volatile("" : "+v"(mx[q][kb]), "+v"(nxt[kb][q][e0]), "+v"(nxt[kb][q][e0 + 1]));
        }
        if (sl >= 26 && (sl & 1) == 0) kr[(sl - 26) >> 1] = kfrag(Kpre, (sl - 26) >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        l_run[q] += ls[q][0] + ls[q][1];
        mt[q] = fmaf(xhalf_max(fmaxf(mx[q][0], mx[q][1])), c, -m_ref[q]);
      }
    };

    // Output of an item: O / l rounded to the input type and turned around in the wave's
    // staging area (row 32qb + j of the item, 16-byte chunk (4n + q4) ^ (row % 16) holds
    // head-dim 32n + 8q4 .. +7), then written as whole rows: copy i stores rows 4i + lane/16,
    // chunk lane % 16. Rows past Lq are dropped; the log-sum-exp is written when asked for.
    // O is reset to zero for the next item.
    auto store_item = [&](const Item& it) {
      o_settle(oacc);
      const int hq = it.hq0 + hw;
      typedef T t4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float l = xhalf_sum(l_run[qb]);
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        const int row = 32 * qb + j;
#pragma unroll
        for (int n = 0; n < NDV; ++n)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            t4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[qb][n][4 * q4 + e] * inv);
            *reinterpret_cast<WF_LDS t4*>(sQw + row * KCH * 16 + (((4 * n + q4) ^ (row & 15)) * 16) + 8 * hf) = o4;
          }
        const int qrow = it.pos0 + qw + row;
        if (a.lse != nullptr && hf == 0 && qrow < a.Lq) {
          const float lse2 = l > 0.f ? (m_run[qb] == -INFINITY ? 0.f : m_run[qb]) + __builtin_log2f(l) : -INFINITY;
          a.lse[((int64_t)it.b * a.Hq + hq) * a.Lq + qrow] = lse2 * kLn2;
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int n = 0; n < NDV; ++n) {
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][n][r] = 0.f;
          asm volatile("" : "+a"(oacc[qb][n]));
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own rows, read back below
      T* obase = (T*)a.o + it.b * a.o_sb + hq * a.o_sh;
      const int ch = lane & 15;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 4 * i + (lane >> 4);
        const u32x4 v16 = lds_read16(sQw + row * KCH * 16 + ((ch ^ (row & 15)) * 16));
        const int qrow = it.pos0 + qw + row;
        if (qrow < a.Lq) *reinterpret_cast<u32x4*>(obase + (int64_t)qrow * a.o_sm + 8 * ch) = v16;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // done with the area before it is restaged
    };

    // ---- start: the first item's Q, the first K tiles (0, 1, 2) and V tile 0 ----
    Item cur_it = item_at(list, 0);
    if (cur_it.n == 0) return;
    Item nxt_it = item_at(list, 1);
    stage_q(cur_it);
    enter(ck, 0, false);
    enter(cv, 0, true);
    issue(ck, false, sK0);
    advance(ck, false);
    issue(ck, false, sK1);
    advance(ck, false);
    issue(ck, false, sK2);
    advance(ck, false);
    issue(cv, true, sV0);
    advance(cv, true);
    wait_vmem();
    __syncthreads();
    read_q();
    f32x16 sc[2][2], sn[2][2];
    s_tile(sK0, sc);
    if (need_mask(0, cur_it.pos0)) apply_mask(0, cur_it.pos0, sc);
    tile_max(sc);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // Q reads done before the area refills
    stage_q(nxt_it);   // landed by the wait below
#pragma unroll
    for (int i = 0; i < 3; ++i) kr[i] = kfrag(sK1, i);
    wait_vmem();
    __syncthreads();   // every wave is done with K_0 before its buffer refills

    // ---- tile loop over the group's items ----
    // Global tile g has K in buffer g % 3 and V in buffer g % 2. Iteration g reads K_{g+1}
    // (S^T of the next tile) and V_g, copies V_{g+1} and K_{g+3} (phase A), and reads the
    // first K fragments of K_{g+2} at the end of phase B. In an item's last iteration the next
    // tile is the next item's first: its Q^T is read from the staging area first; after the
    // item's output has gone through the area, the item after next is staged (and waited for
    // at once when the next item has a single tile, whose last iteration is the next one).
    int u = 0;
    bool done = false;
    auto iter = [&](auto rc) {
      constexpr int R = decltype(rc)::value;
      LP const Kb[3] = {sK0, sK1, sK2};
      LP const Vb[2] = {sV0, sV1};
      f32x16 (*cur)[2] = (R & 1) ? sn : sc;
      f32x16 (*nxt)[2] = (R & 1) ? sc : sn;
      asm volatile("" : "+s"(wofs));
      const bool last = u + 1 == cur_it.n;
      if (last) read_q();
      rescale(cur);
      phase_a(Kb[(R + 1) % 3], Vb[R % 2], Kb[R % 3], Vb[(R + 1) % 2], cur, nxt);
      advance(cv, true);
      advance(ck, false);
      const int kt_n = last ? 0 : u + 1;
      const int pos_n = last ? nxt_it.pos0 : cur_it.pos0;
      if (need_mask(kt_n, pos_n)) apply_mask(kt_n, pos_n, nxt);
      phase_b(Vb[R % 2], Kb[(R + 2) % 3], cur, nxt);
      // V_{g+1} and K_{g+3} (issued in phase A) have landed: after the barrier every wave's
      // copies are visible (K_{g+3}'s first fragments are read at the end of phase B of g+1)
      wait_vmem();
      asm volatile("s_barrier" ::: "memory");
      if (last) {
        store_item(cur_it);
        m_run[0] = m_run[1] = -INFINITY;   // m_ref stays: the next item's first tile used it
        l_run[0] = l_run[1] = 0.f;
        cur_it = nxt_it;
        nxt_it = item_at(list, cur_it.k + 1);
        stage_q(nxt_it);
        if (cur_it.n == 1) wait_vmem();
        u = 0;
        done = cur_it.n == 0;
      } else {
        ++u;
      }
    };
    for (;;) {
      iter(std::integral_constant<int, 0>());
      if (done) break;
      iter(std::integral_constant<int, 1>());
      if (done) break;
      iter(std::integral_constant<int, 2>());
      if (done) break;
      iter(std::integral_constant<int, 3>());
      if (done) break;
      iter(std::integral_constant<int, 4>());
      if (done) break;
      iter(std::integral_constant<int, 5>());
      if (done) break;
    }
    wait_vmem();   // the last copies (empty) and stores
  }
};

template <typename T, int D, int HPW, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_q_kernel(FwdArgs a) {
  typedef AttnFwdQ<T, D, HPW, CAUSAL> K;
  // Separate LDS arrays, so the compiler can tell a tile copy into one buffer from the operand
  // reads of another.
  __shared__ __attribute__((aligned(16384))) char sK0[K::TBYTES];
  __shared__ __attribute__((aligned(16384))) char sK1[K::TBYTES];
  __shared__ __attribute__((aligned(16384))) char sK2[K::TBYTES];
  __shared__ __attribute__((aligned(16384))) char sV0[K::TBYTES];
  __shared__ __attribute__((aligned(16384))) char sV1[K::TBYTES];
  __shared__ __attribute__((aligned(1024))) char sQ[K::NW * K::QBYTES];
  __shared__ __attribute__((aligned(16))) i32x4q list[K::MAX_ITEMS];
  K::run(a, (WF_LDS char*)sK0, (WF_LDS char*)sK1, (WF_LDS char*)sK2, (WF_LDS char*)sV0,
         (WF_LDS char*)sV1, (WF_LDS char*)sQ, (WF_LDS i32x4q*)list);
}

}  // namespace wf
