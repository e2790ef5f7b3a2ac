// Exact attention forward for fp32 inputs on gfx950 (v_mfma_f32_32x32x2_f32).
//
// Same method and transposed formulation as the 16-bit kernel (S^T = K Q^T, O^T += V^T P^T,
// lane l owns query l % 32, online softmax in fp32), with fp32 operands end to end: P is
// not rounded before P V. Four waves of 32 queries per work group, 32-key tiles staged
// through padded LDS rows. The SDPA contract (WorldFoundry "Core 注意力", "选择最窄的入口")
// and the mask rule after its CPU/GPU example apply unchanged.
#include "wf_internal.hpp"

namespace wf {

// One 32-key tile for the wave's 32 queries: S^T = K Q^T from the padded K rows in LDS,
// masks, the online softmax update, O^T += V^T P^T. Ks: BN rows of DQK + 1 floats; Vs: BN
// rows of DV floats; k0: the tile's first key.
template <int DQK, int DV, int MASK, bool CAUSAL>
__device__ __forceinline__ void f32_tile(const FwdArgs& a, const float* Ks, const float* Vs,
                                         const float* qf, int k0, int qrow, const char* mrow,
                                         f32x16* oacc, float& m_run, float& l_run) {
  constexpr int KST = DQK + 1, NS = DQK / 2, NDV = DV / 32;
  const int lane = threadIdx.x & 63, j = lane & 31, hf = lane >> 5;
  const float c = a.scale_log2;
  f32x16 sacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[j * KST + 2 * s + hf], qf[s], sacc, 0, 0, 0);

  float mt = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = k0 + 8 * (r >> 2) + 4 * hf + (r & 3);
    bool ok = key < a.Lk;
    if (CAUSAL) ok = ok && key <= qrow + a.causal_shift;
    float t = sacc[r] * c;
    if constexpr (MASK == MASK_BOOL) {
      if (ok) ok = mrow[key] != 0;
    } else if constexpr (MASK == MASK_F32) {
      if (ok) t += reinterpret_cast<const float*>(mrow)[key] * kLog2e;
    }
    t = ok ? t : -INFINITY;
    sacc[r] = t;
    mt = fmaxf(mt, t);
  }
  mt = xhalf_max(mt);
  if (wave_any(mt > m_run)) {
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
    l_run *= alpha;
#pragma unroll
    for (int n = 0; n < NDV; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[n][r] *= alpha;
    m_run = m_new;
  }
  const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = fast_exp2(sacc[r] + neg_m);
    sacc[r] = p;
    l_run += p;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
#pragma unroll
    for (int n = 0; n < NDV; ++n)
      oacc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * DV + 32 * n + j], sacc[r],
                                                     oacc[n], 0, 0, 0);
  }
}

// Output of the wave's 32 queries (row qrow of this lane's query): O / l, and the lse.
template <int DV>
__device__ __forceinline__ void f32_store(const FwdArgs& a, int b, int hq, int qrow,
                                          const f32x16* oacc, float m_run, float l) {
  constexpr int NDV = DV / 32;
  const int hf = (threadIdx.x & 63) >> 5;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (qrow < a.Lq) {
    float* dst = (float*)a.o + b * a.o_sb + hq * a.o_sh + (int64_t)qrow * a.o_sm;
#pragma unroll
    for (int n = 0; n < NDV; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = oacc[n][4 * q4 + e] * inv;
        *reinterpret_cast<f32x4*>(dst + 32 * n + 8 * q4 + 4 * hf) = o4;
      }
    if (a.lse != nullptr && hf == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.Lq + qrow] =
          l > 0.f ? ((m_run == -INFINITY ? 0.f : m_run) + __builtin_log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int DQK, int DV, int MASK, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_f32_kernel(FwdArgs a) {
  constexpr int BN = 32, NW = 4, BM = NW * 32;
  constexpr int KST = DQK + 1;  // padded K row (floats): lanes reading one column hit distinct banks
  constexpr int NS = DQK / 2, NDV = DV / 32;
  __shared__ __attribute__((aligned(16))) float Ks[BN * KST];
  __shared__ __attribute__((aligned(16))) float Vs[BN * DV];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 31, hf = lane >> 5;

  const int t_q = blockIdx.x % a.n_qtiles;
  const int bh = blockIdx.x / a.n_qtiles;
  const int hq = bh % a.Hq, b = bh / a.Hq;
  const int g = hq / a.G;
  const int qlo = t_q * BM + w * 32;
  const int qrow = qlo + j;
  const int qrow_c = qrow < a.Lq ? qrow : a.Lq - 1;
  const float* qp = (const float*)a.q + b * a.q_sb + hq * a.q_sh + (int64_t)qrow_c * a.q_sm;
  const float* kp = (const float*)a.k + b * a.k_sb + g * a.k_sh;
  const float* vp = (const float*)a.v + b * a.v_sb + g * a.v_sh;

  float qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qf[s] = qp[2 * s + hf];

  const char* mrow = nullptr;
  if constexpr (MASK != MASK_NONE) {
    constexpr int msz = MASK == MASK_BOOL ? 1 : 4;
    mrow = (const char*)a.mask + (b * a.mk_sb + hq * a.mk_sh + (int64_t)qrow_c * a.mk_sm) * msz;
  }

  f32x16 oacc[NDV];
#pragma unroll
  for (int n = 0; n < NDV; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[n][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int n_kt = (a.Lk + BN - 1) / BN;
  int kt_end = n_kt;
  if (CAUSAL) {
    const int lim = t_q * BM + BM - 1 + a.causal_shift;
    kt_end = lim < 0 ? 0 : (lim / BN + 1 < n_kt ? lim / BN + 1 : n_kt);
  }
  for (int kt = 0; kt < kt_end; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();  // previous tile fully consumed
    for (int idx = tid * 4; idx < BN * DQK; idx += 256 * 4) {
      const int r = idx / DQK, col = idx % DQK;
      const int row = k0 + r < a.Lk ? k0 + r : a.Lk - 1;
      const f32x4 x = *reinterpret_cast<const f32x4*>(kp + (int64_t)row * a.k_sm + col);
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[r * KST + col + e] = x[e];
    }
    for (int idx = tid * 4; idx < BN * DV; idx += 256 * 4) {
      const int r = idx / DV, col = idx % DV;
      const int row = k0 + r < a.Lk ? k0 + r : a.Lk - 1;
      *reinterpret_cast<f32x4*>(&Vs[r * DV + col]) =
          *reinterpret_cast<const f32x4*>(vp + (int64_t)row * a.v_sm + col);
    }
    __syncthreads();
    if (CAUSAL && k0 > qlo + 31 + a.causal_shift) continue;
    f32_tile<DQK, DV, MASK, CAUSAL>(a, Ks, Vs, qf, k0, qrow, mrow, oacc, m_run, l_run);
  }
  f32_store<DV>(a, b, hq, qrow, oacc, m_run, xhalf_sum(l_run));
}

// Key-split form for one 32-query tile per (batch, head) (Lq <= 32) over several key tiles:
// the four waves take the key tiles kt = w (mod 4) of the same 32 queries, each through its own
// LDS tile (a wave's LDS accesses run in order, so its loop needs no barrier), and their
// partial (m, l, O) are merged through LDS at the end. In the one-tile-per-wave kernel three of
// the four waves of such a group have no query rows and the fourth walks every key tile.
template <int DQK, int DV, int MASK, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_f32_ks_kernel(FwdArgs a) {
  constexpr int BN = 32, NW = 4;
  constexpr int KST = DQK + 1, NS = DQK / 2, NDV = DV / 32;
  constexpr int KW = BN * KST, VW = BN * DV;  // floats of one wave's K and V tiles
  constexpr int OW = 16 * NDV * 64;           // floats of one wave's O^T fragments
  constexpr int SM = NW * (KW + VW) > NW * (OW + 128) ? NW * (KW + VW) : NW * (OW + 128);
  __shared__ __attribute__((aligned(16))) float smem[SM];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 31, hf = lane >> 5;

  const int hq = blockIdx.x % a.Hq, b = blockIdx.x / a.Hq;
  const int g = hq / a.G;
  const int qrow = j;
  const int qrow_c = qrow < a.Lq ? qrow : a.Lq - 1;
  const float* qp = (const float*)a.q + b * a.q_sb + hq * a.q_sh + (int64_t)qrow_c * a.q_sm;
  const float* kp = (const float*)a.k + b * a.k_sb + g * a.k_sh;
  const float* vp = (const float*)a.v + b * a.v_sb + g * a.v_sh;

  float qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qf[s] = qp[2 * s + hf];

  const char* mrow = nullptr;
  if constexpr (MASK != MASK_NONE) {
    constexpr int msz = MASK == MASK_BOOL ? 1 : 4;
    mrow = (const char*)a.mask + (b * a.mk_sb + hq * a.mk_sh + (int64_t)qrow_c * a.mk_sm) * msz;
  }

  f32x16 oacc[NDV];
#pragma unroll
  for (int n = 0; n < NDV; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[n][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int n_kt = (a.Lk + BN - 1) / BN;
  int kt_end = n_kt;
  if (CAUSAL) {
    const int lim = 31 + a.causal_shift;
    kt_end = lim < 0 ? 0 : (lim / BN + 1 < n_kt ? lim / BN + 1 : n_kt);
  }
  float* Ks = smem + w * (KW + VW);
  float* Vs = Ks + KW;
  for (int kt = w; kt < kt_end; kt += NW) {
    const int k0 = kt * BN;
    for (int idx = lane * 4; idx < BN * DQK; idx += 64 * 4) {
      const int r = idx / DQK, col = idx % DQK;
      const int row = k0 + r < a.Lk ? k0 + r : a.Lk - 1;
      const f32x4 x = *reinterpret_cast<const f32x4*>(kp + (int64_t)row * a.k_sm + col);
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[r * KST + col + e] = x[e];
    }
    for (int idx = lane * 4; idx < BN * DV; idx += 64 * 4) {
      const int r = idx / DV, col = idx % DV;
      const int row = k0 + r < a.Lk ? k0 + r : a.Lk - 1;
      *reinterpret_cast<f32x4*>(&Vs[r * DV + col]) =
          *reinterpret_cast<const f32x4*>(vp + (int64_t)row * a.v_sm + col);
    }
    f32_tile<DQK, DV, MASK, CAUSAL>(a, Ks, Vs, qf, k0, qrow, mrow, oacc, m_run, l_run);
  }

  // Merge: wave v's lane l holds the same (query, head-dim) elements in every wave.
  // O = sum_v 2^(m_v - m) O_v, l = sum_v 2^(m_v - m) l_v with m = max_v m_v; a wave with no
  // kept key (m_v = -inf) contributes nothing, and a query with none in any wave gets 0.
  __syncthreads();  // every wave is done with its tiles: the LDS is reused
  float* Om = smem;               // [wave][16*NDV][64 lanes]
  float* Mm = smem + NW * OW;     // [wave][64]
  float* Lm = Mm + NW * 64;       // [wave][64]
#pragma unroll
  for (int n = 0; n < NDV; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) Om[(w * 16 * NDV + 16 * n + r) * 64 + lane] = oacc[n][r];
  Mm[w * 64 + lane] = m_run;
  Lm[w * 64 + lane] = xhalf_sum(l_run);
  __syncthreads();
  if (w == 0) {
    float mv[NW];
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      mv[v] = Mm[v * 64 + lane];
      m = fmaxf(m, mv[v]);
    }
    const float mref = m == -INFINITY ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int n = 0; n < NDV; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[n][r] = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float alpha = mv[v] == -INFINITY ? 0.f : fast_exp2(mv[v] - mref);
      l += alpha * Lm[v * 64 + lane];
#pragma unroll
      for (int n = 0; n < NDV; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[n][r] += alpha * Om[(v * 16 * NDV + 16 * n + r) * 64 + lane];
    }
    f32_store<DV>(a, b, hq, qrow, oacc, m, l);
  }
}

#define F(DQK, DV, MASK, CAUSAL) {DQK, DV, MASK, CAUSAL, (const void*)&attn_f32_kernel<DQK, DV, MASK, CAUSAL>, 128}
#define FD(DQK, DV) F(DQK, DV, MASK_NONE, false), F(DQK, DV, MASK_NONE, true), \
                    F(DQK, DV, MASK_BOOL, false), F(DQK, DV, MASK_F32, false)
static const F32Entry kTable[] = {
    FD(64, 64), FD(64, 96), FD(64, 128), FD(128, 64), FD(128, 96), FD(128, 128),
};
#undef FD
#undef F

const F32Entry* attn_table_f32(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}

#define F(DQK, DV, MASK, CAUSAL) {DQK, DV, MASK, CAUSAL, (const void*)&attn_f32_ks_kernel<DQK, DV, MASK, CAUSAL>, 32}
#define FD(DQK, DV) F(DQK, DV, MASK_NONE, false), F(DQK, DV, MASK_NONE, true), \
                    F(DQK, DV, MASK_BOOL, false), F(DQK, DV, MASK_F32, false)
static const F32Entry kTableKs[] = {
    FD(64, 64), FD(64, 96), FD(64, 128), FD(128, 64), FD(128, 96), FD(128, 128),
};
#undef FD
#undef F

const F32Entry* attn_table_f32_ks(int* n) {
  *n = (int)(sizeof(kTableKs) / sizeof(kTableKs[0]));
  return kTableKs;
}

}  // namespace wf
