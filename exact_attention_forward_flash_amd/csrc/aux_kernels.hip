// Auxiliary kernels: the varlen tile schedule, the split-KV combine and the block KV cache
// copy / gather.
#include <type_traits>

#include "wf_internal.hpp"

namespace wf {

// ------------------------------------------------------------------------------------------
// Varlen tile schedule (packed sequences given by per-sequence lengths, Ascend "MLA Prefill"
// qSeqLen / kvSeqLen).
//   cu_q, cu_k = exclusive prefix sums of the lengths ([batch + 1]);
//   max_kv >= 0: keys and values are padded per sequence (max_kv rows each), so a sequence's
//   kv length may not exceed max_kv and the packed total is not checked;
//   one work item per (sequence, query tile of bmp positions), sequence by sequence (longest
//   sequences first, each sequence's tiles from its last query tile down).
// One work group of 1024 threads; the attention kernel that follows on the stream takes
// items from the counter this kernel resets.
// ------------------------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kSchedBuckets = 2048;

template <typename I>
__device__ I block_exclusive_scan(I v, I* sm, I* total) {
  const int t = threadIdx.x;
  sm[t] = v;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const I x = t >= off ? sm[t - off] : 0;
    __syncthreads();
    sm[t] += x;
    __syncthreads();
  }
  const I incl = sm[t];
  *total = sm[kSchedThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(
    const int32_t* q_seqlen, const int32_t* kv_seqlen, int batch, int64_t total_q,
    int64_t total_k, int max_kv, int bmp, int bn, int causal, int max_items, int* ws) {
  __shared__ int sm[kSchedThreads];
  __shared__ int64_t sm64[kSchedThreads];  // length sums: 1024 int32 lengths can overflow 32 bits
  __shared__ int hist[kSchedBuckets];
  __shared__ int s_bad;
  (void)causal;   // the order does not depend on the mask: a sequence's last tile is its longest
  int* cu_q = (int*)((char*)ws + VarlenWs::cu_q_off());
  int* cu_k = (int*)((char*)ws + VarlenWs::cu_k_off(batch));
  int2* items = (int2*)((char*)ws + VarlenWs::items_off(batch));
  const int t = threadIdx.x;
  if (t == 0) s_bad = 0;
  for (int i = t; i < kSchedBuckets; i += kSchedThreads) hist[i] = 0;
  __syncthreads();

  // Prefix sums over the batch, 1024 sequences at a time. Totals are kept in 64 bits to
  // reject lengths that overflow.
  int64_t carry_q = 0, carry_k = 0;
  int64_t carry_items = 0;
  for (int base = 0; base < batch; base += kSchedThreads) {
    const int bi = base + t;
    int lq = 0, lk = 0;
    if (bi < batch) {
      lq = q_seqlen[bi];
      lk = kv_seqlen[bi];
      if (lq < 0 || lk < 0 || (max_kv >= 0 && lk > max_kv)) s_bad = 1;
    }
    lq = lq < 0 ? 0 : lq;
    lk = lk < 0 ? 0 : lk;
    int64_t tot_q, tot_k;
    int64_t tot_i;
    const int64_t eq = block_exclusive_scan<int64_t>(lq, sm64, &tot_q);
    const int64_t ek = block_exclusive_scan<int64_t>(lk, sm64, &tot_k);
    const int64_t ntile = ((int64_t)lq + bmp - 1) / bmp;
    block_exclusive_scan<int64_t>(ntile, sm64, &tot_i);
    // Offsets past 2^31 are never used: the totals below flag the call as bad.
    if (bi < batch) {
      cu_q[bi] = (int)(carry_q + eq);
      cu_k[bi] = (int)(carry_k + ek);
    }
    carry_q += tot_q;
    carry_k += tot_k;
    carry_items += tot_i;
    __syncthreads();
  }
  if (t == 0) {
    cu_q[batch] = (int)carry_q;
    cu_k[batch] = (int)carry_k;
    if (carry_q > total_q || (max_kv < 0 && carry_k > total_k) || carry_k > 0x7fffffff ||
        carry_items > max_items)
      s_bad = 1;
  }
  __syncthreads();
  const int bad = s_bad;
  const int n_pairs = bad ? 0 : (int)carry_items;

  // Item order: sequence by sequence, sequences by descending key-tile count (a counting
  // sort over buckets of that count, each sequence taking a contiguous run of slots), and
  // within a sequence its query tiles from the last (most keys under the causal rule) to
  // the first. Work groups that take consecutive items then stream the same sequence's K/V
  // tiles at about the same time, so each tile is fetched once into L2 and read by many;
  // the list still ends with the shortest items. Pass 0 adds each sequence's tile count to
  // its bucket, the exclusive scan turns the sums into slot offsets, pass 1 claims a run of
  // slots per sequence. One thread walks the tiles of one sequence.
  if (!bad) {
    for (int pass = 0; pass < 2; ++pass) {
      for (int base = 0; base < batch; base += kSchedThreads) {
        const int bi = base + t;
        if (bi < batch) {
          const int lq = cu_q[bi + 1] - cu_q[bi];
          const int lk = cu_k[bi + 1] - cu_k[bi];
          const int ntile = (int)(((int64_t)lq + bmp - 1) / bmp);
          const int n_kt = (int)(((int64_t)lk + bn - 1) / bn);
          const int bucket =
              kSchedBuckets - 1 - (n_kt < kSchedBuckets - 1 ? n_kt : kSchedBuckets - 1);
          if (ntile > 0) {
            if (pass == 0) {
              atomicAdd(&hist[bucket], ntile);
            } else {
              const int pos = atomicAdd(&hist[bucket], ntile);
              for (int j = 0; j < ntile; ++j) items[pos + j] = make_int2(bi, ntile - 1 - j);
            }
          }
        }
      }
      __syncthreads();
      if (pass == 0) {  // exclusive scan of the histogram; bucket 0 holds the longest sequences
        int run = 0;
        for (int base = 0; base < kSchedBuckets; base += kSchedThreads) {
          int tot;
          const int ex = block_exclusive_scan<int>(hist[base + t], sm, &tot);
          hist[base + t] = run + ex;
          run += tot;
          __syncthreads();
        }
      }
    }
  }
  if (t < 8) ws[16 + 4 * t] = 0;   // per-XCD work counters
  if (t == 0) {
    ws[0] = 0;        // work counter
    ws[1] = n_pairs;  // number of (sequence, tile) items; heads are expanded by the kernel
    ws[2] = bad;
  }
}

hipError_t launch_varlen_schedule(const int32_t* q_seqlen, const int32_t* kv_seqlen, int batch,
                                  int64_t total_q, int64_t total_k, int max_kv, int bmp, int bn,
                                  int causal, int max_items, int* ws, hipStream_t s) {
  hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, q_seqlen,
                     kv_seqlen, batch, total_q, total_k, max_kv, bmp, bn, causal, max_items, ws);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Split-KV combine: out = sum_s w_s O_s / sum_s w_s with w_s = exp(lse_s - max_s lse_s),
// where O_s is split s's normalised partial output and lse_s its log-sum-exp. A query with
// no kept key in any split gets 0. Splits are summed in index order (deterministic).
// ------------------------------------------------------------------------------------------
// Index arithmetic in I: 32 bits whenever rows * Dv/4 fits (the divisions that split a thread
// index into row, batch and head are then a few instructions instead of a 64-bit division
// sequence each); element offsets stay 64-bit.
template <typename T, typename I>
__global__ __launch_bounds__(256) void split_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int n_splits,
    int B, int Hq, int Lq, int Dv, T* out, int64_t o_sb, int64_t o_sh, int64_t o_sm,
    float* lse) {
  const int64_t rows = (int64_t)B * Hq * Lq;
  const I d4 = (I)(Dv / 4);
  const I gid = (I)blockIdx.x * (I)blockDim.x + (I)threadIdx.x;
  if ((int64_t)gid >= rows * d4) return;
  const I row = gid / d4;
  const int d = (int)(gid - row * d4) * 4;
  // Splits are read in batches of CB with every load of a batch issued before any is used
  // (one memory round trip per batch instead of one per split); sums stay in split order.
  constexpr int CB = 8;
  float mx = -INFINITY;
  for (int s0 = 0; s0 < n_splits; s0 += CB) {
    float ls[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u)
      ls[u] = s0 + u < n_splits ? part_lse[(int64_t)(s0 + u) * rows + row] : -INFINITY;
#pragma unroll
    for (int u = 0; u < CB; ++u) mx = fmaxf(mx, ls[u]);
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (mx != -INFINITY) {
    for (int s0 = 0; s0 < n_splits; s0 += CB) {
      float ls[CB];
      f32x4 o[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const bool in = s0 + u < n_splits;
        ls[u] = in ? part_lse[(int64_t)(s0 + u) * rows + row] : -INFINITY;
        o[u] = in ? *reinterpret_cast<const f32x4*>(part_o + ((int64_t)(s0 + u) * rows + row) * Dv + d)
                  : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const float wgt = __expf(ls[u] - mx);   // 0 past the last split
        den += wgt;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += wgt * o[u][e];
      }
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  // lse of the whole row: the splits' lse merged the same way (-inf when no key is kept)
  if (lse != nullptr && d == 0) lse[row] = den > 0.f ? mx + __logf(den) : -INFINITY;
  const I bh = row / (I)Lq;
  const int q = (int)(row - bh * (I)Lq);
  const I b_ = bh / (I)Hq;
  const int hq = (int)(bh - b_ * (I)Hq);
  const int b = (int)b_;
  T* dst = out + b * o_sb + hq * o_sh + (int64_t)q * o_sm + d;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[e] = (T)(acc[e] * inv);
}

hipError_t launch_split_combine(int dtype, const float* part_o, const float* part_lse,
                                int n_splits, int B, int Hq, int Lq, int Dv, void* out,
                                int64_t o_sb, int64_t o_sh, int64_t o_sm, float* lse,
                                hipStream_t s) {
  const int64_t n = (int64_t)B * Hq * Lq * (Dv / 4);
  const int blocks = (int)((n + 255) / 256);
  const bool i32 = (int64_t)blocks * 256 < ((int64_t)1 << 31);
  auto go = [&](auto tag, auto* o) {
    typedef decltype(tag) I;
    typedef typename std::remove_pointer<decltype(o)>::type T;
    hipLaunchKernelGGL((split_combine_kernel<T, I>), dim3(blocks), dim3(256), 0, s, part_o,
                       part_lse, n_splits, B, Hq, Lq, Dv, o, o_sb, o_sh, o_sm, lse);
  };
  auto by_index = [&](auto* o) {
    if (i32) go(uint32_t(0), o);
    else go(int64_t(0), o);
  };
  if (dtype == DT_BF16) by_index((__bf16*)out);
  else if (dtype == DT_F16) by_index((_Float16*)out);
  else by_index((float*)out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Block KV cache ("Block KV cache 的调用顺序": sink prefix never evicted, window rolls).
// Token t lives in slot t (t < sink) or sink + (t - sink) mod window.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int64_t cache_slot(int64_t t, int64_t sink, int64_t window) {
  return t < sink ? t : sink + (t - sink) % window;
}

template <int U> struct CopyUnit;
template <> struct CopyUnit<16> { typedef u32x4 type; };
template <> struct CopyUnit<4> { typedef uint32_t type; };
template <> struct CopyUnit<2> { typedef uint16_t type; };

// Copies one chunk of new rows into their slots, U bytes per thread. Segment 0 is K,
// segment 1 is V (blockIdx.y). Strides are [b, h, row] in elements.
// Index arithmetic in I (32 bits when every index fits, which keeps the divisions cheap); the
// ring slot of row r is the token itself inside the sink, else sink + (off0 + r) folded once
// into the window, with off0 the window offset of the chunk's first token past the sink
// (negative while the chunk still overlaps the sink).
template <int U, typename I>
__global__ __launch_bounds__(256) void kv_update_kernel(
    int esize, const char* k_new, int64_t kn0, int64_t kn1, int64_t kn2, const char* v_new,
    int64_t vn0, int64_t vn1, int64_t vn2, char* k_cache, int64_t kc0, int64_t kc1, int64_t kc2,
    char* v_cache, int64_t vc0, int64_t vc1, int64_t vc2, int B, int H, int chunk, int Dk, int Dv,
    int64_t tok0, int64_t sink, int64_t window, int64_t off0) {
  typedef typename CopyUnit<U>::type unit;
  const bool isv = blockIdx.y == 1;
  const int D = isv ? Dv : Dk;
  const int per_row = D * esize / U;
  const I n = (I)B * H * chunk * per_row;
  const I gid = (I)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n) return;
  const int piece = (int)(gid % per_row);
  const I r = gid / per_row;
  const int row = (int)(r % chunk);
  const I bh = r / chunk;
  const int h = (int)(bh % H);
  const int b = (int)(bh / H);
  int64_t slot;
  if (tok0 + row < sink) {
    slot = tok0 + row;
  } else {
    int64_t x = off0 + row;
    x = x >= window ? x - window : x;
    slot = sink + x;
  }
  const char* src = isv ? v_new + (b * vn0 + h * vn1 + row * vn2) * esize
                        : k_new + (b * kn0 + h * kn1 + row * kn2) * esize;
  char* dst = isv ? v_cache + (b * vc0 + h * vc1 + slot * vc2) * esize
                  : k_cache + (b * kc0 + h * kc1 + slot * kc2) * esize;
  *reinterpret_cast<unit*>(dst + piece * U) = *reinterpret_cast<const unit*>(src + piece * U);
}

hipError_t launch_kv_update(int unit, int esize, const void* k_new, const int64_t* kn_st,
                            const void* v_new, const int64_t* vn_st, void* k_cache,
                            const int64_t* kc_st, void* v_cache, const int64_t* vc_st, int B,
                            int H, int chunk, int Dk, int Dv, int64_t tok0, int64_t sink,
                            int64_t window, hipStream_t s) {
  const int Dmax = Dk > Dv ? Dk : Dv;
  const int64_t n = (int64_t)B * H * chunk * (Dmax * esize / unit);
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256);
  const int64_t off0 = tok0 >= sink ? (tok0 - sink) % window : tok0 - sink;
  const bool narrow = (int64_t)blocks * 256 < ((int64_t)1 << 31);
#define WF_UPD(U, I)                                                                         \
  hipLaunchKernelGGL((kv_update_kernel<U, I>), dim3(blocks, 2), dim3(256), 0, s, esize,      \
                     (const char*)k_new, kn_st[0], kn_st[1], kn_st[2], (const char*)v_new,   \
                     vn_st[0], vn_st[1], vn_st[2], (char*)k_cache, kc_st[0], kc_st[1],       \
                     kc_st[2], (char*)v_cache, vc_st[0], vc_st[1], vc_st[2], B, H, chunk, Dk, \
                     Dv, tok0, sink, window, off0)
  if (narrow) {
    if (unit == 16) WF_UPD(16, int);
    else if (unit == 4) WF_UPD(4, int);
    else WF_UPD(2, int);
  } else {
    if (unit == 16) WF_UPD(16, int64_t);
    else if (unit == 4) WF_UPD(4, int64_t);
    else WF_UPD(2, int64_t);
  }
#undef WF_UPD
  return hipGetLastError();
}

// Writes the visible tokens in chronological order: position p < min(T, sink) is token p;
// the rest are tokens max(sink, T - window) + (p - min(T, sink)).
template <int U>
__global__ __launch_bounds__(256) void kv_gather_kernel(
    int esize, const char* cache, int64_t c0, int64_t c1, int64_t c2, char* out, int64_t o0,
    int64_t o1, int64_t o2, int B, int H, int64_t n_vis, int D, int64_t T, int64_t sink,
    int64_t window) {
  typedef typename CopyUnit<U>::type unit;
  const int per_row = D * esize / U;
  const int64_t n = (int64_t)B * H * n_vis * per_row;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n) return;
  const int piece = (int)(gid % per_row);
  int64_t r = gid / per_row;
  const int64_t p = r % n_vis; r /= n_vis;
  const int h = (int)(r % H);
  const int b = (int)(r / H);
  const int64_t head = T < sink ? T : sink;
  const int64_t start = (T - window) > sink ? (T - window) : sink;
  const int64_t tok = p < head ? p : start + (p - head);
  const int64_t slot = cache_slot(tok, sink, window);
  const char* src = cache + (b * c0 + h * c1 + slot * c2) * esize;
  char* dst = out + (b * o0 + h * o1 + p * o2) * esize;
  *reinterpret_cast<unit*>(dst + piece * U) = *reinterpret_cast<const unit*>(src + piece * U);
}

hipError_t launch_kv_gather(int unit, int esize, const void* cache, const int64_t* c_st, void* out,
                            const int64_t* o_st, int B, int H, int64_t n_vis, int D,
                            int64_t T, int64_t sink, int64_t window, hipStream_t s) {
  const int64_t n = (int64_t)B * H * n_vis * (D * esize / unit);
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256);
#define WF_GAT(U)                                                                            \
  hipLaunchKernelGGL(kv_gather_kernel<U>, dim3(blocks), dim3(256), 0, s, esize,              \
                     (const char*)cache, c_st[0], c_st[1], c_st[2], (char*)out, o_st[0],     \
                     o_st[1], o_st[2], B, H, n_vis, D, T, sink, window)
  if (unit == 16) WF_GAT(16);
  else if (unit == 4) WF_GAT(4);
  else WF_GAT(2);
#undef WF_GAT
  return hipGetLastError();
}

}  // namespace wf
