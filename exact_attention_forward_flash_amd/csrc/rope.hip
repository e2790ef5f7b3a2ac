// Rotary position embedding of the queries and keys on their way into attention (WorldFoundry
// "Core 注意力": applying RoPE is one of the core's jobs; the page gives no convention). The
// first rot dims of every head turn pairwise by caller-tabulated angles: pair i of a row at
// position p turns by cos[p][i], sin[p][i]; pairs are (i, i + rot/2) ("rotate-half") or
// (2i, 2i + 1) ("interleaved"); dims past rot are copied.
//
// One launch rotates Q and K (blockIdx.y picks the tensor) into contiguous copies that the
// attention kernels then read. The rotation is not done on the attention kernels' K loads:
// every K tile is read by every query tile and every wave of a work group there, so turning it
// on load would redo ~2 FMAs per element per wave per tile in a loop that is already bound by
// its VALU work, while this pass reads and writes Q and K once (bound by HBM).
#include "wf_internal.hpp"

namespace wf {

template <typename T>
struct RopeSeg {
  const T* x;            // input [B, H, L, D], strides in elements
  int64_t sb, sh, sm;
  T* y;                  // output, contiguous [B, H, L, D]
  int H, L;
  int64_t pos0;
  int64_t chunks;        // B * H * L * slots per row
};

// A row is cut into slots of 16 bytes of output: rotate-half, slot u < rot/16 turns the pair
// of chunks (8u, 8u + rot/2) (each element read once; rot % 16 == 0 keeps both chunks
// aligned); interleaved, slot u < rot/8 turns the 4 pairs inside chunk u; the remaining slots
// copy the chunks past rot.
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(RopeSeg<T> s0, RopeSeg<T> s1, int D, int rot,
                                                   int style, const float* __restrict__ cosb,
                                                   const float* __restrict__ sinb) {
  const RopeSeg<T>& s = blockIdx.y == 0 ? s0 : s1;
  const int nrot = style == 0 ? rot / 16 : rot / 8;      // rotating slots per row
  const int spr = nrot + (D - rot) / 8;                  // slots per row
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= s.chunks) return;
  const int64_t row = t / spr;
  const int u = (int)(t % spr);
  const int l = (int)(row % s.L);
  const int64_t bh = row / s.L;
  const int h = (int)(bh % s.H);
  const int64_t b = bh / s.H;
  const T* xr = s.x + b * s.sb + h * s.sh + (int64_t)l * s.sm;
  T* yr = s.y + row * D;
  typedef T t8 __attribute__((ext_vector_type(8)));
  if (u >= nrot) {                                       // past rot: copy
    const int e0 = rot + (u - nrot) * 8;
    *reinterpret_cast<t8*>(yr + e0) = *reinterpret_cast<const t8*>(xr + e0);
    return;
  }
  const int half = rot / 2;
  const float* cr = cosb + (s.pos0 + l) * half;
  const float* sr = sinb + (s.pos0 + l) * half;
  if (style == 0) {
    const int i0 = u * 8;                                // pairs i0 .. i0 + 7
    const t8 xa = *reinterpret_cast<const t8*>(xr + i0);
    const t8 xb = *reinterpret_cast<const t8*>(xr + i0 + half);
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(cr + i0), c1 = *reinterpret_cast<const f32x4*>(cr + i0 + 4);
    const f32x4 n0 = *reinterpret_cast<const f32x4*>(sr + i0), n1 = *reinterpret_cast<const f32x4*>(sr + i0 + 4);
    t8 ya, yb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = e < 4 ? c0[e] : c1[e - 4];
      const float sn = e < 4 ? n0[e] : n1[e - 4];
      const float a = (float)xa[e], bb = (float)xb[e];
      ya[e] = (T)fmaf(a, c, -bb * sn);
      yb[e] = (T)fmaf(bb, c, a * sn);
    }
    *reinterpret_cast<t8*>(yr + i0) = ya;
    *reinterpret_cast<t8*>(yr + i0 + half) = yb;
  } else {
    const int e0 = u * 8, i0 = u * 4;                    // 4 pairs inside the chunk
    const t8 xv = *reinterpret_cast<const t8*>(xr + e0);
    const f32x4 c4 = *reinterpret_cast<const f32x4*>(cr + i0);
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(sr + i0);
    t8 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = (float)xv[2 * i], bb = (float)xv[2 * i + 1];
      out[2 * i] = (T)fmaf(a, c4[i], -bb * s4[i]);
      out[2 * i + 1] = (T)fmaf(bb, c4[i], a * s4[i]);
    }
    *reinterpret_cast<t8*>(yr + e0) = out;
  }
}

template <typename T>
static hipError_t launch_t(const RopeDesc& q, const RopeDesc& k, int D, int rot, int style,
                           const float* cosb, const float* sinb, hipStream_t st) {
  auto seg = [&](const RopeDesc& d) {
    RopeSeg<T> r;
    r.x = (const T*)d.x; r.sb = d.sb; r.sh = d.sh; r.sm = d.sm; r.y = (T*)d.y;
    r.H = d.H; r.L = d.L; r.pos0 = d.pos0;
    const int spr = (style == 0 ? rot / 16 : rot / 8) + (D - rot) / 8;
    r.chunks = (int64_t)d.B * d.H * d.L * spr;           // slots
    return r;
  };
  const RopeSeg<T> a = seg(q), b = seg(k);
  const int64_t n = a.chunks > b.chunks ? a.chunks : b.chunks;
  const int64_t blocks = (n + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_kernel<T>, dim3((unsigned)blocks, 2), dim3(256), 0, st, a, b, D, rot,
                     style, cosb, sinb);
  return hipGetLastError();
}

hipError_t launch_rope(int dtype, const RopeDesc& q, const RopeDesc& k, int D, int rot, int style,
                       const float* cosb, const float* sinb, hipStream_t st) {
  if (dtype == DT_BF16) return launch_t<__bf16>(q, k, D, rot, style, cosb, sinb, st);
  if (dtype == DT_F16) return launch_t<_Float16>(q, k, D, rot, style, cosb, sinb, st);
  return launch_t<float>(q, k, D, rot, style, cosb, sinb, st);
}

}  // namespace wf
