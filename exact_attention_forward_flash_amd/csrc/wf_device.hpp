// Device-side building blocks shared by the gfx950 kernels: vector types, MFMA wrappers,
// LDS transpose reads, cross-half-wave exchange, direct global->LDS copies.
//
// Lane layouts used throughout (wave64, measured on gfx950):
//   v_mfma_f32_32x32x16_{bf16,f16}: A[i][k] comes from lane i + 32*(k/8), element k%8;
//     B[k][j] from lane j + 32*(k/8), element k%8; accumulator element r of lane l holds
//     D[8*(r/4) + 4*(l/32) + r%4][l%32].
//   v_mfma_f32_32x32x2_f32: A[i][k] from lane i + 32*k; B[k][j] from lane j + 32*k; same
//     accumulator layout.
//   ds_read_b64_tr_b16: inside each group of 16 lanes, source lane s names an 8-byte row
//     piece; destination lane t receives element t%4 of the pieces named by lanes
//     4e + t/4, e = 0..3.
//   v_permlane32_swap(x, x): lanes < 32 get (x[l], x[l+32]), lanes >= 32 get
//     (x[l-32], x[l]).
//   global_load_lds_dwordx4: lane l's 16 bytes land at the (wave-uniform) LDS base + 16*l.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define WF_LDS __attribute__((address_space(3)))

template <typename T> struct Mfma16;
template <> struct Mfma16<__bf16> {
  typedef bf16x8 v8;
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8, a),
                                                   __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma16<_Float16> {
  typedef f16x8 v8;
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8, a),
                                                  __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
};

// Round 8 fp32 values to the 16-bit type (nearest even) and pack them as an MFMA operand.
template <typename T>
__device__ __forceinline__ u32x4 pack8(const f32x16& p, int off) {
  typedef typename Mfma16<T>::v8 v8;
  v8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (T)p[off + e];
  return __builtin_bit_cast(u32x4, r);
}

__device__ __forceinline__ float xhalf_max(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 lds_read16(const WF_LDS char* p) {
  return *reinterpret_cast<const WF_LDS u32x4*>(p);
}
__device__ __forceinline__ u32x2 lds_read_tr(const WF_LDS char* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 WF_LDS*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ void dma16(const void* g, WF_LDS char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (WF_LDS void*)lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory loads of this wave are outstanding (they complete in
// issue order): everything but the N most recent.
template <int N>
__device__ __forceinline__ void wait_vmem_n() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__device__ __forceinline__ bool wave_any(bool x) { return __builtin_amdgcn_ballot_w64(x) != 0; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of the 8 16-bit values packed in x, accumulated into acc (fp32): v_dot2c with (1, 1).
// Written out because the compiler's fdot2 builtins, applied to the elements of a vector in
// turn, were seen to read the first element for all of them. A dot2c result may feed the
// next dot2c's accumulator at once, but an ordinary VALU read of it needs 3 wait states
// first (the caller issues them).
template <typename T>
__device__ __forceinline__ float sum8_acc(u32x4 x, float acc);
template <>
__device__ __forceinline__ float sum8_acc<__bf16>(u32x4 x, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) asm("v_dot2c_f32_bf16 %0, 0x3f803f80, %1" : "+v"(acc) : "v"(x[i]));
  return acc;
}
template <>
__device__ __forceinline__ float sum8_acc<_Float16>(u32x4 x, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) asm("v_dot2c_f32_f16 %0, 0x3c003c00, %1" : "+v"(acc) : "v"(x[i]));
  return acc;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace wf
