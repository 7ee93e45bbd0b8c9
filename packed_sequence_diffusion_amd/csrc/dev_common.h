// Device-side helpers shared by the block's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
// Native 16-byte vector for register staging of tiles (HIP's uint4 is a
// class with a union, which keeps arrays of it out of registers).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

#define DIT_DEV __device__ __forceinline__

DIT_DEV float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32).
DIT_DEV bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

// Two floats -> two packed bfloat16 (low = a).
DIT_DEV uint32_t pack2bf(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Streaming accesses (non-temporal: no allocation in the caches) for data a
// kernel touches once, such as the rows of a bandwidth-bound row kernel.
DIT_DEV float4 ld4_stream(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load((const f32x4_t*)p);
  return make_float4(v[0], v[1], v[2], v[3]);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  static DIT_DEV float ld(const float* p) { return *p; }
  static DIT_DEV void st(float* p, float v) { *p = v; }
  // four consecutive elements
  static DIT_DEV float4 ld4(const float* p) { return *(const float4*)p; }
  static DIT_DEV void st4(float* p, float4 v) { *(float4*)p = v; }
  static DIT_DEV void st4_stream(float* p, float4 v) {
    const f32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (f32x4_t*)p);
  }
};
template <> struct Elt<bf16_t> {
  static DIT_DEV float ld(const bf16_t* p) { return bf2f(*p); }
  static DIT_DEV void st(bf16_t* p, float v) { *p = f2bf(v); }
  static DIT_DEV float4 ld4(const bf16_t* p) {
    uint2 u = *(const uint2*)p;
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  static DIT_DEV void st4(bf16_t* p, float4 v) {
    *(uint2*)p = make_uint2(pack2bf(v.x, v.y), pack2bf(v.z, v.w));
  }
  static DIT_DEV void st4_stream(bf16_t* p, float4 v) {
    const u32x2_t w = {pack2bf(v.x, v.y), pack2bf(v.z, v.w)};
    __builtin_nontemporal_store(w, (u32x2_t*)p);
  }
};

// Sum over each 32-lane half of the wave, left in every lane of that half:
// DPP exchanges inside rows of 16 lanes (quad_perm [1,0,3,2] and [2,3,0,1],
// then row_ror by 4 and 8), then one ds_swizzle that swaps the two rows of
// the half (bitmask mode, xor 16).
#define DIT_DPP(v_, ctrl_) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v_), (ctrl_), 0xF, 0xF, false))
DIT_DEV float sum32(float v) {
  v += DIT_DPP(v, 0xB1);   // quad_perm [1,0,3,2]
  v += DIT_DPP(v, 0x4E);   // quad_perm [2,3,0,1]
  v += DIT_DPP(v, 0x124);  // row_ror:4
  v += DIT_DPP(v, 0x128);  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // lane ^ 16
  return v;
}

DIT_DEV float wave_sum(float v) {
  v = sum32(v);
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

DIT_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// max / sum of a value and its copy in the other 32-lane half of the wave
// (lane l and lane l ^ 32), with gfx950's v_permlane32_swap: swapping the
// upper half of one copy with the lower half of another leaves, in every lane,
// the pair {x[l], x[l ^ 32]}.
DIT_DEV float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
DIT_DEV float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The reciprocals below are v_rcp_f32 (about one ulp) rather than an IEEE
// division (a ten-instruction sequence): these feed GEMM epilogues whose
// results are rounded to bf16, or checked at 1e-5 on the fp32 path.  At the
// extremes exp overflows to +inf and rcp(inf) = 0, the limits of the functions.
DIT_DEV float rcp_f(float v) { return __builtin_amdgcn_rcpf(v); }

DIT_DEV float silu_f(float v) { return v * rcp_f(1.0f + __expf(-v)); }

// Tanh-form GELU; tanh(u) = 1 - 2 / (exp(2u) + 1).
DIT_DEV float gelu_tanh_f(float v) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  float u = k0 * (v + 0.044715f * v * v * v);
  float t = 1.0f - 2.0f * rcp_f(__expf(2.0f * u) + 1.0f);
  return 0.5f * v * (1.0f + t);
}

DIT_DEV float tanh_f(float u) { return 1.0f - 2.0f * rcp_f(__expf(2.0f * u) + 1.0f); }
