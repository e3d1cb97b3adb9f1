// Device helpers shared by the connector's gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define IVC_DEV __device__ __forceinline__

typedef uint16_t bf16_t;  // bfloat16 storage
// Native 16-byte vector (HIP's uint4 struct makes arrays of it spill to scratch).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- element conversions ---------------------------------------------------
IVC_DEV float bf16_to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest even; NaN stays a quiet NaN.
IVC_DEV bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename E> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  IVC_DEV static float load(const float* p) { return *p; }
  IVC_DEV static float to_f(float v) { return v; }
  IVC_DEV static float from_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPerVec = 8;
  IVC_DEV static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  IVC_DEV static float to_f(bf16_t v) { return bf16_to_f32(v); }
  IVC_DEV static bf16_t from_f(float v) { return f32_to_bf16(v); }
};

// Unpack a 16-byte vector of E into floats (kPerVec of them).
IVC_DEV void unpack16(const u32x4& v, float* f, float*) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
IVC_DEV void unpack16(const u32x4& v, float* f, bf16_t*) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}
template <typename E> IVC_DEV void unpack(const u32x4& v, float* f) { unpack16(v, f, (E*)nullptr); }

IVC_DEV u32x4 pack16(const float* f, float*) {
  u32x4 v;
  v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
  v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
  return v;
}
IVC_DEV u32x4 pack16(const float* f, bf16_t*) {
  u32x4 v;
  v.x = (uint32_t)f32_to_bf16(f[0]) | ((uint32_t)f32_to_bf16(f[1]) << 16);
  v.y = (uint32_t)f32_to_bf16(f[2]) | ((uint32_t)f32_to_bf16(f[3]) << 16);
  v.z = (uint32_t)f32_to_bf16(f[4]) | ((uint32_t)f32_to_bf16(f[5]) << 16);
  v.w = (uint32_t)f32_to_bf16(f[6]) | ((uint32_t)f32_to_bf16(f[7]) << 16);
  return v;
}
template <typename E> IVC_DEV u32x4 pack(const float* f) { return pack16(f, (E*)nullptr); }

// ---- write-through stores ---------------------------------------------------
// For data that workgroups of one launch hand to each other across XCDs:
// relaxed device-scope atomic stores, which the memory system performs at
// the device's coherence point (nothing left behind in one XCD's L2).
IVC_DEV void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
IVC_DEV void st_coh4(float* p, float4 v) {
  unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
  __hip_atomic_store(q, (unsigned long long)__float_as_uint(v.x) |
                            ((unsigned long long)__float_as_uint(v.y) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, (unsigned long long)__float_as_uint(v.z) |
                                ((unsigned long long)__float_as_uint(v.w) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- XCD-aware workgroup order ------------------------------------------------
// The dispatcher deals workgroups to the 8 XCDs in turn (linear id i runs on
// XCD i % 8), each XCD with its own L2.  This renumbers the n workgroups of
// a launch so that XCD k runs the consecutive range [k n/8, (k+1) n/8): work
// items with nearby numbers, which share operands, then share one L2.  (n
// not a multiple of 8: unchanged.)
IVC_DEV int xcd_major(int i, int n) { return (n & 7) ? i : (i & 7) * (n >> 3) + (i >> 3); }

// ---- wavefront reductions (64 lanes) ---------------------------------------
IVC_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
IVC_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---- moments (mean, sum of squared deviations) of equal-sized groups -------
// Two groups of n values each, (mean a.x, M2 a.y) and (b.x, b.y), combined
// (Chan, Golub and LeVeque's pairwise update with n_a = n_b = n):
//   mean = (a.x + b.x) / 2,  M2 = a.y + b.y + (a.x - b.x)^2 * n / 2.
// half_n = n / 2.  The result depends on the operand order only through
// a.y + b.y and a.x + b.x, both commutative.
IVC_DEV float2 moments_pair(float2 a, float2 b, float half_n) {
  const float d = a.x - b.x;
  return make_float2((a.x + b.x) * 0.5f, fmaf(d * d, half_n, a.y + b.y));
}

// GELU, 0.5 x (1 + erf(x / sqrt 2)), with erf by the approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.28
// (absolute error <= 3e-7):
//   erf(u) = sign(u) (1 - r),  r = 1 / P(|u|)^16,
//   P(v) = 1 + a1 v + a2 v^2 + ... + a6 v^6.
// Then GELU(x) = max(x, 0) - 0.5 |x| r with u = x / sqrt 2, and P(|x| / sqrt 2)
// is a polynomial in |x| whose coefficient k is a_k 2^(-k/2).  One reciprocal,
// no exponential (7.1.26 needs both), the 16th power by four squarings;
// large |x| overflows the power to inf, giving r = 0 (the |x| that r
// multiplies is capped at 1e30, so GELU(+inf) = +inf; NaN stays NaN, and
// GELU(-inf) is NaN, as 0.5 x (1 + erf) gives).  Absolute error <= 1e-6 in
// fp32, far below the bf16 rounding of the outputs.  Branch-free: a library
// erf branches per range, which costs the GEMM epilogues dearly when the
// lanes of a wave fall in different ranges.
IVC_DEV float gelu_erf(float x) {
  const float ax = fabsf(x);
  float p = fmaf(5.3829750000e-06f, ax, 4.8890635643e-05f);
  p = fmaf(p, ax, 3.8003575000e-05f);
  p = fmaf(p, ax, 3.2776263241e-03f);
  p = fmaf(p, ax, 2.1141006150e-02f);
  p = fmaf(p, ax, 4.9867346967e-02f);
  p = fmaf(p, ax, 1.0f);
  p = p * p;
  p = p * p;
  p = p * p;
  p = p * p;
  // max(x, 0) as x - min(x, 0): a NaN x passes through (fmaxf would drop it)
  return fmaf(-0.5f * fminf(ax, 1e30f), __builtin_amdgcn_rcpf(p), x - fminf(x, 0.0f));
}
