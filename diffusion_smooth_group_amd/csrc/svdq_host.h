// svdq_host.h -- host-side helpers of the library (pack, SVD, number formats).
#pragma once
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>

namespace svdq {

int host_threads();
void parallel_for(int64_t n, const std::function<void(int64_t, int64_t)>& f);

// Top-r eigenpairs of a symmetric s x s matrix (Lanczos), descending.
bool lanczos_top(const double* G, int64_t s, int r, double* theta, double* Y, int* steps_out);
// Rank-r truncated SVD of A (K x N row-major): L1 = U_r S_r (K x r),
// L2 = V_r^T (r x N), sigma[r].
bool truncated_svd(const double* A, int64_t K, int64_t N, int r, double* L1, double* L2, double* sigma);

// ---- IEEE number formats (bit exact, round to nearest even) ----
inline uint32_t f2u(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
inline float u2f(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

inline float f16_to_f32(uint16_t h) {
  uint32_t s = uint32_t(h & 0x8000) << 16, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  if (e == 0x1F) return u2f(s | 0x7F800000u | (m << 13));
  if (e == 0) {                       // zero or subnormal: m * 2^-24, exact in fp32
    float v = float(m) * 5.9604644775390625e-08f;
    return s ? -v : v;
  }
  return u2f(s | ((e + 112) << 23) | (m << 13));
}
inline float bf16_to_f32(uint16_t b) { return u2f(uint32_t(b) << 16); }
inline float h16_to_f32(uint16_t v, int dtype) { return dtype == 1 ? bf16_to_f32(v) : f16_to_f32(v); }

inline uint16_t f32_to_f16_rne(float f) {
  uint32_t x = f2u(f);
  uint16_t sign = uint16_t((x >> 16) & 0x8000);
  x &= 0x7FFFFFFFu;
  if (x >= 0x7F800000u) return sign | (x > 0x7F800000u ? 0x7E00 : 0x7C00);
  if (x >= 0x477FF000u) return sign | 0x7C00;               // >= 65520 rounds to inf
  if (x < 0x38800000u) {                                     // below 2^-14: subnormal
    float a = u2f(x) * 16777216.0f;                          // exact: times 2^24
    return sign | uint16_t(std::nearbyint(a));               // half-even, 0..1024
  }
  uint32_t exp = (x >> 23) - 112, mant = x & 0x7FFFFFu;
  uint32_t base = (exp << 10) | (mant >> 13), rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (base & 1u))) ++base;
  return sign | uint16_t(base);
}

inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// float64 -> 16-bit, one rounding (no intermediate fp32).
inline uint16_t f64_to_h16_rne(double x, int dtype) {
  const int p = dtype == 1 ? 8 : 11, emin = dtype == 1 ? -126 : -14;
  const double vmax = dtype == 1 ? 3.3895313892515355e+38 : 65504.0;
  if (std::isnan(x)) return dtype == 1 ? 0x7FC0 : 0x7E00;
  double r;
  if (x == 0.0 || std::isinf(x)) {
    r = x;
  } else {
    int e2;
    std::frexp(std::fabs(x), &e2);
    int e = std::max(e2 - 1, emin);
    double q = std::ldexp(1.0, e - (p - 1));
    r = std::nearbyint(std::fabs(x) / q) * q;
    if (r > vmax) r = INFINITY;
    r = std::copysign(r, x);
  }
  float rf = float(r);                 // exact: r is representable in the 16-bit format
  return dtype == 1 ? uint16_t(f2u(rf) >> 16) : f32_to_f16_rne(rf);
}

// ---- group quantizers (same rules as the GPU activation kernel) ----
// INT4 g64: s = fp16(min(fl32(max|v|/7), 65504)); q = clamp(rint(fl32(v/s)), -7, 7).
inline void quant_int4_group(const float* v, int8_t* q, uint16_t* s_bits) {
  float m = 0.0f;
  for (int i = 0; i < 64; ++i) m = std::fmax(m, std::fabs(v[i]));
  float s = m / 7.0f;
  s = std::fmin(s, 65504.0f);
  uint16_t sh = f32_to_f16_rne(s);
  float s32 = f16_to_f32(sh);
  *s_bits = sh;
  for (int i = 0; i < 64; ++i) {
    if (s32 == 0.0f) { q[i] = 0; continue; }
    float r = std::nearbyint(v[i] / s32);
    r = std::fmin(std::fmax(r, -7.0f), 7.0f);
    q[i] = std::isnan(r) ? 0 : int8_t(r);
  }
}

// INT8, one scale for a whole row of L values (an output channel of R):
// s = fl32(max|v| / 127), q = clamp(rint(fl32(v / s)), -127, 127), 0 if s == 0.
inline void quant_int8_row(const float* v, int64_t L, int8_t* q, float* s_out) {
  float m = 0.0f;
  for (int64_t i = 0; i < L; ++i) m = std::fmax(m, std::fabs(v[i]));
  const float s = m / 127.0f;
  *s_out = s;
  for (int64_t i = 0; i < L; ++i) {
    if (s == 0.0f) { q[i] = 0; continue; }
    float r = std::nearbyint(v[i] / s);
    r = std::fmin(std::fmax(r, -127.0f), 127.0f);
    q[i] = std::isnan(r) ? 0 : int8_t(r);
  }
}

// E2M1 magnitude index of a >= 0, nearest with ties to even, saturating at 6.
inline uint32_t e2m1_index(float a) {
  return uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
         uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
}

// MXFP4 g32: e = smallest biased exponent with 2^(e-127) >= fl32(max|v|/6)
// (0 for an all-zero group, <= 254); code = sign | E2M1(v * 2^(127-e)).
inline void quant_mx_group(const float* v, uint8_t* c, uint8_t* e_out) {
  float m = 0.0f;
  for (int i = 0; i < 32; ++i) m = std::fmax(m, std::fabs(v[i]));
  float t = m / 6.0f;
  uint32_t tb = f2u(t);
  int e = int((tb >> 23) & 0xFF) + ((tb & 0x7FFFFFu) != 0 ? 1 : 0);
  if (t == 0.0f) e = 0;
  if (e > 254) e = 254;
  *e_out = uint8_t(e);
  for (int i = 0; i < 32; ++i) {
    float u = std::ldexp(v[i], 127 - e);
    uint32_t idx = e2m1_index(std::fabs(u));
    c[i] = uint8_t(idx | (std::signbit(v[i]) ? 8u : 0u));
  }
}

}  // namespace svdq
