// RMSNorm and partial RoPE of rows held 8 channels per lane, shared by the pooling epilogue
// and the row kernel.
//
// Sources: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section IV (both branches
// normalise the queries and the compressed KV entries and rotate only the last 64
// dimensions); the MLA walk-through's "The Code: RoPE Helpers" (consecutive pairs read as
// complex numbers, multiplied by e^{i pos f_i}, f_i = theta^(-2i/d)).  RMSNorm is the usual
// y = x / sqrt(mean(x^2) + eps) * gamma.
#pragma once

#include "common.hpp"

namespace csahca {

constexpr int VEC = 8;  // channels per lane

template <typename T>
struct Vec8;

template <>
struct Vec8<uint16_t> {
  u32x4 raw;
  CSAHCA_DEV void load(const uint16_t* p) { raw = *reinterpret_cast<const u32x4*>(p); }
  CSAHCA_DEV void put(uint16_t* p) const { *reinterpret_cast<u32x4*>(p) = raw; }
  CSAHCA_DEV float get(int i) const {
    uint32_t w = raw[i >> 1];
    return (i & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  }
  static CSAHCA_DEV void store(uint16_t* p, const float* v) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = o;
  }
};

template <>
struct Vec8<float> {
  f32x4 a, b;
  CSAHCA_DEV void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  CSAHCA_DEV void put(float* p) const {
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
  }
  CSAHCA_DEV float get(int i) const { return i < 4 ? a[i] : b[i - 4]; }
  static CSAHCA_DEV void store(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};

// What to apply to a row of c channels: RMSNorm (when `norm`) with gain `gamma` ([c] fp32,
// NULL for unit gain), then RoPE on the last `d` channels (d % 8 == 0, 0 = none).
struct NormRope {
  const float* gamma;
  float eps;
  float theta;
  int d;
  int norm;
};

// Sum over the CV consecutive lanes that hold one row (CV a power of two, at most 64,
// groups aligned to CV lanes).
CSAHCA_DEV float row_sum(float v, int CV) {
  for (int o = 1; o < CV; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// cos and sin of pos * f for a rotation frequency f given in double.  The angle is formed
// in double (positions reach 2^20 and more, where a float angle would be off by a sizeable
// fraction of a radian) and reduced by multiples of pi/2 in double (Cody-Waite, pi/2 split
// into two doubles), leaving |x| <= pi/4 and the quadrant.  On that interval the Taylor
// series of sin to x^9 and of cos to x^10 are within 2e-9 of the functions, below half a
// float ulp, so they are evaluated in float by Horner's rule; the quadrant then swaps and
// negates.  (A short, branch-free sequence: the attention kernel runs it with most of its
// registers holding accumulators.)
CSAHCA_DEV void rope_cos_sin(long long pos, double f, float& cs, float& sn) {
  const double a = (double)pos * f;
  const double k = rint(a * 0.6366197723675814);       // 2 / pi
  double r = fma(-k, 1.5707963267948966, a);            // pi/2, high part
  r = fma(-k, 6.123233995736766e-17, r);                // pi/2, low part
  const float x = (float)r, x2 = x * x;
  const float s = x * fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, 1.f / 362880.f, -1.f / 5040.f), 1.f / 120.f),
                                    -1.f / 6.f),
                           1.f);
  const float c = fmaf(x2,
                       fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, -1.f / 3628800.f, 1.f / 40320.f), -1.f / 720.f),
                                     1.f / 24.f),
                            -0.5f),
                       1.f);
  const int q = (int)((long long)k & 3);
  const float s1 = (q & 1) ? c : s, c1 = (q & 1) ? s : c;
  sn = (q & 2) ? -s1 : s1;
  cs = ((q + 1) & 2) ? -c1 : c1;
}

// Frequency of rotated pair i: theta^(-2i/d) = 2^(-2i log2(theta) / d), in double.
CSAHCA_DEV double rope_freq(int i, int d, float theta) {
  return exp2(-2.0 * (double)i * log2((double)theta) / (double)d);
}

// Rotate (a, b) = (x[2i], x[2i+1]) by the angle whose cos and sin are given.
CSAHCA_DEV void rope_apply(float& a, float& b, float cs, float sn) {
  const float a2 = a * cs - b * sn;
  const float b2 = a * sn + b * cs;
  a = a2;
  b = b2;
}

CSAHCA_DEV void rope_rotate(float& a, float& b, long long pos, int i, int d, float theta) {
  float cs, sn;
  rope_cos_sin(pos, rope_freq(i, d, theta), cs, sn);
  rope_apply(a, b, cs, sn);
}

// Gains of channels ch0 .. ch0+7 (1 without a gain vector), loaded as two 16-byte vectors;
// callers issue this early so that the load overlaps their own.
CSAHCA_DEV void load_gain8(const NormRope& nr, int ch0, float (&g)[VEC]) {
  if (nr.gamma) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(nr.gamma + ch0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(nr.gamma + ch0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g[e] = a[e];
      g[4 + e] = b[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) g[e] = 1.f;
  }
}

// Channels ch0 .. ch0+7 of a row whose c channels are spread over CV consecutive lanes;
// g holds their gains (load_gain8).
CSAHCA_DEV void norm_rope8(float (&v)[VEC], const float (&g)[VEC], int ch0, int CV, int c,
                           const NormRope& nr, long long pos) {
  if (nr.norm) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) ss = fmaf(v[e], v[e], ss);
    ss = row_sum(ss, CV);
    const float inv = 1.0f / sqrtf(ss / (float)c + nr.eps);
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] *= inv * g[e];
  }
  const int P = nr.d / 2;  // rotated pairs
  if (P == 0) return;
  if (P <= CV) {
    // one angle per lane: lane li of the row's group forms the cos and sin of pair li,
    // and the lanes holding the rotated channels fetch their four pairs
    const int li = (int)(threadIdx.x & (CV - 1)), base = (int)(threadIdx.x & 63) & ~(CV - 1);
    float cs = 1.f, sn = 0.f;
    if (li < P) rope_cos_sin(pos, rope_freq(li, nr.d, nr.theta), cs, sn);
    const int i0 = (ch0 - (c - nr.d)) / 2;  // negative outside the rotated channels
#pragma unroll
    for (int q = 0; q < VEC / 2; ++q) {
      const int src = base + min(max(i0 + q, 0), P - 1);
      const float cq = __shfl(cs, src, 64), sq = __shfl(sn, src, 64);
      if (i0 >= 0) rope_apply(v[2 * q], v[2 * q + 1], cq, sq);
    }
  } else if (ch0 >= c - nr.d) {
    // the lane's four pairs: f_{i0+q} = f_{i0} * step^q, step = theta^(-2/d)
    const int i0 = (ch0 - (c - nr.d)) / 2;
    const double l2t = log2((double)nr.theta);
    double f = exp2(-2.0 * (double)i0 * l2t / (double)nr.d);
    const double step = exp2(-2.0 * l2t / (double)nr.d);
#pragma unroll
    for (int q = 0; q < VEC / 2; ++q) {
      float cs, sn;
      rope_cos_sin(pos, f, cs, sn);
      rope_apply(v[2 * q], v[2 * q + 1], cs, sn);
      f *= step;
    }
  }
}

// One row's channels cv*8 .. cv*8+7 (the row's c channels held by CV consecutive lanes):
// loaded from x_row, normalised and rotated at position `pos`, rounded once and stored to
// y_row.  Every lane of the row's group calls it (the mean square is a lane sum).
template <typename T>
CSAHCA_DEV void norm_rope_row8(const T* x_row, T* y_row, const NormRope& nr, long long pos, int cv,
                               int CV, int c) {
  Vec8<T> v;
  v.load(x_row + cv * VEC);  // the row and its gains load together
  float g[VEC];
  load_gain8(nr, cv * VEC, g);
  float f[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) f[e] = v.get(e);
  norm_rope8(f, g, cv * VEC, CV, c, nr, pos);
  Vec8<T>::store(y_row + cv * VEC, f);
}

// Host-side check shared by the entry points that take a NormRope.
inline bool norm_rope_args_ok(int c, int d, float eps, float theta) {
  const int CV = c / VEC;
  return c % VEC == 0 && CV >= 1 && CV <= 64 && (CV & (CV - 1)) == 0 && d >= 0 && d <= c &&
         d % 8 == 0 && eps >= 0.f && eps < 1e30f && theta > 0.f && theta < 1e30f;
}

}  // namespace csahca
