// Device code shared by the quantize kernels (nq_kernels.hip) and the fp64
// pass (nq_exact.hip): fp16 conversions and the nearest-codeword decoders.
//
// Pages: NexusQuant blog, E8 walkthrough post, "The Conway-Sloane
// Nearest-Point Algorithm" (round to each coset, fix the parity by moving
// the worst-rounded coordinate, keep the closer candidate) and "The Relaxed
// Parity Discovery" (strict E8 vs the relaxed half-integer coset).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

namespace nq {

// Decisions of the fp32 decoders whose margin -- the squared-distance gap
// between the chosen codeword and the next best one, in units of g = 2y --
// falls below this value are re-taken from y computed in fp64.  In units of
// y it is 1.6e-5: the fp32 computation of y (RoPE removal, Walsh-Hadamard,
// scale) stays within 1.5e-6 of the fp64 value per coordinate on the
// benchmarked caches, so a competitor at lattice distance sqrt(2) can gain
// at most about 6e-6 on the chosen codeword from those errors.
constexpr float kNearTie = 6.4e-5f;

__device__ __forceinline__ float h2f(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}
__device__ __forceinline__ uint16_t f2h_rn(float f) {
  return __half_as_ushort(__float2half_rn(f));
}

// fp64 -> fp16 with a single rounding to nearest-even: round to odd into
// fp32 first (24 bits >= 11 + 2), then round to nearest-even into fp16.
__device__ __forceinline__ uint16_t f64_to_f16_rn(double x) {
  float f = (float)x;
  const double back = (double)f;
  if (back != x) {
    uint32_t b = __float_as_uint(f);
    if (fabs(back) > fabs(x)) b -= 1u;
    b |= 1u;
    f = __uint_as_float(b);
  }
  return f2h_rn(f);
}

// Spread the low 8 bits of x to the even bits of a 16-bit word.
__device__ __forceinline__ uint32_t spread8(uint32_t x) {
  x &= 0xffu;
  x = (x | (x << 4)) & 0x0f0fu;
  x = (x | (x << 2)) & 0x3333u;
  x = (x | (x << 1)) & 0x5555u;
  return x;
}

// (x << n) | (the top n bits of w): v_alignbit_b32
__device__ __forceinline__ uint32_t shift_in(uint32_t x, float w, int n) {
  return __builtin_amdgcn_alignbit(x, __float_as_uint(w), (uint32_t)(32 - n));
}

// cos and sin of the angle p * omega (position times RoPE frequency): the
// angle is formed and reduced to [-pi, pi] in fp64 (2 pi as a two-term
// constant), then the reduced angle is rounded once to fp32 for an fp32
// sincos: both to about one fp32 ulp.  The RoPE table and the kernels that
// form their own rows use this one routine, so their values are identical.
__device__ __forceinline__ void rope_cos_sin(double p, double omega, float& c, float& s) {
  const double ang = p * omega;
  const double n = rint(ang * 0.15915494309189535);
  double r = fma(-n, 6.283185307179586, ang);
  r = fma(-n, 2.4492935982947064e-16, r);
  sincosf((float)r, &s, &c);
}

// The median of three: with b the largest (smallest) and s the second
// largest (smallest) of the values seen so far, median3(b, s, x) is the
// second largest (smallest) once x joins them.  One v_med3_f32 in fp32.
__device__ __forceinline__ float median3(float b, float s, float x) {
  return __builtin_amdgcn_fmed3f(b, s, x);
}
__device__ __forceinline__ double median3(double b, double s, double x) {
  return fmax(fmin(b, s), fmin(fmax(b, s), x));
}
__device__ __forceinline__ uint32_t median3u(uint32_t b, uint32_t s, uint32_t x) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(s), "v"(x));
  return r;
}

// Nearest codeword of the b-bit cube codebook for one 8-group, in fp32 or
// fp64 (F).
//
// Works on g = 2y (exact) and a = |g|: with f = floor(a), the nearest even
// integer to a is f + (f & 1) and the nearest odd one is f | 1 (ties away
// from zero), clamped to the cube (L-2 resp. L-1 in these doubled units).
// The parity step moves the coordinate with the largest "kappa" (|delta| if
// the step toward y stays in the cube, -|delta| if it has to go away) by two;
// its extra squared cost is 4 - 4 kappa, which is also what switching any one
// coordinate to its other neighbour costs.  The closer coset wins, the
// integer coset on ties.  Output: b-bit codes idx = p + L/2 - c/2 packed
// little endian, and the coset bit c.
//
// margin (when non-null): the gap to the next best codeword, in g^2 units.
// Inside a coset it is set by the two cheapest single switches k1 <= k2:
// with the parity step taken, k2 - k1; without one, k1 + k2; on the relaxed
// half coset (no parity) k1.  Across cosets it is |D1 - D0|.
template <int BITS, bool STRICT, typename F>
__device__ __forceinline__ void e8_decode(const F y[8], uint32_t& code, int& coset,
                                          F* margin) {
  constexpr int L = 1 << BITS;
  int P0[8], P1[8];
  F d0[8], d1[8];
  int neg[8];
  F D0 = 0, D1 = 0;
  int S0 = 0, S1 = 0, NS = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const F g = y[k] + y[k];
    neg[k] = signbit(g) ? 1 : 0;
    const F a = fabs(g);
    const int fi = (int)floor(a);
    P0[k] = min(fi + (fi & 1), L - 2);
    P1[k] = min(fi | 1, L - 1);
    d0[k] = a - (F)P0[k];
    d1[k] = a - (F)P1[k];
    D0 = fma(d0[k], d0[k], D0);
    D1 = fma(d1[k], d1[k], D1);
    S0 += P0[k];
    S1 += P1[k];
    NS += neg[k];
  }
  const int odd0 = (S0 >> 1) & 1;
  const int odd1 = STRICT ? (((S1 + 2 * NS) >> 1) & 1) : 0;
  F b0 = -INFINITY, b1 = -INFINITY, s0 = -INFINITY, s1 = -INFINITY;
  int i0 = 0, i1 = 0;
  if (std::is_same<F, float>::value && margin) {
    // fp32 with a margin (the hot paths): the largest and second largest
    // kappa as unsigned keys, no compare masks.  kappa >= 0 (ok) maps to
    // 0x80000000 | bits(|d|), kappa < 0 to 0x7fffffff ^ bits(|d|), so the
    // keys order like kappa; the low 3 bits are replaced by 7 - k, so the
    // lowest index wins exact ties.  Kappas within 8 ulps may pick either
    // coordinate and carry up to 8 ulps (< 2e-6) into the costs, but the
    // gap between them is then far below kNearTie, so those groups are
    // re-decided in fp64 anyway.  ok is the sign bit of d or of P - (L - 3)
    // (resp. L - 2).
    uint32_t kb0 = 0u, ks0 = 0u, kb1 = 0u, ks1 = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t u0 = __float_as_uint((float)d0[k]);
      const uint32_t m0 = (uint32_t)((int32_t)(u0 | (uint32_t)(P0[k] - (L - 3))) >> 31);
      const uint32_t key0 = (((~u0 & 0x7fffffffu) ^ m0) & ~7u) | (uint32_t)(7 - k);
      ks0 = median3u(kb0, ks0, key0);
      kb0 = max(kb0, key0);
      const uint32_t u1 = __float_as_uint((float)d1[k]);
      const uint32_t m1 = (uint32_t)((int32_t)(u1 | (uint32_t)(P1[k] - (L - 2))) >> 31);
      const uint32_t key1 = (((~u1 & 0x7fffffffu) ^ m1) & ~7u) | (uint32_t)(7 - k);
      if (STRICT) ks1 = median3u(kb1, ks1, key1);
      kb1 = max(kb1, key1);
    }
    const auto unkey = [](uint32_t key) -> float {
      const uint32_t kk = key & ~7u;
      return (kk & 0x80000000u) ? __uint_as_float(kk & 0x7fffffffu)
                                : -__uint_as_float(kk ^ 0x7ffffff8u);
    };
    b0 = unkey(kb0);
    s0 = unkey(ks0);
    i0 = 7 - (int)(kb0 & 7u);
    b1 = unkey(kb1);
    s1 = STRICT ? unkey(ks1) : (F)-INFINITY;
    i1 = 7 - (int)(kb1 & 7u);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool ok0 = (d0[k] < 0) || (P0[k] <= L - 4);
      const F k0 = ok0 ? fabs(d0[k]) : -fabs(d0[k]);
      if (margin) s0 = median3(b0, s0, k0);
      if (k0 > b0) { b0 = k0; i0 = k; }
      if (STRICT || margin) {
        const bool ok1 = (d1[k] < 0) || (P1[k] <= L - 3);
        const F k1 = ok1 ? fabs(d1[k]) : -fabs(d1[k]);
        if (STRICT && margin) s1 = median3(b1, s1, k1);
        if (k1 > b1) { b1 = k1; i1 = k; }
      }
    }
  }
  if (odd0) D0 = D0 + fma((F)-4, b0, (F)4);
  if (STRICT && odd1) D1 = D1 + fma((F)-4, b1, (F)4);
  const int c = (D1 < D0) ? 1 : 0;
  if (margin) {
    const F m0 = odd0 ? 4 * (b0 - s0) : 8 - 4 * (b0 + s0);
    const F m1 = !STRICT ? 4 - 4 * b1 : odd1 ? 4 * (b1 - s1) : 8 - 4 * (b1 + s1);
    *margin = fmin(fabs(D1 - D0), c ? m1 : m0);
  }
  const int odd = c ? odd1 : odd0;
  const int is = c ? i1 : i0;
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    int P = c ? P1[k] : P0[k];
    if (odd && k == is) {
      const F dd = c ? d1[k] : d0[k];
      const bool ok = (dd < 0) || (P <= L - 4 + c);
      const int t = (dd >= 0) ? 2 : -2;
      P = ok ? P + t : P - t;
    }
    const int p2 = neg[k] ? -P : P;
    const int idx = (p2 + L - c) >> 1;
    w |= (uint32_t)idx << (BITS * k);
  }
  code = w;
  coset = c;
}

// 2-bit decoder (L = 4) on g = 2y.  With a = |g| and t = a - 1:
//  integer coset: p = 0 if a < 1 else sign(g) (bit B = a >= 1);
//  half coset:    |p| = 1/2 if a < 2 else 3/2 (bit E = a >= 2), sign S;
//  D1 - D0 = sum_k 2 min(|t_k|, 3 - a_k) - 8        (doubled units);
//  integer-coset parity step: the coordinate with the smallest |t| toggles
//  B, extra cost 4 |t|;  strict half-coset step: kappa = |t| (a < 2) or
//  3 - a (a >= 2), extra cost 4 - 4 kappa, toggles E (a >= 1) or S (a < 1).
// The two top bits of g's fp32 pattern are (S, E), so shifting them in for
// k = 7 .. 0 builds the half-coset code word with (S_k, E_k) at bits
// (2k+1, 2k); the sign bit of t gives not-B.  Scanning k downward also makes
// the lowest index win ties.  Code word: 2-bit idx_k = p_k + 2 - c/2 at bits
// [2k, 2k+2): integer coset bit0 = B, bit1 = ~(B & S); half coset
// bit0 = E ^ S, bit1 = ~S.
// `cosets` receives the wave-wide ballot of the coset bit (every lane of the
// wave must be active).  `near` is set when the decision margin (as for
// e8_decode: the cheapest switches 4|t| resp. 4|e| inside the chosen coset,
// |D1 - D0| across) lies below kNearTie.
template <bool STRICT>
__device__ __forceinline__ void e8_decode2(const float g[8], uint32_t& code,
                                           uint64_t& cosets, int& coset, bool& near) {
  // With e = |t| - 1: min(|t|, 3 - a) = 1 - |e| and kappa = 1 - |e| exactly
  // (|t| is a multiple of 2^-24 in [0, 3]), so D1 - D0 = 8 - 2 sum |e|, the
  // strict step takes the smallest |e| (lowest index on ties) and costs
  // 4 |e|.  |.| comes free as a source modifier.  Switching one coordinate
  // to its other neighbour costs 4 |t| on the integer coset and 4 |e| on the
  // half coset, so the second smallest of each bounds the margin.
  //
  // The smallest |t| (|e|) and its coordinate come from one v_min_u32 on
  // keys that hold the bits of |t| with the 3 low mantissa bits replaced by
  // the coordinate index (non-negative floats order like their bits), so
  // equal values pick the lowest index.  Values within 7 ulps may then pick
  // either coordinate and carry up to 7 ulps (< 2e-6) of error into the
  // costs, but the gap between them is then far below kNearTie, so those
  // groups are re-decided in fp64 anyway.
  uint32_t X = 0, Bn = 0;
  float acc = 0.f, b1r = INFINITY;
  uint32_t kb0 = ~0u, ks0 = ~0u, kb1 = ~0u, ks1 = ~0u;
#pragma unroll
  for (int k = 7; k >= 0; --k) {
    const float t = fabsf(g[k]) - 1.0f;
    const float e = fabsf(t) - 1.0f;
    X = shift_in(X, g[k], 2);
    Bn = shift_in(Bn, t, 1);
    acc = acc + fabsf(e);
    const uint32_t k0 = (__float_as_uint(t) & 0x7ffffff8u) | (uint32_t)k;
    ks0 = median3u(kb0, ks0, k0);
    kb0 = min(kb0, k0);
    if (STRICT) {
      const uint32_t k1 = (__float_as_uint(e) & 0x7ffffff8u) | (uint32_t)k;
      ks1 = median3u(kb1, ks1, k1);
      kb1 = min(kb1, k1);
    } else {
      b1r = fminf(b1r, fabsf(e));
    }
  }
  const float best0 = __uint_as_float(kb0 & 0x7ffffff8u);
  const float sec0 = __uint_as_float(ks0 & 0x7ffffff8u);
  const float best1 = STRICT ? __uint_as_float(kb1 & 0x7ffffff8u) : b1r;
  const float sec1 = __uint_as_float(ks1 & 0x7ffffff8u);
  const uint32_t f0 = 1u << (2 * (kb0 & 7u));
  const uint32_t f1 = STRICT ? 1u << (2 * (kb1 & 7u)) : 0u;
  const uint32_t odd0 = __builtin_popcount(Bn) & 1u;
  float lhs = __fmaf_rn(-2.f, acc, 8.f);
  uint32_t odd1 = 0;
  if (STRICT) {
    odd1 = __builtin_popcount(X) & 1u;
    if (odd1) lhs = lhs + 4.f * best1;
  }
  const float rhs = odd0 ? 4.f * best0 : 0.f;
  const int c = lhs < rhs ? 1 : 0;
  cosets = __ballot(lhs < rhs);
  coset = c;
  {
    const float m0 = odd0 ? sec0 - best0 : best0 + sec0;
    const float m1 = !STRICT ? best1 : odd1 ? sec1 - best1 : best1 + sec1;
    near = fminf(fabsf(lhs - rhs), 4.f * (c ? m1 : m0)) < kNearTie;
  }
  // both code words, then a select (no divergent branch)
  const uint32_t Bsp = spread8(~Bn);
  const uint32_t b = Bsp ^ (odd0 ? f0 : 0u);
  const uint32_t w0 = b | (~((b << 1) & X) & 0xaaaau);
  uint32_t x = X;
  if (STRICT) x ^= odd1 ? (f1 & Bsp) | ((f1 & ~Bsp) << 1) : 0u;
  const uint32_t w1 = ((x ^ (x >> 1)) & 0x5555u) | (~x & 0xaaaau);
  code = c ? w1 : w0;
}

}  // namespace nq
