// The fp64 pass of quantize, the RoPE table, and the decoder test hook.
//
// The quantize kernels compute y in fp32 and take each lattice decision in
// fp32.  Every vector with a group whose decision margin falls below
// kNearTie is appended to a queue; exact_kernel then recomputes those
// vectors from their input in fp64 -- RoPE removal with fp64 cos / sin,
// Walsh-Hadamard stages h = 1, 2, ..., n/2, the group maximum, y =
// (L/2) u / a as one correctly rounded division -- decodes them with the same
// two-coset decoder in fp64 and overwrites their codes, coset bits and
// scales.  For fp16 inputs without RoPE, u is exact and the decision is
// taken on the exact quotient with integer arithmetic, so that exact ties
// (coordinates of equal magnitude, equidistant cosets: fp16 sums make them
// common enough to matter) fall to the tie rules and not to rounding.  With
// the queue full the pass recomputes every vector of the call.
//
// Pages: NexusQuant blog, E8 walkthrough post ("Python Implementation": pad,
// per-group scale, nearest lattice point; "The Conway-Sloane Nearest-Point
// Algorithm"); post "The E8 lattice quantizes 8 numbers at once" ("Handling
// outliers": Hadamard rotation); nexusquant-kv 0.5.1 README ("How it works":
// RoPE removal on keys, zero padding).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "nq_device.h"
#include "nq_internal.h"

namespace nq {
namespace {

constexpr int kExBlock = 256;

__device__ __forceinline__ double load_in(const __half* p, int64_t i) {
  return (double)h2f(reinterpret_cast<const uint16_t*>(p)[i]);
}
__device__ __forceinline__ double load_in(const float* p, int64_t i) { return (double)p[i]; }

// The two-coset decoder on the exact quotients g_k = N_k / A (integers, A >
// 0, |N_k| <= L A), the same steps as e8_decode with every comparison exact:
// with r = |N| - P A (the rounding error times A), the distance difference
// is A (D1 - D0) = sum_k (P0_k - P1_k)(r0_k + r1_k), and a parity step adds
// 4A - 4 kappa.  neg_k is the sign bit of g_k (signed zeros included).
template <int BITS, bool STRICT>
__device__ void e8_decode_int(const int64_t N[8], const int neg[8], int64_t A, uint32_t& code,
                              int& coset) {
  constexpr int L = 1 << BITS;
  int P0[8], P1[8];
  int64_t r0[8], r1[8];
  int S0 = 0, S1 = 0, NS = 0;
  int64_t dA = 0;
  const double Ad = (double)A;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t n = N[k] < 0 ? -N[k] : N[k];
    // floor(n / A): the fp64 quotient of the exact n and A, corrected by one
    int fi = (int)floor((double)n / Ad);
    if ((int64_t)fi * A > n) --fi;
    else if ((int64_t)(fi + 1) * A <= n) ++fi;
    P0[k] = min(fi + (fi & 1), L - 2);
    P1[k] = min(fi | 1, L - 1);
    r0[k] = n - (int64_t)P0[k] * A;
    r1[k] = n - (int64_t)P1[k] * A;
    dA += (int64_t)(P0[k] - P1[k]) * (r0[k] + r1[k]);
    S0 += P0[k];
    S1 += P1[k];
    NS += neg[k];
  }
  const int odd0 = (S0 >> 1) & 1;
  const int odd1 = STRICT ? (((S1 + 2 * NS) >> 1) & 1) : 0;
  int64_t b0 = INT64_MIN, b1 = INT64_MIN;
  int i0 = 0, i1 = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool ok0 = (r0[k] < 0) || (P0[k] <= L - 4);
    const int64_t a0 = r0[k] < 0 ? -r0[k] : r0[k];
    const int64_t k0 = ok0 ? a0 : -a0;
    if (k0 > b0) { b0 = k0; i0 = k; }
    if (STRICT) {
      const bool ok1 = (r1[k] < 0) || (P1[k] <= L - 3);
      const int64_t a1 = r1[k] < 0 ? -r1[k] : r1[k];
      const int64_t k1 = ok1 ? a1 : -a1;
      if (k1 > b1) { b1 = k1; i1 = k; }
    }
  }
  if (odd0) dA -= 4 * A - 4 * b0;
  if (STRICT && odd1) dA += 4 * A - 4 * b1;
  const int c = dA < 0 ? 1 : 0;
  const int odd = c ? odd1 : odd0;
  const int is = c ? i1 : i0;
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    int P = c ? P1[k] : P0[k];
    if (odd && k == is) {
      const int64_t dd = c ? r1[k] : r0[k];
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

// One vector per VL = n/8 lanes (lane m holds coordinates 8m .. 8m+7 of the
// padded vector), 64/VL vectors per wave, a grid-stride loop over the items.
// The pass over one tensor by `nblocks` blocks, this being block `block`.
template <int N, int BITS, bool STRICT, typename InT>
__device__ __forceinline__ void exact_body(TensorArgs a, int all, int block, int nblocks) {
  constexpr int VL = N / 8;
  constexpr int VPW = 64 / VL;
  const int lane = threadIdx.x & 63;
  const int m = lane % VL;
  const int row = lane / VL;
  const int64_t n_waves = (int64_t)nblocks * (kExBlock / 64);
  const int64_t wave = (int64_t)block * (kExBlock / 64) + (threadIdx.x >> 6);
  const unsigned long long cnt = all ? 0ull : *a.queue_count;
  const bool every = all || cnt > (unsigned long long)a.queue_cap;
  const int64_t items = every ? a.n_vec : (int64_t)cnt;
  const int h = a.d >> 1;
  const int gl = a.G >> 3;
  const int j0 = 8 * m;
  const InT* x = static_cast<const InT*>(a.x);
  for (int64_t base = wave * VPW; base < items; base += n_waves * VPW) {
    const int64_t item = base + row;
    const bool live = item < items;
    const int64_t vec = live ? (every ? item : a.queue[item]) : 0;
    const int64_t sh = vec / a.T;
    const int64_t t = vec - sh * a.T;
    double v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = j0 < a.d ? load_in(x, vec * a.d + j0 + k) : 0.0;
    if (a.omega != nullptr) {
      // x'_i = x_i c + x_{i+h} s, x'_{i+h} = x_{i+h} c - x_i s: two rounded
      // products and a rounded sum each; c, s from the same fp64 angle and
      // sincos as the fp32 table of the fp32 kernels
      double xp[8];
      if (a.d == 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) xp[k] = v[k ^ 4];
      } else {
        const int hl = h >> 3;
        const int pm = m < hl ? m + hl : (m < 2 * hl ? m - hl : m);
        const int src = lane - m + pm;
#pragma unroll
        for (int k = 0; k < 8; ++k) xp[k] = __shfl(v[k], src);
      }
      if (j0 < a.d) {
        const double pos =
            a.positions != nullptr ? (double)a.positions[t] : (double)(a.pos0 + t);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int j = j0 + k;
          const bool up = j >= h;
          double sn, cs;
          sincos(pos * a.omega[up ? j - h : j], &sn, &cs);
          const double p1 = __dmul_rn(v[k], cs);
          const double p2 = __dmul_rn(xp[k], sn);
          v[k] = up ? __dsub_rn(p1, p2) : __dadd_rn(p1, p2);
        }
      }
    }
    // Walsh-Hadamard stages 1, 2, 4 in the lane, then 8 .. n/2 across lanes;
    // the lower coordinate of each pair keeps a + b, the upper a - b
#pragma unroll
    for (int s = 1; s < 8; s <<= 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if ((k & s) == 0) {
          const double p = v[k], q = v[k + s];
          v[k] = __dadd_rn(p, q);
          v[k + s] = __dsub_rn(p, q);
        }
      }
    }
#pragma unroll
    for (int s = 1; s < VL; s <<= 1) {
      const bool upper = (m & s) != 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const double o = __shfl_xor(v[k], s);
        v[k] = upper ? __dsub_rn(o, v[k]) : __dadd_rn(v[k], o);
      }
    }
    double mx = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = fmax(mx, fabs(v[k]));
    for (int s = 1; s < gl; s <<= 1) mx = fmax(mx, __shfl_xor(mx, s));
    const double am = fmax(mx, a.eps64);
    uint32_t code;
    int c;
    if (std::is_same<InT, __half>::value && a.omega == nullptr && mx > a.eps64) {
      // fp16 inputs without RoPE: u and a are exact multiples of 2^-24
      // below 2^23, so g = 2y = L u / a is decided on exact integers
      int64_t num[8];
      int neg[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        num[k] = (int64_t)(v[k] * (double)(2 << BITS) * 0x1p23);
        neg[k] = signbit(v[k]) ? 1 : 0;
      }
      e8_decode_int<BITS, STRICT>(num, neg, (int64_t)(am * 0x1p24), code, c);
    } else {
      double y[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = (a.half_L64 * v[k]) / am;
      e8_decode<BITS, STRICT, double>(y, code, c, nullptr);
    }
    if (STRICT && a.compact) {
      constexpr uint32_t kBit = 1u << (7 * BITS);
      code = (code & ~kBit) | (c ? kBit : 0u);
    }
    const uint64_t bal = __ballot(c);
    if (live) {
      const int64_t pvec = sh * a.pT + t;
      uint8_t* cp = a.codes + pvec * a.code_bytes + m * BITS;
#pragma unroll
      for (int b = 0; b < BITS; ++b) cp[b] = (uint8_t)(code >> (8 * b));
      if (m == 0 && !a.compact) {
        const uint32_t bits =
            (uint32_t)(bal >> (row * VL)) & (uint32_t)((1ull << VL) - 1ull);
        uint8_t* q = a.cosets + pvec * a.coset_bytes;
        for (int b = 0; b < a.coset_bytes; ++b) q[b] = (uint8_t)(bits >> (8 * b));
      }
      if (m % gl == 0) a.scales[pvec * a.n_scales + m / gl] = f64_to_f16_rn(am * a.sigma_k);
    }
  }
}

template <int N, int BITS, bool STRICT, typename InT>
__global__ __launch_bounds__(kExBlock) void exact_kernel(TensorArgs a, int all) {
  exact_body<N, BITS, STRICT, InT>(a, all, blockIdx.x, gridDim.x);
}

// Both tensors of a call in one launch (the same n, bits and parity): blocks
// 0 .. nk - 1 take the keys, the rest the values.
template <int N, int BITS, bool STRICT, typename InT>
__global__ __launch_bounds__(kExBlock) void exact_kernel2(TensorArgs ak, TensorArgs av, int all,
                                                          int nk) {
  const bool keys = (int)blockIdx.x < nk;
  exact_body<N, BITS, STRICT, InT>(keys ? ak : av, all, keys ? (int)blockIdx.x : (int)blockIdx.x - nk,
                                   keys ? nk : (int)gridDim.x - nk);
}

template <int N>
int64_t exact_blocks(const TensorArgs& a, int all) {
  constexpr int VPB = kExBlock / (N / 8);
  // the queue holds about 1/32 of the vectors and ~1.5e-3 of random vectors
  // are queued: a grid of up to 2048 blocks takes them in one sweep, the
  // blocks past the count exit at once (a full queue falls back to the
  // grid-stride loop over every vector)
  const int64_t vecs = all ? a.n_vec : (a.queue_cap < a.n_vec ? a.queue_cap : a.n_vec);
  int64_t blocks = (vecs + VPB - 1) / VPB;
  const int64_t cap = all ? 65536 : 2048;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return blocks;
}

template <int N, int BITS, typename T>
hipError_t exact_n2(const TensorArgs& ak, const TensorArgs& av, int all, hipStream_t s) {
  const int64_t bk = exact_blocks<N>(ak, all), bv = exact_blocks<N>(av, all);
  const dim3 g((unsigned)(bk + bv)), b(kExBlock);
  if (ak.strict)
    hipLaunchKernelGGL((exact_kernel2<N, BITS, true, T>), g, b, 0, s, ak, av, all, (int)bk);
  else
    hipLaunchKernelGGL((exact_kernel2<N, BITS, false, T>), g, b, 0, s, ak, av, all, (int)bk);
  return hipGetLastError();
}

template <int N, int BITS, typename T>
hipError_t exact_n(const TensorArgs& a, int all, hipStream_t s) {
  const int64_t blocks = exact_blocks<N>(a, all);
  if (a.strict)
    hipLaunchKernelGGL((exact_kernel<N, BITS, true, T>), dim3((unsigned)blocks), dim3(kExBlock),
                       0, s, a, all);
  else
    hipLaunchKernelGGL((exact_kernel<N, BITS, false, T>), dim3((unsigned)blocks), dim3(kExBlock),
                       0, s, a, all);
  return hipGetLastError();
}

template <int BITS, typename T>
hipError_t exact_b(const TensorArgs& a, int all, hipStream_t s) {
  switch (a.n) {
    case 8: return exact_n<8, BITS, T>(a, all, s);
    case 16: return exact_n<16, BITS, T>(a, all, s);
    case 32: return exact_n<32, BITS, T>(a, all, s);
    case 64: return exact_n<64, BITS, T>(a, all, s);
    case 128: return exact_n<128, BITS, T>(a, all, s);
    case 256: return exact_n<256, BITS, T>(a, all, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t exact_t(const TensorArgs& a, int all, hipStream_t s) {
  if (a.bits == 2) return exact_b<2, T>(a, all, s);
  if (a.bits == 3) return exact_b<3, T>(a, all, s);
  return hipErrorInvalidValue;
}

template <int BITS, typename T>
hipError_t exact_b2(const TensorArgs& ak, const TensorArgs& av, int all, hipStream_t s) {
  switch (ak.n) {
    case 8: return exact_n2<8, BITS, T>(ak, av, all, s);
    case 16: return exact_n2<16, BITS, T>(ak, av, all, s);
    case 32: return exact_n2<32, BITS, T>(ak, av, all, s);
    case 64: return exact_n2<64, BITS, T>(ak, av, all, s);
    case 128: return exact_n2<128, BITS, T>(ak, av, all, s);
    case 256: return exact_n2<256, BITS, T>(ak, av, all, s);
    default: return hipErrorInvalidValue;
  }
}

__global__ __launch_bounds__(kExBlock) void rope_table_kernel(
    const int32_t* pos, int64_t pos0, int64_t T, int h, RopeFreqs f, float2* table,
    double* omega, unsigned long long* counters, int n_counters) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (counters != nullptr && i < n_counters) counters[i] = 0ull;
  if (omega != nullptr && i < h) omega[i] = f.omega[i];
  if (i >= T * h) return;
  const int64_t t = i / h;
  const int k = (int)(i % h);
  const double p = pos ? (double)pos[t] : (double)(pos0 + t);
  // cos and sin to about one fp32 ulp, which is all the fp32 kernels need
  // (their near-tie decisions are re-taken in fp64)
  float sn, cs;
  rope_cos_sin(p, f.omega[k], cs, sn);
  table[i] = make_float2(cs, sn);
}

__global__ void clear_counters_kernel(unsigned long long* counters, int n) {
  if ((int)threadIdx.x < n) counters[threadIdx.x] = 0ull;
}

// Nearest point of the whole lattice, no cube limit (the textbook
// Conway-Sloane decoder on D8 and on D8 + 1/2 (strict) or Z^8 + 1/2
// (relaxed)), with the same tie rules as the cube decoder: rounding ties away
// from zero, a parity step toward y (away from zero when y is on the point),
// the lowest index among equal |delta|, the integer coset on equal distance.
// Works on g = 2y, where both cosets round with an exact floor: the nearest
// even integer to |g| is f + (f & 1), the nearest odd one f | 1 (f =
// floor |g|).  Distances in fp64 (exact for fp32 y).  q = 2p.
template <bool STRICT>
__device__ void e8_nearest_free(const float y[8], int q[8], int& coset) {
  int qc[2][8];
  double dist[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    double dl[8];
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float g = y[k] + y[k];
      const int fi = (int)floorf(fabsf(g));
      const int P = c == 0 ? fi + (fi & 1) : (fi | 1);
      const int Q = signbit(g) ? -P : P;
      dl[k] = (double)g - (double)Q;
      qc[c][k] = Q;
      s += Q;
    }
    if ((c == 0 || STRICT) && ((s >> 1) & 1)) {   // sum p = s / 2 is odd
      int is = 0;
      double best = -1.0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (fabs(dl[k]) > best) { best = fabs(dl[k]); is = k; }
      int t = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k == is) t = dl[k] > 0.0 ? 2 : dl[k] < 0.0 ? -2 : (signbit(y[k]) ? -2 : 2);
#pragma unroll
      for (int k = 0; k < 8; ++k) if (k == is) qc[c][k] += t;
    }
    double d = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const double e = (double)y[k] - 0.5 * (double)qc[c][k];
      d += e * e;
    }
    dist[c] = d;
  }
  coset = dist[1] < dist[0] ? 1 : 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) q[k] = coset ? qc[1][k] : qc[0][k];
}

// Decoder alone.  constrained: the cube decoder the quantize kernels use (the
// 2-bit one on g = 2y for b = 2), with the same fp64 re-decision of groups
// whose margin is below kNearTie; otherwise the unconstrained nearest point,
// idx = p - c/2 + L/2 stored as a two's-complement int8.
template <int BITS, bool STRICT>
__global__ __launch_bounds__(kExBlock) void decode_debug_kernel(
    const float* y, int64_t n, int constrained, uint8_t* idx, uint8_t* coset) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = y[i * 8 + k];
  int c;
  if (!constrained) {
    int q[8];
    e8_nearest_free<STRICT>(v, q, c);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      idx[i * 8 + k] = (uint8_t)(int8_t)((q[k] - c + (1 << BITS)) / 2);
    coset[i] = (uint8_t)c;
    return;
  }
  uint32_t code;
  bool near;
  if (BITS == 2) {
    float g[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] = v[k] + v[k];
    uint64_t ball;
    e8_decode2<STRICT>(g, code, ball, c, near);
  } else {
    float mg;
    e8_decode<BITS, STRICT, float>(v, code, c, &mg);
    near = mg < kNearTie;
  }
  if (near) {
    double yd[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) yd[k] = (double)v[k];
    e8_decode<BITS, STRICT, double>(yd, code, c, nullptr);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
    idx[i * 8 + k] = (uint8_t)((code >> (BITS * k)) & ((1u << BITS) - 1u));
  coset[i] = (uint8_t)c;
}

}  // namespace

hipError_t launch_exact(const TensorArgs& a, int in_dtype, int all, hipStream_t s) {
  return in_dtype == 0 ? exact_t<__half>(a, all, s) : exact_t<float>(a, all, s);
}

hipError_t launch_exact2(const TensorArgs& ak, const TensorArgs& av, int in_dtype, int all,
                         hipStream_t s) {
  if (ak.n != av.n || ak.bits != av.bits || ak.strict != av.strict) return hipErrorInvalidValue;
  if (ak.bits == 2)
    return in_dtype == 0 ? exact_b2<2, __half>(ak, av, all, s) : exact_b2<2, float>(ak, av, all, s);
  if (ak.bits == 3)
    return in_dtype == 0 ? exact_b2<3, __half>(ak, av, all, s) : exact_b2<3, float>(ak, av, all, s);
  return hipErrorInvalidValue;
}

hipError_t launch_rope_table(const int32_t* positions, int64_t pos0, int64_t T, int d,
                             const RopeFreqs& f, float2* table, double* omega,
                             unsigned long long* counters, int n_counters,
                             hipStream_t stream) {
  const int h = d / 2;
  int64_t total = T * h;
  if (total < n_counters) total = n_counters;
  const int64_t blocks = (total + kExBlock - 1) / kExBlock;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(kExBlock), 0, stream,
                     positions, pos0, T, h, f, table, omega, counters, n_counters);
  return hipGetLastError();
}

hipError_t launch_clear_counters(unsigned long long* counters, int n, hipStream_t s) {
  hipLaunchKernelGGL(clear_counters_kernel, dim3(1), dim3(64), 0, s, counters, n);
  return hipGetLastError();
}

hipError_t launch_decode_debug(const float* y, int64_t n, int bits, int strict, int constrained,
                               uint8_t* idx, uint8_t* coset, hipStream_t s) {
  const int64_t blocks = (n + kExBlock - 1) / kExBlock;
  const dim3 g((unsigned)blocks), b(kExBlock);
  if (bits == 2 && strict)
    hipLaunchKernelGGL((decode_debug_kernel<2, true>), g, b, 0, s, y, n, constrained, idx, coset);
  else if (bits == 2)
    hipLaunchKernelGGL((decode_debug_kernel<2, false>), g, b, 0, s, y, n, constrained, idx, coset);
  else if (bits == 3 && strict)
    hipLaunchKernelGGL((decode_debug_kernel<3, true>), g, b, 0, s, y, n, constrained, idx, coset);
  else if (bits == 3)
    hipLaunchKernelGGL((decode_debug_kernel<3, false>), g, b, 0, s, y, n, constrained, idx, coset);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace nq
