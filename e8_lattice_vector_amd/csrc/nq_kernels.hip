// HIP kernels for E8 lattice KV-cache quantization on gfx950 (MI355X).
//
// Layout on the wave: one 8-group (8 consecutive coordinates of the padded
// head vector) per lane, n/8 consecutive lanes per vector, 64/(n/8) vectors
// per wave64.  The Walsh-Hadamard butterflies over strides 1, 2, 4 run inside
// the lane; strides 8 .. n/2 pair lanes m and m ^ (stride/8).  Every
// butterfly is one correctly rounded fp32 add or subtract and the stages run
// in the order 1, 2, 4, ..., n/2, so the rotated vector -- and the scaled
// value y on which the lattice decision is taken -- is reproducible bit for
// bit by any implementation of the same stage order.
//
// Pages: NexusQuant blog, E8 walkthrough post ("The Conway-Sloane
// Nearest-Point Algorithm", "Python Implementation", "Why Per-Group
// Scaling?", "The Relaxed Parity Discovery"); post "The E8 lattice quantizes
// 8 numbers at once" ("Handling outliers": Hadamard rotation);
// nexusquant-kv 0.5.1 README ("How it works": RoPE removal, zero padding);
// Nedelkoski et al., "E8 Lattice Key Quantization for Low-Bit KV-Cache
// Compression" (Abstract, Table 3: scoring packed keys without
// dequantizing).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "nq_internal.h"
#include "nq_device.h"

namespace nq {
namespace {

constexpr int kBlock = 256;

// min / max of 64-bit values (HIP's unqualified min / max of two int64_t
// resolve to the int overloads and truncate)
__host__ __device__ constexpr int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ constexpr int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

typedef float nq_f2 __attribute__((ext_vector_type(2)));
typedef float nq_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t nq_u4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Io;

template <>
struct Io<__half> {
  static __device__ __forceinline__ void load8(const void* base, int64_t off,
                                               float v[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(base) + off);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = h2f((uint16_t)(u[i] & 0xffffu));
      v[2 * i + 1] = h2f((uint16_t)(u[i] >> 16));
    }
  }
  static __device__ __forceinline__ void store8(void* base, int64_t off,
                                                const float v[8]) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = (uint32_t)f2h_rn(v[2 * i]) | ((uint32_t)f2h_rn(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) =
        make_uint4(u[0], u[1], u[2], u[3]);
  }
  static __device__ __forceinline__ float load1(const void* base, int64_t off) {
    return h2f(static_cast<const uint16_t*>(base)[off]);
  }
  using Raw = uint4;
  static __device__ __forceinline__ Raw load_raw(const void* base, int64_t off) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  }
  static __device__ __forceinline__ void cvt(const Raw& w, float v[8]) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = h2f((uint16_t)(u[i] & 0xffffu));
      v[2 * i + 1] = h2f((uint16_t)(u[i] >> 16));
    }
  }
};

template <>
struct Io<float> {
  static __device__ __forceinline__ void load8(const void* base, int64_t off,
                                               float v[8]) {
    const float4* p =
        reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store8(void* base, int64_t off,
                                                const float v[8]) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  static __device__ __forceinline__ float load1(const void* base, int64_t off) {
    return static_cast<const float*>(base)[off];
  }
  struct Raw {
    float4 a, b;
  };
  static __device__ __forceinline__ Raw load_raw(const void* base, int64_t off) {
    const float4* p =
        reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    return Raw{p[0], p[1]};
  }
  static __device__ __forceinline__ void cvt(const Raw& w, float v[8]) {
    v[0] = w.a.x; v[1] = w.a.y; v[2] = w.a.z; v[3] = w.a.w;
    v[4] = w.b.x; v[5] = w.b.y; v[6] = w.b.z; v[7] = w.b.w;
  }
};

// Walsh-Hadamard stages 1, 2, 4 inside the lane.
__device__ __forceinline__ void fwht_lane(float v[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if ((k & h) == 0) {
        const float a = v[k], b = v[k + h];
        v[k] = __fadd_rn(a, b);
        v[k + h] = __fsub_rn(a, b);
      }
    }
  }
}

// Stages 2 and 4 inside the lane (stage 1 already done).
__device__ __forceinline__ void fwht_lane_24(float v[8]) {
#pragma unroll
  for (int h = 2; h < 8; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if ((k & h) == 0) {
        const float a = v[k], b = v[k + h];
        v[k] = __fadd_rn(a, b);
        v[k + h] = __fsub_rn(a, b);
      }
    }
  }
}

// Load 8 fp16 values and apply Walsh-Hadamard stage 1 in the same
// instructions: v_fma_mix_f32 reads both fp16 halves of a word (exactly
// widened) and rounds a*1 + b (or a*1 - b) once to fp32, i.e. fl(a + b).
__device__ __forceinline__ void load8_h_stage1(const void* p, float v[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    asm("v_fma_mix_f32 %0, %2, 1.0, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %1, %2, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[1,0,1]"
        : "=&v"(v[2 * i]), "=&v"(v[2 * i + 1])
        : "v"(u[i]));
  }
}

// Stages 8 .. 4*VL across the VL lanes of one vector (lane m holds
// coordinates 8m .. 8m+7).  The lane with the stride bit clear keeps a + b,
// its partner a - b.
template <int VL>
__device__ __forceinline__ void fwht_cross(float v[8], int m) {
#pragma unroll
  for (int s = 1; s < VL; s <<= 1) {
    const bool upper = (m & s) != 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float o = __shfl_xor(v[k], s);
      v[k] = upper ? __fsub_rn(o, v[k]) : __fadd_rn(v[k], o);
    }
  }
}

// Split-half RoPE on the lane's 8 coordinates.  inverse: x'_i = x_i c + x_{i+h}
// s, x'_{i+h} = x_{i+h} c - x_i s; forward flips the sign of s.  Products and
// sums are rounded separately.  All lanes of the wave must call this.
template <bool INVERSE>
__device__ __forceinline__ void rope_lane(float v[8], int m, int d,
                                          const float2* row) {
  const int h = d >> 1;
  const int j0 = 8 * m;
  float xp[8];
  if (d == 8) {
#pragma unroll
    for (int k = 0; k < 8; ++k) xp[k] = v[k ^ 4];
  } else {
    const int hl = h >> 3;
    const int pm = (m < hl) ? m + hl : m - hl;
    const int src = (int)(threadIdx.x & 63) - m + pm;
#pragma unroll
    for (int k = 0; k < 8; ++k) xp[k] = __shfl(v[k], src);
  }
  if (j0 < d) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k;
      const bool up = j >= h;
      const float2 cs = row[up ? j - h : j];
      const float a = __fmul_rn(v[k], cs.x);
      const float b = __fmul_rn(xp[k], cs.y);
      v[k] = (up == INVERSE) ? __fsub_rn(a, b) : __fadd_rn(a, b);
    }
  }
}

// ---------------------------------------------------------------------------
// Fast path for n <= 128 (one 16-lane DPP row or less per vector).
//
// Lane relabelling: the cross-lane butterfly stages pair lanes l and l ^ a_k
// with a = (1, 2, 7, 15), which are the DPP patterns quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror and row_mirror.  Lane l of a row holds
// 8-group m(l) = A^-1 l, A = [a_0 a_1 a_2 a_3] over GF(2); then the stage-k
// pair (l, l ^ a_k) is exactly the group pair (m, m ^ 2^k), i.e. the stride
// 8 * 2^k butterfly of the textbook transform, in the textbook order.
//
// Sign twist: lane l keeps w = sigma_l * u.  Every lane then computes
// w + coef_k * w_partner with one v_fmac_f32_dpp (coef_k = -1 where bit k of m
// is set, else +1); the sum is rounded once, exactly like a + b or a - b, and
// sigma_l = (-1)^popcount(m) is folded into the scale at the end.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_group(int l) {
  return l ^ (((l >> 2) & 1) * 3) ^ (((l >> 3) & 1) * 4);
}
__device__ __forceinline__ int group_lane(int m) {
  return (m & 1) ^ (m & 2) ^ (((m >> 2) & 1) * 7) ^ (((m >> 3) & 1) * 15);
}

#define NQ_FMAC8(CTRL, v, c)                                            \
  asm volatile("s_nop 1\n\t"                                             \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"  \
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), \
                 "+v"(v[5]), "+v"(v[6]), "+v"(v[7])                       \
               : "v"(c))

// x * c + partner(x) * s for 8 values: the partner read goes through DPP.
#define NQ_MULDPP8(CTRL, out, v, s)                                      \
  asm volatile("s_nop 1\n\t"                                             \
               "v_mul_f32_dpp %0, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_mul_f32_dpp %1, %9, %17 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_mul_f32_dpp %2, %10, %18 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_mul_f32_dpp %3, %11, %19 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_mul_f32_dpp %4, %12, %20 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_mul_f32_dpp %5, %13, %21 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_mul_f32_dpp %6, %14, %22 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
               "v_mul_f32_dpp %7, %15, %23 " CTRL " row_mask:0xf bank_mask:0xf"  \
               : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3]), \
                 "=&v"(out[4]), "=&v"(out[5]), "=&v"(out[6]), "=&v"(out[7]) \
               : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]),   \
                 "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(s[0]), "v"(s[1]),  \
                 "v"(s[2]), "v"(s[3]), "v"(s[4]), "v"(s[5]), "v"(s[6]),   \
                 "v"(s[7]))

#define NQ_DPP_A0 "quad_perm:[1,0,3,2]"
#define NQ_DPP_A1 "quad_perm:[2,3,0,1]"
#define NQ_DPP_A2 "row_half_mirror"
#define NQ_DPP_A3 "row_mirror"

template <int K>
__device__ __forceinline__ void stage_fmac(float v[8], float c) {
  if (K == 0) NQ_FMAC8(NQ_DPP_A0, v, c);
  if (K == 1) NQ_FMAC8(NQ_DPP_A1, v, c);
  if (K == 2) NQ_FMAC8(NQ_DPP_A2, v, c);
  if (K == 3) NQ_FMAC8(NQ_DPP_A3, v, c);
}

template <int K>
__device__ __forceinline__ void partner_mul(float out[8], const float v[8],
                                            const float s[8]) {
  if (K == 0) NQ_MULDPP8(NQ_DPP_A0, out, v, s);
  if (K == 1) NQ_MULDPP8(NQ_DPP_A1, out, v, s);
  if (K == 2) NQ_MULDPP8(NQ_DPP_A2, out, v, s);
  if (K == 3) NQ_MULDPP8(NQ_DPP_A3, out, v, s);
}

template <int K>
__device__ __forceinline__ float dpp_a(float x) {
  constexpr int ctrl = K == 0 ? 0xB1 : K == 1 ? 0x4E : K == 2 ? 0x141 : 0x140;
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), ctrl, 0xF, 0xF, true));
}
template <int K>
__device__ __forceinline__ uint32_t dpp_a_u(uint32_t x) {
  constexpr int ctrl = K == 0 ? 0xB1 : K == 1 ? 0x4E : K == 2 ? 0x141 : 0x140;
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, ctrl, 0xF, 0xF, true);
}

// Max over the lanes of one scale group (gl = G/8 lanes, a subspace spanned
// by a_0 .. a_{log2 gl - 1}).
// max |v_k| over the lane's 8 values (v_max3_f32 with abs modifiers)
__device__ __forceinline__ float abs_max8(const float v[8]) {
  float m;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|\n\t"
      "v_max3_f32 %0, %0, |%4|, |%5|\n\t"
      "v_max3_f32 %0, %0, |%6|, |%7|\n\t"
      "v_max_f32_e64 %0, %0, |%8|"
      : "=&v"(m)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]),
        "v"(v[6]), "v"(v[7]));
  return m;
}

#define NQ_DPP_MAX(CTRL, x)                                                  \
  asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 " CTRL                  \
               " row_mask:0xf bank_mask:0xf"                                   \
               : "+v"(x))

// Max over the lanes of one scale group (gl = G/8 lanes, a subspace spanned
// by a_0 .. a_{log2 gl - 1}).
template <int VL>
__device__ __forceinline__ float group_max(float x, int gl) {
  if (VL > 1 && gl > 1) NQ_DPP_MAX(NQ_DPP_A0, x);
  if (VL > 2 && gl > 2) NQ_DPP_MAX(NQ_DPP_A1, x);
  if (VL > 4 && gl > 4) NQ_DPP_MAX(NQ_DPP_A2, x);
  if (VL > 8 && gl > 8) NQ_DPP_MAX(NQ_DPP_A3, x);
  return x;
}
template <int VL>
__device__ __forceinline__ uint32_t row_or(uint32_t x) {
  if (VL > 1) x |= dpp_a_u<0>(x);
  if (VL > 2) x |= dpp_a_u<1>(x);
  if (VL > 4) x |= dpp_a_u<2>(x);
  if (VL > 8) x |= dpp_a_u<3>(x);
  return x;
}

// fl(1/a): the hardware reciprocal estimate refined by one Newton step whose
// residual 1 - a*r0 is formed by a fused multiply-add.  On gfx950 this equals
// the correctly rounded quotient 1/a for every normal a below 2^126, i.e.
// wherever 1/a is normal (compared against IEEE division for every fp32
// mantissa of every such binade); the callers keep the true division above.
__device__ __forceinline__ float rcp_rn(float a) {
  const float r0 = __builtin_amdgcn_rcpf(a);
  const float e = __builtin_fmaf(-a, r0, 1.0f);
  return __builtin_fmaf(e, r0, r0);
}

// Coset words from a wave-wide ballot: bit VL*row + l of `mask` is the coset
// bit of lane l of that row; move it to bit VL*row + lane_group(l), i.e.
// reverse the nibbles at odd nibble positions (l ^ 3 where bit 2 of l is
// set), then for VL = 16 swap nibbles 2 and 3 of each 16-bit row word
// (l ^ 4 where bit 3 is set).  Runs on the scalar unit.
template <int VL>
__device__ __forceinline__ uint64_t coset_rows(uint64_t x) {
  if (VL >= 8) {
    const uint64_t odd = x & 0xF0F0F0F0F0F0F0F0ull;
    x = (x & 0x0F0F0F0F0F0F0F0Full) | ((odd & 0x1010101010101010ull) << 3) |
        ((odd & 0x8080808080808080ull) >> 3) | ((odd & 0x2020202020202020ull) << 1) |
        ((odd & 0x4040404040404040ull) >> 1);
  }
  if (VL == 16) {
    x = (x & 0x00FF00FF00FF00FFull) | ((x & 0x0F000F000F000F00ull) << 4) |
        ((x & 0xF000F000F000F000ull) >> 4);
  }
  return x;
}

// Compact strict packing: bit 7b of a group's code bits (the low bit of
// idx_7) holds the coset bit.  A strict codeword has an even index sum, so
// the low bit of idx_7 is the parity of the low bits of idx_0 .. idx_6.
template <int BITS>
struct Compact {
  static constexpr uint32_t kBit = 1u << (7 * BITS);
  static constexpr uint32_t kLow7 = BITS == 2 ? 0x1555u : 0x49249u;
  static __device__ __forceinline__ uint32_t fold(uint32_t w, int c) {
    return (w & ~kBit) | (c ? kBit : 0u);
  }
  // parity of idx_0..idx_6's low bits (the low bit of idx_7)
  static __device__ __forceinline__ uint32_t low7(uint32_t w) {
    return (uint32_t)__builtin_popcount(w & kLow7) & 1u;
  }
  static __device__ __forceinline__ uint32_t unfold(uint32_t w, int& c) {
    c = (w & kBit) ? 1 : 0;
    return (w & ~kBit) | (low7(w) ? kBit : 0u);
  }
};

// Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
// that consecutive logical workgroups share an XCD and its L2.  The wave
// order is then either tile-fastest (neighbouring waves stream neighbouring
// memory and share the cache lines of the small coset / scale planes: the
// memory-bound dequantize) or tile-major (the waves walking different
// (slab, head) chunks of one token tile are neighbours and share its RoPE
// rows in L2: the ALU-bound quantize, which wants many short waves).
// gridDim.x is a multiple of 8.
__device__ __forceinline__ int64_t xcd_wave_id() {
  const uint32_t nb = gridDim.x;
  const uint32_t lb = (blockIdx.x & 7u) * (nb >> 3) + (blockIdx.x >> 3);
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  return (int64_t)lb * (kBlock / 64) + w;
}

// What a wave needs to append to the queue of the fp64 pass, kept in LDS so
// that the hot loop holds none of it in registers: the counter, the queue,
// its capacity, and the index of the wave's first vector with the stride
// between the (slab, head) planes it walks.
struct QueueSlot {
  unsigned long long* count;
  int64_t* queue;
  int64_t cap;
  int64_t base;    // vector index of plane sh0, token t0 of the wave
  int64_t stride;  // vectors per plane (T)
};

__device__ __forceinline__ void queue_slot_init(QueueSlot* slot, const TensorArgs& a,
                                                int64_t base) {
  if ((threadIdx.x & 63) == 0) *slot = QueueSlot{a.queue_count, a.queue, a.queue_cap, base, a.T};
}

// Appends vector slot.base + it * slot.stride + off of every lane with `push`
// set to the call's queue of vectors whose lattice decisions are re-taken in
// fp64 (one atomic add per wave; entries past the queue's capacity are
// dropped, and the fp64 pass then recomputes every vector).  All lanes of
// the wave must call this.
__device__ __forceinline__ void queue_push(const QueueSlot* slot, bool push, int it, int off) {
  const uint64_t b = __ballot(push);
  if (b == 0) return;
  const QueueSlot q = *slot;
  const int lane = threadIdx.x & 63;
  const int first = __builtin_ctzll(b);
  unsigned long long base = 0;
  if (lane == first) base = atomicAdd(q.count, (unsigned long long)__popcll(b));
  base = __shfl(base, first);
  if (push) {
    const unsigned long long r = base + (unsigned long long)__popcll(b & ((1ull << lane) - 1ull));
    if (r < (unsigned long long)q.cap) q.queue[r] = q.base + (int64_t)it * q.stride + off;
  }
}

// ROPE: 0 none, 1 partner through DPP (d == n >= 16), 2 partner through
// ds_bpermute (other d, a multiple of 16), 3 partner inside the lane (d == 8).
template <int N, int BITS, bool STRICT, typename InT, int ROPE, bool PAD>
__global__ __launch_bounds__(kBlock) void quantize_fast_kernel(TensorArgs a,
                                                               int sh_chunk,
                                                               int tile_major) {
  constexpr int VL = N / 8;
  constexpr int TPW = 64 / VL;  // tokens per wave iteration
  const int lane = threadIdx.x & 63;
  const int row = lane / VL;
  const int l = lane % VL;
  const int m = lane_group(l);
  const int64_t n_tt = (a.T + TPW - 1) / TPW;
  const int64_t SH = a.n_vec / a.T;
  const int64_t wave = xcd_wave_id();
  const int64_t n_shc = (SH + sh_chunk - 1) / sh_chunk;
  const int64_t tt = tile_major ? wave / n_shc : wave % n_tt;
  const int64_t sh0 = (tile_major ? wave % n_shc : wave / n_tt) * sh_chunk;
  if (tt >= n_tt || sh0 >= SH) return;
  const int64_t sh1 = min64(SH, sh0 + sh_chunk);
  const int64_t t = tt * TPW + row;
  __shared__ QueueSlot qslots[kBlock / 64];
  QueueSlot* qslot = &qslots[threadIdx.x >> 6];
  queue_slot_init(qslot, a, sh0 * a.T + tt * TPW);
  const bool tvalid = t < a.T;
  const int64_t tc = tvalid ? t : a.T - 1;
  const int j0 = 8 * m;
  const bool data_lane = j0 < a.d;
  const int h = a.d >> 1;
  const int gl = a.G >> 3;

  // RoPE table slice for this lane's token and coordinates, kept in registers
  float rc[8], rs[8];
  int pl = 0;
  if (ROPE != 0) {
    const float2* row_p = a.rope + tc * h;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k;
      const bool up = j >= h;
      const float2 cs = data_lane ? row_p[up ? j - h : j] : make_float2(0.f, 0.f);
      rc[k] = cs.x;
      rs[k] = up ? -cs.y : cs.y;
    }
    if (ROPE == 2) {
      const int hl = h >> 3;
      const int pm = (m < hl) ? m + hl : (m < 2 * hl ? m - hl : m);
      pl = (lane - l) + group_lane(pm);
    }
  }
  // per-lane butterfly coefficients and final sign
  float coef[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) coef[k] = ((m >> k) & 1) ? -1.f : 1.f;
  const bool neg_sigma = (__builtin_popcount(m) & 1) != 0;
  // decision scale 2r (2-bit decoder on 2y) or r, with the lane's sign
  const float kr = (neg_sigma ? -a.half_L : a.half_L) * (BITS == 2 ? 2.f : 1.f);
  const float kq = (neg_sigma ? -1.f : 1.f) * (BITS == 2 ? 2.f : 1.f);
  const int row_shift = row * VL;
  constexpr uint32_t kRowMask = VL >= 32 ? 0xffffffffu : (1u << VL) - 1u;
  // Scale conversions are batched over gl iterations: lane m keeps the group
  // maximum of iteration (m % gl) of the batch and converts it at the flush.
  const int mg = m % gl;

  // per-lane byte offsets inside one (slab, head) plane (the host keeps
  // them below 2^31); the plane bases advance uniformly with sh
  const uint32_t off_x = (uint32_t)(tc * a.d + j0) * (uint32_t)sizeof(InT);
  const uint32_t off_c = (uint32_t)(tc * a.code_bytes) + (uint32_t)(m * BITS);
  const uint32_t off_s = (uint32_t)(tc * a.coset_bytes);
  const uint32_t off_g = (uint32_t)(tc * a.n_scales) + (uint32_t)(m / gl);
  const int64_t plane_x = a.T * a.d * (int64_t)sizeof(InT);
  const int64_t plane_c = a.pT * a.code_bytes;
  const int64_t plane_s = a.pT * a.coset_bytes;
  const int64_t plane_g = a.pT * a.n_scales;
  const uint32_t off_gb = (off_g + (uint32_t)mg * (uint32_t)plane_g) * 2u;
  float keep = 0.f;
  // uniform plane bases in scalar registers, lane offsets in 32-bit vector
  // registers (global_load/store with an SGPR base); the empty asm keeps the
  // offsets from being folded into per-lane 64-bit pointers
  const int n_it = (int)(sh1 - sh0);
  const char* xb = static_cast<const char*>(a.x) + sh0 * plane_x;
  uint8_t* cb = a.codes + sh0 * plane_c;
  uint8_t* qb = a.cosets + sh0 * plane_s;
  char* gb = reinterpret_cast<char*>(a.scales) + sh0 * plane_g * 2;
  uint32_t ox = off_x, oc = off_c, os = off_s;
  for (int it = 0; it < n_it; ++it, xb += plane_x, cb += plane_c, qb += plane_s) {
    asm volatile("" : "+v"(ox), "+v"(oc), "+v"(os));
    float v[8];
    constexpr bool kFuse = ROPE == 0 && std::is_same<InT, __half>::value;
    if (!PAD || data_lane) {
      if constexpr (kFuse) load8_h_stage1(xb + ox, v);
      else Io<InT>::load8(xb + ox, 0, v);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = 0.f;
    }
    if (ROPE == 1) {
      float pv[8];
      constexpr int KR = N == 128 ? 3 : N == 64 ? 2 : N == 32 ? 1 : 0;
      partner_mul<KR>(pv, v, rs);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __fmaf_rn(v[k], rc[k], pv[k]);
    } else if (ROPE == 2) {
      float pv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pv[k] = __shfl(v[k], pl);
      if (data_lane) {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __fmaf_rn(v[k], rc[k], __fmul_rn(pv[k], rs[k]));
      }
    } else if (ROPE == 3) {
      float x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = v[k];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __fmaf_rn(x[k], rc[k], __fmul_rn(x[k ^ 4], rs[k]));
    }
    if constexpr (kFuse) fwht_lane_24(v);
    else fwht_lane(v);
    if (VL > 1) stage_fmac<0>(v, coef[0]);
    if (VL > 2) stage_fmac<1>(v, coef[1]);
    if (VL > 4) stage_fmac<2>(v, coef[2]);
    if (VL > 8) stage_fmac<3>(v, coef[3]);
    float mx = abs_max8(v);
    mx = group_max<VL>(mx, gl);
    float amax;
    asm("v_max_f32 %0, %1, %2" : "=v"(amax) : "s"(a.eps), "v"(mx));
    // r = fl((L/2) / amax) = (L/2) fl(1/amax) (a power-of-two multiple);
    // fp16 inputs keep amax below 2^25
    float rs;
    if (std::is_same<InT, __half>::value || amax < 0x1p126f)
      rs = __fmul_rn(rcp_rn(amax), kr);
    else
      rs = __fmul_rn(__fdiv_rn(a.half_L, amax), kq);
    uint32_t code;
    uint64_t cball;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(v[k], rs);
    int c;
    bool near;
    if (BITS == 2) {
      e8_decode2<STRICT>(y, code, cball, c, near);
    } else {
      float mgn;
      e8_decode<BITS, STRICT, float>(y, code, c, &mgn);
      near = mgn < kNearTie;
      cball = __ballot(c);
    }
    {
      // a vector with any near-tie group goes to the fp64 pass
      const uint64_t nb = __ballot(near);
      if (nb != 0) {
        const bool lead = l == 0 && tvalid && ((nb >> row_shift) & kRowMask) != 0;
        queue_push(qslot, lead, it, row);
      }
    }
    if (STRICT && a.compact) code = Compact<BITS>::fold(code, c);
    const uint64_t cmask = coset_rows<VL>(cball);
    const int slot = it & (gl - 1);
    if (mg == slot) keep = amax;
    if (tvalid) {
      uint8_t* cp = cb + oc;
      if (BITS == 2) {
        *reinterpret_cast<uint16_t*>(cp) = (uint16_t)code;
      } else {
        cp[0] = (uint8_t)(code & 0xffu);
        cp[1] = (uint8_t)((code >> 8) & 0xffu);
        cp[2] = (uint8_t)(code >> 16);
      }
      if (m == 0 && !a.compact) {
        const uint32_t cw = (uint32_t)(cmask >> row_shift) & kRowMask;
        uint8_t* q = qb + os;
        if (VL > 8) *reinterpret_cast<uint16_t*>(q) = (uint16_t)cw;
        else q[0] = (uint8_t)cw;
      }
    }
    if (slot == gl - 1 || it == n_it - 1) {
      if (tvalid && mg <= slot) {
        char* sb = gb + (int64_t)(it - slot) * plane_g * 2;
        *reinterpret_cast<uint16_t*>(sb + off_gb) =
            f64_to_f16_rn((double)keep * a.sigma_k);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Keys with split-half RoPE at d = n = 128, fp16 input, one or two scales
// per vector: the RoPE removal fused with the stride-64 butterfly.
//
// Lane l of an 8-lane row holds input coordinates 8m .. 8m+7 and their RoPE
// partners 64 + 8m .. 64 + 8m+7 (m = lane_group(l), l < 8).  For a pair
// (i, p = i + 64) whose angle has cosine c and sine s, the removal gives
// x'_i = x_i c + x_p s and x'_p = x_p c - x_i s, and the stride-64 stage of
// the transform then forms
//     x'_i + x'_p = x_i (c - s) + x_p (c + s),
//     x'_i - x'_p = x_i (c + s) - x_p (c - s),
// each as one rounded product and one fused multiply-add straight from the
// fp16 words (v_fma_mix), with the lane's (c - s, c + s) in registers: no
// partner exchange and one cross-lane stage fewer than the fast path.
// Stages 1, 2, 4 run inside the lane on both halves, stages 8, 16, 32
// across the 8 lanes through DPP with the fast path's sign twist (the GF(2)
// lane relabelling restricted to a = (1, 2, 7)).  The lane then holds output
// groups m and m + 8 and decodes both.  The fp32 rounding order differs from
// the textbook one; the decision margins and the fp64 pass make the codes
// those of the fp64 definition all the same.
// ---------------------------------------------------------------------------

// x_i (c - s) + x_p (c + s) and x_i (c + s) - x_p (c - s) for the two pairs
// of one 32-bit word of fp16 inputs (lo: word wi, partner word wp).
#define NQ_PAIR_HALF(SEL, wi, wp, cm, cp, lo, hi)                                 \
  do {                                                                            \
    float t1_, t2_;                                                               \
    asm("v_fma_mix_f32 %2, %5, %7, 0 op_sel:[" SEL ",0,0] op_sel_hi:[1,0,0]\n\t"    \
        "v_fma_mix_f32 %3, %5, %6, 0 op_sel:[" SEL ",0,0] op_sel_hi:[1,0,0]\n\t"    \
        "v_fma_mix_f32 %0, %4, %6, %2 op_sel:[" SEL ",0,0] op_sel_hi:[1,0,0]\n\t"   \
        "v_fma_mix_f32 %1, %4, %7, -%3 op_sel:[" SEL ",0,0] op_sel_hi:[1,0,0]"      \
        : "=&v"(lo), "=&v"(hi), "=&v"(t1_), "=&v"(t2_)                            \
        : "v"(wi), "v"(wp), "v"(cm), "v"(cp));                                    \
  } while (0)

__device__ __forceinline__ void rope_stage64(const uint4& wl, const uint4& wh,
                                             const float cm[8], const float cp[8],
                                             float lo[8], float hi[8]) {
  const uint32_t ui[4] = {wl.x, wl.y, wl.z, wl.w};
  const uint32_t up[4] = {wh.x, wh.y, wh.z, wh.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    NQ_PAIR_HALF("0", ui[i], up[i], cm[2 * i], cp[2 * i], lo[2 * i], hi[2 * i]);
    NQ_PAIR_HALF("1", ui[i], up[i], cm[2 * i + 1], cp[2 * i + 1], lo[2 * i + 1], hi[2 * i + 1]);
  }
}

// max |v_k| over 16 values
__device__ __forceinline__ float abs_max16(const float a[8], const float b[8]) {
  float m;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|\n\t"
      "v_max3_f32 %0, %0, |%4|, |%5|\n\t"
      "v_max3_f32 %0, %0, |%6|, |%7|\n\t"
      "v_max3_f32 %0, %0, |%8|, |%9|\n\t"
      "v_max3_f32 %0, %0, |%10|, |%11|\n\t"
      "v_max3_f32 %0, %0, |%12|, |%13|\n\t"
      "v_max3_f32 %0, %0, |%14|, |%15|\n\t"
      "v_max_f32_e64 %0, %0, |%16|"
      : "=&v"(m)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
        "v"(a[7]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]),
        "v"(b[6]), "v"(b[7]));
  return m;
}

// One 8-group: scale, decode, margin.  `code` gets the packed indices (with
// the coset bit folded in for compact packing), `c` the coset.
template <int BITS, bool STRICT>
__device__ __forceinline__ void pair_decode(const float v[8], float rs, int compact,
                                            uint32_t& code, uint64_t& cball, bool& near) {
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(v[k], rs);
  int c;
  if (BITS == 2) {
    e8_decode2<STRICT>(y, code, cball, c, near);
  } else {
    float mgn;
    e8_decode<BITS, STRICT, float>(y, code, c, &mgn);
    near = mgn < kNearTie;
    cball = __ballot(c);
  }
  if (STRICT && compact) code = Compact<BITS>::fold(code, c);
}

template <int BITS>
__device__ __forceinline__ void store_code(uint8_t* p, uint32_t code) {
  if (BITS == 2) {
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)code;
  } else {
    p[0] = (uint8_t)(code & 0xffu);
    p[1] = (uint8_t)((code >> 8) & 0xffu);
    p[2] = (uint8_t)(code >> 16);
  }
}

// NS scales per vector: 1 (G = 128) or 2 (G = 64, one per half).
template <int BITS, bool STRICT, int NS>
__global__ __launch_bounds__(kBlock) void quantize_pair_kernel(TensorArgs a, int sh_chunk) {
  constexpr int TPW = 8;          // tokens per wave iteration
  constexpr int BATCH = 8 / NS;   // iterations per batch of scale stores
  const int lane = threadIdx.x & 63;
  const int row = lane >> 3;
  const int l = lane & 7;
  const int m = lane_group(l);
  const int64_t n_tt = (a.T + TPW - 1) / TPW;
  const int64_t SH = a.n_vec / a.T;
  const int64_t wave = xcd_wave_id();
  const int64_t n_shc = (SH + sh_chunk - 1) / sh_chunk;
  const int64_t tt = wave / n_shc;
  const int64_t sh0 = (wave % n_shc) * sh_chunk;
  if (tt >= n_tt) return;
  const int64_t sh1 = min64(SH, sh0 + sh_chunk);
  const int64_t t = tt * TPW + row;
  __shared__ QueueSlot qslots[kBlock / 64];
  QueueSlot* qslot = &qslots[threadIdx.x >> 6];
  queue_slot_init(qslot, a, sh0 * a.T + tt * TPW);
  const bool tvalid = t < a.T;
  const int64_t tc = tvalid ? t : a.T - 1;
  const int j0 = 8 * m;

  // (c - s, c + s) of the lane's 8 pairs for its token
  float cm[8], cp[8];
  {
    const float2* rp = a.rope + tc * 64 + j0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float2 cs = rp[k];
      cm[k] = __fsub_rn(cs.x, cs.y);
      cp[k] = __fadd_rn(cs.x, cs.y);
    }
  }
  const float coef0 = (m & 1) ? -1.f : 1.f;
  const float coef1 = (m & 2) ? -1.f : 1.f;
  const float coef2 = (m & 4) ? -1.f : 1.f;
  const bool neg_sigma = (__builtin_popcount(m) & 1) != 0;
  const float kr = (neg_sigma ? -a.half_L : a.half_L) * (BITS == 2 ? 2.f : 1.f);
  const int row_shift = row * 8;
  // scale batching: lane m keeps scale (m % NS) of iteration m / NS of the batch
  const int mi = m / NS;
  const int which = m % NS;

  // per-lane byte offsets inside one (slab, head) plane (below 2^31: the
  // host checks); the plane bases advance uniformly
  const uint32_t off_x = (uint32_t)(tc * 128 + j0) * 2u;
  const uint32_t off_c = (uint32_t)(tc * a.code_bytes) + (uint32_t)(m * BITS);
  const uint32_t off_s = (uint32_t)(tc * a.coset_bytes);
  const int64_t plane_x = a.T * 128 * 2;
  const int64_t plane_c = a.pT * a.code_bytes;
  const int64_t plane_s = a.pT * a.coset_bytes;
  const int64_t plane_g = a.pT * NS;
  const uint32_t off_gb = ((uint32_t)(tc * NS + which) + (uint32_t)mi * (uint32_t)plane_g) * 2u;
  float keep = 0.f;
  const int n_it = (int)(sh1 - sh0);
  const char* xb = static_cast<const char*>(a.x) + sh0 * plane_x;
  uint8_t* cbp = a.codes + sh0 * plane_c;
  uint8_t* qb = a.cosets + sh0 * plane_s;
  char* gb = reinterpret_cast<char*>(a.scales) + sh0 * plane_g * 2;
  uint32_t ox = off_x, oc = off_c, os = off_s;
  for (int it = 0; it < n_it; ++it, xb += plane_x, cbp += plane_c, qb += plane_s) {
    asm volatile("" : "+v"(ox), "+v"(oc), "+v"(os));
    const uint4 wl = *reinterpret_cast<const uint4*>(xb + ox);
    const uint4 wh = *reinterpret_cast<const uint4*>(xb + ox + 128);
    float lo[8], hi[8];
    rope_stage64(wl, wh, cm, cp, lo, hi);
    fwht_lane(lo);
    fwht_lane(hi);
    stage_fmac<0>(lo, coef0);
    stage_fmac<0>(hi, coef0);
    stage_fmac<1>(lo, coef1);
    stage_fmac<1>(hi, coef1);
    stage_fmac<2>(lo, coef2);
    stage_fmac<2>(hi, coef2);
    float amax_lo, amax_hi, rs_lo, rs_hi;
    if (NS == 1) {
      float mx = abs_max16(lo, hi);
      mx = group_max<8>(mx, 8);
      asm("v_max_f32 %0, %1, %2" : "=v"(amax_lo) : "s"(a.eps), "v"(mx));
      amax_hi = amax_lo;
      // r = fl((L/2) / amax) = (L/2) fl(1/amax); fp16 inputs keep amax < 2^25
      rs_lo = __fmul_rn(rcp_rn(amax_lo), kr);
      rs_hi = rs_lo;
    } else {
      float ml = abs_max8(lo), mh = abs_max8(hi);
      ml = group_max<8>(ml, 8);
      mh = group_max<8>(mh, 8);
      asm("v_max_f32 %0, %1, %2" : "=v"(amax_lo) : "s"(a.eps), "v"(ml));
      asm("v_max_f32 %0, %1, %2" : "=v"(amax_hi) : "s"(a.eps), "v"(mh));
      rs_lo = __fmul_rn(rcp_rn(amax_lo), kr);
      rs_hi = __fmul_rn(rcp_rn(amax_hi), kr);
    }
    uint32_t code_lo, code_hi;
    uint64_t cb_lo, cb_hi;
    bool near_lo, near_hi;
    pair_decode<BITS, STRICT>(lo, rs_lo, a.compact, code_lo, cb_lo, near_lo);
    pair_decode<BITS, STRICT>(hi, rs_hi, a.compact, code_hi, cb_hi, near_hi);
    {
      // a vector with any near-tie group goes to the fp64 pass
      const uint64_t nb = __ballot(near_lo || near_hi);
      if (nb != 0) {
        const bool lead = l == 0 && tvalid && ((nb >> row_shift) & 0xffull) != 0;
        queue_push(qslot, lead, it, row);
      }
    }
    const uint64_t cm_lo = coset_rows<8>(cb_lo);
    const uint64_t cm_hi = coset_rows<8>(cb_hi);
    const int slot = it & (BATCH - 1);
    if (mi == slot) keep = (NS == 2 && which) ? amax_hi : amax_lo;
    if (tvalid) {
      store_code<BITS>(cbp + oc, code_lo);
      store_code<BITS>(cbp + oc + 8 * BITS, code_hi);
      if (l == 0 && !a.compact) {
        const uint32_t cw = (uint32_t)((cm_lo >> row_shift) & 0xffull) |
                            ((uint32_t)((cm_hi >> row_shift) & 0xffull) << 8);
        *reinterpret_cast<uint16_t*>(qb + os) = (uint16_t)cw;
      }
    }
    if (slot == BATCH - 1 || it == n_it - 1) {
      if (tvalid && mi <= slot) {
        char* sb = gb + (int64_t)(it - slot) * plane_g * 2;
        *reinterpret_cast<uint16_t*>(sb + off_gb) = f64_to_f16_rn((double)keep * a.sigma_k);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Quantize with the rotation on the matrix cores: vectors without RoPE
// (values, or keys when no RoPE is removed), n = 128 with d = 128 or 96 (the
// lanes of the padding coordinates feed zeros), 2-bit codes, one scale per
// vector (NS = 1) or per 64 coordinates (NS = 2), fp16 input.
//
// The Walsh-Hadamard product u = H x of 16 vectors is a 128 x 128 by
// 128 x 16 matrix product: 8 output tiles x 4 K chunks of
// v_mfma_f32_16x16x32_f16.  The inputs are fp16 numbers and the entries of H
// are +-1, so every product is exact and only the fp32 sums round.  Both
// sides are relabelled.  Lane l (v = l & 15, p = l >> 4) feeds K slot 8p + j
// of chunk k with input coordinate j + 8k + 32p of vector v (its four chunks
// are one 64-byte run), and row m of output tile tau is output coordinate
//     (m & 3) + 4 (tau & 1) + 8 (tau >> 1) + 32 (m >> 2).
// Then (-1)^popcount(out & in) splits into a per-lane pattern chosen by
// tau & 1 times the tile-uniform sign (-1)^((tau >> 1 & 1) (k & 1) +
// (tau >> 2) (k >> 1)), so four fragments of H (two patterns and their
// negatives) serve all 32 products.  Lane l receives rows 4p .. 4p+3 of
// column v of every tile: the 8-groups 4p + h (h = tau >> 1) of vector v,
// element e of group h at tile 2h + (e >> 2), row e & 3, so each lane decodes
// four consecutive groups and stores their 8 code bytes at once.
//
// Waves walk kQmChunk (slab, head) planes of one 16-token tile, and
// neighbouring waves take neighbouring tiles of the same planes, so the
// loads in flight at any time cover a few contiguous stretches of each plane.
// ---------------------------------------------------------------------------
typedef _Float16 nq_f16x8 __attribute__((ext_vector_type(8)));

constexpr int kQmChunk = 8;  // (slab, head) planes per wave

template <bool STRICT, int NS>
__global__ __launch_bounds__(kBlock) void quantize_mfma_kernel(TensorArgs a, int sh_chunk) {
  static_assert(NS == 1 || NS == 2, "one scale per vector or per 64 coordinates");
  const int lane = threadIdx.x & 63;
  const int v = lane & 15;
  const int p = lane >> 4;
  const int64_t n_tt = (a.T + 15) / 16;
  const int64_t SH = a.n_vec / a.T;
  const int64_t wave = xcd_wave_id();
  const int64_t tt = wave % n_tt;
  const int64_t sh0 = (wave / n_tt) * sh_chunk;
  if (sh0 >= SH) return;
  const int64_t sh1 = min64(SH, sh0 + sh_chunk);
  const int64_t t = tt * 16 + v;
  __shared__ QueueSlot qslots[kBlock / 64];
  QueueSlot* qslot = &qslots[threadIdx.x >> 6];
  queue_slot_init(qslot, a, sh0 * a.T + tt * 16);
  const bool tvalid = t < a.T;
  const int64_t tc = tvalid ? t : a.T - 1;

  // H's fragments: the two per-lane sign patterns and their negatives
  nq_f16x8 Ap[2], An[2];
#pragma unroll
  for (int t0 = 0; t0 < 2; ++t0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int par =
          __builtin_popcount(v & j & 3) + t0 * (j >> 2) + __builtin_popcount((v >> 2) & p);
      Ap[t0][j] = (par & 1) ? (_Float16)-1.0f : (_Float16)1.0f;
      An[t0][j] = (par & 1) ? (_Float16)1.0f : (_Float16)-1.0f;
    }
  }
  const float kr = a.half_L * 2.f;  // the 2-bit decoder works on g = 2y

  // input rows of d fp16 (d = 96 or 128): lane p feeds coordinates
  // 32p .. 32p+31, zeros (no load) where they are padding
  const int row_x = 2 * a.d;
  const bool data_lane = 32 * p < a.d;
  const uint32_t off_x = (uint32_t)(tc * row_x) + 64u * (uint32_t)p;
  const uint32_t off_c = (uint32_t)(tc * a.code_bytes) + 8u * (uint32_t)p;
  const uint32_t off_s = (uint32_t)(tc * a.coset_bytes);
  const int64_t plane_x = a.T * row_x;
  const int64_t plane_c = a.pT * a.code_bytes;
  const int64_t plane_s = a.pT * a.coset_bytes;
  const int64_t plane_g = a.pT * NS;  // NS fp16 scales per vector
  // scale batching: lane p stores scale (p >> 1 for NS = 2) of iteration
  // it0 + p (NS = 1) or it0 + (p & 1) (NS = 2) of a batch starting at it0
  const int which = NS == 2 ? (p >> 1) : 0;
  const int mi = NS == 2 ? (p & 1) : p;
  const uint32_t off_gb = (uint32_t)(tc * NS + which + (int64_t)mi * plane_g) * 2u;
  const int n_it = (int)(sh1 - sh0);
  const char* xb = static_cast<const char*>(a.x) + sh0 * plane_x;
  uint8_t* cb = a.codes + sh0 * plane_c;
  uint8_t* qb = a.cosets + sh0 * plane_s;
  char* gb = reinterpret_cast<char*>(a.scales) + sh0 * plane_g * 2;
  uint32_t ox = off_x, oc = off_c, os = off_s;
  float keep = 0.f;
  // the next plane's input is in flight while one is decoded (zeros on
  // padding lanes)
  uint4 nxt[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    nxt[k] = data_lane ? *reinterpret_cast<const uint4*>(xb + ox + 16 * k) : make_uint4(0, 0, 0, 0);
  for (int it = 0; it < n_it; ++it, xb += plane_x, cb += plane_c, qb += plane_s) {
    asm volatile("" : "+v"(ox), "+v"(oc), "+v"(os));
    uint4 raw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[k] = nxt[k];
    if (it + 1 < n_it && data_lane) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        nxt[k] = *reinterpret_cast<const uint4*>(xb + plane_x + ox + 16 * k);
    }
    nq_f4 acc[8];
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) acc[tau] = nq_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const nq_f16x8 B = __builtin_bit_cast(nq_f16x8, raw[k]);
#pragma unroll
      for (int tau = 0; tau < 8; ++tau) {
        const bool neg = ((((tau >> 1) & 1) * (k & 1) + ((tau >> 2) & 1) * (k >> 1)) & 1) != 0;
        acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(neg ? An[tau & 1] : Ap[tau & 1], B,
                                                          acc[tau], 0, 0, 0);
      }
    }
    // maximum of |u| over the scale group: the lane's 32 values, then the
    // lanes of the vector 16 apart (lanes p, p ^ 1 hold coordinates 0..63 or
    // 64..127) and, with one scale per vector, 32 apart
    float mx = 0.f;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[tau][r]));
    {
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                        false, false);
      mx = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
      if (NS == 1) {
        const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                          __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
      }
    }
    float amax;
    asm("v_max_f32 %0, %1, %2" : "=v"(amax) : "s"(a.eps), "v"(mx));
    const float rs = __fmul_rn(rcp_rn(amax), kr);
    uint32_t cw = 0, words[2] = {0u, 0u};
    bool near_any = false;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = __fmul_rn(acc[2 * h + (e >> 2)][e & 3], rs);
      uint32_t code;
      uint64_t cball;
      int c;
      bool near;
      e8_decode2<STRICT>(y, code, cball, c, near);
      near_any = near_any || near;
      if (STRICT && a.compact) code = Compact<2>::fold(code, c);
      cw |= (uint32_t)c << h;
      words[h >> 1] |= code << (16 * (h & 1));
    }
    {
      // token v's groups sit in lanes v, v + 16, v + 32, v + 48
      const uint64_t nb = __ballot(near_any);
      if (nb != 0) {
        const uint64_t f = nb | (nb >> 16) | (nb >> 32) | (nb >> 48);
        const bool lead = p == 0 && tvalid && ((f >> v) & 1u) != 0;
        queue_push(qslot, lead, it, v);
      }
    }
    if (tvalid) *reinterpret_cast<uint2*>(cb + oc) = make_uint2(words[0], words[1]);
    // coset word of the vector: bits 4p .. 4p+3 from lane p
    {
      uint32_t x = cw << (4 * p);
      const auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
      x = s16[0] | s16[1];
      const auto s32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      x = s32[0] | s32[1];
      if (tvalid && p == 0 && !a.compact) *reinterpret_cast<uint16_t*>(qb + os) = (uint16_t)x;
    }
    // scales: in batches of 4 / NS iterations, lane p keeps and stores the
    // scale `which` of the batch's iteration mi
    constexpr int BATCH = 4 / NS;
    const int slot = it & (BATCH - 1);
    if (mi == slot) keep = amax;
    if (slot == BATCH - 1 || it == n_it - 1) {
      if (tvalid && mi <= slot) {
        char* sb = gb + (int64_t)(it - slot) * plane_g * 2;
        *reinterpret_cast<uint16_t*>(sb + off_gb) = f64_to_f16_rn((double)keep * a.sigma_k);
      }
    }
  }
}

template <int N, int BITS, bool STRICT, typename InT>
__global__ __launch_bounds__(kBlock) void quantize_kernel(TensorArgs a) {
  constexpr int VL = N / 8;
  constexpr int VPB = kBlock / VL;
  const int m = threadIdx.x % VL;
  const int64_t vec = (int64_t)blockIdx.x * VPB + threadIdx.x / VL;
  const bool live = vec < a.n_vec;
  const int64_t vv = live ? vec : 0;
  const int j0 = 8 * m;
  float v[8];
  if (j0 < a.d) {
    Io<InT>::load8(a.x, vv * a.d + j0, v);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.f;
  }
  const int64_t t = vv % a.T;
  const int64_t pvec = (vv - t) / a.T * a.pT + t;   // index in the packed planes
  if (a.rope != nullptr) rope_lane<true>(v, m, a.d, a.rope + t * (a.d >> 1));
  fwht_lane(v);
  fwht_cross<VL>(v, m);
  float mx = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fabsf(v[k]));
  const int gl = a.G >> 3;
  for (int s = 1; s < gl; s <<= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
  const float amax = fmaxf(mx, a.eps);
  const float r = __fdiv_rn(a.half_L, amax);
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(v[k], r);
  uint32_t code;
  int c;
  float mgn;
  e8_decode<BITS, STRICT, float>(y, code, c, &mgn);
  const uint64_t bal = __ballot(c);
  {
    const uint64_t nb = __ballot(mgn < kNearTie);
    if (nb != 0) {
      __shared__ QueueSlot qslots[kBlock / 64];
      QueueSlot* qslot = &qslots[threadIdx.x >> 6];
      queue_slot_init(qslot, a, vv - (threadIdx.x & 63) / VL);
      const int lane = threadIdx.x & 63;
      const uint64_t rows = nb >> (lane - m);
      const bool lead = m == 0 && live &&
                        (rows & (VL >= 64 ? ~0ull : ((1ull << VL) - 1ull))) != 0;
      queue_push(qslot, lead, 0, lane / VL);
    }
  }
  if (!live) return;
  if (STRICT && a.compact) code = Compact<BITS>::fold(code, c);
  uint8_t* cp = a.codes + pvec * a.code_bytes + m * BITS;
  if (BITS == 2) {
    *reinterpret_cast<uint16_t*>(cp) = (uint16_t)code;
  } else {
    cp[0] = (uint8_t)(code & 0xffu);
    cp[1] = (uint8_t)((code >> 8) & 0xffu);
    cp[2] = (uint8_t)(code >> 16);
  }
  if (m == 0 && !a.compact) {
    const int lane = threadIdx.x & 63;
    const uint32_t bits = (uint32_t)(bal >> lane) &
                          (VL >= 32 ? 0xffffffffu : ((1u << VL) - 1u));
    uint8_t* q = a.cosets + pvec * a.coset_bytes;
    for (int b = 0; b < a.coset_bytes; ++b) q[b] = (uint8_t)(bits >> (8 * b));
  }
  if (m % gl == 0) {
    a.scales[pvec * a.n_scales + m / gl] = f64_to_f16_rn((double)amax * a.sigma_k);
  }
}

template <typename T>
struct OutIo;
// Dequantized output: written once, read by a later consumer, and far
// larger than the caches, so the stores are non-temporal (they do not fill
// the L2 with dirty lines that a following kernel then has to wait behind).
constexpr int kStoreNT = 2;   // cache-policy bits of a raw buffer store: nt

template <>
struct OutIo<__half> {
  // fp16 RNE, two values per v_cvt_pk_f16_f32; `flip` xors the sign bits
  static __device__ __forceinline__ void store8(void* base, int64_t off,
                                                const float v[8], uint32_t flip) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = __builtin_bit_cast(uint32_t, __floats2half2_rn(v[2 * i], v[2 * i + 1])) ^ flip;
    const nq_u4 w = {u[0], u[1], u[2], u[3]};
    __builtin_nontemporal_store(w, reinterpret_cast<nq_u4*>(static_cast<uint16_t*>(base) + off));
  }
  static constexpr uint32_t kFlip = 0x80008000u;
};
template <>
struct OutIo<float> {
  static __device__ __forceinline__ void store8(void* base, int64_t off,
                                                const float v[8], uint32_t flip) {
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = __uint_as_float(__float_as_uint(v[i]) ^ flip);
    nq_f4* p = reinterpret_cast<nq_f4*>(static_cast<float*>(base) + off);
    __builtin_nontemporal_store(nq_f4{w[0], w[1], w[2], w[3]}, p);
    __builtin_nontemporal_store(nq_f4{w[4], w[5], w[6], w[7]}, p + 1);
  }
  static constexpr uint32_t kFlip = 0x80000000u;
};

// Inverse path with the quantize kernel's wave layout: lane l holds 8-group
// m(l); z = s16 / sqrt(n) * (idx - L/2 + c/2) goes through the same
// sign-twisted DPP butterflies, so lane l ends with sigma_l * x^; sigma_l is
// removed by flipping sign bits at the store.  Keys then get RoPE forward:
// x_i = y_i c - y_{i+h} s, x_{i+h} = y_{i+h} c + y_i s.
template <int N, int BITS, typename OutT, int ROPE, bool CMP>
__global__ __launch_bounds__(kBlock) void dequantize_fast_kernel(TensorArgs a,
                                                                 int sh_chunk,
                                                                 int tile_major) {
  constexpr int VL = N / 8;
  constexpr int TPW = 64 / VL;
  constexpr int L = 1 << BITS;
  const int lane = threadIdx.x & 63;
  const int row = lane / VL;
  const int l = lane % VL;
  const int m = lane_group(l);
  const int64_t n_tt = (a.T + TPW - 1) / TPW;
  const int64_t SH = a.n_vec / a.T;
  const int64_t wave = xcd_wave_id();
  const int64_t n_shc = (SH + sh_chunk - 1) / sh_chunk;
  const int64_t tt = tile_major ? wave / n_shc : wave % n_tt;
  const int64_t sh0 = (tile_major ? wave % n_shc : wave / n_tt) * sh_chunk;
  if (tt >= n_tt || sh0 >= SH) return;
  const int64_t sh1 = min64(SH, sh0 + sh_chunk);
  const int64_t t = tt * TPW + row;
  const bool tvalid = t < a.T;
  const int64_t tc = tvalid ? t : a.T - 1;
  const int j0 = 8 * m;
  const bool data_lane = j0 < a.d;
  const int h = a.d >> 1;
  const int gl = a.G >> 3;
  const bool neg_sigma = (__builtin_popcount(m) & 1) != 0;
  float coef[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) coef[k] = ((m >> k) & 1) ? -1.f : 1.f;

  // RoPE forward, in the twisted frame: lane value w = sigma y, so
  // sigma x = w c + w_partner * (sigma sigma_partner) * s_fwd; for the DPP
  // partner sigma sigma_partner = -1.
  float rc[8], rs[8];
  int pl = 0;
  bool pneg = false;
  if (ROPE != 0) {
    const float2* row_p = a.rope + tc * h;
    int pm = m;
    if (ROPE == 2) {
      const int hl = h >> 3;
      pm = (m < hl) ? m + hl : (m < 2 * hl ? m - hl : m);
      pl = (lane - l) + group_lane(pm);
      pneg = ((__builtin_popcount(m) ^ __builtin_popcount(pm)) & 1) != 0;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k;
      const bool up = j >= h;
      const float2 cs = data_lane ? row_p[up ? j - h : j] : make_float2(0.f, 0.f);
      const float sf = up ? cs.y : -cs.y;        // forward sign
      rc[k] = cs.x;
      rs[k] = (ROPE == 1) ? -sf : (ROPE == 2 ? (pneg ? -sf : sf) : sf);
    }
  }
  const uint32_t flip = neg_sigma ? OutIo<OutT>::kFlip : 0u;

  // code word, coset byte and scale of the next (slab, head) are loaded one
  // iteration ahead
  auto load_meta = [&](int64_t vec, uint32_t& code, uint32_t& cbyte, uint16_t& sbits) {
    const uint8_t* cp = a.codes + vec * a.code_bytes + m * BITS;
    if (BITS == 2) {
      code = *reinterpret_cast<const uint16_t*>(cp);
    } else {
      code = (uint32_t)cp[0] | ((uint32_t)cp[1] << 8) | ((uint32_t)cp[2] << 16);
    }
    cbyte = CMP ? 0u : a.cosets[vec * a.coset_bytes + (m >> 3)];
    sbits = a.scales[vec * a.n_scales + m / gl];
  };  // `vec` indexes the packed planes (token stride pT)
  uint32_t code_n, cbyte_n;
  uint16_t sbits_n;
  load_meta(sh0 * a.pT + tc, code_n, cbyte_n, sbits_n);
  for (int64_t sh = sh0; sh < sh1; ++sh) {
    const int64_t vec = sh * a.T + tc;
    const uint32_t code_r = code_n, cbyte = cbyte_n;
    const uint16_t sbits = sbits_n;
    if (sh + 1 < sh1) load_meta((sh + 1) * a.pT + tc, code_n, cbyte_n, sbits_n);
    int c = (int)((cbyte >> (m & 7)) & 1u);
    const uint32_t code = CMP ? Compact<BITS>::unfold(code_r, c) : code_r;
    const float sc = h2f(sbits) * a.inv_sqrt_n;
    const float off = (0.5f * (float)c - a.half_L) * sc;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t idx = (code >> (BITS * k)) & (uint32_t)(L - 1);
      v[k] = __fmaf_rn((float)idx, sc, off);
    }
    fwht_lane(v);
    if (VL > 1) stage_fmac<0>(v, coef[0]);
    if (VL > 2) stage_fmac<1>(v, coef[1]);
    if (VL > 4) stage_fmac<2>(v, coef[2]);
    if (VL > 8) stage_fmac<3>(v, coef[3]);
    if (ROPE == 1) {
      float pv[8];
      constexpr int KR = N == 128 ? 3 : N == 64 ? 2 : N == 32 ? 1 : 0;
      partner_mul<KR>(pv, v, rs);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __fmaf_rn(v[k], rc[k], pv[k]);
    } else if (ROPE == 2) {
      float pv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pv[k] = __shfl(v[k], pl);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __fmaf_rn(v[k], rc[k], pv[k] * rs[k]);
    } else if (ROPE == 3) {
      float x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = v[k];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __fmaf_rn(x[k], rc[k], x[k ^ 4] * rs[k]);
    }
    if (tvalid && data_lane) OutIo<OutT>::store8(a.y, vec * a.d + j0, v, flip);
  }
}

// Copies n >= 1 elements from global memory to a wave-private LDS slice: U
// loads per lane are issued before any of them is written, so that they
// are in flight together (a load-then-write loop waits out each one).
// Lanes past the end copy element n - 1 again, onto itself: no write is
// conditional, so the compiler cannot sink a load into a branch.
template <int U, typename E>
__device__ __forceinline__ void wave_copy(E* l, const E* g, int n, int lane) {
  for (int b = 0; b < n; b += 64 * U) {
    E t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) t[u] = g[min(b + lane + 64 * u, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) l[min(b + lane + 64 * u, n - 1)] = t[u];
  }
}

// ---------------------------------------------------------------------------
// Dequantize keys with the rotation on the matrix cores (RoPE, d = n = 128,
// 2-bit codes, one scale per vector, fp16 output).
//
// The B operand of chunk k holds 8-group 4p + k of vector v (lane
// l = 16p + v) as fp16 numbers 1024 + 2 idx + c (2p + 1028 for the codeword
// point p = idx - 2 + c/2): exact, and so is every sum of 128 of them, so
// u' = H (2p + 1028) comes out of the matrix cores exact in fp32.  Since
// H 1 = 128 e_0, H p = (u' - 1028 * 128 e_0) / 2, and x = (s16 / sqrt(n)) H p
// takes one rounded product per coordinate.  Row m of output tile tau is
// output coordinate (m & 7) + 8 (tau & 1) + 16 (tau >> 1 & 1) + 32 (m >> 3)
// + 64 (tau >> 2), so a coordinate and its RoPE partner (+ 64) sit in tiles
// tau and tau ^ 4 of the same lane; (-1)^popcount(out & in) splits into a
// per-lane pattern chosen by tau >> 2 times the tile-uniform sign
// (-1)^((tau & 1)(k & 1) + (tau >> 1 & 1)(k >> 1)).  The fp16 results pass
// through the wave's LDS tile so that every global store writes 1 KiB of
// contiguous output.  Lane l needs cos / sin of its token at the 16 angles
// (coordinate mod 64) 4 p0 + 32 p1 + 8 q0 + 16 q1 + r (q, r < 4).
// ---------------------------------------------------------------------------
struct DmFrags {
  nq_f16x8 Ap[2], An[2];   // H's fragments: two per-lane sign patterns, negated
};

__device__ __forceinline__ DmFrags dm_frags(int v, int p) {
  DmFrags h;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int par = __builtin_popcount(v & j & 7) + ((v >> 3) & 1) * (p & 1) + q * (p >> 1);
      h.Ap[q][j] = (par & 1) ? (_Float16)-1.0f : (_Float16)1.0f;
      h.An[q][j] = (par & 1) ? (_Float16)1.0f : (_Float16)-1.0f;
    }
  }
  return h;
}

__device__ __forceinline__ int dm_freq(int p, int q, int r) {
  return 4 * (p & 1) + 32 * (p >> 1) + 8 * (q & 1) + 16 * (q >> 1) + r;
}

// cos / sin of the lane's 16 angles at position pos (the same values as the
// RoPE table's).  The frequencies are read 8 at a time before any of them
// is used, so their loads are in flight together.
__device__ __forceinline__ void dm_cos_sin(double pos, const RopeFreqs& f, int p,
                                           float (&rc)[4][4], float (&rn)[4][4]) {
#pragma unroll
  for (int q0 = 0; q0 < 4; q0 += 2) {
    double om[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) om[q][r] = f.omega[dm_freq(p, q0 + q, r)];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) rope_cos_sin(pos, om[q][r], rc[q0 + q][r], rn[q0 + q][r]);
  }
}

// A lane's packed words of one token: code word pair (8-groups 4p .. 4p + 3),
// coset bits, scale bits.
struct DmMeta {
  uint2 cw;
  uint32_t cs, sb;
};

// Raw buffer (gfx9-family format word) over `bytes` bytes (< 2^31) at p.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dm_rsrc(char* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)bytes, 0x00020000);
}

// One 16-token tile of one plane -> 16 rows of 256 B at byte yoff of the
// buffer yr.  Rows from `rows` on are not stored: their stores take an
// offset past the buffer's end, which the hardware drops, so no store is
// conditional and the compiler's wait counts stay exact.  The stores are
// non-temporal, as every dequantized output is.  ROPE = false skips the
// rotation (rc, rn unused).
template <bool CMP, bool ROPE = true>
__device__ __forceinline__ void dm_tile(const DmFrags& h, const DmMeta& m, float half_rs,
                                        const float (&rc)[4][4], const float (&rn)[4][4],
                                        char* tile, int v, int p, __amdgpu_buffer_rsrc_t yr,
                                        uint32_t yoff, int rows) {
  nq_f4 acc[8];
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) acc[tau] = nq_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t w = ((k < 2 ? m.cw.x : m.cw.y) >> (16 * (k & 1))) & 0xffffu;
    int c = (int)((m.cs >> (4 * p + k)) & 1u);
    if (CMP) w = Compact<2>::unfold(w, c);
    // fp16 1024 + 2 idx + c for the group's 8 coordinates, two per word
    const uint32_t base = 0x64006400u | (c ? 0x00010001u : 0u);
    uint32_t bw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t nib = (w >> (4 * q)) & 0xfu;
      bw[q] = (((nib | (nib << 14)) & 0x00030003u) << 1) | base;
    }
    const nq_f16x8 B = __builtin_bit_cast(nq_f16x8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      const bool neg = (((tau & 1) * (k & 1) + ((tau >> 1) & 1) * (k >> 1)) & 1) != 0;
      acc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_f16(neg ? h.An[tau >> 2] : h.Ap[tau >> 2], B,
                                                        acc[tau], 0, 0, 0);
    }
  }
  // coordinate 0 (lane p = 0, tile 0, row 0) carries the 1028 * 128 offset
  if (p == 0) acc[0][0] -= 131584.f;
  const float f = h2f((uint16_t)m.sb) * half_rs;
  // per pair of tiles (q, q + 4): scale, RoPE forward (x_i c - x_{i+64} s
  // in the lower half, x_{i+64} c + x_i s in the upper), fp16 results into
  // the wave's LDS tile (16 tokens x 256 B; the 16-byte chunks of token row
  // v rotated by v against bank conflicts)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float xl[4], xu[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lo = acc[q][r] * f, up = acc[q + 4][r] * f;
      if (ROPE) {
        xl[r] = __fmaf_rn(lo, rc[q][r], -(up * rn[q][r]));
        xu[r] = __fmaf_rn(up, rc[q][r], lo * rn[q][r]);
      } else {
        xl[r] = lo;
        xu[r] = up;
      }
    }
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const float* x = hi ? xu : xl;
      const int tau = q + 4 * hi;
      const uint32_t u0 = __builtin_bit_cast(uint32_t, __floats2half2_rn(x[0], x[1]));
      const uint32_t u1 = __builtin_bit_cast(uint32_t, __floats2half2_rn(x[2], x[3]));
      // byte 8 p0 + 64 p1 + 16 tau0 + 32 tau1 + 128 tau2 of row v
      const int ch = 4 * (p >> 1) + (tau & 1) + 2 * ((tau >> 1) & 1) + 8 * (tau >> 2);
      *reinterpret_cast<uint2*>(tile + v * 256 + ((ch ^ v) << 4) + 8 * (p & 1)) =
          make_uint2(u0, u1);
    }
    // one pair at a time: the scheduler would otherwise form every pair's
    // products first and hold them all in registers
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // store i, lane l: token row 4i + p of the tile, 16-byte chunk v
    const int row = 4 * i + p;
    const uint4 val = *reinterpret_cast<const uint4*>(tile + row * 256 + ((v ^ row) << 4));
    const uint32_t off = row < rows ? yoff + 1024u * i + 16u * (16u * p + v) : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(nq_u4, val), yr, (int)off, 0,
                                           kStoreNT);
  }
  __builtin_amdgcn_wave_barrier();
}

// Plane-walking form (explicit positions): a wave keeps its 16-token tile
// (and the tile's cos / sin in registers) while it walks kDmChunk (slab,
// head) planes; neighbouring waves take neighbouring tiles.
constexpr int kDmChunk = 32;

template <bool CMP>
__global__ __launch_bounds__(kBlock) void dequantize_mfma_kernel(TensorArgs a, int sh_chunk,
                                                                 RopeFreqs f) {
  const int lane = threadIdx.x & 63;
  const int v = lane & 15;
  const int p = lane >> 4;
  const int64_t n_tt = (a.T + 15) / 16;
  const int64_t SH = a.n_vec / a.T;
  const int64_t wave = xcd_wave_id();
  const int64_t tt = wave % n_tt;
  const int64_t sh0 = (wave / n_tt) * sh_chunk;
  if (sh0 >= SH) return;
  const int64_t sh1 = min64(SH, sh0 + sh_chunk);
  const int64_t t = tt * 16 + v;
  const int64_t tc = t < a.T ? t : a.T - 1;
  const DmFrags h = dm_frags(v, p);
  // this lane's cos / sin, formed once for all the wave's planes (the same
  // values as the RoPE table's)
  float rc[4][4], rn[4][4];
  dm_cos_sin(a.positions != nullptr ? (double)a.positions[tc] : (double)(a.pos0 + tc), f, p, rc,
             rn);
  const float half_rs = 0.5f * a.inv_sqrt_n;
  const uint32_t off_c = (uint32_t)(tc * a.code_bytes) + 8u * (uint32_t)p;
  const uint32_t off_s = (uint32_t)(tc * a.coset_bytes);
  const uint32_t off_g = (uint32_t)tc * 2u;
  const uint32_t off_y = (uint32_t)(tt * 16 * 256);   // the tile's 4 KiB stretch
  const int rows = (int)min64(16, a.T - tt * 16);
  __shared__ __align__(16) char lds_tiles[kBlock / 64][16 * 256];
  char* tile = lds_tiles[threadIdx.x >> 6];
  const int64_t plane_y = a.T * 256;
  const int64_t plane_c = a.pT * a.code_bytes;
  const int64_t plane_s = a.pT * a.coset_bytes;
  const int64_t plane_g = a.pT * 2;
  const int n_it = (int)(sh1 - sh0);
  char* yb = static_cast<char*>(a.y) + sh0 * plane_y;
  const uint8_t* cb = a.codes + sh0 * plane_c;
  const uint8_t* qb = a.cosets + sh0 * plane_s;
  const char* gb = reinterpret_cast<const char*>(a.scales) + sh0 * plane_g;
  // plane min(it, n_it - 1): the one-ahead load past the last plane reloads it
  auto load_meta = [&](int it, DmMeta& m) {
    const int q = min(it, n_it - 1);
    m.cw = *reinterpret_cast<const uint2*>(cb + q * plane_c + off_c);
    m.cs = CMP ? 0u : (uint32_t)*reinterpret_cast<const uint16_t*>(qb + q * plane_s + off_s);
    m.sb = (uint32_t)*reinterpret_cast<const uint16_t*>(gb + q * plane_g + off_g);
  };
  auto step = [&](int it, const DmMeta& m) {
    dm_tile<CMP>(h, m, half_rs, rc, rn, tile, v, p, dm_rsrc(yb + it * plane_y, plane_y), off_y,
                 rows);
  };
  // the next plane's words are loaded one ahead, into two register sets used
  // in turn, so that no copy of a word still in flight makes the wave wait
  DmMeta m0, m1;
  load_meta(0, m0);
#pragma unroll 1
  for (int it = 0; it < n_it; it += 2) {
    load_meta(it + 1, m1);
    step(it, m0);
    if (it + 1 >= n_it) break;
    load_meta(it + 2, m0);
    step(it + 1, m1);
  }
}

// Token-walking form (positions pos0 + t): a wave walks a run of kDtRun
// tiles of one (slab, head) plane, so each wave writes one contiguous
// stretch of output (32 KiB).  It copies the packed words of kDtChunk tiles
// at a time into its LDS slice; the tiles of a chunk then issue no global
// load, only stores, which therefore never wait for one another (with a
// tile's words loaded from global memory in the loop, the wait for them also
// waited out the previous tile's stores).  The lane's cos / sin are formed
// at the run's first tile and rotated by the angle of 16 tokens
// (host-computed cos / sin of 16 omega) from tile to tile: after at most
// kDtRun - 1 rotations they are within 4e-7 of the directly formed
// values.  Runs of one chunk measured faster than runs of 16 or 32 tiles,
// although each run forms its 16 cos / sin pairs afresh.  Without ROPE
// (values, keys with theta = 0) no cos / sin are formed and the tile is
// only scaled; f is then not read.  One scale per vector only: with a scale
// per 64 coordinates the scales would apply before the inverse rotation,
// inside the product, not to its output.
constexpr int kDtRun = 8;
// Runs without RoPE (no cos / sin to form): 4 tiles measured fastest
// (0.417 ms at the Llama values against 0.436 / 0.453 / 0.614 ms for runs
// of 8 / 2 / 1 and 0.474 / 0.494 ms for 16 / 32; keys with RoPE took
// 0.538 ms with runs of 4 against 0.452 ms with runs of 8).
constexpr int kDtRunV = 4;
constexpr int kDtChunk = 8;
constexpr int kDtTok = 16 * kDtChunk;   // tokens per chunk

template <bool CMP, bool ROPE>
__global__ __launch_bounds__(kBlock) void dequantize_mfma_tw_kernel(TensorArgs a, RopeFreqs f) {
  const int lane = threadIdx.x & 63;
  const int v = lane & 15;
  const int p = lane >> 4;
  constexpr int kRun = ROPE ? kDtRun : kDtRunV;   // tiles a wave walks
  const int64_t n_tt = (a.T + 15) / 16;
  const int64_t n_run = (n_tt + kRun - 1) / kRun;
  const int64_t SH = a.n_vec / a.T;
  const int64_t wave = xcd_wave_id();
  const int64_t sh = wave / n_run;
  if (sh >= SH) return;                     // whole wave; no block barrier below
  const int64_t tt0 = (wave % n_run) * kRun;
  const int nt = (int)min64((int64_t)16 * kRun, a.T - tt0 * 16);   // tokens of the run
  const int n_it = (nt + 15) / 16;
  // the wave's LDS slice: a chunk's code rows (32 B a token), coset words
  // and scales, then the step's cos / sin for lane group p ([p][0 .. 15]
  // cos, [p][16 .. 31] sin, in (q, r) order)
  __shared__ __align__(16) char lds_meta[kBlock / 64][kDtTok * 36 + 512];
  __shared__ __align__(16) char lds_tiles[kBlock / 64][16 * 256];
  char* mc = lds_meta[threadIdx.x >> 6];
  uint16_t* mq = reinterpret_cast<uint16_t*>(mc + kDtTok * 32);
  uint16_t* mg = mq + kDtTok;
  float* mst = reinterpret_cast<float*>(mc + kDtTok * 36);
  char* tile = lds_tiles[threadIdx.x >> 6];
  if (ROPE) {
    const int k = dm_freq(p, (lane >> 2) & 3, lane & 3);
    mst[32 * p + (lane & 15)] = f.step_c[k];
    mst[32 * p + 16 + (lane & 15)] = f.step_s[k];
  }
  const DmFrags h = dm_frags(v, p);
  float rc[4][4] = {}, rn[4][4] = {};
  if (ROPE) dm_cos_sin((double)(a.pos0 + tt0 * 16 + v), f, p, rc, rn);
  const float4* stp = reinterpret_cast<const float4*>(mst + 32 * p);
  const float half_rs = 0.5f * a.inv_sqrt_n;
  const __amdgpu_buffer_rsrc_t yr =
      dm_rsrc(static_cast<char*>(a.y) + (sh * a.T + tt0 * 16) * 256, (int64_t)nt * 256);
  const int64_t v0 = sh * a.pT + tt0 * 16;
#pragma unroll 1
  for (int c0 = 0; c0 < n_it; c0 += kDtChunk) {
    // the chunk's tokens ct0 .. ct0 + cnt - 1 of the run into the slice (the
    // previous chunk's reads of it have all returned: their values are used)
    const int ct0 = 16 * c0;
    const int cnt = min(kDtTok, nt - ct0);
    wave_copy<2 * kDtTok / 64>(reinterpret_cast<uint4*>(mc),
                               reinterpret_cast<const uint4*>(a.codes + (v0 + ct0) * 32),
                               2 * cnt, lane);
    if (!CMP)
      wave_copy<kDtTok / 64>(mq, reinterpret_cast<const uint16_t*>(a.cosets) + v0 + ct0, cnt,
                             lane);
    wave_copy<kDtTok / 64>(mg, a.scales + v0 + ct0, cnt, lane);
    // the slice is written and read by this wave only; the wait makes the
    // copies visible
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    const int c1 = min(n_it, c0 + kDtChunk);
#pragma unroll 1
    for (int it = c0; it < c1; ++it) {
      const int t = min(16 * it + v, nt - 1) - ct0;   // token within the chunk
      DmMeta m;
      m.cw = *reinterpret_cast<const uint2*>(mc + 32 * t + 8 * p);
      m.cs = CMP ? 0u : (uint32_t)mq[t];
      m.sb = (uint32_t)mg[t];
      dm_tile<CMP, ROPE>(h, m, half_rs, rc, rn, tile, v, p, yr, 4096u * (uint32_t)it,
                   min(16, nt - 16 * it));
      // the step's cos / sin are read after the tile, not held through it
      __builtin_amdgcn_sched_barrier(0);
      if (!ROPE) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 dc4 = stp[q], dn4 = stp[4 + q];
        const float dc[4] = {dc4.x, dc4.y, dc4.z, dc4.w}, dn[4] = {dn4.x, dn4.y, dn4.z, dn4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float c = rc[q][r], sn = rn[q][r];
          rc[q][r] = __fmaf_rn(c, dc[r], -(sn * dn[r]));
          rn[q][r] = __fmaf_rn(sn, dc[r], c * dn[r]);
        }
      }
    }
  }
}

// Token-walking variant for tensors without RoPE (values; keys with theta =
// 0), n = 64 or 128: wave -> ((slab, head) plane, run of kTwTiles token
// tiles).  The wave first copies the run's packed bytes (codes, cosets,
// scales: each a contiguous stretch of its plane) into its LDS slice with
// 16-byte loads, then walks the tiles reading only LDS, so its stores are
// never held up by a load and each wave writes one contiguous stretch of the
// output.  (The plane-walking kernel keeps each lane's RoPE rows in
// registers, which needs a fixed token tile per wave.)
constexpr int kTwTiles = 32;

__device__ __forceinline__ int align16(int x) { return (x + 15) & ~15; }

// bytes of one wave's LDS slice
__host__ __device__ __forceinline__ int tw_slice_bytes(int run, int code_bytes,
                                                       int coset_bytes, int n_scales) {
  return ((run * code_bytes + 15) & ~15) + ((run * coset_bytes + 15) & ~15) +
         ((run * n_scales * 2 + 15) & ~15);
}

template <int N, int BITS, typename OutT, bool CMP>
__global__ __launch_bounds__(kBlock) void dequantize_tw_kernel(TensorArgs a) {
  constexpr int VL = N / 8;
  constexpr int TPW = 64 / VL;
  constexpr int L = 1 << BITS;
  constexpr int CB = N * BITS / 8;          // code bytes per vector (16 .. 48)
  constexpr int RUN = kTwTiles * TPW;       // tokens per run
  static_assert(CB % 16 == 0, "16-byte staging of the code rows");
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int row = lane / VL;
  const int l = lane % VL;
  const int m = lane_group(l);
  const int csb = a.coset_bytes, ns = a.n_scales;
  uint8_t* lc = smem + (threadIdx.x >> 6) * tw_slice_bytes(RUN, CB, csb, ns);
  uint8_t* lq = lc + RUN * CB;
  uint16_t* lg = reinterpret_cast<uint16_t*>(lq + align16(RUN * csb));
  const int64_t n_tt = (a.T + TPW - 1) / TPW;
  const int64_t n_run = (n_tt + kTwTiles - 1) / kTwTiles;
  const int64_t SH = a.n_vec / a.T;
  const int64_t wave = xcd_wave_id();
  const int64_t sh = wave / n_run;
  if (sh >= SH) return;                     // whole wave; no block barrier below
  const int64_t tt0 = (wave % n_run) * kTwTiles;
  const int64_t tok0 = tt0 * TPW;
  const int nt = (int)min64((int64_t)RUN, a.T - tok0);   // tokens of this run
  const int64_t v0 = sh * a.pT + tok0;                 // first packed vector
  {
    // codes: nt * CB bytes, 16-byte aligned at both ends
    const uint4* gc = reinterpret_cast<const uint4*>(a.codes + v0 * CB);
    uint4* dc = reinterpret_cast<uint4*>(lc);
    for (int i = lane; i < nt * (CB / 16); i += 64) dc[i] = gc[i];
    if (!CMP) {
      const uint8_t* gq = a.cosets + v0 * csb;
      for (int i = lane; i < nt * csb; i += 64) lq[i] = gq[i];
    }
    const uint16_t* gg = a.scales + v0 * ns;
    for (int i = lane; i < nt * ns; i += 64) lg[i] = gg[i];
  }
  // the slice is written and read by this wave only; LDS operations of a
  // wave complete in order, and the wait makes the writes visible
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const int j0 = 8 * m;
  const bool data_lane = j0 < a.d;
  const int gl = a.G >> 3;
  const bool neg_sigma = (__builtin_popcount(m) & 1) != 0;
  float coef[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) coef[k] = ((m >> k) & 1) ? -1.f : 1.f;
  const uint32_t flip = neg_sigma ? OutIo<OutT>::kFlip : 0u;
  const int n_tiles = (nt + TPW - 1) / TPW;
  for (int it = 0; it < n_tiles; ++it) {
    const int lt = min(it * TPW + row, nt - 1);   // token within the run
    uint32_t code;
    if (BITS == 2) {
      code = *reinterpret_cast<const uint16_t*>(lc + lt * CB + m * BITS);
    } else {
      const uint8_t* cp = lc + lt * CB + m * BITS;
      code = (uint32_t)cp[0] | ((uint32_t)cp[1] << 8) | ((uint32_t)cp[2] << 16);
    }
    int c = CMP ? 0 : (int)((lq[lt * csb + (m >> 3)] >> (m & 7)) & 1u);
    if (CMP) code = Compact<BITS>::unfold(code, c);
    const float sc = h2f(lg[lt * ns + m / gl]) * a.inv_sqrt_n;
    const float off = (0.5f * (float)c - a.half_L) * sc;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t idx = (code >> (BITS * k)) & (uint32_t)(L - 1);
      v[k] = __fmaf_rn((float)idx, sc, off);
    }
    fwht_lane(v);
    if (VL > 1) stage_fmac<0>(v, coef[0]);
    if (VL > 2) stage_fmac<1>(v, coef[1]);
    if (VL > 4) stage_fmac<2>(v, coef[2]);
    if (VL > 8) stage_fmac<3>(v, coef[3]);
    if (it * TPW + row < nt && data_lane)
      OutIo<OutT>::store8(a.y, (sh * a.T + tok0 + it * TPW + row) * a.d + j0, v, flip);
  }
}

template <int N, int BITS, typename OutT>
__global__ __launch_bounds__(kBlock) void dequantize_kernel(TensorArgs a) {
  constexpr int VL = N / 8;
  constexpr int VPB = kBlock / VL;
  constexpr int L = 1 << BITS;
  const int m = threadIdx.x % VL;
  const int64_t vec = (int64_t)blockIdx.x * VPB + threadIdx.x / VL;
  const bool live = vec < a.n_vec;
  const int64_t vv = live ? vec : 0;
  const int64_t t = vv % a.T;
  const int64_t pvec = (vv - t) / a.T * a.pT + t;   // index in the packed planes
  const uint8_t* cp = a.codes + pvec * a.code_bytes + m * BITS;
  uint32_t code;
  if (BITS == 2) {
    code = *reinterpret_cast<const uint16_t*>(cp);
  } else {
    code = (uint32_t)cp[0] | ((uint32_t)cp[1] << 8) | ((uint32_t)cp[2] << 16);
  }
  int c = a.compact ? 0 : (a.cosets[pvec * a.coset_bytes + (m >> 3)] >> (m & 7)) & 1;
  if (a.compact) code = Compact<BITS>::unfold(code, c);
  const int gl = a.G >> 3;
  const float s = h2f(a.scales[pvec * a.n_scales + m / gl]) * a.inv_sqrt_n;
  const float off = 0.5f * (float)c - a.half_L;
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int idx = (int)((code >> (BITS * k)) & (L - 1));
    v[k] = ((float)idx + off) * s;
  }
  fwht_lane(v);
  fwht_cross<VL>(v, m);
  if (a.rope != nullptr) rope_lane<false>(v, m, a.d, a.rope + t * (a.d >> 1));
  const int j0 = 8 * m;
  if (live && j0 < a.d) OutIo<OutT>::store8(a.y, vec * a.d + j0, v, 0u);
}

// One key per thread; the rotated queries of the GQA group (q~ = H pad(q))
// sit in LDS and are read as broadcasts.  score = s16 . sum_j q~_j p_j / sqrt(n).
constexpr int kScoreKeys = 1024;
constexpr int kMaxGroup = 8;

template <int N, int BITS, typename QT>
__global__ __launch_bounds__(kBlock) void score_kernel(ScoreArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int CB = N * BITS / 8;
  extern __shared__ float qt[];
  const int64_t s = blockIdx.z;
  const int h = blockIdx.y;
  const int grp = a.Hq / a.H;
  for (int i = threadIdx.x; i < grp * N; i += blockDim.x) {
    const int g = i / N, j = i % N;
    const int64_t qh = s * a.Hq + (int64_t)h * grp + g;
    qt[i] = (j < a.d) ? Io<QT>::load1(a.q, qh * a.d + j) : 0.f;
  }
  __syncthreads();
  for (int hs = 1; hs < N; hs <<= 1) {
    for (int i = threadIdx.x; i < grp * (N / 2); i += blockDim.x) {
      const int g = i / (N / 2), r = i % (N / 2);
      const int j = (r / hs) * 2 * hs + (r % hs);
      const float x0 = qt[g * N + j], x1 = qt[g * N + j + hs];
      qt[g * N + j] = x0 + x1;
      qt[g * N + j + hs] = x0 - x1;
    }
    __syncthreads();
  }
  const int64_t t_end = min64(a.T, (int64_t)(blockIdx.x + 1) * kScoreKeys);
  const int gl = a.G >> 3;
  for (int64_t t = (int64_t)blockIdx.x * kScoreKeys + threadIdx.x; t < t_end;
       t += blockDim.x) {
    const int64_t vec = (s * a.H + h) * a.pT + t;   // packed planes: token stride pT
    uint8_t cb[CB];
    const uint8_t* cp = a.codes + vec * a.code_bytes;
#pragma unroll
    for (int i = 0; i < CB; ++i) cb[i] = cp[i];
    const uint8_t* csp = a.cosets + vec * a.coset_bytes;
    for (int g0 = 0; g0 < grp; g0 += kMaxGroup) {
      const int gn = min(kMaxGroup, grp - g0);
      float acc[kMaxGroup];
#pragma unroll
      for (int g = 0; g < kMaxGroup; ++g) acc[g] = 0.f;
      for (int sg = 0; sg < N / (gl * 8); ++sg) {
        float part[kMaxGroup];
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) part[g] = 0.f;
        for (int mm = sg * gl; mm < (sg + 1) * gl; ++mm) {
          // group mm's 8b code bits start at byte mm * b
          uint32_t w = (uint32_t)cb[mm * BITS] | ((uint32_t)cb[mm * BITS + 1] << 8);
          if (BITS == 3) w |= (uint32_t)cb[mm * BITS + 2] << 16;
          int c = a.compact ? 0 : (csp[mm >> 3] >> (mm & 7)) & 1;
          if (a.compact) w = Compact<BITS>::unfold(w, c);
          const float off = 0.5f * (float)c - a.half_L;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int j = 8 * mm + k;
            const int idx = (int)((w >> (BITS * k)) & (L - 1));
            const float p = (float)idx + off;
            for (int g = 0; g < gn; ++g) part[g] = fmaf(qt[(g0 + g) * N + j], p, part[g]);
          }
        }
        const float sc = h2f(a.scales[vec * a.n_scales + sg]);
        for (int g = 0; g < gn; ++g) acc[g] = fmaf(part[g], sc, acc[g]);
      }
      for (int g = 0; g < gn; ++g) {
        const int64_t qh = s * a.Hq + (int64_t)h * grp + g0 + g;
        a.out[qh * a.T + t] = acc[g] * a.inv_sqrt_n;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Table-based asymmetric scoring (Nedelkoski et al., Abstract and Table 3:
// q.k from packed keys without dequantizing them).
//
// With q~ = H pad(q) (unnormalised) and p = idx - L/2 + c/2,
//   q . D0(k) = (1/sqrt n) sum_g s_g sum_{j in g} q~_j p_j .
// The code index is linear in the packed bits (idx_j = sum_b bit * 2^b), so
// every code byte contributes sum_{bits i} (bit_i - 1/2) w_i with
// w_i = q~_{j(i)} 2^{b(i)}: one 256-entry table per code byte covers 2- and
// 3-bit codes alike.  Each coset byte adds sum_i Q_{m(i)} (bit_i - 1) / 2 with
// Q_m the sum of q~ over 8-group m; the centring constant sum_j q~_j (L-1)/2 -
// sum_m Q_m L/2 + sum_m Q_m / 2 cancels exactly.  Tables hold HPP query heads
// side by side so one LDS vector read serves all of them.
// Compact packing: the code bit that holds c takes the coset weight
// (c ? 0 : -Q_m / 2), and the tables of the coset bytes are keyed instead by
// the per-key mask of the groups' idx_7 low bits (the parity of idx_0..idx_6,
// computed with popcounts): entry sum_i (bit_i - 1/2) q~_{8 m(i) + 7}.  The
// constant still cancels.
// ---------------------------------------------------------------------------
constexpr int kLutBlock = 512;

// Table entries: HPP floats side by side.  2 and 4 heads use native vector
// types and vector accumulation, so that each lookup stays one 8- or 16-byte
// LDS read (per-component use lets the compiler split it into scalar reads).
template <int HPP>
struct LutVec;
template <> struct LutVec<1> { using T = float; };
template <> struct LutVec<2> { using T = nq_f2; };
template <> struct LutVec<3> { using T = float3; };
template <> struct LutVec<4> { using T = nq_f4; };

template <typename V>
struct LutAcc {   // vector accumulator for native vectors
  V v;
  __device__ __forceinline__ void zero() { v = V(0.f); }
  __device__ __forceinline__ void add(V x) { v = v + x; }
  __device__ __forceinline__ float get(int i) const { return v[i]; }
};
template <>
struct LutAcc<float3> {
  float v[3];
  __device__ __forceinline__ void zero() { v[0] = v[1] = v[2] = 0.f; }
  __device__ __forceinline__ void add(float3 x) { v[0] += x.x; v[1] += x.y; v[2] += x.z; }
  __device__ __forceinline__ float get(int i) const { return v[i]; }
};
template <>
struct LutAcc<float> {
  float v;
  __device__ __forceinline__ void zero() { v = 0.f; }
  __device__ __forceinline__ void add(float x) { v += x; }
  __device__ __forceinline__ float get(int) const { return v; }
};


// NS = scale groups per key (n / G: 1, 2 or 4); a compile-time count keeps
// the per-key lookups free of branches, so their LDS reads overlap.
template <int BITS, int N, int HPP, typename QT, bool CMP, int NS>
__global__ __launch_bounds__(kLutBlock) void score_lut_kernel(ScoreArgs a,
                                                              int n_pass,
                                                              int64_t chunk) {
  constexpr int CB = N * BITS / 8;        // code bytes per key
  constexpr int NG = N / 8;               // 8-groups per key
  constexpr int CSB = (NG + 7) / 8;       // coset bytes per key
  constexpr int NT = CB + CSB;            // tables
  using V = typename LutVec<HPP>::T;
  extern __shared__ __align__(16) float lds[];   // 16-byte table entries
  float* lut = lds;                       // [NT][256][HPP]
  float* qt = lds + NT * 256 * HPP;       // [HPP][N] rotated queries
  float* qm = qt + HPP * N;               // [HPP][NG] group sums
  const int64_t s = blockIdx.z;
  const int h = blockIdx.y / n_pass;
  const int pass = blockIdx.y % n_pass;
  const int grp = a.Hq / a.H;
  const int hq0 = h * grp + pass * HPP;
  const int nh = min(HPP, h * grp + grp - hq0);  // heads in this pass

  // rotated queries q~ = H pad(q) (in LDS), then group sums
  for (int i = threadIdx.x; i < HPP * N; i += blockDim.x) {
    const int hh = i / N, j = i % N;
    qt[i] = (hh < nh && j < a.d)
                ? Io<QT>::load1(a.q, (s * a.Hq + hq0 + hh) * (int64_t)a.d + j)
                : 0.f;
  }
  __syncthreads();
  for (int hs = 1; hs < N; hs <<= 1) {
    for (int i = threadIdx.x; i < HPP * (N / 2); i += blockDim.x) {
      const int hh = i / (N / 2), r = i % (N / 2);
      const int j = (r / hs) * 2 * hs + (r % hs);
      const float x0 = qt[hh * N + j], x1 = qt[hh * N + j + hs];
      qt[hh * N + j] = x0 + x1;
      qt[hh * N + j + hs] = x0 - x1;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < HPP * NG; i += blockDim.x) {
    const int hh = i / NG, mm = i % NG;
    float sum = 0.f;
    for (int k = 0; k < 8; ++k) sum += qt[hh * N + 8 * mm + k];
    qm[i] = sum;
  }
  __syncthreads();
  // Tables.  Bit i of a table's byte adds A_i when set and B_i when clear:
  //   code bit            A = +w/2, B = -w/2 (w = q~_j 2^b for its coordinate)
  //   coset bit           A = 0,    B = -Q_m/2 (also the folded c of compact)
  //   compact parity bit  A = +q~_{8m+7}/2, B = -q~_{8m+7}/2
  // Each work item (table, head, high nibble h) forms the 16 low-nibble sums
  // from two 4-entry pair tables and writes entries 16 h .. 16 h + 15.
  for (int item = threadIdx.x; item < NT * HPP * 16; item += blockDim.x) {
    const int h = item & 15;
    const int hh = (item >> 4) % HPP;
    const int tb = (item >> 4) / HPP;
    float A[8], B[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (tb < CB) {
        const int bit = 8 * tb + i;           // position in the key's bit stream
        if (CMP && bit % (8 * BITS) == 7 * BITS) {   // the folded coset bit
          A[i] = 0.f;
          B[i] = -0.5f * qm[hh * NG + bit / (8 * BITS)];
        } else {
          const float w = qt[hh * N + bit / BITS] * (float)(1 << (bit % BITS));
          A[i] = 0.5f * w;
          B[i] = -0.5f * w;
        }
      } else {
        const int mm = 8 * (tb - CB) + i;
        if (mm >= NG) {
          A[i] = 0.f;
          B[i] = 0.f;
        } else if (CMP) {
          A[i] = 0.5f * qt[hh * N + 8 * mm + 7];
          B[i] = -A[i];
        } else {
          A[i] = 0.f;
          B[i] = -0.5f * qm[hh * NG + mm];
        }
      }
    }
    float hi = 0.f;
#pragma unroll
    for (int i = 4; i < 8; ++i) hi += ((h >> (i - 4)) & 1) ? A[i] : B[i];
    float p01[4], p23[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      p01[u] = ((u & 1) ? A[0] : B[0]) + ((u & 2) ? A[1] : B[1]);
      p23[u] = ((u & 1) ? A[2] : B[2]) + ((u & 2) ? A[3] : B[3]);
    }
    float* row = lut + ((size_t)tb * 256 + h * 16) * HPP + hh;
#pragma unroll
    for (int u = 0; u < 16; ++u) row[u * HPP] = (p01[u & 3] + p23[u >> 2]) + hi;
  }
  __syncthreads();

  const V* lutv = reinterpret_cast<const V*>(__builtin_assume_aligned(lut, 16));
  constexpr int CBG = CB / NS;             // code bytes per scale group
  constexpr int KG = CSB / NS;             // coset (parity) bytes per scale group
  static_assert(CB % NS == 0 && CSB % NS == 0, "scale groups must cover whole bytes");
  const int64_t t0 = (int64_t)blockIdx.x * chunk;
  const int64_t t1 = min64(a.T, t0 + chunk);
  const int64_t base = (s * a.H + h) * a.pT;   // packed planes: token stride pT
  for (int64_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
    const int64_t vec = base + t;
    uint32_t cw[CB / 4 + 1];
    const uint8_t* cp = a.codes + vec * CB;
    if (CB % 16 == 0) {
#pragma unroll
      for (int i = 0; i < CB / 16; ++i) {
        const uint4 w = reinterpret_cast<const uint4*>(cp)[i];
        cw[4 * i] = w.x; cw[4 * i + 1] = w.y; cw[4 * i + 2] = w.z; cw[4 * i + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < CB / 4; ++i) cw[i] = reinterpret_cast<const uint32_t*>(cp)[i];
    }
    uint32_t cs = 0;   // coset bits, or (compact) the groups' idx_7 low bits
    if (CMP) {
      cw[CB / 4] = 0u;
#pragma unroll
      for (int mm = 0; mm < NG; ++mm) {
        const int o = mm * 8 * BITS;
        const uint64_t x = (uint64_t)cw[o >> 5] | ((uint64_t)cw[(o >> 5) + 1] << 32);
        cs |= Compact<BITS>::low7((uint32_t)(x >> (o & 31))) << mm;
      }
    } else {
      const uint8_t* csp = a.cosets + vec * CSB;
#pragma unroll
      for (int i = 0; i < CSB; ++i) cs |= (uint32_t)csp[i] << (8 * i);
    }
    float score[HPP];
#pragma unroll
    for (int hh = 0; hh < HPP; ++hh) score[hh] = 0.f;
#pragma unroll
    for (int g = 0; g < NS; ++g) {
      LutAcc<V> acc;
      acc.zero();
#pragma unroll
      for (int b = g * CBG; b < (g + 1) * CBG; ++b) {
        const uint32_t v = (cw[b >> 2] >> (8 * (b & 3))) & 0xffu;
        acc.add(lutv[b * 256 + v]);
      }
#pragma unroll
      for (int k = g * KG; k < (g + 1) * KG; ++k) {
        const uint32_t v = (cs >> (8 * k)) & 0xffu;
        acc.add(lutv[(CB + k) * 256 + v]);
      }
      const float sc = h2f(a.scales[vec * a.n_scales + g]);
#pragma unroll
      for (int hh = 0; hh < HPP; ++hh) score[hh] = fmaf(acc.get(hh), sc, score[hh]);
    }
#pragma unroll
    for (int hh = 0; hh < HPP; ++hh)
      if (hh < nh) a.out[(s * a.Hq + hq0 + hh) * a.T + t] = score[hh] * a.inv_sqrt_n;
  }
}

// ---------------------------------------------------------------------------
// Value half of decode attention on the packed cache:
//   out[s][h] = sum_t w[s][h][t] * D(V)[s][h / (Hq/H)][t].
// D is linear, so the sum is taken in the codec frame,
//   z = sum_t w_t s_t (idx_t - L/2 + c_t/2),   out = (H z / sqrt n)[:d],
// with one Walsh-Hadamard transform per query head instead of one per key.
// One workgroup per (slab, KV head, head pass); each VL-lane row takes one
// key per step, lane m accumulates its 8-group; rows and waves are reduced
// through LDS in a fixed order (deterministic).
// ---------------------------------------------------------------------------
// Threads per workgroup: 1024, or 512 where the accumulators (HPP heads x 8
// coordinates), the in-flight weights and 3-bit code words need more than
// the 128 registers a lane has at 1024 threads (8 heads per pass; 4 heads of
// 3-bit codes); no instance spills.
template <int BITS, int HPP>
constexpr int att_block() { return (HPP >= 8 || (HPP >= 4 && BITS == 3)) ? 512 : 1024; }

template <int BITS, int N, int HPP, bool CMP>
__global__ __launch_bounds__((att_block<BITS, HPP>())) void attend_kernel(AttendArgs a, int n_pass) {
  constexpr int VL = N / 8;
  constexpr int KPW = 64 / VL;             // keys per wave per step
  constexpr int L = 1 << BITS;
  extern __shared__ float lds[];           // [n_waves][HPP][N]
  const int64_t s = blockIdx.z;
  const int h = blockIdx.y / n_pass;
  const int pass = blockIdx.y % n_pass;
  const int grp = a.Hq / a.H;
  const int hq0 = h * grp + pass * HPP;
  const int nh = min(HPP, h * grp + grp - hq0);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int row = lane / VL;
  const int m = lane % VL;
  const int gl = a.G >> 3;
  float acc[HPP][8];
  float offacc[HPP];
#pragma unroll
  for (int g = 0; g < HPP; ++g) {
    offacc[g] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[g][k] = 0.f;
  }
  const int64_t base = (s * a.H + h) * a.pT;   // packed planes: token stride pT
  const float* wrow = a.w + (s * a.Hq + hq0) * a.T;
  const int64_t stride = (int64_t)nw * KPW;
  // U keys per row per step, all loads issued before any use so that U
  // HBM round trips overlap
  constexpr int U = 8;
  for (int64_t t0 = (int64_t)wv * KPW + row; t0 < a.T; t0 += U * stride) {
    uint32_t code[U], cbyte[U];
    uint16_t sbits[U];
    float wt[U][HPP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tu = t0 + u * stride;
      const bool ok = tu < a.T;
      const int64_t vec = base + (ok ? tu : t0);
      const uint8_t* cp = a.codes + vec * a.code_bytes + m * BITS;
      if (BITS == 2) {
        code[u] = *reinterpret_cast<const uint16_t*>(cp);
      } else {
        code[u] = (uint32_t)cp[0] | ((uint32_t)cp[1] << 8) | ((uint32_t)cp[2] << 16);
      }
      cbyte[u] = CMP ? 0u : a.cosets[vec * a.coset_bytes + (m >> 3)];
      sbits[u] = a.scales[vec * a.n_scales + m / gl];
#pragma unroll
      for (int g = 0; g < HPP; ++g)
        wt[u][g] = (ok && g < nh) ? wrow[(int64_t)g * a.T + tu] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int c = (int)((cbyte[u] >> (m & 7)) & 1u);
      const uint32_t cw = CMP ? Compact<BITS>::unfold(code[u], c) : code[u];
      const float sc = h2f(sbits[u]);
      const float off = 0.5f * (float)c - a.half_L;
      float p[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        p[k] = (float)((cw >> (BITS * k)) & (uint32_t)(L - 1));
#pragma unroll
      for (int g = 0; g < HPP; ++g) {
        const float ws = wt[u][g] * sc;
        offacc[g] = fmaf(ws, off, offacc[g]);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[g][k] = fmaf(ws, p[k], acc[g][k]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < HPP; ++g) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[g][k] += offacc[g];
  }
  // rows of a wave hold the same 8-group: add lanes l, l + VL, l + 2 VL, ...
#pragma unroll
  for (int sft = VL; sft < 64; sft <<= 1) {
#pragma unroll
    for (int g = 0; g < HPP; ++g) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[g][k] += __shfl_xor(acc[g][k], sft);
    }
  }
  if (lane < VL) {
#pragma unroll
    for (int g = 0; g < HPP; ++g) {
#pragma unroll
      for (int k = 0; k < 8; ++k) lds[(wv * HPP + g) * N + 8 * m + k] = acc[g][k];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HPP * N; i += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < nw; ++w) sum += lds[w * HPP * N + i];
    lds[i] = sum;
  }
  __syncthreads();
  for (int hs = 1; hs < N; hs <<= 1) {
    for (int i = threadIdx.x; i < HPP * (N / 2); i += blockDim.x) {
      const int g = i / (N / 2), r = i % (N / 2);
      const int j = (r / hs) * 2 * hs + (r % hs);
      const float x0 = lds[g * N + j], x1 = lds[g * N + j + hs];
      lds[g * N + j] = x0 + x1;
      lds[g * N + j + hs] = x0 - x1;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < nh * a.d; i += blockDim.x) {
    const int g = i / a.d, j = i % a.d;
    a.out[(s * a.Hq + hq0 + g) * (int64_t)a.d + j] = lds[g * N + j] * a.inv_sqrt_n;
  }
}

// The same value sum on the matrix cores, for 2-bit values with one scale per
// vector at n = 128 (one 16 x 16 x 32 bf16 product per 32 tokens and 16
// coordinates).  z_h[j] = sum_t (w_h,t s_t) (idx_t,j - 2 + c_t/2) is a dense
// contraction over tokens: the A operand holds the weights (rows: query heads),
// the B operand the code values (columns: the 8-groups), K runs over tokens.
//  * B: 64 (idx - 2 + c/2) is a signed byte: (idx ^ 2) in its two top bits and
//    the coset bit below them; it converts exactly to fp32 and to bf16, so the
//    centred values (no cancellation against the sum of the weights) carry no
//    rounding.  The factor 64 is removed at the end.
//  * A: w s in fp32, split into its top 16 bits (hi, rows 0..7) and the bf16
//    truncation of the remainder (lo, rows 8..15); hi + lo differs from w s
//    by less than 2^-14 |w s|.  D = hi-rows + lo-rows.
// Lane l supplies A row l % 16 and B column l % 16 for the 8 tokens
// 8 (l / 16) .. + 7 of the chunk, and holds D rows 4 (l / 16) .. + 3 of
// column l % 16.  Column g of block (q, half) is coordinate 8 g + 4 half + q.
// This form serves passes of 5..8 query heads; up to 4 heads use the table
// form further down, which needs fewer instructions per token.
// ---------------------------------------------------------------------------
typedef __bf16 nq_bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float i8_to_f(uint32_t x, int byte) {
  return (float)(int)(int8_t)(x >> (8 * byte));
}

// One lane's share of a 32-token chunk: the group words of its 8-group for
// tokens tb .. tb + 7 (two per word), their coset words (two per word), their
// scales (two per word) and its query head's weights.
struct AttChunk {
  uint32_t cw[4], cs[4], sw[4];
  float wt[8];
};

// FULL: tokens tb .. tb + 7 all exist and the scale / coset planes and the
// weight rows are 16-byte aligned there.  Otherwise indices are clamped to
// the last token and the weights of missing tokens are 0.
template <bool FULL, bool CMP>
__device__ __forceinline__ void att_load(AttChunk& k, const uint8_t* __restrict__ cp,
                                         const uint16_t* __restrict__ csp,
                                         const uint16_t* __restrict__ scp,
                                         const float* __restrict__ wr, int tb, int T,
                                         bool arow) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t0 = FULL ? tb + 2 * j : min(tb + 2 * j, T - 1);
    const uint32_t t1 = FULL ? tb + 2 * j + 1 : min(tb + 2 * j + 1, T - 1);
    k.cw[j] = (uint32_t)*reinterpret_cast<const uint16_t*>(cp + t0 * 32u) |
              ((uint32_t)*reinterpret_cast<const uint16_t*>(cp + t1 * 32u) << 16);
    if (!FULL) {
      k.sw[j] = (uint32_t)scp[t0] | ((uint32_t)scp[t1] << 16);
      if (!CMP) k.cs[j] = (uint32_t)csp[t0] | ((uint32_t)csp[t1] << 16);
    }
  }
  if (FULL) {
    const uint4 sv = *reinterpret_cast<const uint4*>(scp + (uint32_t)tb);
    k.sw[0] = sv.x; k.sw[1] = sv.y; k.sw[2] = sv.z; k.sw[3] = sv.w;
    if (!CMP) {
      const uint4 cv = *reinterpret_cast<const uint4*>(csp + (uint32_t)tb);
      k.cs[0] = cv.x; k.cs[1] = cv.y; k.cs[2] = cv.z; k.cs[3] = cv.w;
    }
  }
  if (arow) {
    if (FULL) {
      const float4 w0 = *reinterpret_cast<const float4*>(wr + (uint32_t)tb);
      const float4 w1 = *reinterpret_cast<const float4*>(wr + (uint32_t)tb + 4);
      k.wt[0] = w0.x; k.wt[1] = w0.y; k.wt[2] = w0.z; k.wt[3] = w0.w;
      k.wt[4] = w1.x; k.wt[5] = w1.y; k.wt[6] = w1.z; k.wt[7] = w1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) k.wt[i] = tb + i < T ? wr[(uint32_t)(tb + i)] : 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) k.wt[i] = 0.f;
  }
}

template <bool CMP>
__device__ __forceinline__ void att_mma(nq_f4 (&acc)[4][2], const AttChunk& k, int col,
                                        uint32_t pmask) {
  nq_u4 av;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float x[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float ws = k.wt[2 * j + e] * h2f((uint16_t)(k.sw[j] >> (16 * e)));
      x[e] = ws - __uint_as_float(__float_as_uint(ws) & pmask);
    }
    av[j] = __builtin_amdgcn_perm(__float_as_uint(x[1]), __float_as_uint(x[0]), 0x07060302u);
  }
  const nq_bf16x8 A = __builtin_bit_cast(nq_bf16x8, av);
  uint32_t xa[4], C[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t x = k.cw[j];
    uint32_t cb;
    if (CMP) {
      cb = (x >> 14) & 0x00010001u;
      const uint32_t p0 = (uint32_t)__builtin_popcount(x & 0x00001555u) & 1u;
      const uint32_t p1 = (uint32_t)__builtin_popcount(x & 0x15550000u) & 1u;
      x = (x & ~0x40004000u) | (p0 << 14) | (p1 << 30);
    } else {
      cb = (k.cs[j] >> col) & 0x00010001u;
    }
    C[j] = __umul24(cb, 0x2020u);
    xa[j] = x ^ 0xaaaaaaaau;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    nq_bf16x8 B0, B1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t t = ((xa[j] << (6 - 2 * q)) & 0xc0c0c0c0u) | C[j];
      B0[2 * j] = (__bf16)i8_to_f(t, 0);
      B0[2 * j + 1] = (__bf16)i8_to_f(t, 2);
      B1[2 * j] = (__bf16)i8_to_f(t, 1);
      B1[2 * j + 1] = (__bf16)i8_to_f(t, 3);
    }
    acc[q][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B0, acc[q][0], 0, 0, 0);
    acc[q][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B1, acc[q][1], 0, 0, 0);
  }
}

template <int HPP, bool CMP>
__global__ __launch_bounds__(1024) void attend_mfma_kernel(AttendArgs a, int n_pass) {
  constexpr int N = 128;
  constexpr int U = 2;                     // chunks of 32 tokens per wave per step
  extern __shared__ float lds[];           // [n_waves][HPP][N]
  const int64_t s = blockIdx.z;
  const int h = blockIdx.y / n_pass;
  const int pass = blockIdx.y % n_pass;
  const int grp = a.Hq / a.H;
  const int hq0 = h * grp + pass * HPP;
  const int nh = min(HPP, h * grp + grp - hq0);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int col = lane & 15;               // B column = 8-group; A row
  const int kg = lane >> 4;                // tokens 8 kg .. 8 kg + 7 of a chunk
  const int hh = col & 7;                  // the A row's query head
  const bool arow = hh < nh;
  const uint32_t pmask = col >= 8 ? 0xffff0000u : 0u;
  const int T = (int)a.T;
  const int64_t base = (s * a.H + h) * a.pT;
  const float* wr = a.w + (s * a.Hq + hq0 + (arow ? hh : 0)) * a.T;
  const uint8_t* cp = a.codes + base * (N / 4) + 2 * col;
  const uint16_t* csp = reinterpret_cast<const uint16_t*>(a.cosets) + base;
  const uint16_t* scp = a.scales + base;
  const bool vec = (T & 3) == 0 &&
                   (((uintptr_t)scp | (CMP ? (uintptr_t)0 : (uintptr_t)csp)) & 15) == 0;
  nq_f4 acc[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q][0] = acc[q][1] = nq_f4{0.f, 0.f, 0.f, 0.f};
  const int step = nw * 32;
  for (int c0 = wv * 32; c0 < T; c0 += U * step) {
    AttChunk k[U];
    if (vec && c0 + (U - 1) * step + 32 <= T) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        att_load<true, CMP>(k[u], cp, csp, scp, wr, c0 + u * step + 8 * kg, T, arow);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
        att_load<false, CMP>(k[u], cp, csp, scp, wr, c0 + u * step + 8 * kg, T, arow);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) att_mma<CMP>(acc, k[u], col, pmask);
  }
  // rows 8..15 (lanes 32..63) hold the low parts of rows 0..7 (lanes 0..31)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[q][hf][r] + __shfl_xor(acc[q][hf][r], 32);
        const int head = 4 * kg + r;
        if (kg < 2 && head < HPP) lds[(wv * HPP + head) * N + 8 * col + 4 * hf + q] = v;
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HPP * N; i += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < nw; ++w) sum += lds[w * HPP * N + i];
    lds[i] = sum;
  }
  __syncthreads();
  for (int hs = 1; hs < N; hs <<= 1) {
    for (int i = threadIdx.x; i < HPP * (N / 2); i += blockDim.x) {
      const int g = i / (N / 2), r = i % (N / 2);
      const int j = (r / hs) * 2 * hs + (r % hs);
      const float x0 = lds[g * N + j], x1 = lds[g * N + j + hs];
      lds[g * N + j] = x0 + x1;
      lds[g * N + j + hs] = x0 - x1;
    }
    __syncthreads();
  }
  const float osc = a.inv_sqrt_n * (1.f / 64.f);
  for (int i = threadIdx.x; i < nh * a.d; i += blockDim.x) {
    const int g = i / a.d, j = i % a.d;
    a.out[(s * a.Hq + hq0 + g) * (int64_t)a.d + j] = lds[g * N + j] * osc;
  }
}


// The 2-bit code values of one byte as bf16 (entry c * 256 + byte holds
// idx - 2 + c/2 for the byte's 4 coordinates, exact in bf16, low coordinate
// first), in kTblCopies copies: entry e of copy r at uint2 index
// e * kTblCopies + r, and lane l reads copy l % kTblCopies.  On gfx950's 64
// four-byte LDS banks an 8-byte entry of copy r then sits in bank pair r or
// r + 16 only, so of the 32 lanes one ds_read_b64 pass serves, at most two
// can contend for a bank pair (about 2.3x fewer conflict stalls than random
// lookups in one copy, measured).
constexpr int kTblCopies = 16;    // copies for the scorer and the attention kernels
// Entry e of the value table: the bf16 of idx - 2 + c/2 for the 4
// coordinates of code byte e & 255 with coset bit e >> 8.
__device__ __forceinline__ uint2 value_entry(int e) {
  const int c = e >> 8, byte = e & 255;
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float lo = (float)((byte >> (4 * h)) & 3) - 2.f + 0.5f * (float)c;
    const float hi = (float)((byte >> (4 * h + 2)) & 3) - 2.f + 0.5f * (float)c;
    w[h] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  return make_uint2(w[0], w[1]);
}
// The table in TC copies, entry e of copy r at index e * TC + r.  Copy 0 is
// computed (one entry per thread), then replicated by every thread
// (neighbouring lanes write neighbouring copies of one entry).  Ends with a
// barrier.
template <int TC>
__device__ __forceinline__ void value_table_copies(uint2* tbl) {
  for (int e = threadIdx.x; e < 512; e += blockDim.x) tbl[e * TC] = value_entry(e);
  __syncthreads();
  for (int i = threadIdx.x; i < 512 * TC; i += blockDim.x)
    if (i % TC != 0) tbl[i] = tbl[i - i % TC];
  __syncthreads();
}

// Variant for up to 4 query heads a pass: the 16 A rows are (head, hi / lo
// part, sub) and the two bf16 of a K-slot pair are two coordinates of one
// token (sub 0 and 1), so a lookup in a 4 KB LDS table -- entry (c, code byte)
// holds the bf16 of idx - 2 + c/2 for the byte's 4 coordinates -- yields B
// operand words directly.  Column g of block b holds coordinates 8 g + 2 b
// (sub 0) and 8 g + 2 b + 1 (sub 1); the A row of sub 0 carries the weight in
// the low bf16 of each pair and 0 in the high one, sub 1 the reverse.
template <bool CMP, int TC>
__device__ __forceinline__ void att_mma4(nq_f4 (&acc)[4], const AttChunk& k,
                                         const uint2* __restrict__ tbl, int col,
                                         uint32_t pmask, uint32_t asel) {
  static_assert(TC == 1 || TC == 16, "table copies");
  const char* tb = reinterpret_cast<const char*>(tbl);
  // this lane's table copy (entry e of copy r at byte 8 (TC e + r)), as a
  // byte offset in both 16-bit halves
  const uint32_t lane_copy = (uint32_t)((threadIdx.x & 63) % TC) * 8u * 0x00010001u;
#pragma unroll
  for (int hc = 0; hc < 2; ++hc) {
    nq_u4 av;
    uint32_t bw[4][4];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int w = 2 * hc + jp;           // tokens 2 w and 2 w + 1 of the lane
      uint32_t cw = k.cw[w];
      uint32_t cc;                          // their coset bits at bits 0 and 16
      if (CMP) {
        cc = (cw >> 14) & 0x00010001u;
        const uint32_t p0 = (uint32_t)__builtin_popcount(cw & 0x00001555u) & 1u;
        const uint32_t p1 = (uint32_t)__builtin_popcount(cw & 0x15550000u) & 1u;
        cw = (cw & ~0x40004000u) | (p0 << 14) | (p1 << 30);
      } else {
        cc = (k.cs[w] >> col) & 0x00010001u;
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int j = 2 * jp + e;
        const float ws = k.wt[2 * w + e] * h2f((uint16_t)(k.sw[w] >> (16 * e)));
        const float x = ws - __uint_as_float(__float_as_uint(ws) & pmask);
        av[j] = __builtin_amdgcn_perm(__float_as_uint(x), __float_as_uint(x), asel);
        // 16-bit halves: table indices (code byte 0 | c << 8), (code byte 1 | c << 8)
        const uint32_t ix = __builtin_amdgcn_perm(cc, cw, e ? 0x06030602u : 0x04010400u);
        const uint32_t ad = TC == 1 ? ((ix << 3) & 0xfff8fff8u)
                                    : (((ix << 7) & 0xff80ff80u) | lane_copy);
        const uint2 e0 = *reinterpret_cast<const uint2*>(tb + (ad & 0xffffu));
        const uint2 e1 = *reinterpret_cast<const uint2*>(tb + (ad >> 16));
        bw[0][j] = e0.x;
        bw[1][j] = e0.y;
        bw[2][j] = e1.x;
        bw[3][j] = e1.y;
      }
    }
    const nq_bf16x8 A = __builtin_bit_cast(nq_bf16x8, av);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const nq_u4 bv = {bw[b][0], bw[b][1], bw[b][2], bw[b][3]};
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(nq_bf16x8, bv),
                                                       acc[b], 0, 0, 0);
    }
  }
}

template <int HPP, bool CMP>
__global__ __launch_bounds__(1024) void attend_mfma4_kernel(AttendArgs a, int n_pass) {
  static_assert(HPP <= 4, "rows are (head, part, sub)");
  constexpr int N = 128;
  constexpr int U = 2;                     // chunks of 32 tokens per wave per step
  extern __shared__ float red[];           // [n_waves][HPP][N]
  __shared__ uint2 tbl[512 * kTblCopies];  // entry c * 256 + code byte, kTblCopies copies
  value_table_copies<kTblCopies>(tbl);
  const int64_t s = blockIdx.z;
  const int h = blockIdx.y / n_pass;
  const int pass = blockIdx.y % n_pass;
  const int grp = a.Hq / a.H;
  const int hq0 = h * grp + pass * HPP;
  const int nh = min(HPP, h * grp + grp - hq0);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int col = lane & 15;               // B column = 8-group; A row
  const int kg = lane >> 4;                // tokens 8 kg .. 8 kg + 7 of a chunk
  const int hh = col & 3;                  // the A row's query head, part, sub
  const bool arow = hh < nh;
  const uint32_t pmask = (col & 4) ? 0xffff0000u : 0u;
  const uint32_t asel = (col & 8) ? 0x03020c0cu : 0x0c0c0302u;
  const int T = (int)a.T;
  const int64_t base = (s * a.H + h) * a.pT;
  const float* wr = a.w + (s * a.Hq + hq0 + (arow ? hh : 0)) * a.T;
  const uint8_t* cp = a.codes + base * (N / 4) + 2 * col;
  const uint16_t* csp = reinterpret_cast<const uint16_t*>(a.cosets) + base;
  const uint16_t* scp = a.scales + base;
  const bool vec = (T & 3) == 0 &&
                   (((uintptr_t)scp | (CMP ? (uintptr_t)0 : (uintptr_t)csp)) & 15) == 0;
  nq_f4 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = nq_f4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  const int step = nw * 32;
  for (int c0 = wv * 32; c0 < T; c0 += U * step) {
    AttChunk k[U];
    if (vec && c0 + (U - 1) * step + 32 <= T) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        att_load<true, CMP>(k[u], cp, csp, scp, wr, c0 + u * step + 8 * kg, T, arow);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
        att_load<false, CMP>(k[u], cp, csp, scp, wr, c0 + u * step + 8 * kg, T, arow);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) att_mma4<CMP, kTblCopies>(acc, k[u], tbl, col, pmask, asel);
  }
  // rows 4..7 / 12..15 (lanes 16..31 / 48..63) hold the low parts of rows
  // 0..3 / 8..11 (lanes 0..15 / 32..47); lanes 0..15 have sub 0, 32..47 sub 1
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = acc[b][r] + __shfl_xor(acc[b][r], 16);
      if ((kg & 1) == 0 && r < HPP)
        red[(wv * HPP + r) * N + 8 * col + 2 * b + (kg >> 1)] = v;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HPP * N; i += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < nw; ++w) sum += red[w * HPP * N + i];
    red[i] = sum;
  }
  __syncthreads();
  for (int hs = 1; hs < N; hs <<= 1) {
    for (int i = threadIdx.x; i < HPP * (N / 2); i += blockDim.x) {
      const int g = i / (N / 2), r = i % (N / 2);
      const int j = (r / hs) * 2 * hs + (r % hs);
      const float x0 = red[g * N + j], x1 = red[g * N + j + hs];
      red[g * N + j] = x0 + x1;
      red[g * N + j + hs] = x0 - x1;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < nh * a.d; i += blockDim.x) {
    const int g = i / a.d, j = i % a.d;
    a.out[(s * a.Hq + hq0 + g) * (int64_t)a.d + j] = red[g * N + j] * a.inv_sqrt_n;
  }
}

// q~ = H pad(q) of the pass's query heads, in place in LDS (qt: HPP rows of
// 128 floats, filled and followed by a barrier).
template <int HPP>
__device__ __forceinline__ void rotate_queries(float* qt) {
  constexpr int N = 128;
  for (int hs = 1; hs < N; hs <<= 1) {
    for (int i = threadIdx.x; i < HPP * (N / 2); i += blockDim.x) {
      const int hh = i / (N / 2), r = i % (N / 2);
      const int j = (r / hs) * 2 * hs + (r % hs);
      const float x0 = qt[hh * N + j], x1 = qt[hh * N + j + hs];
      qt[hh * N + j] = x0 + x1;
      qt[hh * N + j + hs] = x0 - x1;
    }
    __syncthreads();
  }
}

// The A operands of the four 16x16x32 products: lane (row col = lane & 15,
// k-group kg = lane >> 4) holds coordinates 8 (4 kg + b) .. + 7 of row col,
// which is head col / 2's hi part (even rows) or lo part (odd rows).
template <int HPP>
__device__ __forceinline__ void score_a_operands(const float* qt, int nh, int lane,
                                                 nq_bf16x8 (&A)[4]) {
  constexpr int N = 128;
  const int col = lane & 15, kg = lane >> 4;
  const int hh = col >> 1;
  const bool part = (col & 1) != 0;
  const bool arow = hh < nh;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    nq_u4 av;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t pr = 0;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float v = arow ? qt[hh * N + 8 * (4 * kg + b) + 2 * e + k] : 0.f;
        const float hi = (float)(__bf16)v;
        const float x = part ? v - hi : v;
        const uint32_t bits = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
        pr |= bits << (16 * k);
      }
      av[e] = pr;
    }
    A[b] = __builtin_bit_cast(nq_bf16x8, av);
  }
}

// One 16-key block: the four products over the key's code words w (8-groups
// 4 kg .. 4 kg + 3 of key col), cosets cs (the key's coset word), and the
// scores of heads 2 kg and 2 kg + 1 scaled by f.  TC table copies; lane_copy
// is the lane's copy as a byte offset in both 16-bit halves.
template <bool CMP, int TC>
__device__ __forceinline__ void score_block(const nq_bf16x8 (&A)[4], uint2 cw, uint32_t cs,
                                            int kg, const char* tb, uint32_t lane_copy, float f,
                                            float& v0, float& v1) {
  constexpr int kShift = TC == 16 ? 7 : TC == 8 ? 6 : TC == 4 ? 5 : TC == 2 ? 4 : 3;
  static_assert((1 << (kShift - 3)) == TC, "TC a power of two up to 16");
  uint32_t w[2] = {cw.x, cw.y};
  uint32_t cc[2];
  if (CMP) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      cc[d] = (w[d] >> 14) & 0x00010001u;
      const uint32_t p0 = (uint32_t)__builtin_popcount(w[d] & 0x00001555u) & 1u;
      const uint32_t p1 = (uint32_t)__builtin_popcount(w[d] & 0x15550000u) & 1u;
      w[d] = (w[d] & ~0x40004000u) | (p0 << 14) | (p1 << 30);
    }
  } else {
    // coset bits of groups 4 kg .. 4 kg + 3 spread to bytes 0..3
    const uint32_t sp = __umul24((cs >> (4 * kg)) & 15u, 0x00204081u) & 0x01010101u;
    cc[0] = cc[1] = sp;
  }
  nq_f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // 16-bit halves: table entries (code byte 0 | c << 8), (code byte 1 | c << 8)
    const uint32_t sel = CMP ? ((b & 1) ? 0x06030602u : 0x04010400u)
                             : (0x04010400u + 0x01000100u * (uint32_t)b +
                                ((b & 1) ? 0x00020002u : 0u));
    const uint32_t ix = __builtin_amdgcn_perm(cc[b >> 1], w[b >> 1], sel);
    // entries ix.lo and ix.hi (< 512 each) of this lane's copy: byte offsets
    // (ix * TC + copy) * 8 in the two 16-bit halves
    const uint32_t ad = (ix << kShift) | lane_copy;
    const uint2 e0 = *reinterpret_cast<const uint2*>(tb + (ad & 0xffffu));
    const uint2 e1 = *reinterpret_cast<const uint2*>(tb + (ad >> 16));
    const nq_u4 bv = {e0.x, e0.y, e1.x, e1.y};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[b], __builtin_bit_cast(nq_bf16x8, bv), acc,
                                                  0, 0, 0);
  }
  // rows 4 kg .. 4 kg + 3: (head 2 kg hi, lo, head 2 kg + 1 hi, lo)
  v0 = (acc[0] + acc[1]) * f;
  v1 = (acc[2] + acc[3]) * f;
}

// ---------------------------------------------------------------------------
// Packed-key scores on the matrix cores, for 2-bit keys with one scale per
// vector at n = 128.  With q~ = H pad(q) and p = idx - 2 + c/2,
//   score = (s / sqrt n) sum_j q~_j p_j ,
// a dense contraction over the coordinates j: for 16 keys at a time,
// D[row][key] = sum_j A[row][j] B[j][key], B from the value table (exact
// bf16) and A the rotated queries, split into bf16 hi and lo parts (error
// below 2^-16 |q~_j| each).  Four 16x16x32 products
// cover the 128 coordinates.  Lane (key l % 16, group block g = l / 16)
// takes the 8-groups 4 g .. 4 g + 3 of its key (8 contiguous code bytes);
// product b uses 8-group 4 g + b, whose two table entries are that lane's B
// operand as they come.  Row 2h + part holds the hi or lo part of head h,
// so the lane of group block g receives both parts of heads 2g and 2g + 1 and
// adds them itself.  Each wave scores 32 consecutive keys per step with the
// next step's loads in flight, and two workgroups share a CU.
// ---------------------------------------------------------------------------
constexpr int kScoreMfmaBlock = 1024;

template <int HPP, typename QT, bool CMP>
__global__ __launch_bounds__(kScoreMfmaBlock, 8) void score_mfma_kernel(ScoreArgs a, int n_pass,
                                                                     int64_t chunk) {
  static_assert(HPP <= 8, "rows are (head, part)");
  constexpr int N = 128;
  constexpr int U = 2;                     // 16-key blocks per wave per step
  extern __shared__ float qt[];            // [HPP][N] rotated queries
  __shared__ uint2 tbl[512 * kTblCopies];  // the value table, kTblCopies copies
  const int64_t s = blockIdx.z;
  const int h = blockIdx.y / n_pass;
  const int pass = blockIdx.y % n_pass;
  const int grp = a.Hq / a.H;
  const int hq0 = h * grp + pass * HPP;
  const int nh = min(HPP, h * grp + grp - hq0);
  // one query coordinate per thread (HPP * N <= 1024 threads), loaded
  // while the table is built
  static_assert(HPP * N <= kScoreMfmaBlock, "one query coordinate per thread");
  const int qi = threadIdx.x;
  float qv = 0.f;
  if (qi < HPP * N && qi / N < nh && qi % N < a.d)
    qv = Io<QT>::load1(a.q, (s * a.Hq + hq0 + qi / N) * (int64_t)a.d + qi % N);
  value_table_copies<kTblCopies>(tbl);
  if (qi < HPP * N) qt[qi] = qv;
  __syncthreads();
  rotate_queries<HPP>(qt);
  const int lane = threadIdx.x & 63;
  // wave index in a scalar register: the key loop's control stays uniform
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nw = blockDim.x >> 6;
  const int col = lane & 15;               // key of the block; A row
  const int kg = lane >> 4;                // 8-groups 4 kg .. 4 kg + 3; heads 2 kg, 2 kg + 1
  nq_bf16x8 A[4];
  score_a_operands<HPP>(qt, nh, lane, A);
  const char* tb = reinterpret_cast<const char*>(tbl);
  // this workgroup's keys t0 .. t0 + nk - 1 (nk < 2^26: 32-bit offsets)
  const int64_t t0 = (int64_t)blockIdx.x * chunk;
  const int nk = (int)(min64(a.T, t0 + chunk) - t0);
  const int64_t base = (s * a.H + h) * a.pT + t0;
  const uint8_t* cp = a.codes + base * (N / 4);
  const uint16_t* csp = reinterpret_cast<const uint16_t*>(a.cosets) + base;
  const uint16_t* scp = a.scales + base;
  float* op = a.out + (s * a.Hq + hq0) * a.T + t0;
  // rows 0 .. nh-1 of the pass, keys t0 .. t0 + nk - 1 (below 2^31 bytes:
  // T < 2^26 and nh <= 8); dword 3 is the gfx9-family raw buffer format
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      op, 0, (int)(((uint32_t)(nh - 1) * (uint32_t)a.T + (uint32_t)nk) * 4u), 0x00020000);
  const uint32_t cofs = 8u * (uint32_t)kg;
  // 16-byte score stores need 16-byte aligned rows and chunk starts
  const bool vec_store = (a.T & 3) == 0 && (chunk & 3) == 0;
  // this lane's table copy, as a byte offset in both 16-bit halves
  const uint32_t lane_copy = (uint32_t)(lane % kTblCopies) * 8u * 0x00010001u;
  // codes, coset words and scales of a step's U blocks, in two register
  // sets used in turn: the next step's loads are in flight while a step
  // computes, and no register holding a load in flight is copied
  struct StepData {
    uint2 cw[U];
    uint32_t cs[U], sc[U];
  };
  auto load_step = [&](int kb_, StepData& d) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t t = (uint32_t)min(kb_ + 16 * u + col, nk - 1);
      d.cw[u] = *reinterpret_cast<const uint2*>(cp + (t * (uint32_t)(N / 4) + cofs));
      d.cs[u] = CMP ? 0u : (uint32_t)csp[t];
      d.sc[u] = scp[t];
    }
  };
  auto compute_step = [&](int kb, const StepData& sd) {
    const uint2* cw = sd.cw;
    const uint32_t* cs = sd.cs;
    const uint32_t* sc = sd.sc;
    float v[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u)
      score_block<CMP, kTblCopies>(A, cw[u], cs[u], kg, tb, lane_copy,
                                   h2f((uint16_t)sc[u]) * a.inv_sqrt_n, v[u][0], v[u][1]);
    // Stores through a buffer resource: every lane issues them, and a lane
    // with nothing to store (tail key, or head beyond nh) gets an offset past
    // the resource's range, which the hardware drops.  No store sits behind
    // a branch, so the waits for the next step's loads need not wait for
    // these stores.
    if (HPP > 4 && vec_store && kb + 16 * U <= nk) {
      // a whole step: transpose the (block u, head part j) values of each
      // quad of keys, so lane q = 2u + j of quad i holds keys 16u + 4i ..
      // 16u + 4i + 3 of head 2 kg + j, and store them as 16 bytes (each
      // head's 32 keys are one 128-byte line).  Measured: 1.3 % faster at
      // 5 heads a pass, 2.5 % slower at 4, where half the lanes store
      // nothing either way.
      static_assert(U == 2, "four values a lane");
      float x[4] = {v[0][0], v[0][1], v[1][0], v[1][1]};
      const int q = col & 3;
      float y[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) y[b] = dpp_a<0>(x[b ^ 1]);   // lane q ^ 1
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if ((b & 1) != (q & 1)) x[b] = y[b];
#pragma unroll
      for (int b = 0; b < 4; ++b) y[b] = dpp_a<1>(x[b ^ 2]);   // lane q ^ 2
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if ((b & 2) != (q & 2)) x[b] = y[b];
      const int head = 2 * kg + (q & 1);
      const int t = kb + 16 * (q >> 1) + (col & ~3);
      const uint32_t off =
          head < nh ? ((uint32_t)head * (uint32_t)a.T + (uint32_t)t) * 4u : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(nq_u4, make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                                               __float_as_uint(x[2]), __float_as_uint(x[3]))),
          orsrc, (int)off, 0, 0);
      return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = kb + 16 * u + col;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int head = 2 * kg + j;
        const bool ok = t < nk && head < nh;
        const uint32_t off = ok ? ((uint32_t)head * (uint32_t)a.T + (uint32_t)t) * 4u : 0xFFFFFFFCu;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[u][j]), orsrc, (int)off, 0, 0);
      }
    }
  };
  const int kstep = 16 * U * nw;
  StepData d0, d1;
  int kb = 16 * U * wv;
  if (kb < nk) load_step(kb, d0);
  // the scheduling barriers keep the prefetch loads ahead of the step's work
  for (; kb < nk; kb += 2 * kstep) {
    load_step(min(kb + kstep, nk - 1), d1);
    __builtin_amdgcn_sched_barrier(0);
    compute_step(kb, d0);
    if (kb + kstep >= nk) break;
    load_step(min(kb + 2 * kstep, nk - 1), d0);
    __builtin_amdgcn_sched_barrier(0);
    compute_step(kb + kstep, d1);
  }
}

// ---------------------------------------------------------------------------
// Packed-key scores on the matrix cores for 3-bit keys at n = 128 with one
// scale per vector or one per 64 coordinates (no compact packing): the same
// contraction as score_mfma_kernel, with the B operand formed arithmetically
// instead of from a table.  Lane (key col, k-group kg) loads the 12 code
// bytes of 8-groups 4 kg .. 4 kg + 3 of its key (group 4 kg + b at bits
// 24 b .. 24 b + 23 of the three words); for product b its 8 coordinates
// enter as bf16 of 2 p = 2 idx - 8 + c (exact small integers), and the
// factor 1/2 joins the scale.  With two scales the halves (coordinates 0..63
// in k-groups 0, 1; 64..127 in k-groups 2, 3) accumulate separately: each
// product runs twice, with the B operand of the other half's lanes zeroed.
// ---------------------------------------------------------------------------
template <int NS>
__device__ __forceinline__ void score_block3(const nq_bf16x8 (&A)[4], uint3 cw, uint32_t cs,
                                             int kg, float f0, float f1, float& v0, float& v1) {
  // coset bits of groups 4 kg .. 4 kg + 3
  const uint32_t cb = (cs >> (4 * kg)) & 15u;
  nq_f4 acc[NS];
#pragma unroll
  for (int hh = 0; hh < NS; ++hh) acc[hh] = nq_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // the group's 24-bit code word: 8 fields idx_j at bits 3 j
    uint32_t g;
    if (b == 0) g = cw.x;
    else if (b == 1) g = __builtin_amdgcn_alignbit(cw.y, cw.x, 24);
    else if (b == 2) g = __builtin_amdgcn_alignbit(cw.z, cw.y, 16);
    else g = cw.z >> 8;
    // 2 p - c + 8 = 2 idx; 2 p = 2 idx + c - 8
    const int off = (int)((cb >> b) & 1u) - 8;
    uint32_t bw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = (float)((int)((g >> (6 * e)) & 7u) * 2 + off);
      const float hi = (float)((int)((g >> (6 * e + 3)) & 7u) * 2 + off);
      // bf16 of both (exact: integers below 16 in magnitude), low first
      bw[e] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
    if (NS == 1) {
      const nq_bf16x8 B = __builtin_bit_cast(nq_bf16x8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[b], B, acc[0], 0, 0, 0);
    } else {
#pragma unroll
      for (int hh = 0; hh < NS; ++hh) {
        const bool mine = (kg >> 1) == hh;   // this lane's coordinates are in half hh
        const nq_bf16x8 B = __builtin_bit_cast(
            nq_bf16x8, make_uint4(mine ? bw[0] : 0u, mine ? bw[1] : 0u, mine ? bw[2] : 0u,
                                  mine ? bw[3] : 0u));
        acc[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[b], B, acc[hh], 0, 0, 0);
      }
    }
  }
  // rows 4 kg .. 4 kg + 3: (head 2 kg hi, lo, head 2 kg + 1 hi, lo)
  if (NS == 1) {
    v0 = (acc[0][0] + acc[0][1]) * f0;
    v1 = (acc[0][2] + acc[0][3]) * f0;
  } else {
    v0 = (acc[0][0] + acc[0][1]) * f0 + (acc[NS - 1][0] + acc[NS - 1][1]) * f1;
    v1 = (acc[0][2] + acc[0][3]) * f0 + (acc[NS - 1][2] + acc[NS - 1][3]) * f1;
  }
}

// Two workgroups per CU with one scale per vector (64 VGPRs); with two, the
// second accumulator and the masked operands need one workgroup's registers.
template <int HPP, typename QT, int NS>
__global__ __launch_bounds__(kScoreMfmaBlock, NS == 1 ? 8 : 4) void score_mfma3_kernel(
    ScoreArgs a, int n_pass, int64_t chunk) {
  static_assert(HPP <= 8, "rows are (head, part)");
  static_assert(NS == 1 || NS == 2, "one scale per vector or per 64 coordinates");
  constexpr int N = 128;
  constexpr int CB = 48;                   // code bytes per key
  constexpr int U = 2;                     // 16-key blocks per wave per step
  extern __shared__ float qt[];            // [HPP][N] rotated queries
  const int64_t s = blockIdx.z;
  const int h = blockIdx.y / n_pass;
  const int pass = blockIdx.y % n_pass;
  const int grp = a.Hq / a.H;
  const int hq0 = h * grp + pass * HPP;
  const int nh = min(HPP, h * grp + grp - hq0);
  static_assert(HPP * N <= kScoreMfmaBlock, "one query coordinate per thread");
  const int qi = threadIdx.x;
  float qv = 0.f;
  if (qi < HPP * N && qi / N < nh && qi % N < a.d)
    qv = Io<QT>::load1(a.q, (s * a.Hq + hq0 + qi / N) * (int64_t)a.d + qi % N);
  if (qi < HPP * N) qt[qi] = qv;
  __syncthreads();
  rotate_queries<HPP>(qt);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nw = blockDim.x >> 6;
  const int col = lane & 15;               // key of the block; A row
  const int kg = lane >> 4;                // 8-groups 4 kg .. 4 kg + 3; heads 2 kg, 2 kg + 1
  nq_bf16x8 A[4];
  score_a_operands<HPP>(qt, nh, lane, A);
  const int64_t t0 = (int64_t)blockIdx.x * chunk;
  const int nk = (int)(min64(a.T, t0 + chunk) - t0);
  const int64_t base = (s * a.H + h) * a.pT + t0;
  const uint8_t* cp = a.codes + base * CB;
  const uint16_t* csp = reinterpret_cast<const uint16_t*>(a.cosets) + base;
  const uint16_t* scp = a.scales + base * NS;
  float* op = a.out + (s * a.Hq + hq0) * a.T + t0;
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      op, 0, (int)(((uint32_t)(nh - 1) * (uint32_t)a.T + (uint32_t)nk) * 4u), 0x00020000);
  const uint32_t cofs = 12u * (uint32_t)kg;
  // the scale factor carries the 1/2 of the doubled code values
  const float fs = 0.5f * a.inv_sqrt_n;
  struct StepData {
    uint3 cw[U];
    uint32_t cs[U], sc[U];
  };
  auto load_step = [&](int kb_, StepData& d) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t t = (uint32_t)min(kb_ + 16 * u + col, nk - 1);
      d.cw[u] = *reinterpret_cast<const uint3*>(cp + (t * (uint32_t)CB + cofs));
      d.cs[u] = (uint32_t)csp[t];
      d.sc[u] = NS == 2 ? *reinterpret_cast<const uint32_t*>(scp + 2 * t) : (uint32_t)scp[t];
    }
  };
  auto compute_step = [&](int kb, const StepData& sd) {
    float v[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u)
      score_block3<NS>(A, sd.cw[u], sd.cs[u], kg, h2f((uint16_t)(sd.sc[u] & 0xffffu)) * fs,
                       h2f((uint16_t)(sd.sc[u] >> 16)) * fs, v[u][0], v[u][1]);
    // buffer stores: lanes with nothing to store take an offset past the
    // resource's range, which the hardware drops
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = kb + 16 * u + col;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int head = 2 * kg + j;
        const bool ok = t < nk && head < nh;
        const uint32_t off = ok ? ((uint32_t)head * (uint32_t)a.T + (uint32_t)t) * 4u : 0xFFFFFFFCu;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[u][j]), orsrc, (int)off, 0, 0);
      }
    }
  };
  const int kstep = 16 * U * nw;
  StepData d0, d1;
  int kb = 16 * U * wv;
  if (kb < nk) load_step(kb, d0);
  for (; kb < nk; kb += 2 * kstep) {
    load_step(min(kb + kstep, nk - 1), d1);
    __builtin_amdgcn_sched_barrier(0);
    compute_step(kb, d0);
    if (kb + kstep >= nk) break;
    load_step(min(kb + 2 * kstep, nk - 1), d0);
    __builtin_amdgcn_sched_barrier(0);
    compute_step(kb + kstep, d1);
  }
}

// Pipelined form of the table variant: each wave keeps kAttStages 32-token
// chunks in flight in LDS stages, filled by direct global -> LDS loads (no
// registers held for data in flight).  A stage holds the chunk's codes
// (1024 B, token t at 32 sigma(t), sigma spreading the tokens a lane group
// reads over distinct banks), the weights of up to 4 heads (128 B each), the
// 32 scales and the 32 coset words.  Two loads per chunk: the codes (64
// lanes x 16 B), then weights / scales / cosets (lanes 0..39).  The wait
// before a chunk's use counts the loads issued after it; no other vector
// memory operation is issued inside the loop.
// ---------------------------------------------------------------------------
constexpr int kAttStages = 3;
constexpr int kAttStage = 1664;           // bytes per stage

// token -> 32-byte slot of the stage's code area
__device__ __forceinline__ int att_sigma(int t) { return (t & ~7) | ((t + 2 * (t >> 3)) & 7); }
__device__ __forceinline__ int att_sigma_inv(int p) { return (p & ~7) | ((p - 2 * (p >> 3)) & 7); }

__device__ __forceinline__ void att_dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(src) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void att_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

template <int HPP, bool CMP>
__global__ __launch_bounds__(1024) void attend_dma_kernel(AttendArgs a, int n_pass) {
  static_assert(HPP <= 4, "rows are (head, part, sub)");
  constexpr int N = 128;
  constexpr int R = kAttStages;
  extern __shared__ __align__(16) char dyn[];   // stages; reduction buffer afterwards
  __shared__ uint2 tbl[512 * kTblCopies];   // kTblCopies copies of the value table
  value_table_copies<kTblCopies>(tbl);
  const int64_t s = blockIdx.z;
  const int h = blockIdx.y / n_pass;
  const int pass = blockIdx.y % n_pass;
  const int grp = a.Hq / a.H;
  const int hq0 = h * grp + pass * HPP;
  const int nh = min(HPP, h * grp + grp - hq0);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const int hh = col & 3;
  const bool arow = hh < nh;
  const uint32_t pmask = (col & 4) ? 0xffff0000u : 0u;
  const uint32_t asel = (col & 8) ? 0x03020c0cu : 0x0c0c0302u;
  const int T = (int)a.T;
  const int64_t base = (s * a.H + h) * a.pT;
  const float* wrow = a.w + (s * a.Hq + hq0) * a.T;
  const uint8_t* cp = a.codes + base * (N / 4);
  const uint16_t* csp = reinterpret_cast<const uint16_t*>(a.cosets) + base;
  const uint16_t* scp = a.scales + base;
  // this lane's sources for the two loads of a chunk at token c0:
  //  codes: cp + 32 c0 + goff;   rest: src1 + c0 * eb1 (active: act1)
  const int goff = 32 * att_sigma_inv(lane >> 1) + 16 * (lane & 1);
  const char* src1;
  int eb1;
  bool act1;
  if (lane < 32) {
    act1 = (lane >> 3) < nh;
    src1 = reinterpret_cast<const char*>(wrow + (int64_t)min(lane >> 3, nh - 1) * a.T + 4 * (lane & 7));
    eb1 = 4;
  } else if (lane < 36) {
    act1 = true;
    src1 = reinterpret_cast<const char*>(scp + 8 * (lane - 32));
    eb1 = 2;
  } else {
    act1 = !CMP && lane < 40;
    src1 = reinterpret_cast<const char*>(csp + 8 * (CMP ? 0 : lane - 36));
    eb1 = 2;
  }
  const uint32_t dyn0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dyn;
  const uint32_t wbase = dyn0 + (uint32_t)(wv * R * kAttStage);
  const char* wst = dyn + wv * R * kAttStage;        // this wave's stages
  nq_f4 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = nq_f4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  const int nfull = T >> 5;
  const int nk = nfull > wv ? (nfull - 1 - wv) / nw + 1 : 0;   // this wave's full chunks
  auto issue = [&](int k) {
    const int c0 = (wv + k * nw) * 32;
    const uint32_t sb = wbase + (uint32_t)((k % R) * kAttStage);
    att_dma16(cp + (int64_t)c0 * 32 + goff, __builtin_amdgcn_readfirstlane(sb));
    if (act1) att_dma16(src1 + (int64_t)c0 * eb1, __builtin_amdgcn_readfirstlane(sb + 1024));
  };
#pragma unroll
  for (int k = 0; k < R - 1; ++k)
    if (k < nk) issue(k);
  for (int k = 0; k < nk; ++k) {
    if (k + R - 1 < nk) issue(k + R - 1);
    // loads issued after chunk k's: 2 per later chunk
    const int later = min(R - 1, nk - 1 - k);
    if (later >= 3) att_wait_vm<6>();
    else if (later == 2) att_wait_vm<4>();
    else if (later == 1) att_wait_vm<2>();
    else att_wait_vm<0>();
    const char* st = wst + (k % R) * kAttStage;
    AttChunk ch;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t0 = 8 * kg + 2 * j;
      const uint32_t g0 = *reinterpret_cast<const uint16_t*>(st + 32 * att_sigma(t0) + 2 * col);
      const uint32_t g1 = *reinterpret_cast<const uint16_t*>(st + 32 * att_sigma(t0 + 1) + 2 * col);
      ch.cw[j] = g0 | (g1 << 16);
    }
    const uint4 sv = *reinterpret_cast<const uint4*>(st + 1536 + 16 * kg);
    ch.sw[0] = sv.x; ch.sw[1] = sv.y; ch.sw[2] = sv.z; ch.sw[3] = sv.w;
    if (!CMP) {
      const uint4 cv = *reinterpret_cast<const uint4*>(st + 1600 + 16 * kg);
      ch.cs[0] = cv.x; ch.cs[1] = cv.y; ch.cs[2] = cv.z; ch.cs[3] = cv.w;
    }
    if (arow) {
      const float4 w0 = *reinterpret_cast<const float4*>(st + 1024 + 128 * hh + 32 * kg);
      const float4 w1 = *reinterpret_cast<const float4*>(st + 1024 + 128 * hh + 32 * kg + 16);
      ch.wt[0] = w0.x; ch.wt[1] = w0.y; ch.wt[2] = w0.z; ch.wt[3] = w0.w;
      ch.wt[4] = w1.x; ch.wt[5] = w1.y; ch.wt[6] = w1.z; ch.wt[7] = w1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) ch.wt[i] = 0.f;
    }
    att_mma4<CMP, kTblCopies>(acc, ch, tbl, col, pmask, asel);
  }
  // the partial chunk (T not a multiple of 32), through registers
  if ((T & 31) != 0 && wv == nfull % nw) {
    AttChunk ch;
    const float* wr = wrow + (int64_t)(arow ? hh : 0) * a.T;
    att_load<false, CMP>(ch, cp + 2 * col, csp, scp, wr, nfull * 32 + 8 * kg, T, arow);
    att_mma4<CMP, kTblCopies>(acc, ch, tbl, col, pmask, asel);
  }
  att_wait_vm<0>();
  __syncthreads();                              // stages become the reduction buffer
  float* red = reinterpret_cast<float*>(dyn);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = acc[b][r] + __shfl_xor(acc[b][r], 16);
      if ((kg & 1) == 0 && r < HPP)
        red[(wv * HPP + r) * N + 8 * col + 2 * b + (kg >> 1)] = v;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HPP * N; i += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < nw; ++w) sum += red[w * HPP * N + i];
    red[i] = sum;
  }
  __syncthreads();
  for (int hs = 1; hs < N; hs <<= 1) {
    for (int i = threadIdx.x; i < HPP * (N / 2); i += blockDim.x) {
      const int g = i / (N / 2), r = i % (N / 2);
      const int j = (r / hs) * 2 * hs + (r % hs);
      const float x0 = red[g * N + j], x1 = red[g * N + j + hs];
      red[g * N + j] = x0 + x1;
      red[g * N + j + hs] = x0 - x1;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < nh * a.d; i += blockDim.x) {
    const int g = i / a.d, j = i % a.d;
    a.out[(s * a.Hq + hq0 + g) * (int64_t)a.d + j] = red[g * N + j] * a.inv_sqrt_n;
  }
}

// (slab, head) pairs per wave: about 8192 waves in all (32 per CU, the
// resident limit at <= 64 VGPRs), so that on long caches each wave walks all
// pairs of its token tile and reads its RoPE rows once.
inline int sh_chunk_for(int64_t SH, int64_t n_tt) {
  int64_t n_shc = (8192 + n_tt - 1) / n_tt;
  if (n_shc < 1) n_shc = 1;
  if (n_shc > SH) n_shc = SH;
  return (int)((SH + n_shc - 1) / n_shc);
}

// (slab, head) planes per quantize wave: up to 64, so that a wave reads its
// token tile's RoPE rows once for many planes, but no fewer than about 16384
// waves in all (short caches would otherwise leave most SIMDs idle; at the
// Mistral-7B shape 16384 waves measured 1.2 % faster than 8192 and the same
// as 32768).
inline int quantize_chunk(int64_t SH, int64_t n_tt) {
  int64_t c = SH * n_tt / 16384;
  if (c > 64) c = 64;
  if (c > SH) c = SH;
  if (c < 1) c = 1;
  return (int)c;
}

template <int N, int BITS, bool STRICT, typename T, int ROPE, bool PAD>
hipError_t quantize_fast_launch(const TensorArgs& a, hipStream_t s) {
  constexpr int TPW = 64 / (N / 8);
  const int64_t SH = a.n_vec / a.T;
  const int64_t n_tt = (a.T + TPW - 1) / TPW;
  const int chunk = quantize_chunk(SH, n_tt);
  const int64_t waves = n_tt * ((SH + chunk - 1) / chunk);
  const int64_t blocks = ((waves + kBlock / 64 - 1) / (kBlock / 64) + 7) / 8 * 8;
  hipLaunchKernelGGL((quantize_fast_kernel<N, BITS, STRICT, T, ROPE, PAD>),
                     dim3((unsigned)blocks), dim3(kBlock), 0, s, a, chunk, 1);
  return hipGetLastError();
}

template <int N, int BITS, bool STRICT, typename T>
hipError_t quantize_fast_rope(const TensorArgs& a, hipStream_t s) {
  if (a.rope == nullptr) {
    return a.d == N ? quantize_fast_launch<N, BITS, STRICT, T, 0, false>(a, s)
                    : quantize_fast_launch<N, BITS, STRICT, T, 0, true>(a, s);
  }
  if (a.d == 8) return quantize_fast_launch<N, BITS, STRICT, T, 3, false>(a, s);
  if (N >= 16 && a.d == N) return quantize_fast_launch<N, BITS, STRICT, T, 1, false>(a, s);
  return quantize_fast_launch<N, BITS, STRICT, T, 2, true>(a, s);
}

// 8 tokens per wave, up to 64 (slab, head) planes per wave, tile-major (the waves
// sharing a token tile are neighbours and share its RoPE rows in L2).
template <int BITS, bool STRICT, int NS>
hipError_t quantize_pair_launch(const TensorArgs& a, hipStream_t s) {
  const int64_t SH = a.n_vec / a.T;
  const int64_t n_tt = (a.T + 7) / 8;
  const int chunk = quantize_chunk(SH, n_tt);
  const int64_t waves = n_tt * ((SH + chunk - 1) / chunk);
  const int64_t blocks = ((waves + kBlock / 64 - 1) / (kBlock / 64) + 7) / 8 * 8;
  hipLaunchKernelGGL((quantize_pair_kernel<BITS, STRICT, NS>), dim3((unsigned)blocks),
                     dim3(kBlock), 0, s, a, chunk);
  return hipGetLastError();
}

template <int BITS>
hipError_t quantize_pair(const TensorArgs& a, hipStream_t s) {
  if (a.n_scales == 1)
    return a.strict ? quantize_pair_launch<BITS, true, 1>(a, s)
                    : quantize_pair_launch<BITS, false, 1>(a, s);
  return a.strict ? quantize_pair_launch<BITS, true, 2>(a, s)
                  : quantize_pair_launch<BITS, false, 2>(a, s);
}

// 16 tokens per wave, kQmChunk (slab, head) planes per wave, tile-fastest.
template <bool STRICT, int NS>
hipError_t quantize_mfma_launch(const TensorArgs& a, hipStream_t s) {
  const int64_t SH = a.n_vec / a.T;
  const int64_t n_tt = (a.T + 15) / 16;
  const int chunk = (int)(SH < kQmChunk ? SH : kQmChunk);
  const int64_t waves = n_tt * ((SH + chunk - 1) / chunk);
  const int64_t blocks = ((waves + kBlock / 64 - 1) / (kBlock / 64) + 7) / 8 * 8;
  hipLaunchKernelGGL((quantize_mfma_kernel<STRICT, NS>), dim3((unsigned)blocks), dim3(kBlock), 0,
                     s, a, chunk);
  return hipGetLastError();
}

template <int N, int BITS, typename T>
hipError_t quantize_n(const TensorArgs& a, hipStream_t s) {
  if constexpr (N <= 128) {
    // per-lane byte offsets are 32-bit, in the dense planes and the packed ones
    if (max64(a.T, a.pT) * a.d * (int64_t)sizeof(T) < ((int64_t)1 << 31)) {
      if constexpr (N == 128 && BITS == 2 && std::is_same<T, __half>::value) {
        // d = 128, or 96 (padded to 128: the last lane quarter feeds zeros)
        if ((a.d == 128 || a.d == 96) && a.rope == nullptr) {
          if (a.n_scales == 1)
            return a.strict ? quantize_mfma_launch<true, 1>(a, s) : quantize_mfma_launch<false, 1>(a, s);
          if (a.n_scales == 2)
            return a.strict ? quantize_mfma_launch<true, 2>(a, s) : quantize_mfma_launch<false, 2>(a, s);
        }
      }
      if constexpr (N == 128 && std::is_same<T, __half>::value) {
        if (a.d == 128 && a.rope != nullptr && (a.n_scales == 1 || a.n_scales == 2))
          return quantize_pair<BITS>(a, s);
      }
      return a.strict ? quantize_fast_rope<N, BITS, true, T>(a, s)
                      : quantize_fast_rope<N, BITS, false, T>(a, s);
    }
  }
  constexpr int VPB = kBlock / (N / 8);
  const int64_t blocks = (a.n_vec + VPB - 1) / VPB;
  if (a.strict)
    hipLaunchKernelGGL((quantize_kernel<N, BITS, true, T>), dim3((unsigned)blocks),
                       dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((quantize_kernel<N, BITS, false, T>), dim3((unsigned)blocks),
                       dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int N, int BITS, typename T, int ROPE>
hipError_t dequantize_fast_launch(const TensorArgs& a, hipStream_t s) {
  constexpr int TPW = 64 / (N / 8);
  const int64_t SH = a.n_vec / a.T;
  const int64_t n_tt = (a.T + TPW - 1) / TPW;
  const int chunk = sh_chunk_for(SH, n_tt);
  const int64_t waves = n_tt * ((SH + chunk - 1) / chunk);
  const int64_t blocks = ((waves + kBlock / 64 - 1) / (kBlock / 64) + 7) / 8 * 8;
  if (a.compact)
    hipLaunchKernelGGL((dequantize_fast_kernel<N, BITS, T, ROPE, true>), dim3((unsigned)blocks),
                       dim3(kBlock), 0, s, a, chunk, 0);
  else
    hipLaunchKernelGGL((dequantize_fast_kernel<N, BITS, T, ROPE, false>), dim3((unsigned)blocks),
                       dim3(kBlock), 0, s, a, chunk, 0);
  return hipGetLastError();
}

template <int N, int BITS, typename T>
hipError_t dequantize_tw_launch(const TensorArgs& a, hipStream_t s) {
  constexpr int TPW = 64 / (N / 8);
  constexpr int RUN = kTwTiles * TPW;
  const int64_t SH = a.n_vec / a.T;
  const int64_t n_tt = (a.T + TPW - 1) / TPW;
  const int64_t waves = SH * ((n_tt + kTwTiles - 1) / kTwTiles);
  const int64_t blocks = ((waves + kBlock / 64 - 1) / (kBlock / 64) + 7) / 8 * 8;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = (size_t)(kBlock / 64) *
                     tw_slice_bytes(RUN, N * BITS / 8, a.coset_bytes, a.n_scales);
  auto kern = a.compact ? dequantize_tw_kernel<N, BITS, T, true>
                        : dequantize_tw_kernel<N, BITS, T, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

// 16 tokens per wave, kDmChunk (slab, head) planes per wave, tile-fastest.
inline hipError_t dequantize_mfma_launch(const TensorArgs& a, const RopeFreqs& f, hipStream_t s) {
  const int64_t SH = a.n_vec / a.T;
  const int64_t n_tt = (a.T + 15) / 16;
  if (a.positions == nullptr) {
    const int64_t waves = SH * ((n_tt + kDtRun - 1) / kDtRun);
    const int64_t blocks = ((waves + kBlock / 64 - 1) / (kBlock / 64) + 7) / 8 * 8;
    if (a.compact)
      hipLaunchKernelGGL((dequantize_mfma_tw_kernel<true, true>), dim3((unsigned)blocks),
                         dim3(kBlock), 0, s, a, f);
    else
      hipLaunchKernelGGL((dequantize_mfma_tw_kernel<false, true>), dim3((unsigned)blocks),
                         dim3(kBlock), 0, s, a, f);
    return hipGetLastError();
  }
  const int chunk = (int)(SH < kDmChunk ? SH : kDmChunk);
  const int64_t waves = n_tt * ((SH + chunk - 1) / chunk);
  const int64_t blocks = ((waves + kBlock / 64 - 1) / (kBlock / 64) + 7) / 8 * 8;
  if (a.compact)
    hipLaunchKernelGGL((dequantize_mfma_kernel<true>), dim3((unsigned)blocks), dim3(kBlock), 0, s,
                       a, chunk, f);
  else
    hipLaunchKernelGGL((dequantize_mfma_kernel<false>), dim3((unsigned)blocks), dim3(kBlock), 0, s,
                       a, chunk, f);
  return hipGetLastError();
}

// Vectors without RoPE (values) on the same token-walking matrix-core
// kernel: d = n = 128, 2 bits, one scale per vector, fp16 output.
inline hipError_t dequantize_mfma_tw_norope_launch(const TensorArgs& a, hipStream_t s) {
  static const RopeFreqs none{};   // not read without RoPE
  const int64_t SH = a.n_vec / a.T;
  const int64_t n_tt = (a.T + 15) / 16;
  const int64_t waves = SH * ((n_tt + kDtRunV - 1) / kDtRunV);
  const int64_t blocks = ((waves + kBlock / 64 - 1) / (kBlock / 64) + 7) / 8 * 8;
  if (a.compact)
    hipLaunchKernelGGL((dequantize_mfma_tw_kernel<true, false>), dim3((unsigned)blocks),
                       dim3(kBlock), 0, s, a, none);
  else
    hipLaunchKernelGGL((dequantize_mfma_tw_kernel<false, false>), dim3((unsigned)blocks),
                       dim3(kBlock), 0, s, a, none);
  return hipGetLastError();
}

// Keys with RoPE that the matrix-core kernel dequantizes, forming its own
// cos / sin rows: d = n = 128, 2 bits, one scale per vector, fp16 output, and
// per-lane byte offsets that fit 32 bits in the dense and packed planes.
bool forms_rope_rows(const TensorArgs& a, int out_dtype) {
  return out_dtype == 0 && a.n == 128 && a.bits == 2 && a.d == 128 && a.n_scales == 1 &&
         max64(a.T, a.pT) * 256 < ((int64_t)1 << 31);
}

template <int N, int BITS, typename T>
hipError_t dequantize_n(const TensorArgs& a, const RopeFreqs* f, hipStream_t s) {
  if constexpr (N == 128 && BITS == 2 && std::is_same<T, __half>::value) {
    if (f != nullptr && forms_rope_rows(a, 0)) return dequantize_mfma_launch(a, *f, s);
    if (a.rope == nullptr && a.n == 128 && a.d == 128 && a.n_scales == 1 &&
        max64(a.T, a.pT) * 256 < ((int64_t)1 << 31))
      return dequantize_mfma_tw_norope_launch(a, s);
  }
  if constexpr ((N == 64 || N == 128) && (N * BITS / 8) % 16 == 0) {
    if (a.rope == nullptr) return dequantize_tw_launch<N, BITS, T>(a, s);
  }
  if constexpr (N <= 128) {
    if (a.rope == nullptr) return dequantize_fast_launch<N, BITS, T, 0>(a, s);
    if (a.d == 8) return dequantize_fast_launch<N, BITS, T, 3>(a, s);
    if (N >= 16 && a.d == N) return dequantize_fast_launch<N, BITS, T, 1>(a, s);
    return dequantize_fast_launch<N, BITS, T, 2>(a, s);
  }
  constexpr int VPB = kBlock / (N / 8);
  const int64_t blocks = (a.n_vec + VPB - 1) / VPB;
  hipLaunchKernelGGL((dequantize_kernel<N, BITS, T>), dim3((unsigned)blocks),
                     dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int BITS, int N, int HPP, typename T, int NS>
hipError_t score_lut_launch(const ScoreArgs& a, int n_pass, hipStream_t s) {
  constexpr int CB = N * BITS / 8, NG = N / 8, CSB = (NG + 7) / 8;
  const size_t lds = sizeof(float) * ((size_t)(CB + CSB) * 256 * HPP + HPP * N + HPP * NG);
  auto kern = a.compact ? score_lut_kernel<BITS, N, HPP, T, true, NS>
                        : score_lut_kernel<BITS, N, HPP, T, false, NS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // The tables take most of a CU's LDS, so one workgroup runs per CU: with
  // 256 or more (slab, head, pass) triples each builds its tables once and
  // streams all its keys; fewer are split over token chunks to cover the CUs.
  const int64_t pairs = a.S * a.H * n_pass;
  int64_t n_chunks = (256 + pairs - 1) / pairs;
  const int64_t min_chunk = 4 * kLutBlock;
  n_chunks = max64(1, min64(n_chunks, (a.T + min_chunk - 1) / min_chunk));
  const int64_t chunk = (a.T + n_chunks - 1) / n_chunks;
  const dim3 grid((unsigned)n_chunks, (unsigned)(a.H * n_pass), (unsigned)a.S);
  hipLaunchKernelGGL(kern, grid, dim3(kLutBlock), lds, s, a, n_pass, chunk);
  return hipGetLastError();
}

// Query heads whose tables fit in a CU's 160 KB of LDS (the launcher picks
// hpp from the device's limit, never above this).
template <int BITS, int N>
constexpr int lut_max_hpp() {
  constexpr int CB = N * BITS / 8, NG = N / 8, CSB = (NG + 7) / 8;
  constexpr int per_head = 4 * ((CB + CSB) * 256 + N + NG);
  return 160 * 1024 / per_head;
}

template <int HPP, typename T>
hipError_t score_mfma_launch(const ScoreArgs& a, int n_pass, hipStream_t s) {
  const size_t lds = sizeof(float) * HPP * 128;
  auto kern = a.compact ? score_mfma_kernel<HPP, T, true> : score_mfma_kernel<HPP, T, false>;
  // two workgroups per CU: 512 (slab, head, pass, token chunk) blocks or more
  const int64_t pairs = a.S * a.H * n_pass;
  int64_t n_chunks = (512 + pairs - 1) / pairs;
  const int64_t min_chunk = 4096;
  n_chunks = max64(1, min64(n_chunks, (a.T + min_chunk - 1) / min_chunk));
  const int64_t chunk = (a.T + n_chunks - 1) / n_chunks;
  const dim3 grid((unsigned)n_chunks, (unsigned)(a.H * n_pass), (unsigned)a.S);
  hipLaunchKernelGGL(kern, grid, dim3(kScoreMfmaBlock), lds, s, a, n_pass, chunk);
  return hipGetLastError();
}

template <int HPP, typename T, int NS>
hipError_t score_mfma3_launch(const ScoreArgs& a, int n_pass, hipStream_t s) {
  const size_t lds = sizeof(float) * HPP * 128;
  const int64_t pairs = a.S * a.H * n_pass;
  int64_t n_chunks = (512 + pairs - 1) / pairs;
  const int64_t min_chunk = 4096;
  n_chunks = max64(1, min64(n_chunks, (a.T + min_chunk - 1) / min_chunk));
  const int64_t chunk = (a.T + n_chunks - 1) / n_chunks;
  const dim3 grid((unsigned)n_chunks, (unsigned)(a.H * n_pass), (unsigned)a.S);
  hipLaunchKernelGGL((score_mfma3_kernel<HPP, T, NS>), grid, dim3(kScoreMfmaBlock), lds, s, a,
                     n_pass, chunk);
  return hipGetLastError();
}

template <typename T, int NS>
hipError_t score_mfma3(const ScoreArgs& a, hipStream_t s) {
  const int grp = a.Hq / a.H;
  const int n_pass = (grp + 7) / 8;
  const int hpp = (grp + n_pass - 1) / n_pass;
  switch (hpp) {
    case 1: return score_mfma3_launch<1, T, NS>(a, n_pass, s);
    case 2: return score_mfma3_launch<2, T, NS>(a, n_pass, s);
    case 3: return score_mfma3_launch<3, T, NS>(a, n_pass, s);
    case 4: return score_mfma3_launch<4, T, NS>(a, n_pass, s);
    case 5: return score_mfma3_launch<5, T, NS>(a, n_pass, s);
    case 6: return score_mfma3_launch<6, T, NS>(a, n_pass, s);
    case 7: return score_mfma3_launch<7, T, NS>(a, n_pass, s);
    default: return score_mfma3_launch<8, T, NS>(a, n_pass, s);
  }
}

template <typename T>
hipError_t score_mfma(const ScoreArgs& a, hipStream_t s) {
  const int grp = a.Hq / a.H;
  const int n_pass = (grp + 7) / 8;
  const int hpp = (grp + n_pass - 1) / n_pass;
  switch (hpp) {
    case 1: return score_mfma_launch<1, T>(a, n_pass, s);
    case 2: return score_mfma_launch<2, T>(a, n_pass, s);
    case 3: return score_mfma_launch<3, T>(a, n_pass, s);
    case 4: return score_mfma_launch<4, T>(a, n_pass, s);
    case 5: return score_mfma_launch<5, T>(a, n_pass, s);
    case 6: return score_mfma_launch<6, T>(a, n_pass, s);
    case 7: return score_mfma_launch<7, T>(a, n_pass, s);
    default: return score_mfma_launch<8, T>(a, n_pass, s);
  }
}

template <int BITS, int N, typename T, int NS>
hipError_t score_lut_hpp(const ScoreArgs& a, int hpp, int n_pass, hipStream_t s) {
  constexpr int kMax = lut_max_hpp<BITS, N>();
  if (hpp == 1) return score_lut_launch<BITS, N, 1, T, NS>(a, n_pass, s);
  if constexpr (kMax >= 2) {
    if (hpp == 2) return score_lut_launch<BITS, N, 2, T, NS>(a, n_pass, s);
  }
  if constexpr (kMax >= 3) {
    if (hpp == 3) return score_lut_launch<BITS, N, 3, T, NS>(a, n_pass, s);
  }
  if constexpr (kMax >= 4) {
    if (hpp == 4) return score_lut_launch<BITS, N, 4, T, NS>(a, n_pass, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS, int N, typename T>
hipError_t score_lut_n(const ScoreArgs& a, int max_lds, hipStream_t s) {
  constexpr int CB = N * BITS / 8, NG = N / 8, CSB = (NG + 7) / 8;
  const int grp = a.Hq / a.H;
  const size_t per_head = sizeof(float) * ((size_t)(CB + CSB) * 256 + N + NG);
  int hpp_max = (int)((size_t)max_lds / per_head);
  if (hpp_max < 1) return hipErrorInvalidValue;
  if (hpp_max > 4) hpp_max = 4;
  const int n_pass = (grp + hpp_max - 1) / hpp_max;
  const int hpp = (grp + n_pass - 1) / n_pass;
  const int ns = N / a.G;   // 1, 2 or 4 (G = n or a multiple of 64)
  if (ns == 1) return score_lut_hpp<BITS, N, T, 1>(a, hpp, n_pass, s);
  if constexpr (N >= 128) {
    if (ns == 2) return score_lut_hpp<BITS, N, T, 2>(a, hpp, n_pass, s);
  }
  if constexpr (N >= 256) {
    if (ns == 4) return score_lut_hpp<BITS, N, T, 4>(a, hpp, n_pass, s);
  }
  return hipErrorInvalidValue;
}

template <int N, int BITS, typename T>
hipError_t score_n(const ScoreArgs& a, hipStream_t s) {
  if constexpr (N == 128 && BITS == 2) {
    if (a.n_scales == 1 && a.T < ((int64_t)1 << 26)) return score_mfma<T>(a, s);
  }
  if constexpr (N == 128 && BITS == 3) {
    // 4-byte code loads need the token stride to keep them aligned (48 B a
    // key: always), the 2-scale words need 4-byte aligned scale rows
    if (!a.compact && a.T < ((int64_t)1 << 26)) {
      if (a.n_scales == 1) return score_mfma3<T, 1>(a, s);
      if (a.n_scales == 2 && ((uintptr_t)a.scales & 3) == 0) return score_mfma3<T, 2>(a, s);
    }
  }
  if constexpr (N >= 64) {
    const bool coset_bytes_align = (a.G == N) || (a.G % 64 == 0);
    int dev = 0, max_lds = 0;
    if (coset_bytes_align && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock,
                              dev) == hipSuccess &&
        max_lds >= 32 * 1024) {
      return score_lut_n<BITS, N, T>(a, max_lds, s);
    }
  }
  const dim3 grid((unsigned)((a.T + kScoreKeys - 1) / kScoreKeys), (unsigned)a.H,
                  (unsigned)a.S);
  const size_t lds = sizeof(float) * (size_t)(a.Hq / a.H) * N;
  hipLaunchKernelGGL((score_kernel<N, BITS, T>), grid, dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

#define NQ_DISPATCH_N(n, FN, BITS, T, ...)                \
  switch (n) {                                            \
    case 8: return FN<8, BITS, T>(__VA_ARGS__);           \
    case 16: return FN<16, BITS, T>(__VA_ARGS__);         \
    case 32: return FN<32, BITS, T>(__VA_ARGS__);         \
    case 64: return FN<64, BITS, T>(__VA_ARGS__);         \
    case 128: return FN<128, BITS, T>(__VA_ARGS__);       \
    case 256: return FN<256, BITS, T>(__VA_ARGS__);       \
    default: return hipErrorInvalidValue;                 \
  }

template <typename T>
hipError_t quantize_t(const TensorArgs& a, hipStream_t s) {
  if (a.bits == 2) { NQ_DISPATCH_N(a.n, quantize_n, 2, T, a, s) }
  if (a.bits == 3) { NQ_DISPATCH_N(a.n, quantize_n, 3, T, a, s) }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t dequantize_t(const TensorArgs& a, const RopeFreqs* f, hipStream_t s) {
  if (a.bits == 2) { NQ_DISPATCH_N(a.n, dequantize_n, 2, T, a, f, s) }
  if (a.bits == 3) { NQ_DISPATCH_N(a.n, dequantize_n, 3, T, a, f, s) }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t score_t(const ScoreArgs& a, hipStream_t s) {
  if (a.bits == 2) { NQ_DISPATCH_N(a.n, score_n, 2, T, a, s) }
  if (a.bits == 3) { NQ_DISPATCH_N(a.n, score_n, 3, T, a, s) }
  return hipErrorInvalidValue;
}


template <int BITS, int N, int HPP>
hipError_t attend_launch(const AttendArgs& a, hipStream_t s) {
  const int grp = a.Hq / a.H;
  const int n_pass = (grp + HPP - 1) / HPP;
  const size_t lds = sizeof(float) * (size_t)(att_block<BITS, HPP>() / 64) * HPP * N;
  auto kern = a.compact ? attend_kernel<BITS, N, HPP, true> : attend_kernel<BITS, N, HPP, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid(1u, (unsigned)(a.H * n_pass), (unsigned)a.S);
  hipLaunchKernelGGL(kern, grid, dim3(att_block<BITS, HPP>()), lds, s, a, n_pass);
  return hipGetLastError();
}

template <int HPP>
hipError_t attend_mfma_launch(const AttendArgs& a, hipStream_t s) {
  constexpr int kThreads = 1024;
  const int grp = a.Hq / a.H;
  const int n_pass = (grp + HPP - 1) / HPP;
  const size_t lds = sizeof(float) * (size_t)(kThreads / 64) * HPP * 128;
  auto kern = a.compact ? attend_mfma_kernel<HPP, true> : attend_mfma_kernel<HPP, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid(1u, (unsigned)(a.H * n_pass), (unsigned)a.S);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a, n_pass);
  return hipGetLastError();
}

template <int HPP>
hipError_t attend_mfma4_launch(const AttendArgs& a, hipStream_t s) {
  constexpr int kThreads = 1024;
  const int grp = a.Hq / a.H;
  const int n_pass = (grp + HPP - 1) / HPP;
  const size_t lds = sizeof(float) * (size_t)(kThreads / 64) * HPP * 128;
  auto kern = a.compact ? attend_mfma4_kernel<HPP, true> : attend_mfma4_kernel<HPP, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid(1u, (unsigned)(a.H * n_pass), (unsigned)a.S);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a, n_pass);
  return hipGetLastError();
}

template <int HPP>
hipError_t attend_dma_launch(const AttendArgs& a, hipStream_t s) {
  constexpr int kThreads = 1024;
  const int grp = a.Hq / a.H;
  const int n_pass = (grp + HPP - 1) / HPP;
  const size_t lds = std::max((size_t)(kThreads / 64) * kAttStages * kAttStage,
                              sizeof(float) * (size_t)(kThreads / 64) * HPP * 128) + 512;
  auto kern = a.compact ? attend_dma_kernel<HPP, true> : attend_dma_kernel<HPP, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid(1u, (unsigned)(a.H * n_pass), (unsigned)a.S);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a, n_pass);
  return hipGetLastError();
}
// Direct-to-LDS loads move 16 aligned bytes per lane: the weight rows (T a
// multiple of 4) and every plane's scale and coset rows (token stride a
// multiple of 8, 16-byte aligned planes) must allow it.
bool attend_dma_ok(const AttendArgs& a) {
  const auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  return (a.T & 3) == 0 && (a.pT & 7) == 0 && al(a.w) && al(a.codes) && al(a.scales) &&
         (a.compact || al(a.cosets));
}

template <int BITS, int N>
hipError_t attend_n(const AttendArgs& a, hipStream_t s) {
  const int grp = a.Hq / a.H;
  if constexpr (BITS == 2 && N == 128) {
    if (a.n_scales == 1 && a.T < ((int64_t)1 << 26)) {
      if (grp <= 4 && attend_dma_ok(a)) {
        if (grp <= 1) return attend_dma_launch<1>(a, s);
        if (grp <= 2) return attend_dma_launch<2>(a, s);
        return attend_dma_launch<4>(a, s);
      }
      if (grp <= 1) return attend_mfma4_launch<1>(a, s);
      if (grp <= 2) return attend_mfma4_launch<2>(a, s);
      if (grp <= 4) return attend_mfma4_launch<4>(a, s);
      return attend_mfma_launch<8>(a, s);
    }
  }
  if (grp <= 1) return attend_launch<BITS, N, 1>(a, s);
  if (grp <= 2) return attend_launch<BITS, N, 2>(a, s);
  if (grp <= 4 || N > 128) return attend_launch<BITS, N, 4>(a, s);
  return attend_launch<BITS, N, 8>(a, s);
}

template <int BITS>
hipError_t attend_b(const AttendArgs& a, hipStream_t s) {
  switch (a.n) {
    case 8: return attend_n<BITS, 8>(a, s);
    case 16: return attend_n<BITS, 16>(a, s);
    case 32: return attend_n<BITS, 32>(a, s);
    case 64: return attend_n<BITS, 64>(a, s);
    case 128: return attend_n<BITS, 128>(a, s);
    case 256: return attend_n<BITS, 256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.bits == 2) return attend_b<2>(a, s);
  if (a.bits == 3) return attend_b<3>(a, s);
  return hipErrorInvalidValue;
}

namespace {
}  // namespace

hipError_t launch_quantize(const TensorArgs& a, int in_dtype, hipStream_t s) {
  return in_dtype == 0 ? quantize_t<__half>(a, s) : quantize_t<float>(a, s);
}

bool dequantize_forms_rope_rows(const TensorArgs& a, int out_dtype) {
  return forms_rope_rows(a, out_dtype);
}

hipError_t launch_dequantize(const TensorArgs& a, int out_dtype, const RopeFreqs* f,
                             hipStream_t s) {
  return out_dtype == 0 ? dequantize_t<__half>(a, f, s) : dequantize_t<float>(a, f, s);
}

hipError_t launch_score(const ScoreArgs& a, int in_dtype, hipStream_t s) {
  return in_dtype == 0 ? score_t<__half>(a, s) : score_t<float>(a, s);
}

}  // namespace nq
