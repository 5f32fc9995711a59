// Internal interface between the C-ABI front end (nq_api.cpp) and the HIP
// kernels (nq_kernels.hip).  Not installed; the public ABI is include/nq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nq.h"

namespace nq {

// One KV tensor pass (quantize or dequantize).
struct TensorArgs {
  const void* x;        // quantize: input [S][H][T][d]
  void* y;              // dequantize: output [S][H][T][d]
  uint8_t* codes;       // packed planes (quantize writes, dequantize reads)
  uint8_t* cosets;
  uint16_t* scales;     // fp16 bits
  const float2* rope;   // [T][d/2] (cos, sin), or nullptr: no RoPE step
  int64_t n_vec;        // S * H * T
  int64_t T;            // tokens of this call (dense x / y planes hold T)
  int64_t pT;           // token stride of the packed planes (>= T); the plane
                        // bases already point at the call's first token
  int d, n, G, bits, strict, code_bytes, coset_bytes, n_scales;
  int compact;          // coset bit folded into idx_7's low bit (no coset plane)
  float eps;            // fp32(1e-8 * sqrt(n)): floor of the group maximum of |H v|
  float half_L;         // L / 2
  double sigma_k;       // 1 / ((L/2) * sqrt(n)): stored scale = a * sigma_k
  float inv_sqrt_n;     // fp32(1 / sqrt(n))
  // quantize only: the fp64 pass
  const double* omega;             // RoPE frequencies [d/2] in fp64, or nullptr
  const int32_t* positions;        // RoPE positions [T], or nullptr: pos0 + t
  int64_t pos0;
  unsigned long long* queue_count; // vectors queued for the fp64 pass
  int64_t* queue;                  // their indices (slab * H + head) * T + t
  int64_t queue_cap;               // entries the queue holds
  double eps64;                    // 1e-8 * sqrt(n)
  double half_L64;                 // L / 2
};

struct ScoreArgs {
  const uint8_t* codes;
  const uint8_t* cosets;
  const uint16_t* scales;
  const void* q;        // [S][Hq][d]
  float* out;           // [S][Hq][T]
  int64_t S, T;
  int64_t pT;           // token stride of the packed planes (>= T)
  int H, Hq, d, n, G, bits, code_bytes, coset_bytes, n_scales;
  int compact;          // coset bit folded into idx_7's low bit (no coset plane)
  float half_L;
  float inv_sqrt_n;
};

struct AttendArgs {
  const uint8_t* codes;
  const uint8_t* cosets;
  const uint16_t* scales;
  const float* w;       // [S][Hq][T]
  float* out;           // [S][Hq][d]
  int64_t S, T;
  int64_t pT;           // token stride of the packed planes (>= T)
  int H, Hq, d, n, G, bits, code_bytes, coset_bytes, n_scales;
  int compact;          // coset bit folded into idx_7's low bit (no coset plane)
  float half_L;
  float inv_sqrt_n;
};

constexpr int kMaxHalfDim = 128;
struct RopeFreqs {
  double omega[kMaxHalfDim];  // theta^(-2i/d), computed on the host
  // cos and sin of 16 omega_i (the angle step of a 16-token tile), rounded
  // once to fp32 on the host
  float step_c[kMaxHalfDim], step_s[kMaxHalfDim];
};

// cos / sin of positions[t] (or pos0 + t when positions is null) times
// omega_i, rounded once to fp32, into `table`.  Also copies the frequencies
// to `omega` and clears the n_counters queue counters (each if not null).
hipError_t launch_rope_table(const int32_t* positions, int64_t pos0, int64_t T,
                             int d, const RopeFreqs& f, float2* table,
                             double* omega, unsigned long long* counters,
                             int n_counters, hipStream_t stream);
hipError_t launch_clear_counters(unsigned long long* counters, int n, hipStream_t s);
// The fp64 pass: the queued vectors (all = 0) or every vector (all = 1).
hipError_t launch_exact(const TensorArgs& a, int in_dtype, int all, hipStream_t s);
// The fp64 pass over both tensors of a call in one launch (same n, bits and
// parity).
hipError_t launch_exact2(const TensorArgs& ak, const TensorArgs& av, int in_dtype, int all,
                         hipStream_t s);
hipError_t launch_quantize(const TensorArgs& a, int in_dtype, hipStream_t s);
// The body of nq_quantize_kv (argument checks, launches) on a given workspace.
int quantize_impl(const nq_config* cfg, const void* k, const void* v, int64_t S, int32_t H,
                  int64_t T, const int32_t* positions, const nq_packed* pk, const nq_packed* pv,
                  void* ws, size_t ws_bytes, void* stream);
// Dequantize; for keys with RoPE, f holds the frequencies (a kernel that
// forms its own cos / sin rows uses f, the others the table at a.rope).
hipError_t launch_dequantize(const TensorArgs& a, int out_dtype, const RopeFreqs* f,
                             hipStream_t s);
// Whether dequantize forms the cos / sin rows itself for these keys (then
// no table is built).
bool dequantize_forms_rope_rows(const TensorArgs& a, int out_dtype);
hipError_t launch_score(const ScoreArgs& a, int in_dtype, hipStream_t s);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);
hipError_t launch_decode_debug(const float* y, int64_t n_groups, int bits,
                               int strict, int constrained, uint8_t* idx,
                               uint8_t* coset, hipStream_t s);

}  // namespace nq
