/*
 * nq.h -- C ABI of libnq: E8 lattice quantization of a transformer KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page and section):
 *  [Walk]  NexusQuant blog (nexusquant.hashnode.dev), E8 walkthrough post:
 *          "The E8 Lattice, Briefly", "The Conway-Sloane Nearest-Point
 *          Algorithm", "Python Implementation", "Why Per-Group Scaling?",
 *          "The Relaxed Parity Discovery", "Bit Rate Accounting",
 *          "What Makes This Hard in Practice".
 *  [Had]   Same blog, post "The E8 lattice quantizes 8 numbers at once",
 *          "Handling outliers".
 *  [RM]    nexusquant-kv 0.5.1 README, "How it works", "API reference"
 *          (compress_kv_cache: head_dim, rope_base, bits), "Results".
 *  [E8KQ]  Nedelkoski et al., "E8 Lattice Key Quantization for Low-Bit
 *          KV-Cache Compression", Abstract and Table 3 (table-based
 *          asymmetric scoring of packed keys).
 *
 * Conventions for every entry point
 *  - Device pointers are HIP device (or managed) memory; host pointers are
 *    marked "host".  The caller owns every buffer; the library allocates
 *    nothing, keeps no state between calls and may be called from several
 *    host threads at once (on different output buffers).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; the call returns once it is enqueued.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    negative nq_status means nothing was launched.  NQ_ERR_HIP reports a
 *    launch failure.  Faults during execution surface at the caller's next
 *    synchronisation.  Nothing throws across the ABI.
 *  - Device pointers must be 16-byte aligned.
 *  - Tensors are row-major.  A KV tensor is [S][H][T][d] ("slabs" S =
 *    layers x batch, H KV heads, T tokens, head_dim d), fp16 (or fp32 when
 *    cfg->in_dtype == NQ_DTYPE_F32).
 *  - Inputs that are not finite, or whose group scale overflows fp16, give
 *    unspecified codes (not checked).
 */
#ifndef NQ_H_
#define NQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NQ_OK = 0,
  NQ_ERR_INVALID_ARG = -1, /* null / misaligned pointer, bad size or shape */
  NQ_ERR_UNSUPPORTED = -2, /* valid but not implemented (see nq_config)    */
  NQ_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  NQ_ERR_HIP = -4          /* a HIP launch or API call failed              */
} nq_status;

enum { NQ_PARITY_STRICT = 0, NQ_PARITY_RELAXED = 1 };
enum { NQ_ROPE_SCALING_NONE = 0, NQ_ROPE_SCALING_LINEAR = 1, NQ_ROPE_SCALING_LLAMA3 = 2 };
enum { NQ_PACKING_STANDARD = 0, NQ_PACKING_COMPACT = 1 };
enum { NQ_DTYPE_F16 = 0, NQ_DTYPE_F32 = 1 };
enum { NQ_PLANE_CODES = 0, NQ_PLANE_COSETS = 1, NQ_PLANE_SCALES = 2 };

/* Codec parameters ([RM] "API reference": head_dim, rope_base, bits;
 * [Walk] "Why Per-Group Scaling?": scale group; "The Relaxed Parity
 * Discovery": parity mode).
 *  head_dim    d, a multiple of 8 in [8, 256]; vectors are zero-padded to
 *              n = the next power of two >= d ([RM] "How it works" step 4).
 *              With rope_theta > 0, d must be 8 or a multiple of 16.
 *  bits_k/v    2 or 3 bits per coordinate for keys / values (levels L = 2^b,
 *              [Walk] "Python Implementation": 4 levels = 2-bit, 8 = 3-bit).
 *  scale_group G: coordinates per fp16 scale; a multiple of 8 dividing n,
 *              or 0 for G = n (one scale per head vector).
 *  parity      NQ_PARITY_STRICT: E8 = D8 u (D8 + 1/2) (even coordinate sum
 *              on both cosets); NQ_PARITY_RELAXED: D8 u (Z^8 + 1/2).
 *  in_dtype    NQ_DTYPE_F16 or NQ_DTYPE_F32 for K/V/query inputs and for
 *              dequantized outputs.
 *  rope_theta  > 0: keys carry split-half RoPE with base theta (frequency
 *              theta^(-2i/d), pair (i, i + d/2)); it is removed before
 *              quantizing and re-applied on dequantize.  0: keys are
 *              quantized as given (the README's "fast" mode, no RoPE removal).
 *
 * RoPE frequency scaling ([RM] "API reference": rope_scaling, the model
 * config's dict, for Llama-3.1 and similar; "Limitations": linear scaling and
 * Llama-3.1 at long context).  Each frequency w_i = theta^(-2i/d) becomes:
 *  NQ_ROPE_SCALING_NONE    w_i (the remaining fields are ignored)
 *  NQ_ROPE_SCALING_LINEAR  w_i / rope_factor
 *  NQ_ROPE_SCALING_LLAMA3  with wavelength l = 2 pi / w_i and the original
 *      context C = rope_original_max: w_i where l < C / high_freq_factor;
 *      w_i / rope_factor where l > C / low_freq_factor; between the two,
 *      (1 - a) w_i / rope_factor + a w_i with
 *      a = (C / l - low_freq_factor) / (high_freq_factor - low_freq_factor).
 * Everything is evaluated in fp64 in that order on the host.  Requirements:
 * rope_factor > 0; LLAMA3 also 0 < low_freq_factor < high_freq_factor and
 * rope_original_max > 0; otherwise NQ_ERR_INVALID_ARG.
 *
 * packing ([Walk] "Bit Rate Accounting": b bits per coordinate; "The Relaxed
 * Parity Discovery": strict E8 keeps an even coordinate sum on both cosets)
 *  NQ_PACKING_STANDARD  codes plus a coset plane (one bit per 8-group)
 *  NQ_PACKING_COMPACT   strict parity only (else NQ_ERR_INVALID_ARG): a
 *      strict codeword's index sum is even, so the low bit of idx_7 is the
 *      parity of the low bits of idx_0..idx_6; that bit position stores the
 *      coset bit instead.  Exactly 8b bits per group; the coset plane has 0
 *      bytes and its pointer may be NULL.
 *
 * exact ([Walk] "The Conway-Sloane Nearest-Point Algorithm": the code of a
 * group is the nearest lattice point of its scaled coordinates y; the pages
 * fix no precision for y, read here as fp64 from the exact input values)
 *  0  y and the decisions in fp32; every vector with a group whose decision
 *     margin (squared-distance gap to the next best codeword) is below
 *     1.6e-5 in units of y is recomputed in fp64 -- RoPE removal, transform,
 *     group maximum, y = (L/2) u / a correctly rounded -- and decided there.
 *     The result equals the fp64 definition except where fp64 itself cannot
 *     separate two codewords.
 *  1  every vector takes the fp64 path (a reference mode, many times slower).
 */
typedef struct {
  int32_t head_dim;
  int32_t bits_k;
  int32_t bits_v;
  int32_t scale_group;
  int32_t parity;
  int32_t in_dtype;
  double rope_theta;
  int32_t rope_scaling;          /* NQ_ROPE_SCALING_*                       */
  int32_t rope_original_max;     /* LLAMA3: original context length C       */
  double rope_factor;            /* LINEAR, LLAMA3                          */
  double rope_low_freq_factor;   /* LLAMA3                                  */
  double rope_high_freq_factor;  /* LLAMA3                                  */
  int32_t packing;               /* NQ_PACKING_*                            */
  int32_t exact;                 /* 0 or 1, see above                       */
} nq_config;

/* Packed form of one KV tensor: three device planes, each row-major over
 * [S][H][token_capacity] vectors ([Walk] "Bit Rate Accounting": b bits per
 * coordinate plus a 16-bit scale; one coset bit per 8-group is added so both
 * cosets fit):
 *   codes  : n*b/8 bytes per vector; coordinate j at bits [j*b, j*b+b) of the
 *            vector's little-endian bit stream, value idx = p - c/2 + L/2
 *   cosets : ceil(n/64) bytes per vector; bit m = 1 when 8-group m lies on
 *            the half-integer coset
 *   scales : n/G fp16 per vector, sigma = max|z| / (L/2) over the group, z the
 *            orthonormally rotated vector
 * The three pointers must be 16-byte aligned; sizes from nq_packed_bytes for
 * S * H * token_capacity vectors.  With NQ_PACKING_COMPACT the coset plane
 * is empty (cosets may be NULL) and bit 7b of each group's code bits holds
 * the coset bit in place of the low bit of idx_7.
 *
 * Token window (decode-time append, [RM] "HuggingFace ecosystem": the cache
 * keeps growing during decode): a call on n_tokens tokens touches tokens
 * [token_offset, token_offset + n_tokens) of every (slab, head) plane.
 * token_capacity = 0 means token_offset + n_tokens; otherwise the window must
 * fit (NQ_ERR_INVALID_ARG).  Both 0 is a dense cache of exactly n_tokens.
 * With positions == NULL, keys take RoPE positions token_offset + t. */
typedef struct {
  void* codes;
  void* cosets;
  void* scales;
  int64_t token_capacity;  /* tokens per (slab, head) plane, or 0          */
  int64_t token_offset;    /* first token of the call inside each plane    */
} nq_packed;

/* Host.  Bytes of one plane for n_vectors vectors of keys (is_value = 0) or
 * values (is_value = 1).  Returns 0 for an invalid config or plane. */
size_t nq_packed_bytes(const nq_config* cfg, int is_value, int64_t n_vectors,
                       int plane);

/* Host.  Workspace bytes that quantize needs for a call on n_slabs x
 * n_kv_heads x n_tokens vectors; dequantize takes the same workspace (it uses
 * its first part only).  In order, each part rounded up to 256 bytes: the
 * RoPE cos/sin table in fp32 (T * d/2 * 8 bytes) and the fp64 frequencies
 * (d/2 * 8 bytes), both only when rope_theta > 0; 256 bytes of queue
 * counters; two
 * queues (keys, values) of the vectors that take the fp64 path, 8 bytes per
 * entry, min(S*H*T, max(1024, S*H*T / 32)) entries each.  Returns 0 for an
 * invalid config or shape.  Scoring and attention need no workspace. */
size_t nq_workspace_bytes(const nq_config* cfg, int64_t n_slabs, int32_t n_kv_heads,
                          int64_t n_tokens);

/* Host.  Static text for a status code. */
const char* nq_status_string(int status);

/* Quantize + pack a post-prefill KV cache ([RM] "How it works" steps 3-5,
 * [Walk] "Python Implementation").  Per token and head: keys lose RoPE
 * (rope_theta > 0), the vector is zero-padded to n and rotated by the
 * Walsh-Hadamard matrix, scaled per group of G, and each 8-group is replaced
 * by its nearest codeword of the lattice restricted to b-bit coordinates.
 * Arithmetic: fp32, with the fp64 pass of cfg->exact for near-ties, so that
 * codes, coset bits and scales are those of the fp64 definition (y = (L/2)
 * u / a, u = H pad(RoPE^-1(x)), a the group maximum of |u| floored at
 * 1e-8 sqrt(n)), up to codeword pairs fp64 cannot separate.  The fp32
 * transform runs as butterfly stages, or for fp16 vectors without RoPE at
 * d = n = 128, 2 bits, one scale per vector, as a +-1 matrix product on the
 * matrix cores (exact products, fp32 sums).
 *  k, v        device [S][H][T][d] inputs; either may be NULL (then the
 *              matching packed planes are not touched)
 *  positions   device int32 [T] token positions for RoPE, or NULL for
 *              token_offset + (0..T-1); values must be >= 0
 *  pk, pv      host structs holding device plane pointers (outputs)
 *  workspace   device scratch of nq_workspace_bytes(cfg, S, H, T) bytes; its
 *              contents on entry do not matter, and calls that share one
 *              workspace must not overlap in time
 * Errors: NQ_ERR_INVALID_ARG (sizes <= 0, null config, misalignment),
 * NQ_ERR_UNSUPPORTED (see nq_config), NQ_ERR_WORKSPACE, NQ_ERR_HIP. */
int nq_quantize_kv(const nq_config* cfg, const void* k, const void* v,
                   int64_t n_slabs, int32_t n_kv_heads, int64_t n_tokens,
                   const int32_t* positions, const nq_packed* pk,
                   const nq_packed* pv, void* workspace, size_t ws_bytes,
                   void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments and results as nq_quantize_kv, with no workspace
 * argument.  Its workspace is a library-owned device array of 32 MiB per
 * GPU (allocated when the library's code is loaded on that GPU and held until
 * the process ends), so calls that need more -- nq_workspace_bytes(cfg, S, H,
 * T) > 32 MiB, e.g. more than about 55K tokens at d = 128 with RoPE --
 * return NQ_ERR_WORKSPACE before anything is enqueued.  It calls no
 * allocating routine.  Every call on one GPU shares that array: calls whose
 * work overlaps in time on one GPU (other streams, other host threads) race
 * and give undefined results; calls in one stream are ordered and safe.
 * The array's contents between calls do not matter (each call clears what it
 * counts). */
int nq_quantize_kv_noalloc(const nq_config* cfg, const void* k, const void* v,
                           int64_t n_slabs, int32_t n_kv_heads, int64_t n_tokens,
                           const int32_t* positions, const nq_packed* pk,
                           const nq_packed* pv, void* stream);

/* Inverse path ([Walk] "What Makes This Hard in Practice", item 3: unpack on
 * the device; [RM] "How it works": RoPE re-applied after quantization):
 * p = idx - L/2 + c/2, z = s16 * p, x = (H z / sqrt(n))[:d], keys get RoPE
 * at `positions` (rope_theta > 0), rounded to the output dtype (RNE).
 * Arithmetic: fp32.  For fp16 output at d = n = 128, 2 bits, one scale per
 * vector (keys with RoPE, and vectors without it), H p is formed exactly on
 * the matrix cores and scaled by s16 / sqrt(n) once; otherwise
 * z = s16 / sqrt(n) * p goes through butterfly stages.  RoPE cos / sin: fp64
 * angle reduction, then fp32 sincos (the quantize path's values), except
 * for those matrix-core keys with positions == NULL: there the kernel forms
 * them at the start of each 128-token run and rotates them by the 16-token
 * angle step (within 4e-7 of the directly formed values), so a window read
 * at token_offset may differ from a read with explicit positions by one step
 * of the output dtype.
 *  k_out, v_out  device [S][H][T][d] outputs (either may be NULL)
 *  workspace     with keys and rope_theta > 0: at least the fp32 RoPE table
 *                (T * d/2 * 8 bytes, e.g. a workspace of nq_workspace_bytes);
 *                otherwise unused (may be NULL)
 * Errors as nq_quantize_kv. */
int nq_dequantize_kv(const nq_config* cfg, const nq_packed* pk,
                     const nq_packed* pv, int64_t n_slabs, int32_t n_kv_heads,
                     int64_t n_tokens, const int32_t* positions, void* k_out,
                     void* v_out, void* workspace, size_t ws_bytes,
                     void* stream);

/* Table-based asymmetric q.k scoring on packed keys without dequantizing
 * them ([E8KQ] Abstract, Table 3).  For query head h of slab s:
 *   scores[s][h][t] = q[s][h] . D0(K)[s][h / (n_q_heads / n_kv_heads)][t]
 * where D0 is the dequantization without the RoPE step (scores are taken in
 * the codec frame; with rope_theta == 0 they are plain q.k logits).
 *  q       device [S][n_q_heads][d] queries (in_dtype)
 *  scores  device fp32 [S][n_q_heads][T]
 * n_q_heads must be a positive multiple of n_kv_heads.  workspace may be NULL.
 * Arithmetic: fp32 sums.  For 2-bit keys with one scale per vector at
 * n = 128 the per-coordinate products run on bf16 matrix cores, with the
 * code values exact and each rotated query coordinate split into two bf16
 * parts (relative error below 2^-16 per term).
 * Errors as nq_quantize_kv. */
int nq_score_packed_keys(const nq_config* cfg, const nq_packed* pk,
                         int64_t n_slabs, int32_t n_kv_heads,
                         int32_t n_q_heads, int64_t n_tokens, const void* q,
                         float* scores, void* workspace, size_t ws_bytes,
                         void* stream);

/* Value half of decode attention on the packed cache ([Walk] "What Makes
 * This Hard in Practice", item 3: the packed form stays on the device and is
 * used there; [E8KQ] Abstract: attention over the compressed cache):
 *   out[s][h][:] = sum_t weights[s][h][t] * D(V)[s][h / (n_q_heads / n_kv_heads)][t][:]
 * with D the dequantization of the values (no RoPE), summed in the codec
 * frame (one inverse Walsh-Hadamard transform per query head).
 *  pv       packed values (bits_v, scale_group, parity from cfg)
 *  weights  device fp32 [S][n_q_heads][T] (e.g. softmax of the scores)
 *  out      device fp32 [S][n_q_heads][d]
 * n_q_heads must be a positive multiple of n_kv_heads.  The result is
 * deterministic (fixed reduction order).  Arithmetic: fp32 sums; for 2-bit
 * values with one scale per vector at n = 128 the per-token products run on
 * bf16 matrix cores, with the code values exact and each weight * scale
 * split into two bf16 parts (relative error below 2^-14 per term).
 * Errors as nq_quantize_kv. */
int nq_attend_packed_values(const nq_config* cfg, const nq_packed* pv,
                            int64_t n_slabs, int32_t n_kv_heads,
                            int32_t n_q_heads, int64_t n_tokens,
                            const float* weights, float* out, void* stream);

/* Test hook: the nearest-point decoder alone ([Walk] "The Conway-Sloane
 * Nearest-Point Algorithm") on caller-given groups y (lattice units).
 *  y            device fp32 [n_groups][8]
 *  constrained  1: the cube-limited decoder the quantize kernels use (for
 *               b = 2 the same 2-bit decoder), valid for |y_k| <= L/2 (the
 *               range the scale step produces); idx in [0, L-1]
 *               0: nearest point of the whole lattice (E8, or D8 u (Z^8 + 1/2)
 *               relaxed), no cube limit; idx = p - c/2 + L/2 written as a
 *               two's-complement int8 (|y_k| <= 60)
 *  idx_out      device uint8 [n_groups][8], idx = p - c/2 + L/2 (L = 2^bits)
 *  coset_out    device uint8 [n_groups]
 * bits 2 or 3; parity NQ_PARITY_STRICT or NQ_PARITY_RELAXED. */
int nq_e8_decode_debug(const float* y, int64_t n_groups, int32_t bits,
                       int32_t parity, int32_t constrained, uint8_t* idx_out,
                       uint8_t* coset_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NQ_H_ */
