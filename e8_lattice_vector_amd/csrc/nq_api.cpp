// C-ABI front end of libnq: argument validation, layout arithmetic and
// kernel launches.  Every check runs on the host before anything is
// enqueued; nothing is allocated and no state is kept between calls.
#include <math.h>
#include <string.h>

#include "../../include/nq.h"
#include "nq_internal.h"

namespace {

struct Layout {
  int d, n, G, bits, L, code_bytes, coset_bytes, n_scales, compact;
};

int next_pow2_min8(int d) {
  int n = 8;
  while (n < d) n <<= 1;
  return n;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validates the parts of the config that do not depend on K vs V.
int check_config(const nq_config* c) {
  if (c == nullptr) return NQ_ERR_INVALID_ARG;
  const int d = c->head_dim;
  if (d < 8 || d > 256 || (d % 8) != 0) return NQ_ERR_UNSUPPORTED;
  if (!(c->bits_k == 2 || c->bits_k == 3)) return NQ_ERR_UNSUPPORTED;
  if (!(c->bits_v == 2 || c->bits_v == 3)) return NQ_ERR_UNSUPPORTED;
  if (c->parity != NQ_PARITY_STRICT && c->parity != NQ_PARITY_RELAXED)
    return NQ_ERR_INVALID_ARG;
  if (c->in_dtype != NQ_DTYPE_F16 && c->in_dtype != NQ_DTYPE_F32)
    return NQ_ERR_INVALID_ARG;
  if (!(c->rope_theta >= 0.0) || !isfinite(c->rope_theta)) return NQ_ERR_INVALID_ARG;
  if (c->rope_theta > 0.0 && !(d == 8 || d % 16 == 0)) return NQ_ERR_UNSUPPORTED;
  if (c->rope_scaling == NQ_ROPE_SCALING_LINEAR || c->rope_scaling == NQ_ROPE_SCALING_LLAMA3) {
    if (!(c->rope_factor > 0.0) || !isfinite(c->rope_factor)) return NQ_ERR_INVALID_ARG;
  } else if (c->rope_scaling != NQ_ROPE_SCALING_NONE) {
    return NQ_ERR_INVALID_ARG;
  }
  if (c->packing != NQ_PACKING_STANDARD && c->packing != NQ_PACKING_COMPACT)
    return NQ_ERR_INVALID_ARG;
  if (c->packing == NQ_PACKING_COMPACT && c->parity != NQ_PARITY_STRICT)
    return NQ_ERR_INVALID_ARG;
  if (c->exact != 0 && c->exact != 1) return NQ_ERR_INVALID_ARG;
  if (c->rope_scaling == NQ_ROPE_SCALING_LLAMA3) {
    if (!(c->rope_low_freq_factor > 0.0) || !isfinite(c->rope_high_freq_factor) ||
        !(c->rope_high_freq_factor > c->rope_low_freq_factor) || c->rope_original_max <= 0)
      return NQ_ERR_INVALID_ARG;
  }
  const int n = next_pow2_min8(d);
  const int G = c->scale_group == 0 ? n : c->scale_group;
  if (G < 8 || G > n || (G % 8) != 0 || (n % G) != 0) return NQ_ERR_UNSUPPORTED;
  return NQ_OK;
}

Layout layout(const nq_config* c, int is_value) {
  Layout l;
  l.d = c->head_dim;
  l.n = next_pow2_min8(l.d);
  l.G = c->scale_group == 0 ? l.n : c->scale_group;
  l.bits = is_value ? c->bits_v : c->bits_k;
  l.L = 1 << l.bits;
  l.code_bytes = l.n * l.bits / 8;
  l.compact = c->packing == NQ_PACKING_COMPACT ? 1 : 0;
  l.coset_bytes = l.compact ? 0 : (l.n / 8 + 7) / 8;
  l.n_scales = l.n / l.G;
  return l;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace of a call on S x H x T vectors, in this order (each part
// 256-byte aligned): the fp32 RoPE table [T][d/2] (cos, sin) -- the only part
// dequantize uses --, the fp64 RoPE frequencies [d/2], two queue counters
// (keys, values) and the key and value queues of the fp64 pass.
struct WsLayout {
  size_t rope32, omega, counters, queue_k, queue_v, total;
  int64_t queue_cap;
};

int64_t queue_capacity(int64_t n_vec) {
  // ~1e-3 of random vectors have a near-tie group; a queue of 1/32 of the
  // vectors (at least 1024) leaves a wide margin, and a full queue makes the
  // fp64 pass recompute every vector instead
  int64_t cap = n_vec / 32;
  if (cap < 1024) cap = 1024;
  if (cap > n_vec) cap = n_vec;
  return cap;
}

WsLayout ws_layout(const nq_config* c, int64_t S, int64_t H, int64_t T) {
  WsLayout w;
  const bool rope = c->rope_theta > 0.0;
  const size_t th = (size_t)T * (size_t)(c->head_dim / 2);
  w.rope32 = 0;
  w.omega = round256(rope ? th * sizeof(float2) : 0);
  w.counters = w.omega + round256(rope ? (size_t)(c->head_dim / 2) * sizeof(double) : 0);
  w.queue_k = w.counters + 256;
  w.queue_cap = queue_capacity(S * H * T);
  const size_t qb = round256((size_t)w.queue_cap * sizeof(int64_t));
  w.queue_v = w.queue_k + qb;
  w.total = w.queue_v + qb;
  return w;
}

size_t rope_bytes(const nq_config* c, int64_t T) {
  if (c->rope_theta <= 0.0) return 0;
  return round256((size_t)T * (size_t)(c->head_dim / 2) * sizeof(float2));
}

constexpr int64_t kMaxTokens = (int64_t)1 << 40;

// Pointers, alignment and the token window [token_offset, token_offset + T)
// of a call inside planes of token_capacity tokens per (slab, head).
int check_packed(const nq_packed* p, int64_t T, const nq_config* c) {
  const bool need_cosets = c->packing != NQ_PACKING_COMPACT;
  if (p == nullptr || p->codes == nullptr || (need_cosets && p->cosets == nullptr) ||
      p->scales == nullptr)
    return NQ_ERR_INVALID_ARG;
  if (!aligned16(p->codes) || !aligned16(p->cosets) || !aligned16(p->scales))
    return NQ_ERR_INVALID_ARG;
  if (p->token_offset < 0 || p->token_offset > kMaxTokens || p->token_capacity < 0 ||
      p->token_capacity > kMaxTokens)
    return NQ_ERR_INVALID_ARG;
  if (p->token_capacity != 0 && p->token_offset + T > p->token_capacity)
    return NQ_ERR_INVALID_ARG;
  return NQ_OK;
}

// The call's window: plane token stride and plane bases advanced to the
// window's first token (the same shift as starting at a later vector, so the
// kernels' alignment assumptions still hold).
struct PackedView {
  uint8_t* codes;
  uint8_t* cosets;
  uint16_t* scales;
  int64_t pT, t0;
};

PackedView packed_view(const nq_packed* p, const Layout& l, int64_t T) {
  PackedView v;
  v.t0 = p->token_offset;
  v.pT = p->token_capacity != 0 ? p->token_capacity : p->token_offset + T;
  v.codes = static_cast<uint8_t*>(p->codes) + v.t0 * l.code_bytes;
  v.cosets = static_cast<uint8_t*>(p->cosets) + v.t0 * l.coset_bytes;
  v.scales = static_cast<uint16_t*>(p->scales) + v.t0 * l.n_scales;
  return v;
}

int check_shape(int64_t S, int32_t H, int64_t T) {
  if (S <= 0 || H <= 0 || T <= 0) return NQ_ERR_INVALID_ARG;
  // vector counts must fit the 1-D launch grids (2^31 - 1 blocks of >= 8)
  if ((double)S * (double)H * (double)T > 8.0e9) return NQ_ERR_UNSUPPORTED;
  return NQ_OK;
}

nq::TensorArgs tensor_args(const nq_config* c, const Layout& l, int64_t S,
                           int32_t H, int64_t T, const nq_packed* p) {
  nq::TensorArgs a;
  memset(&a, 0, sizeof(a));
  const PackedView pv = packed_view(p, l, T);
  a.codes = pv.codes;
  a.cosets = pv.cosets;
  a.scales = pv.scales;
  a.n_vec = S * (int64_t)H * T;
  a.T = T;
  a.pT = pv.pT;
  a.d = l.d;
  a.n = l.n;
  a.G = l.G;
  a.bits = l.bits;
  a.strict = c->parity == NQ_PARITY_STRICT ? 1 : 0;
  a.compact = l.compact;
  a.code_bytes = l.code_bytes;
  a.coset_bytes = l.coset_bytes;
  a.n_scales = l.n_scales;
  a.eps = (float)(1e-8 * sqrt((double)l.n));
  a.half_L = (float)(l.L / 2);
  a.sigma_k = 1.0 / ((l.L / 2.0) * sqrt((double)l.n));
  a.inv_sqrt_n = (float)(1.0 / sqrt((double)l.n));
  a.eps64 = 1e-8 * sqrt((double)l.n);
  a.half_L64 = l.L / 2.0;
  return a;
}

// Frequency i of the rotary embedding, with the config's frequency scaling
// (the formulas of nq_config, in fp64, in the order written there).
double rope_freq(const nq_config* c, int i) {
  const int d = c->head_dim;
  const double w = pow(c->rope_theta, -(2.0 * i) / d);
  if (c->rope_scaling == NQ_ROPE_SCALING_LINEAR) return w / c->rope_factor;
  if (c->rope_scaling != NQ_ROPE_SCALING_LLAMA3) return w;
  const double C = (double)c->rope_original_max;
  const double lo = c->rope_low_freq_factor, hi = c->rope_high_freq_factor;
  const double wavelen = 2.0 * M_PI / w;
  if (wavelen < C / hi) return w;
  if (wavelen > C / lo) return w / c->rope_factor;
  const double a = (C / wavelen - lo) / (hi - lo);
  return (1.0 - a) * w / c->rope_factor + a * w;
}

// Builds the fp32 cos/sin table at the start of the workspace when keys need
// RoPE; in the same launch copies the fp64 frequencies to `omega` and clears
// the n_counters queue counters at `counters` (each when not null).
void rope_freqs(const nq_config* c, nq::RopeFreqs* f) {
  for (int i = 0; i < c->head_dim / 2; ++i) {
    f->omega[i] = rope_freq(c, i);
    f->step_c[i] = (float)cos(16.0 * f->omega[i]);
    f->step_s[i] = (float)sin(16.0 * f->omega[i]);
  }
}

int prepare_rope(const nq_config* c, int64_t T, const int32_t* positions, int64_t pos0,
                 void* ws, double* omega, unsigned long long* counters, int n_counters,
                 hipStream_t s, const float2** out) {
  *out = nullptr;
  nq::RopeFreqs f;
  const int d = c->head_dim;
  rope_freqs(c, &f);
  float2* table = static_cast<float2*>(ws);
  if (nq::launch_rope_table(positions, pos0, T, d, f, table, omega, counters, n_counters, s) !=
      hipSuccess)
    return NQ_ERR_HIP;
  *out = table;
  return NQ_OK;
}

}  // namespace

namespace nq {

// nq_quantize_kv with the workspace supplied by the entry point.
int quantize_impl(const nq_config* cfg, const void* k, const void* v, int64_t S, int32_t H,
                  int64_t T, const int32_t* positions, const nq_packed* pk, const nq_packed* pv,
                  void* ws, size_t ws_bytes, void* stream) {
  int st = check_config(cfg);
  if (st != NQ_OK) return st;
  if ((st = check_shape(S, H, T)) != NQ_OK) return st;
  if (k == nullptr && v == nullptr) return NQ_ERR_INVALID_ARG;
  if (k != nullptr && (!aligned16(k) || (st = check_packed(pk, T, cfg)) != NQ_OK))
    return st != NQ_OK ? st : NQ_ERR_INVALID_ARG;
  if (v != nullptr && (!aligned16(v) || (st = check_packed(pv, T, cfg)) != NQ_OK))
    return st != NQ_OK ? st : NQ_ERR_INVALID_ARG;
  if (positions != nullptr && !aligned16(positions)) return NQ_ERR_INVALID_ARG;
  const WsLayout w = ws_layout(cfg, S, H, T);
  if (ws == nullptr || ws_bytes < w.total) return NQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return NQ_ERR_INVALID_ARG;
  char* wb = static_cast<char*>(ws);
  auto* counters = reinterpret_cast<unsigned long long*>(wb + w.counters);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float2* rope = nullptr;
  double* omega = nullptr;
  if (k != nullptr && cfg->rope_theta > 0.0) {
    omega = reinterpret_cast<double*>(wb + w.omega);
    if ((st = prepare_rope(cfg, T, positions, pk->token_offset, ws, omega, counters, 2, s,
                           &rope)) != NQ_OK)
      return st;
  } else if (nq::launch_clear_counters(counters, 2, s) != hipSuccess) {
    return NQ_ERR_HIP;
  }
  // each tensor's fp32 kernel (which queues near-tie vectors), then the fp64
  // pass over the queues, one launch for both tensors when they share bits;
  // with cfg->exact every vector takes the fp64 pass
  nq::TensorArgs args[2];
  for (int is_v = 0; is_v < 2; ++is_v) {
    const void* x = is_v ? v : k;
    if (x == nullptr) continue;
    nq::TensorArgs& a = args[is_v];
    a = tensor_args(cfg, layout(cfg, is_v), S, H, T, is_v ? pv : pk);
    a.x = x;
    a.rope = is_v ? nullptr : rope;
    a.omega = is_v ? nullptr : omega;
    a.positions = positions;
    a.pos0 = (is_v ? pv : pk)->token_offset;
    a.queue_count = counters + is_v;
    a.queue = reinterpret_cast<int64_t*>(wb + (is_v ? w.queue_v : w.queue_k));
    a.queue_cap = w.queue_cap;
    if (!cfg->exact && nq::launch_quantize(a, cfg->in_dtype, s) != hipSuccess) return NQ_ERR_HIP;
  }
  if (k != nullptr && v != nullptr && args[0].bits == args[1].bits) {
    if (nq::launch_exact2(args[0], args[1], cfg->in_dtype, cfg->exact, s) != hipSuccess)
      return NQ_ERR_HIP;
  } else {
    for (int is_v = 0; is_v < 2; ++is_v) {
      if ((is_v ? v : k) == nullptr) continue;
      if (nq::launch_exact(args[is_v], cfg->in_dtype, cfg->exact, s) != hipSuccess)
        return NQ_ERR_HIP;
    }
  }
  return NQ_OK;
}

}  // namespace nq

extern "C" {

size_t nq_packed_bytes(const nq_config* cfg, int is_value, int64_t n_vectors,
                       int plane) {
  if (check_config(cfg) != NQ_OK || n_vectors < 0) return 0;
  const Layout l = layout(cfg, is_value);
  switch (plane) {
    case NQ_PLANE_CODES: return (size_t)n_vectors * l.code_bytes;
    case NQ_PLANE_COSETS: return (size_t)n_vectors * l.coset_bytes;
    case NQ_PLANE_SCALES: return (size_t)n_vectors * l.n_scales * 2;
    default: return 0;
  }
}

size_t nq_workspace_bytes(const nq_config* cfg, int64_t n_slabs, int32_t n_kv_heads,
                          int64_t n_tokens) {
  if (check_config(cfg) != NQ_OK || check_shape(n_slabs, n_kv_heads, n_tokens) != NQ_OK) return 0;
  return ws_layout(cfg, n_slabs, n_kv_heads, n_tokens).total;
}

const char* nq_status_string(int status) {
  switch (status) {
    case NQ_OK: return "ok";
    case NQ_ERR_INVALID_ARG: return "invalid argument";
    case NQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case NQ_ERR_WORKSPACE: return "workspace missing or too small";
    case NQ_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int nq_quantize_kv(const nq_config* cfg, const void* k, const void* v,
                   int64_t S, int32_t H, int64_t T, const int32_t* positions,
                   const nq_packed* pk, const nq_packed* pv, void* ws,
                   size_t ws_bytes, void* stream) {
  return nq::quantize_impl(cfg, k, v, S, H, T, positions, pk, pv, ws, ws_bytes, stream);
}

int nq_dequantize_kv(const nq_config* cfg, const nq_packed* pk,
                     const nq_packed* pv, int64_t S, int32_t H, int64_t T,
                     const int32_t* positions, void* k_out, void* v_out,
                     void* ws, size_t ws_bytes, void* stream) {
  int st = check_config(cfg);
  if (st != NQ_OK) return st;
  if ((st = check_shape(S, H, T)) != NQ_OK) return st;
  if (k_out == nullptr && v_out == nullptr) return NQ_ERR_INVALID_ARG;
  if (k_out != nullptr && (!aligned16(k_out) || (st = check_packed(pk, T, cfg)) != NQ_OK))
    return st != NQ_OK ? st : NQ_ERR_INVALID_ARG;
  if (v_out != nullptr && (!aligned16(v_out) || (st = check_packed(pv, T, cfg)) != NQ_OK))
    return st != NQ_OK ? st : NQ_ERR_INVALID_ARG;
  if (positions != nullptr && !aligned16(positions)) return NQ_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (k_out != nullptr) {
    nq::TensorArgs a = tensor_args(cfg, layout(cfg, 0), S, H, T, pk);
    a.y = k_out;
    nq::RopeFreqs f;
    const bool rope = rope_bytes(cfg, T) != 0;
    if (rope) {
      if (ws == nullptr || ws_bytes < rope_bytes(cfg, T)) return NQ_ERR_WORKSPACE;
      if (!aligned16(ws)) return NQ_ERR_INVALID_ARG;
      rope_freqs(cfg, &f);
      a.positions = positions;
      a.pos0 = pk->token_offset;
      // the matrix-core kernel forms its own cos / sin rows; the others
      // read the table
      if (!nq::dequantize_forms_rope_rows(a, cfg->in_dtype)) {
        const float2* table = nullptr;
        if ((st = prepare_rope(cfg, T, positions, pk->token_offset, ws, nullptr, nullptr, 0, s,
                               &table)) != NQ_OK)
          return st;
        a.rope = table;
      }
    }
    if (nq::launch_dequantize(a, cfg->in_dtype, rope ? &f : nullptr, s) != hipSuccess)
      return NQ_ERR_HIP;
  }
  if (v_out != nullptr) {
    nq::TensorArgs a = tensor_args(cfg, layout(cfg, 1), S, H, T, pv);
    a.y = v_out;
    if (nq::launch_dequantize(a, cfg->in_dtype, nullptr, s) != hipSuccess) return NQ_ERR_HIP;
  }
  return NQ_OK;
}

int nq_score_packed_keys(const nq_config* cfg, const nq_packed* pk, int64_t S,
                         int32_t H, int32_t Hq, int64_t T, const void* q,
                         float* scores, void* ws, size_t ws_bytes,
                         void* stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_config(cfg);
  if (st != NQ_OK) return st;
  if ((st = check_shape(S, H, T)) != NQ_OK) return st;
  if (Hq <= 0 || Hq % H != 0) return NQ_ERR_INVALID_ARG;
  if (S > 65535 || H > 65535) return NQ_ERR_UNSUPPORTED;
  if ((st = check_packed(pk, T, cfg)) != NQ_OK) return st;
  if (q == nullptr || scores == nullptr || !aligned16(q) || !aligned16(scores))
    return NQ_ERR_INVALID_ARG;
  const Layout l = layout(cfg, 0);
  if ((size_t)(Hq / H) * l.n * sizeof(float) > 64 * 1024) return NQ_ERR_UNSUPPORTED;
  nq::ScoreArgs a;
  memset(&a, 0, sizeof(a));
  const PackedView pv = packed_view(pk, l, T);
  a.codes = pv.codes;
  a.cosets = pv.cosets;
  a.scales = pv.scales;
  a.q = q;
  a.out = scores;
  a.S = S;
  a.T = T;
  a.pT = pv.pT;
  a.H = H;
  a.Hq = Hq;
  a.d = l.d;
  a.n = l.n;
  a.G = l.G;
  a.bits = l.bits;
  a.code_bytes = l.code_bytes;
  a.coset_bytes = l.coset_bytes;
  a.n_scales = l.n_scales;
  a.compact = l.compact;
  a.half_L = (float)(l.L / 2);
  a.inv_sqrt_n = (float)(1.0 / sqrt((double)l.n));
  if (nq::launch_score(a, cfg->in_dtype, static_cast<hipStream_t>(stream)) != hipSuccess)
    return NQ_ERR_HIP;
  return NQ_OK;
}

int nq_attend_packed_values(const nq_config* cfg, const nq_packed* pv,
                            int64_t S, int32_t H, int32_t Hq, int64_t T,
                            const float* weights, float* out, void* stream) {
  int st = check_config(cfg);
  if (st != NQ_OK) return st;
  if ((st = check_shape(S, H, T)) != NQ_OK) return st;
  if (Hq <= 0 || Hq % H != 0) return NQ_ERR_INVALID_ARG;
  if (S > 65535 || (int64_t)H * ((Hq / H + 3) / 4 + 1) > 65535) return NQ_ERR_UNSUPPORTED;
  if ((st = check_packed(pv, T, cfg)) != NQ_OK) return st;
  if (weights == nullptr || out == nullptr || !aligned16(weights) || !aligned16(out))
    return NQ_ERR_INVALID_ARG;
  const Layout l = layout(cfg, 1);
  nq::AttendArgs a;
  memset(&a, 0, sizeof(a));
  const PackedView view = packed_view(pv, l, T);
  a.codes = view.codes;
  a.cosets = view.cosets;
  a.scales = view.scales;
  a.w = weights;
  a.out = out;
  a.S = S;
  a.T = T;
  a.pT = view.pT;
  a.H = H;
  a.Hq = Hq;
  a.d = l.d;
  a.n = l.n;
  a.G = l.G;
  a.bits = l.bits;
  a.code_bytes = l.code_bytes;
  a.coset_bytes = l.coset_bytes;
  a.n_scales = l.n_scales;
  a.compact = l.compact;
  a.half_L = (float)(l.L / 2);
  a.inv_sqrt_n = (float)(1.0 / sqrt((double)l.n));
  if (nq::launch_attend(a, static_cast<hipStream_t>(stream)) != hipSuccess) return NQ_ERR_HIP;
  return NQ_OK;
}

int nq_e8_decode_debug(const float* y, int64_t n_groups, int32_t bits,
                       int32_t parity, int32_t constrained, uint8_t* idx_out,
                       uint8_t* coset_out, void* stream) {
  if (y == nullptr || idx_out == nullptr || coset_out == nullptr || n_groups <= 0)
    return NQ_ERR_INVALID_ARG;
  if (!(bits == 2 || bits == 3)) return NQ_ERR_UNSUPPORTED;
  if (parity != NQ_PARITY_STRICT && parity != NQ_PARITY_RELAXED)
    return NQ_ERR_INVALID_ARG;
  if (constrained != 0 && constrained != 1) return NQ_ERR_INVALID_ARG;
  if (n_groups > ((int64_t)1 << 38)) return NQ_ERR_UNSUPPORTED;
  if (nq::launch_decode_debug(y, n_groups, bits, parity == NQ_PARITY_STRICT,
                              constrained, idx_out, coset_out,
                              static_cast<hipStream_t>(stream)) != hipSuccess)
    return NQ_ERR_HIP;
  return NQ_OK;
}

}  // extern "C"
