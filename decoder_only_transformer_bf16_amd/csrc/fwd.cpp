// C-ABI implementation of libfwd.so: configuration checks, weight packing into
// library-owned HBM, workspace, and the launch sequence of the prefill forward.
// See include/fwd.h for the contract of every entry point.
#include "fwd.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using fwdk::DType;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define TIMED(model, kind, expr)              \
  do {                                        \
    if (int rc_ = (model)->tick(kind)) return rc_; \
    HIP_TRY(expr);                            \
    if (int rc_ = (model)->tock()) return rc_; \
  } while (0)

#define HIP_TRY(expr)                                                                              \
  do {                                                                                             \
    hipError_t e_ = (expr);                                                                        \
    if (e_ != hipSuccess) return fail(FWD_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// sqrt(hidden) rounded to 8 significant bits, ties to even ("pegainfer issue #878":
// the embedding scale is the bf16-rounded value).
float bf16_sqrt(int hidden) {
  const double r = std::sqrt((double)hidden);
  int e = 0;
  const double m = std::frexp(r, &e);                    // r = m * 2^e, m in [0.5, 1)
  const double q = std::nearbyint(std::ldexp(m, 8));    // default rounding: nearest, ties to even
  return (float)std::ldexp(q, e - 8);
}

int check_config(const fwd_config* c) {
  if (!c) return fail(FWD_E_ARG, "config is NULL");
  if (c->n_layers < 0 || c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->ffn <= 0 || c->vocab <= 0)
    return fail(FWD_E_CONFIG, "geometry fields must be positive (n_layers >= 0)");
  if (c->n_heads % c->n_kv_heads) return fail(FWD_E_CONFIG, "n_heads must be a multiple of n_kv_heads");
  if (c->dtype != FWD_DTYPE_BF16 && c->dtype != FWD_DTYPE_F32) return fail(FWD_E_CONFIG, "dtype");
  const DType dt = DType(c->dtype);
  if (!fwdk::attention_supported(dt, c->head_dim))
    return fail(FWD_E_CONFIG, dt == DType::BF16 ? "bf16 head_dim must be 64, 128 or 256"
                                                : "f32 head_dim must be 16, 32 or 64");
  const int vec = dt == DType::BF16 ? 8 : 4;
  if (c->hidden % vec || c->ffn % vec || (c->n_heads * c->head_dim) % vec)
    return fail(FWD_E_CONFIG, "hidden, ffn and n_heads*head_dim must be multiples of 8 (bf16) / 4 (f32)");
  if (dt == DType::BF16 && (c->hidden % 32 || c->ffn % 32 || (c->n_heads * c->head_dim) % 32 ||
                            (c->n_kv_heads * c->head_dim) % 32))
    return fail(FWD_E_CONFIG, "bf16 needs hidden, ffn and head widths that are multiples of 32");
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps)) return fail(FWD_E_CONFIG, "rms_eps must be positive");
  if (!(c->rope_theta > 1.0) || !std::isfinite(c->rope_theta)) return fail(FWD_E_CONFIG, "rope_theta must be > 1");
  if (std::isnan(c->final_logit_softcap) || c->final_logit_softcap < 0.f || std::isinf(c->final_logit_softcap))
    return fail(FWD_E_CONFIG, "final_logit_softcap must be positive, or 0 for off");
  if (c->embed_scale_mode != FWD_EMBED_SCALE_NONE && c->embed_scale_mode != FWD_EMBED_SCALE_BF16_SQRT_HIDDEN)
    return fail(FWD_E_CONFIG, "embed_scale_mode");
  if (c->norm_placement != FWD_NORM_PRE && c->norm_placement != FWD_NORM_SANDWICH)
    return fail(FWD_E_CONFIG, "norm_placement");
  if (c->sliding_window < 0) return fail(FWD_E_CONFIG, "sliding_window must be >= 0");
  if (c->layer_kind)
    for (int l = 0; l < c->n_layers; ++l)
      if (c->layer_kind[l] != FWD_LAYER_GLOBAL && c->layer_kind[l] != FWD_LAYER_LOCAL)
        return fail(FWD_E_CONFIG, "layer_kind entries must be FWD_LAYER_GLOBAL or FWD_LAYER_LOCAL");
  if (c->max_tokens <= 0) return fail(FWD_E_CONFIG, "max_tokens must be positive");
  if ((c->qk_norm != 0 && c->qk_norm != 1) || (c->norm_gain_offset != 0 && c->norm_gain_offset != 1))
    return fail(FWD_E_CONFIG, "qk_norm and norm_gain_offset must be 0 or 1");
  if (c->ffn_act != FWD_FFN_SILU && c->ffn_act != FWD_FFN_GELU_TANH) return fail(FWD_E_CONFIG, "ffn_act");
  if (c->rope_theta_local != 0.0 && (!(c->rope_theta_local > 1.0) || !std::isfinite(c->rope_theta_local)))
    return fail(FWD_E_CONFIG, "rope_theta_local must be > 1, or 0 for rope_theta");
  if (c->n_experts < 0 || (c->n_experts == 0 && c->ffn_kind))
    for (int l = 0; c->ffn_kind && l < c->n_layers; ++l)
      if (c->ffn_kind[l] != FWD_FFN_DENSE) return fail(FWD_E_CONFIG, "ffn_kind names MoE layers but n_experts is 0");
  if (c->n_experts < 0) return fail(FWD_E_CONFIG, "n_experts must be >= 0");
  if (c->n_experts > 0) {
    if (c->dtype != FWD_DTYPE_BF16) return fail(FWD_E_CONFIG, "mixture of experts needs dtype bf16");
    if (c->n_experts > fwdk::kMoeMaxExperts) return fail(FWD_E_CONFIG, "n_experts must be at most 256");
    if (c->n_experts_per_tok < 1 || c->n_experts_per_tok > std::min(fwdk::kMoeMaxTopK, (int)c->n_experts))
      return fail(FWD_E_CONFIG, "n_experts_per_tok must be in 1 .. min(8, n_experts)");
    if (c->moe_ffn <= 0 || c->moe_ffn % 32) return fail(FWD_E_CONFIG, "moe_ffn must be a positive multiple of 32");
    if (c->moe_norm_topk != 0 && c->moe_norm_topk != 1) return fail(FWD_E_CONFIG, "moe_norm_topk must be 0 or 1");
    for (int l = 0; c->ffn_kind && l < c->n_layers; ++l)
      if (c->ffn_kind[l] != FWD_FFN_DENSE && c->ffn_kind[l] != FWD_FFN_MOE)
        return fail(FWD_E_CONFIG, "ffn_kind entries must be FWD_FFN_DENSE or FWD_FFN_MOE");
  }
  if (c->rope_scaling != FWD_ROPE_NONE) {
    if (c->rope_scaling != FWD_ROPE_LLAMA3 && c->rope_scaling != FWD_ROPE_LONGROPE)
      return fail(FWD_E_CONFIG, "rope_scaling");
    if (!(c->rope_factor > 0.f) || !std::isfinite(c->rope_factor) || c->rope_original_max_pos <= 0)
      return fail(FWD_E_CONFIG, "rope scaling needs rope_factor > 0 and rope_original_max_pos > 0");
    if (c->rope_scaling == FWD_ROPE_LLAMA3 &&
        !(c->rope_low_freq_factor > 0.f && c->rope_high_freq_factor > c->rope_low_freq_factor &&
          std::isfinite(c->rope_high_freq_factor)))
      return fail(FWD_E_CONFIG, "llama3 rope scaling needs 0 < rope_low_freq_factor < rope_high_freq_factor");
    if (c->rope_scaling == FWD_ROPE_LONGROPE) {
      if (!c->rope_short_factor || !c->rope_long_factor)
        return fail(FWD_E_CONFIG, "longrope needs rope_short_factor and rope_long_factor");
      for (int k = 0; k < c->head_dim / 2; ++k)
        if (!(c->rope_short_factor[k] > 0.f) || !(c->rope_long_factor[k] > 0.f) ||
            !std::isfinite(c->rope_short_factor[k]) || !std::isfinite(c->rope_long_factor[k]))
          return fail(FWD_E_CONFIG, "longrope factors must be positive and finite");
    }
  }
  return FWD_OK;
}

// bf16 GEMM operands (weights, normalised activations, attention and SwiGLU
// outputs) are kept K-tiled (16 x 32 tiles, rows padded to 16); f32 is row-major.
// (value, column) pairs the sliced argmax of a small batch may use (rows x slices <= 2 x 256)
constexpr int64_t kArgPartPairs = 1024;

struct Geometry {
  int64_t esize, H, Hq, Hkv, D, F, V, L, T, qkv_rows, logit_chunk, rope_tables;
  int64_t E = 0, topk = 0, Fe = 0, moe_layers = 0;  // mixture of experts
  int64_t moe_rows() const { return round_up(T * topk + 16 * E, 16); }  // permuted rows (16-aligned segments)
  int64_t moe_tiles() const { return (T * topk + fwdk::kMoeTileRows - 1) / fwdk::kMoeTileRows + E; }
  bool tiled;
  int64_t rows(int64_t r) const { return tiled ? round_up(r, 16) : r; }  // allocated rows of an operand
  int64_t weight_bytes() const {
    const int64_t per_layer =
        (rows(qkv_rows) * H + rows(H) * Hq * D + rows(2 * F) * H + rows(H) * F) * esize + 4 * H * 4;
    const int64_t moe_delta = moe_layers * ((rows(E) * H + E * (rows(2 * Fe) * H + rows(H) * Fe) -
                                             (rows(2 * F) * H + rows(H) * F)) * esize);
    return rows(V) * H * esize + H * 4 + L * per_layer + moe_delta;
  }
  // Logit chunk (few rows, fp32) or the fused head's argmax keys (8 bytes each).
  int64_t logit_ws_bytes() const {
    return std::max<int64_t>(logit_chunk * V * 4, fwdk::head_argmax_part_keys((int)T, (int)V) * 8);
  }
  // Workspace (bytes, each buffer rounded to 256) for up to T tokens.
  int64_t workspace_bytes(bool sandwich) const {
    auto r = [](int64_t b) { return round_up(b, 256); };
    int64_t w = 2 * r(T * H * 4);                       // residual stream, mid-layer copy
    w += r(rows(T) * H * esize);                        // normalised activations
    w += r(T * (Hq + 2 * Hkv) * D * esize);             // rotated q | rotated k | v
    w += r(8 * T * Hkv * D * esize);                    // transposed v, padded keys
    w += r(rows(T) * Hq * D * esize);                   // attention output
    w += r(rows(T) * F * esize);                        // SwiGLU output
    if (sandwich) w += r(T * H * 4);                    // sublayer output before its norm
    if (sandwich && tiled) w += r(dense_split_floats() * 4);  // split-K partials of its products
    w += r(T * 4) + r(T * 4) + 256;                     // ids, argmax, flag
    w += r(logit_ws_bytes());                           // logits when the caller wants none / argmax keys
    w += r(kArgPartPairs * 8);                          // sliced argmax partials
    w += rope_tables * r(T * (D / 2) * 8);              // RoPE cos/sin tables
    if (tiled) w += r(skinny_part_floats() * 4) + r(skinny_counters() * 4) + r(fwdk::skinny_groups((int)H) * 64 * 4);
    if (E > 0) {
      const int64_t A = T * topk, nch = fwdk::moe_chunks(A);
      w += r(T * E * 4) + 3 * r(A * 4) + 2 * r(nch * E * 4) + 4 * r((E + 1) * 4);
      w += r(moe_rows() * H * esize) + r(moe_rows() * Fe * esize) + r(moe_rows() * H * 4);
    }
    return w;
  }
  // Split-K workspace of the few-row products (bf16, at most kSkinnyRows rows):
  // the largest partial set over the five projections, one counter per 64 outputs.
  int64_t skinny_part_floats() const {
    const int Mk = (int)std::min<int64_t>(T, fwdk::kSkinnyRows);
    const int64_t nk[5][2] = {{qkv_rows, H}, {H, Hq * D}, {2 * F, H}, {H, F}, {V, H}};
    int64_t f = 0;
    for (const auto& p : nk) f = std::max(f, fwdk::skinny_part_floats(Mk, (int)p[0], (int)p[1]));
    return f;
  }
  int64_t skinny_counters() const { return fwdk::skinny_groups((int)std::max({qkv_rows, H, 2 * F, V})); }
  // Split-K partials of the sandwich products (O and down, whose outputs are stored
  // before their norm): the largest need over every row count up to T. It depends on
  // the rows only through their 128-row tile count, so the last row count of each
  // tile count bounds it.
  int64_t dense_split_floats() const {
    int64_t f = 0;
    for (int64_t c = 1; c <= (T + 127) / 128; ++c) {
      const int M = (int)std::min(128 * c, T);
      f = std::max({f, fwdk::dense_split_floats(M, (int)H, (int)(Hq * D), true),
                    fwdk::dense_split_floats(M, (int)H, (int)F, true)});
    }
    return f;
  }
};

Geometry geometry(const fwd_config* c) {
  Geometry g;
  g.esize = c->dtype == FWD_DTYPE_BF16 ? 2 : 4;
  g.H = c->hidden;
  g.Hq = c->n_heads;
  g.Hkv = c->n_kv_heads;
  g.D = c->head_dim;
  g.F = c->ffn;
  g.V = c->vocab;
  g.L = c->n_layers;
  g.T = c->max_tokens;
  g.qkv_rows = (g.Hq + 2 * g.Hkv) * g.D;
  g.logit_chunk = std::min<int64_t>(g.T, 1024);  // a multiple of 16 whenever it splits T
  g.tiled = c->dtype == FWD_DTYPE_BF16;
  bool any_local = false;
  for (int l = 0; c->layer_kind && l < c->n_layers; ++l) any_local |= c->layer_kind[l] == FWD_LAYER_LOCAL;
  g.rope_tables = (any_local && c->rope_theta_local > 0.0 && c->rope_theta_local != c->rope_theta ? 2 : 1) *
                  (c->rope_scaling == FWD_ROPE_LONGROPE ? 2 : 1);
  if (c->n_experts > 0) {
    g.E = c->n_experts;
    g.topk = c->n_experts_per_tok;
    g.Fe = c->moe_ffn;
    for (int l = 0; l < c->n_layers; ++l) g.moe_layers += !c->ffn_kind || c->ffn_kind[l] == FWD_FFN_MOE;
  }
  return g;
}

}  // namespace

struct fwd_model {
  fwd_config cfg{};
  std::vector<int32_t> kinds;
  DType dt = DType::BF16;
  Geometry g{};
  hipStream_t stream = nullptr;
  float embed_scale = 1.f;
  std::vector<void*> allocs;

  void* embed = nullptr;
  float* final_norm = nullptr;
  struct Layer {
    float *attn_norm, *ffn_norm, *post_attn, *post_ffn, *q_norm, *k_norm;
    void *wqkv, *wo, *wgu, *wdown;  // MoE layers: wgu / wdown are the experts' stacks
    void* router;                   // MoE layers: [E, H]
    bool moe;
  };
  std::vector<Layer> layers;

  float* x = nullptr;   // residual stream (updated in place when no hidden slots are requested)
  float* xb = nullptr;  // mid-layer residual when slots are requested
  void* n = nullptr;
  void* qk = nullptr;
  void* vt = nullptr;
  void* o = nullptr;
  void* a = nullptr;
  float* u = nullptr;
  int32_t* ids = nullptr;
  int32_t* amax = nullptr;
  int* flag = nullptr;
  float* logits_ws = nullptr;
  float* argpart = nullptr;  // partial (value, column) pairs of the sliced argmax for few rows
  float2* rope_tab[4] = {};  // [2 * local + long factors]: RoPE (cos, sin) tables of max_tokens rows
  std::vector<float> rope_short, rope_long;  // longrope factors (the config's arrays are borrowed)
  fwdk::SplitK sk{};  // workspace of the few-row products (bf16)
  fwdk::DenseSplit ds{};  // split-K partials of the sandwich products (bf16)
  // mixture-of-experts workspace (models with MoE layers)
  float* moe_logits = nullptr;  // [T, E]
  int32_t* moe_idx = nullptr;   // [T, k]
  float* moe_w = nullptr;       // [T, k]
  fwdk::MoePlan plan{};
  void* moe_x = nullptr;        // [moe_rows, H] bf16 K-tiled: token rows in expert order
  void* moe_a = nullptr;        // [moe_rows, Fe] bf16 K-tiled: gated FFN activations
  float* moe_y = nullptr;       // [moe_rows, H] fp32: expert outputs
  float* ssq = nullptr;  // [H / 64][kSkinnyRows] row sums of squares left by a few-row residual product

  // per-kernel-class event timing (fwd_set_timing)
  bool timing = false;
  std::vector<hipEvent_t> events;
  size_t events_used = 0;
  std::vector<int> marks;  // kernel class of each (start, stop) event pair
  double class_ms[FWD_KERNEL_CLASSES] = {};
  int64_t class_n[FWD_KERNEL_CLASSES] = {};

  // Record the start event of a launch of `kind` (no-op when timing is off).
  int tick(int kind) {
    if (!timing) return FWD_OK;
    if (events_used + 2 > events.size()) {
      for (int i = 0; i < 2; ++i) {
        hipEvent_t e;
        HIP_TRY(hipEventCreate(&e));
        events.push_back(e);
      }
    }
    marks.push_back(kind);
    HIP_TRY(hipEventRecord(events[events_used], stream));
    return FWD_OK;
  }
  int tock() {
    if (!timing) return FWD_OK;
    HIP_TRY(hipEventRecord(events[events_used + 1], stream));
    events_used += 2;
    return FWD_OK;
  }
  // After the stream is synchronised: fold the recorded pairs into the totals.
  int collect() {
    if (!timing) return FWD_OK;
    for (size_t i = 0; i < marks.size(); ++i) {
      float ms = 0.f;
      HIP_TRY(hipEventElapsedTime(&ms, events[2 * i], events[2 * i + 1]));
      class_ms[marks[i]] += ms;
      class_n[marks[i]] += 1;
    }
    marks.clear();
    events_used = 0;
    return FWD_OK;
  }

  int alloc(void** p, int64_t bytes) {
    *p = nullptr;
    if (bytes <= 0) return FWD_OK;
    HIP_TRY(hipMalloc(p, (size_t)round_up(bytes, 256)));
    allocs.push_back(*p);
    return FWD_OK;
  }
  ~fwd_model() {
    if (stream) (void)hipStreamSynchronize(stream);
    else (void)hipDeviceSynchronize();
    for (void* p : allocs) (void)hipFree(p);
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
  }
};

// KV-cache session: per-layer K and V caches [Bmax, Hkv, Smax, D] and the chunk
// partials of the decode attention; borrows its model.
struct fwd_session {
  fwd_model* m = nullptr;
  int Bmax = 0, Smax = 0;
  int B = 0, len = 0;  // sequences and their common length after the last call
  std::vector<void*> allocs;
  char* kc = nullptr;  // layer l at kc + l * layer_bytes
  char* vc = nullptr;
  int64_t layer_bytes = 0;
  float* part = nullptr;
  unsigned* count = nullptr;  // [Bmax, Hkv] arrival counters of the decode attention
  float2* rope_tab[4] = {};   // as the model's, [Smax, D / 2] each
  ~fwd_session() {
    if (m && m->stream) (void)hipStreamSynchronize(m->stream);
    else (void)hipDeviceSynchronize();
    for (void* p : allocs) (void)hipFree(p);
  }
};

namespace {

// RoPE (cos, sin) tables [rows, D/2] for one layer kind and longrope factor set:
// angle(t, k) = t * f_k with f_k from the base (rope_theta, or rope_theta_local on
// local layers) and the scaling of the config, both entries times the longrope
// multiplier; computed in double on the host ("N7 · model/forward-parity", intro:
// RoPE; Theorem statement: llama3 rope scaling, phi3 longrope, gemma3 local layers).
std::vector<double> rope_frequencies(const fwd_model* m, bool local, bool long_set, double* mult) {
  const fwd_config& c = m->cfg;
  const int64_t D = m->g.D, half = D / 2;
  const double theta = local && c.rope_theta_local > 0.0 ? c.rope_theta_local : c.rope_theta;
  std::vector<double> f(half);
  for (int64_t k = 0; k < half; ++k) f[k] = std::pow(theta, -2.0 * (double)k / (double)D);
  *mult = 1.0;
  if (c.rope_scaling == FWD_ROPE_LLAMA3) {
    const double L0 = c.rope_original_max_pos, s = c.rope_factor;
    const double lo = c.rope_low_freq_factor, hi = c.rope_high_freq_factor;
    for (double& fk : f) {
      const double wavelen = 2.0 * M_PI / fk;
      if (wavelen < L0 / hi) continue;  // high frequencies unchanged
      if (wavelen > L0 / lo) {
        fk /= s;
      } else {
        const double t = (L0 / wavelen - lo) / (hi - lo);
        fk = (1.0 - t) * fk / s + t * fk;
      }
    }
  } else if (c.rope_scaling == FWD_ROPE_LONGROPE) {
    const std::vector<float>& e = long_set ? m->rope_long : m->rope_short;
    for (int64_t k = 0; k < half; ++k) f[k] = 1.0 / ((double)e[k] * std::pow(theta, 2.0 * (double)k / (double)D));
    const double s = c.rope_factor;
    if (s > 1.0) *mult = std::sqrt(1.0 + std::log(s) / std::log((double)c.rope_original_max_pos));
  }
  return f;
}

int rope_tables(fwd_model* m, float2* (&out)[4], int64_t rows, std::vector<void*>& owner) {
  const int64_t half = m->g.D / 2;
  bool any_local = false;
  for (int32_t k : m->kinds) any_local |= k == FWD_LAYER_LOCAL;
  const bool two_bases = any_local && m->cfg.rope_theta_local > 0.0 && m->cfg.rope_theta_local != m->cfg.rope_theta;
  const bool two_sets = m->cfg.rope_scaling == FWD_ROPE_LONGROPE;
  for (int i = 0; i < 4; ++i) out[i] = nullptr;
  for (int local = 0; local < (two_bases ? 2 : 1); ++local)
    for (int set = 0; set < (two_sets ? 2 : 1); ++set) {
      double mult = 1.0;
      const std::vector<double> f = rope_frequencies(m, local, set, &mult);
      std::vector<float2> cs((size_t)rows * half);
      for (int64_t t = 0; t < rows; ++t)
        for (int64_t k = 0; k < half; ++k) {
          const double ang = (double)t * f[k];
          cs[(size_t)t * half + k] = float2{(float)(mult * std::cos(ang)), (float)(mult * std::sin(ang))};
        }
      void* p = nullptr;
      HIP_TRY(hipMalloc(&p, (size_t)round_up((int64_t)cs.size() * 8, 256)));
      owner.push_back(p);
      out[2 * local + set] = (float2*)p;
      HIP_TRY(hipMemcpyAsync(p, cs.data(), cs.size() * 8, hipMemcpyHostToDevice, m->stream));
      HIP_TRY(hipStreamSynchronize(m->stream));  // the host table dies at scope end
    }
  // a kind or set without a table of its own uses the one it equals
  for (int local = 0; local < 2; ++local)
    for (int set = 0; set < 2; ++set)
      if (!out[2 * local + set]) out[2 * local + set] = out[2 * (two_bases ? local : 0) + (two_sets ? set : 0)];
  return FWD_OK;
}

// Packed row order of a q or k projection: within each head, the rotate-half pair
// (k, k + D/2) is placed C rows apart in the same 2C-row group, so the GEMM
// epilogue receives both members of a pair together (C = fwdk::pair_chunk).
std::vector<int32_t> rope_row_map(int heads, int D, int C, int offset) {
  std::vector<int32_t> map((size_t)heads * D);
  const int half = D / 2;
  for (int h = 0; h < heads; ++h)
    for (int d = 0; d < D; ++d) {
      const int k = d < half ? d : d - half, second = d < half ? 0 : 1;
      const int packed = (2 * (k / C) + second) * C + (k % C);
      map[(size_t)h * D + d] = offset + h * D + packed;
    }
  return map;
}

// Gate row f and up row f land C rows apart in the same 2C-row group.
std::vector<int32_t> glu_row_map(int F, int C, int second) {
  std::vector<int32_t> map(F);
  for (int f = 0; f < F; ++f) map[f] = (2 * (f / C) + second) * C + (f % C);
  return map;
}

std::vector<int32_t> identity_map(int rows, int offset) {
  std::vector<int32_t> map(rows);
  for (int r = 0; r < rows; ++r) map[r] = offset + r;
  return map;
}

bool device_is_gfx950() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return false;
  return std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
}

}  // namespace

extern "C" {

int fwd_available(void) { return device_is_gfx950() ? 1 : 0; }

const char* fwd_last_error(void) { return g_err.c_str(); }

int fwd_output_sizes(const fwd_config* cfg, int32_t B, int32_t S, fwd_sizes* out) {
  if (int rc = check_config(cfg)) return rc;
  if (!out || B < 0 || S < 0) return fail(FWD_E_ARG, "bad B, S or NULL output");
  const Geometry g = geometry(cfg);
  const int64_t T = (int64_t)B * S;
  out->logits_elems = T * g.V;
  out->hidden_elems = (g.L + 2) * T * g.H;
  out->argmax_elems = T;
  out->weight_bytes = g.weight_bytes();
  out->workspace_bytes = g.workspace_bytes(cfg->norm_placement == FWD_NORM_SANDWICH);
  return FWD_OK;
}

int fwd_create(const fwd_config* cfg, const fwd_weights* w, void* hip_stream, fwd_model** out) {
  if (!out) return fail(FWD_E_ARG, "out is NULL");
  *out = nullptr;
  if (int rc = check_config(cfg)) return rc;
  if (!w || !w->embed || !w->final_norm || (cfg->n_layers > 0 && !w->layers))
    return fail(FWD_E_WEIGHTS, "embed, final_norm and layers are required");
  const bool sandwich = cfg->norm_placement == FWD_NORM_SANDWICH;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const fwd_layer_weights& L = w->layers[l];
    const bool moe = cfg->n_experts > 0 && (!cfg->ffn_kind || cfg->ffn_kind[l] == FWD_FFN_MOE);
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.ffn_norm ||
        (!moe && (!L.w_gate || !L.w_up || !L.w_down)) ||
        (moe && (!L.router || !L.expert_gate || !L.expert_up || !L.expert_down)) ||
        (sandwich && (!L.post_attn_norm || !L.post_ffn_norm)) || (cfg->qk_norm && (!L.q_norm || !L.k_norm)))
      return fail(FWD_E_WEIGHTS, "layer " + std::to_string(l) + " is missing a weight pointer");
  }
  if (!device_is_gfx950()) return fail(FWD_E_UNAVAILABLE, "no gfx950 device is available");

  fwd_model* m = new fwd_model();
  m->cfg = *cfg;
  m->kinds.assign(cfg->n_layers, FWD_LAYER_GLOBAL);
  if (cfg->layer_kind) m->kinds.assign(cfg->layer_kind, cfg->layer_kind + cfg->n_layers);
  m->cfg.layer_kind = nullptr;
  if (cfg->rope_scaling == FWD_ROPE_LONGROPE) {
    m->rope_short.assign(cfg->rope_short_factor, cfg->rope_short_factor + cfg->head_dim / 2);
    m->rope_long.assign(cfg->rope_long_factor, cfg->rope_long_factor + cfg->head_dim / 2);
  }
  m->cfg.rope_short_factor = m->cfg.rope_long_factor = nullptr;
  m->cfg.ffn_kind = nullptr;  // (read into each layer's flag at packing)
  m->dt = DType(cfg->dtype);
  m->g = geometry(cfg);
  m->stream = (hipStream_t)hip_stream;
  m->embed_scale = cfg->embed_scale_mode == FWD_EMBED_SCALE_BF16_SQRT_HIDDEN ? bf16_sqrt(cfg->hidden) : 1.f;
  const Geometry& g = m->g;
  hipStream_t s = m->stream;
  const int C = fwdk::pair_chunk(m->dt);

  auto run = [&]() -> int {
    // ---- weights ----
    // row maps, uploaded once
    std::vector<int32_t> maps;
    auto append = [&](const std::vector<int32_t>& v) {
      const size_t off = maps.size();
      maps.insert(maps.end(), v.begin(), v.end());
      return off;
    };
    const size_t mq = append(rope_row_map((int)g.Hq, (int)g.D, C, 0));
    const size_t mk = append(rope_row_map((int)g.Hkv, (int)g.D, C, (int)(g.Hq * g.D)));
    const size_t mv = append(identity_map((int)(g.Hkv * g.D), (int)((g.Hq + g.Hkv) * g.D)));
    const size_t mg = append(glu_row_map((int)g.F, C, 0));
    const size_t mu = append(glu_row_map((int)g.F, C, 1));
    const size_t mid = append(identity_map((int)std::max({g.V, g.H, g.F, g.E}), 0));
    const size_t mge = append(glu_row_map((int)std::max<int64_t>(g.Fe, 1), C, 0));
    const size_t mue = append(glu_row_map((int)std::max<int64_t>(g.Fe, 1), C, 1));
    int32_t* dmaps = nullptr;
    HIP_TRY(hipMalloc((void**)&dmaps, maps.size() * 4));
    struct Free {
      int32_t* p;
      ~Free() { (void)hipFree(p); }
    } free_maps{dmaps};
    HIP_TRY(hipMemcpyAsync(dmaps, maps.data(), maps.size() * 4, hipMemcpyHostToDevice, s));

    // dst[map[r], :] = src[r, :] for an operand of `rows` (allocated g.rows(rows)) x K,
    // K-tiled for bf16 (padding rows cleared), row-major for f32
    auto place = [&](void* dst, int64_t dst_rows, const void* src, size_t map, int rows, int64_t K) -> int {
      if (g.tiled) {
        HIP_TRY(hipMemsetAsync(dst, 0, g.rows(dst_rows) * K * g.esize, s));
        HIP_TRY(fwdk::pack_tiled(dst, src, dmaps + map, rows, (int)K, s));
      } else {
        HIP_TRY(fwdk::copy_rows(dst, src, dmaps + map, rows, K * g.esize, s));
      }
      return FWD_OK;
    };
    auto alloc_operand = [&](void** p, int64_t rows, int64_t K) { return m->alloc(p, g.rows(rows) * K * g.esize); };

    if (int rc = alloc_operand(&m->embed, g.V, g.H)) return rc;
    if (int rc = place(m->embed, g.V, w->embed, mid, (int)g.V, g.H)) return rc;
    if (int rc = m->alloc((void**)&m->final_norm, g.H * 4)) return rc;
    const float goff = (float)cfg->norm_gain_offset;
    HIP_TRY(fwdk::gains_to_f32(m->dt, w->final_norm, m->final_norm, (int)g.H, goff, s));

    m->layers.resize(g.L);
    for (int l = 0; l < g.L; ++l) {
      const fwd_layer_weights& W = w->layers[l];
      fwd_model::Layer& L = m->layers[l];
      L = fwd_model::Layer{};
      if (int rc = m->alloc((void**)&L.attn_norm, g.H * 4)) return rc;
      if (int rc = m->alloc((void**)&L.ffn_norm, g.H * 4)) return rc;
      HIP_TRY(fwdk::gains_to_f32(m->dt, W.attn_norm, L.attn_norm, (int)g.H, goff, s));
      HIP_TRY(fwdk::gains_to_f32(m->dt, W.ffn_norm, L.ffn_norm, (int)g.H, goff, s));
      if (cfg->qk_norm) {
        if (int rc = m->alloc((void**)&L.q_norm, g.D * 4)) return rc;
        if (int rc = m->alloc((void**)&L.k_norm, g.D * 4)) return rc;
        HIP_TRY(fwdk::gains_to_f32(m->dt, W.q_norm, L.q_norm, (int)g.D, goff, s));
        HIP_TRY(fwdk::gains_to_f32(m->dt, W.k_norm, L.k_norm, (int)g.D, goff, s));
      }
      if (sandwich) {
        if (int rc = m->alloc((void**)&L.post_attn, g.H * 4)) return rc;
        if (int rc = m->alloc((void**)&L.post_ffn, g.H * 4)) return rc;
        HIP_TRY(fwdk::gains_to_f32(m->dt, W.post_attn_norm, L.post_attn, (int)g.H, goff, s));
        HIP_TRY(fwdk::gains_to_f32(m->dt, W.post_ffn_norm, L.post_ffn, (int)g.H, goff, s));
      }
      if (int rc = alloc_operand(&L.wqkv, g.qkv_rows, g.H)) return rc;
      if (g.tiled) HIP_TRY(hipMemsetAsync(L.wqkv, 0, g.rows(g.qkv_rows) * g.H * g.esize, s));
      // (three sources into one operand: clear once, then pack each)
      auto put = [&](void* dst, const void* src, size_t map, int rows, int64_t K) -> int {
        if (g.tiled) HIP_TRY(fwdk::pack_tiled(dst, src, dmaps + map, rows, (int)K, s));
        else HIP_TRY(fwdk::copy_rows(dst, src, dmaps + map, rows, K * g.esize, s));
        return FWD_OK;
      };
      if (int rc = put(L.wqkv, W.wq, mq, (int)(g.Hq * g.D), g.H)) return rc;
      if (int rc = put(L.wqkv, W.wk, mk, (int)(g.Hkv * g.D), g.H)) return rc;
      if (int rc = put(L.wqkv, W.wv, mv, (int)(g.Hkv * g.D), g.H)) return rc;
      L.moe = g.E > 0 && (!cfg->ffn_kind || cfg->ffn_kind[l] == FWD_FFN_MOE);
      if (!L.moe) {
        if (int rc = alloc_operand(&L.wgu, 2 * g.F, g.H)) return rc;
        if (g.tiled) HIP_TRY(hipMemsetAsync(L.wgu, 0, g.rows(2 * g.F) * g.H * g.esize, s));
        if (int rc = put(L.wgu, W.w_gate, mg, (int)g.F, g.H)) return rc;
        if (int rc = put(L.wgu, W.w_up, mu, (int)g.F, g.H)) return rc;
        if (int rc = alloc_operand(&L.wdown, g.H, g.F)) return rc;
        if (int rc = place(L.wdown, g.H, W.w_down, mid, (int)g.H, g.F)) return rc;
      } else {
        // router [E, H]; per expert e: gate/up rows interleaved like the dense layer's
        // at wgu + e * rows(2 Fe) * H, down at wdown + e * rows(H) * Fe (all K-tiled)
        if (int rc = alloc_operand(&L.router, g.E, g.H)) return rc;
        if (int rc = place(L.router, g.E, W.router, mid, (int)g.E, g.H)) return rc;
        const int64_t gu_e = g.rows(2 * g.Fe) * g.H, d_e = g.rows(g.H) * g.Fe;
        if (int rc = m->alloc(&L.wgu, g.E * gu_e * g.esize)) return rc;
        if (int rc = m->alloc(&L.wdown, g.E * d_e * g.esize)) return rc;
        HIP_TRY(hipMemsetAsync(L.wgu, 0, g.E * gu_e * g.esize, s));
        HIP_TRY(hipMemsetAsync(L.wdown, 0, g.E * d_e * g.esize, s));
        for (int64_t e = 0; e < g.E; ++e) {
          char* gu = (char*)L.wgu + e * gu_e * g.esize;
          const char* src_g = (const char*)W.expert_gate + e * g.Fe * g.H * g.esize;
          const char* src_u = (const char*)W.expert_up + e * g.Fe * g.H * g.esize;
          const char* src_d = (const char*)W.expert_down + e * g.H * g.Fe * g.esize;
          if (int rc = put(gu, src_g, mge, (int)g.Fe, g.H)) return rc;
          if (int rc = put(gu, src_u, mue, (int)g.Fe, g.H)) return rc;
          if (int rc = put((char*)L.wdown + e * d_e * g.esize, src_d, mid, (int)g.H, g.Fe)) return rc;
        }
      }
      if (int rc = alloc_operand(&L.wo, g.H, g.Hq * g.D)) return rc;
      if (int rc = place(L.wo, g.H, W.wo, mid, (int)g.H, g.Hq * g.D)) return rc;
    }
    HIP_TRY(hipStreamSynchronize(s));  // the row maps are freed at scope end

    // ---- RoPE table ----
    if (int rc = rope_tables(m, m->rope_tab, g.T, m->allocs)) return rc;

    // ---- workspace ----
    const int64_t T = g.T;
    if (int rc = m->alloc((void**)&m->x, T * g.H * 4)) return rc;
    if (int rc = m->alloc((void**)&m->xb, T * g.H * 4)) return rc;
    if (int rc = m->alloc(&m->n, g.rows(T) * g.H * g.esize)) return rc;
    if (int rc = m->alloc(&m->qk, T * (g.Hq + 2 * g.Hkv) * g.D * g.esize)) return rc;
    if (int rc = m->alloc(&m->vt, 8 * T * g.Hkv * g.D * g.esize)) return rc;
    if (int rc = m->alloc(&m->o, g.rows(T) * g.Hq * g.D * g.esize)) return rc;
    if (int rc = m->alloc(&m->a, g.rows(T) * g.F * g.esize)) return rc;
    if (sandwich)
      if (int rc = m->alloc((void**)&m->u, T * g.H * 4)) return rc;
    if (sandwich && g.tiled) {
      m->ds.part_floats = g.dense_split_floats();
      if (int rc = m->alloc((void**)&m->ds.part, m->ds.part_floats * 4)) return rc;
    }
    if (int rc = m->alloc((void**)&m->ids, T * 4)) return rc;
    if (int rc = m->alloc((void**)&m->amax, T * 4)) return rc;
    if (int rc = m->alloc((void**)&m->flag, 256)) return rc;
    if (int rc = m->alloc((void**)&m->logits_ws, g.logit_ws_bytes())) return rc;
    if (int rc = m->alloc((void**)&m->argpart, kArgPartPairs * 8)) return rc;
    if (g.E > 0) {
      const int64_t A = T * g.topk, nch = fwdk::moe_chunks(A);
      if (int rc = m->alloc((void**)&m->moe_logits, T * g.E * 4)) return rc;
      if (int rc = m->alloc((void**)&m->moe_idx, A * 4)) return rc;
      if (int rc = m->alloc((void**)&m->moe_w, A * 4)) return rc;
      if (int rc = m->alloc((void**)&m->plan.pos, A * 4)) return rc;
      if (int rc = m->alloc((void**)&m->plan.chunk_count, nch * g.E * 4)) return rc;
      if (int rc = m->alloc((void**)&m->plan.chunk_base, nch * g.E * 4)) return rc;
      if (int rc = m->alloc((void**)&m->plan.total, g.E * 4)) return rc;
      if (int rc = m->alloc((void**)&m->plan.seg_start, g.E * 4)) return rc;
      if (int rc = m->alloc((void**)&m->plan.seg_count, g.E * 4)) return rc;
      if (int rc = m->alloc((void**)&m->plan.mtile_start, (g.E + 1) * 4)) return rc;
      if (int rc = m->alloc(&m->moe_x, g.moe_rows() * g.H * g.esize)) return rc;
      if (int rc = m->alloc(&m->moe_a, g.moe_rows() * g.Fe * g.esize)) return rc;
      if (int rc = m->alloc((void**)&m->moe_y, g.moe_rows() * g.H * 4)) return rc;
    }
    if (g.tiled) {
      m->sk.part_floats = g.skinny_part_floats();
      m->sk.count_len = g.skinny_counters();
      if (int rc = m->alloc((void**)&m->sk.part, std::max<int64_t>(m->sk.part_floats, 1) * 4)) return rc;
      if (int rc = m->alloc((void**)&m->sk.count, m->sk.count_len * 4)) return rc;
      HIP_TRY(hipMemsetAsync(m->sk.count, 0, m->sk.count_len * 4, s));  // the kernels leave them zero
      if (int rc = m->alloc((void**)&m->ssq, fwdk::skinny_groups((int)g.H) * fwdk::kSkinnyRows * 4)) return rc;
    }
    HIP_TRY(hipStreamSynchronize(s));
    return FWD_OK;
  };
  const int rc = run();
  if (rc != FWD_OK) {
    delete m;
    return rc;
  }
  *out = m;
  return FWD_OK;
}

}  // extern "C"

namespace {

// The forward pass over B sequences of S new tokens each, at positions pos0 .. pos0 +
// S - 1. Without a session: the plain prefill (pos0 = 0). With one: every layer's
// rotated keys and values are also stored in the cache; when `decode` is set (S = 1,
// pos0 = the cached length) attention runs over the cache instead of the prefill
// kernel. Shapes are checked by the callers.
int forward(fwd_model* m, fwd_session* sess, const int32_t* ids_host, int32_t B, int32_t S, int pos0, bool decode,
            const fwd_outputs* out) {
  const int64_t T = (int64_t)B * S;
  const int V = (int)m->g.V;
  const fwd_outputs none{nullptr, nullptr, nullptr};
  const fwd_outputs& o = out ? *out : none;

  const Geometry& g = m->g;
  const DType dt = m->dt;
  hipStream_t s = m->stream;
  const int H = (int)g.H, Hq = (int)g.Hq, Hkv = (int)g.Hkv, D = (int)g.D, F = (int)g.F, L = (int)g.L;
  const int M = (int)T;
  const float eps = m->cfg.rms_eps;
  const bool sandwich = m->cfg.norm_placement == FWD_NORM_SANDWICH;
  const int64_t TH = T * H;
  float* hidden = o.hidden;
  const bool tl = g.tiled;
  const fwdk::SplitK* sk = tl ? &m->sk : nullptr;  // used by products of at most kSkinnyRows rows

  m->marks.clear();
  m->events_used = 0;
  HIP_TRY(hipMemcpyAsync(m->ids, ids_host, T * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemsetAsync(m->flag, 0, 4, s));

  float* cur = hidden ? hidden : m->x;
  TIMED(m, FWD_KERNEL_EMBED, fwdk::embed(dt, m->ids, m->embed, cur, M, H, m->embed_scale, tl, s));
  // first layer's input norm; every later sublayer input norm is fused below
  if (L > 0) TIMED(m, FWD_KERNEL_NORM, fwdk::rmsnorm(dt, cur, m->layers[0].attn_norm, m->n, nullptr, M, H, eps, tl, s));
  // Few rows, pre-norm, no hidden slots: each residual product also leaves its rows' sums
  // of squares, and the next product normalises its input itself (no norm launches
  // after the first).
  const bool fuse = tl && M <= fwdk::kSkinnyRows && !sandwich && !hidden && L > 0 && g.moe_layers == 0;
  // RoPE tables of this call: per layer kind, and the longrope factor set its length selects
  float2* const* rope_tabs = sess ? sess->rope_tab : m->rope_tab;
  const int rope_set =
      m->cfg.rope_scaling == FWD_ROPE_LONGROPE && (int64_t)pos0 + S > m->cfg.rope_original_max_pos ? 1 : 0;
  const int ngroups = (int)fwdk::skinny_groups(H);
  auto normx = [&](const float* x, const float* w) { return fwdk::RowNormX{x, w, m->ssq, ngroups, eps}; };

  const int ldvt = (int)round_up(S, 8);
  char* qk = (char*)m->qk;
  for (int l = 0; l < L; ++l) {
    const fwd_model::Layer& w = m->layers[l];
    float* xin = cur;
    float* xmid = hidden ? m->xb : m->x;
    float* xout = hidden ? hidden + (int64_t)(l + 1) * TH : m->x;
    const bool last = l + 1 == L;
    const float* next_norm = last ? m->final_norm : m->layers[l + 1].attn_norm;

    // attention sublayer (its input norm is already in m->n)
    // with a session, the rotated keys and the values are also stored in the cache: by
    // the QKV epilogue, or with QK-norm by the pass that normalises and rotates
    void* kc = sess ? sess->kc + l * sess->layer_bytes : nullptr;
    void* vc = sess ? sess->vc + l * sess->layer_bytes : nullptr;
    const bool local = m->kinds[l] == FWD_LAYER_LOCAL;
    const float2* cs = rope_tabs[2 * (local ? 1 : 0) + rope_set];
    const bool qkn = m->cfg.qk_norm != 0;
    fwdk::RopeArgs ra{m->qk, cs, Hq, Hkv, D, S, pos0, qkn ? nullptr : kc, qkn ? nullptr : vc,
                      sess && !qkn ? sess->Smax : 0, !qkn};
    const fwdk::RowNormX nq = normx(xin, w.attn_norm);
    TIMED(m, FWD_KERNEL_QKV_ROPE,
          fwdk::gemm_qkv_rope(dt, m->n, w.wqkv, ra, M, H, tl, s, sk, fuse && l > 0 ? &nq : nullptr));
    const int64_t ldqkv = (int64_t)(Hq + 2 * Hkv) * D;
    if (qkn) {
      fwdk::QkNormArgs qa{m->qk, ldqkv, Hq, Hkv, D, S, pos0, cs, w.q_norm, w.k_norm, eps, kc, vc,
                          sess ? sess->Smax : 0};
      TIMED(m, FWD_KERNEL_QK_NORM, fwdk::qk_norm_rope(dt, qa, M, s));
    }
    const int window = local ? m->cfg.sliding_window : 0;
    if (sess) {
      if (decode) {
        TIMED(m, FWD_KERNEL_ATTENTION, fwdk::attention_decode(dt, qk, ldqkv, kc, vc, sess->Smax, pos0 + 1, B, Hq, Hkv,
                                                              D, window, m->o, (int64_t)Hq * D, tl, sess->part, sess->count,
                                                              s));
      }
    }
    if (!decode) {
    TIMED(m, FWD_KERNEL_V_TRANSPOSE,
          fwdk::transpose_v(dt, qk + (int64_t)(Hq + Hkv) * D * g.esize, ldqkv, m->vt, ldvt, B, S, Hkv * D, s));
    fwdk::AttnArgs aa{};
    aa.q = qk;
    aa.k = qk + (int64_t)Hq * D * g.esize;
    aa.vt = m->vt;
    aa.o = m->o;
    aa.ldq = aa.ldk = ldqkv;
    aa.ldo = (int64_t)Hq * D;
    aa.ldvt = ldvt;
    aa.B = B;
    aa.S = S;
    aa.Hq = Hq;
    aa.Hkv = Hkv;
    aa.D = D;
    aa.window = window;
    aa.o_tiled = tl;
    TIMED(m, FWD_KERNEL_ATTENTION, fwdk::attention(dt, aa, s));
    }
    if (fuse) {
      TIMED(m, FWD_KERNEL_O_PROJ, fwdk::gemm_residual(dt, m->o, w.wo, xin, xmid, M, H, Hq * D, tl, s, sk, m->ssq));
    } else if (!sandwich) {
      TIMED(m, FWD_KERNEL_O_PROJ, fwdk::gemm_residual(dt, m->o, w.wo, xin, xmid, M, H, Hq * D, tl, s, sk));
      TIMED(m, FWD_KERNEL_NORM, fwdk::rmsnorm(dt, xmid, w.ffn_norm, m->n, nullptr, M, H, eps, tl, s));
    } else {
      TIMED(m, FWD_KERNEL_O_PROJ, fwdk::gemm_store(dt, m->o, w.wo, m->u, H, M, H, Hq * D, 0.f, tl, s, sk, nullptr, &m->ds));
      TIMED(m, FWD_KERNEL_NORM, fwdk::add_norm(dt, xin, m->u, w.post_attn, xmid, w.ffn_norm, m->n, nullptr, M, H, eps, tl, s));
    }

    // feed-forward sublayer
    float* final32 = (last && hidden) ? hidden + (int64_t)(L + 1) * TH : nullptr;
    if (w.moe) {
      // mixture of experts on the normalised rows in m->n: route, permute by expert,
      // grouped expert products, weighted combination (+ the residual for pre-norm)
      const int E = (int)g.E, k = (int)g.topk, Fe = (int)g.Fe, A = M * k;
      TIMED(m, FWD_KERNEL_MOE_ROUTE, fwdk::gemm_store(dt, m->n, w.router, m->moe_logits, E, M, E, H, 0.f, tl, s, sk));
      TIMED(m, FWD_KERNEL_MOE_ROUTE, fwdk::moe_route(m->moe_logits, M, E, k, m->cfg.moe_norm_topk != 0, m->moe_idx,
                                                     m->moe_w, s));
      TIMED(m, FWD_KERNEL_MOE_ROUTE, fwdk::moe_plan(m->moe_idx, A, E, m->plan, s));
      TIMED(m, FWD_KERNEL_MOE_ROUTE, fwdk::moe_gather(m->n, m->plan.pos, A, k, H, m->moe_x, s));
      const int max_tiles = (A + fwdk::kMoeTileRows - 1) / fwdk::kMoeTileRows + E;
      const fwdk::GroupArgs gu{m->plan.seg_start, m->plan.seg_count, m->plan.mtile_start, E, g.rows(2 * g.Fe) * H,
                               max_tiles};
      const fwdk::GroupArgs gd{m->plan.seg_start, m->plan.seg_count, m->plan.mtile_start, E, g.rows(g.H) * g.Fe,
                               max_tiles};
      TIMED(m, FWD_KERNEL_MOE_EXPERTS,
            fwdk::gemm_grouped_swiglu(m->moe_x, w.wgu, m->moe_a, Fe, H, gu, m->cfg.ffn_act, s));
      TIMED(m, FWD_KERNEL_MOE_EXPERTS, fwdk::gemm_grouped_store(m->moe_a, w.wdown, m->moe_y, H, Fe, gd, s));
      if (!sandwich) {
        TIMED(m, FWD_KERNEL_MOE_COMBINE,
              fwdk::moe_combine(m->moe_y, m->plan.pos, m->moe_w, M, k, H, xmid, xout, s));
        TIMED(m, FWD_KERNEL_NORM, fwdk::rmsnorm(dt, xout, next_norm, m->n, final32, M, H, eps, tl, s));
      } else {
        TIMED(m, FWD_KERNEL_MOE_COMBINE,
              fwdk::moe_combine(m->moe_y, m->plan.pos, m->moe_w, M, k, H, nullptr, m->u, s));
        TIMED(m, FWD_KERNEL_NORM,
              fwdk::add_norm(dt, xmid, m->u, w.post_ffn, xout, next_norm, m->n, final32, M, H, eps, tl, s));
      }
      cur = xout;
      continue;
    }
    const fwdk::RowNormX nf = normx(xmid, w.ffn_norm);
    TIMED(m, FWD_KERNEL_GATE_UP,
          fwdk::gemm_swiglu(dt, m->n, w.wgu, m->a, M, F, H, tl, s, sk, fuse ? &nf : nullptr, m->cfg.ffn_act));
    if (fuse) {
      TIMED(m, FWD_KERNEL_DOWN_PROJ, fwdk::gemm_residual(dt, m->a, w.wdown, xmid, xout, M, H, F, tl, s, sk, m->ssq));
    } else if (!sandwich) {
      TIMED(m, FWD_KERNEL_DOWN_PROJ, fwdk::gemm_residual(dt, m->a, w.wdown, xmid, xout, M, H, F, tl, s, sk));
      TIMED(m, FWD_KERNEL_NORM, fwdk::rmsnorm(dt, xout, next_norm, m->n, final32, M, H, eps, tl, s));
    } else {
      TIMED(m, FWD_KERNEL_DOWN_PROJ, fwdk::gemm_store(dt, m->a, w.wdown, m->u, H, M, H, F, 0.f, tl, s, sk, nullptr, &m->ds));
      TIMED(m, FWD_KERNEL_NORM, fwdk::add_norm(dt, xmid, m->u, w.post_ffn, xout, next_norm, m->n, final32, M, H, eps, tl, s));
    }
    cur = xout;
  }
  if (L == 0) {
    float* final32 = hidden ? hidden + TH : nullptr;
    TIMED(m, FWD_KERNEL_NORM, fwdk::rmsnorm(dt, cur, m->final_norm, m->n, final32, M, H, eps, tl, s));
  }

  // tied LM head (+ softcap) and argmax
  const float cap = m->cfg.final_logit_softcap;
  int32_t* am = o.argmax ? o.argmax : m->amax;
  const fwdk::RowNormX nh = normx(cur, m->final_norm);
  const fwdk::RowNormX* nhp = fuse ? &nh : nullptr;
  if (dt == fwdk::DType::BF16 && tl && M > fwdk::kSkinnyRows) {
    // argmax folded into the head's epilogue; logits written only when requested
    int nchunk = 0;
    uint64_t* keys = (uint64_t*)m->logits_ws;
    TIMED(m, FWD_KERNEL_LM_HEAD,
          fwdk::gemm_head_keys(m->n, m->embed, o.logits, V, M, V, H, cap, keys, &nchunk, m->flag, s));
    TIMED(m, FWD_KERNEL_ARGMAX, fwdk::argmax_keys(keys, nchunk, M, am, s));
  } else if (o.logits) {
    TIMED(m, FWD_KERNEL_LM_HEAD, fwdk::gemm_store(dt, m->n, m->embed, o.logits, V, M, V, H, cap, tl, s, sk, nhp));
    TIMED(m, FWD_KERNEL_ARGMAX, fwdk::argmax_rows(o.logits, V, M, V, am, m->flag, s, m->argpart, kArgPartPairs));
  } else {
    const int64_t chunk = g.logit_chunk;
    for (int64_t r0 = 0; r0 < T; r0 += chunk) {
      const int rows = (int)std::min<int64_t>(chunk, T - r0);
      const char* nrow = (const char*)m->n + r0 * H * g.esize;  // (r0 is a multiple of 16: a tile row)
      TIMED(m, FWD_KERNEL_LM_HEAD,
            fwdk::gemm_store(dt, nrow, m->embed, m->logits_ws, V, rows, V, H, cap, tl, s, sk, nhp));  // (fused: one chunk)
      TIMED(m, FWD_KERNEL_ARGMAX,
            fwdk::argmax_rows(m->logits_ws, V, rows, V, am + r0, m->flag, s, m->argpart, kArgPartPairs));
    }
  }
  int flag = 0;
  HIP_TRY(hipMemcpyAsync(&flag, m->flag, 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (int rc = m->collect()) return rc;
  if (flag) return fail(FWD_E_NONFINITE, "non-finite logits");
  return FWD_OK;
}

int check_ids(const int32_t* ids_host, int64_t T, int V) {
  if (!ids_host) return fail(FWD_E_ARG, "ids is NULL");
  for (int64_t i = 0; i < T; ++i)
    if (ids_host[i] < 0 || ids_host[i] >= V)
      return fail(FWD_E_TOKEN_RANGE, "token id " + std::to_string(ids_host[i]) + " at index " + std::to_string(i) +
                                         " is outside [0, " + std::to_string(V) + ")");
  return FWD_OK;
}

}  // namespace

extern "C" {

int fwd_prefill(fwd_model* m, const int32_t* ids_host, int32_t B, int32_t S, const fwd_outputs* out) {
  if (!m) return fail(FWD_E_ARG, "model is NULL");
  if (B < 0 || S < 0) return fail(FWD_E_ARG, "B and S must be >= 0");
  const int64_t T = (int64_t)B * S;
  if (T == 0) return FWD_OK;
  if (T > m->g.T) return fail(FWD_E_TOO_LARGE, "B*S = " + std::to_string(T) + " exceeds max_tokens " +
                                                   std::to_string(m->g.T));
  if (int rc = check_ids(ids_host, T, (int)m->g.V)) return rc;
  return forward(m, nullptr, ids_host, B, S, 0, false, out);
}

int fwd_session_create(fwd_model* m, int32_t max_batch, int32_t max_seq, fwd_session** out) {
  if (!out) return fail(FWD_E_ARG, "out is NULL");
  *out = nullptr;
  if (!m) return fail(FWD_E_ARG, "model is NULL");
  if (max_batch <= 0 || max_seq <= 0) return fail(FWD_E_ARG, "max_batch and max_seq must be positive");
  if (max_batch > m->g.T) return fail(FWD_E_TOO_LARGE, "max_batch exceeds the model's max_tokens");
  const Geometry& g = m->g;
  if (g.Hq / g.Hkv > 16) return fail(FWD_E_CONFIG, "decode supports at most 16 query heads per kv head");
  fwd_session* se = new fwd_session();
  se->m = m;
  se->Bmax = max_batch;
  se->Smax = max_seq;
  auto run = [&]() -> int {
    se->layer_bytes = round_up((int64_t)max_batch * g.Hkv * max_seq * g.D * g.esize, 256);
    const int64_t cache = std::max<int64_t>(g.L, 1) * se->layer_bytes;
    void* p = nullptr;
    HIP_TRY(hipMalloc(&p, (size_t)cache));
    se->allocs.push_back(p);
    se->kc = (char*)p;
    HIP_TRY(hipMalloc(&p, (size_t)cache));
    se->allocs.push_back(p);
    se->vc = (char*)p;
    const int64_t nsplit = (max_seq + fwdk::kDecodeChunk - 1) / fwdk::kDecodeChunk;
    HIP_TRY(hipMalloc(&p, (size_t)round_up((int64_t)max_batch * g.Hq * nsplit * (g.D + 2) * 4, 256)));
    se->allocs.push_back(p);
    se->part = (float*)p;
    HIP_TRY(hipMalloc(&p, (size_t)round_up((int64_t)max_batch * g.Hkv * 4, 256)));
    se->allocs.push_back(p);
    se->count = (unsigned*)p;
    HIP_TRY(hipMemsetAsync(p, 0, (size_t)max_batch * g.Hkv * 4, m->stream));  // the kernel leaves them zero
    return rope_tables(m, se->rope_tab, max_seq, se->allocs);
  };
  if (int rc = run()) {
    delete se;
    return rc;
  }
  *out = se;
  return FWD_OK;
}

int fwd_session_prefill(fwd_session* se, const int32_t* ids_host, int32_t B, int32_t S, const fwd_outputs* out) {
  if (!se) return fail(FWD_E_ARG, "session is NULL");
  if (B <= 0 || S <= 0) return fail(FWD_E_ARG, "B and S must be positive");
  if (B > se->Bmax || S > se->Smax)
    return fail(FWD_E_TOO_LARGE, "B or S exceeds the session's max_batch / max_seq");
  const int64_t T = (int64_t)B * S;
  if (T > se->m->g.T) return fail(FWD_E_TOO_LARGE, "B*S exceeds the model's max_tokens");
  if (int rc = check_ids(ids_host, T, (int)se->m->g.V)) return rc;
  se->B = 0;
  se->len = 0;
  if (int rc = forward(se->m, se, ids_host, B, S, 0, false, out)) return rc;
  se->B = B;
  se->len = S;
  return FWD_OK;
}

int fwd_session_decode(fwd_session* se, const int32_t* ids_host, const fwd_outputs* out) {
  if (!se) return fail(FWD_E_ARG, "session is NULL");
  if (se->len <= 0) return fail(FWD_E_ARG, "decode needs a prefilled session");
  if (se->len >= se->Smax) return fail(FWD_E_TOO_LARGE, "the session is full (max_seq tokens)");
  if (int rc = check_ids(ids_host, se->B, (int)se->m->g.V)) return rc;
  if (int rc = forward(se->m, se, ids_host, se->B, 1, se->len, true, out)) return rc;
  se->len += 1;
  return FWD_OK;
}

int32_t fwd_session_length(const fwd_session* se) { return se ? se->len : -1; }

void fwd_session_destroy(fwd_session* se) { delete se; }

}  // extern "C"

namespace {
// fwd_gemm's split partials come from a memory pool of the library's own on each device,
// allocated and freed in stream order (so calls on concurrent streams never share them),
// with a release threshold that keeps the freed memory in the pool between calls
// instead of returning it to the driver at every synchronisation.
hipError_t split_pool(hipMemPool_t* out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static hipMemPool_t pools[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!pools[dev]) {
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    if ((e = hipMemPoolCreate(&p, &props)) != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    if ((e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) return e;
    pools[dev] = p;
  }
  *out = pools[dev];
  return hipSuccess;
}

// Argument checks shared by fwd_gemm and fwd_gemm_noalloc: FWD_OK to go on, `done`
// set when there is nothing to compute.
int gemm_args(const void* X, const void* W, const float* Y, int32_t P, int32_t in, int32_t out, int32_t dtype,
              bool* done) {
  *done = false;
  if (dtype != FWD_DTYPE_BF16 && dtype != FWD_DTYPE_F32) return fail(FWD_E_ARG, "dtype");
  if (P < 0 || in <= 0 || out < 0) return fail(FWD_E_ARG, "sizes must be P >= 0, in > 0, out >= 0");
  if (in % (dtype == FWD_DTYPE_BF16 ? 8 : 4)) return fail(FWD_E_ARG, "in must be a multiple of 8 (bf16) / 4 (f32)");
  if ((int64_t)P * out == 0) {
    *done = true;
    return FWD_OK;
  }
  if (!X || !W || !Y) return fail(FWD_E_ARG, "NULL buffer");
  if (!device_is_gfx950()) return fail(FWD_E_UNAVAILABLE, "no gfx950 device is available");
  return FWD_OK;
}
}  // namespace

extern "C" {

int fwd_gemm(const void* X, const void* W, float* Y, int32_t P, int32_t in, int32_t out, int32_t dtype,
             void* hip_stream) {
  bool done = false;
  if (int rc = gemm_args(X, W, Y, P, in, out, dtype, &done)) return rc;
  if (done) return FWD_OK;
  const hipStream_t s = (hipStream_t)hip_stream;
  fwdk::DenseSplit ds{nullptr, dtype == FWD_DTYPE_BF16 ? fwdk::dense_split_floats(P, out, in, false) : 0};
  if (ds.part_floats > 0) {  // split partials, stream-ordered: concurrent calls on other streams do not share them
    hipMemPool_t pool = nullptr;
    HIP_TRY(split_pool(&pool));
    HIP_TRY(hipMallocFromPoolAsync((void**)&ds.part, (size_t)ds.part_floats * 4, pool, s));
  }
  const hipError_t e = fwdk::gemm_store(DType(dtype), X, W, Y, out, P, out, in, 0.f, false, s, nullptr, nullptr, &ds);
  if (ds.part) HIP_TRY(hipFreeAsync(ds.part, s));
  HIP_TRY(e);
  return FWD_OK;
}

int fwd_gemm_noalloc(const void* X, const void* W, float* Y, int32_t P, int32_t in, int32_t out, int32_t dtype,
                     void* hip_stream) {
  bool done = false;
  if (int rc = gemm_args(X, W, Y, P, in, out, dtype, &done)) return rc;
  if (done) return FWD_OK;
  const int64_t need = dtype == FWD_DTYPE_BF16 ? fwdk::dense_split_floats(P, out, in, false) : 0;
  if (need > fwdk::kStaticSplitFloats)
    return fail(FWD_E_TOO_LARGE, "this product's split partials need " + std::to_string(need * 4) +
                                     " bytes; the static scratch holds " +
                                     std::to_string(fwdk::kStaticSplitFloats * 4));
  fwdk::DenseSplit ds{nullptr, 0};
  if (need > 0) {
    HIP_TRY(fwdk::static_split_scratch(&ds.part));
    ds.part_floats = fwdk::kStaticSplitFloats;
  }
  HIP_TRY(fwdk::gemm_store(DType(dtype), X, W, Y, out, P, out, in, 0.f, false, (hipStream_t)hip_stream, nullptr,
                           nullptr, &ds));
  return FWD_OK;
}

int fwd_attention(const void* q, const void* k, const void* v_t, void* o, int32_t B, int32_t S, int32_t n_heads,
                  int32_t n_kv_heads, int32_t head_dim, int32_t window, int32_t dtype, void* hip_stream) {
  if (dtype != FWD_DTYPE_BF16 && dtype != FWD_DTYPE_F32) return fail(FWD_E_ARG, "dtype");
  if (B < 0 || S < 0 || n_heads <= 0 || n_kv_heads <= 0 || window < 0) return fail(FWD_E_ARG, "bad sizes");
  if (n_heads % n_kv_heads) return fail(FWD_E_CONFIG, "n_heads must be a multiple of n_kv_heads");
  if (!fwdk::attention_supported(DType(dtype), head_dim)) return fail(FWD_E_CONFIG, "unsupported head_dim");
  if ((int64_t)B * S == 0) return FWD_OK;
  if (!q || !k || !v_t || !o) return fail(FWD_E_ARG, "NULL buffer");
  if (!device_is_gfx950()) return fail(FWD_E_UNAVAILABLE, "no gfx950 device is available");
  fwdk::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.vt = v_t;
  a.o = o;
  a.ldq = a.ldo = (int64_t)n_heads * head_dim;
  a.ldk = (int64_t)n_kv_heads * head_dim;
  a.ldvt = (int)round_up(S, 8);
  a.B = B;
  a.S = S;
  a.Hq = n_heads;
  a.Hkv = n_kv_heads;
  a.D = head_dim;
  a.window = window;
  a.o_tiled = false;
  HIP_TRY(fwdk::attention(DType(dtype), a, (hipStream_t)hip_stream));
  return FWD_OK;
}

int fwd_rmsnorm(const float* x, const void* w, void* y, int32_t rows, int32_t hidden, float eps, int32_t dtype,
                void* hip_stream) {
  if (dtype != FWD_DTYPE_BF16 && dtype != FWD_DTYPE_F32) return fail(FWD_E_ARG, "dtype");
  if (rows < 0 || hidden <= 0 || hidden % 4) return fail(FWD_E_ARG, "rows >= 0 and hidden a positive multiple of 4");
  if (rows == 0) return FWD_OK;
  if (!x || !w || !y) return fail(FWD_E_ARG, "NULL buffer");
  if (!device_is_gfx950()) return fail(FWD_E_UNAVAILABLE, "no gfx950 device is available");
  HIP_TRY(fwdk::rmsnorm(DType(dtype), x, (const float*)w, y, nullptr, rows, hidden, eps, false,
                        (hipStream_t)hip_stream));
  return FWD_OK;
}

int fwd_moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t norm_topk, int32_t* idx, float* w,
                  void* hip_stream) {
  if (T < 0 || E <= 0 || E > fwdk::kMoeMaxExperts || k < 1 || k > std::min(fwdk::kMoeMaxTopK, (int)E))
    return fail(FWD_E_ARG, "need T >= 0, 1 <= E <= 256 and 1 <= k <= min(8, E)");
  if (norm_topk != 0 && norm_topk != 1) return fail(FWD_E_ARG, "norm_topk must be 0 or 1");
  if (T == 0) return FWD_OK;
  if (!logits || !idx || !w) return fail(FWD_E_ARG, "NULL buffer");
  if (!device_is_gfx950()) return fail(FWD_E_UNAVAILABLE, "no gfx950 device is available");
  HIP_TRY(fwdk::moe_route(logits, T, E, k, norm_topk != 0, idx, w, (hipStream_t)hip_stream));
  return FWD_OK;
}

int fwd_set_timing(fwd_model* m, int32_t enable) {
  if (!m) return fail(FWD_E_ARG, "model is NULL");
  m->timing = enable != 0;
  m->marks.clear();
  m->events_used = 0;
  for (int k = 0; k < FWD_KERNEL_CLASSES; ++k) {
    m->class_ms[k] = 0.0;
    m->class_n[k] = 0;
  }
  return FWD_OK;
}

int fwd_get_timing(const fwd_model* m, int32_t kernel_class, double* total_ms, int64_t* launches) {
  if (!m || kernel_class < 0 || kernel_class >= FWD_KERNEL_CLASSES) return fail(FWD_E_ARG, "bad model or class");
  if (total_ms) *total_ms = m->class_ms[kernel_class];
  if (launches) *launches = m->class_n[kernel_class];
  return FWD_OK;
}

void fwd_destroy(fwd_model* m) { delete m; }

}  // extern "C"
