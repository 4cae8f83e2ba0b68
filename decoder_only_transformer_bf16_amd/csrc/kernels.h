// Host-side launchers of the gfx950 kernels. Every launcher only enqueues work on
// `stream` and returns the launch status; shapes are validated by the caller
// (the C-ABI layer) before any launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fwdk {

enum class DType { F32 = 0, BF16 = 1 };

// Pair distance of the fused pair epilogues (RoPE, SwiGLU): the two members of a
// pair sit `pair_chunk(dt)` packed columns apart. The weight packing of the runtime
// and the GEMM epilogues both follow it.
inline int pair_chunk(DType dt) { return dt == DType::BF16 ? 32 : 1; }

// ---- projections Y = X·Wᵀ (X [M, K], W [N, K]) ----
// `tiled`: X and W are both in the K-tiled layout of common.h (bf16 only, K a
// multiple of 32, rows padded to 16 and readable); otherwise both are row-major.
// `sk`: workspace of the split-K kernel for few rows (bf16 K-tiled, M <= kSkinnyRows,
// e.g. a decode step); without one every product takes the tiled kernels.
// Y fp32 [M, N] (ldy), optional softcap (0 = off).
constexpr int kSkinnyRows = 64;
struct SplitK {
  float* part;          // fp32 partial tiles, skinny_part_floats() of them
  unsigned* count;      // one arrival counter per 64-column group; zero between launches
  int64_t part_floats;  // capacity of part
  int64_t count_len;    // capacity of count
};
// Partial floats and counters a product of M rows, N outputs and K inputs needs.
int64_t skinny_part_floats(int M, int N, int K);
int64_t skinny_groups(int N);
// The few-row kernel can take X as RMSNorm(x; w) of fp32 rows instead of a bf16 operand
// (`nx`), given the per-row sums of squares that a residual product over the same rows
// left as partials (`ssq_out` of gemm_residual): ssq[g * kSkinnyRows + r] is row r's
// sum over output columns [64 g, 64 g + 64). Both need `sk` and M <= kSkinnyRows.
struct RowNormX {
  const float* x;    // [M, K] fp32 row-major
  const float* w;    // [K] gains
  const float* ssq;  // [groups][kSkinnyRows]
  int groups;        // ceil(K / 64)
  float eps;
};
// Products with few output tiles and a long K are cut into K ranges whose fp32 partial
// tiles a second launch adds in range order (deterministic) when `ds` holds room for
// dense_split_floats(M, N, K, tiled) partials (bf16 only; 0 floats: the product is not
// split). The plan depends on the operand layout: K-tiled products may take ranges of
// 256 x 256 tiles, row-major ones take 128 x 128 tiles.
struct DenseSplit {
  float* part;
  int64_t part_floats;
};
int64_t dense_split_floats(int M, int N, int K, bool tiled);
// For callers that cannot allocate: a static device array of kStaticSplitFloats floats
// that serves as the split-K partial buffer. static_split_scratch gives its address on
// the current device (looked up once per device). Calls that use it concurrently on one
// device race.
constexpr int64_t kStaticSplitFloats = (int64_t)4 << 20;  // 16 MiB
hipError_t static_split_scratch(float** ptr);
hipError_t gemm_store(DType dt, const void* X, const void* W, float* Y, int64_t ldy, int M, int N, int K,
                      float softcap, bool tiled, hipStream_t s, const SplitK* sk = nullptr,
                      const RowNormX* nx = nullptr, const DenseSplit* ds = nullptr);
// Tied LM head with the per-position argmax fused (bf16 K-tiled operands, K a multiple
// of 32, M > kSkinnyRows): logits as gemm_store when Y is set (Y may be null: argmax
// only), plus per row the best (value, lowest column) key of each column chunk in
// part[row * nchunk + chunk] (head_argmax_part_keys(M, N) keys bound the size);
// *flag = 1 if any logit is not finite. argmax_keys then reduces the chunks: out[r] =
// argmax over the N logits of row r, lowest index on ties.
int64_t head_argmax_part_keys(int M, int N);
hipError_t gemm_head_keys(const void* X, const void* W, float* Y, int64_t ldy, int M, int N, int K, float softcap,
                         uint64_t* part, int* nchunk, int* flag, hipStream_t s);
hipError_t argmax_keys(const uint64_t* part, int nchunk, int M, int32_t* out, hipStream_t s);
// xout[M, N] = xin + X·Wᵀ (fp32 residual stream, row stride N; xin may equal xout).
hipError_t gemm_residual(DType dt, const void* X, const void* W, const float* xin, float* xout, int M, int N,
                         int K, bool tiled, hipStream_t s, const SplitK* sk = nullptr, float* ssq_out = nullptr);
// a[M, F] = silu(g) * u with W packed as interleaved gate/up chunks (N = 2F); with
// `tiled`, a is written K-tiled too (it is the down projection's X).
// act 0: silu(g) (SwiGLU); 1: GELU in its tanh form.
hipError_t gemm_swiglu(DType dt, const void* X, const void* W, void* a, int M, int F, int K, bool tiled,
                       hipStream_t s, const SplitK* sk = nullptr, const RowNormX* nx = nullptr, int act = 0);
// QKV projection with RoPE on q and k; N = (Hq + 2 Hkv) D with packed q/k rows.
// Writes qkv [M, (Hq + 2 Hkv) D]: rotated q heads, rotated k heads, then the value
// heads, each in natural dim order. Rows are b * S + t (t = position).
struct RopeArgs {
  void* qkv;
  const float2* cs;  // [positions, D / 2] (cos, sin)
  int Hq, Hkv, D, S;
  int pos0;          // row r is at position pos0 + r % S (0 for a prefill)
  void* kc = nullptr;  // optional KV cache of the layer, K and V each [B, Hkv, Smax, D]:
  void* vc = nullptr;  // row r's rotated k and its v also go to sequence r / S, position pos0 + r % S
  int Smax = 0;
  bool rotate = true;  // false: q and k stored as projected (natural order), no cache stores
};
hipError_t gemm_qkv_rope(DType dt, const void* X, const void* W, const RopeArgs& r, int M, int K, bool tiled,
                         hipStream_t s, const SplitK* sk = nullptr, const RowNormX* nx = nullptr);

// ---- attention ----
struct AttnArgs {
  const void* q;
  const void* k;
  const void* vt;
  void* o;
  int64_t ldq, ldk, ldo;  // elements between consecutive tokens
  int ldvt;               // elements between consecutive dims of vt (>= S, multiple of 8)
  int B, S, Hq, Hkv, D, window;
  bool o_tiled;           // o K-tiled (bf16) with row width ldo = Hq * D, rows padded to 16
};
hipError_t attention(DType dt, const AttnArgs& a, hipStream_t s);
// vt[b, c, t] = src[(b * S + t) * ld + c] for c < C = Hkv * D (values transposed so that
// keys are contiguous); rows of vt are ldvt long (ldvt >= S rounded up to 8).
hipError_t transpose_v(DType dt, const void* src, int64_t ld, void* vt, int ldvt, int B, int S, int C,
                       hipStream_t s);
bool attention_supported(DType dt, int D);

// ---- KV cache (decode) ----
// Cache of one layer: K and V each [Bmax, Hkv, Smax, D] (dtype dt), positions contiguous,
// filled by gemm_qkv_rope (RopeArgs::kc / vc).
// One query per sequence: o[b, h, :] = softmax over cached keys j < len (and
// len - 1 - j < window when window > 0) of q·k_j / sqrt(D), times v_j. q rows b of
// the qkv buffer (stride ldq); o bf16 K-tiled (o_tiled) or row-major with stride ldo.
// Flash-decoding: key chunks of kDecodeChunk per workgroup, fp32 throughout, merged
// by rescaling. `part` holds B * Hq * ceil(len / kDecodeChunk) * (D + 2) floats;
// `count` B * Hkv arrival counters, zero between launches (each launch leaves them
// zero), used by the bf16 kernel that merges in place (without it a second kernel
// merges).
constexpr int kDecodeChunk = 256;
hipError_t attention_decode(DType dt, const void* q, int64_t ldq, const void* kc, const void* vc, int Smax, int len,
                            int B, int Hq, int Hkv, int D, int window, void* o, int64_t ldo, bool o_tiled,
                            float* part, unsigned* count, hipStream_t s);

// ---- row kernels ----
// y = RMSNorm(x; w) (w fp32 gains); y of dtype dt (K-tiled with `tiled`: bf16, H a
// multiple of 32); optional fp32 copy y32 (row-major).
hipError_t rmsnorm(DType dt, const float* x, const float* w, void* y, float* y32, int rows, int H, float eps,
                   bool tiled, hipStream_t s);
// xout = xin + RMSNorm(u; wpost); y = RMSNorm(xout; wnext) (dtype dt, K-tiled with
// `tiled`), y32 optional row-major fp32 copy of y.
hipError_t add_norm(DType dt, const float* xin, const float* u, const float* wpost, float* xout, const float* wnext,
                    void* y, float* y32, int rows, int H, float eps, bool tiled, hipStream_t s);
// x[t, :] = E[ids[t], :] * scale (fp32 out); E K-tiled with `tiled`.
hipError_t embed(DType dt, const int32_t* ids, const void* E, float* x, int rows, int H, float scale, bool tiled,
                 hipStream_t s);
// out[r] = argmax_v z[r, v] (lowest index on ties); *flag = 1 if any z is not finite.
// With `part` (room for part_pairs (value, column) pairs: 2 * part_pairs floats), the
// rows of a small batch are split into up to kArgmaxMaxSlices column slices whose
// partial results a second launch merges.
constexpr int kArgmaxMaxSlices = 64;
hipError_t argmax_rows(const float* z, int64_t ldz, int rows, int V, int32_t* out, int* flag, hipStream_t s,
                       float* part = nullptr, int64_t part_pairs = 0);

// ---- packing ----
// dst[map[r], :] = src[r, :] for r < rows; rows of `row_bytes` bytes (multiple of 4).
hipError_t copy_rows(void* dst, const void* src, const int32_t* map, int rows, int64_t row_bytes, hipStream_t s);
// K-tiled bf16 dst (rows padded to 16, cleared by the caller): row map[r] of dst =
// row r of the row-major [rows, K] src; K a multiple of 32.
hipError_t pack_tiled(void* dst, const void* src, const int32_t* map, int rows, int K, hipStream_t s);
// dst[i] = offset + float(src[i]) for a gain vector of dtype dt (offset 1: (1 + w) gains).
hipError_t gains_to_f32(DType dt, const void* src, float* dst, int n, float offset, hipStream_t s);

// ---- mixture of experts ----
// Routing, permutation and combination of the MoE feed-forward (moe.hip); the expert
// products are gemm_grouped_* below.
constexpr int kMoeMaxExperts = 256, kMoeMaxTopK = 8;
constexpr int kMoeTileRows = 256;  // rows per tile of the grouped products
// idx[t, j], w[t, j] (j < k): the k largest logits of row t of logits [T, E] (lowest
// index first on ties) and their softmax probabilities, renormalised when `norm`.
hipError_t moe_route(const float* logits, int T, int E, int k, bool norm, int32_t* idx, float* w, hipStream_t s);
// Device buffers of the permutation: chunk_count / chunk_base [moe_chunks(A) * E],
// total / seg_start / seg_count [E], mtile_start [E + 1], pos [A].
struct MoePlan {
  int *chunk_count, *chunk_base, *total, *seg_start, *seg_count, *mtile_start;
  int32_t* pos;
};
int64_t moe_chunks(int64_t A);
// For the A = T * k assignments idx[]: pos[i] = the row of assignment i in the
// expert-ordered matrix (expert segments 16-row aligned, token order inside), and per
// expert seg_start / seg_count and mtile_start (prefix of ceil(count / kMoeTileRows)).
hipError_t moe_plan(const int32_t* idx, int A, int E, const MoePlan& p, hipStream_t s);
// xp row pos[i] = n row i / k (bf16 K-tiled, row width H).
hipError_t moe_gather(const void* n, const int32_t* pos, int A, int k, int H, void* xp, hipStream_t s);
// out[t] = (xin[t] if xin) + sum_j w[t, j] * y[pos[t * k + j]] (fp32 rows of H).
hipError_t moe_combine(const float* y, const int32_t* pos, const float* w, int T, int k, int H, const float* xin,
                       float* out, hipStream_t s);
// Grouped products over the expert segments: X rows [seg_start[e], + seg_count[e]) times
// expert e's W (W + e * w_stride elements, K-tiled), one launch for all experts.
struct GroupArgs {
  const int *seg_start, *seg_count, *mtile_start;
  int E;
  int64_t w_stride;
  int max_tiles;  // upper bound of mtile_start[E] (sizes the grid)
};
// a[rows, F] = act(g) * u (K-tiled bf16, act as gemm_swiglu) with each expert's W packed
// as interleaved gate/up chunks.
hipError_t gemm_grouped_swiglu(const void* X, const void* W, void* a, int F, int K, const GroupArgs& g, int act,
                               hipStream_t s);
// Y[rows, N] fp32 (row stride N).
hipError_t gemm_grouped_store(const void* X, const void* W, float* Y, int N, int K, const GroupArgs& g, hipStream_t s);

// ---- QK-norm ----
// In place on qkv [rows, ld] (as gemm_qkv_rope writes it without rotation): every q head
// (gains gq [D]) and k head (gains gk [D]) is RMS-normalised over its D values, then
// rotated by RoPE at position pos0 + row % S (table cs [positions, D / 2]); with kc / vc
// (KV cache [B, Hkv, Smax, D]) the rotated k heads and the v heads of row r are stored
// for sequence r / S at that position.
struct QkNormArgs {
  void* qkv;
  int64_t ld;
  int Hq, Hkv, D, S, pos0;
  const float2* cs;
  const float *gq, *gk;
  float eps;
  void *kc, *vc;
  int Smax;
};
hipError_t qk_norm_rope(DType dt, const QkNormArgs& a, int rows, hipStream_t s);

}  // namespace fwdk
