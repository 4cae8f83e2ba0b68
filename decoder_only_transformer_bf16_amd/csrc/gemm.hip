// Projections Y = X·Wᵀ ("N9 · metalgemm", Theorem 1: X [P, in], W [out, in],
// both row-major, fp32 accumulation) with the fused epilogues of the forward pass:
// plain fp32 store (+ final-logit softcap, "pegainfer issue #878"), the tied head with
// the per-position argmax, residual add, SwiGLU, and RoPE on the query/key heads
// ("N7 · model/forward-parity", intro and Theorem 1).
//
// bf16 path: CDNA4 MFMA v_mfma_f32_32x32x16_bf16 on operands staged through LDS by
// buffer->LDS loads: a two-group ping-pong kernel with 256 x 256 tiles for large
// problems (K-tiled operands: 32-wide K slices in four LDS stages; row-major ones:
// 64-wide slices in two), a 128 x 128 software-pipelined kernel for small ones (with an
// optional split of K over workgroups), and a split-K 16x16x32 kernel for few rows.
// f32 path: v_mfma_f32_32x32x2_f32 on 64 x 64 tiles through LDS (the fp32 configuration is tiny).
#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace fwdk {
namespace {

// ------------------------------------------------------------------ epilogues
// Every epilogue receives pairs of accumulator values (v0 at packed column c,
// v1 at packed column c + C) of one output row. ok0 / ok1 flag columns < N.
// batch() takes R rows of one column pair at once (row[q] < 0: skip); the default
// loops over pair(). Epilogues that read memory override it to issue every load
// before the first store (the output may alias the input, so the compiler could
// not reorder them itself).
template <class E, int R>
__device__ __forceinline__ void batch_pairs(const E& e, const int (&row)[R], int c, const float (&v0)[R],
                                            const float (&v1)[R], bool ok0, bool ok1) {
#pragma unroll
  for (int q = 0; q < R; ++q)
    if (row[q] >= 0) e.pair(row[q], c, v0[q], v1[q], ok0, ok1);
}

template <int C>
struct EpiStore {
  float* Y;
  int64_t ldy;
  float cap;  // 0 = off
  __device__ __forceinline__ float apply(float v) const {
    if (cap > 0.f) {
      // c * tanh(v / c) with tanh(y) = sign(y) (1 - e^{-2|y|}) / (1 + e^{-2|y|})
      const float y = fabsf(v) * fast_rcp(cap);
      const float e = fast_exp2(-2.f * kLog2e * y);
      const float t = (1.f - e) * fast_rcp(1.f + e);
      return copysignf(cap * t, v);
    }
    return v;
  }
  __device__ __forceinline__ void pair(int row, int c, float v0, float v1, bool ok0, bool ok1) const {
    float* y = Y + (int64_t)row * ldy + c;
    if (ok0) y[0] = apply(v0);
    if (ok1) y[C] = apply(v1);
  }
  template <int R>
  __device__ __forceinline__ void batch(const int (&row)[R], int c, const float (&v0)[R], const float (&v1)[R],
                                        bool ok0, bool ok1) const {
    batch_pairs(*this, row, c, v0, v1, ok0, ok1);
  }
};

// Tied LM head with the per-position argmax folded in ("N7 · model/forward-parity",
// Theorem 1: per-position argmax; "pegainfer issue #878", Acceptance Criteria: lowest
// index on ties, non-finite logits fail the call). Logits (after the optional softcap)
// are stored only when Y is set. Each lane keeps, per row, its best value and column;
// it meets its columns in increasing order, so a strict comparison keeps the lowest
// column among equal values. A running sum of v * 0 turns NaN as soon as any value is
// infinite or NaN. write_tile then encodes each row's best as one 64-bit key that
// orders by value first and by lower column second (the value's bits made monotone as
// an unsigned integer, -0 counted as +0 since the two compare equal; the low word the
// complement of the column), reduces the keys across lanes and stores one per (row,
// column chunk) into part[row * nchunk + chunk]; argmax_partials_kernel reduces the
// chunks.
template <int C>
struct EpiHead {
  float* Y;  // optional [M, ldy] fp32 logits
  int64_t ldy;
  float cap;  // 0 = off
  uint64_t* part;
  int nchunk;
  int* flag;  // set to 1 when a logit is not finite
  static __device__ __forceinline__ uint64_t key(float v, int col) {
    uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)col;
  }
  // Rows rtile .. rtile + 31 (wave-uniform) hold every row of the batch. Logit stores are
  // 4-byte buffer stores relative to that band; rows past M and columns past N get an
  // out-of-range offset, which the hardware drops, and the comparisons use selects, so
  // the batch has no per-element branches.
  template <int R>
  __device__ __forceinline__ void batch_best(const int (&row)[R], int c, const float (&v0)[R], const float (&v1)[R],
                                             bool ok0, bool ok1, float (&bv)[R], int (&bi)[R], float& chk,
                                             int rtile) const {
    if (cap > 0.f) best_rows<true>(row, c, v0, v1, ok0, ok1, bv, bi, chk, rtile);
    else best_rows<false>(row, c, v0, v1, ok0, ok1, bv, bi, chk, rtile);
  }
  template <bool CAP, int R>
  __device__ __forceinline__ void best_rows(const int (&row)[R], int c, const float (&v0)[R], const float (&v1)[R],
                                            bool ok0, bool ok1, float (&bv)[R], int (&bi)[R], float& chk,
                                            int rtile) const {
    const EpiStore<C> st{Y, ldy, cap};
    // (without Y: a null range, never stored through)
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(Y ? Y + (int64_t)rtile * ldy : nullptr, Y ? (int64_t)32 * ldy * 4 : 0);
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const bool u0 = row[q] >= 0 && ok0, u1 = row[q] >= 0 && ok1;
      const float a = CAP ? st.apply(v0[q]) : v0[q], b = CAP ? st.apply(v1[q]) : v1[q];
      if (Y) {
        const uint32_t off = ((uint32_t)(row[q] - rtile) * (uint32_t)ldy + (uint32_t)c) * 4u;  // (used if u0 / u1)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), ry, (int)(u0 ? off : 0x80000000u), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(b), ry, (int)(u1 ? off + 4u * C : 0x80000000u), 0, 0);
      }
      chk = fmaf(u0 ? a : 0.f, 0.f, chk);
      chk = fmaf(u1 ? b : 0.f, 0.f, chk);
      const float a2 = u0 ? a : -INFINITY, b2 = u1 ? b : -INFINITY;
      const bool ga = a2 > bv[q];
      bv[q] = ga ? a2 : bv[q];
      bi[q] = ga ? c : bi[q];
      const bool gb = b2 > bv[q];
      bv[q] = gb ? b2 : bv[q];
      bi[q] = gb ? c + C : bi[q];
    }
  }
};

// Epilogues with kInit = true take the residual into the accumulators before the K loop
// (init_acc): the tile's residual loads then travel with the first operand loads, and
// the epilogue only stores.
template <class E, class = void>
struct kInitAcc : std::false_type {};
template <class E>
struct kInitAcc<E, std::void_t<decltype(E::kInit)>> : std::true_type {};

// xout = xin + X·Wᵀ for the tiled kernels: the accumulators start from xin (init_acc),
// the epilogue stores them.
template <int C>
struct EpiResidualInit {
  static constexpr bool kInit = true;
  const float* xin;
  float* xout;
  int64_t ld;
  template <int R>
  __device__ __forceinline__ void batch(const int (&row)[R], int c, const float (&v0)[R], const float (&v1)[R],
                                        bool ok0, bool ok1) const {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      if (row[q] < 0) continue;
      float* y = xout + (int64_t)row[q] * ld + c;
      if (ok0) y[0] = v0[q];
      if (ok1) y[C] = v1[q];
    }
  }
};

template <class E, class = void>
struct kHasBest : std::false_type {};
template <class E>
struct kHasBest<E, std::void_t<decltype(&E::template batch_best<16>)>> : std::true_type {};

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// The 32 lanes of each half-wavefront hold keys of the same 16 rows (register q of
// the 32x32 accumulator layout) for different columns. Four exchange steps halve the
// rows each lane keeps (the lane keeps the half its bit selects and receives the
// partner's keys of that half), a fifth combines the last pair, so lane l ends with
// the maximum over all 32 lanes of row q = (l >> 1) & 15.
__device__ __forceinline__ uint64_t reduce_rows16(uint64_t (&k)[16], int lane) {
#pragma unroll
  for (int n = 8; n >= 1; n >>= 1) {
    // all ones where this lane keeps the upper half (lane bit 16, 8, 4, 2 for n = 8, 4, 2, 1);
    // selected by masks rather than by index so that k stays in registers
    const uint64_t m = (lane & (2 * n)) ? ~0ull : 0ull;
#pragma unroll
    for (int q = 0; q < n; ++q) {
      const uint64_t lo = k[q], up = k[q + n];
      const uint64_t send = (lo & m) | (up & ~m), keep = (up & m) | (lo & ~m);
      k[q] = max_u64(keep, shfl_xor_u64(send, 2 * n));
    }
  }
  return max_u64(k[0], shfl_xor_u64(k[0], 1));
}

template <int C>
struct EpiResidual {
  const float* xin;
  float* xout;
  int64_t ld;
  float* ssq = nullptr;  // optional [groups][kSkinnyRows]: per 64-column group, sum of squares of each stored row
  // Same as batch(), and sq[q] = the sum of squares of the (up to two) values stored in row q.
  template <int R>
  __device__ __forceinline__ void batch_sq(const int (&row)[R], int c, const float (&v0)[R], const float (&v1)[R],
                                           bool ok0, bool ok1, float (&sq)[R]) const {
    float a[R], b[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int64_t i = (int64_t)(row[q] < 0 ? 0 : row[q]) * ld + c;
      a[q] = (row[q] >= 0 && ok0) ? xin[i] : 0.f;
      b[q] = (row[q] >= 0 && ok1) ? xin[i + C] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      sq[q] = 0.f;
      if (row[q] < 0) continue;
      const int64_t i = (int64_t)row[q] * ld + c;
      const float x0 = a[q] + v0[q], x1 = b[q] + v1[q];
      if (ok0) {
        xout[i] = x0;
        sq[q] = x0 * x0;
      }
      if (ok1) {
        xout[i + C] = x1;
        sq[q] += x1 * x1;
      }
    }
  }
  __device__ __forceinline__ void pair(int row, int c, float v0, float v1, bool ok0, bool ok1) const {
    const int64_t i = (int64_t)row * ld + c;
    if (ok0) xout[i] = xin[i] + v0;
    if (ok1) xout[i + C] = xin[i + C] + v1;
  }
  template <int R>
  __device__ __forceinline__ void batch(const int (&row)[R], int c, const float (&v0)[R], const float (&v1)[R],
                                        bool ok0, bool ok1) const {
    float a[R], b[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {  // all loads first
      const int64_t i = (int64_t)(row[q] < 0 ? 0 : row[q]) * ld + c;
      a[q] = (row[q] >= 0 && ok0) ? xin[i] : 0.f;
      b[q] = (row[q] >= 0 && ok1) ? xin[i + C] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      if (row[q] < 0) continue;
      const int64_t i = (int64_t)row[q] * ld + c;
      if (ok0) xout[i] = a[q] + v0[q];
      if (ok1) xout[i + C] = b[q] + v1[q];
    }
  }
};

// ACT 0: silu(g) = g / (1 + e^-g) (SwiGLU); ACT 1: GELU in its tanh form,
// 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))), tanh(y) = 1 - 2 / (1 + e^{2y}).
template <int C, typename T, int ACT = 0>
struct EpiSwiGLU {
  T* a;
  int F;
  bool tiled;  // a in the K-tiled layout (it is the next GEMM's X operand)
  bool buf = false;  // the K-tiled output spans less than 2^31 bytes (32-bit buffer offsets)
  __device__ __forceinline__ void pair(int row, int c, float g, float u, bool ok0, bool) const {
    if (!ok0) return;
    const int f = (c / (2 * C)) * C + (c % C);
    Elem<T>::store(a + (tiled ? tiled_index(row, f, F) : (int64_t)row * F + f), act(g) * u);
  }
  static __device__ __forceinline__ float act(float g) {
    if constexpr (ACT == 0) {
      return g * fast_rcp(1.f + fast_exp2(-kLog2e * g));
    } else {
      const float y = 0.7978845608028654f * (g + 0.044715f * g * g * g);
      return 0.5f * g * (2.f - 2.f * fast_rcp(1.f + fast_exp2(2.f * kLog2e * y)));
    }
  }
  template <int R>
  __device__ __forceinline__ void batch(const int (&row)[R], int c, const float (&v0)[R], const float (&v1)[R],
                                        bool ok0, bool ok1) const {
    if constexpr (std::is_same<T, bf16_t>::value && C == 32 && R % 2 == 0) {
      if (tiled && buf) {
        // Adjacent lanes hold adjacent outputs f, f + 1 of the same R rows. Each pair
        // swaps half its results (even lanes give away rows R/2.., odd lanes rows
        // ..R/2) so that every lane stores two neighbouring bf16 outputs with one
        // 4-byte buffer store: the even lane rows q < R/2, the odd lane rows q + R/2.
        // Rows past the end get an offset outside the buffer, which the hardware
        // drops, so there is no branch per row. Selections between the two halves use
        // bit masks, not indices, so that the arrays stay in registers. (F is a
        // multiple of 32 for the K-tiled layout, so ok0 is the same for both lanes of
        // a pair.)
        if (!ok0) return;
        const uint32_t m = (threadIdx.x & 1) ? ~0u : 0u;
        const int f2 = ((c / (2 * C)) * C + (c % C)) & ~1;
        const uint32_t colpart = (uint32_t)(f2 >> 5) * 1024u + (uint32_t)(f2 & 31) * 2u;
        const uint32_t tilerow = (uint32_t)F * 32u;  // bytes per 16-row band of the K-tiled output
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a, 0x7FFFFFF0);
        uint32_t s[R];
#pragma unroll
        for (int q = 0; q < R; ++q) s[q] = __float_as_uint(act(v0[q]) * v1[q]);
#pragma unroll
        for (int q = 0; q < R / 2; ++q) {
          const uint32_t mine = s[q], other = s[q + R / 2];
          const uint32_t send = (mine & m) | (other & ~m);
          const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, true);  // partner
          const float lo = __uint_as_float((recv & m) | (mine & ~m));
          const float hi = __uint_as_float((other & m) | (recv & ~m));
          const int r = (int)(((uint32_t)row[q] & ~m) | ((uint32_t)row[q + R / 2] & m));
          const uint32_t off = r < 0 ? 0x80000000u : (uint32_t)(r >> 4) * tilerow + (uint32_t)(r & 15) * 64u + colpart;
          __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(lo, hi), rs, (int)off, 0, 0);
        }
        return;
      }
    }
    batch_pairs(*this, row, c, v0, v1, ok0, ok1);
  }
};

// KV: also store the rotated keys and the values in a KV cache (a separate
// instantiation, so that the plain prefill keeps the lean epilogue).
// bf16 stores of R rows of one column per lane into a row-major buffer (rs, `rowbytes`
// per row), where lanes 2k and 2k + 1 hold neighbouring columns of the same rows (the
// accumulator layouts of every kernel here): each pair swaps half its values by one DPP
// move so that every lane stores two neighbouring outputs with one 4-byte store (the
// even lane rows q < R/2, the odd lane rows q + R/2). `colbytes` is this lane's column
// in bytes. Rows past the end (row < 0) get an out-of-range offset, which the hardware
// drops; halves are selected by bit masks, not indices, so the arrays stay in registers.
template <int R>
__device__ __forceinline__ void store_pairs_rows(__amdgpu_buffer_rsrc_t rs, const int (&row)[R], uint32_t colbytes,
                                                 const float (&v)[R], uint32_t rowbytes) {
  static_assert(R % 2 == 0, "rows are split between the two lanes of a pair");
  const uint32_t m = (threadIdx.x & 1) ? ~0u : 0u;
  const uint32_t cb = colbytes & ~3u;
#pragma unroll
  for (int q = 0; q < R / 2; ++q) {
    const uint32_t mine = __float_as_uint(v[q]), other = __float_as_uint(v[q + R / 2]);
    const uint32_t send = (mine & m) | (other & ~m);
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    const float lo = __uint_as_float((recv & m) | (mine & ~m));
    const float hi = __uint_as_float((other & m) | (recv & ~m));
    const int r = (int)(((uint32_t)row[q] & ~m) | ((uint32_t)row[q + R / 2] & m));
    const uint32_t off = r < 0 ? 0x80000000u : (uint32_t)r * rowbytes + cb;
    __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(lo, hi), rs, (int)off, 0, 0);
  }
}

template <int C, typename T, bool KV, bool ROT = true>
struct EpiRope {
  T* qkv;  // [M, (Hq + 2 Hkv) D]: rotated q, rotated k, plain v, natural dim order
  const float2* cs;
  int Hq, Hkv, D, S, pos0;  // row r is sequence r / S at position pos0 + r % S
  T *kc, *vc;               // with KV: the cache [B, Hkv, Smax, D]
  int Smax;
  bool buf = false;  // bf16 qkv spans less than 2^31 bytes: pair-packed buffer stores (rotating path, no cache)
  __device__ __forceinline__ T* cache(T* base, int row, int head, int d) const {
    return base + (((int64_t)(row / S) * Hkv + head) * Smax + pos0 + row % S) * D + d;
  }
  template <int R>
  __device__ __forceinline__ void batch(const int (&row)[R], int c, const float (&v0)[R], const float (&v1)[R],
                                        bool ok0, bool ok1) const {
    const int qsz = Hq * D, ksz = Hkv * D;
    if (!ok0) return;
    if constexpr (std::is_same<T, bf16_t>::value && C == 32 && ROT && !KV && R % 2 == 0) {
      if (buf) {  // (sections start at multiples of 32 columns: both lanes of a pair take the same path)
        const uint32_t rowbytes = (uint32_t)(qsz + 2 * ksz) * 2u;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(qkv, 0x7FFFFFF0);
        if (c >= qsz + ksz) {
          store_pairs_rows(rs, row, (uint32_t)c * 2u, v0, rowbytes);
          if (ok1) store_pairs_rows(rs, row, (uint32_t)(c + C) * 2u, v1, rowbytes);
          return;
        }
        const int sec = c < qsz ? 0 : qsz;
        const int cc = c - sec;
        const int head = cc / D, pd = cc - head * D;
        const int k = (pd / (2 * C)) * C + (pd % C);
        float2 r[R];
#pragma unroll
        for (int q = 0; q < R; ++q)  // all table loads first
          r[q] = cs[(int64_t)((row[q] < 0 ? 0 : row[q]) % S + pos0) * (D / 2) + k];
        float a[R], b[R];
#pragma unroll
        for (int q = 0; q < R; ++q) {
          a[q] = v0[q] * r[q].x - v1[q] * r[q].y;
          b[q] = v0[q] * r[q].y + v1[q] * r[q].x;
        }
        const uint32_t col = (uint32_t)(sec + head * D + k) * 2u;
        store_pairs_rows(rs, row, col, a, rowbytes);
        store_pairs_rows(rs, row, col + (uint32_t)D, b, rowbytes);  // dim k + D/2: D/2 columns of 2 bytes
        return;
      }
    }
    if (c >= qsz + ksz) {  // value columns: plain stores
      batch_pairs(*this, row, c, v0, v1, ok0, ok1);
      return;
    }
    const int sec = c < qsz ? 0 : qsz;
    const int cc = c - sec;
    const int head = cc / D, pd = cc - head * D;
    const int k = (pd / (2 * C)) * C + (pd % C);  // rotation index in [0, D/2)
    if constexpr (!ROT) {  // projected q / k in natural order
#pragma unroll
      for (int q = 0; q < R; ++q) {
        if (row[q] < 0) continue;
        T* dst = qkv + (int64_t)row[q] * (qsz + 2 * ksz) + sec + head * D + k;
        Elem<T>::store(dst, v0[q]);
        Elem<T>::store(dst + D / 2, v1[q]);
      }
      return;
    }
    float2 r[R];
#pragma unroll
    for (int q = 0; q < R; ++q)  // all table loads first
      r[q] = cs[(int64_t)((row[q] < 0 ? 0 : row[q]) % S + pos0) * (D / 2) + k];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      if (row[q] < 0) continue;
      T* dst = qkv + (int64_t)row[q] * (qsz + 2 * ksz) + sec + head * D + k;
      const float a = v0[q] * r[q].x - v1[q] * r[q].y, b = v0[q] * r[q].y + v1[q] * r[q].x;
      Elem<T>::store(dst, a);
      Elem<T>::store(dst + D / 2, b);
      if (KV && sec) {
        T* kd = cache(kc, row[q], head, k);
        Elem<T>::store(kd, a);
        Elem<T>::store(kd + D / 2, b);
      }
    }
  }
  __device__ __forceinline__ void pair(int row, int c, float v0, float v1, bool ok0, bool ok1) const {
    if (!ok0) return;
    const int qsz = Hq * D, ksz = Hkv * D;
    T* out = qkv + (int64_t)row * (qsz + 2 * ksz);
    if (c < qsz + ksz) {
      const int t = row % S + pos0;
      const int sec = c < qsz ? 0 : qsz;
      const int cc = c - sec;
      const int head = cc / D, pd = cc - head * D;
      const int k = (pd / (2 * C)) * C + (pd % C);  // rotation index in [0, D/2)
      T* dst = out + sec + head * D + k;
      if constexpr (!ROT) {
        Elem<T>::store(dst, v0);
        Elem<T>::store(dst + D / 2, v1);
        return;
      }
      const float2 r = cs[(int64_t)t * (D / 2) + k];
      const float a = v0 * r.x - v1 * r.y, b = v0 * r.y + v1 * r.x;
      Elem<T>::store(dst, a);
      Elem<T>::store(dst + D / 2, b);
      if (KV && sec) {
        T* kd = cache(kc, row, head, k);
        Elem<T>::store(kd, a);
        Elem<T>::store(kd + D / 2, b);
      }
    } else {  // value columns are not permuted
      Elem<T>::store(out + c, v0);
      if (ok1) Elem<T>::store(out + c + C, v1);
      if (KV) {
        const int vcol = c - qsz - ksz, vh = vcol / D, vd = vcol - vh * D;
        Elem<T>::store(cache(vc, row, vh, vd), v0);
        if (ok1) {
          const int vcol1 = vcol + C, vh1 = vcol1 / D, vd1 = vcol1 - vh1 * D;
          Elem<T>::store(cache(vc, row, vh1, vd1), v1);
        }
      }
    }
  }
};

// ------------------------------------------------------------------ tile order
// Workgroups are handed to the 8 XCDs round-robin (id % 8). Remap so that each XCD
// works on a contiguous range of tiles, and walk that range in groups of GM tile
// rows so that concurrently running tiles share X rows and W rows in the XCD's L2.
__device__ __forceinline__ void tile_coords(int pid, int nTM, int nTN, int& tm, int& tn) {
  constexpr int kXcd = 8, GM = 8;
  const int total = nTM * nTN;
  const int q = total / kXcd, r = total % kXcd;
  const int x = pid % kXcd, local = pid / kXcd;
  const int lin = x * q + min(x, r) + local;
  const int group = lin / (GM * nTN);
  const int first = group * GM;
  const int gsz = min(nTM - first, GM);
  const int in = lin - group * GM * nTN;
  tm = first + in % gsz;
  tn = in / gsz;
}

// ------------------------------------------------------------------ bf16 MFMA kernel
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Physical 16-byte chunk of logical chunk c in row r of a tile whose rows hold BK
// bf16. gfx950's LDS serves a ds_read_b128 16 lanes (256 bytes, 64 banks) at a
// time; a fragment read touches one chunk column of 16 consecutive rows, so the
// swizzle must give those 16 rows distinct (row parity, chunk) bank slots. For
// 128-byte rows, c ^ (r & 7) ^ ((r >> 3) & 1) does (and 8 consecutive rows still
// land on 8 distinct chunks).
template <int BK>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (BK == 64) return c ^ (r & 7) ^ ((r >> 3) & 1);
  else return c ^ ((r >> 2) & 3);  // 64-byte rows: 16 rows -> (r & 3, chunk) distinct
}
template <int BK>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * BK + (swz<BK>(r, c) << 3);
}

// Global -> LDS copy of 1 KiB of a BK-wide K slice of a ROWS-row operand tile with
// buffer_load_dwordx4 ... lds (no VGPR staging): 64 lanes x 16 bytes. Lane l lands
// at byte 16 l of block `blk`, i.e. tile row blk * (64 / CH) + l / CH and physical
// chunk l % CH, so it fetches the logical chunk the swizzled layout keeps there.
// Row-major operands: row r of the tile starts at r * K. K-tiled operands (BK = 32):
// block `blk` of slice k0 is the 1 KiB tile (blk, k0 / 32) of the operand tile.
template <int BK, bool TILED>
__device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t rs, bf16_t* lds, int K, int k0, int blk, int lane) {
  constexpr int CH = BK / 8, RPB = 64 / CH;  // chunks per row, rows per 1 KiB block
  static_assert(!TILED || BK == 32, "the K-tiled layout has 32-wide tiles");
  const int row = blk * RPB + lane / CH;
  const int ch = swz<BK>(row, lane % CH);  // the swizzle is an involution
  uint32_t off;
  if constexpr (TILED) {
    off = (uint32_t)((blk * (K / 32) + k0 / 32) * 512 + (lane / CH) * 32 + ch * 8) * 2u;
  } else {
    const int kk = k0 + ch * 8;
    off = kk < K ? (uint32_t)(row * K + kk) * 2u : 0x80000000u;
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lds + blk * 512), 16, off, 0, 0, 0);
}

// The VGPR route: the same 1 KiB piece fetched into registers; put_block writes it
// to the LDS position the DMA route would have used (byte 16 l of the piece).
template <int BK>
__device__ __forceinline__ u32x4_t fetch_block(__amdgpu_buffer_rsrc_t rs, int K, int k0, int blk, int lane) {
  constexpr int CH = BK / 8, RPB = 64 / CH;
  const int row = blk * RPB + lane / CH;
  const int kk = k0 + swz<BK>(row, lane % CH) * 8;
  const uint32_t off = kk < K ? (uint32_t)(row * K + kk) * 2u : 0x80000000u;
  return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
}
__device__ __forceinline__ void put_block(bf16_t* lds, int blk, int lane, const u32x4_t& v) {
  *reinterpret_cast<u32x4_t*>(lds + blk * 512 + lane * 8) = v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// acc[i][j] of a wavefront whose sub-tile starts at (r0, c0) := xin at the positions the
// accumulator layout below gives its registers (zero outside M x N).
template <int TM, int TN, class Epi>
__device__ __forceinline__ void init_acc(const Epi& epi, floatx16_t (&acc)[TM][TN], int r0, int c0, int M, int N,
                                         int lane) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), col = c0 + j * 32 + (lane & 31);
        acc[i][j][r] = (row < M && col < N) ? epi.xin[(int64_t)row * epi.ld + col] : 0.f;
      }
}

// Accumulator layout of v_mfma_f32_32x32x16: register r of lane l holds row
// 8 (r / 4) + 4 (l / 32) + r % 4 and column l % 32 of the 32x32 sub-tile. Hands a
// wavefront's TM x TN sub-tiles (origin r0, c0) to the epilogue, 16 rows of one
// column pair at a time.
template <int TM, int TN, class Epi>
__device__ __forceinline__ void write_tile(const Epi& epi, const floatx16_t (&acc)[TM][TN], int r0, int c0, int M,
                                           int N, int lane) {
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float bv[16], chk = 0.f;  // (argmax epilogues) per-row best value and column, finiteness check
    int bi[16];
    if constexpr (kHasBest<Epi>::value) {
#pragma unroll
      for (int r = 0; r < 16; ++r) bv[r] = -INFINITY, bi[r] = 0x7FFFFFFF;
    }
#pragma unroll
    for (int jp = 0; jp < TN / 2; ++jp) {
      const int c = c0 + jp * 64 + lr;
      const bool ok0 = c < N, ok1 = c + 32 < N;
      int rows[16];
      float v0[16], v1[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
        rows[r] = row < M ? row : -1;
        v0[r] = acc[i][2 * jp][r];
        v1[r] = acc[i][2 * jp + 1][r];
      }
      if constexpr (kHasBest<Epi>::value) epi.batch_best(rows, c, v0, v1, ok0, ok1, bv, bi, chk, r0 + i * 32);
      else epi.batch(rows, c, v0, v1, ok0, ok1);
    }
    if constexpr (kHasBest<Epi>::value) {
      // one key per (row, chunk of the wavefront's TN * 32 columns)
      uint64_t keys[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) keys[r] = Epi::key(bv[r], bi[r]);
      const uint64_t k = reduce_rows16(keys, lane);
      const int q = (lane >> 1) & 15;
      const int row = r0 + i * 32 + 8 * (q >> 2) + 4 * lk + (q & 3);
      if ((lane & 1) == 0 && row < M && c0 < N) epi.part[(int64_t)row * epi.nchunk + c0 / (TN * 32)] = k;
      if (chk != chk) *epi.flag = 1;
    }
  }
}

// Tile configuration: BM x BN output tile, BK-wide K slices, STAGES LDS buffers,
// WM x WN wavefronts (each owning a (BM/WM) x (BN/WN) block of 32x32 MFMA tiles).
template <int BM_, int BN_, int BK_, int STAGES_, int WM_, int WN_, int OCC_ = 1, int BPOS_ = 1, int RPM_ = 2,
          int LSPAN_ = 0>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WM = WM_, WN = WN_;
  static constexpr int OCC = OCC_;    // workgroups per CU the register budget is sized for
  static constexpr int BPOS = BPOS_;  // the slice barrier precedes MFMA BPOS of the last sub-step
  static constexpr int RPM = RPM_;    // fragment reads issued after each MFMA
  // With two stages the refill of slice t + 1 must land before barrier t: its loads
  // go out over the first LSPAN MFMAs of slice t (default: half the slice).
  static constexpr int LSPAN = LSPAN_ > 0 ? LSPAN_ : (BK / 16) * (BM / WM / 32) * (BN / WN / 32) / 2;
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32, KS = BK / 16;
  static constexpr int LOADS_A = BM * (BK / 8) / 64 / NW;      // 1 KiB buffer loads per wave per slice
  static constexpr int LOADS = (BM + BN) * (BK / 8) / 64 / NW;
  static_assert(LOADS_A * NW * 64 == BM * (BK / 8) && LOADS * NW * 64 == (BM + BN) * (BK / 8), "load split");
  static constexpr int LDS_BYTES = STAGES * (BM + BN) * BK * 2;
  static_assert(LDS_BYTES * OCC <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2, "one buffer being read, one being filled");
  static_assert(TN % 2 == 0, "pair epilogues need an even number of 32-column sub-tiles");
  static_assert(KS % 2 == 0, "fragment register buffers alternate per sub-step");
  static_assert(BPOS >= 0 && BPOS + (TM + TN - 1) / RPM < TM * TN, "next-slice reads fit after the barrier");
};

// Fragment reads in the order the MFMAs of a sub-step consume them (MFMA x uses A
// tile x % TM and B tile x / TM): A0, B0, A1 .. A(TM-1), B1 .. B(TN-1). Index f < TM
// names A tile f, f >= TM names B tile f - TM.
template <int TM>
__device__ constexpr int need_frag(int n) {
  return n == 0 ? 0 : n == 1 ? TM : n <= TM ? n - 1 : n;
}

// Grouped launches: m-tile gm belongs to the last expert whose first tile is at or
// before it (so experts without rows are skipped). group_tile gives the tile's
// coordinates within that expert, the expert's first row and its row count, or false
// past the last expert's tiles.
__device__ __forceinline__ int group_expert(const GroupArgs& g, int gm) {
  int lo = 0, hi = g.E;  // mtile_start[lo] <= gm < mtile_start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.mtile_start[mid] <= gm) lo = mid;
    else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ bool group_tile(const GroupArgs& g, int block, int nTN, int& tm, int& tn, int& row0,
                                           int& rows) {
  const int gm = block / nTN;
  if (gm >= g.mtile_start[g.E]) return false;
  const int e = group_expert(g, gm);
  tm = gm - g.mtile_start[e];
  tn = block - gm * nTN;
  row0 = g.seg_start[e];
  rows = g.seg_count[e];
  return true;
}

// SPLIT: workgroup b takes tile b % tiles and K slices [kps (b / tiles), + kps) of it;
// the epilogue (a plain store) writes that split's fp32 partial tile to
// epi.Y + (b / tiles) M ldy, and a second launch adds the splits in order.
template <class C, class Epi, bool TILED, bool SPLIT = false>
__global__ __launch_bounds__(C::NT, C::OCC) void gemm_bf16_kernel(const bf16_t* __restrict__ X,
                                                                  const bf16_t* __restrict__ W, int M, int N, int K,
                                                                  Epi epi, int kps = 0) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, ST = C::STAGES, NW = C::NW;
  constexpr int WTM = C::WTM, WTN = C::WTN, TM = C::TM, TN = C::TN, KS = C::KS;
  constexpr int SLICE = (BM + BN) * BK;  // elements per stage
  __shared__ __attribute__((aligned(1024))) bf16_t lds[ST * SLICE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int nTM = (M + BM - 1) / BM, nTN = (N + BN - 1) / BN;
  int pid = blockIdx.x, kt0 = 0, nk = (K + BK - 1) / BK;
  if constexpr (SPLIT) {
    const int sp = pid / (nTM * nTN);
    pid -= sp * nTM * nTN;
    kt0 = sp * kps;
    nk = min(nk - kt0, kps);
    epi.Y += (int64_t)sp * M * epi.ldy;
  }
  int tm, tn;
  tile_coords(pid, nTM, nTN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  // (K-tiled operands are read in whole 16-row tiles: rows are padded to 16)
  const int mr = TILED ? (M + 15) / 16 * 16 : M, nr = TILED ? (N + 15) / 16 * 16 : N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(X + (int64_t)m0 * K, (int64_t)min(BM, mr - m0) * K * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(W + (int64_t)n0 * K, (int64_t)min(BN, nr - n0) * K * 2);

  floatx16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16_t{};
  if constexpr (kInitAcc<Epi>::value) init_acc<TM, TN>(epi, acc, m0 + wm * WTM, n0 + wn * WTN, M, N, lane);

  // Software pipeline over K slices; slice t lives in LDS buffer t % ST.
  // One barrier per slice, early in its last sub-step (whose fragments were read
  // during the previous sub-step): past barrier t every wavefront is done with
  // buffer (t - 1) % ST and slice t + 1 has landed. While computing slice t, the
  // wavefront refills buffer (t - 1) % ST with slice t + ST - 1, its LT
  // buffer->LDS loads spread evenly over the slice's MFMAs so the address and data
  // paths see a steady stream rather than a burst. Fragment reads for sub-step
  // kk + 1 (for the last sub-step: the next slice's first, after the barrier) go
  // out RPM per MFMA, front-loaded and in the order the MFMAs consume them, into
  // the register set the current MFMAs are not using.
  constexpr int MF = TM * TN, FR = TM + TN, LA = C::LOADS_A, LT = C::LOADS, RPM = C::RPM;
  constexpr int G = KS * MF;                   // MFMAs per slice
  constexpr int GB = (KS - 1) * MF + C::BPOS;  // the barrier sits before MFMA GB
  // load p of a refill follows MFMA (p * LS) / LT; LPRE of them precede the barrier.
  // With ST >= 3 the refill (slice t + ST - 1) may straddle the barrier; with two
  // stages it is slice t + 1 itself and must be issued before it.
  constexpr int LS = ST == 2 ? (C::LSPAN < GB ? C::LSPAN : GB) : G;
  constexpr int LPRE = (GB * LT + LS - 1) / LS < LT ? (GB * LT + LS - 1) / LS : LT;
  static_assert(ST > 2 || LPRE == LT, "two stages: every refill load precedes the barrier");
  constexpr int WAIT_STEADY = ST == 2 ? 0 : (ST - 3) * LT + LPRE;  // loads allowed in flight at a barrier
  static_assert(WAIT_STEADY < 64, "vmcnt range");
  auto issue_load = [&](int p, bf16_t* buf, int k0) {  // load p of this wave's share of one slice
    if (p < LA) load_block<BK, TILED>(ra, buf, K, k0, wave + p * NW, lane);
    else load_block<BK, TILED>(rb, buf + BM * BK, K, k0, wave + (p - LA) * NW, lane);
  };
#pragma unroll
  for (int q = 0; q < ST - 1; ++q)
    if (q < nk)
#pragma unroll
      for (int p = 0; p < LT; ++p) issue_load(p, lds + q * SLICE, (kt0 + q) * BK);
  const int lr = lane & 31, lk = lane >> 5;
  const int arow = wm * WTM + lr, brow = BM + wn * WTN + lr;  // tile rows this lane reads (+32 i / +32 j)
  bf16x8_t fa[2][TM], fb[2][TN];
  auto read_frag = [&](const bf16_t* base, int f, int kk, int buf) {
    if (f < TM) fa[buf][f] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(base + lds_off<BK>(arow + f * 32, kk * 2 + lk)));
    else fb[buf][f - TM] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(base + lds_off<BK>(brow + (f - TM) * 32, kk * 2 + lk)));
  };
  if (nk >= ST - 1) wait_vmcnt<(ST - 2) * LT>();  // slice 0 has landed
  else wait_vmcnt<0>();
  lds_barrier();
#pragma unroll
  for (int f = 0; f < FR; ++f) read_frag(lds, f, 0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    const bf16_t* cur = lds + (kt % ST) * SLICE;
    const bf16_t* nxt = lds + ((kt + 1) % ST) * SLICE;
    bf16_t* fill = lds + ((kt + ST - 1) % ST) * SLICE;
    const bool refill = kt + ST - 1 < nk;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int rb_ = kk & 1, wb = rb_ ^ 1;  // register buffers: read from rb_, prefetch into wb
#pragma unroll
      for (int x = 0; x < MF; ++x) {
        const int g = kk * MF + x;
        if (g == GB) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // all of slice kt is in registers
          if (refill) wait_vmcnt<WAIT_STEADY>();  // slice kt + 1 has landed
          else wait_vmcnt<0>();
          lds_barrier();
        }
        const int i = x % TM, j = x / TM;
        acc[i][j] = mfma_32x32x16_bf16(fa[rb_][i], fb[rb_][j], acc[i][j]);
        if (kk + 1 < KS) {
#pragma unroll
          for (int n = x * RPM; n < (x + 1) * RPM && n < FR; ++n) read_frag(cur, need_frag<TM>(n), kk + 1, wb);
        } else if (x >= C::BPOS) {
          const int y = x - C::BPOS;
          // (on the last slice this reads a stale but in-bounds buffer; never used)
#pragma unroll
          for (int n = y * RPM; n < (y + 1) * RPM && n < FR; ++n) read_frag(nxt, need_frag<TM>(n), 0, wb);
        }
        if (refill) {
#pragma unroll
          for (int p = 0; p < LT; ++p)
            if ((p * LS) / LT == g) issue_load(p, fill, (kt0 + kt + ST - 1) * BK);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  write_tile<TM, TN>(epi, acc, m0 + wm * WTM, n0 + wn * WTN, M, N, lane);
}

template <class C, class Epi, bool TILED = false>
hipError_t launch_cfg(const void* X, const void* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  const int grid = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<C, Epi, TILED>), dim3(grid), dim3(C::NT), 0, s, (const bf16_t*)X,
                     (const bf16_t*)W, M, N, K, epi);
  return hipGetLastError();
}

using CfgSmall = Cfg<128, 128, 32, 4, 2, 2>;
// 64 x 128 tiles (4 wavefronts of 32 x 64) for problems that give the 128 x 128 kernel
// fewer tiles than the chip has CUs (a 512-token prefill of a 576-wide model: 20 -> 40
// tiles; a 1024-row, 3840-wide product: 240 -> 480, K 15360 in 141-162 us instead of
// 146-175 us interleaved).
using CfgNarrow = Cfg<64, 128, 32, 4, 2, 2, 1, 0>;


// ------------------------------------------------------------------ ping-pong kernel
// 8 wavefronts, two per SIMD, in two groups of four (waves 0-3 and 4-7, one of
// each group per SIMD). The groups alternate between a compute phase (all MFMAs
// of one K slice on fragments already in registers) and a memory phase (the
// fragment reads of the next slice from LDS, plus a share of the buffer->LDS
// loads of a later slice), one workgroup barrier apart, so that each SIMD's
// matrix pipe is fed by one wavefront while the other waits on memory.
//   group 0: memory(s) in step 2s,     compute(s) in step 2s + 1
//   group 1: memory(s) in step 2s + 1, compute(s) in step 2s + 2
// Slice s lives in buffer s % ST; memory(s) also loads slice s + ST - 1 into
// buffer (s - 1) % ST, free since the barrier ending step 2s - 1. Every barrier
// ending an odd step has slice s + 1 landed (each wavefront waits for its own
// loads of it first), which memory(s + 1) of group 0 needs at step 2s + 2.
template <int BM_, int BN_, int BK_, int STAGES_, int WM_, int WN_, int RS_ = 0>
struct PPCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, WM = WM_, WN = WN_;
  static constexpr int RS = RS_;  // 0: buffer->LDS DMA; else slices staged in registers (VGPR route)
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32, KS = BK / 16;
  static constexpr int LOADS_A = BM * (BK / 8) / 64 / NW;
  static constexpr int LOADS = (BM + BN) * (BK / 8) / 64 / NW;
  static_assert(NW == 8, "two groups of four wavefronts");
  static_assert(LOADS_A * NW * 64 == BM * (BK / 8) && LOADS * NW * 64 == (BM + BN) * (BK / 8), "load split");
  static constexpr int LDS_BYTES = STAGES * (BM + BN) * BK * 2;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 3, "the lagging group still reads slice s - 1 while slice s + ST - 1 loads");
  static_assert(TN % 2 == 0, "pair epilogues need an even number of 32-column sub-tiles");
  static_assert((STAGES - 2) * LOADS < 64, "vmcnt range");
};

// SPLIT: workgroup b takes tile b % tiles over K slices [kps (b / tiles), + kps) and the
// epilogue (a plain store) writes that range's fp32 partial tile at epi.Y + (b / tiles) M ldy.
template <class C, class Epi, bool TILED, bool GROUPED = false, bool SPLIT = false>
__global__ __launch_bounds__(C::NT) void gemm_pp_kernel(const bf16_t* __restrict__ X, const bf16_t* __restrict__ W,
                                                        int M, int N, int K, Epi epi, GroupArgs grp = GroupArgs{},
                                                        int kps = 0) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, ST = C::STAGES, NW = C::NW;
  constexpr int WTM = C::WTM, WTN = C::WTN, TM = C::TM, TN = C::TN, KS = C::KS;
  constexpr int SLICE = (BM + BN) * BK, LA = C::LOADS_A, LT = C::LOADS, FR = TM + TN;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[ST * SLICE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int nTN = (N + BN - 1) / BN;
  static_assert(!(SPLIT && GROUPED) && (!SPLIT || C::RS == 0), "split ranges: plain tiles, buffer->LDS route");
  int tm, tn, row0 = 0, kt0 = 0;
  if constexpr (GROUPED) {
    if (!group_tile(grp, blockIdx.x, nTN, tm, tn, row0, M)) return;
    X += (int64_t)row0 * K;
    W += (int64_t)group_expert(grp, blockIdx.x / nTN) * grp.w_stride;
  } else {
    int pid = blockIdx.x;
    if constexpr (SPLIT) {
      const int tiles = ((M + BM - 1) / BM) * nTN, sp = pid / tiles;
      pid -= sp * tiles;
      kt0 = sp * kps;
      epi.Y += (int64_t)sp * M * epi.ldy;
    }
    tile_coords(pid, (M + BM - 1) / BM, nTN, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;
  // (K-tiled operands are read in whole 16-row tiles: rows are padded to 16)
  const int mr = TILED ? (M + 15) / 16 * 16 : M, nr = TILED ? (N + 15) / 16 * 16 : N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(X + (int64_t)m0 * K, (int64_t)min(BM, mr - m0) * K * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(W + (int64_t)n0 * K, (int64_t)min(BN, nr - n0) * K * 2);
  const int nk = SPLIT ? min((K + BK - 1) / BK - kt0, kps) : (K + BK - 1) / BK;  // slices of this workgroup
  auto issue_load = [&](int p, bf16_t* buf, int k0) {
    if (p < LA) load_block<BK, TILED>(ra, buf, K, k0, wave + p * NW, lane);
    else load_block<BK, TILED>(rb, buf + BM * BK, K, k0, wave + (p - LA) * NW, lane);
  };
  const int lr = lane & 31, lk = lane >> 5;
  const int arow = wm * WTM + lr, brow = BM + wn * WTN + lr;
  bf16x8_t fa[KS][TM], fb[KS][TN];
  auto read_slice = [&](const bf16_t* base) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int n = 0; n < FR; ++n) {
        const int f = need_frag<TM>(n);
        if (f < TM) fa[kk][f] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(base + lds_off<BK>(arow + f * 32, kk * 2 + lk)));
        else fb[kk][f - TM] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(base + lds_off<BK>(brow + (f - TM) * 32, kk * 2 + lk)));
      }
    }
  };

  floatx16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16_t{};
  if constexpr (kInitAcc<Epi>::value) init_acc<TM, TN>(epi, acc, row0 + m0 + wm * WTM, n0 + wn * WTN, row0 + M, N, lane);

  constexpr int RS = C::RS;
  u32x4_t stage[RS > 0 ? RS : 1][LT];  // VGPR route: slices in flight in registers
  auto fetch = [&](int slot, int k0) {
#pragma unroll
    for (int p = 0; p < LT; ++p)
      stage[slot][p] = p < LA ? fetch_block<BK>(ra, K, k0, wave + p * NW, lane)
                              : fetch_block<BK>(rb, K, k0, wave + (p - LA) * NW, lane);
  };
  auto put = [&](int slot, bf16_t* buf) {
#pragma unroll
    for (int p = 0; p < LT; ++p) {
      if (p < LA) put_block(buf, wave + p * NW, lane, stage[slot][p]);
      else put_block(buf + BM * BK, wave + (p - LA) * NW, lane, stage[slot][p]);
    }
  };
  auto compute = [&]() {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int x = 0; x < TM * TN; ++x) {
        const int i = x % TM, j = x / TM;
        acc[i][j] = mfma_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j]);
      }
  };

  if constexpr (RS == 0) {
#pragma unroll
    for (int q = 0; q < ST - 1; ++q)
      if (q < nk)
#pragma unroll
        for (int p = 0; p < LT; ++p) issue_load(p, lds + q * SLICE, (kt0 + q) * BK);
    if (nk >= ST - 1) wait_vmcnt<(ST - 2) * LT>();  // slice 0 has landed
    else wait_vmcnt<0>();
    lds_barrier();
    if (group == 1) lds_barrier();  // group 1 runs one step behind

    for (int s = 0; s < nk; ++s) {
      // memory(s)
      read_slice(lds + (s % ST) * SLICE);
      const bool refill = s + ST - 1 < nk;
      if (refill) {
        bf16_t* fill = lds + ((s + ST - 1) % ST) * SLICE;
#pragma unroll
        for (int p = 0; p < LT; ++p) issue_load(p, fill, (kt0 + s + ST - 1) * BK);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // fragments in registers, buffer s % ST read
      if (group == 1) {  // this barrier ends an odd step: slice s + 1 must have landed
        if (refill) wait_vmcnt<(ST - 2) * LT>();
        else wait_vmcnt<0>();
      }
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      compute();  // compute(s)
      __builtin_amdgcn_sched_barrier(0);
      if (group == 0) {  // this barrier ends an odd step
        if (refill) wait_vmcnt<(ST - 2) * LT>();
        else wait_vmcnt<0>();
      }
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // VGPR route: memory(s) writes slice s + 1 from registers into buffer (s + 1) % ST,
    // refills those registers with slice s + 1 + RS, then reads slice s's fragments.
    // Slice s + 1 is visible after the barrier ending step 2s + 1 (both groups have
    // written their parts and drained lgkmcnt); buffer (s + 1) % ST last held slice
    // s + 1 - ST, read by group 1 in step 2s + 3 - 2 ST < 2s.
    static_assert(ST >= 3, "buffer reuse distance");
    static_assert(RS == 1, "register slots are indexed by slice parity only when RS == 1");
    fetch(0, 0);
    wait_vmcnt<0>();
    put(0, lds);
#pragma unroll
    for (int q = 1; q <= RS; ++q)
      if (q < nk) fetch(q % RS, q * BK);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    lds_barrier();
    if (group == 1) lds_barrier();

    for (int s = 0; s < nk; ++s) {
      if (s + 1 < nk) {
        if (s + RS < nk) wait_vmcnt<(RS - 1) * LT>();  // slice s + 1 is in registers
        else wait_vmcnt<0>();
        put((s + 1) % RS, lds + ((s + 1) % ST) * SLICE);
        if (s + 1 + RS < nk) fetch((s + 1) % RS, (s + 1 + RS) * BK);
      }
      read_slice(lds + (s % ST) * SLICE);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      compute();
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (group == 0) lds_barrier();  // matches group 1's extra barrier

  write_tile<TM, TN>(epi, acc, row0 + m0 + wm * WTM, n0 + wn * WTN, row0 + M, N, lane);
}

// 8 wavefronts (two per SIMD) in ping-pong, 64 x 128 outputs each, four K slices of
// 32 in flight
using CfgBig = PPCfg<256, 256, 32, 4, 4, 2>;

template <class C, class Epi, bool TILED = false>
hipError_t launch_pp(const void* X, const void* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  const int grid = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((gemm_pp_kernel<C, Epi, TILED>), dim3(grid), dim3(C::NT), 0, s, (const bf16_t*)X,
                     (const bf16_t*)W, M, N, K, epi);
  return hipGetLastError();
}

// ------------------------------------------------------------------ ping-pong, 64-wide slices
// The same two-group alternation for row-major operands (the standalone product), with
// 64-wide K slices in two LDS stages of 64 KiB: each row then contributes one full
// 128-byte cache line per slice (eight rows per 1 KiB load), where a 32-wide slice
// reads half lines and costs the texture address unit twice the cycles per load. Group
// 0 issues every buffer->LDS load of slice s + 1 at the start of its memory(s) phase,
// into the buffer both groups finished reading by the barrier ending step 2s - 1, and
// waits for them before the barrier ending step 2s + 1, which group 0's memory(s + 1)
// needs; group 1 only reads fragments. Interleaved in one process on operands uniform in
// [-1, 1): 7.5% faster than the 32-wide kernel on [4096, 4096, 14336], 1% on
// [8192, 4096, 128256], bitwise equal (every accumulator takes the same MFMAs in the
// same K order). On K-tiled operands inside the forward (weights N(0, 0.02)) it was
// 5.8% slower per prefill (223.6 vs 211.2 ms interleaved, the down product 53.5 vs
// 47.2 ms): two steps of prefetch do not cover the memory latency there, where the
// 32-wide kernel keeps three slices in flight. K-tiled operands stay supported (two
// 32-wide sub-slices per slice, each laid out as in the 32-wide kernels).
template <int BM_, int BN_, int WM_, int WN_>
struct PP64Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, STAGES = 2, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32, KS = BK / 16;
  static constexpr int BLK_A = BM * BK / 512, BLK = (BM + BN) * BK / 512;  // 1 KiB blocks per slice
  static constexpr int LOADS = BLK / (NW / 2);                              // per group-0 wavefront
  static_assert(NW == 8, "two groups of four wavefronts");
  static_assert(LOADS * (NW / 2) == BLK && BM % 16 == 0 && BN % 16 == 0, "load split");
  static_assert(STAGES * (BM + BN) * BK * 2 <= 160 * 1024, "LDS budget");
  static_assert(TN % 2 == 0, "pair epilogues need an even number of 32-column sub-tiles");
  static_assert(LOADS < 64, "vmcnt range");
};

// LDS element offset of 8-element chunk c (0..7) of row r in a 64-wide slice region of R rows.
template <int R, bool TILED>
__device__ __forceinline__ int lds_off64(int r, int c) {
  if constexpr (TILED) return (c >> 2) * (R * 32) + r * 32 + (swz<32>(r, c & 3) << 3);
  else return lds_off<64>(r, c);
}

// 1 KiB block `blk` of a 64-wide slice (k0) of an R-row operand tile into its region.
// K-tiled: block (sub, rb) = (blk / (R / 16), blk % (R / 16)) is the 16 x 32 tile
// (rb, k0 / 32 + sub). Row-major: rows 8 blk .. 8 blk + 7, 128 bytes each.
template <int R, bool TILED>
__device__ __forceinline__ void load_block64(__amdgpu_buffer_rsrc_t rs, bf16_t* region, int K, int k0, int blk,
                                             int lane) {
  if constexpr (TILED) {
    const int sub = blk / (R / 16), rb = blk - sub * (R / 16);
    const int row = lane >> 2, ch = swz<32>(row, lane & 3);
    // (past the last K tile, when K is an odd number of 32-wide tiles: zeros)
    const uint32_t off = k0 / 32 + sub < K / 32
                             ? (uint32_t)((rb * (K / 32) + k0 / 32 + sub) * 512 + row * 32 + ch * 8) * 2u
                             : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(region + blk * 512), 16, off, 0, 0, 0);
  } else {
    load_block<64, false>(rs, region, K, k0, blk, lane);
  }
}

template <class C, class Epi, bool TILED, bool GROUPED = false>
__global__ __launch_bounds__(C::NT) void gemm_pp64_kernel(const bf16_t* __restrict__ X,
                                                          const bf16_t* __restrict__ W, int M, int N, int K, Epi epi,
                                                          GroupArgs grp = GroupArgs{}) {
  constexpr int BM = C::BM, BN = C::BN, BK = 64;
  constexpr int WTM = C::WTM, WTN = C::WTN, TM = C::TM, TN = C::TN, KS = C::KS;
  constexpr int SLICE = (BM + BN) * BK, FR = TM + TN, LT = C::LOADS;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[2 * SLICE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int nTN = (N + BN - 1) / BN;
  int tm, tn, row0 = 0;
  if constexpr (GROUPED) {
    if (!group_tile(grp, blockIdx.x, nTN, tm, tn, row0, M)) return;
    X += (int64_t)row0 * K;
    W += (int64_t)group_expert(grp, blockIdx.x / nTN) * grp.w_stride;
  } else {
    tile_coords(blockIdx.x, (M + BM - 1) / BM, nTN, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int mr = TILED ? (M + 15) / 16 * 16 : M, nr = TILED ? (N + 15) / 16 * 16 : N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(X + (int64_t)m0 * K, (int64_t)min(BM, mr - m0) * K * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(W + (int64_t)n0 * K, (int64_t)min(BN, nr - n0) * K * 2);
  const int nk = (K + BK - 1) / BK;
  // group 0 only: wave w (0..3) takes blocks w, w + 4, ... of the slice (A blocks first)
  auto issue_slice = [&](bf16_t* buf, int k0) {
#pragma unroll
    for (int p = 0; p < LT; ++p) {
      const int blk = wave + p * (C::NW / 2);
      if (blk < C::BLK_A) load_block64<BM, TILED>(ra, buf, K, k0, blk, lane);
      else load_block64<BN, TILED>(rb, buf + BM * BK, K, k0, blk - C::BLK_A, lane);
    }
  };
  const int lr = lane & 31, lk = lane >> 5;
  const int arow = wm * WTM + lr, brow = wn * WTN + lr;
  bf16x8_t fa[KS][TM], fb[KS][TN];
  auto read_slice = [&](const bf16_t* base) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int n = 0; n < FR; ++n) {
        const int f = need_frag<TM>(n);
        if (f < TM)
          fa[kk][f] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(base + lds_off64<BM, TILED>(arow + f * 32, kk * 2 + lk)));
        else
          fb[kk][f - TM] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
              base + BM * BK + lds_off64<BN, TILED>(brow + (f - TM) * 32, kk * 2 + lk)));
      }
    }
  };

  floatx16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16_t{};
  if constexpr (kInitAcc<Epi>::value) init_acc<TM, TN>(epi, acc, row0 + m0 + wm * WTM, n0 + wn * WTN, row0 + M, N, lane);

  if (group == 0) {
    issue_slice(lds, 0);
    wait_vmcnt<0>();
  }
  lds_barrier();
  if (group == 1) lds_barrier();  // group 1 runs one step behind

  for (int s = 0; s < nk; ++s) {
    // memory(s): fragments of slice s; group 0 also starts slice s + 1
    read_slice(lds + (s & 1) * SLICE);
    if (group == 0 && s + 1 < nk) issue_slice(lds + ((s + 1) & 1) * SLICE, (s + 1) * BK);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)  // compute(s)
#pragma unroll
      for (int x = 0; x < TM * TN; ++x) {
        const int i = x % TM, j = x / TM;
        acc[i][j] = mfma_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j]);
      }
    __builtin_amdgcn_sched_barrier(0);
    if (group == 0) wait_vmcnt<0>();  // this barrier ends an odd step: slice s + 1 has landed
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (group == 0) lds_barrier();  // matches group 1's extra barrier

  write_tile<TM, TN>(epi, acc, row0 + m0 + wm * WTM, n0 + wn * WTN, row0 + M, N, lane);
}

using Cfg64 = PP64Cfg<256, 256, 4, 2>;

// ------------------------------------------------------------------ split K
// Products with few output tiles and a long K (the Gemma-style sandwich down product,
// small standalone products) leave most CUs idle on the tiled kernels. There the K
// slices are cut into nsplit ranges: workgroup b computes tile b % tiles over range b / tiles and
// stores its fp32 partial tile into part[split][M][N]; splitk_sum_kernel then adds the
// partials of every output in split order and applies the softcap, so the result does
// not depend on timing and repeats bit for bit.
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* __restrict__ part, int nsplit, int M, int N,
                                                         float* __restrict__ Y, int64_t ldy, float cap) {
  const EpiStore<32> st{nullptr, 0, cap};
  const int64_t MN = (int64_t)M * N;
  if ((N & 3) == 0 && (ldy & 3) == 0) {  // four outputs of a row per thread, 16-byte accesses
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < MN / 4; q += (int64_t)gridDim.x * blockDim.x) {
      const int64_t e = 4 * q, r = e / N, c = e - r * N;
      float4 acc = *reinterpret_cast<const float4*>(part + e);
      for (int sp = 1; sp < nsplit; ++sp) {
        const float4 v = *reinterpret_cast<const float4*>(part + sp * MN + e);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
      *reinterpret_cast<float4*>(Y + r * ldy + c) = float4{st.apply(acc.x), st.apply(acc.y), st.apply(acc.z),
                                                           st.apply(acc.w)};
    }
    return;
  }
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < MN; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / N, c = e - r * N;
    float acc = part[e];
    for (int sp = 1; sp < nsplit; ++sp) acc += part[sp * MN + e];
    Y[r * ldy + c] = st.apply(acc);
  }
}

// nsplit ranges of kps 32-wide K slices each (nsplit = 1: no split).
struct DenseSplitPlan {
  int nsplit, kps;
  bool big = false;  // ranges of 256 x 256 ping-pong tiles (K-tiled operands), else of 128 x 128 tiles
};
DenseSplitPlan split_ranges(int K, int ns) {
  const int nk = (K + 31) / 32;
  ns = std::max(1, std::min(ns, nk));
  const int kps = (nk + ns - 1) / ns;
  return {(nk + kps - 1) / kps, kps};
}

template <class C, bool TILED>
hipError_t launch_split(const void* X, const void* W, int M, int N, int K, float* Y, int64_t ldy, float cap,
                        float* part, const DenseSplitPlan& p, hipStream_t s) {
  static_assert(C::BK == 32, "split ranges count 32-wide slices");
  const int tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<C, EpiStore<32>, TILED, true>), dim3(tiles * p.nsplit), dim3(C::NT), 0, s,
                     (const bf16_t*)X, (const bf16_t*)W, M, N, K, EpiStore<32>{part, N, 0.f}, p.kps);
  const int64_t work = ((N & 3) == 0 && (ldy & 3) == 0) ? (int64_t)M * N / 4 : (int64_t)M * N;
  const int blocks = (int)std::min<int64_t>((work + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_sum_kernel, dim3(blocks), dim3(256), 0, s, (const float*)part, p.nsplit, M, N, Y, ldy,
                     cap);
  return hipGetLastError();
}

// The same over ranges of 256 x 256 ping-pong tiles (K-tiled operands).
hipError_t launch_split_pp(const void* X, const void* W, int M, int N, int K, float* Y, int64_t ldy, float cap,
                           float* part, const DenseSplitPlan& p, hipStream_t s) {
  const int tiles = ((M + CfgBig::BM - 1) / CfgBig::BM) * ((N + CfgBig::BN - 1) / CfgBig::BN);
  hipLaunchKernelGGL((gemm_pp_kernel<CfgBig, EpiStore<32>, true, false, true>), dim3(tiles * p.nsplit),
                     dim3(CfgBig::NT), 0, s, (const bf16_t*)X, (const bf16_t*)W, M, N, K, EpiStore<32>{part, N, 0.f},
                     GroupArgs{}, p.kps);
  const int64_t work = ((N & 3) == 0 && (ldy & 3) == 0) ? (int64_t)M * N / 4 : (int64_t)M * N;
  const int blocks = (int)std::min<int64_t>((work + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_sum_kernel, dim3(blocks), dim3(256), 0, s, (const float*)part, p.nsplit, M, N, Y, ldy,
                     cap);
  return hipGetLastError();
}

template <class C, class Epi, bool TILED = false>
hipError_t launch_pp64(const void* X, const void* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  const int grid = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((gemm_pp64_kernel<C, Epi, TILED>), dim3(grid), dim3(C::NT), 0, s, (const bf16_t*)X,
                     (const bf16_t*)W, M, N, K, epi);
  return hipGetLastError();
}

// ------------------------------------------------------------------ f32 kernel
// fp32 products on the matrix cores (v_mfma_f32_32x32x2_f32): a 64 x 64 output tile
// per workgroup, one 32 x 32 quarter per wavefront, K slices of 16 through LDS. The
// tile returns through LDS so that the epilogue is called with the same (row, column
// pair) per thread as everywhere else: 4 rows x 2 pairs per thread.
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                                                      int M, int N, int K, Epi epi) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  __shared__ float Cs[64][64 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // this wavefront's 32 x 32 quarter of the tile
  const int nTN = (N + 63) / 64;
  const int m0 = (blockIdx.x / nTN) * 64, n0 = (blockIdx.x % nTN) * 64;
  floatx16_t acc = floatx16_t{};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int e = tid + p * 256, r = e >> 4, k = e & 15;
      As[k][r] = (m0 + r < M && k0 + k < K) ? X[(int64_t)(m0 + r) * K + k0 + k] : 0.f;
      Bs[k][r] = (n0 + r < N && k0 + k < K) ? W[(int64_t)(n0 + r) * K + k0 + k] : 0.f;
    }
    __syncthreads();
    // v_mfma_f32_32x32x2_f32: lane l holds row (A) / column (B) l % 32 at k = l / 32
#pragma unroll
    for (int kk = 0; kk < 16; kk += 2) {
      const float av = As[kk + (lane >> 5)][wm * 32 + (lane & 31)];
      const float bv = Bs[kk + (lane >> 5)][wn * 32 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
  for (int r = 0; r < 16; ++r) Cs[wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][wn * 32 + (lane & 31)] = acc[r];
  __syncthreads();
  const int tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int c = n0 + tx * 4 + 2 * jp;
      epi.pair(row, c, Cs[ty * 4 + i][tx * 4 + 2 * jp], Cs[ty * 4 + i][tx * 4 + 2 * jp + 1], c < N, c + 1 < N);
    }
  }
}

// ------------------------------------------------------------------ few rows (split K)
// Products with at most 64 rows (one token per sequence in a decode step) are bound by
// streaming W once from HBM, and a tiled kernel would start too few workgroups for
// that. Here a workgroup owns a 64-column group (four 16-column blocks, so that packed
// columns c and c + 32 meet in one thread for the pair epilogues) and a range of K
// tiles; its four wavefronts take every fourth K tile of the range. Each 16 x 32 tile
// of W (1 KiB, contiguous in the K-tiled layout) is one 16-byte load per lane and
// feeds one v_mfma_f32_16x16x32_bf16 per 16-row block of X (lane l holds row or
// column l % 16 and K elements 8 (l / 16) .. + 7 of both operands; the product's
// register r of lane l is row 4 (l / 16) + r, column l % 16). The wavefronts' sums
// meet in LDS. When K is split over several workgroups, each writes its fp32 partial
// tile, and the last to arrive at the group's counter adds the partials in split
// order (so the result does not depend on the arrival order), runs the epilogue and
// re-arms the counter.
constexpr int kSkUnroll = 8;     // K tiles per wavefront in flight
constexpr int kSkUnrollNorm = 4; // the same with the normalised X operand (three times the loads)
// Workgroups a launch aims for: about one resident round when X is normalised on the
// fly (three times the loads per K tile), half that for a bf16 X, whose splits otherwise
// spend more on the partial round trip than they save (interleaved decode steps of the
// Llama shape: O 0.453 -> 0.412 ms and down 0.907 -> 0.856 ms per step at 224; QKV with
// the fused norm 0.593 -> 0.697 ms, so it keeps 448).
constexpr int kSkTarget = 448;
constexpr int kSkMinTiles = 8;   // fewest K tiles per split
constexpr int kSkWaves = 4;      // wavefronts per workgroup, each on every kSkWaves-th K tile

template <class E, class = void>
struct kHasSq : std::false_type {};
template <class E>
struct kHasSq<E, std::void_t<decltype(&E::template batch_sq<2>)>> : std::true_type {};

struct SkinnyPlan {
  int groups, nsplit, kps;  // 64-column groups, K splits, K tiles per split
};
SkinnyPlan skinny_plan(int N, int K, int target) {
  SkinnyPlan p;
  const int KT = K / 32;
  p.groups = (N + 63) / 64;
  int ns = std::max(1, std::min((target + p.groups - 1) / p.groups, KT / kSkMinTiles));
  p.kps = (KT + ns - 1) / ns;
  p.nsplit = (KT + p.kps - 1) / p.kps;
  return p;
}
int skinny_blocks(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }  // 16-row blocks of the tile

// X operand of the few-row kernel: bf16 K-tiled (XTiled) or RMSNorm(x; w) built on the
// fly from fp32 rows (XNorm), whose per-row sums of squares a residual epilogue left
// as partials over 64-column groups.
struct XTiled {
  const bf16_t* X;
};
struct XNorm {
  const float* x;    // [M, K] fp32 row-major
  const float* w;    // [K] gains
  const float* ssq;  // [groups][kSkinnyRows] partial sums of squares of x's rows
  int groups;
  float eps;
};

template <int MB, class XOp, class Epi>
__global__ __launch_bounds__(64 * kSkWaves) void gemm_skinny_kernel(XOp xop, const bf16_t* __restrict__ W, int M,
                                                                   int N, int K,
                                                         int nsplit, int kps, float* __restrict__ part,
                                                         unsigned* __restrict__ count, float* __restrict__ ssq_out,
                                                         Epi epi) {
  constexpr bool kNorm = std::is_same<XOp, XNorm>::value;
  constexpr int RW = 16 * MB, LD = 64 + 4, U = kNorm ? kSkUnrollNorm / MB : kSkUnroll;
  constexpr int NW = kSkWaves, NT = 64 * NW;
  __shared__ float red[NW][RW][LD];
  __shared__ float rinv_s[RW];
  __shared__ int last;
  const int KT = K >> 5;
  const int g = blockIdx.x / nsplit, sp = blockIdx.x - g * nsplit;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kt0 = sp * kps, kt1 = min(KT, kt0 + kps);
  const int64_t npad = ((int64_t)N + 15) & ~(int64_t)15;  // W rows are padded to 16 (zeros)
  const int64_t wrows = npad - (int64_t)g * 64 < 64 ? npad - (int64_t)g * 64 : 64;
  const auto wrs = make_rsrc(W + (int64_t)g * 64 * K, wrows * K * 2);
  const uint32_t lo = (uint32_t)((lane & 15) * 32 + (lane >> 4) * 8) * 2u;

  __amdgpu_buffer_rsrc_t xrs, grs;
  float rinv[MB];
  if constexpr (kNorm) {
    // 1 / rms of each row from the partials, added in group order by every workgroup alike
    constexpr int SL = NT / RW;  // slices of the groups per row
    float* sums = &red[0][0][0];  // [SL][RW], free until the K loop ends
    const int r = threadIdx.x % RW, sl = threadIdx.x / RW;
    float sacc = 0.f;
    for (int j = sl; j < xop.groups; j += SL) sacc += xop.ssq[(int64_t)j * kSkinnyRows + r];
    sums[sl * RW + r] = sacc;
    __syncthreads();
    if (threadIdx.x < RW) {
      float t = 0.f;
      for (int j = 0; j < SL; ++j) t += sums[j * RW + threadIdx.x];
      rinv_s[threadIdx.x] = threadIdx.x < M ? fast_rsqrt(t / (float)K + xop.eps) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) rinv[rb] = rinv_s[rb * 16 + (lane & 15)];
    xrs = make_rsrc(xop.x, (int64_t)M * K * 4);  // rows past M read as zeros
    grs = make_rsrc(xop.w, (int64_t)K * 4);
  } else {
    xrs = make_rsrc(xop.X, (int64_t)((M + 15) & ~15) * K * 2);
  }

  floatx4_t acc[MB][4];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[rb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  for (int base = kt0 + wave; base < kt1; base += NW * U) {
    // every load of the batch first (past the range the offsets leave the buffers:
    // zeros), then conversions and products; the scheduling barrier keeps the
    // compiler from trading loads in flight for registers
    u32x4_t wv[U][4], xv[U][MB];
    u32x4_t xa[kNorm ? U : 1][kNorm ? MB : 1][2], ga[kNorm ? U : 1][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = base + NW * u;
      const bool ok = kt < kt1;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        wv[u][nb] = __builtin_amdgcn_raw_buffer_load_b128(wrs, ok ? (uint32_t)(nb * KT + kt) * 1024u + lo : 0x80000000u,
                                                          0, 0);
      if constexpr (kNorm) {
        // this lane's elements k .. k + 7 of row rb * 16 + lane % 16, and their gains
        const int k = kt * 32 + (lane >> 4) * 8;
        const uint32_t go = ok ? (uint32_t)k * 4u : 0x80000000u;
        ga[u][0] = __builtin_amdgcn_raw_buffer_load_b128(grs, go, 0, 0);
        ga[u][1] = __builtin_amdgcn_raw_buffer_load_b128(grs, go + 16u, 0, 0);
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
          const uint32_t xo = ok ? (uint32_t)((rb * 16 + (lane & 15)) * K + k) * 4u : 0x80000000u;
          xa[u][rb][0] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo, 0, 0);
          xa[u][rb][1] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 16u, 0, 0);
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
          xv[u][rb] = __builtin_amdgcn_raw_buffer_load_b128(
              xrs, ok ? (uint32_t)(rb * KT + kt) * 1024u + lo : 0x80000000u, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (kNorm) {  // x * gain * (1 / rms), rounded to bf16
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
          u32x4_t packed;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e)
              packed[2 * h + e] = pack_bf16x2(
                  __uint_as_float(xa[u][rb][h][2 * e]) * __uint_as_float(ga[u][h][2 * e]) * rinv[rb],
                  __uint_as_float(xa[u][rb][h][2 * e + 1]) * __uint_as_float(ga[u][h][2 * e + 1]) * rinv[rb]);
          xv[u][rb] = packed;
        }
      }
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[rb][nb] = mfma_16x16x32_bf16(as_bf16x8(xv[u][rb]), as_bf16x8(wv[u][nb]), acc[rb][nb]);
    }
  }

#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][rb * 16 + 4 * (lane >> 4) + r][nb * 16 + (lane & 15)] = acc[rb][nb][r];
  __syncthreads();

  // thread -> column pair (p, p + 32) and rows rq, rq + 8, ...
  constexpr int NR = NT / 32, R = RW / NR;  // row slots, rows per thread
  const int p = threadIdx.x & 31, rq = threadIdx.x >> 5;
  float v0[R], v1[R];
  int rows[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int row = rq + NR * q;
    v0[q] = 0.f;
    v1[q] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      v0[q] += red[w][row][p];
      v1[q] += red[w][row][p + 32];
    }
    rows[q] = row < M ? row : -1;
  }
  if (nsplit > 1) {
    // Partials travel as device-coherent (agent-scope) stores and loads, which the
    // XCDs' separate L2s do not keep; the counter is bumped only after every store of
    // the workgroup has completed, and read back before any partial is loaded. (A
    // release/acquire fence pair would write back and invalidate the whole L2 in
    // every workgroup instead.)
    float* mine = part + ((int64_t)g * nsplit + sp) * RW * 64;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      __hip_atomic_store(mine + (rq + NR * q) * 64 + p, v0[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(mine + (rq + NR * q) * 64 + p + 32, v1[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
      last = __hip_atomic_fetch_add(count + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(nsplit - 1);
    __syncthreads();
    if (!last) return;
    const float* all = part + (int64_t)g * nsplit * RW * 64;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      v0[q] = 0.f;
      v1[q] = 0.f;
    }
    constexpr int TB = 8;  // partials loaded per round trip, then added in split order
    for (int t0 = 0; t0 < nsplit; t0 += TB) {
      float a0[TB][R], a1[TB][R];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int t = t0 + u < nsplit ? t0 + u : t0;  // (surplus loads repeat t0, unused)
#pragma unroll
        for (int q = 0; q < R; ++q) {
          const float* at = all + (int64_t)t * RW * 64 + (rq + NR * q) * 64 + p;
          a0[u][q] = __hip_atomic_load(at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          a1[u][q] = __hip_atomic_load(at + 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int u = 0; u < TB; ++u)
        if (t0 + u < nsplit)
#pragma unroll
          for (int q = 0; q < R; ++q) {
            v0[q] += a0[u][q];
            v1[q] += a1[u][q];
          }
    }
    if (threadIdx.x == 0) __hip_atomic_store(count + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int c = g * 64 + p;
  if constexpr (kHasSq<Epi>::value) {
    if (ssq_out) {
      // per-row sums of squares of this group's stored values: 32 lanes per row, one store
      float sq[R];
      epi.batch_sq(rows, c, v0, v1, c < N, c + 32 < N, sq);
#pragma unroll
      for (int q = 0; q < R; ++q) {
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) sq[q] += __shfl_xor(sq[q], o, 32);
        if (p == 0) ssq_out[(int64_t)g * kSkinnyRows + rq + NR * q] = sq[q];
      }
      return;
    }
  }
  epi.batch(rows, c, v0, v1, c < N, c + 32 < N);
}

template <class XOp, class Epi>
hipError_t launch_skinny(const XOp& xop, const void* W, int M, int N, int K, const Epi& epi, const SplitK& sk,
                         float* ssq_out, hipStream_t s) {
  const SkinnyPlan p = skinny_plan(N, K, std::is_same<XOp, XNorm>::value ? kSkTarget : kSkTarget / 2);
  const int MB = skinny_blocks(M);
  if (p.nsplit > 1 && ((int64_t)p.groups * p.nsplit * 16 * MB * 64 > sk.part_floats || p.groups > sk.count_len))
    return hipErrorInvalidValue;  // workspace sized for fewer rows or outputs
  const dim3 grid(p.groups * p.nsplit), block(64 * kSkWaves);
  const bf16_t* w = (const bf16_t*)W;
  switch (MB) {
    case 1:
      hipLaunchKernelGGL((gemm_skinny_kernel<1, XOp, Epi>), grid, block, 0, s, xop, w, M, N, K, p.nsplit, p.kps,
                         sk.part, sk.count, ssq_out, epi);
      break;
    case 2:
      hipLaunchKernelGGL((gemm_skinny_kernel<2, XOp, Epi>), grid, block, 0, s, xop, w, M, N, K, p.nsplit, p.kps,
                         sk.part, sk.count, ssq_out, epi);
      break;
    default:
      hipLaunchKernelGGL((gemm_skinny_kernel<4, XOp, Epi>), grid, block, 0, s, xop, w, M, N, K, p.nsplit, p.kps,
                         sk.part, sk.count, ssq_out, epi);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ dispatch
// The tile kernels (no few-row path): 256 x 256 ping-pong tiles from 256 such tiles up
// (32-wide slices on K-tiled operands, 64-wide on row-major ones), 128 x 128 tiles from 256
// of those, 64 x 128 tiles below.
template <class Epi>
hipError_t launch_dense(const void* X, const void* W, int M, int N, int K, const Epi& epi, bool tiled, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (tiled && K % 32) return hipErrorInvalidValue;
  const int64_t big = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  const int64_t small = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  if (tiled) {
    if (big >= 256) return launch_pp<CfgBig, Epi, true>(X, W, M, N, K, epi, s);
    if (small >= 256) return launch_cfg<CfgSmall, Epi, true>(X, W, M, N, K, epi, s);
    return launch_cfg<CfgNarrow, Epi, true>(X, W, M, N, K, epi, s);
  }
  if (big >= 256) return launch_pp64<Cfg64, Epi, false>(X, W, M, N, K, epi, s);
  if (small >= 256) return launch_cfg<CfgSmall, Epi, false>(X, W, M, N, K, epi, s);
  return launch_cfg<CfgNarrow, Epi, false>(X, W, M, N, K, epi, s);
}

// Both operands row-major, or both K-tiled (K a multiple of 32).
template <class Epi>
hipError_t launch_bf16(const void* X, const void* W, int M, int N, int K, const Epi& epi, bool tiled, hipStream_t s,
                       const SplitK* sk, const RowNormX* nx = nullptr, float* ssq_out = nullptr) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (tiled && K % 32) return hipErrorInvalidValue;
  const bool few = tiled && sk && M <= kSkinnyRows;
  if ((nx || ssq_out) && !few) return hipErrorInvalidValue;  // only the few-row kernel fuses the norm
  if (few) {
    if (nx) return launch_skinny(XNorm{nx->x, nx->w, nx->ssq, nx->groups, nx->eps}, W, M, N, K, epi, *sk, ssq_out, s);
    return launch_skinny(XTiled{(const bf16_t*)X}, W, M, N, K, epi, *sk, ssq_out, s);
  }
  return launch_dense(X, W, M, N, K, epi, tiled, s);
}

template <class Epi>
hipError_t launch_f32(const void* X, const void* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int grid = ((M + 63) / 64) * ((N + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<Epi>), dim3(grid), dim3(256), 0, s, (const float*)X, (const float*)W, M, N,
                     K, epi);
  return hipGetLastError();
}

// out[row] = the column of the largest key among the row's nchunk partial keys (see
// EpiHead). One wavefront per row, four rows per workgroup.
__global__ __launch_bounds__(256) void argmax_partials_kernel(const uint64_t* __restrict__ part, int nchunk,
                                                             int rows, int32_t* __restrict__ out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint64_t* p = part + (int64_t)row * nchunk;
  uint64_t k = 0;
  for (int j = lane; j < nchunk; j += 64) k = max_u64(k, p[j]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) k = max_u64(k, shfl_xor_u64(k, o));
  if (lane == 0) out[row] = (int32_t)~(uint32_t)k;
}

}  // namespace

namespace {
template <class Epi>
hipError_t launch_grouped(const void* X, const void* W, int N, int K, const Epi& epi, const GroupArgs& g,
                          hipStream_t s) {
  static_assert(CfgBig::BM == kMoeTileRows, "the plan counts tiles of the grouped product's height");
  if (g.max_tiles <= 0 || N <= 0) return hipSuccess;
  if (K % 32 || g.E <= 0 || g.E > kMoeMaxExperts) return hipErrorInvalidValue;
  const int grid = g.max_tiles * ((N + CfgBig::BN - 1) / CfgBig::BN);
  hipLaunchKernelGGL((gemm_pp_kernel<CfgBig, Epi, true, true>), dim3(grid), dim3(CfgBig::NT), 0, s,
                     (const bf16_t*)X, (const bf16_t*)W, 0, N, K, epi, g);
  return hipGetLastError();
}
}  // namespace

hipError_t gemm_grouped_swiglu(const void* X, const void* W, void* a, int F, int K, const GroupArgs& g, int act,
                               hipStream_t s) {
  if (act == 1) return launch_grouped(X, W, 2 * F, K, EpiSwiGLU<32, bf16_t, 1>{(bf16_t*)a, F, true}, g, s);
  if (act != 0) return hipErrorInvalidValue;
  return launch_grouped(X, W, 2 * F, K, EpiSwiGLU<32, bf16_t>{(bf16_t*)a, F, true}, g, s);
}

hipError_t gemm_grouped_store(const void* X, const void* W, float* Y, int N, int K, const GroupArgs& g,
                              hipStream_t s) {
  return launch_grouped(X, W, N, K, EpiStore<32>{Y, N, 0.f}, g, s);
}

int64_t skinny_part_floats(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K < 32) return 0;
  const SkinnyPlan p = skinny_plan(N, K, kSkTarget);  // the larger of the two split counts
  return p.nsplit > 1 ? (int64_t)p.groups * p.nsplit * 16 * skinny_blocks(std::min(M, kSkinnyRows)) * 64 : 0;
}
int64_t skinny_groups(int N) { return N > 0 ? (N + 63) / 64 : 0; }

namespace {
// Which products to split, from interleaved timings: a long K (>= 8192) with fewer than
// 256 tiles of 128 x 128, on 128 x 128 tiles, the split count aiming at two workgroups
// per CU with at least 128 slices per range (a 1024 x 3840 product over K 15360, K-tiled:
// 2 ranges 133 us, 3 ranges 145 us, 4 ranges 149 us, against 165-174 us unsplit on
// 64 x 128 tiles). A split did not pay below that: the same product over K 4096 took
// 46 us unsplit and 50-80 us in 2-8 ranges; 256 x 1536 over K 1536 gained 1.5 us from 3
// ranges on 64 x 128 tiles, less than the standalone product's stream-ordered
// allocation of the partials costs (about 15 us per call).
constexpr int kCUs = 256;
DenseSplitPlan dense_split_plan(int M, int N, int K, bool tiled) {
  const DenseSplitPlan none{1, 0};
  if (M <= 0 || N <= 0 || K <= 0) return none;
  const int64_t small = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  const int nk = (K + 31) / 32;
  if (small >= 256 || nk < 256) return none;
  const int64_t big = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  if (tiled && big >= 16) {
    // About one round of 256 x 256 tiles over the ranges, each range at least 64 slices
    // (the Gemma3-style down product, 1024 x 3840 over K 15360: 60 tiles x 4 ranges,
    // 6.88 -> 5.60 ms over its 48 layers against 2 ranges of 128 x 128 tiles,
    // interleaved in one process)
    DenseSplitPlan p = split_ranges(K, (int)std::max<int64_t>(2, std::min<int64_t>(kCUs / big, nk / 64)));
    p.big = true;
    return p;
  }
  const int ns = (int)std::min<int64_t>(std::max<int64_t>((2 * kCUs + small / 2) / small, 2), nk / 128);
  return split_ranges(K, ns);
}
}  // namespace

// The static split-K scratch. In host code `scratch` names a host-side stand-in, not
// device memory: kernels get the address hipGetSymbolAddress returns for each device.
static __device__ __align__(256) float scratch[kStaticSplitFloats];

hipError_t static_split_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int64_t dense_split_floats(int M, int N, int K, bool tiled) {
  const DenseSplitPlan p = dense_split_plan(M, N, K, tiled);
  return p.nsplit > 1 ? (int64_t)p.nsplit * M * N : 0;
}

hipError_t gemm_store(DType dt, const void* X, const void* W, float* Y, int64_t ldy, int M, int N, int K,
                      float softcap, bool tiled, hipStream_t s, const SplitK* sk, const RowNormX* nx,
                      const DenseSplit* ds) {
  if (dt == DType::BF16 && ds && !nx && !(tiled && sk && M <= kSkinnyRows) && M > 0 && N > 0) {
    const DenseSplitPlan p = dense_split_plan(M, N, K, tiled);
    if (p.nsplit > 1) {
      if (tiled && K % 32) return hipErrorInvalidValue;
      if ((int64_t)p.nsplit * M * N > ds->part_floats || !ds->part) return hipErrorInvalidValue;
      if (p.big) return launch_split_pp(X, W, M, N, K, Y, ldy, softcap, ds->part, p, s);
      return tiled ? launch_split<CfgSmall, true>(X, W, M, N, K, Y, ldy, softcap, ds->part, p, s)
                   : launch_split<CfgSmall, false>(X, W, M, N, K, Y, ldy, softcap, ds->part, p, s);
    }
  }
  if (dt == DType::BF16) return launch_bf16(X, W, M, N, K, EpiStore<32>{Y, ldy, softcap}, tiled, s, sk, nx);
  if (tiled || nx) return hipErrorInvalidValue;
  return launch_f32(X, W, M, N, K, EpiStore<1>{Y, ldy, softcap}, s);
}

int64_t head_argmax_part_keys(int M, int N) {
  if (M <= 0 || N <= 0) return 0;
  return (int64_t)M * ((N + 63) / 64);  // the narrowest wavefront column span (64) bounds every config
}

hipError_t gemm_head_keys(const void* X, const void* W, float* Y, int64_t ldy, int M, int N, int K, float softcap,
                         uint64_t* part, int* nchunk, int* flag, hipStream_t s) {
  *nchunk = 0;
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % 32 || M <= kSkinnyRows || !part || !flag) return hipErrorInvalidValue;
  EpiHead<32> epi{Y, ldy, softcap, part, 0, flag};
  if ((int64_t)((M + 255) / 256) * ((N + 255) / 256) >= 256) {
    *nchunk = epi.nchunk = (N + CfgBig::WTN - 1) / CfgBig::WTN;
    return launch_pp<CfgBig, EpiHead<32>, true>(X, W, M, N, K, epi, s);
  }
  *nchunk = epi.nchunk = (N + CfgSmall::WTN - 1) / CfgSmall::WTN;
  return launch_cfg<CfgSmall, EpiHead<32>, true>(X, W, M, N, K, epi, s);
}

hipError_t argmax_keys(const uint64_t* part, int nchunk, int M, int32_t* out, hipStream_t s) {
  if (M <= 0 || nchunk <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_partials_kernel, dim3((M + 3) / 4), dim3(256), 0, s, part, nchunk, M, out);
  return hipGetLastError();
}

hipError_t gemm_residual(DType dt, const void* X, const void* W, const float* xin, float* xout, int M, int N,
                         int K, bool tiled, hipStream_t s, const SplitK* sk, float* ssq_out) {
  if (dt == DType::BF16) {
    if ((tiled && sk && M <= kSkinnyRows) || ssq_out)  // few rows: split-K kernel, residual added at the end
      return launch_bf16(X, W, M, N, K, EpiResidual<32>{xin, xout, N}, tiled, s, sk, nullptr, ssq_out);
    return launch_dense(X, W, M, N, K, EpiResidualInit<32>{xin, xout, N}, tiled, s);
  }
  if (tiled || ssq_out) return hipErrorInvalidValue;
  return launch_f32(X, W, M, N, K, EpiResidual<1>{xin, xout, N}, s);
}

hipError_t gemm_swiglu(DType dt, const void* X, const void* W, void* a, int M, int F, int K, bool tiled,
                       hipStream_t s, const SplitK* sk, const RowNormX* nx, int act) {
  if (act != 0 && act != 1) return hipErrorInvalidValue;
  if (dt == DType::BF16) {
    const bool fits = tiled && (int64_t)((M + 15) / 16 * 16) * F * 2 <= 0x7FFFFFF0LL;
    if (act == 1)
      return launch_bf16(X, W, M, 2 * F, K, EpiSwiGLU<32, bf16_t, 1>{(bf16_t*)a, F, tiled, fits}, tiled, s, sk, nx);
    return launch_bf16(X, W, M, 2 * F, K, EpiSwiGLU<32, bf16_t>{(bf16_t*)a, F, tiled, fits}, tiled, s, sk, nx);
  }
  if (tiled || nx) return hipErrorInvalidValue;
  if (act == 1) return launch_f32(X, W, M, 2 * F, K, EpiSwiGLU<1, float, 1>{(float*)a, F, false}, s);
  return launch_f32(X, W, M, 2 * F, K, EpiSwiGLU<1, float>{(float*)a, F, false}, s);
}

hipError_t gemm_qkv_rope(DType dt, const void* X, const void* W, const RopeArgs& r, int M, int K, bool tiled,
                         hipStream_t s, const SplitK* sk, const RowNormX* nx) {
  const int N = (r.Hq + 2 * r.Hkv) * r.D;
  if ((r.kc == nullptr) != (r.vc == nullptr) || (!r.rotate && r.kc)) return hipErrorInvalidValue;
  if (!r.rotate) {  // projections only (a QK-norm pass rotates afterwards)
    if (dt == DType::BF16)
      return launch_bf16(X, W, M, N, K,
                         EpiRope<32, bf16_t, false, false>{(bf16_t*)r.qkv, r.cs, r.Hq, r.Hkv, r.D, r.S, r.pos0,
                                                           nullptr, nullptr, 0},
                         tiled, s, sk, nx);
    if (tiled || nx) return hipErrorInvalidValue;
    return launch_f32(X, W, M, N, K,
                      EpiRope<1, float, false, false>{(float*)r.qkv, r.cs, r.Hq, r.Hkv, r.D, r.S, r.pos0, nullptr,
                                                      nullptr, 0},
                      s);
  }
  if (dt == DType::BF16) {
    if (r.kc)
      return launch_bf16(X, W, M, N, K,
                         EpiRope<32, bf16_t, true>{(bf16_t*)r.qkv, r.cs, r.Hq, r.Hkv, r.D, r.S, r.pos0, (bf16_t*)r.kc,
                                                   (bf16_t*)r.vc, r.Smax},
                         tiled, s, sk, nx);
    const bool fits = (int64_t)M * N * 2 <= 0x7FFFFFF0LL;
    return launch_bf16(
        X, W, M, N, K,
        EpiRope<32, bf16_t, false>{(bf16_t*)r.qkv, r.cs, r.Hq, r.Hkv, r.D, r.S, r.pos0, nullptr, nullptr, 0, fits},
        tiled, s, sk, nx);
  }
  if (tiled || nx) return hipErrorInvalidValue;
  if (r.kc)
    return launch_f32(X, W, M, N, K,
                      EpiRope<1, float, true>{(float*)r.qkv, r.cs, r.Hq, r.Hkv, r.D, r.S, r.pos0, (float*)r.kc,
                                              (float*)r.vc, r.Smax},
                      s);
  return launch_f32(X, W, M, N, K,
                    EpiRope<1, float, false>{(float*)r.qkv, r.cs, r.Hq, r.Hkv, r.D, r.S, r.pos0, nullptr, nullptr, 0},
                    s);
}

}  // namespace fwdk
