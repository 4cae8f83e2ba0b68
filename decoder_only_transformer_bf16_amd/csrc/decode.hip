// Decode side of the forward pass: the per-layer KV cache and the one-query-per-
// sequence attention over it.
//
// A cached session prefills a prompt and then extends every sequence by one token per
// step, and a step must give the logits a cacheless forward over the whole sequence
// gives at its last position ("N7 · model/forward-parity", Theorem 1: the cached
// session prefill agrees with the cacheless forward; greedy continuation). The cache
// holds each layer's rotated keys and values, [B, Hkv, Smax, D] with positions
// contiguous, written by the QKV projection's epilogue.
//
// attention_decode is flash-decoding: the visible keys of a sequence are cut into
// chunks of kDecodeChunk, one workgroup per (chunk, kv head, sequence) computes the
// scores of all Hq / Hkv query heads that share the kv head, their chunk-local
// softmax statistics and the chunk's share of P·V, and the chunks are merged by
// rescaling to a common maximum. The work is HBM-bound: each cached key and value is
// read once per step.
//
// bf16 (at most 8 query heads per kv head): a wavefront reads its 64 keys and values
// as 1 KiB pieces, D / 8 lanes per key row (16 bytes each), so every load is
// contiguous; a lane's partial dot products are summed across its key's lanes with
// DPP moves, and its share of P·V stays in registers until one LDS reduction. The
// last workgroup of a (sequence, kv head) to finish merges the chunks itself. For
// 128-wide heads in groups of 1, 2, 4 or 8 a kernel with the group size fixed at
// compile time takes bf16 dot products (v_dot2) for the scores and for P·V, with the
// probabilities rounded to bf16; the other bf16 shapes accumulate fp32 products. The
// fp32 configuration (and wider groups) use a plain one-thread-per-key kernel and a
// separate merge kernel.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace fwdk {
namespace {

template <typename T> struct Vec16;  // 16 bytes of T widened to fp32
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[8]) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float (&v)[4]) {
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
};

constexpr int kMaxGroup = 16;  // query heads per kv head

// Workgroup (chunk c, kv head g, sequence b); one thread per key of the chunk.
// part[((b * Hq + h) * nsplit + c) * (D + 2) + ...] = (o[0..D), m, l) of the chunk, with
// o = sum_j 2^(s_j - m) v_j and l = sum_j 2^(s_j - m), s_j the score in log2 units.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_decode_kernel(const T* __restrict__ q, int64_t ldq,
                                                         const T* __restrict__ kc, const T* __restrict__ vc, int Smax,
                                                         int len, int Hq, int Hkv, int window, float* __restrict__ part,
                                                         int nsplit, float scale_log2) {
  constexpr int CH = kDecodeChunk;
  static_assert(CH == 256, "one thread per key");
  __shared__ float qs[kMaxGroup][D];
  __shared__ float ps[CH][kMaxGroup + 1];
  __shared__ float stat[2][kMaxGroup];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int G = Hq / Hkv;
  const int lo = window > 0 ? max(0, len - window) : 0;
  const int j0 = lo + c * CH, j1 = min(len, j0 + CH);
  const int64_t head = ((int64_t)b * Hkv + g) * Smax;

  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, d = i - h * D;
    qs[h][d] = Elem<T>::load(q + (int64_t)b * ldq + (int64_t)(g * G + h) * D + d);
  }
  __syncthreads();

  // scores, one key per thread
  {
    const int j = j0 + tid;
    float acc[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) acc[h] = 0.f;
    if (j < j1) {
      const T* krow = kc + (head + j) * D;
      constexpr int E = Vec16<T>::N;
      for (int d0 = 0; d0 < D; d0 += E) {
        float kv[E];
        Vec16<T>::load(krow + d0, kv);
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h < G) {
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h] = fmaf(qs[h][d0 + e], kv[e], acc[h]);
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
      if (h < G) ps[tid][h] = j < j1 ? acc[h] * scale_log2 : -INFINITY;
  }
  __syncthreads();

  // chunk max and sum per head; one wavefront per head
  const int wave = tid >> 6, lane = tid & 63;
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY;
    for (int i = lane; i < CH; i += 64) m = fmaxf(m, ps[i][h]);
    m = wave_max(m);
    float l = 0.f;
    for (int i = lane; i < CH; i += 64) {
      const float p = ps[i][h] == -INFINITY ? 0.f : exp2f(ps[i][h] - m);
      ps[i][h] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      stat[0][h] = m;
      stat[1][h] = l;
    }
  }
  __syncthreads();

  // P·V: thread per (head, dim)
  const int n = j1 - j0;
  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, d = i - h * D;
    const T* vcol = vc + head * D + (int64_t)j0 * D + d;
    float acc = 0.f;
    for (int k = 0; k < n; ++k) acc = fmaf(ps[k][h], Elem<T>::load(vcol + (int64_t)k * D), acc);
    float* out = part + (((int64_t)b * Hq + g * G + h) * nsplit + c) * (D + 2);
    out[d] = acc;
    if (d == 0) {
      out[D] = stat[0][h];
      out[D + 1] = stat[1][h];
    }
  }
}

// Merge the chunks of one (sequence, head): thread per dim.
template <typename T>
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(const float* __restrict__ part, int nsplit, int Hq,
                                                               int D, T* __restrict__ o, int64_t ldo, bool o_tiled) {
  const int bh = blockIdx.x, b = bh / Hq, h = bh - b * Hq;
  const float* p = part + (int64_t)bh * nsplit * (D + 2);
  float M = -INFINITY;
  for (int c = 0; c < nsplit; ++c) M = fmaxf(M, p[c * (D + 2) + D]);
  float L = 0.f;
  for (int c = 0; c < nsplit; ++c) L += p[c * (D + 2) + D + 1] * exp2f(p[c * (D + 2) + D] - M);
  const float inv = 1.f / L;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int c = 0; c < nsplit; ++c) acc += p[c * (D + 2) + d] * exp2f(p[c * (D + 2) + D] - M);
    const int col = h * D + d;
    Elem<T>::store(o + (o_tiled ? tiled_index(b, col, (int)ldo) : (int64_t)b * ldo + col), acc * inv);
  }
}


// ------------------------------------------------------------------ bf16 kernel
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct DecodeArgs {
  const bf16_t* q;
  int64_t ldq;
  const bf16_t *kc, *vc;
  int Smax, len, Hq, Hkv, window, nsplit;
  float scale_log2;
  float* part;       // [B, Hq, nsplit, D + 2]: chunk outputs (unnormalised), max, sum
  unsigned* count;   // [B, Hkv] arrival counters, zero between launches
  bf16_t* o;
  int64_t ldo;
  bool o_tiled;
};

// Workgroup (chunk c, kv head g, sequence b), 4 wavefronts x 64 keys. Lane l of a
// wavefront holds dims 8 (l % LPK) .. + 7 of key l / LPK of each 1 KiB piece.
template <int D, int GM>
__global__ __launch_bounds__(256) void attn_decode_bf16_kernel(DecodeArgs a) {
  constexpr int CH = kDecodeChunk, LPK = D / 8, KPL = 64 / LPK, NL = 64 / KPL;
  constexpr int NB = NL < 16 ? NL : 16;  // pieces per tensor in flight per lane
  constexpr int RS = GM * D + 4;         // row stride of the partial outputs (floats)
  static_assert(CH == 256 && D % 64 == 0 && D <= 256, "4 x 64 keys per chunk, D in {64, 128, 256}");
  __shared__ float ps[CH][GM + 1];
  __shared__ __align__(16) float ored[4 * KPL * RS];
  __shared__ float stat[2][GM];
  __shared__ int last;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane % LPK, kk = lane / LPK;
  const int G = a.Hq / a.Hkv;
  const int lo = a.window > 0 ? max(0, a.len - a.window) : 0;
  const int j0 = lo + c * CH, j1 = min(a.len, j0 + CH);
  const int64_t head = ((int64_t)b * a.Hkv + g) * a.Smax;
  // keys at or past j1 (including cache rows not written yet) read as zeros
  const auto krs = make_rsrc(a.kc + head * D, (int64_t)j1 * D * 2);
  const auto vrs = make_rsrc(a.vc + head * D, (int64_t)j1 * D * 2);
  auto piece = [&](int i) {  // byte offset of this lane's 16 bytes of piece i
    return (uint32_t)(j0 + wave * 64 + i * KPL + kk) * (D * 2) + sub * 16;
  };

  // loads complete in issue order: the query first, then the keys, then the values,
  // which arrive while the scores are computed
  u32x4_t qv[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {  // (heads past G load head 0 again, unused: no branch)
    const int hh = h < G ? h : 0;
    qv[h] = *reinterpret_cast<const u32x4_t*>(a.q + (int64_t)b * a.ldq + (int64_t)(g * G + hh) * D + sub * 8);
  }
  u32x4_t kv[NB], vv[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) kv[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, piece(i), 0, 0);
#pragma unroll
  for (int i = 0; i < NB; ++i) vv[i] = __builtin_amdgcn_raw_buffer_load_b128(vrs, piece(i), 0, 0);
  float qr[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h) unpack8(qv[h], qr[h]);

  // scores (log2 units), -inf past the last key
#pragma unroll
  for (int i0 = 0; i0 < NL; i0 += NB) {
    if (i0 > 0) {
#pragma unroll
      for (int i = 0; i < NB; ++i) kv[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, piece(i0 + i), 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      float k8[8];
      unpack8(kv[i], k8);
      const int jl = wave * 64 + (i0 + i) * KPL + kk;
      const bool ok = j0 + jl < j1;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          float sdot = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) sdot = fmaf(qr[h][e], k8[e], sdot);
          sdot = group_sum<LPK>(sdot);
          if (sub == 0) ps[jl][h] = ok ? sdot * a.scale_log2 : -INFINITY;
        }
      }
    }
  }
  __syncthreads();

  // chunk maximum and sum per head, one wavefront per head
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY;
    for (int i = lane; i < CH; i += 64) m = fmaxf(m, ps[i][h]);
    m = wave_max(m);
    float l = 0.f;
    for (int i = lane; i < CH; i += 64) {
      const float p = ps[i][h] == -INFINITY ? 0.f : fast_exp2(ps[i][h] - m);
      ps[i][h] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      stat[0][h] = m;
      stat[1][h] = l;
    }
  }
  __syncthreads();

  // P·V in registers
  float acc[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int i0 = 0; i0 < NL; i0 += NB) {
    if (i0 > 0) {
#pragma unroll
      for (int i = 0; i < NB; ++i) vv[i] = __builtin_amdgcn_raw_buffer_load_b128(vrs, piece(i0 + i), 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      float v8[8];
      unpack8(vv[i], v8);
      const int jl = wave * 64 + (i0 + i) * KPL + kk;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          const float p = ps[jl][h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, v8[e], acc[h][e]);
        }
      }
    }
  }
  float* orow = ored + (wave * KPL + kk) * RS + sub * 8;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < G) {
      *reinterpret_cast<float4*>(orow + h * D) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *reinterpret_cast<float4*>(orow + h * D + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  __syncthreads();

  auto put_o = [&](int h, int d, float v) {
    const int col = (g * G + h) * D + d;
    Elem<bf16_t>::store(a.o + (a.o_tiled ? tiled_index(b, col, (int)a.ldo) : (int64_t)b * a.ldo + col), v);
  };
  const int items = G * D;
  float* pbase = a.part + ((int64_t)b * a.Hq + g * G) * a.nsplit * (D + 2);  // head g * G + h at h * nsplit * (D + 2)
  for (int it = tid; it < items; it += 256) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 4 * KPL; ++r) sum += ored[r * RS + it];
    const int h = it / D, d = it - h * D;
    if (a.nsplit == 1) put_o(h, d, sum / stat[1][h]);
    else store_agent(pbase + ((int64_t)h * a.nsplit + c) * (D + 2) + d, sum);
  }
  if (a.nsplit == 1) return;
  if (tid < G) {
    store_agent(pbase + ((int64_t)tid * a.nsplit + c) * (D + 2) + D, stat[0][tid]);
    store_agent(pbase + ((int64_t)tid * a.nsplit + c) * (D + 2) + D + 1, stat[1][tid]);
  }
  // the last chunk of this (sequence, kv head) to finish merges all of them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  unsigned* cnt = a.count + (int64_t)b * a.Hkv + g;
  if (tid == 0)
    last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(a.nsplit - 1);
  __syncthreads();
  if (!last) return;
  // one pass over the chunks in order per (head, dim), rescaling to the running maximum
  const int ns = a.nsplit;
  for (int it = tid; it < items; it += 256) {
    const int h = it / D, d = it - h * D;
    const float* ph = pbase + (int64_t)h * ns * (D + 2);
    float M = -INFINITY, L = 0.f, O = 0.f;
    constexpr int TB = 8;  // chunks loaded per round trip
    for (int t0 = 0; t0 < ns; t0 += TB) {
      float ov[TB], mv[TB], lv[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int t = t0 + u < ns ? t0 + u : t0;  // (surplus loads repeat t0, unused)
        ov[u] = load_agent(ph + (int64_t)t * (D + 2) + d);
        mv[u] = load_agent(ph + (int64_t)t * (D + 2) + D);
        lv[u] = load_agent(ph + (int64_t)t * (D + 2) + D + 1);
      }
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        if (t0 + u >= ns) break;
        const float Mn = fmaxf(M, mv[u]);
        const float r = fast_exp2(M - Mn), e = fast_exp2(mv[u] - Mn);  // (first chunk: r = 0)
        O = O * r + ov[u] * e;
        L = L * r + lv[u] * e;
        M = Mn;
      }
    }
    put_o(h, d, O / L);
  }
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------- D = 128, exact group size
// The same workgroup layout (256 keys, 4 wavefronts x 64 keys, 16 lanes per key
// holding 8 dims each) with the group size a template constant, so no per-head branch.
// Scores: v_dot2_f32_bf16 on the bf16 (q, k) pairs (exact products, fp32 sums), then
// the G per-head partial sums of a key are reduced over its 16 lanes together
// (head_sums). P·V: two keys at a time, their values for one dim paired by v_perm_b32
// and weighted by the bf16 probabilities with v_dot2. The probabilities are rounded
// to bf16 before the chunk sum, so the weights and the normaliser agree.

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
// DPP controls within a row of 16 lanes: exchange across lane bit 0 / bit 1
// (quad_perm [1,0,3,2] / [2,3,0,1]) and rotations by 4 and 8 lanes (row_ror), which
// keep bits 0 and 1 of the lane and flip bit 2 / bit 3 respectively.
template <int BIT>
__device__ __forceinline__ float dpp_bit(float v) {
  if constexpr (BIT == 0) return dpp_mov<0xB1>(v);
  else if constexpr (BIT == 1) return dpp_mov<0x4E>(v);
  else if constexpr (BIT == 2) return dpp_mov<0x124>(v);
  else return dpp_mov<0x128>(v);
}
// v[0 .. G) are this lane's partial sums of G heads; the key's 16 lanes form one DPP
// row. For each of the lane bits t < log2(G) in turn, a lane keeps the half of its
// remaining heads selected by bit t of its index and adds the partner's (the lane
// with bit t flipped and the same lower bits) partial of that half; the bits from
// log2(G) to 3 are then summed by exchanges that keep the lower bits. Returns the
// complete sum of head head_of_lane<G>(sub).
template <int G, int T = 0>
__device__ __forceinline__ void halve(float (&v)[G], int sub) {
  if constexpr ((G >> T) > 1) {
    constexpr int H = (G >> T) / 2;
    const bool b = (sub >> T) & 1;
#pragma unroll
    for (int k = 0; k < H; ++k) {
      const float keep = b ? v[k + H] : v[k];
      const float send = b ? v[k] : v[k + H];
      v[k] = keep + dpp_bit<T>(send);
    }
    halve<G, T + 1>(v, sub);
  }
}
template <int G>
__device__ __forceinline__ float head_sums(float (&v)[G], int sub) {
  halve<G>(v, sub);
  constexpr int LB = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  float r = v[0];
  if constexpr (LB <= 0) r += dpp_bit<0>(r);
  if constexpr (LB <= 1) r += dpp_bit<1>(r);
  if constexpr (LB <= 2) r += dpp_bit<2>(r);
  r += dpp_bit<3>(r);
  return r;
}
template <int G>
__device__ __forceinline__ int head_of_lane(int sub) {
  int h = 0;
#pragma unroll
  for (int t = 0; (G >> t) > 1; ++t) h += ((sub >> t) & 1) * ((G >> t) / 2);
  return h;
}

template <int G>
__global__ __launch_bounds__(256) void attn_decode_d128_kernel(DecodeArgs a) {
  constexpr int D = 128, CH = kDecodeChunk, LPK = 16, KPL = 4, NL = 16;
  constexpr int RS = G * D + 4;  // row stride of the partial outputs (floats)
  static_assert(CH == 256 && (G == 1 || G == 2 || G == 4 || G == 8), "4 x 64 keys per chunk, G in {1, 2, 4, 8}");
  __shared__ __align__(16) float ps[CH][G];
  __shared__ __align__(16) float ored[4 * KPL * RS];
  __shared__ float stat[2][G];
  __shared__ int last;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane % LPK, kk = lane / LPK;
  const int lo = a.window > 0 ? max(0, a.len - a.window) : 0;
  const int j0 = lo + c * CH, j1 = min(a.len, j0 + CH);
  const int64_t head = ((int64_t)b * a.Hkv + g) * a.Smax;
  // keys at or past j1 (including cache rows not written yet) read as zeros
  const auto krs = make_rsrc(a.kc + head * D, (int64_t)j1 * D * 2);
  const auto vrs = make_rsrc(a.vc + head * D, (int64_t)j1 * D * 2);
  auto piece = [&](int i) {  // byte offset of this lane's 16 bytes of piece i
    return (uint32_t)(j0 + wave * 64 + i * KPL + kk) * (D * 2) + sub * 16;
  };

  // loads complete in issue order: the query first, then the keys, then the values
  u32x4_t qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qv[h] = *reinterpret_cast<const u32x4_t*>(a.q + (int64_t)b * a.ldq + (int64_t)(g * G + h) * D + sub * 8);
  u32x4_t kv[NL], vv[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) kv[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, piece(i), 0, 0);
#pragma unroll
  for (int i = 0; i < NL; ++i) vv[i] = __builtin_amdgcn_raw_buffer_load_b128(vrs, piece(i), 0, 0);

  // scores (log2 units), -inf past the last key
  const int hl = head_of_lane<G>(sub);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    float sh[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) d = dot2_bf16(qv[h][w], kv[i][w], d);
      sh[h] = d;
    }
    const float tot = head_sums<G>(sh, sub);
    const int jl = wave * 64 + i * KPL + kk;
    if (sub < G) ps[jl][hl] = j0 + jl < j1 ? tot * a.scale_log2 : -INFINITY;
  }
  __syncthreads();

  // chunk maximum and sum per head (probabilities rounded to bf16), one wavefront per head
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY;
    for (int i = lane; i < CH; i += 64) m = fmaxf(m, ps[i][h]);
    m = wave_max(m);
    float l = 0.f;
    for (int i = lane; i < CH; i += 64) {
      const float e = ps[i][h] == -INFINITY ? 0.f : fast_exp2(ps[i][h] - m);
      const float p = __uint_as_float(pack_bf16x2(e, 0.f) << 16);
      ps[i][h] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      stat[0][h] = m;
      stat[1][h] = l;
    }
  }
  __syncthreads();

  // P·V, two keys (pieces i, i + 1) per step: acc[h][e] += p_i v_i[e] + p_{i+1} v_{i+1}[e]
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < NL; i += 2) {
    const int ja = wave * 64 + i * KPL + kk, jb = ja + KPL;
    uint32_t pp[G];
#pragma unroll
    for (int h = 0; h < G; ++h)  // both probabilities are bf16 values: their high halves
      pp[h] = __builtin_amdgcn_perm(__float_as_uint(ps[jb][h]), __float_as_uint(ps[ja][h]), 0x07060302u);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t xl = __builtin_amdgcn_perm(vv[i + 1][w], vv[i][w], 0x05040100u);  // dim 2w of both keys
      const uint32_t xh = __builtin_amdgcn_perm(vv[i + 1][w], vv[i][w], 0x07060302u);  // dim 2w + 1
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc[h][2 * w] = dot2_bf16(pp[h], xl, acc[h][2 * w]);
        acc[h][2 * w + 1] = dot2_bf16(pp[h], xh, acc[h][2 * w + 1]);
      }
    }
  }
  float* orow = ored + (wave * KPL + kk) * RS + sub * 8;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    *reinterpret_cast<float4*>(orow + h * D) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
    *reinterpret_cast<float4*>(orow + h * D + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
  }
  __syncthreads();

  auto put_o = [&](int h, int d, float v) {
    const int col = (g * G + h) * D + d;
    Elem<bf16_t>::store(a.o + (a.o_tiled ? tiled_index(b, col, (int)a.ldo) : (int64_t)b * a.ldo + col), v);
  };
  constexpr int items = G * D;
  float* pbase = a.part + ((int64_t)b * a.Hq + g * G) * a.nsplit * (D + 2);  // head g * G + h at h * nsplit * (D + 2)
  for (int it = tid; it < items; it += 256) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 4 * KPL; ++r) sum += ored[r * RS + it];
    const int h = it / D, d = it - h * D;
    if (a.nsplit == 1) put_o(h, d, sum / stat[1][h]);
    else store_agent(pbase + ((int64_t)h * a.nsplit + c) * (D + 2) + d, sum);
  }
  if (a.nsplit == 1) return;
  if (tid < G) {
    store_agent(pbase + ((int64_t)tid * a.nsplit + c) * (D + 2) + D, stat[0][tid]);
    store_agent(pbase + ((int64_t)tid * a.nsplit + c) * (D + 2) + D + 1, stat[1][tid]);
  }
  // the last chunk of this (sequence, kv head) to finish merges all of them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  unsigned* cnt = a.count + (int64_t)b * a.Hkv + g;
  if (tid == 0)
    last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(a.nsplit - 1);
  __syncthreads();
  if (!last) return;
  // one pass over the chunks in order per (head, dim), rescaling to the running maximum
  const int ns = a.nsplit;
  for (int it = tid; it < items; it += 256) {
    const int h = it / D, d = it - h * D;
    const float* ph = pbase + (int64_t)h * ns * (D + 2);
    float M = -INFINITY, L = 0.f, O = 0.f;
    constexpr int TB = 8;  // chunks loaded per round trip
    for (int t0 = 0; t0 < ns; t0 += TB) {
      float ov[TB], mv[TB], lv[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int t = t0 + u < ns ? t0 + u : t0;  // (surplus loads repeat t0, unused)
        ov[u] = load_agent(ph + (int64_t)t * (D + 2) + d);
        mv[u] = load_agent(ph + (int64_t)t * (D + 2) + D);
        lv[u] = load_agent(ph + (int64_t)t * (D + 2) + D + 1);
      }
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        if (t0 + u >= ns) break;
        const float Mn = fmaxf(M, mv[u]);
        const float r = fast_exp2(M - Mn), e = fast_exp2(mv[u] - Mn);  // (first chunk: r = 0)
        O = O * r + ov[u] * e;
        L = L * r + lv[u] * e;
        M = Mn;
      }
    }
    put_o(h, d, O / L);
  }
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace

namespace {
template <typename T, int D>
hipError_t decode_impl(const void* q, int64_t ldq, const void* kc, const void* vc, int Smax, int len, int B, int Hq,
                       int Hkv, int window, void* o, int64_t ldo, bool o_tiled, float* part, hipStream_t s) {
  const int lo = window > 0 ? std::max(0, len - window) : 0;
  const int nsplit = (len - lo + kDecodeChunk - 1) / kDecodeChunk;
  const float sl = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((attn_decode_kernel<T, D>), dim3(nsplit, Hkv, B), dim3(256), 0, s, (const T*)q, ldq,
                     (const T*)kc, (const T*)vc, Smax, len, Hq, Hkv, window, part, nsplit, sl);
  hipLaunchKernelGGL(attn_decode_merge_kernel<T>, dim3(B * Hq), dim3(D < 256 ? D : 256), 0, s, part, nsplit, Hq, D,
                     (T*)o, ldo, o_tiled);
  return hipGetLastError();
}

template <int D, int GM>
hipError_t decode_bf16(const DecodeArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((attn_decode_bf16_kernel<D, GM>), dim3(a.nsplit, a.Hkv, B), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <int G>
hipError_t decode_d128(const DecodeArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((attn_decode_d128_kernel<G>), dim3(a.nsplit, a.Hkv, B), dim3(256), 0, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t attention_decode(DType dt, const void* q, int64_t ldq, const void* kc, const void* vc, int Smax, int len,
                            int B, int Hq, int Hkv, int D, int window, void* o, int64_t ldo, bool o_tiled,
                            float* part, unsigned* count, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (len <= 0 || len > Smax || Hq % Hkv || Hq / Hkv > kMaxGroup) return hipErrorInvalidValue;
  if (o_tiled && (dt != DType::BF16 || ldo != (int64_t)Hq * D || ldo % 32)) return hipErrorInvalidValue;
  const int G = Hq / Hkv;
  if (dt == DType::BF16 && G <= 8 && count && (D == 64 || D == 128 || D == 256) && ldq % 8 == 0) {
    DecodeArgs a{(const bf16_t*)q, ldq, (const bf16_t*)kc, (const bf16_t*)vc, Smax, len, Hq, Hkv, window, 0,
                 kLog2e / sqrtf((float)D), part, count, (bf16_t*)o, ldo, o_tiled};
    const int lo = window > 0 ? std::max(0, len - window) : 0;
    a.nsplit = (len - lo + kDecodeChunk - 1) / kDecodeChunk;
    switch (D) {
      case 64: return G <= 4 ? decode_bf16<64, 4>(a, B, s) : decode_bf16<64, 8>(a, B, s);
      case 128:
        switch (G) {
          case 1: return decode_d128<1>(a, B, s);
          case 2: return decode_d128<2>(a, B, s);
          case 4: return decode_d128<4>(a, B, s);
          case 8: return decode_d128<8>(a, B, s);
        }
        return G <= 4 ? decode_bf16<128, 4>(a, B, s) : decode_bf16<128, 8>(a, B, s);
      default: return G <= 4 ? decode_bf16<256, 4>(a, B, s) : decode_bf16<256, 8>(a, B, s);
    }
  }
  if (dt == DType::BF16) {
    switch (D) {
      case 64: return decode_impl<bf16_t, 64>(q, ldq, kc, vc, Smax, len, B, Hq, Hkv, window, o, ldo, o_tiled, part, s);
      case 128: return decode_impl<bf16_t, 128>(q, ldq, kc, vc, Smax, len, B, Hq, Hkv, window, o, ldo, o_tiled, part, s);
      case 256: return decode_impl<bf16_t, 256>(q, ldq, kc, vc, Smax, len, B, Hq, Hkv, window, o, ldo, o_tiled, part, s);
    }
  } else {
    switch (D) {
      case 16: return decode_impl<float, 16>(q, ldq, kc, vc, Smax, len, B, Hq, Hkv, window, o, ldo, false, part, s);
      case 32: return decode_impl<float, 32>(q, ldq, kc, vc, Smax, len, B, Hq, Hkv, window, o, ldo, false, part, s);
      case 64: return decode_impl<float, 64>(q, ldq, kc, vc, Smax, len, B, Hq, Hkv, window, o, ldo, false, part, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fwdk
