// Decode side of the forward pass: the per-layer KV cache and the one-query-per-
// sequence attention over it.
//
// A cached session prefills a prompt and then extends every sequence by one token per
// step, and a step must give the logits a cacheless forward over the whole sequence
// gives at its last position ("N7 · model/forward-parity", Theorem 1: the cached
// session prefill agrees with the cacheless forward; greedy continuation). The cache
// holds each layer's rotated keys and values, [B, Hkv, Smax, D] with positions
// contiguous, written by kv_store from the QKV projection's output.
//
// attention_decode is flash-decoding: the visible keys of a sequence are cut into
// chunks of kDecodeChunk, one workgroup per (chunk, kv head, sequence) computes the
// scores of all Hq / Hkv query heads that share the kv head, their chunk-local
// softmax statistics and the chunk's share of P·V, all in fp32; a second kernel merges
// the chunks. The work is HBM-bound (each cached key and value is read once per step).
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

// k and v of token row r = b * S + s go to position pos0 + s of sequence b.
template <typename T>
__global__ __launch_bounds__(256) void kv_store_kernel(const T* __restrict__ qkv, int64_t ldqkv, int Hq, int Hkv,
                                                      int D, int S, int pos0, T* __restrict__ kc, T* __restrict__ vc,
                                                      int Smax) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte piece
  const int r = blockIdx.x, b = r / S, s = r % S;
  const int width = Hkv * D;
  const T* krow = qkv + (int64_t)r * ldqkv + (int64_t)Hq * D;
  const T* vrow = krow + width;
  for (int c = threadIdx.x * E; c < width; c += 256 * E) {
    const int g = c / D, d = c - g * D;
    const int64_t at = (((int64_t)b * Hkv + g) * Smax + pos0 + s) * D + d;
    *reinterpret_cast<u32x4_t*>(kc + at) = *reinterpret_cast<const u32x4_t*>(krow + c);
    *reinterpret_cast<u32x4_t*>(vc + at) = *reinterpret_cast<const u32x4_t*>(vrow + c);
  }
}

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

}  // namespace

hipError_t kv_store(DType dt, const void* qkv, int64_t ldqkv, int Hq, int Hkv, int D, int B, int S, int pos0,
                    void* kc, void* vc, int Smax, hipStream_t s) {
  if (B <= 0 || S <= 0) return hipSuccess;
  if (pos0 < 0 || pos0 + S > Smax || D % (dt == DType::BF16 ? 8 : 4)) return hipErrorInvalidValue;
  if (dt == DType::BF16)
    hipLaunchKernelGGL(kv_store_kernel<bf16_t>, dim3(B * S), dim3(256), 0, s, (const bf16_t*)qkv, ldqkv, Hq, Hkv, D,
                       S, pos0, (bf16_t*)kc, (bf16_t*)vc, Smax);
  else
    hipLaunchKernelGGL(kv_store_kernel<float>, dim3(B * S), dim3(256), 0, s, (const float*)qkv, ldqkv, Hq, Hkv, D, S,
                       pos0, (float*)kc, (float*)vc, Smax);
  return hipGetLastError();
}

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
}  // namespace

hipError_t attention_decode(DType dt, const void* q, int64_t ldq, const void* kc, const void* vc, int Smax, int len,
                            int B, int Hq, int Hkv, int D, int window, void* o, int64_t ldo, bool o_tiled,
                            float* part, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (len <= 0 || len > Smax || Hq % Hkv || Hq / Hkv > kMaxGroup) return hipErrorInvalidValue;
  if (o_tiled && (dt != DType::BF16 || ldo != (int64_t)Hq * D || ldo % 32)) return hipErrorInvalidValue;
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
