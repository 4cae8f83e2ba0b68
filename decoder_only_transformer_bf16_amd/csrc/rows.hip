// Row-wise, HBM-bound kernels of the forward pass: scaled embedding gather,
// RMSNorm (plain, and the sandwich variant fused with the residual add), the
// per-position argmax with the non-finite check, and weight packing copies.
// One 64-lane wavefront per row, 16-byte vector accesses along the row.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace fwdk {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 wavefronts of 64 lanes

template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
  static __device__ __forceinline__ float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <> struct Vec4<bf16_t> {
  static __device__ __forceinline__ void store(bf16_t* p, float4 v) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
  }
  static __device__ __forceinline__ float4 load(const bf16_t* p) {
    const u32x2_t u = *reinterpret_cast<const u32x2_t*>(p);
    return float4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xFFFF0000u), __uint_as_float(u[1] << 16),
                  __uint_as_float(u[1] & 0xFFFF0000u)};
  }
};

__device__ __forceinline__ float sumsq4(float4 v) { return v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w; }
__device__ __forceinline__ float4 mul4(float4 a, float4 b, float s) {
  return float4{a.x * b.x * s, a.y * b.y * s, a.z * b.z * s, a.w * b.w * s};
}

// Rows of up to kMaxV * 256 elements are held in registers (kMaxV float4 per lane),
// so every load of a row is in flight before the reduction; longer rows loop.
constexpr int kMaxV = 16;

// y = x * w / sqrt(mean(x^2) + eps)  ("N7 · model/forward-parity", intro: RMSNorm)
// One wavefront per row (rows past the grid are walked with a grid stride). The gains
// are loaded together with the row, before the reduction, so that no load waits after
// it (Llama-shape rows: 84 -> 77 us per launch).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                     T* __restrict__ y, float* __restrict__ y32, int rows, int H,
                                                     float eps, bool tiled) {
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x * kRowsPerBlock;
  int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (H <= kMaxV * 256) {
    float4 g[kMaxV];
#pragma unroll
    for (int j = 0; j < kMaxV; ++j) {
      const int i = lane * 4 + j * 256;
      g[j] = i < H ? Vec4<float>::load(w + i) : float4{0.f, 0.f, 0.f, 0.f};
    }
    for (; row < rows; row += stride) {
      const float* xr = x + (int64_t)row * H;
      float4 v[kMaxV];
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxV; ++j) {
        const int i = lane * 4 + j * 256;
        v[j] = i < H ? Vec4<float>::load(xr + i) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < kMaxV; ++j) ss += sumsq4(v[j]);
      ss = wave_sum(ss);
      const float r = fast_rsqrt(ss / (float)H + eps);
#pragma unroll
      for (int j = 0; j < kMaxV; ++j) {
        const int i = lane * 4 + j * 256;
        if (i >= H) continue;
        const float4 o = mul4(v[j], g[j], r);
        Vec4<T>::store(y + (tiled ? tiled_index(row, i, H) : (int64_t)row * H + i), o);
        if (y32) Vec4<float>::store(y32 + (int64_t)row * H + i, o);
      }
    }
    return;
  }
  for (; row < rows; row += stride) {
    const float* xr = x + (int64_t)row * H;
    float ss = 0.f;
    for (int i = lane * 4; i < H; i += 256) ss += sumsq4(Vec4<float>::load(xr + i));
    ss = wave_sum(ss);
    const float r = fast_rsqrt(ss / (float)H + eps);
    for (int i = lane * 4; i < H; i += 256) {
      const float4 v = mul4(Vec4<float>::load(xr + i), Vec4<float>::load(w + i), r);
      Vec4<T>::store(y + (tiled ? tiled_index(row, i, H) : (int64_t)row * H + i), v);
      if (y32) Vec4<float>::store(y32 + (int64_t)row * H + i, v);
    }
  }
}

// Sandwich placement ("N7 · model/forward-parity", intro: topology-selected norm
// placement): xout = xin + RMSNorm(u; wpost), then y = RMSNorm(xout; wnext), the
// input of the next sublayer.
template <typename T>
__global__ __launch_bounds__(256) void add_norm_kernel(const float* __restrict__ xin, const float* __restrict__ u,
                                                      const float* __restrict__ wpost, float* __restrict__ xout,
                                                      const float* __restrict__ wnext, T* __restrict__ y,
                                                      float* __restrict__ y32, int rows, int H, float eps,
                                                      bool tiled) {
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t off = (int64_t)row * H;
  if (H <= kMaxV * 256) {
    // gains go out with the rows (post-norm gains) and before the second reduction
    // (next-norm gains), so no load waits behind a reduction
    float4 uv[kMaxV], xv[kMaxV], g[kMaxV];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxV; ++j) {
      const int i = lane * 4 + j * 256;
      uv[j] = i < H ? Vec4<float>::load(u + off + i) : float4{0.f, 0.f, 0.f, 0.f};
      xv[j] = i < H ? Vec4<float>::load(xin + off + i) : float4{0.f, 0.f, 0.f, 0.f};
      g[j] = i < H ? Vec4<float>::load(wpost + i) : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kMaxV; ++j) ss += sumsq4(uv[j]);
    ss = wave_sum(ss);
    const float ru = fast_rsqrt(ss / (float)H + eps);
    float sx = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxV; ++j) {
      const int i = lane * 4 + j * 256;
      if (i >= H) continue;
      const float4 n = mul4(uv[j], g[j], ru);
      xv[j] = float4{xv[j].x + n.x, xv[j].y + n.y, xv[j].z + n.z, xv[j].w + n.w};
      Vec4<float>::store(xout + off + i, xv[j]);
      sx += sumsq4(xv[j]);
    }
#pragma unroll
    for (int j = 0; j < kMaxV; ++j) {
      const int i = lane * 4 + j * 256;
      g[j] = i < H ? Vec4<float>::load(wnext + i) : float4{0.f, 0.f, 0.f, 0.f};
    }
    sx = wave_sum(sx);
    const float rx = fast_rsqrt(sx / (float)H + eps);
#pragma unroll
    for (int j = 0; j < kMaxV; ++j) {
      const int i = lane * 4 + j * 256;
      if (i >= H) continue;
      const float4 v = mul4(xv[j], g[j], rx);
      Vec4<T>::store(y + (tiled ? tiled_index(row, i, H) : off + i), v);
      if (y32) Vec4<float>::store(y32 + off + i, v);
    }
    return;
  }
  float ss = 0.f;
  for (int i = lane * 4; i < H; i += 256) ss += sumsq4(Vec4<float>::load(u + off + i));
  ss = wave_sum(ss);
  const float ru = fast_rsqrt(ss / (float)H + eps);
  float sx = 0.f;
  for (int i = lane * 4; i < H; i += 256) {
    const float4 n = mul4(Vec4<float>::load(u + off + i), Vec4<float>::load(wpost + i), ru);
    const float4 xi = Vec4<float>::load(xin + off + i);
    const float4 xo = float4{xi.x + n.x, xi.y + n.y, xi.z + n.z, xi.w + n.w};
    Vec4<float>::store(xout + off + i, xo);
    sx += sumsq4(xo);
  }
  sx = wave_sum(sx);
  const float rx = fast_rsqrt(sx / (float)H + eps);
  for (int i = lane * 4; i < H; i += 256) {
    // each lane re-reads only what it wrote itself
    const float4 v = mul4(Vec4<float>::load(xout + off + i), Vec4<float>::load(wnext + i), rx);
    Vec4<T>::store(y + (tiled ? tiled_index(row, i, H) : off + i), v);
    if (y32) Vec4<float>::store(y32 + off + i, v);
  }
}

// x[t] = E[ids[t]] * scale ("pegainfer issue #878", Proposed Plan: scaled embedding)
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids, const T* __restrict__ E,
                                                   float* __restrict__ x, int rows, int H, float scale, bool tiled) {
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t id = ids[row];
  for (int i = lane * 4; i < H; i += 256) {
    const float4 v = Vec4<T>::load(E + (tiled ? tiled_index(id, i, H) : id * H + i));
    Vec4<float>::store(x + (int64_t)row * H + i, float4{v.x * scale, v.y * scale, v.z * scale, v.w * scale});
  }
}

// argmax over a row, lowest index on ties ("N7 · model/forward-parity", Theorem 1:
// per-position argmax); any non-finite value raises the flag ("pegainfer issue
// #878", Acceptance Criteria). 256 threads per row.
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// Blocks (row, slice): columns [slice * span, min(V, slice * span + span)) of the row.
// With one slice the block writes out[row]; otherwise its best (value, column) goes to
// pv / pi[row * gridDim.y + slice] and argmax_merge_kernel picks among the slices (a
// few rows, e.g. a decode step, would otherwise keep only a handful of workgroups busy).
__global__ __launch_bounds__(256) void argmax_kernel(const float* __restrict__ z, int64_t ldz, int V, int span,
                                                    int32_t* __restrict__ out, float* __restrict__ pv,
                                                    int* __restrict__ pi, int* __restrict__ flag) {
  const int row = blockIdx.x, tid = threadIdx.x;
  const int c0 = blockIdx.y * span, c1 = min(V, c0 + span);
  const float* zr = z + (int64_t)row * ldz;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  bool bad = false;
  const bool vec = (V % 4 == 0) && ((ldz % 4) == 0) && (span % 4 == 0);
  if (vec) {
    for (int i = c0 + tid * 4; i < c1; i += 1024) {
      const float4 v = *reinterpret_cast<const float4*>(zr + i);
      bad |= !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
      better(bv, bi, v.x, i);
      better(bv, bi, v.y, i + 1);
      better(bv, bi, v.z, i + 2);
      better(bv, bi, v.w, i + 3);
    }
  } else {
    for (int i = c0 + tid; i < c1; i += 256) {
      const float v = zr[i];
      bad |= !isfinite(v);
      better(bv, bi, v, i);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    better(bv, bi, ov, oi);
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int sbad[4];
  const int wave = tid >> 6;
  const bool wbad = __any(bad);
  if ((tid & 63) == 0) {
    sv[wave] = bv;
    si[wave] = bi;
    sbad[wave] = wbad;
  }
  __syncthreads();
  if (tid == 0) {
    float v = sv[0];
    int i = si[0];
    int anybad = sbad[0];
    for (int w = 1; w < 4; ++w) {
      better(v, i, sv[w], si[w]);
      anybad |= sbad[w];
    }
    if (gridDim.y == 1) {
      if (out) out[row] = i;
    } else {
      pv[row * gridDim.y + blockIdx.y] = v;
      pi[row * gridDim.y + blockIdx.y] = i;
    }
    if (anybad) *flag = 1;
  }
}

// out[row] = the best of the row's `slices` partial (value, column) pairs (lowest column
// among equal values, as `better` orders them).
__global__ __launch_bounds__(64) void argmax_merge_kernel(const float* __restrict__ pv, const int* __restrict__ pi,
                                                         int slices, int rows, int32_t* __restrict__ out) {
  const int row = blockIdx.x * 64 + threadIdx.x;
  if (row >= rows) return;
  float v = pv[row * slices];
  int i = pi[row * slices];
  for (int j = 1; j < slices; ++j) better(v, i, pv[row * slices + j], pi[row * slices + j]);
  out[row] = i;
}

// Packing copy: dst row map[r] <- src row r.
__global__ __launch_bounds__(256) void copy_rows_kernel(uint8_t* __restrict__ dst, const uint8_t* __restrict__ src,
                                                       const int32_t* __restrict__ map, int64_t row_bytes) {
  const int r = blockIdx.x;
  const uint8_t* s = src + (int64_t)r * row_bytes;
  uint8_t* d = dst + (int64_t)map[r] * row_bytes;
  if (row_bytes % 16 == 0) {
    for (int64_t i = threadIdx.x * 16; i < row_bytes; i += 256 * 16)
      *reinterpret_cast<u32x4_t*>(d + i) = *reinterpret_cast<const u32x4_t*>(s + i);
  } else {
    for (int64_t i = threadIdx.x * 4; i < row_bytes; i += 256 * 4)
      *reinterpret_cast<uint32_t*>(d + i) = *reinterpret_cast<const uint32_t*>(s + i);
  }
}

// dst (K-tiled, bf16) row map[r] = src row r (row-major, K elements); one 16-byte
// piece (8 elements, inside one 32-wide tile) per thread.
__global__ __launch_bounds__(256) void pack_tiled_kernel(bf16_t* __restrict__ dst, const bf16_t* __restrict__ src,
                                                        const int32_t* __restrict__ map, int K) {
  const int r = blockIdx.x;
  const bf16_t* srow = src + (int64_t)r * K;
  const int64_t d = map[r];
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8)
    *reinterpret_cast<u32x4_t*>(dst + tiled_index(d, c, K)) = *reinterpret_cast<const u32x4_t*>(srow + c);
}

template <typename T>
__global__ void gains_kernel(const T* __restrict__ src, float* __restrict__ dst, int n, float offset) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = offset + Elem<T>::load(src + i);
}

// QK-norm then RoPE, in place on the q and k heads of each token row (qwen3 / gemma3
// family axis of "N7 · model/forward-parity", Theorem statement): a head's D values
// are scaled by gain / sqrt(mean of squares + eps), then each pair (k, k + D/2) turns
// by the row's table entry. With a cache, the rotated k heads and the v heads are also
// stored at the row's position. One wavefront per head, a lane per pair.
// bf16: D / 16 lanes per head; a lane holds elements 8 j .. 8 j + 7 of both halves,
// i.e. eight whole rotation pairs, with 16-byte loads and stores.
template <int D>
__global__ __launch_bounds__(256) void qk_norm_rope_bf16_kernel(QkNormArgs a, int rows) {
  constexpr int LPH = D / 16, HPW = 64 / LPH, half = D / 2;
  const int lane = threadIdx.x & 63, j = lane % LPH;
  const int nh = a.Hq + a.Hkv, heads = nh + (a.vc ? a.Hkv : 0);
  const int64_t gh = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * HPW + lane / LPH;
  if (gh >= (int64_t)rows * heads) return;  // (whole groups of LPH lanes leave together)
  const int row = (int)(gh / heads), h = (int)(gh - (int64_t)row * heads);
  const int b = row / a.S, pos = a.pos0 + row % a.S;
  bf16_t* x = (bf16_t*)a.qkv + (int64_t)row * a.ld + (int64_t)h * D + 8 * j;
  const u32x4_t u0 = *reinterpret_cast<const u32x4_t*>(x), u1 = *reinterpret_cast<const u32x4_t*>(x + half);
  if (h >= nh) {  // a value head: cache copy only
    bf16_t* dst = (bf16_t*)a.vc + (((int64_t)b * a.Hkv + (h - nh)) * a.Smax + pos) * D + 8 * j;
    *reinterpret_cast<u32x4_t*>(dst) = u0;
    *reinterpret_cast<u32x4_t*>(dst + half) = u1;
    return;
  }
  const bool is_k = h >= a.Hq;
  const float* gain = (is_k ? a.gk : a.gq) + 8 * j;
  const float4* cs4 = reinterpret_cast<const float4*>(a.cs + (int64_t)pos * half + 8 * j);  // 8 (cos, sin)
  float p[8], q[8];
  unpack8(u0, p);
  unpack8(u1, q);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += p[e] * p[e] + q[e] * q[e];
  ss = group_sum<LPH>(ss);
  const float r = fast_rsqrt(ss / (float)D + a.eps);
  float o0[8], o1[8];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    const float4 c = cs4[e2];  // pairs 2 e2 and 2 e2 + 1
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int e = 2 * e2 + t;
      const float cx = t ? c.z : c.x, sy = t ? c.w : c.y;
      const float u = p[e] * r * gain[e], v = q[e] * r * gain[e + half];
      o0[e] = u * cx - v * sy;
      o1[e] = u * sy + v * cx;
    }
  }
  const u32x4_t w0 = pack8(o0), w1 = pack8(o1);
  *reinterpret_cast<u32x4_t*>(x) = w0;
  *reinterpret_cast<u32x4_t*>(x + half) = w1;
  if (is_k && a.kc) {
    bf16_t* kd = (bf16_t*)a.kc + (((int64_t)b * a.Hkv + (h - a.Hq)) * a.Smax + pos) * D + 8 * j;
    *reinterpret_cast<u32x4_t*>(kd) = w0;
    *reinterpret_cast<u32x4_t*>(kd + half) = w1;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(QkNormArgs a) {
  const int row = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = a.D / 2, nh = a.Hq + a.Hkv, heads = nh + (a.vc ? a.Hkv : 0);
  const int b = row / a.S, pos = a.pos0 + row % a.S;
  T* base = (T*)a.qkv + (int64_t)row * a.ld;
  for (int h = blockIdx.y * 4 + wave; h < heads; h += gridDim.y * 4) {
    T* x = base + (int64_t)h * a.D;
    if (h >= nh) {  // a value head: cache copy only
      const int g = h - nh;
      T* dst = (T*)a.vc + (((int64_t)b * a.Hkv + g) * a.Smax + pos) * a.D;
      for (int d = lane; d < a.D; d += 64) dst[d] = x[d];
      continue;
    }
    const bool is_k = h >= a.Hq;
    const float* gain = is_k ? a.gk : a.gq;
    float ss = 0.f;
    for (int k = lane; k < half; k += 64) {
      const float u = Elem<T>::load(x + k), v = Elem<T>::load(x + k + half);
      ss += u * u + v * v;
    }
    ss = wave_sum(ss);
    const float r = fast_rsqrt(ss / (float)a.D + a.eps);
    const float2* cs = a.cs + (int64_t)pos * half;
    T* kd = is_k && a.kc ? (T*)a.kc + (((int64_t)b * a.Hkv + (h - a.Hq)) * a.Smax + pos) * a.D : nullptr;
    for (int k = lane; k < half; k += 64) {
      const float u = Elem<T>::load(x + k) * r * gain[k], v = Elem<T>::load(x + k + half) * r * gain[k + half];
      const float2 c = cs[k];
      const float o0 = u * c.x - v * c.y, o1 = u * c.y + v * c.x;
      Elem<T>::store(x + k, o0);
      Elem<T>::store(x + k + half, o1);
      if (kd) {
        Elem<T>::store(kd + k, o0);
        Elem<T>::store(kd + k + half, o1);
      }
    }
  }
}

inline int row_blocks(int rows) { return (rows + kRowsPerBlock - 1) / kRowsPerBlock; }
// RMSNorm grids stop at 2048 workgroups (8 per CU); larger batches walk rows with the grid
// stride, each wavefront loading the gains once for all its rows. Llama-shape rows
// (16384 x 4096), interleaved in one process: 5.39 -> 5.16 ms over the 65 norms of a
// prefill, the same at 1024 workgroups.
constexpr int kNormMaxBlocks = 2048;

}  // namespace

hipError_t rmsnorm(DType dt, const float* x, const float* w, void* y, float* y32, int rows, int H, float eps,
                   bool tiled, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (tiled && (dt != DType::BF16 || H % 32)) return hipErrorInvalidValue;
  if (dt == DType::BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3(std::min(row_blocks(rows), kNormMaxBlocks)), dim3(256), 0, s, x, w,
                       (bf16_t*)y, y32, rows, H, eps, tiled);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(row_blocks(rows)), dim3(256), 0, s, x, w,
                       (float*)y, y32, rows, H, eps, false);
  return hipGetLastError();
}

hipError_t add_norm(DType dt, const float* xin, const float* u, const float* wpost, float* xout, const float* wnext,
                    void* y, float* y32, int rows, int H, float eps, bool tiled, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (tiled && (dt != DType::BF16 || H % 32)) return hipErrorInvalidValue;
  if (dt == DType::BF16)
    hipLaunchKernelGGL(add_norm_kernel<bf16_t>, dim3(row_blocks(rows)), dim3(256), 0, s, xin, u, wpost, xout,
                       wnext, (bf16_t*)y, y32, rows, H, eps, tiled);
  else
    hipLaunchKernelGGL(add_norm_kernel<float>, dim3(row_blocks(rows)), dim3(256), 0, s, xin, u, wpost, xout, wnext,
                       (float*)y, y32, rows, H, eps, false);
  return hipGetLastError();
}

hipError_t embed(DType dt, const int32_t* ids, const void* E, float* x, int rows, int H, float scale, bool tiled,
                 hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (tiled && (dt != DType::BF16 || H % 32)) return hipErrorInvalidValue;
  if (dt == DType::BF16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(row_blocks(rows)), dim3(256), 0, s, ids, (const bf16_t*)E, x,
                       rows, H, scale, tiled);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(row_blocks(rows)), dim3(256), 0, s, ids, (const float*)E, x, rows,
                       H, scale, false);
  return hipGetLastError();
}

hipError_t argmax_rows(const float* z, int64_t ldz, int rows, int V, int32_t* out, int* flag, hipStream_t s,
                       float* part, int64_t part_pairs) {
  if (rows <= 0) return hipSuccess;
  // split long rows of small batches so that at least ~256 workgroups run
  int slices = 1;
  if (part && out) {
    const int want = std::min<int>(kArgmaxMaxSlices, (256 + rows - 1) / rows);
    slices = std::max(1, std::min(want, (V + 4095) / 4096));
    if ((int64_t)rows * slices > part_pairs) slices = 1;
  }
  const int span = ((V + slices - 1) / slices + 1023) & ~1023;  // a multiple of 1024 columns
  slices = (V + span - 1) / span;
  float* pv = slices > 1 ? part : nullptr;
  int* pi = slices > 1 ? reinterpret_cast<int*>(part + (int64_t)rows * slices) : nullptr;
  hipLaunchKernelGGL(argmax_kernel, dim3(rows, slices), dim3(256), 0, s, z, ldz, V, span, out, pv, pi, flag);
  if (slices > 1) {
    if (hipError_t e = hipGetLastError()) return e;
    hipLaunchKernelGGL(argmax_merge_kernel, dim3((rows + 63) / 64), dim3(64), 0, s, pv, pi, slices, rows, out);
  }
  return hipGetLastError();
}

hipError_t copy_rows(void* dst, const void* src, const int32_t* map, int rows, int64_t row_bytes, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(rows), dim3(256), 0, s, (uint8_t*)dst, (const uint8_t*)src, map,
                     row_bytes);
  return hipGetLastError();
}

hipError_t pack_tiled(void* dst, const void* src, const int32_t* map, int rows, int K, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_tiled_kernel, dim3(rows), dim3(256), 0, s, (bf16_t*)dst, (const bf16_t*)src, map, K);
  return hipGetLastError();
}

hipError_t gains_to_f32(DType dt, const void* src, float* dst, int n, float offset, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dt == DType::BF16)
    hipLaunchKernelGGL(gains_kernel<bf16_t>, dim3((n + 255) / 256), dim3(256), 0, s, (const bf16_t*)src, dst, n,
                       offset);
  else
    hipLaunchKernelGGL(gains_kernel<float>, dim3((n + 255) / 256), dim3(256), 0, s, (const float*)src, dst, n,
                       offset);
  return hipGetLastError();
}

hipError_t qk_norm_rope(DType dt, const QkNormArgs& a, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (a.D % 2 || a.D > 512 || (a.kc == nullptr) != (a.vc == nullptr)) return hipErrorInvalidValue;
  const int heads = a.Hq + a.Hkv + (a.vc ? a.Hkv : 0);
  if (dt == DType::BF16 && (a.D == 64 || a.D == 128 || a.D == 256) && a.ld % 8 == 0) {
    const int64_t per_block = 4LL * (64 / (a.D / 16));  // heads per workgroup
    const dim3 grid((unsigned)(((int64_t)rows * heads + per_block - 1) / per_block));
    switch (a.D) {
      case 64: hipLaunchKernelGGL(qk_norm_rope_bf16_kernel<64>, grid, dim3(256), 0, s, a, rows); break;
      case 128: hipLaunchKernelGGL(qk_norm_rope_bf16_kernel<128>, grid, dim3(256), 0, s, a, rows); break;
      default: hipLaunchKernelGGL(qk_norm_rope_bf16_kernel<256>, grid, dim3(256), 0, s, a, rows);
    }
    return hipGetLastError();
  }
  const dim3 grid(rows, (heads + 3) / 4);
  if (dt == DType::BF16) hipLaunchKernelGGL(qk_norm_rope_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(qk_norm_rope_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fwdk
