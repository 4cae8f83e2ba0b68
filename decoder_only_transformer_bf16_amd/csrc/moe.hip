// Mixture-of-experts feed-forward: routing, the expert-ordered permutation of the
// token rows, and the weighted combination of the expert outputs (qwen3moe family
// axis of "N7 · model/forward-parity", Theorem statement; the intro lists the MoE FFN).
//
// A token's router logits pick its top-k experts (the softmax over all experts is
// monotone, so by logit, lowest index first on ties); their softmax probabilities,
// optionally renormalised to sum 1, weight the experts' outputs. Assignments (token t,
// slot j) are laid out expert by expert, in token order within an expert, each
// expert's segment starting on a 16-row boundary so that its rows form whole tiles of
// the K-tiled operand layout; the grouped products then run one expert per tile, and
// the combination adds a token's k outputs in slot order. Every step is deterministic
// (integer counting only, no floating-point atomics).
#include "common.h"
#include "kernels.h"

namespace fwdk {
namespace {

constexpr int kChunk = 256;  // assignments per counting workgroup

// One wavefront per token. Lane l holds logits l, l + 64, ...
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                       bool norm, int32_t* __restrict__ idx, float* __restrict__ w) {
  constexpr int MAXV = kMoeMaxExperts / 64;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* z = logits + (int64_t)t * E;
  float v[MAXV];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < MAXV; ++q) {
    const int e = lane + 64 * q;
    v[q] = e < E ? z[e] : -INFINITY;
    m = fmaxf(m, v[q]);
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < MAXV; ++q) s += lane + 64 * q < E ? fast_exp2((v[q] - m) * kLog2e) : 0.f;
  s = wave_sum(s);
  float picked_sum = 0.f, picked[kMoeMaxTopK];
  int picked_e[kMoeMaxTopK];
#pragma unroll
  for (int j = 0; j < kMoeMaxTopK; ++j) {
    if (j >= k) break;
    // the largest remaining logit, lowest expert index on ties
    float best = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < MAXV; ++q) {
      const int e = lane + 64 * q;
      if (e < E && (v[q] > best || (v[q] == best && e < be))) {
        best = v[q];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ob = __shfl_xor(best, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ob > best || (ob == best && oe < be)) {
        best = ob;
        be = oe;
      }
    }
#pragma unroll
    for (int q = 0; q < MAXV; ++q)
      if (lane + 64 * q == be) v[q] = -INFINITY;  // (a picked expert is never picked again)
    const float p = fast_exp2((best - m) * kLog2e) / s;
    picked[j] = p;
    picked_e[j] = be;
    picked_sum += p;
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < kMoeMaxTopK; ++j) {
      if (j >= k) break;
      idx[(int64_t)t * k + j] = picked_e[j];
      w[(int64_t)t * k + j] = norm ? picked[j] / picked_sum : picked[j];
    }
  }
}

// Per chunk of kChunk assignments: how many go to each expert.
__global__ __launch_bounds__(kChunk) void moe_count_kernel(const int32_t* __restrict__ idx, int A, int E,
                                                           int* __restrict__ chunk_count) {
  __shared__ int hist[kMoeMaxExperts];
  for (int e = threadIdx.x; e < E; e += kChunk) hist[e] = 0;
  __syncthreads();
  const int i = blockIdx.x * kChunk + threadIdx.x;
  if (i < A) atomicAdd(&hist[idx[i]], 1);  // (integer counts: the order of the adds does not matter)
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunk) chunk_count[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Exclusive prefix sum over the 256 threads of a workgroup; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w2 = 0; w2 < wave; ++w2) base += lds[w2];
  *total = lds[0] + lds[1] + lds[2] + lds[3];
  __syncthreads();
  return base + incl - v;
}

// Workgroup per expert: each chunk's first row within the expert's segment (chunk
// order), and the expert's total.
__global__ __launch_bounds__(256) void moe_expert_scan_kernel(const int* __restrict__ chunk_count, int nchunks,
                                                              int E, int* __restrict__ chunk_base,
                                                              int* __restrict__ total) {
  __shared__ int lds[4];
  const int e = blockIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const int v = c < nchunks ? chunk_count[(int64_t)c * E + e] : 0;
    int tot;
    const int ex = block_exclusive_scan(v, lds, &tot);
    if (c < nchunks) chunk_base[(int64_t)c * E + e] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) total[e] = carry;
}

// One workgroup, thread per expert: segments (16-row aligned) and first 128-row tiles.
__global__ __launch_bounds__(256) void moe_segments_kernel(const int* __restrict__ total, int E,
                                                           int* __restrict__ seg_start, int* __restrict__ seg_count,
                                                           int* __restrict__ mtile_start) {
  __shared__ int lds[4];
  const int e = threadIdx.x;  // E <= 256
  const int n = e < E ? total[e] : 0;
  int rows_total, tiles_total;
  const int rows0 = block_exclusive_scan((n + 15) / 16 * 16, lds, &rows_total);
  const int tile0 = block_exclusive_scan((n + kMoeTileRows - 1) / kMoeTileRows, lds, &tiles_total);
  if (e < E) {
    seg_start[e] = rows0;
    seg_count[e] = n;
    mtile_start[e] = tile0;
  }
  if (e == 0) mtile_start[E] = tiles_total;
}

// Row of every assignment: its expert's chunk base, plus the assignments of the same
// expert earlier in the chunk (earlier wavefronts, then earlier lanes).
__global__ __launch_bounds__(kChunk) void moe_place_kernel(const int32_t* __restrict__ idx, int A, int E,
                                                           const int* __restrict__ chunk_base,
                                                           const int* __restrict__ seg_start,
                                                           int32_t* __restrict__ pos) {
  __shared__ int hist[kChunk / 64][kMoeMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < (kChunk / 64) * E; i += kChunk) hist[i / E][i % E] = 0;
  __syncthreads();
  const int i = blockIdx.x * kChunk + threadIdx.x;
  const int e = i < A ? idx[i] : -1;
  int r = 0;
  for (int j = 0; j < 64; ++j) {
    const int ej = __shfl(e, j, 64);
    r += (j < lane && ej == e) ? 1 : 0;
  }
  if (e >= 0) atomicAdd(&hist[wave][e], 1);
  __syncthreads();
  if (e < 0) return;
  for (int w2 = 0; w2 < wave; ++w2) r += hist[w2][e];
  pos[i] = seg_start[e] + chunk_base[(int64_t)blockIdx.x * E + e] + r;
}

// X_perm row pos[i] = n row i / k (both bf16 K-tiled with row width H).
__global__ __launch_bounds__(256) void moe_gather_kernel(const bf16_t* __restrict__ n, const int32_t* __restrict__ pos,
                                                         int A, int k, int H, bf16_t* __restrict__ xp) {
  const int i = blockIdx.x;
  if (i >= A) return;
  const int src = i / k, dst = pos[i];
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8)
    *reinterpret_cast<u32x4_t*>(xp + tiled_index(dst, c, H)) =
        *reinterpret_cast<const u32x4_t*>(n + tiled_index(src, c, H));
}

// out[t] = (xin[t] +) sum over slots j in order of w[t, j] * y[pos[t, j]].
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ pos,
                                                          const float* __restrict__ w, int k, int H,
                                                          const float* __restrict__ xin, float* __restrict__ out) {
  const int t = blockIdx.x;
  for (int h = threadIdx.x * 4; h < H; h += 256 * 4) {
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const float wj = w[(int64_t)t * k + j];
      const float4 v = *reinterpret_cast<const float4*>(y + (int64_t)pos[(int64_t)t * k + j] * H + h);
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
      acc.z = fmaf(wj, v.z, acc.z);
      acc.w = fmaf(wj, v.w, acc.w);
    }
    if (xin) {
      const float4 x = *reinterpret_cast<const float4*>(xin + (int64_t)t * H + h);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    *reinterpret_cast<float4*>(out + (int64_t)t * H + h) = acc;
  }
}

}  // namespace

hipError_t moe_route(const float* logits, int T, int E, int k, bool norm, int32_t* idx, float* w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (E <= 0 || E > kMoeMaxExperts || k <= 0 || k > kMoeMaxTopK || k > E) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_route_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, norm, idx, w);
  return hipGetLastError();
}

int64_t moe_chunks(int64_t A) { return (A + kChunk - 1) / kChunk; }

hipError_t moe_plan(const int32_t* idx, int A, int E, const MoePlan& p, hipStream_t s) {
  if (A <= 0) return hipSuccess;
  if (E <= 0 || E > kMoeMaxExperts) return hipErrorInvalidValue;
  const int nch = (int)moe_chunks(A);
  hipLaunchKernelGGL(moe_count_kernel, dim3(nch), dim3(kChunk), 0, s, idx, A, E, p.chunk_count);
  hipLaunchKernelGGL(moe_expert_scan_kernel, dim3(E), dim3(256), 0, s, p.chunk_count, nch, E, p.chunk_base,
                     p.total);
  hipLaunchKernelGGL(moe_segments_kernel, dim3(1), dim3(256), 0, s, p.total, E, p.seg_start, p.seg_count,
                     p.mtile_start);
  hipLaunchKernelGGL(moe_place_kernel, dim3(nch), dim3(kChunk), 0, s, idx, A, E, p.chunk_base, p.seg_start, p.pos);
  return hipGetLastError();
}

hipError_t moe_gather(const void* n, const int32_t* pos, int A, int k, int H, void* xp, hipStream_t s) {
  if (A <= 0) return hipSuccess;
  if (H % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_gather_kernel, dim3(A), dim3(256), 0, s, (const bf16_t*)n, pos, A, k, H, (bf16_t*)xp);
  return hipGetLastError();
}

hipError_t moe_combine(const float* y, const int32_t* pos, const float* w, int T, int k, int H, const float* xin,
                       float* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (H % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(T), dim3(256), 0, s, y, pos, w, k, H, xin, out);
  return hipGetLastError();
}

}  // namespace fwdk
