// Causal grouped-query attention with an optional sliding window
// ("N7 · model/forward-parity", intro: causal multi-head/GQA attention;
// "pegainfer issue #878", Description: a window of W keeps keys with i - j < W).
//
//   o[b,i,h,:] = sum_j p_ij v[b,j,g,:],  p_ij = softmax_j(q[b,i,h,:]·k[b,j,g,:] / sqrt(D)),
//   g = h / (Hq / Hkv), over keys j <= i (and i - j < W when W > 0).
//
// bf16 path (D in {64, 128, 256}): flash-style single pass with an online softmax.
// The score tile is computed transposed, Sᵀ = K·Qᵀ with v_mfma_f32_16x16x32_bf16,
// so that every lane owns one query column: the softmax statistics are per lane
// except for one cross-lane max over the four 16-lane groups. The probabilities
// then feed Oᵀ += Vᵀ·Pᵀ straight from registers as the MFMA B operand; values are
// kept transposed (keys contiguous) so the A operand is a 16-byte LDS read.
// K and Vᵀ slices of 32 keys are double-buffered in LDS.
//
// f32 path (D <= 64): one wavefront per query row on the vector ALUs.
#include "common.h"
#include "kernels.h"

namespace fwdk {
namespace {

constexpr int KB = 32;  // keys per slice

// Key j of a slice (j = 8 g + 4 t + r) is stored in LDS row 16 t + 4 g + r, so that
// row m of the t-th 16-row MFMA tile holds key 8 (m / 4) + 4 t + m % 4 and lane group
// g of the transposed score tile ends up owning keys 8 g .. 8 g + 7.
__device__ __forceinline__ int key_row(int j) { return ((j >> 2) & 1) * 16 + (j >> 3) * 4 + (j & 3); }

// LDS layouts (16-byte chunks XOR-swizzled so that the 16 lanes an LDS read serves
// together, which read one chunk column of 16 consecutive rows, hit distinct banks).
template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {  // K tile: [32 rows][D]
  return row * D + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 3);
}
__device__ __forceinline__ int v_off(int d, int chunk) {  // Vᵀ tile: [D rows][32 keys], 4 chunks per row
  return d * KB + ((chunk ^ ((d >> 2) & 3)) << 3);
}

template <int D>
struct KVLoader {
  static constexpr int kPer = D / 64;  // (32 * D / 8) chunks / 256 threads, same for K and Vᵀ
  u32x4_t kv[kPer], vv[kPer];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ kbase, int64_t ldk,
                                       const bf16_t* __restrict__ vbase, int ldvt, int j0, int S, int tid) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int q = tid + p * 256;
      const int j = q / (D / 8), c = q % (D / 8);
      kv[p] = (j0 + j < S) ? *reinterpret_cast<const u32x4_t*>(kbase + (int64_t)(j0 + j) * ldk + c * 8)
                           : u32x4_t{0u, 0u, 0u, 0u};
      const int d = q >> 2, cv = q & 3;
      const int key = j0 + cv * 8;
      u32x4_t x = u32x4_t{0u, 0u, 0u, 0u};
      if (key < S) {
        x = *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)d * ldvt + key);
        if (key + 8 > S) {  // keys past the sequence end hold padding: zero them
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k0 = key + 2 * e;
            uint32_t w = x[e];
            if (k0 >= S) w &= 0xFFFF0000u;
            if (k0 + 1 >= S) w &= 0x0000FFFFu;
            x[e] = w;
          }
        }
      }
      vv[p] = x;
    }
  }
  __device__ __forceinline__ void store(bf16_t* klds, bf16_t* vlds, int tid) const {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int q = tid + p * 256;
      const int j = q / (D / 8), c = q % (D / 8);
      *reinterpret_cast<u32x4_t*>(klds + k_off<D>(key_row(j), c)) = kv[p];
      *reinterpret_cast<u32x4_t*>(vlds + v_off(q >> 2, q & 3)) = vv[p];
    }
  }
};

template <int D, int NQ>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a, float scale_log2) {
  constexpr int BQ = 4 * 16 * NQ;  // queries per workgroup (4 wavefronts)
  constexpr int DS = D / 32;       // 32-wide d slices of the score contraction
  constexpr int DT = D / 16;       // 16-row d tiles of the output
  __shared__ __attribute__((aligned(16))) bf16_t klds[2][KB * D];
  __shared__ __attribute__((aligned(16))) bf16_t vlds[2][D * KB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int qb = gridDim.x - 1 - blockIdx.x;  // longest query blocks first
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.Hq / a.Hkv);
  const int S = a.S, W = a.window;
  const int q0 = qb * BQ;
  const int wq0 = q0 + wave * 16 * NQ;
  const int wq1 = min(wq0 + 16 * NQ, S) - 1;  // last valid query of this wavefront

  const bf16_t* qbase = (const bf16_t*)a.q + (int64_t)b * S * a.ldq + h * D;
  const bf16_t* kbase = (const bf16_t*)a.k + (int64_t)b * S * a.ldk + g * D;
  const bf16_t* vbase = (const bf16_t*)a.vt + (int64_t)(b * a.Hkv + g) * D * a.ldvt;

  // Qᵀ fragments (MFMA B operand): lane owns query wq0 + 16 nq + ln, d chunk 32 ds + 8 lg.
  bf16x8_t qf[NQ][DS];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const int qi = wq0 + nq * 16 + ln;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (qi < S) v = *reinterpret_cast<const u32x4_t*>(qbase + (int64_t)qi * a.ldq + ds * 32 + lg * 8);
      qf[nq][ds] = as_bf16x8(v);
    }
  }

  floatx4_t o[DT][NQ];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) o[dt][nq] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m[NQ], l[NQ];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    m[nq] = -INFINITY;
    l[nq] = 0.f;
  }

  const int kv_end = min(S, q0 + BQ);
  const int kv_begin = W > 0 ? max(0, q0 - W + 1) : 0;
  const int kb0 = kv_begin / KB, kb1 = (kv_end + KB - 1) / KB;

  KVLoader<D> ld;
  if (kb0 < kb1) {
    ld.load(kbase, a.ldk, vbase, a.ldvt, kb0 * KB, S, tid);
    ld.store(klds[0], vlds[0], tid);
  }
  __syncthreads();

  for (int kb = kb0; kb < kb1; ++kb) {
    const int cur = (kb - kb0) & 1;
    if (kb + 1 < kb1) ld.load(kbase, a.ldk, vbase, a.ldvt, (kb + 1) * KB, S, tid);

    const int j0 = kb * KB;
    const bool active = wq0 < S && j0 <= wq1 && !(W > 0 && j0 + KB - 1 < wq0 - W + 1);
    if (active) {
      const bf16_t* K = klds[cur];
      const bf16_t* V = vlds[cur];
      // Sᵀ[key, query]: tile t covers LDS rows 16 t .. 16 t + 15
      floatx4_t s[2][NQ];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) s[t][nq] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(K + k_off<D>(16 * t + ln, ds * 4 + lg)));
#pragma unroll
          for (int nq = 0; nq < NQ; ++nq) s[t][nq] = mfma_16x16x32_bf16(kf, qf[nq][ds], s[t][nq]);
        }
      }
      // register r of tile t in lane (ln, lg) is key j0 + 8 lg + 4 t + r, query wq0 + 16 nq + ln.
      // Blocks strictly below the diagonal and inside the window need no mask.
      const bool full = j0 + KB - 1 <= wq0 && (W <= 0 || wq1 - j0 < W);
      bf16x8_t pf[NQ];
      float mx[NQ];
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) {
        if (!full) {
          const int qi = wq0 + nq * 16 + ln;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int kj = j0 + 8 * lg + 4 * t + r;
              const bool vis = kj <= qi && kj < S && (W <= 0 || qi - kj < W);
              if (!vis) s[t][nq][r] = -INFINITY;
            }
        }
        float v = fmaxf(fmaxf(fmaxf(s[0][nq][0], s[0][nq][1]), fmaxf(s[0][nq][2], s[0][nq][3])),
                        fmaxf(fmaxf(s[1][nq][0], s[1][nq][1]), fmaxf(s[1][nq][2], s[1][nq][3])));
        v = fmaxf(v, __shfl_xor(v, 16, 64));
        v = fmaxf(v, __shfl_xor(v, 32, 64));
        mx[nq] = v * scale_log2;  // block max of the query's scaled scores (log2 units)
      }
      // Lazy rescaling: a query's reference max m moves only when the block max
      // exceeds it by more than 2^8, so probabilities stay <= 256 and the O / l
      // rescale (exact, by powers computed with exp2) is skipped on most blocks.
      bool need = false;
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) need |= mx[nq] > m[nq] + 8.f;
      if (__any(need)) {
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) {
          const float mnew = mx[nq] > m[nq] + 8.f ? mx[nq] : m[nq];
          const float corr = mnew == -INFINITY ? 1.f : fast_exp2(m[nq] - mnew);
          m[nq] = mnew;
          l[nq] *= corr;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt][nq] *= corr;
        }
      }
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) {
        const float mo = m[nq] == -INFINITY ? 0.f : m[nq];
        float p[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[4 * t + r] = fast_exp2(fmaf(s[t][nq][r], scale_log2, -mo));
        l[nq] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pf[nq] = as_bf16x8(u32x4_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                   pack_bf16x2(p[6], p[7])});
      }
      // Oᵀ[d, query] += Vᵀ[d, keys] · Pᵀ[keys, query]
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8_t vf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(V + v_off(dt * 16 + ln, lg)));
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) o[dt][nq] = mfma_16x16x32_bf16(vf, pf[nq], o[dt][nq]);
      }
    }
    if (kb + 1 < kb1) ld.store(klds[cur ^ 1], vlds[cur ^ 1], tid);
    __syncthreads();
  }

  // normalise and store: register r of d tile dt is dim 16 dt + 4 lg + r of query wq0 + 16 nq + ln
  bf16_t* obase = (bf16_t*)a.o + (int64_t)b * S * a.ldo + h * D;
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    float lt = l[nq];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const float inv = 1.f / lt;
    const int qi = wq0 + nq * 16 + ln;
    if (qi < S) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const floatx4_t v = o[dt][nq] * inv;
        *reinterpret_cast<u32x2_t*>(obase + (int64_t)qi * a.ldo + dt * 16 + lg * 4) =
            u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

// f32 path: one wavefront per (query, head); lanes stride over keys with their own
// running max / sum / accumulator, merged across the wavefront at the end.
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a, float scale_log2) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int g = h / (a.Hq / a.Hkv);
  const int S = a.S, W = a.window;
  const float* q = (const float*)a.q + ((int64_t)b * S + i) * a.ldq + h * D;
  const float* kbase = (const float*)a.k + (int64_t)b * S * a.ldk + g * D;
  const float* vbase = (const float*)a.vt + (int64_t)(b * a.Hkv + g) * D * a.ldvt;
  float qv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = q[d];
  float m = -INFINITY, l = 0.f, acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  const int jlo = W > 0 ? max(0, i - W + 1) : 0;
  for (int j = jlo + lane; j <= i; j += 64) {
    const float* k = kbase + (int64_t)j * a.ldk;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], k[d], s);
    s *= scale_log2;
    const float mn = fmaxf(m, s);
    const float corr = fast_exp2(m - mn), p = fast_exp2(s - mn);
    l = l * corr + p;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = acc[d] * corr + p * vbase[(int64_t)d * a.ldvt + j];
    m = mn;
  }
  const float mall = wave_max(m);
  const float f = m == -INFINITY ? 0.f : fast_exp2(m - mall);
  const float lt = wave_sum(l * f);
  float* o = (float*)a.o + ((int64_t)b * S + i) * a.ldo + h * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float v = wave_sum(acc[d] * f);
    if (lane == 0) o[d] = v / lt;
  }
}

// 64 tokens x 64 value columns per workgroup through an LDS tile.
template <typename T>
__global__ __launch_bounds__(256) void transpose_v_kernel(const T* __restrict__ src, int64_t ld, T* __restrict__ vt,
                                                         int ldvt, int S, int C) {
  constexpr int kV = 16 / sizeof(T);  // elements per 16-byte access
  constexpr int kPad = kV;
  __shared__ T tile[64][64 + kPad];
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64, b = blockIdx.z;
  for (int q = threadIdx.x; q < 64 * 64 / kV; q += 256) {
    const int r = q / (64 / kV), cv = (q % (64 / kV)) * kV;
    const int t = t0 + r, c = c0 + cv;
    T v[kV];
    if (t < S && c < C) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(src + ((int64_t)b * S + t) * ld + c);
      __builtin_memcpy(v, &x, 16);
    } else {
#pragma unroll
      for (int e = 0; e < kV; ++e) v[e] = T(0);
    }
#pragma unroll
    for (int e = 0; e < kV; ++e) tile[r][cv + e] = v[e];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * 64 / kV; q += 256) {
    const int ci = q / (64 / kV), tv = (q % (64 / kV)) * kV;
    const int c = c0 + ci, t = t0 + tv;
    if (c < C && t < S) {
      T v[kV];
#pragma unroll
      for (int e = 0; e < kV; ++e) v[e] = tile[tv + e][ci];
      u32x4_t x;
      __builtin_memcpy(&x, v, 16);
      *reinterpret_cast<u32x4_t*>(vt + ((int64_t)b * C + c) * ldvt + t) = x;
    }
  }
}

template <int D>
hipError_t launch_bf16(const AttnArgs& a, hipStream_t s) {
  const float sl = kLog2e / sqrtf((float)D);
  const int64_t heads = (int64_t)a.B * a.Hq;
  constexpr int kMaxNQ = D >= 256 ? 2 : 4;
  // largest per-wave query count that still gives >= 512 workgroups
  int nq = kMaxNQ;
  while (nq > 1 && heads * ((a.S + 64 * nq - 1) / (64 * nq)) < 512) nq >>= 1;
  const dim3 blk(256);
  switch (nq) {
    case 4:
      if constexpr (kMaxNQ >= 4) {
        hipLaunchKernelGGL((attn_bf16_kernel<D, 4>), dim3((a.S + 255) / 256, a.Hq, a.B), blk, 0, s, a, sl);
        break;
      }
      [[fallthrough]];
    case 2:
      hipLaunchKernelGGL((attn_bf16_kernel<D, 2>), dim3((a.S + 127) / 128, a.Hq, a.B), blk, 0, s, a, sl);
      break;
    default:
      hipLaunchKernelGGL((attn_bf16_kernel<D, 1>), dim3((a.S + 63) / 64, a.Hq, a.B), blk, 0, s, a, sl);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3(a.S, a.Hq, a.B), dim3(64), 0, s, a, kLog2e / sqrtf((float)D));
  return hipGetLastError();
}

}  // namespace

hipError_t transpose_v(DType dt, const void* src, int64_t ld, void* vt, int ldvt, int B, int S, int C,
                       hipStream_t s) {
  if (B <= 0 || S <= 0) return hipSuccess;
  const dim3 grid((S + 63) / 64, (C + 63) / 64, B);
  if (dt == DType::BF16)
    hipLaunchKernelGGL(transpose_v_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)src, ld, (bf16_t*)vt, ldvt,
                       S, C);
  else
    hipLaunchKernelGGL(transpose_v_kernel<float>, grid, dim3(256), 0, s, (const float*)src, ld, (float*)vt, ldvt, S,
                       C);
  return hipGetLastError();
}

bool attention_supported(DType dt, int D) {
  if (dt == DType::BF16) return D == 64 || D == 128 || D == 256;
  return D == 16 || D == 32 || D == 64;
}

hipError_t attention(DType dt, const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.S <= 0) return hipSuccess;
  if (dt == DType::BF16) {
    switch (a.D) {
      case 64: return launch_bf16<64>(a, s);
      case 128: return launch_bf16<128>(a, s);
      case 256: return launch_bf16<256>(a, s);
    }
  } else {
    switch (a.D) {
      case 16: return launch_f32<16>(a, s);
      case 32: return launch_f32<32>(a, s);
      case 64: return launch_f32<64>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fwdk
