// Projections Y = X·Wᵀ ("N9 · metalgemm", Theorem 1: X [P, in], W [out, in],
// both row-major, fp32 accumulation) with the fused epilogues of the forward pass:
// plain fp32 store (+ final-logit softcap, "pegainfer issue #878"), residual add,
// SwiGLU, and RoPE on the query/key heads ("N7 · model/forward-parity", intro).
//
// bf16 path: CDNA4 MFMA v_mfma_f32_32x32x16_bf16, one 64-wide wavefront per
// (BM/WM) x (BN/WN) sub-tile, K staged through LDS in 64-wide slices, double
// buffered, with the next slice's global loads in flight during the MFMAs.
// f32 path: an LDS-tiled VALU kernel (the fp32 configuration is tiny).
#include "common.h"
#include "kernels.h"

namespace fwdk {
namespace {

// ------------------------------------------------------------------ epilogues
// Every epilogue receives pairs of accumulator values (v0 at packed column c,
// v1 at packed column c + C) of one output row. ok0 / ok1 flag columns < N.

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
};

template <int C>
struct EpiResidual {
  const float* xin;
  float* xout;
  int64_t ld;
  __device__ __forceinline__ void pair(int row, int c, float v0, float v1, bool ok0, bool ok1) const {
    const int64_t i = (int64_t)row * ld + c;
    if (ok0) xout[i] = xin[i] + v0;
    if (ok1) xout[i + C] = xin[i + C] + v1;
  }
};

template <int C, typename T>
struct EpiSwiGLU {
  T* a;
  int F;
  __device__ __forceinline__ void pair(int row, int c, float g, float u, bool ok0, bool) const {
    if (!ok0) return;
    const int f = (c / (2 * C)) * C + (c % C);
    // silu(g) = g / (1 + e^{-g})
    const float s = g * fast_rcp(1.f + fast_exp2(-kLog2e * g));
    Elem<T>::store(a + (int64_t)row * F + f, s * u);
  }
};

template <int C, typename T>
struct EpiRope {
  T* qk;
  T* vt;
  const float2* cs;
  int Hq, Hkv, D, S, ldvt;
  __device__ __forceinline__ void pair(int row, int c, float v0, float v1, bool ok0, bool) const {
    if (!ok0) return;
    const int qsz = Hq * D, ksz = Hkv * D;
    const int b = row / S, t = row - b * S;
    if (c < qsz + ksz) {
      const int sec = c < qsz ? 0 : qsz;
      const int cc = c - sec;
      const int head = cc / D, pd = cc - head * D;
      const int k = (pd / (2 * C)) * C + (pd % C);  // rotation index in [0, D/2)
      const float2 r = cs[(int64_t)t * (D / 2) + k];
      const float a = v0 * r.x - v1 * r.y;
      const float bb = v0 * r.y + v1 * r.x;
      T* dst = qk + (int64_t)row * (qsz + ksz) + sec + head * D + k;
      Elem<T>::store(dst, a);
      Elem<T>::store(dst + D / 2, bb);
    } else {
      const int cc = c - qsz - ksz;  // value columns are not permuted
      const int g = cc / D, d = cc - g * D;
      T* dst = vt + ((int64_t)(b * Hkv + g) * D + d) * ldvt + t;
      Elem<T>::store(dst, v0);
      Elem<T>::store(dst + (int64_t)C * ldvt, v1);
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
constexpr int BK = 64;  // K slice staged in LDS: 8 chunks of 16 bytes per row

// LDS element offset of 16-byte chunk c of tile row r (XOR swizzle on chunks so
// that the 32-row fragment reads and the row-wise writes spread over all banks).
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }

template <int ROWS, int NT>
struct SliceLoader {
  static constexpr int kPer = ROWS * (BK / 8) / NT;
  static_assert(kPer * NT == ROWS * (BK / 8), "tile rows must fill the workgroup");
  u32x4_t v[kPer];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ base, int64_t ld, int row0, int nrows, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int q = tid + p * NT;
      const int r = q >> 3, c = q & 7;
      const int gr = row0 + r, gk = k0 + c * 8;
      if (gr < nrows && gk < K)
        v[p] = *reinterpret_cast<const u32x4_t*>(base + (int64_t)gr * ld + gk);
      else
        v[p] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int q = tid + p * NT;
      *reinterpret_cast<u32x4_t*>(lds + lds_off(q >> 3, q & 7)) = v[p];
    }
  }
};

template <int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(const bf16_t* __restrict__ X,
                                                               const bf16_t* __restrict__ W, int M, int N,
                                                               int K, Epi epi) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TN % 2 == 0, "pair epilogues need an even number of 32-column sub-tiles");
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][(BM + BN) * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int nTM = (M + BM - 1) / BM, nTN = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, nTM, nTN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  floatx16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16_t{};

  SliceLoader<BM, NT> la;
  SliceLoader<BN, NT> lb;
  const int nk = (K + BK - 1) / BK;
  la.load(X, K, m0, M, 0, K, tid);
  lb.load(W, K, n0, N, 0, K, tid);
  la.store(lds[0], tid);
  lb.store(lds[0] + BM * BK, tid);
  __syncthreads();

  const int lr = lane & 31, lk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(X, K, m0, M, (kt + 1) * BK, K, tid);
      lb.load(W, K, n0, N, (kt + 1) * BK, K, tid);
    }
    const bf16_t* As = lds[cur];
    const bf16_t* Bs = lds[cur] + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(As + lds_off(wm * WTM + i * 32 + lr, kk * 2 + lk)));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(Bs + lds_off(wn * WTN + j * 32 + lr, kk * 2 + lk)));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16_bf16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      la.store(lds[cur ^ 1], tid);
      lb.store(lds[cur ^ 1] + BM * BK, tid);
    }
    __syncthreads();
  }

  // Accumulator layout of v_mfma_f32_32x32x16: register r of lane l holds
  // row 8 (r / 4) + 4 (l / 32) + r % 4 and column l % 32 of the 32x32 sub-tile.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jp = 0; jp < TN / 2; ++jp) {
      const int c = n0 + wn * WTN + jp * 64 + lr;
      const bool ok0 = c < N, ok1 = c + 32 < N;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
        if (row < M) epi.pair(row, c, acc[i][2 * jp][r], acc[i][2 * jp + 1][r], ok0, ok1);
      }
    }
}

// ------------------------------------------------------------------ f32 VALU kernel
// 64x64 output tile, 256 threads, 4x4 outputs per thread, K slices of 16.
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                                                      int M, int N, int K, Epi epi) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int nTN = (N + 63) / 64;
  const int m0 = (blockIdx.x / nTN) * 64, n0 = (blockIdx.x % nTN) * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int e = tid + p * 256, r = e >> 4, k = e & 15;
      As[k][r] = (m0 + r < M && k0 + k < K) ? X[(int64_t)(m0 + r) * K + k0 + k] : 0.f;
      Bs[k][r] = (n0 + r < N && k0 + k < K) ? W[(int64_t)(n0 + r) * K + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int c = n0 + tx * 4 + 2 * jp;
      epi.pair(row, c, acc[i][2 * jp], acc[i][2 * jp + 1], c < N, c + 1 < N);
    }
  }
}

// ------------------------------------------------------------------ dispatch
template <class Epi>
hipError_t launch_bf16(const void* X, const void* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int64_t big = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  if (big >= 256) {
    const int grid = ((M + 255) / 256) * ((N + 255) / 256);
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 2, Epi>), dim3(grid), dim3(256), 0, s,
                       (const bf16_t*)X, (const bf16_t*)W, M, N, K, epi);
  } else {
    const int grid = ((M + 127) / 128) * ((N + 127) / 128);
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, Epi>), dim3(grid), dim3(256), 0, s,
                       (const bf16_t*)X, (const bf16_t*)W, M, N, K, epi);
  }
  return hipGetLastError();
}

template <class Epi>
hipError_t launch_f32(const void* X, const void* W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int grid = ((M + 63) / 64) * ((N + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<Epi>), dim3(grid), dim3(256), 0, s, (const float*)X, (const float*)W, M, N,
                     K, epi);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_store(DType dt, const void* X, const void* W, float* Y, int64_t ldy, int M, int N, int K,
                      float softcap, hipStream_t s) {
  if (dt == DType::BF16) return launch_bf16(X, W, M, N, K, EpiStore<32>{Y, ldy, softcap}, s);
  return launch_f32(X, W, M, N, K, EpiStore<1>{Y, ldy, softcap}, s);
}

hipError_t gemm_residual(DType dt, const void* X, const void* W, const float* xin, float* xout, int M, int N,
                         int K, hipStream_t s) {
  if (dt == DType::BF16) return launch_bf16(X, W, M, N, K, EpiResidual<32>{xin, xout, N}, s);
  return launch_f32(X, W, M, N, K, EpiResidual<1>{xin, xout, N}, s);
}

hipError_t gemm_swiglu(DType dt, const void* X, const void* W, void* a, int M, int F, int K, hipStream_t s) {
  if (dt == DType::BF16) return launch_bf16(X, W, M, 2 * F, K, EpiSwiGLU<32, bf16_t>{(bf16_t*)a, F}, s);
  return launch_f32(X, W, M, 2 * F, K, EpiSwiGLU<1, float>{(float*)a, F}, s);
}

hipError_t gemm_qkv_rope(DType dt, const void* X, const void* W, const RopeArgs& r, int M, int K, hipStream_t s) {
  const int N = (r.Hq + 2 * r.Hkv) * r.D;
  if (dt == DType::BF16)
    return launch_bf16(X, W, M, N, K,
                       EpiRope<32, bf16_t>{(bf16_t*)r.qk, (bf16_t*)r.vt, r.cs, r.Hq, r.Hkv, r.D, r.S, r.ldvt}, s);
  return launch_f32(X, W, M, N, K,
                    EpiRope<1, float>{(float*)r.qk, (float*)r.vt, r.cs, r.Hq, r.Hkv, r.D, r.S, r.ldvt}, s);
}

}  // namespace fwdk
