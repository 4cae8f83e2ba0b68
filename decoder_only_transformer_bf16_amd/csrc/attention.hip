// Causal grouped-query attention with an optional sliding window
// ("N7 · model/forward-parity", intro: causal multi-head/GQA attention;
// "pegainfer issue #878", Description: a window of W keeps keys with i - j < W).
//
//   o[b,i,h,:] = sum_j p_ij v[b,j,g,:],  p_ij = softmax_j(q[b,i,h,:]·k[b,j,g,:] / sqrt(D)),
//   g = h / (Hq / Hkv), over keys j <= i (and i - j < W when W > 0).
//
// bf16 path (D in {64, 128, 256}): flash-style single pass with an online softmax.
// The score tile is computed transposed, Sᵀ = K·Qᵀ with v_mfma_f32_32x32x16_bf16,
// so that every lane owns one query column and 16 contiguous keys of a 32-key block:
// the softmax statistics are per lane except for one cross-lane max. The
// probabilities then feed Oᵀ += Vᵀ·Pᵀ straight from registers as the MFMA B operand;
// values are kept transposed (keys contiguous) so the A operand is a 16-byte LDS
// read. K and Vᵀ blocks stream global -> LDS by buffer loads through a 3-deep ring
// (two blocks in flight), and the score MFMAs of block j + 1 are issued before the
// softmax of block j so the two overlap. Registers are held to two wavefronts per
// SIMD, so one wavefront's softmax also overlaps the other's MFMAs.
//
// f32 path (D <= 64): one wavefront per query row on the vector ALUs.
#include "common.h"
#include "kernels.h"

namespace fwdk {
namespace {

constexpr int KB = 32;  // keys per block
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// K block in LDS: row R = 8 a + 4 g + b holds key 16 g + 4 a + b, so that in the
// transposed score tile Sᵀ = K·Qᵀ (v_mfma_f32_32x32x16_bf16, whose register r of lane
// (n, g) is row 8 (r / 4) + 4 g + r % 4) lane group g = l / 32 owns the 16 contiguous
// keys 16 g + r. Those 16 probabilities then feed Oᵀ += Vᵀ·Pᵀ directly as two MFMA B
// operands (keys 16 g + 8 m + 0..7 in MFMA m), matched by 16-byte reads of Vᵀ rows.
__device__ __forceinline__ int key_of_row(int R) { return ((R >> 2) & 1) * 16 + (R >> 3) * 4 + (R & 3); }

// 16-byte chunk swizzles: the 16 lanes an LDS read serves together read one chunk
// column of 16 consecutive rows, so (row's bank half, chunk) must differ across them.
template <int D>
__device__ __forceinline__ int kswz(int R, int c) {
  if constexpr (D == 64) return c ^ ((R >> 1) & 7);  // 128-byte rows: two rows per bank sweep
  else return c ^ (R & 15);                          // >= 256-byte rows
}
__device__ __forceinline__ int vswz(int d, int c) { return c ^ ((d >> 2) & 3); }  // 64-byte rows

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 1 KiB piece (64 lanes x 16 bytes) of a K or Vᵀ block, global -> LDS directly.
// Pieces 0 .. D/16-1 are K, D/16 .. D/8-1 are Vᵀ. Keys past the sequence read as zero
// (out of the buffer's range); the partial 8-key chunk at the end of Vᵀ rows reads the
// row padding, whose weight is exactly zero.
template <int D>
__device__ __forceinline__ void load_piece(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int64_t ldk, int ldvt,
                                           bf16_t* klds, bf16_t* vlds, int j0, int S, int piece, int lane) {
  constexpr int CH = D / 8, RPB = 64 / CH;  // K: chunks per row, rows per piece
  if (piece < D / 16) {
    const int R = piece * RPB + lane / CH;
    const int c = kswz<D>(R, lane % CH);
    const int key = j0 + key_of_row(R);
    const uint32_t off = key < S ? (uint32_t)(key * ldk + c * 8) * 2u : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(klds + piece * 512), 16, off, 0, 0, 0);
  } else {
    const int vp = piece - D / 16;
    const int d = vp * 16 + lane / 4;
    const int c = vswz(d, lane & 3);
    const int key = j0 + c * 8;
    const uint32_t off = key < S ? (uint32_t)(d * ldvt + key) * 2u : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(vlds + vp * 512), 16, off, 0, 0, 0);
  }
}

template <int D, int QT, int ST>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a, float scale_log2) {
  constexpr int QW = 32 * QT;      // queries per wavefront
  constexpr int BQ = 4 * QW;       // queries per workgroup
  constexpr int DS = D / 16;       // k-steps of the score contraction
  constexpr int DT = D / 32;       // 32-row d tiles of the output
  constexpr int PIECES = D / 8;    // 1 KiB loads per K+Vᵀ block
  constexpr int LPW = PIECES / 4;  // ... per wavefront
  constexpr int KSZ = KB * D, VSZ = D * KB;
  __shared__ __attribute__((aligned(1024))) bf16_t lds[ST * (KSZ + VSZ)];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 31, lg = lane >> 5;
  // One linear grid, decoded so that workgroups are dispatched longest query block
  // first across all heads and batch rows (causal work grows with the block index),
  // and so that the query heads of one KV head keep the same id modulo the number of
  // (batch row, KV head) pairs, which sends them to the same XCD when that number is
  // a multiple of 8.
  const int G = a.Hq / a.Hkv, BG = a.B * a.Hkv;
  const int per = a.Hq * a.B, nqb = gridDim.x / per;
  const int id = blockIdx.x, qo = id / per, rem = id - qo * per;
  const int hi = rem / BG, bg = rem - hi * BG;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv, h = g * G + hi;
  const int qb = nqb - 1 - qo;
  const int S = a.S, W = a.window;
  const int q0 = qb * BQ;
  const int wq0 = q0 + wave * QW;
  const int wq1 = min(wq0 + QW, S) - 1;  // last valid query of this wavefront

  const bf16_t* qbase = (const bf16_t*)a.q + (int64_t)b * S * a.ldq + h * D;
  const bf16_t* kbase = (const bf16_t*)a.k + (int64_t)b * S * a.ldk + g * D;
  const bf16_t* vbase = (const bf16_t*)a.vt + (int64_t)(b * a.Hkv + g) * D * a.ldvt;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, (int64_t)S * a.ldk * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, (int64_t)D * a.ldvt * 2);

  // Qᵀ fragments (MFMA B operand): lane owns query wq0 + 32 qt + ln, dims 16 ds + 8 lg .. + 7
  bf16x8_t qf[QT][DS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qi = wq0 + qt * 32 + ln;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (qi < S) v = *reinterpret_cast<const u32x4_t*>(qbase + (int64_t)qi * a.ldq + ds * 16 + lg * 8);
      qf[qt][ds] = as_bf16x8(v);
    }
  }
  wait_vmcnt<0>();

  // key blocks of the workgroup, and the active sub-range of this wavefront
  const int kv_end = min(S, q0 + BQ);
  const int kv_begin = W > 0 ? max(0, q0 - W + 1) : 0;
  const int kb0 = kv_begin / KB, kb1 = (kv_end + KB - 1) / KB;
  const int wb0 = W > 0 ? max(kb0, (wq0 - W + 1) / KB) : kb0;
  const int wb1 = wq0 < S ? min(kb1, wq1 / KB + 1) : kb0;  // empty when the wave has no queries
  auto active = [&](int kb) { return kb >= wb0 && kb < wb1; };

  auto issue_block = [&](int kb) {
    bf16_t* kl = lds + (kb % ST) * (KSZ + VSZ);
#pragma unroll
    for (int p = 0; p < LPW; ++p)
      load_piece<D>(rk, rv, a.ldk, a.ldvt, kl, kl + KSZ, kb * KB, S, wave + 4 * p, lane);
  };
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (kb0 + s < kb1) issue_block(kb0 + s);

  floatx16_t o[DT][QT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) o[dt][qt] = floatx16_t{};
  float m[QT], l[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.f;
  }

  // Sᵀ of block kb (K from its LDS buffer)
  auto scores = [&](int kb, floatx16_t (&sc)[QT]) {
    const bf16_t* K = lds + (kb % ST) * (KSZ + VSZ);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) sc[qt] = floatx16_t{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(K + ln * D + (kswz<D>(ln, 2 * ds + lg) << 3)));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) sc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qt][ds], sc[qt], 0, 0, 0);
    }
  };

  floatx16_t sc[QT], sn[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) sc[qt] = sn[qt] = floatx16_t{};
  if (kb0 < kb1) {
    if (kb0 + ST - 2 < kb1) wait_vmcnt<(ST - 2) * LPW>();
    else wait_vmcnt<0>();
  }
  lds_barrier();
  if (active(kb0)) scores(kb0, sc);

  for (int kb = kb0; kb < kb1; ++kb) {
    if (kb + 1 < kb1) {
      if (kb + ST - 2 < kb1) wait_vmcnt<(ST - 3) * LPW>();  // block kb + 1 has landed
      else wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_barrier();  // ... for everyone; and everyone is done with block kb - 1
      if (kb + ST - 1 < kb1) issue_block(kb + ST - 1);  // refill block kb - 1's buffer
      if (active(kb + 1)) scores(kb + 1, sn);  // MFMAs that overlap the softmax below
    }
    if (active(kb)) {
      const int j0 = kb * KB;
      // lane (ln, lg), register r of q tile qt: key j0 + 16 lg + r, query wq0 + 32 qt + ln.
      // Blocks strictly below the diagonal and inside the window need no mask.
      const bool full = j0 + KB - 1 <= wq0 && (W <= 0 || wq1 - j0 < W);
      float mx[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (!full) {
          // key j0 + 16 lg + r is visible from query qi iff 0 <= qi - key < window
          // (window = W if W > 0, else unbounded) and key < S
          const int qi = wq0 + qt * 32 + ln;
          const int d0 = qi - (j0 + 16 * lg);            // qi - key for r = 0
          const int wlim = W > 0 ? W : 0x7FFFFFFF;
          const int klim = S - (j0 + 16 * lg);           // r < klim <=> key < S
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int dd = d0 - r;
            const bool vis = (unsigned)dd < (unsigned)wlim && r < klim;
            sc[qt][r] = vis ? sc[qt][r] : -INFINITY;
          }
        }
        float v = sc[qt][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) v = fmaxf(v, sc[qt][r]);
        mx[qt] = v;
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) mx[qt] = fmaxf(mx[qt], __shfl_xor(mx[qt], 32, 64)) * scale_log2;
      // Lazy rescaling: the reference max m of a query moves only when a block max
      // exceeds it by more than 2^8, so probabilities stay <= 256 and the O / l
      // rescale (exact powers of exp2) is skipped on most blocks.
      bool need = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) need |= mx[qt] > m[qt] + 8.f;
      if (__any(need)) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float mnew = mx[qt] > m[qt] + 8.f ? mx[qt] : m[qt];
          const float corr = mnew == -INFINITY ? 1.f : fast_exp2(m[qt] - mnew);
          m[qt] = mnew;
          l[qt] *= corr;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt][qt] *= corr;
        }
      }
      bf16x8_t pf[QT][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mo = m[qt] == -INFINITY ? 0.f : m[qt];
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(sc[qt][r], scale_log2, -mo));
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) ps += p[r];
        l[qt] += ps;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
          pf[qt][mm] = as_bf16x8(u32x4_t{pack_bf16x2(p[8 * mm + 0], p[8 * mm + 1]), pack_bf16x2(p[8 * mm + 2], p[8 * mm + 3]),
                                         pack_bf16x2(p[8 * mm + 4], p[8 * mm + 5]), pack_bf16x2(p[8 * mm + 6], p[8 * mm + 7])});
      }
      // Oᵀ[d, query] += Vᵀ[d, keys] · Pᵀ[keys, query]
      const bf16_t* V = lds + (kb % ST) * (KSZ + VSZ) + KSZ;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 32 + ln;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const bf16x8_t vf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(V + d * KB + (vswz(d, 2 * lg + mm) << 3)));
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qt][mm], o[dt][qt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) sc[qt] = sn[qt];
  }

  // normalise and store: register r of d tile dt is dim 32 dt + 8 (r / 4) + 4 lg + r % 4
  // o row b * S + qi, columns h * D + d: row-major with stride ldo, or K-tiled with
  // row width ldo (four consecutive columns never cross a 32-wide tile)
  bf16_t* obase = (bf16_t*)a.o + (a.o_tiled ? 0 : (int64_t)b * S * a.ldo + h * D);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float lt = l[qt];
    lt += __shfl_xor(lt, 32, 64);
    const float inv = 1.f / lt;
    const int qi = wq0 + qt * 32 + ln;
    if (qi < S) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const floatx16_t& v = o[dt][qt];
          const int d = dt * 32 + a4 * 8 + lg * 4;
          const int64_t at = a.o_tiled ? tiled_index((int64_t)b * S + qi, h * D + d, (int)a.ldo) : (int64_t)qi * a.ldo + d;
          *reinterpret_cast<u32x2_t*>(obase + at) =
              u32x2_t{pack_bf16x2(v[4 * a4] * inv, v[4 * a4 + 1] * inv), pack_bf16x2(v[4 * a4 + 2] * inv, v[4 * a4 + 3] * inv)};
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
  const dim3 blk(256);
  // two 32-query tiles per wavefront only where they fit beside two wavefronts per
  // SIMD without spilling (D = 64), and only when the grid stays full
  if constexpr (D == 64) {
    if (heads * ((a.S + 255) / 256) >= 512) {
      hipLaunchKernelGGL((attn_bf16_kernel<D, 2, 3>), dim3((a.S + 255) / 256 * heads), blk, 0, s, a, sl);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_bf16_kernel<D, 1, 3>), dim3((a.S + 127) / 128 * heads), blk, 0, s, a, sl);
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
  if (a.o_tiled && (dt != DType::BF16 || a.ldo != (int64_t)a.Hq * a.D || a.ldo % 32)) return hipErrorInvalidValue;
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
