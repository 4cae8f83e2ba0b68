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
// read. K and Vᵀ blocks stream global -> LDS by buffer loads through a 3-deep ring.
// Each step of the block loop issues the next block's score MFMAs in one basic block
// with this block's exponentials, then the value MFMAs (for D = 64 all the step's MFMA
// fragments are read from LDS first). The normaliser sums the bf16 probabilities the
// value product uses. With two or three wavefronts per SIMD, one wavefront's vector
// work overlaps another's MFMAs.
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

// One K + Vᵀ block, global -> LDS by buffer loads into `kl` (1 KiB pieces of 64 lanes x
// 16 bytes; pieces 0 .. D/16 - 1 are K, the rest Vᵀ; this wavefront takes pieces
// wave + 4 p, so p < LPW / 2 are K pieces). loff[p] is the lane's byte offset relative
// to the block's first key. The buffer resources start at the block: K keys past S
// fall outside the K range and read as zero; Vᵀ chunks (8 keys) at or past S are given
// an offset outside the range in the last block, and the partial chunk before S reads
// the zero padding of the Vᵀ rows. (A device function, not a lambda: a lambda in a
// kernel is also compiled for the host, where the resource type does not exist.)
template <int D>
__device__ __forceinline__ void load_block(const bf16_t* kbase, const bf16_t* vbase, int64_t ldk, int ldvt, int S,
                                           int j0, bf16_t* kl, const uint32_t* loff, int wave, int lane) {
  constexpr int LPW = D / 32, KSZ = KB * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (int64_t)j0 * ldk, (int64_t)(S - j0) * ldk * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + j0, ((int64_t)D * ldvt - j0) * 2);
  const bool tail = j0 + KB > S;
#pragma unroll
  for (int p = 0; p < LPW; ++p) {
    const int piece = wave + 4 * p;
    if (p < LPW / 2) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(kl + piece * 512), 16, loff[p], 0, 0, 0);
    } else {
      const int vp = piece - D / 16;
      uint32_t off = loff[p];
      if (tail) {
        const int d = vp * 16 + lane / 4;
        if (j0 + vswz(d, lane & 3) * 8 >= S) off = 0x80000000u;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(kl + KSZ + vp * 512), 16, off, 0, 0, 0);
    }
  }
}

// Cross-half maximum: lanes l and l ^ 32 (the two halves of one query's keys) swap
// values by one v_permlane32_swap, no LDS round trip.
__device__ __forceinline__ float max_halves(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

// Wavefronts per SIMD the registers are held to, and whether a block's MFMA fragments
// are read from LDS ahead of its softmax. D = 128: three (three 48 KiB workgroups per
// CU), fragments read just before their MFMAs; in the Llama-shape forward this is 8%
// faster than two wavefronts reading ahead. D = 64: two, reading ahead (11% faster).
template <int D>
constexpr int attn_waves_per_simd() { return D == 128 ? 3 : 2; }
template <int D, int QT>
constexpr bool attn_read_ahead() { return QT == 1 && D == 64; }

template <int D, int QT, int ST>
__global__ __launch_bounds__(256, (attn_waves_per_simd<D>())) void attn_bf16_kernel(AttnArgs a, float scale_log2) {
  constexpr int QW = 32 * QT;      // queries per wavefront
  constexpr int BQ = 4 * QW;       // queries per workgroup
  constexpr int DS = D / 16;       // k-steps of the score contraction
  constexpr int DT = D / 32;       // 32-row d tiles of the output
  constexpr int LPW = D / 32;      // 1 KiB pieces per wavefront per block: D / 8 over 4 wavefronts
  constexpr int KSZ = KB * D, VSZ = D * KB, SLOT = KSZ + VSZ;
  // The loop is unrolled so that both the ring slot of a block (its index since the
  // first block, modulo ST) and the score buffer it uses (modulo 2) are constants:
  // LDS reads then take immediate offsets, and no scores are copied between buffers.
  constexpr int UNROLL = ST % 2 ? 2 * ST : ST;
  constexpr bool READ_AHEAD = attn_read_ahead<D, QT>();
  __shared__ __attribute__((aligned(1024))) bf16_t lds[ST * SLOT];

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

  // Block loads: 1 KiB pieces (64 lanes x 16 bytes) global -> LDS by buffer loads.
  // Pieces 0 .. D/16 - 1 are the K block, the rest its Vᵀ block; this wavefront takes
  // pieces wave + 4 p, so that p < LPW / 2 are K pieces. Byte offsets relative to the
  // block's first key are the same for every block.
  uint32_t loff[LPW];
#pragma unroll
  for (int p = 0; p < LPW; ++p) {
    const int piece = wave + 4 * p;
    if (p < LPW / 2) {
      constexpr int CH = D / 8, RPB = 64 / CH;  // chunks per K row, rows per piece
      const int R = piece * RPB + lane / CH;
      loff[p] = (uint32_t)(key_of_row(R) * a.ldk + kswz<D>(R, lane % CH) * 8) * 2u;
    } else {
      const int d = (piece - D / 16) * 16 + lane / 4;
      loff[p] = (uint32_t)(d * a.ldvt + vswz(d, lane & 3) * 8) * 2u;
    }
  }
  // key blocks of the workgroup, and the active sub-range of this wavefront
  const int kv_end = min(S, q0 + BQ);
  const int kv_begin = W > 0 ? max(0, q0 - W + 1) : 0;
  const int kb0 = kv_begin / KB, kb1 = (kv_end + KB - 1) / KB;
  const int wb0 = W > 0 ? max(kb0, (wq0 - W + 1) / KB) : kb0;
  const int wb1 = wq0 < S ? min(kb1, wq1 / KB + 1) : kb0;  // empty when the wave has no queries
  auto active = [&](int kb) { return kb >= wb0 && kb < wb1; };

#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (kb0 + s < kb1) load_block<D>(kbase, vbase, a.ldk, a.ldvt, S, (kb0 + s) * KB, lds + s * SLOT, loff, wave, lane);

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
  floatx16_t sb[2][QT];  // scores of the current block and of the next one

  // Sᵀ of the block in ring slot `slot` into score buffer `par`
  auto scores = [&](int slot, int par) __attribute__((always_inline)) {
    const bf16_t* K = lds + slot * SLOT;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) sb[par][qt] = floatx16_t{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(K + ln * D + (kswz<D>(ln, 2 * ds + lg) << 3)));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        sb[par][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qt][ds], sb[par][qt], 0, 0, 0);
    }
  };
  // Causal / window / length mask of block kb: lane (ln, lg), register r of q tile qt
  // is key j0 + 16 lg + r against query wq0 + 32 qt + ln.
  auto mask = [&](int kb, int par) __attribute__((always_inline)) {
    const int j0 = kb * KB;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      // key j0 + 16 lg + r is visible from query qi iff 0 <= qi - key < window
      // (window = W if W > 0, else unbounded) and key < S
      const int qi = wq0 + qt * 32 + ln;
      const int d0 = qi - (j0 + 16 * lg);  // qi - key for r = 0
      const int wlim = W > 0 ? W : 0x7FFFFFFF;
      const int klim = S - (j0 + 16 * lg);  // r < klim <=> key < S
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dd = d0 - r;
        const bool vis = (unsigned)dd < (unsigned)wlim && r < klim;
        sb[par][qt][r] = vis ? sb[par][qt][r] : -INFINITY;
      }
    }
  };
  // Row maxima (scaled to log2 units), and the lazy rescaling: the reference max m of
  // a query moves only when a block max exceeds it by more than 2^8, so probabilities
  // stay <= 256 and the O / l rescale (exact powers of exp2) is skipped on most blocks.
  auto max_and_rescale = [&](int par) __attribute__((always_inline)) {
    float mx[QT];
    bool need = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float v = sb[par][qt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) v = fmaxf(v, sb[par][qt][r]);
      mx[qt] = max_halves(v) * scale_log2;
      need |= mx[qt] > m[qt] + 8.f;
    }
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
  };
  // Probabilities p = exp2(s log2e / sqrt(D) - m) as bf16 MFMA B operands. The
  // normaliser l sums the same bf16 values the value product weights (two per
  // v_dot2 with ones), so the weights of a query sum to one.
  auto probs = [&](int par, bf16x8_t (&pf)[QT][2]) __attribute__((always_inline)) {
    const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float nmo = m[qt] == -INFINITY ? 0.f : -m[qt];
      uint32_t pk[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pk[i] = pack_bf16x2(fast_exp2(fmaf(sb[par][qt][2 * i], scale_log2, nmo)),
                            fast_exp2(fmaf(sb[par][qt][2 * i + 1], scale_log2, nmo)));
      float s = l[qt];
#pragma unroll
      for (int i = 0; i < 8; ++i) s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[i]), ones, s, false);
      l[qt] = s;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
        pf[qt][mm] = as_bf16x8(u32x4_t{pk[4 * mm], pk[4 * mm + 1], pk[4 * mm + 2], pk[4 * mm + 3]});
    }
  };
  // Oᵀ[d, query] += Vᵀ[d, keys] · Pᵀ[keys, query], the d tiles innermost so that
  // consecutive MFMAs accumulate into different registers
  auto pv = [&](int slot, const bf16x8_t (&pf)[QT][2]) __attribute__((always_inline)) {
    const bf16_t* V = lds + slot * SLOT + KSZ;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 32 + ln;
        const bf16x8_t vf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(V + d * KB + (vswz(d, 2 * lg + mm) << 3)));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qt][mm], o[dt][qt], 0, 0, 0);
      }
  };
  // The same two products from fragments read ahead: all K fragments of a block and all
  // Vᵀ fragments are read from LDS before the block's softmax, so that no MFMA waits on
  // the LDS read issued just before it.
  auto read_k = [&](int slot, bf16x8_t (&kf)[DS]) __attribute__((always_inline)) {
    const bf16_t* K = lds + slot * SLOT;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      kf[ds] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(K + ln * D + (kswz<D>(ln, 2 * ds + lg) << 3)));
  };
  auto read_v = [&](int slot, bf16x8_t (&vf)[2][DT]) __attribute__((always_inline)) {
    const bf16_t* V = lds + slot * SLOT + KSZ;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 32 + ln;
        vf[mm][dt] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(V + d * KB + (vswz(d, 2 * lg + mm) << 3)));
      }
  };
  auto scores_from = [&](const bf16x8_t (&kf)[DS], int par) __attribute__((always_inline)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) sb[par][qt] = floatx16_t{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        sb[par][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds], qf[qt][ds], sb[par][qt], 0, 0, 0);
  };
  auto pv_from = [&](const bf16x8_t (&vf)[2][DT], const bf16x8_t (&pf)[QT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[mm][dt], pf[qt][mm], o[dt][qt], 0, 0, 0);
  };

  if (kb0 < kb1) {
    if (kb0 + ST - 2 < kb1) wait_vmcnt<(ST - 2) * LPW>();
    else wait_vmcnt<0>();
  }
  lds_barrier();
  if (active(kb0)) scores(0, 0);

  for (int kb = kb0; kb < kb1; kb += UNROLL) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = kb + u;
      if (k >= kb1) break;
      const int slot = u % ST, par = u & 1;
      const bool has_next = k + 1 < kb1;
      if (has_next) {
        if (k + ST - 2 < kb1) wait_vmcnt<(ST - 3) * LPW>();  // block k + 1 has landed
        else wait_vmcnt<0>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();  // ... for everyone; and everyone is done with block k - 1
        if (k + ST - 1 < kb1)  // refill block k - 1's slot
          load_block<D>(kbase, vbase, a.ldk, a.ldvt, S, (k + ST - 1) * KB, lds + (u + ST - 1) % ST * SLOT, loff, wave,
                        lane);
      }
      const bool act = active(k), act1 = has_next && active(k + 1);
      const int j0 = k * KB;
      // blocks strictly below the diagonal and inside the window need no mask
      const bool full = j0 + KB - 1 <= wq0 && (W <= 0 || wq1 - j0 < W);
      if (act && READ_AHEAD) {
        bf16x8_t kf[DS], vf[2][DT], pf[QT][2];
        read_k((u + 1) % ST, kf);
        read_v(slot, vf);
        if (!full) mask(k, par);
        max_and_rescale(par);
        // one basic block: the next block's score MFMAs interleave with this block's
        // exponentials (after the wavefront's last block they read a stale slot and
        // are not used)
        scores_from(kf, par ^ 1);
        probs(par, pf);
        pv_from(vf, pf);
        // issue order: each score MFMA of the next block followed by a share of the
        // vector work that makes the first half of P, then the first half's value
        // MFMAs each followed by a share of the second half's, then the rest
#pragma unroll
        for (int i = 0; i < DS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 24 / DS, 0);
        }
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 26 / DT, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, DT, 0);
      } else if (act) {
        if (!full) mask(k, par);
        max_and_rescale(par);
        bf16x8_t pf[QT][2];
        scores((u + 1) % ST, par ^ 1);
        probs(par, pf);
        pv(slot, pf);
      } else if (act1) {
        scores((u + 1) % ST, par ^ 1);
      }
    }
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
