// Shared device helpers for the gfx950 kernels: element types, vector types,
// conversions, wavefront reductions and the MFMA wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fwdk {

typedef uint16_t bf16_t;  // bf16 storage: the upper 16 bits of an IEEE binary32

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> bf16 conversions in one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return bf16_t(pack_bf16x2(f, 0.f) & 0xFFFFu); }

// Element type traits: load/store one value through fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Wavefront-wide reductions (64 lanes) through cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 dword3: 32-bit data
// format, the value untyped loads require). Loads whose offset lies past `bytes`
// return zero, which pads the ragged edges of a tile without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Every lane of an aligned group of N lanes (N = 4, 8, 16 or 32) gets the group's sum,
// through DPP moves within rows of 16 lanes (and one shuffle across rows for 32).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group of 4, 8, 16 or 32 lanes");
  v += dpp_mov<0xB1>(v);                          // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);                          // quad_perm [2, 3, 0, 1]: quad sums
  if constexpr (N >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror: lane i <- 7 - i within 8 lanes
  if constexpr (N >= 16) v += dpp_mov<0x140>(v);  // row_mirror: lane i <- 15 - i
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

// 8 bf16 values (16 bytes) widened to fp32, and packed back with rounding to nearest even.
__device__ __forceinline__ void unpack8(const u32x4_t& u, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ u32x4_t pack8(const float (&f)[8]) {
  u32x4_t u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return u;
}

// exp2 on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// 1/x and 1/sqrt(x) on the hardware units (v_rcp_f32, v_rsq_f32).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

// K-tiled bf16 operand layout: a [rows, K] matrix (K a multiple of 32) stored as
// 16 x 32 tiles of 1 KiB, tile (r / 16, c / 32) at element ((r / 16) * (K / 32) +
// c / 32) * 512, row-major inside the tile. A GEMM reads one tile per 64-lane
// 16-byte load, i.e. 1 KiB of contiguous memory, where a row-major layout would
// touch sixteen half cache lines. Row count is padded to a multiple of 16.
__device__ __forceinline__ int64_t tiled_index(int64_t r, int c, int K) {
  return ((r >> 4) * (K >> 5) + (c >> 5)) * 512 + (r & 15) * 32 + (c & 31);
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence makes
// the compiler drain every outstanding buffer->LDS load (vmcnt(0)) first, which
// would empty a multi-stage load pipeline at each step. Callers wait for exactly
// what they need (s_waitcnt vmcnt / lgkmcnt) before calling it; the "memory"
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

constexpr float kLog2e = 1.4426950408889634f;

// MFMA wrappers (CDNA4): D = A * B + C with fp32 accumulation.
__device__ __forceinline__ floatx16_t mfma_32x32x16_bf16(const bf16x8_t& a, const bf16x8_t& b,
                                                         const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4_t mfma_16x16x32_bf16(const bf16x8_t& a, const bf16x8_t& b,
                                                        const floatx4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace fwdk
