// Device-side helpers shared by the gfx950 kernels of the Palu library.
// CDNA4 only: 64-lane wavefronts, MFMA matrix cores, LDS DMA and LDS
// transpose reads.  Lane layouts used below were checked on gfx950:
//   v_mfma_f32_16x16x32_{f16,bf16}: A lane l -> row l%16, k = 8*(l/16)+[0..7];
//     B lane l -> col l%16, same k; C lane l -> col l%16, rows 4*(l/16)+[0..3].
//   v_mfma_f32_16x16x4_f32: A lane l -> row l%16, k = l/16; B col l%16, k = l/16.
//   ds_read_b64_tr_b16: in each 16-lane group, source lane s = 4e+q addresses
//     4 consecutive 16-bit elements (row e, columns 4q..4q+3) of a row-major
//     tile; result lane i receives element i of rows e = 0..3.
//   global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace palu {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define PALU_LDS __attribute__((address_space(3)))

// 8 x 16-bit operand of a 16x16x32 MFMA, for element type T.
template <class T> struct Vec8;
template <> struct Vec8<_Float16> { typedef f16x8 type; };
template <> struct Vec8<__bf16> { typedef bf16x8 type; };

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16-byte global -> LDS copy; `lds_wave_base` must be wave-uniform, lane l
// writes bytes [16*l, 16*l+16) after it.  Issued from an asm block (M0 is set
// in the same block; there are no register outputs) so that the compiler
// does not order later LDS reads of other buffers behind it: callers wait
// with wait_vmcnt<N>() and a barrier before reading the destination.
__device__ __forceinline__ void dma16(const void* gsrc, unsigned lds_wave_base) {
  const unsigned lds = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(gsrc)
               : "memory", "m0");
}
// 16-byte global -> LDS copy from a wave-uniform base plus a per-lane 32-bit
// byte offset; lane l lands at LDS byte `lds_wave_base` + 16*l.
__device__ __forceinline__ void dma16s(const void* base, unsigned voff, unsigned lds_wave_base) {
  const uint64_t a = (uint64_t)base;
  // (readfirstlane returns int: each half goes through unsigned, so that the
  // low half is zero-extended)
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  const unsigned lds = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sb)
               : "memory", "m0");
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(const PALU_LDS void*)p;
}

// s_waitcnt vmcnt(N) leaving lgkmcnt / expcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}
// Workgroup barrier without the memory fence of __syncthreads(): outstanding
// LDS-DMA prefetches are not drained.  Callers order their own accesses.
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

// Scalar load of a wave-uniform 32-bit value (waits in the same block; it
// counts in lgkmcnt, so it leaves the vector-memory counter of DMA in flight
// alone).
__device__ __forceinline__ int sload_i32(const int* ptr) {
  const uint64_t a = (uint64_t)ptr;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(u) : "memory");
  return v;
}

__device__ __forceinline__ i16x4 ds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((PALU_LDS i16x4*)lds_addr);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48) with the
// gfx950 row-swap permutes (VALU only).  permlane16_swap(a, b) exchanges the
// odd rows of a with the even rows of b; permlane32_swap(a, b) exchanges the
// upper half of a with the lower half of b.  With a == b == x the two
// results of each swap hold the row pair, so every lane ends with the same
// value, summed in the same order.
__device__ __forceinline__ float rows4_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows4_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Reductions over each half-wave (32 lanes): DPP butterflies inside a 16-lane
// row (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror), then the row pair through permlane16_swap.  Every lane of the
// half receives the result (sums may differ by rounding order between lanes).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max32(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float sum32(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
// x + (value of lane l ^ 32)
__device__ __forceinline__ float halves_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, 64); }

// Round-to-nearest-even conversions from binary32.
template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

template <class T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace palu
