// Symmetric int4 quantisation of latent rows (gfx950).
//
// Quantization stacks with the low-rank cache (arXiv 2407.21118v2 abstract:
// low-rank-aware quantization compatibility; PALU page, section "Rollout",
// route C).  The pages do not define the quantizer; this one is plain
// symmetric int4 with one binary16 scale per 32 consecutive elements of a
// token's latent row:  s = fp16(amax / 7) (IEEE binary32 divide, round to
// nearest even), code = clamp(rint(z / s), -7, 7) (binary32 divide, ties to
// even), code = 0 where s == 0; element 2i in the low nibble of byte i.
#include "common.h"
#include "quant.h"
#include "int4.h"

#include <type_traits>

namespace palu {

// One thread per (row, 32-element chunk).  Stores 16 bytes of codes and one
// binary16 scale.  The chunk's 32 loads are issued before any is used (the
// index is clamped inside the row, values past the rank are dropped after).
// code = rint(fl(z / s)) needs the correctly rounded binary32 quotient only
// where it decides the rounding: t = z * fl(1 / s) lies within 1.5e-6 of
// fl(z / s) for |t| < 8 (two roundings of relative size 2^-24 each), so
// rint(t) is the code unless t is within 4e-6 of a half-integer, where the
// exact quotient is formed; beyond |t| >= 8 both clamp to +-7.
template <class T>
__global__ void __launch_bounds__(256) palu_quant_kernel(const T* __restrict__ z, int64_t n_rows, int r,
                                                         int64_t stride, uint8_t* __restrict__ codes,
                                                         _Float16* __restrict__ scales) {
  const int nc = cdiv(r, 32);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_rows * nc) return;
  const int64_t row = idx / nc;
  const int c = (int)(idx - row * nc);
  const T* zr = z + row * stride + c * 32;
  const int n = min(32, r - c * 32);
  T raw[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) raw[i] = zr[min(i, n - 1)];
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = i < n ? to_f32(raw[i]) : 0.f;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const float s32 = __fdiv_rn(amax, 7.0f);
  const _Float16 s16 = (_Float16)s32;
  const float sf = (float)s16;
  unsigned int words[4] = {0u, 0u, 0u, 0u};
  if (sf != 0.f) {
    const float inv = __fdiv_rn(1.0f, sf);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float t = v[i] * inv;
      float qf = rintf(t);
      if (fabsf(t) < 8.f && fabsf(fabsf(t - qf) - 0.5f) < 4e-6f) qf = rintf(__fdiv_rn(v[i], sf));
      qf = fminf(fmaxf(qf, -7.f), 7.f);
      const int q = i < n ? (int)qf : 0;
      words[i >> 3] |= (unsigned int)(q & 0xF) << (4 * (i & 7));
    }
  }
  uint4 packed = make_uint4(words[0], words[1], words[2], words[3]);
  *(uint4*)(codes + row * (int64_t)(16 * nc) + 16 * c) = packed;
  scales[row * nc + c] = s16;
}

template <class T>
static hipError_t launch_q(const void* z, int64_t n_rows, int r, int64_t stride, void* codes, void* scales,
                           hipStream_t stream) {
  const int nc = cdiv(r, 32);
  const int64_t work = n_rows * nc;
  if (work == 0) return hipSuccess;
  const int64_t blocks = cdiv64(work, 256);
  hipLaunchKernelGGL(palu_quant_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, stream, (const T*)z, n_rows, r,
                     stride, (uint8_t*)codes, (_Float16*)scales);
  return hipGetLastError();
}

// The chunks (32 elements) of one (sequence, group) block are numbered
// c = t * nch + chunk; codes, scales and output rows are then plain arrays
// of chunks (16, 2 and 64 bytes each), and rows t < L are exactly the chunks
// c < L * nch.  A wave expands 64 consecutive chunks: in round k its lane l
// takes the 8-element piece (quarter l % 4 of chunk 16 k + l / 4), so that
// every load and store instruction of the wave covers contiguous memory
// (256 bytes of codes in, 1 KB out); the four rounds' loads are issued
// before any is used.  The decode consumes the int4 latent
// z_hat = code * scale (PALU page, section "Rollout", route C: quantization
// on top of the low-rank cache); the product is exact in fp32 and is
// rounded once to the 16-bit format, or (split mode, what the decode
// attends over on shapes that do not read the codes directly) kept exactly
// as a hi + lo pair of 16-bit values.
template <class T>
__global__ void __launch_bounds__(256) palu_dequant_kernel(const DequantParams p) {
  const int b = blockIdx.y / p.G, j = blockIdx.y - b * p.G;
  const DequantSide& d = p.side[blockIdx.z];
  const unsigned nch = (unsigned)d.nch[j];
  int L = p.seq_lens ? p.seq_lens[b] : p.max_len;
  L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
  const unsigned n_chunks = (unsigned)L * nch;
  const int l = threadIdx.x & 63;
  const unsigned c0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 64 + (l >> 2);   // chunk of round 0
  if (c0 >= n_chunks) return;
  const uint8_t* codes = d.codes + b * d.seq_c + d.goff_c[j] + 4 * (l & 3);
  const uint8_t* scales = d.scales + b * d.seq_s + d.goff_s[j];
  uint8_t* out = d.out + b * d.seq_o + d.goff_o[j];
  unsigned w[4];
  float s[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned c = c0 + 16 * k;
    if (c < n_chunks) {
      w[k] = *(const unsigned*)(codes + 16 * (int64_t)c);
      s[k] = (float)*(const _Float16*)(scales + 2 * (int64_t)c);
    }
  }
  const int tail = d.rank[j] & 31;   // elements in a row's last chunk (0: a whole chunk)
  auto mask_tail = [&](uint4& o, unsigned c) {
    if (tail != 0 && c - __umulhi(c, d.magic[j]) * nch == nch - 1) {
      // the row's last chunk: zero from the rank on (elements e0 .. e0+7 here)
      const int nv = tail - 8 * (l & 3);
      unsigned* h = (unsigned*)&o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        h[q] &= (2 * q < nv ? 0xFFFFu : 0u) | (2 * q + 1 < nv ? 0xFFFF0000u : 0u);
    }
  };
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned c = c0 + 16 * k;
    if (c < n_chunks) {
      if (p.split) {
        uint4 hi, lo;
        split8<T>(w[k], s[k], hi, lo);
        mask_tail(hi, c);
        mask_tail(lo, c);
        // (the out pointer already holds this lane's 16-byte piece offset)
        *(uint4*)(out + 128 * (int64_t)c + 16 * (l & 3)) = hi;
        *(uint4*)(out + 128 * (int64_t)c + 64 + 16 * (l & 3)) = lo;
      } else {
        uint4 o = expand8<T>(w[k], s[k]);
        mask_tail(o, c);
        *(uint4*)(out + 64 * (int64_t)c + 16 * (l & 3)) = o;
      }
    }
  }
}

// One thread per 8 columns of one row of B': rows 64 c + i and 64 c + 32 + i
// both copy row 32 c + i of B (zero past the rank).
template <class T>
__global__ void __launch_bounds__(256) palu_dup_factor_kernel(const DupParams p) {
  const int side = blockIdx.z, j = blockIdx.y;
  const int r = p.rank[side][j], rr = 64 * cdiv(r, 32);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = p.w / 8;                      // 8-column pieces per row
  if (idx >= (int64_t)rr * cpr) return;
  const int row = (int)(idx / cpr), col = (int)(idx - (int64_t)row * cpr) * 8;
  const int src_row = 32 * (row / 64) + (row & 31);
  uint4 v = uint4{0u, 0u, 0u, 0u};
  if (src_row < r) v = *(const uint4*)((const T*)p.src[side] + p.soff[side][j] + (int64_t)src_row * p.w + col);
  *(uint4*)((T*)p.dst[side] + p.doff[side][j] + (int64_t)row * p.w + col) = v;
}

hipError_t launch_dup_factor(const DupParams& p, hipStream_t stream) {
  if (p.G == 0) return hipSuccess;
  if (p.w % 8 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)cdiv64((int64_t)p.max_rows * (p.w / 8), 256), (unsigned)p.G, 2);
  hipLaunchKernelGGL(palu_dup_factor_kernel<uint16_t>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_dequant(int out_dtype, const DequantParams& p, hipStream_t stream) {
  if (p.batch == 0 || p.G == 0) return hipSuccess;
  const uint64_t chunks = (uint64_t)p.max_len * (uint64_t)p.max_nch;
  if (chunks * (uint64_t)p.max_nch >= (1ull << 32)) return hipErrorInvalidValue;
  // 256 chunks per block of 256 threads
  if (p.n_sides != 1 && p.n_sides != 2) return hipErrorInvalidValue;
  const dim3 grid((unsigned)cdiv64((int64_t)chunks, 256), (unsigned)(p.batch * p.G), (unsigned)p.n_sides);
  if (out_dtype == 1)
    hipLaunchKernelGGL(palu_dequant_kernel<_Float16>, grid, dim3(256), 0, stream, p);
  else if (out_dtype == 2)
    hipLaunchKernelGGL(palu_dequant_kernel<__bf16>, grid, dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quant(int dtype, const void* z, int64_t n_rows, int r, int64_t stride, void* codes,
                        void* scales, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_q<float>(z, n_rows, r, stride, codes, scales, stream);
    case 1: return launch_q<_Float16>(z, n_rows, r, stride, codes, scales, stream);
    case 2: return launch_q<__bf16>(z, n_rows, r, stride, codes, scales, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace palu
