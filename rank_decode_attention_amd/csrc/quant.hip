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

namespace palu {

template <class T>
__device__ __forceinline__ float load_f32(const T* p) { return to_f32(*p); }

// One thread per (row, 32-element chunk).  Stores 16 bytes of codes and one
// binary16 scale.
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
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = i < n ? load_f32(zr + i) : 0.f;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const float s32 = __fdiv_rn(amax, 7.0f);
  const _Float16 s16 = (_Float16)s32;
  const float sf = (float)s16;
  unsigned int words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int q = 0;
    if (sf != 0.f && i < n) {
      float qf = rintf(__fdiv_rn(v[i], sf));
      qf = fminf(fmaxf(qf, -7.f), 7.f);
      q = (int)qf;
    }
    words[i >> 3] |= (unsigned int)(q & 0xF) << (4 * (i & 7));
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

// One thread per (row, chunk slot): 16 bytes of codes and one scale in,
// 32 values out (four 16-byte stores).  The decode consumes the int4 latent
// ẑ = code * scale (PALU page, section "Rollout", route C: quantization on
// top of the low-rank cache); the product is exact in fp32 and is rounded
// once, to the activation format that the decode's MFMA takes.
template <class T>
__global__ void __launch_bounds__(256) palu_dequant_kernel(const DequantParams p) {
  const int b = blockIdx.y / p.G, j = blockIdx.y - b * p.G;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int t = (int)(idx >> p.cs_log2), ch = (int)(idx & ((1 << p.cs_log2) - 1));
  if (t >= p.max_len || ch >= p.nch[j]) return;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
  if (t >= L) return;
  const int nch = p.nch[j];
  const uint8_t* cr = p.codes + b * p.seq_c + p.goff_c[j] + (int64_t)t * (16 * nch) + 16 * ch;
  const uint8_t* sr = p.scales + b * p.seq_s + p.goff_s[j] + (int64_t)t * (2 * nch) + 2 * ch;
  uint8_t* orow = p.out + b * p.seq_o + p.goff_o[j] + (int64_t)t * (64 * nch) + 64 * ch;
  const uint4 c = *(const uint4*)cr;
  const float s = (float)*(const _Float16*)sr;
  const unsigned w[4] = {c.x, c.y, c.z, c.w};
  T v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int nib = (int)((w[i >> 3] >> (4 * (i & 7))) & 0xF);
    const int q = nib >= 8 ? nib - 16 : nib;   // 4-bit two's complement
    v[i] = from_f32<T>(32 * ch + i < p.rank[j] ? (float)q * s : 0.0f);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) ((uint4*)orow)[k] = *(const uint4*)&v[8 * k];
}

hipError_t launch_dequant(int out_dtype, const DequantParams& p, hipStream_t stream) {
  if (p.batch == 0 || p.G == 0) return hipSuccess;
  if (p.cs_log2 < 0 || p.cs_log2 > 5) return hipErrorInvalidValue;
  const dim3 grid((unsigned)cdiv64((int64_t)p.max_len << p.cs_log2, 256), (unsigned)(p.batch * p.G), 1);
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
