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
