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

// Four lanes per (row, 32-element chunk), lane i of the quad owning
// elements 8i .. 8i + 7, so that each of a wave's load rounds covers sixteen
// chunks of contiguous row memory.  The chunk's amax is reduced
// over the quad with DPP; every lane forms the same scale, quantises its 8
// elements and stores their 4 bytes of codes (a chunk's 16 bytes are the
// quad's 4 stores); lane 0 stores the scale.
// code = rint(fl(z / s)) needs the correctly rounded binary32 quotient only
// where it decides the rounding: with 1/s known within one ulp, t = z * (1/s)
// lies within 1.9e-6 of fl(z / s) for |t| < 8 (relative errors 2^-23 for the
// reciprocal, 2^-24 for the product and 2^-24 for fl(z / s) itself), so
// rint(t) is the code unless t is within 4e-6 of a half-integer, where the
// exact quotient is formed (also beyond |t| >= 8, where both clamp to +-7).
// A lane's 8 elements are read as the whole 16-byte blocks that hold them
// (two for 16-bit elements, three for binary32) and realigned in registers;
// blocks are addressed by 32-bit byte offsets from a 16-byte-aligned,
// wave-uniform row base, each clamped to the block of the piece's last byte
// (a lane without elements reads the base block), so every load reads a
// block holding bytes of the input and none leaves its pages; loads and
// realignment are separate steps so that a wave issues several pieces'
// loads before it uses any.
template <class T>
struct Piece {
  static constexpr int NS = 8 * (int)sizeof(T) / 16 + 1;   // 16-byte blocks a piece can touch
  uint4 seg[NS];
  unsigned sh;                                           // the piece's byte offset in its first block
};

// zb: 16-byte aligned and wave-uniform; off: the piece's byte offset from
// zb; n: its elements (0..8)
template <class T>
__device__ __forceinline__ void piece_load(Piece<T>& pc, const char* zb, unsigned off, int n) {
  pc.sh = off & 15u;
  const unsigned first = n > 0 ? off & ~15u : 0u;
  const unsigned last = n > 0 ? (off + (unsigned)n * (unsigned)sizeof(T) - 1u) & ~15u : 0u;
#pragma unroll
  for (int i = 0; i < Piece<T>::NS; ++i) pc.seg[i] = *(const uint4*)(zb + min(first + 16u * i, last));
}

template <class T>
__device__ __forceinline__ void piece_values(const Piece<T>& pc, int n, float (&v)[8]) {
  constexpr int ND = 2 * (int)sizeof(T);                 // dwords of 8 elements
  unsigned d[4 * Piece<T>::NS];
#pragma unroll
  for (int i = 0; i < Piece<T>::NS; ++i) {
    d[4 * i] = pc.seg[i].x;
    d[4 * i + 1] = pc.seg[i].y;
    d[4 * i + 2] = pc.seg[i].z;
    d[4 * i + 3] = pc.seg[i].w;
  }
  const unsigned b = pc.sh & 3;
  // dword offset sh / 4 in two bitwise selects (by 2, then by 1; written
  // as masks so that the compiler keeps the words in registers instead of
  // indexing an array)
  const unsigned m2 = 0u - ((pc.sh >> 3) & 1u), m1 = 0u - ((pc.sh >> 2) & 1u);
  unsigned f2[ND + 2], e[ND + 1];
#pragma unroll
  for (int j = 0; j < ND + 2; ++j) f2[j] = (d[j + 2] & m2) | (d[j] & ~m2);
#pragma unroll
  for (int j = 0; j <= ND; ++j) e[j] = (f2[j + 1] & m1) | (f2[j] & ~m1);
  unsigned o[ND];
#pragma unroll
  for (int k = 0; k < ND; ++k) o[k] = __builtin_amdgcn_alignbyte(e[k + 1], e[k], b);
  const T* el = (const T*)o;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = i < n ? to_f32(el[i]) : 0.f;
}

// fl(a / 7) for finite a >= 0 without a divide: q0 = fl(a * fl(1/7)) is
// corrected once by its exact residual a - 7 q0 (an fma, exact in binary32).
// Checked against the correctly rounded quotient for every non-negative
// finite binary32 a (tests/test_quant_host.py: on a sample of every
// binade, and on all 2^31 - 2^23 values with PALU_EXHAUSTIVE=1).
__device__ __forceinline__ float div7_rn(float a) {
  const float c = 1.0f / 7.0f;   // fl(1/7), folded at compile time
  const float q0 = a * c;
  return __builtin_fmaf(__builtin_fmaf(-q0, 7.0f, a), c, q0);
}

// t within 4e-6 of a half-integer (|t - rint(t)| <= 1/2 always; beyond
// |t| >= 8 the exact quotient clamps to the same code as t)
__device__ __forceinline__ bool near_half(float t, float rt) { return fabsf(t - rt) > 0.5f - 4e-6f; }

// Rotated chunks (the low-rank-aware variant): before the amax, every full
// 32-element chunk is replaced by z H (H the Sylvester Hadamard matrix of
// order 32, entries +-1), formed by the fast Walsh-Hadamard butterflies in
// binary32 - stages h = 1, 2, 4 inside a lane's 8 elements, h = 8 and 16
// between the quad's lanes (DPP) - the pair (i, i + h) becoming
// (a + b, a - b).  A trailing partial chunk is quantised as it is.
__device__ __forceinline__ void fwht32(float (&v)[8], int qi) {
#pragma unroll
  for (int h = 1; h < 8; h *= 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  // h = 8: lanes qi and qi ^ 1; h = 16: lanes qi and qi ^ 2 (the lower lane
  // holds a, the upper lane b)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = dpp<0xB1>(v[i]);
    v[i] = (qi & 1) ? p - v[i] : v[i] + p;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = dpp<0x4E>(v[i]);
    v[i] = (qi & 2) ? p - v[i] : v[i] + p;
  }
}

// One quad's chunk: its 8 elements v (zero past the row's rank),
// rotated first for ROT where the chunk is full; the quad's amax, the
// chunk's scale, this lane's 4 bytes of codes and (lane 0) the scale.  All
// four lanes of the quad run it together (the amax crosses the quad by DPP).
template <bool ROT>
__device__ __forceinline__ void quant_quad(float (&v)[8], int qi, int c, int r, bool live, uint8_t* crow,
                                           _Float16* srow) {
  if constexpr (ROT) {
    // (every lane of the quad runs the butterflies; chunks that are not full
    // keep their values)
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = v[i];
    fwht32(w, qi);
    if (32 * c + 32 <= r) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = w[i];
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, dpp<0xB1>(amax));
  amax = fmaxf(amax, dpp<0x4E>(amax));
  float s32 = div7_rn(amax);
  // (held as binary32: the compiler would otherwise fuse the last fma with
  // the conversion below into one fma rounding straight to fp16)
  asm volatile("" : "+v"(s32));
  const _Float16 s16 = (_Float16)s32;
  const float sf = (float)s16;
  unsigned word = 0u;   // element 8 qi + i in nibble i
  if (sf != 0.f) {
    // 1/s within one ulp: the hardware reciprocal and one Newton step
    const float r0 = __builtin_amdgcn_rcpf(sf);
    const float inv = __builtin_fmaf(r0, __builtin_fmaf(-sf, r0, 1.0f), r0);
    float qf[8];
    float dmax = 0.f;   // the largest |t - rint(t)| of the lane's elements
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = v[i] * inv;
      qf[i] = rintf(t);
      dmax = fmaxf(dmax, fabsf(t - qf[i]));
    }
    if (dmax > 0.5f - 4e-6f) {   // (rare) the exact quotient where it decides the rounding
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = v[i] * inv;
        if (near_half(t, rintf(t))) qf[i] = rintf(__fdiv_rn(v[i], sf));
      }
    }
    // nibble i = q_i & 15: 0x88888888 + sum q_i 16^i holds q_i + 8 (1 .. 15,
    // no carries) in nibble i, and q + 8 = (q & 15) ^ 8 for -8 <= q <= 7
    // The clamp to +-7 only acts when the scale is an fp16 subnormal: a
    // normal fp16 scale is within 2^-11 of amax / 7, so |t| < 7.01 and
    // rint(t) lies in -7 .. 7 already (an infinite scale gives t = 0).
    if (sf < 0x1p-14f) {   // (rare)
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[i] = __builtin_amdgcn_fmed3f(qf[i], -7.f, 7.f);
    }
    word = 0x88888888u;
#pragma unroll
    for (int i = 0; i < 8; ++i) word += (unsigned)(int)qf[i] << (4 * i);   // (elements past the row: code 0)
    word ^= 0x88888888u;
  }
  if (live) {
    *(unsigned*)(crow + 16 * c + 4 * qi) = word;
    if (qi == 0) srow[c] = s16;
  }
}

// A wave quantises 32 consecutive chunks (of the flattened (row, chunk)
// list) in kQRounds rounds of 16: in round k, lane l takes quarter l % 4 of
// chunk 16 k + l / 4.  Both rounds' loads are issued before any chunk is
// quantised (measured: two rounds per wave, twice the waves, about 3%
// faster than four rounds, which leave the last wave of blocks of each CU
// partly idle).
constexpr int kQRounds = 2;

template <class T, bool ROT>
__global__ void __launch_bounds__(256) palu_quant_kernel(const T* __restrict__ z, int64_t n_rows, int r,
                                                         int64_t stride, uint8_t* __restrict__ codes,
                                                         _Float16* __restrict__ scales, unsigned nc_magic) {
  const int nc = cdiv(r, 32);
  const int qi = threadIdx.x & 3;
  const int64_t work = n_rows * nc;
  // the wave's first chunk and its (row, chunk) (wave-uniform); a lane's
  // chunk in round k lies rel = c0 + 16 k + l / 4 chunks past the start of
  // row row0, i.e. in row row0 + rel / nc (rel / nc by a multiply with
  // ceil(2^32 / nc), exact for rel < 2^32 / nc; nc = 1 needs none)
  const int64_t w0 = ((int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * (16 * kQRounds);
  // (the last block's waves past the work end here: their row base would lie
  // past the input, and lanes without elements read the base block)
  if (w0 >= work) return;
  const int64_t row0 = w0 / nc;
  const int c0 = (int)(w0 - row0 * nc);
  const T* zrow0 = z + row0 * stride;
  // the wave's 16-byte-aligned base and each lane's 32-bit offsets from it
  // (the host bounds the row stride so that 34 rows fit in 32 bits)
  const unsigned zoff = (unsigned)((uintptr_t)zrow0 & 15);
  const char* zb = (const char*)zrow0 - zoff;   // (pointer arithmetic keeps the global address space)
  const unsigned stride_b = (unsigned)stride * (unsigned)sizeof(T);
  uint8_t* crow0 = codes + row0 * (int64_t)(16 * nc);
  _Float16* srow0 = scales + row0 * nc;
  Piece<T> pc[kQRounds];
  unsigned rrel[kQRounds];
  int c[kQRounds], n[kQRounds];
  bool live[kQRounds];
#pragma unroll
  for (int k = 0; k < kQRounds; ++k) {
    const unsigned rel = (unsigned)c0 + 16u * k + ((threadIdx.x & 63) >> 2);
    rrel[k] = nc == 1 ? rel : __umulhi(rel, nc_magic);
    c[k] = (int)(rel - rrel[k] * (unsigned)nc);
    live[k] = w0 + (int64_t)(16 * k) + ((threadIdx.x & 63) >> 2) < work;
    const int e0 = 32 * c[k] + 8 * qi;            // this lane's first element in the row
    int m = live[k] ? r - e0 : 0;
    n[k] = m < 0 ? 0 : (m > 8 ? 8 : m);
    piece_load<T>(pc[k], zb, zoff + rrel[k] * stride_b + (unsigned)e0 * (unsigned)sizeof(T), n[k]);
  }
  // (the whole wave takes part; quads past the end carry zeros)
#pragma unroll
  for (int k = 0; k < kQRounds; ++k) {
    float v[8];
    piece_values<T>(pc[k], n[k], v);
    quant_quad<ROT>(v, qi, c[k], r, live[k], crow0 + rrel[k] * (16u * nc), srow0 + rrel[k] * (unsigned)nc);
  }
}

template <class T, bool ROT>
static hipError_t launch_q(const void* z, int64_t n_rows, int r, int64_t stride, void* codes, void* scales,
                           hipStream_t stream) {
  const int nc = cdiv(r, 32);
  const int64_t work = n_rows * nc;     // chunks, 4 lanes each, 16 kQRounds per wave
  if (work == 0) return hipSuccess;
  const unsigned magic = (unsigned)((0xFFFFFFFFull / (unsigned)nc) + 1);   // ceil(2^32 / nc) for nc > 1
  const int64_t blocks = cdiv64(work, 4 * 16 * kQRounds);
  hipLaunchKernelGGL((palu_quant_kernel<T, ROT>), dim3((unsigned)blocks), dim3(256), 0, stream, (const T*)z, n_rows,
                     r, stride, (uint8_t*)codes, (_Float16*)scales, nc == 1 ? 0u : magic);
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

template <bool ROT>
static hipError_t launch_quant_r(int dtype, const void* z, int64_t n_rows, int r, int64_t stride, void* codes,
                                 void* scales, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_q<float, ROT>(z, n_rows, r, stride, codes, scales, stream);
    case 1: return launch_q<_Float16, ROT>(z, n_rows, r, stride, codes, scales, stream);
    case 2: return launch_q<__bf16, ROT>(z, n_rows, r, stride, codes, scales, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quant(int dtype, const void* z, int64_t n_rows, int r, int64_t stride, void* codes,
                        void* scales, hipStream_t stream, bool rotate) {
  return rotate ? launch_quant_r<true>(dtype, z, n_rows, r, stride, codes, scales, stream)
                : launch_quant_r<false>(dtype, z, n_rows, r, stride, codes, scales, stream);
}

}  // namespace palu
