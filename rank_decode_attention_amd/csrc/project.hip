// Prefill latent projection z = x A on MFMA, writing the latent cache (gfx950).
//
// PALU page, section "Inference flow", prefill steps 3-4: instead of K/V the
// attention layer computes the low-rank latents z_k = x A_k, z_v = x A_v and
// caches them.  Optional int4 output quantises each 32-element chunk of a
// token's latent row (quantization composing with low rank: arXiv
// 2407.21118v2 abstract).
//
// Layout: x [n_tok][D] row-major; A is passed as its transpose A^T
// [n_lat][D] (the weight layout of a Linear(D -> n_lat)), so both MFMA
// operands are 16-byte contiguous runs of D.  Block = 256 tokens x up to 160
// latent channels of one latent row (group j of keys or values); 8 waves of
// 32 tokens x 160 channels (two per SIMD); K-steps of 128 bytes staged by LDS
// DMA, double-buffered.
#include "common.h"
#include "project.h"

#include <type_traits>

namespace palu {

template <class T_>
struct PrjCfg {
  typedef T_ T;
  static constexpr bool F32 = std::is_same<T, float>::value;
  static constexpr int ESZ = sizeof(T);
  static constexpr int BM = 256, BN = 160, BK = F32 ? 32 : 64, NW = 8, NT = 512;
  static constexpr int MT = BM / (16 * NW), NTL = 10;    // m-tiles / n-tiles per wave
  static constexpr int CPR = BK * ESZ / 16;              // 16-byte chunks per staged row
  static constexpr int PIT = CPR + 1;                    // padded LDS row pitch (slots)
  static constexpr int SX = cdiv(BM * PIT, 64 * NW) * 64 * NW;   // x slots (whole instructions)
  static constexpr int SA = cdiv(BN * PIT, 64 * NW) * 64 * NW;
  static constexpr int NIX = SX / (64 * NW), NIA = SA / (64 * NW);
  static constexpr int NDMA = NIX + NIA;
  static constexpr int BUF = (SX + SA);                  // slots per stage
  static constexpr int KCH = 2;                          // operand chunks (4 x 16 bytes) per K-step per row
};

template <class C, class OT>
__device__ __forceinline__ void store_elem(uint8_t* base, OT v) { *(OT*)base = v; }

template <class C>
__global__ void __launch_bounds__(C::NT, 1) palu_project_kernel(const ProjectParams p) {
  typedef typename C::T T;
  typedef typename std::conditional<C::F32, f32x4, typename Vec8<typename std::conditional<C::F32, _Float16, T>::type>::type>::type op_t;
  __shared__ uint4 st0[C::BUF];
  __shared__ uint4 st1[C::BUF];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int64_t m0 = (int64_t)blockIdx.x * C::BM;
  const int j = blockIdx.y;                       // latent row: keys of groups 0..G-1, then values
  const int r = p.rank[j];
  const int n0 = blockIdx.z * C::BN;
  if (n0 >= r) return;
  const int64_t col0 = p.col_off[j] + n0;         // first row of A^T for this block
  const int nvalid = min(C::BN, r - n0);
  const T* X = (const T*)p.x;
  const T* A = (const T*)p.A;
  const int64_t D = p.d_model;

  // per-lane DMA geometry (slot -> row, chunk)
  int gx[C::NIX], ga[C::NIA];
#pragma unroll
  for (int m = 0; m < C::NIX; ++m) {
    const int slot = (m * C::NW + w) * 64 + l;
    int row = slot / C::PIT, pos = slot - row * C::PIT;
    row = row < C::BM ? row : C::BM - 1;
    pos = pos < C::CPR ? pos : 0;
    int64_t tok = m0 + row;
    tok = tok < p.n_tok ? tok : p.n_tok - 1;
    gx[m] = (int)((tok - m0) << 8) | pos;
  }
#pragma unroll
  for (int m = 0; m < C::NIA; ++m) {
    const int slot = (m * C::NW + w) * 64 + l;
    int row = slot / C::PIT, pos = slot - row * C::PIT;
    row = row < nvalid ? row : nvalid - 1;
    pos = pos < C::CPR ? pos : 0;
    ga[m] = (row << 8) | pos;
  }
  auto issue = [&](uint4* buf, int64_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < C::NIX; ++m) {
      const T* src = X + (m0 + (gx[m] >> 8)) * D + k0 + (gx[m] & 0xFF) * (16 / C::ESZ);
      dma16(src, lds_addr(buf) + 16u * ((m * C::NW + w) * 64));
    }
#pragma unroll
    for (int m = 0; m < C::NIA; ++m) {
      const T* src = A + (col0 + (ga[m] >> 8)) * D + k0 + (ga[m] & 0xFF) * (16 / C::ESZ);
      dma16(src, lds_addr(buf) + 16u * (C::SX + (m * C::NW + w) * 64));
    }
  };

  f32x4 acc[C::MT][C::NTL];
#pragma unroll
  for (int a = 0; a < C::MT; ++a)
#pragma unroll
    for (int b = 0; b < C::NTL; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ntl = cdiv(nvalid, 16);

  auto compute = [&](const uint4* buf) __attribute__((always_inline)) {
    const int kq = l >> 4, rr = l & 15;
#pragma unroll
    for (int kc = 0; kc < C::KCH; ++kc) {
      op_t xa[C::MT];
#pragma unroll
      for (int a = 0; a < C::MT; ++a) {
        const int row = C::MT * 16 * w + 16 * a + rr;
        // 16-bit: chunk 4*kc + kq holds k = 32 kc + 8 kq .. +7; fp32: 4 floats
        xa[a] = *(const op_t*)(buf + row * C::PIT + 4 * kc + kq);
      }
      // Every n-tile runs (branch-free, so the operand reads go out ahead of
      // the MFMAs; a runtime bound here puts each read and its MFMAs in a
      // basic block of its own): rows of A^T past the valid channels are
      // copies of the last valid row in LDS, and their columns are not stored.
#pragma unroll
      for (int b = 0; b < C::NTL; ++b) {
        const op_t bv = *(const op_t*)(buf + C::SX + (16 * b + rr) * C::PIT + 4 * kc + kq);
#pragma unroll
        for (int a = 0; a < C::MT; ++a) {
          if constexpr (C::F32) {
            f32x4 c = acc[a][b];
            c = mfma16x16x4(xa[a][0], bv[0], c);
            c = mfma16x16x4(xa[a][1], bv[1], c);
            c = mfma16x16x4(xa[a][2], bv[2], c);
            c = mfma16x16x4(xa[a][3], bv[3], c);
            acc[a][b] = c;
          } else {
            acc[a][b] = mfma16x16x32(xa[a], bv, acc[a][b]);
          }
        }
      }
    }
  };

  const int nk = (int)(D / C::BK);
  issue(st0, 0);
  for (int ks = 0; ks < nk; ks += 2) {
    // stage ks in st0, ks + 1 in st1
    if (ks + 1 < nk) {
      issue(st1, (int64_t)(ks + 1) * C::BK);
      wait_vmcnt<C::NDMA>();
    } else {
      wait_vmcnt<0>();
    }
    barrier();
    compute(st0);
    wait_lgkm0();
    barrier();
    if (ks + 1 < nk) {
      if (ks + 2 < nk) {
        issue(st0, (int64_t)(ks + 2) * C::BK);
        wait_vmcnt<C::NDMA>();
      } else {
        wait_vmcnt<0>();
      }
      barrier();
      compute(st1);
      wait_lgkm0();
      barrier();
    }
  }

  // ---- epilogue
  const int kq = l >> 4, rr = l & 15;
  const int gj = j % p.G, is_v = j >= p.G;
  const int pitch = is_v ? p.pv[gj] : p.pk[gj];
  // block of latent row t of the written sequence (paged: the page holding
  // t, with t counted inside it)
  auto blk_of = [&](int64_t t, int64_t& tin) __attribute__((always_inline)) {
    if (p.block_table) {
      tin = t & ((1 << p.page_shift) - 1);
      return (int64_t)p.block_table[(int64_t)p.seq * p.max_pages + (t >> p.page_shift)];
    }
    tin = t;
    return (int64_t)p.seq;
  };
  auto zrow = [&](int64_t t) __attribute__((always_inline)) {
    int64_t tin;
    const int64_t blk = blk_of(t, tin);
    return (is_v ? p.zv : p.zk) + blk * (is_v ? p.seq_bytes_v : p.seq_bytes_k) + (is_v ? p.goff_v[gj] : p.goff_k[gj]) +
           tin * pitch;
  };
  if (p.quant == 0) {
#pragma unroll
    for (int a = 0; a < C::MT; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t tok = m0 + C::MT * 16 * w + 16 * a + 4 * kq + e;
        if (tok < p.n_tok) {
          uint8_t* rowp = zrow(p.pos0 + tok);
#pragma unroll
          for (int b = 0; b < C::NTL; ++b) {
            const int n = n0 + 16 * b + rr;
            if (b < ntl && n < r) store_elem<C, T>(rowp + n * C::ESZ, from_f32<T>(acc[a][b][e]));
          }
          // zero the row padding (pitch beyond the rank) once, from the last block
          if (n0 + C::BN >= r) {
            const int padn = pitch / C::ESZ;
            for (int n = r + rr; n < padn; n += 16) store_elem<C, T>(rowp + n * C::ESZ, from_f32<T>(0.f));
          }
        }
      }
  } else {
    // Quantise per (token, 32-element chunk) exactly as palu_quant_latent.
    // Each wave stages one 16-token m-tile at a time in its own LDS region,
    // transposed ([column][token], 16-byte vector writes of the lane's four
    // consecutive tokens), then its lanes take one (token, chunk) each.
    // The region reuses a stage buffer: every wave has passed the main
    // loop's final barrier, so no stage data is read any more.
    constexpr int TP = 20;                                  // floats per staged column (16 tokens + pad)
    static_assert((C::NW / 2) * C::BN * TP * 4 <= C::BUF * 16, "staging");
    float* zs = (float*)(w < C::NW / 2 ? st0 : st1) + (w % (C::NW / 2)) * (C::BN * TP);
    const int nc_row = cdiv(r, 32);
    auto srow = [&](int64_t t) __attribute__((always_inline)) {
      int64_t tin;
      const int64_t blk = blk_of(t, tin);
      return (is_v ? p.sv : p.sk) + blk * (is_v ? p.seq_sbytes_v : p.seq_sbytes_k) +
             (is_v ? p.soff_v[gj] : p.soff_k[gj]) + tin * 2 * nc_row;
    };
    const int nchunk = cdiv(nvalid, 32);
#pragma unroll
    for (int a = 0; a < C::MT; ++a) {
#pragma unroll
      for (int b = 0; b < C::NTL; ++b) *(f32x4*)(zs + (16 * b + rr) * TP + 4 * kq) = acc[a][b];
      wait_lgkm0();
      for (int it = l; it < 16 * nchunk; it += 64) {
        const int trow = it & 15, c = it >> 4;
        const int64_t tok = m0 + C::MT * 16 * w + 16 * a + trow;
        const int cg = n0 / 32 + c;                // chunk index within the latent row
        const int n = min(32, r - cg * 32);
        if (tok < p.n_tok) {
          const float* v = zs + (32 * c) * TP + trow;
          float amax = 0.f;
          for (int i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(v[i * TP]));
          const float s32 = __fdiv_rn(amax, 7.0f);
          const _Float16 s16 = (_Float16)s32;
          const float sf = (float)s16;
          unsigned int words[4] = {0u, 0u, 0u, 0u};
          for (int i = 0; i < n; ++i) {
            int q = 0;
            if (sf != 0.f) {
              float qf = rintf(__fdiv_rn(v[i * TP], sf));
              qf = fminf(fmaxf(qf, -7.f), 7.f);
              q = (int)qf;
            }
            words[i >> 3] |= (unsigned int)(q & 0xF) << (4 * (i & 7));
          }
          *(uint4*)(zrow(p.pos0 + tok) + 16 * cg) = make_uint4(words[0], words[1], words[2], words[3]);
          ((_Float16*)srow(p.pos0 + tok))[cg] = s16;
        }
      }
      wait_lgkm0();   // this m-tile's reads are done before the next one is staged
    }
  }
}

template <class C>
static hipError_t launch_c(const ProjectParams& p, int max_rank, hipStream_t stream) {
  dim3 grid((unsigned)cdiv64(p.n_tok, C::BM), (unsigned)(2 * p.G), (unsigned)cdiv(max_rank, C::BN));
  hipLaunchKernelGGL(palu_project_kernel<C>, grid, dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_project(int dtype, const ProjectParams& p, int max_rank, hipStream_t stream) {
  if (p.n_tok == 0) return hipSuccess;
  switch (dtype) {
    case 0: return launch_c<PrjCfg<float>>(p, max_rank, stream);
    case 1: return launch_c<PrjCfg<_Float16>>(p, max_rank, stream);
    case 2: return launch_c<PrjCfg<__bf16>>(p, max_rank, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace palu
