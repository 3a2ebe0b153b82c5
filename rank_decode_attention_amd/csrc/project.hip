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
// operands are 16-byte contiguous runs of D.  The latent channels are cut
// into column tiles of at most 160 channels of one latent row (group j of
// keys or values); a block computes 256 tokens x two consecutive column
// tiles, 8 waves of 64 tokens x one tile (two per SIMD), with K-steps of 64
// bytes per row staged by LDS DMA in a ring of 4 stages (3 requested ahead).
#include "common.h"
#include "project.h"

#include <hip/hip_ext.h>
#include <type_traits>

namespace palu {

template <class T_>
struct PrjCfg {
  typedef T_ T;
  static constexpr bool F32 = std::is_same<T, float>::value;
  static constexpr int ESZ = sizeof(T);
  static constexpr int BM = 256, TN = kColTile, NTB = 2, NW = 8, NT = 512;   // tokens, channels of a column tile, tiles per block
  static constexpr int WM = 4;                           // wave w: tokens 64 (w % 4) .., column tile w / 4
  static constexpr int MT = BM / (16 * WM);              // m-tiles per wave (4)
  static constexpr int NTL = TN / 16;                    // n-tiles per wave (10)
  static constexpr int ROWB = 64;                        // bytes of a row per K-step: four 16-byte chunks
  static constexpr int BK = ROWB / ESZ;                  // K per step (32 for 16-bit, 16 for fp32)
  static constexpr int SXS = BM * 4, SAS = NTB * TN * 4; // 16-byte slots of the x and A^T tiles of a stage
  static constexpr int NIX = SXS / (64 * NW);            // DMA instructions per wave (x)
  static constexpr int NIA = cdiv(SAS, 64 * NW);         // (A^T; the last one only for waves inside the tile)
  static constexpr int STG = SXS + SAS;                  // slots per stage (36 KB)
  static constexpr int NS = 4;                           // stages: 3 requested ahead of the one computed
  static constexpr int TP = 20;                          // int4 epilogue: floats per staged column (16 tokens + pad)
  static_assert(SXS % (64 * NW) == 0 && SAS % 64 == 0, "DMA slots");
  static_assert(NW * TN * TP <= NS * STG * 4, "epilogue staging");
};

template <class C, class OT>
__device__ __forceinline__ void store_elem(uint8_t* base, OT v) { *(OT*)base = v; }

template <class C>
__global__ void __launch_bounds__(C::NT, 1) palu_project_kernel(const ProjectParams p) {
  typedef typename C::T T;
  typedef typename std::conditional<C::F32, f32x4, typename Vec8<typename std::conditional<C::F32, _Float16, T>::type>::type>::type op_t;
  __shared__ uint4 stg[C::NS * C::STG];

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // (wave-uniform: scalar registers)
  const int wm = w % C::WM, wt = w / C::WM;
  const int64_t m0 = (int64_t)blockIdx.x * C::BM;
  // the block's two column tiles (an odd tile count leaves the last block
  // one tile: its second tile repeats the first and is not stored)
  const int tb = 2 * blockIdx.y;
  const int tile[2] = {tb, min(tb + 1, p.ntiles - 1)};
  int jt[2], n0t[2], nvt[2];
  int64_t colt[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    jt[t] = p.tile[tile[t]] >> 16;
    n0t[t] = p.tile[tile[t]] & 0xFFFF;
    nvt[t] = min(C::TN, p.rank[jt[t]] - n0t[t]);
    colt[t] = p.col_off[jt[t]] + n0t[t];          // first row of A^T of the tile
  }
  const bool store = wt == 0 || tb + 1 < p.ntiles;   // (wave-uniform)
  const T* X = (const T*)p.x;
  const T* A = (const T*)p.A;
  const int64_t D = p.d_model;

  // Stage layout: row-major tiles of 64-byte rows (x: BM token rows, then
  // A^T: TN channel rows of each column tile), the four 16-byte chunks of
  // row R stored at chunk position c ^ ((R >> 1) & 3): the LDS serves a
  // 16-byte-per-lane read 8 lanes (128 bytes) at a time, and the 8 rows of
  // such a group (same logical chunk) then cover 8 distinct 16-byte slots
  // of a 128-byte line (measured: no bank conflicts, where c ^ ((R >> 2) & 3)
  // had two-way ones).  DMA instruction m of wave w fills slots
  // (m * NW + w) * 64 + l of a region: row slot / 4, physical chunk
  // slot % 4.  Rows past the tokens or a tile's valid channels load the
  // last valid row (never stored).  Sources are a wave-uniform base plus a
  // per-lane 32-bit byte offset; the bases advance by one K-step per stage.
  constexpr int EPC = 16 / C::ESZ;                 // elements per 16-byte chunk
  unsigned xoff[C::NIX], aoff[C::NIA];
#pragma unroll
  for (int m = 0; m < C::NIX; ++m) {
    const int slot = (m * C::NW + w) * 64 + l;
    const int row = slot >> 2, lc = (slot & 3) ^ ((row >> 1) & 3);
    const int64_t tok = min(m0 + row, p.n_tok - 1);
    xoff[m] = (unsigned)(((tok - m0) * D + lc * EPC) * C::ESZ);
  }
#pragma unroll
  for (int m = 0; m < C::NIA; ++m) {
    const int slot = min((m * C::NW + w) * 64 + l, C::SAS - 1);
    const int row = slot >> 2, lc = (slot & 3) ^ ((row >> 1) & 3);
    const int t = row / C::TN, r = min(row - t * C::TN, nvt[t] - 1);
    aoff[m] = (unsigned)(((colt[t] + r) * D + lc * EPC) * C::ESZ);
  }
  const T* xblk = X + m0 * D;
  // (waves whose slots of an A^T instruction lie past the tiles skip it:
  // they issue one DMA instruction fewer per stage)
  const bool afull = (C::NIA - 1) * C::NW * 64 + w * 64 < C::SAS;
  // stage ks into buffer BUF (a compile-time constant)
  auto issue = [&](auto bufc, int ks) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    const unsigned base = lds_addr(stg) + 16u * (unsigned)(BUF * C::STG);
    const T* xb = xblk + (int64_t)ks * C::BK;
    const T* ab = A + (int64_t)ks * C::BK;
#pragma unroll
    for (int m = 0; m < C::NIX; ++m) dma16s(xb, xoff[m], base + 16u * ((m * C::NW + w) * 64));
#pragma unroll
    for (int m = 0; m < C::NIA; ++m)
      if (m < C::NIA - 1 || afull) dma16s(ab, aoff[m], base + 16u * (C::SXS + (m * C::NW + w) * 64));
  };
  // wait until at most `after` stages issued after the next one are in flight
  auto wait_stages = [&](int after) __attribute__((always_inline)) {
    constexpr int NF = C::NIX + C::NIA, NP = NF - 1;
    if (afull) {
      if (after >= 2) wait_vmcnt<2 * NF>(); else if (after == 1) wait_vmcnt<NF>(); else wait_vmcnt<0>();
    } else {
      if (after >= 2) wait_vmcnt<2 * NP>(); else if (after == 1) wait_vmcnt<NP>(); else wait_vmcnt<0>();
    }
  };

  f32x4 acc[C::MT][C::NTL];
#pragma unroll
  for (int a = 0; a < C::MT; ++a)
#pragma unroll
    for (int b = 0; b < C::NTL; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int kq = l >> 4, rr = l & 15;
  // operand read offset of this lane inside a 16-row tile: row rr, logical
  // chunk kq (16-bit: k = 8 kq .. +7 of the step; fp32: k = 4 kq .. +3)
  const int lo = rr * C::ROWB + 16 * (kq ^ ((rr >> 1) & 3));

  // Every n-tile runs (branch-free, so the operand reads go out ahead of the
  // MFMAs): rows of A^T past the valid channels are copies of the last valid
  // row in LDS, and their columns are not stored.
  auto step_mma = [&](auto bufc) __attribute__((always_inline)) {
    const uint8_t* sb = (const uint8_t*)stg + decltype(bufc)::value * C::STG * 16;
    op_t xa[C::MT], bv[C::NTL];
#pragma unroll
    for (int a = 0; a < C::MT; ++a) xa[a] = *(const op_t*)(sb + (64 * wm + 16 * a) * C::ROWB + lo);
#pragma unroll
    for (int b = 0; b < C::NTL; ++b) bv[b] = *(const op_t*)(sb + 16 * C::SXS + (C::TN * wt + 16 * b) * C::ROWB + lo);
#pragma unroll
    for (int b = 0; b < C::NTL; ++b)
#pragma unroll
      for (int a = 0; a < C::MT; ++a) {
        if constexpr (C::F32) {
          f32x4 c = acc[a][b];
          c = mfma16x16x4(xa[a][0], bv[b][0], c);
          c = mfma16x16x4(xa[a][1], bv[b][1], c);
          c = mfma16x16x4(xa[a][2], bv[b][2], c);
          c = mfma16x16x4(xa[a][3], bv[b][3], c);
          acc[a][b] = c;
        } else {
          acc[a][b] = mfma16x16x32(xa[a], bv[b], acc[a][b]);
        }
      }
  };
  auto sync = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    barrier();
    asm volatile("" ::: "memory");
  };

  // K loop: stage ks lives in buffer ks % NS, and NS - 1 stages are
  // requested ahead.  Step ks waits for stage ks, refills the buffer of
  // stage ks - 1 (every wave past the barrier has used its operands) and
  // runs stage ks's operand reads and MFMAs.  One barrier per step; the
  // loop is unrolled over the ring, so that every buffer index and LDS
  // address offset is a constant.
  const int nk = (int)(D / C::BK);
  static_assert(C::NS == 4, "buffer constants below");
  if (0 < nk) issue(std::integral_constant<int, 0>{}, 0);
  if (1 < nk) issue(std::integral_constant<int, 1>{}, 1);
  if (2 < nk) issue(std::integral_constant<int, 2>{}, 2);
  auto step = [&](auto bufc, int ks) __attribute__((always_inline)) {
    constexpr int B = decltype(bufc)::value;
    wait_stages(min(nk - 1, ks + C::NS - 2) - ks);
    sync();
    if (ks + C::NS - 1 < nk) issue(std::integral_constant<int, (B + C::NS - 1) % C::NS>{}, ks + C::NS - 1);
    step_mma(bufc);
  };
  for (int ks = 0; ks < nk; ks += C::NS) {
    step(std::integral_constant<int, 0>{}, ks);
    if (ks + 1 < nk) step(std::integral_constant<int, 1>{}, ks + 1);
    if (ks + 2 < nk) step(std::integral_constant<int, 2>{}, ks + 2);
    if (ks + 3 < nk) step(std::integral_constant<int, 3>{}, ks + 3);
  }

  // ---- epilogue: this wave's column tile
  const int j = jt[wt], n0 = n0t[wt], nvalid = nvt[wt], r = p.rank[j];
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
    if (!store) return;
#pragma unroll
    for (int a = 0; a < C::MT; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t tok = m0 + 64 * wm + 16 * a + 4 * kq + e;
        if (tok < p.n_tok) {
          uint8_t* rowp = zrow(p.pos0 + tok);
#pragma unroll
          for (int b = 0; b < C::NTL; ++b) {
            const int n = 16 * b + rr;
            if (n < nvalid) store_elem<C, T>(rowp + (n0 + n) * C::ESZ, from_f32<T>(acc[a][b][e]));
          }
          // zero the row padding (pitch beyond the rank) once, from the row's last tile
          if (n0 + C::TN >= r) {
            const int padn = pitch / C::ESZ;
            for (int n = r + rr; n < padn; n += 16) store_elem<C, T>(rowp + n * C::ESZ, from_f32<T>(0.f));
          }
        }
      }
  } else {
    // Quantise per (token, 32-element chunk) exactly as palu_quant_latent.
    // Each wave stages one 16-token m-tile at a time in its own LDS region,
    // transposed ([channel][token], 16-byte writes of a lane's four
    // consecutive tokens), then four lanes take each (token, chunk).
    wait_lgkm0();
    __syncthreads();   // every wave's operand reads of the stages are done
    if (!store) return;
    float* zs = (float*)stg + w * (C::TN * C::TP);
    const int nc_row = cdiv(r, 32);
    auto srow = [&](int64_t t) __attribute__((always_inline)) {
      int64_t tin;
      const int64_t blk = blk_of(t, tin);
      return (is_v ? p.sv : p.sk) + blk * (is_v ? p.seq_sbytes_v : p.seq_sbytes_k) +
             (is_v ? p.soff_v[gj] : p.soff_k[gj]) + tin * 2 * nc_row;
    };
    const int nchunk = cdiv(nvalid, 32);
    // lane l: token l / 4 of the m-tile, elements 8 (l % 4) .. + 7 of every
    // chunk (the quad's amax crosses its four lanes by DPP); one round per
    // 32-element chunk of the tile
    const int qi = l & 3, trow = l >> 2;
#pragma unroll
    for (int a = 0; a < C::MT; ++a) {
      wait_lgkm0();   // (the previous m-tile's reads are done before it is overwritten)
#pragma unroll
      for (int b = 0; b < C::NTL; ++b) *(f32x4*)(zs + (16 * b + rr) * C::TP + 4 * kq) = acc[a][b];
      wait_lgkm0();
      const int64_t tok = m0 + 64 * wm + 16 * a + trow;
      const bool live = tok < p.n_tok;        // (the same for the four lanes of a quad)
      uint8_t* crow = nullptr;
      _Float16* srw = nullptr;
      if (live) {
        crow = zrow(p.pos0 + tok);
        srw = (_Float16*)srow(p.pos0 + tok);
      }
#pragma unroll
      for (int c = 0; c < C::TN / 32; ++c) {
        if (c >= nchunk) break;                // (wave-uniform)
        const int cg = n0 / 32 + c;            // chunk index within the latent row
        const int nv = min(32, r - cg * 32) - 8 * qi;   // valid elements of this lane
        const float* vs = zs + (32 * c + 8 * qi) * C::TP + trow;
        float v[8];
        if (cg * 32 + 32 <= r) {               // (wave-uniform) a whole chunk: no masking
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = vs[i * C::TP];
        } else {                               // the row's last, partial chunk: zero past the rank
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = i < nv ? vs[i * C::TP] : 0.f;
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = fmaxf(amax, dpp<0xB1>(amax));
        amax = fmaxf(amax, dpp<0x4E>(amax));
        // s = fl(amax / 7): the product by fl(1/7) corrected once by its exact
        // residual (equal to the correctly rounded quotient for every
        // non-negative binary32), held as binary32 before the fp16 rounding
        const float q0 = amax * (1.0f / 7.0f);
        float s32 = __builtin_fmaf(__builtin_fmaf(-q0, 7.0f, amax), 1.0f / 7.0f, q0);
        asm volatile("" : "+v"(s32));
        const _Float16 s16 = (_Float16)s32;
        const float sf = (float)s16;
        unsigned word = 0u;   // element 8 qi + i in nibble i
        if (sf != 0.f) {
          // code = rint(fl(z / s)): with 1/s within one ulp, t = z * (1/s) is
          // within 1.9e-6 of fl(z / s) for |t| < 8, so rint(t) is the code
          // unless t lies within 4e-6 of a half-integer, where the correctly
          // rounded quotient is formed (for |t| >= 8 both clamp to +-7)
          const float r0 = __builtin_amdgcn_rcpf(sf);
          const float inv = __builtin_fmaf(r0, __builtin_fmaf(-sf, r0, 1.0f), r0);
          float qf[8];
          bool near = false;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float t = v[i] * inv;
            qf[i] = rintf(t);
            near |= fabsf(t - qf[i]) > 0.5f - 4e-6f;
          }
          if (near) {   // (rare)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float t = v[i] * inv;
              if (fabsf(t - rintf(t)) > 0.5f - 4e-6f) qf[i] = rintf(__fdiv_rn(v[i], sf));
            }
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int q = (int)__builtin_amdgcn_fmed3f(qf[i], -7.f, 7.f);
            word |= (unsigned)(q & 0xF) << (4 * i);
          }
        }
        if (live) {
          *(unsigned*)(crow + 16 * cg + 4 * qi) = word;
          if (qi == 0) srw[cg] = s16;
        }
      }
    }
  }
}

template <class C>
static hipError_t launch_c(const ProjectParams& p, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  dim3 grid((unsigned)cdiv64(p.n_tok, C::BM), (unsigned)cdiv(p.ntiles, C::NTB));
  if (t0 && t1)
    hipExtLaunchKernelGGL(palu_project_kernel<C>, grid, dim3(C::NT), 0, stream, t0, t1, 0, p);
  else
    hipLaunchKernelGGL(palu_project_kernel<C>, grid, dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_project(int dtype, ProjectParams& p, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (p.n_tok == 0) return hipSuccess;
  // column tiles of at most 160 channels: every latent row in order, split
  // where its rank exceeds 160; a block takes two consecutive tiles
  p.ntiles = 0;
  for (int j = 0; j < 2 * p.G; ++j)
    for (int n0 = 0; n0 < p.rank[j]; n0 += kColTile) {
      if (p.ntiles >= kMaxColTiles || n0 > 0xFFFF) return hipErrorInvalidValue;
      p.tile[p.ntiles++] = j << 16 | n0;
    }
  if (p.ntiles == 0) return hipSuccess;
  switch (dtype) {
    case 0: return launch_c<PrjCfg<float>>(p, stream, t0, t1);
    case 1: return launch_c<PrjCfg<_Float16>>(p, stream, t0, t1);
    case 2: return launch_c<PrjCfg<__bf16>>(p, stream, t0, t1);
  }
  return hipErrorInvalidValue;
}

}  // namespace palu
