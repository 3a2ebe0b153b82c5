// Fused decode attention for MHA head-groups on gfx950: one wave per kv head.
//
// Method: PALU page, section "Low-rank projection decomposition" (K = z_k B_k,
// V = z_v B_v) and section "Inference flow" (decode: read the latents,
// rebuild, attend); arXiv 2407.21118v2 abstract (keys rebuilt on the fly,
// RoPE-based attention, fused kernels).  Same results and split records as
// palu_decode_kernel; this instantiation covers head-groups of 4 kv heads with
// one query head each, head_dim 128, ranks <= 256, 16-bit latents, RoPE.
//
// Design (ours):
//  * Block = the 4 kv heads of a head-group = 4 waves, one per SIMD, so each
//    wave has 512 registers: wave c keeps B_k^T of kv head c (128 dims x 256
//    ranks, 256 registers) for the whole block.  A wave owns whole heads, so
//    its scores are complete in registers and the online softmax runs inside
//    the wave: one block barrier per tile.
//  * 32-token tiles stream HBM -> LDS through LDS DMA, two tiles ahead, into
//    unpadded XOR-swizzled rows (keys: 16-byte chunk index ^ (row & 15);
//    values: ^ ((row & 3) << 1)), so MFMA operand reads and transpose reads
//    are bank-conflict-free and every DMA instruction is fully used.  Key
//    tiles use a ring of 3 buffers, value tiles a ring of 4: the value tile
//    of step n is consumed in step n + 1.
//  * The RoPE angles of a tile (64 frequencies x 32 positions) are formed
//    once per block into a shared table (each lane advances 8 of them by a
//    32-token rotation, re-seeded exactly in fp64 at every segment start and
//    every 64 tiles) one step ahead of use.
//  * Step n: softmax of tile n-1 (scores kept in registers), P . z_v of tile
//    n-1 on MFMA, then the key rebuild of tile n (64 MFMA per 16 tokens) with
//    RoPE and the query dot on the fp32 accumulators.  The running maximum is
//    raised only when a tile's maximum exceeds it by more than 2^8, so the
//    accumulator rescale is rare; P <= 2^8 is split into hi + lo 16-bit parts.
#include "common.h"
#include "decode.h"

#include <hip/hip_ext.h>
#include <type_traits>

namespace palu {
namespace {

template <class LT_>
struct MhaCfg {
  typedef LT_ LT;
  static constexpr int DH = 128, NW = 4, NT = 256, TT = 32;
  static constexpr int RK = 256, RV = 256;
  static constexpr int NKC = RK / 32;          // 32-deep k-chunks of the key rebuild
  static constexpr int NMT = DH / 16;          // 16-row M-tiles per wave (one kv head)
  static constexpr int NNT = RV / 16;          // value n-tiles
  static constexpr int ROWB = RK * 2;          // bytes per LDS latent row (512)
  static constexpr int TILEB = TT * ROWB;      // 16 KB per latent tile
  static constexpr int NDT = TILEB / (16 * NT);   // DMA instructions per wave per latent tile (4)
  static constexpr int NDMA = 2 * NDT + 1;     // per tile step: keys, values, query
  static constexpr int NKB = 3, NVB = 4;       // key / value buffer rings
  static constexpr int AP = 17;                // angle-table row pitch in 16-byte units (68 floats)
  static constexpr int STGB = 32 * DH * NW * 2;   // bytes of one staged B_k chunk (32 ranks x 512 columns)
  static_assert(NDT * 16 * NT == TILEB, "tile DMA");
  static_assert(STGB <= NKB * TILEB && 2 * STGB <= NVB * TILEB, "B_k staging");
};

constexpr float kTau = 8.0f;   // lazy-rescale threshold (log2 domain)

__device__ __forceinline__ void sincos_turns(double t, double theta_turns, float* c, float* s) {
  double rev = t * theta_turns;
  rev -= rint(rev);
  const float r = (float)rev;
  *c = __builtin_amdgcn_cosf(r);
  *s = __builtin_amdgcn_sinf(r);
}

// Scalar load of a wave-uniform 32-bit value (waits in the same block).
__device__ __forceinline__ int sload_i32(const int* ptr) {
  const uint64_t a = (uint64_t)ptr;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(u) : "memory");
  return v;
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

// Reductions over a 16-lane row (DPP only); every lane of the row receives
// the result.
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

}  // namespace

template <class LT>
__global__ void __launch_bounds__(256, 1) palu_decode_mha_kernel(const DecodeParams p) {
  typedef MhaCfg<LT> C;
  typedef typename Vec8<LT>::type op_t;
  typedef short s8 __attribute__((ext_vector_type(8)));
  __shared__ uint4 zkb[C::NKB * C::TILEB / 16];
  __shared__ uint4 zvb[C::NVB * C::TILEB / 16];
  __shared__ f32x4 angc[2 * C::TT * C::AP];       // [table][position][frequency / 4]
  __shared__ f32x4 angs[2 * C::TT * C::AP];
  __shared__ uint4 qst[3][C::NW][16];             // raw query of each wave, one per tile step in flight
  __shared__ double theta[C::DH / 2];             // rotation frequencies in turns per token
  __shared__ f32x4 stpc[C::DH / 8], stps[C::DH / 8];   // rotation by 32 tokens per frequency
  __shared__ int tstart[kMaxBatch + 1];
  __shared__ int wsum[C::NW];
  __shared__ f32x4 pbc[C::NW][C::TT / 4];          // per wave: P of the previous tile, broadcast to all lanes

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = l >> 4, s = l & 15;
  const int g = blockIdx.x % p.G, pb = blockIdx.x / p.G;
  const int batch = p.batch;

  // ---------------------------------------------------------------- tile prefix sums
  {
    constexpr int MAXPER = kMaxBatch / C::NT;
    const int per = cdiv(batch, C::NT);
    int loc[MAXPER];
    int sacc = 0;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int bb = tid * per + i;
      int v = 0;
      if (i < per && bb < batch) {
        int L = p.seq_lens[bb];
        L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
        v = cdiv(L, C::TT);
      }
      loc[i] = v;
      sacc += v;
    }
    int incl = sacc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (l >= d) incl += o;
    }
    if (l == 63) wsum[w] = incl;
    __syncthreads();
    int run = incl - sacc;
    for (int i = 0; i < w; ++i) run += wsum[i];
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int bb = tid * per + i;
      if (i < per && bb < batch) tstart[bb] = run;
      run += loc[i];
    }
    if (tid == C::NT - 1) tstart[batch] = run;
    if (tid < C::DH / 2) {
      const double th = exp2(-(2.0 * tid / C::DH) * log2(p.rope_base)) * 0.15915494309189535;
      theta[tid] = th;
      float c, sn;
      sincos_turns(32.0, th, &c, &sn);
      ((float*)stpc)[tid] = c;
      ((float*)stps)[tid] = sn;
    }
    __syncthreads();
  }
  const int total = tstart[batch];
  if (g == 0 && pb == 0) {
    for (int i = tid; i <= batch; i += C::NT) p.hdr[i] = tstart[i];
  }
  const int tpb = cdiv(total, p.P);
  const int n_begin = pb * tpb;
  const int n_end = min(total, n_begin + tpb);
  if (n_begin >= n_end) return;

  const int rk = p.rk[g];
  const int pk = p.pk[g], pv = p.pv[g];
  const int cprk = pk >> 4, cprv = pv >> 4;
  const uint8_t* zk_seq = p.zk + p.goff_k[g];
  const uint8_t* zv_seq = p.zv + p.goff_v[g];
  const int64_t sbk = p.seq_bytes_k, sbv = p.seq_bytes_v;
  const int h = g * C::NW + w;                    // query head of this wave (one per kv head)

  // ---------------------------------------------------------------- B_k^T of kv head w into registers
  op_t breg[C::NKC][C::NMT];   // [k-chunk][M-tile]
  {
    const LT* Bg = (const LT*)p.Bk + p.boff_k[g];   // [rk][4 * DH]
    constexpr int W = C::NW * C::DH;
    constexpr int NSI = C::STGB / (16 * C::NT);     // DMA instructions per wave per staged chunk (8)
    uint8_t* const slots[3] = {(uint8_t*)zkb, (uint8_t*)zvb, (uint8_t*)zvb + C::STGB};
    auto stage = [&](int slot, int kc) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < NSI; ++m) {
        const int q = (m * C::NW + w) * 64 + l;     // 16-byte slot of the staged chunk
        const int row = q >> 6, col = (q & 63) * 8;
        const int kr = min(kc * 32 + row, rk - 1);
        dma16(Bg + (int64_t)kr * W + col, lds_addr(slots[slot]) + 16u * ((m * C::NW + w) * 64));
      }
    };
    auto gather = [&](int slot, int kc) __attribute__((always_inline)) {
      const LT* sb = (const LT*)slots[slot];
#pragma unroll
      for (int mt = 0; mt < C::NMT; ++mt) {
        const int j = mt >> 1, hh = mt & 1;
        const int i0 = w * C::DH + hh * (C::DH / 2) + 16 * j;
        // (the rank is a multiple of 32: every staged row is a real row of B_k)
        const i16x4 lo = ds_read_tr16(sb + (8 * kq + (s >> 2)) * W + i0 + 4 * (s & 3));
        const i16x4 hi = ds_read_tr16(sb + (8 * kq + 4 + (s >> 2)) * W + i0 + 4 * (s & 3));
        const s8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        // move the operand into the AGPR file once; it stays there
        op_t v = __builtin_bit_cast(op_t, both), av;
        asm volatile("" : "=a"(av) : "0"(v));
        breg[kc][mt] = av;
      }
    };
    const int nkc = cdiv(rk, 32);
    stage(0, 0);
    if (1 < nkc) stage(1, 1);
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc) {
      if (kc < nkc) {
        if (kc + 1 < nkc) wait_vmcnt<NSI>(); else wait_vmcnt<0>();
        barrier();
        if (kc + 2 < nkc) stage((kc + 2) % 3, kc + 2);
        gather(kc % 3, kc);
      } else {
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt) {
          op_t z = op_t{}, az;
          asm volatile("" : "=a"(az) : "0"(z));
          breg[kc][mt] = az;
        }
      }
    }
    wait_lgkm0();
    barrier();   // staging buffers are free before the tile DMA overwrites them
  }

  // ---------------------------------------------------------------- per-lane constants
  // DMA slots: instruction m of wave w fills 16-byte slots (m*NW + w)*64 + l of
  // a tile = row q >> 5, physical chunk q & 31, holding the logical chunk
  // given by the swizzle; chunks past a row's data load chunk 0 (finite, and
  // multiplied by zero rows of B_k or ignored by the merge).
  // (row, key chunk byte, value chunk byte) of DMA slot m of this lane
  auto dslot = [&](int m, int& row, int& ck, int& cv) __attribute__((always_inline)) {
    const int q = (m * C::NW + w) * 64 + l;
    const int pc = q & 31;
    row = q >> 5;
    const int lck = pc ^ (row & 15), lcv = pc ^ ((row & 3) << 1);
    ck = 16 * (lck < cprk ? lck : 0);
    cv = 16 * (lcv < cprv ? lcv : 0);
  };
  unsigned koff[C::NDT], voff[C::NDT];          // byte offsets inside a full tile
#pragma unroll
  for (int m = 0; m < C::NDT; ++m) {
    int row, ck, cv;
    dslot(m, row, ck, cv);
    koff[m] = (unsigned)(row * pk + ck);
    voff[m] = (unsigned)(row * pv + cv);
  }
  // key operand reads: token row 16u + s, logical chunk 4 kc + kq
  const int sh = s >> 2, sl = s & 3;
  int kaddr[4];
#pragma unroll
  for (int b4 = 0; b4 < 4; ++b4) kaddr[b4] = s * C::ROWB + 16 * (kq ^ sl) + 64 * (b4 ^ sh);
  // value reads: lane l accumulates ranks 4l .. 4l+3 (logical chunk l/2, half l%2)
  int vofs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) vofs[r] = 16 * ((l >> 1) ^ (2 * r)) + 8 * (l & 1);
  // angle-table writer: position tau, frequency quads f4a and f4a + 8
  const int tau = tid & 31, f4a = tid >> 5;

  // ---------------------------------------------------------------- tile cursors (wave-uniform)
  // A cursor walks the block's tiles in order: tile n of sequence b starts at
  // token t0 of a history of L tokens; empty sequences hold no tiles.
  auto len_of = [&](int b) __attribute__((always_inline)) {
    int L = sload_i32(p.seq_lens + b);
    return L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
  };
  struct Cur { int n, b, t0, L; };
  Cur c0;
  {
    int b = 0;
    while (tstart[b + 1] <= n_begin) ++b;
    b = __builtin_amdgcn_readfirstlane(b);
    c0.n = n_begin;
    c0.b = b;
    c0.t0 = __builtin_amdgcn_readfirstlane((n_begin - tstart[b]) * C::TT);
    c0.L = len_of(b);
  }
  auto advance = [&](Cur& c) __attribute__((always_inline)) {
    ++c.n;
    c.t0 += C::TT;
    if (c.t0 >= c.L && c.n < n_end) {
      int b = c.b + 1, L = len_of(b);
      while (L == 0) L = len_of(++b);
      c.b = b;
      c.L = L;
      c.t0 = 0;
    }
  };
  auto seg_start = [&](const Cur& c) __attribute__((always_inline)) { return c.t0 == 0 || c.n == n_begin; };
  auto seg_end = [&](const Cur& c) __attribute__((always_inline)) { return c.t0 + C::TT >= c.L || c.n == n_end - 1; };

  auto issue = [&](const Cur& c) __attribute__((always_inline)) {
    const uint8_t* kb = zk_seq + (int64_t)c.b * sbk + (int64_t)c.t0 * pk;
    const uint8_t* vb = zv_seq + (int64_t)c.b * sbv + (int64_t)c.t0 * pv;
    const unsigned kdst = lds_addr(zkb) + (unsigned)((c.n % C::NKB) * C::TILEB);
    const unsigned vdst = lds_addr(zvb) + (unsigned)((c.n % C::NVB) * C::TILEB);
    const int lim = c.L - 1 - c.t0;
    if (lim >= C::TT - 1) {
#pragma unroll
      for (int m = 0; m < C::NDT; ++m) dma16s(kb, koff[m], kdst + 16u * ((m * C::NW + w) * 64));
#pragma unroll
      for (int m = 0; m < C::NDT; ++m) dma16s(vb, voff[m], vdst + 16u * ((m * C::NW + w) * 64));
    } else {
      // last tile of a history: rows past it repeat its last row
#pragma unroll
      for (int m = 0; m < C::NDT; ++m) {
        int row, ck, cv;
        dslot(m, row, ck, cv);
        dma16s(kb, (unsigned)(min(row, lim) * pk + ck), kdst + 16u * ((m * C::NW + w) * 64));
      }
#pragma unroll
      for (int m = 0; m < C::NDT; ++m) {
        int row, ck, cv;
        dslot(m, row, ck, cv);
        dma16s(vb, (unsigned)(min(row, lim) * pv + cv), vdst + 16u * ((m * C::NW + w) * 64));
      }
    }
    // this wave's query (256 bytes, lanes 0-15; loaded at every step so that
    // every step issues the same number of DMA instructions)
    const uint8_t* qb = (const uint8_t*)p.q + ((int64_t)c.b * p.H + h) * (C::DH * 2);
    if (l < 16) dma16s(qb, 16u * l, lds_addr(&qst[c.n % 3][w][0]));
  };

  // Angle table of tile c.n from the table of tile c.n - 1 (same entries of
  // this lane, rotated by 32 positions), or seeded exactly.  The previous
  // entries and the rotation are read first (ang_fetch) so that their LDS
  // latency passes while other work runs.
  struct AngIn { f32x4 pc0, pc1, ps0, ps1, rc0, rc1, rs0, rs1; };
  auto ang_fetch = [&](const Cur& c, AngIn& in) __attribute__((always_inline)) {
    const f32x4* pc = angc + ((c.n - 1) & 1) * (C::TT * C::AP) + tau * C::AP;
    const f32x4* ps = angs + ((c.n - 1) & 1) * (C::TT * C::AP) + tau * C::AP;
    in.pc0 = pc[f4a];
    in.pc1 = pc[f4a + 8];
    in.ps0 = ps[f4a];
    in.ps1 = ps[f4a + 8];
    in.rc0 = stpc[f4a];
    in.rc1 = stpc[f4a + 8];
    in.rs0 = stps[f4a];
    in.rs1 = stps[f4a + 8];
  };
  auto angles = [&](const Cur& c, const AngIn& in, bool have_prev) __attribute__((always_inline)) {
    f32x4 oc0, oc1, os0, os1;
    if (!have_prev || seg_start(c) || ((c.n - n_begin) & 63) == 0) {
      // exact seed at this tile's first position
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float cv, sv;
        sincos_turns((double)(c.t0 + tau), theta[4 * f4a + i], &cv, &sv);
        oc0[i] = cv;
        os0[i] = sv;
        sincos_turns((double)(c.t0 + tau), theta[4 * (f4a + 8) + i], &cv, &sv);
        oc1[i] = cv;
        os1[i] = sv;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        oc0[i] = in.pc0[i] * in.rc0[i] - in.ps0[i] * in.rs0[i];
        os0[i] = in.ps0[i] * in.rc0[i] + in.pc0[i] * in.rs0[i];
        oc1[i] = in.pc1[i] * in.rc1[i] - in.ps1[i] * in.rs1[i];
        os1[i] = in.ps1[i] * in.rc1[i] + in.pc1[i] * in.rs1[i];
      }
    }
    f32x4* tc = angc + (c.n & 1) * (C::TT * C::AP) + tau * C::AP;
    f32x4* ts = angs + (c.n & 1) * (C::TT * C::AP) + tau * C::AP;
    tc[f4a] = oc0;
    tc[f4a + 8] = oc1;
    ts[f4a] = os0;
    ts[f4a + 8] = os1;
  };

  // ---------------------------------------------------------------- running state
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};         // ranks 4l .. 4l+3 of sum_t P_t z_v[t]
  float m_run = -INFINITY, l_run = 0.f;
  float qlo[4][4], qhi[4][4];
  float sc0 = 0.f, sc1 = 0.f;                     // scores of the previous tile
  Cur prev = c0;
  float* const pb_w = (float*)&pbc[w][0];         // this wave's P of the previous tile

  // online softmax of the previous tile; its P goes to pb_w
  auto softmax_prev = [&]() __attribute__((always_inline)) {
    const float x0 = (prev.t0 + s < prev.L) ? sc0 : -INFINITY;
    const float x1 = (prev.t0 + 16 + s < prev.L) ? sc1 : -INFINITY;
    // every row of the wave holds the same 16 token pairs: the maximum is uniform
    const float tmax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(max16(fmaxf(x0, x1)))));
    if (tmax > m_run + kTau) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - tmax);
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= alpha;
      m_run = tmax;
    }
    const float p0 = __builtin_amdgcn_exp2f(x0 - m_run);
    const float p1 = __builtin_amdgcn_exp2f(x1 - m_run);
    l_run += sum16(p0 + p1);
    if (kq == 0) {
      pb_w[s] = p0;
      pb_w[16 + s] = p1;
    }
  };

  // P z_v of the previous tile for tokens 4k .. 4k+3 (P broadcast from LDS)
  auto pv_part = [&](const uint8_t* zv, const f32x4& pq, int k) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * k + i;
      const float pt = pq[i];
      const uint2 z = *(const uint2*)(zv + t * C::ROWB + vofs[t & 3]);
      if constexpr (std::is_same<LT, _Float16>::value) {
        const _Float16* zh = (const _Float16*)&z;
        acc[0] = fmaf(pt, (float)zh[0], acc[0]);
        acc[1] = fmaf(pt, (float)zh[1], acc[1]);
        acc[2] = fmaf(pt, (float)zh[2], acc[2]);
        acc[3] = fmaf(pt, (float)zh[3], acc[3]);
      } else {
        acc[0] = fmaf(pt, __uint_as_float(z.x << 16), acc[0]);
        acc[1] = fmaf(pt, __uint_as_float(z.x & 0xFFFF0000u), acc[1]);
        acc[2] = fmaf(pt, __uint_as_float(z.y << 16), acc[2]);
        acc[3] = fmaf(pt, __uint_as_float(z.y & 0xFFFF0000u), acc[3]);
      }
    }
  };

  auto record_prev = [&]() __attribute__((always_inline)) {
    float* rec = p.rec + ((int64_t)g * (p.P + batch) + pb + prev.b) * p.rec_stride;
    *(f32x4*)(rec + 2 * C::NW + w * p.rvp + 4 * l) = acc;
    if (l == 0) {
      rec[2 * w] = m_run;
      rec[2 * w + 1] = l_run;
    }
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  };

  // RoPE on the rebuilt keys of one 16-token half and the query dot (pairs of
  // frequency blocks j0 .. j1-1)
  auto rope_part = [&](const f32x4 (&kt)[C::NMT], const f32x4 (&cj)[4], const f32x4 (&sj)[4], int j0, int j1,
                       float part) __attribute__((always_inline)) {
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const f32x4 c4 = cj[j], s4 = sj[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = kt[2 * j][e], bq = kt[2 * j + 1][e];
        const float klo = a * c4[e] - bq * s4[e];
        const float khi = a * s4[e] + bq * c4[e];
        part = fmaf(qlo[j][e], klo, part);
        part = fmaf(qhi[j][e], khi, part);
      }
    }
    return part;
  };

  // ---------------------------------------------------------------- pipeline
  Cur cd = c0;                 // next tile to load
  issue(cd);
  advance(cd);
  if (cd.n < n_end) { issue(cd); advance(cd); }
  Cur ca = c0;                 // next angle table
  {
    AngIn in0;
    angles(ca, in0, false);
  }
  advance(ca);
  Cur cc = c0;                 // tile to rebuild

  for (int n = n_begin; n <= n_end; ++n) {
    if (n < n_end) {
      if (n + 1 < n_end) wait_vmcnt<C::NDMA>(); else wait_vmcnt<0>();
    }
    barrier();   // tile n and angle table n visible; every wave finished step n - 1
    const bool have = n < n_end, had = n > n_begin;
    AngIn ain;
    const bool do_ang = ca.n < n_end;
    if (do_ang) ang_fetch(ca, ain);
    if (have && seg_start(cc)) {
      // segment start: rotate this wave's query to its position, pre-scaled
      const int pos = p.q_pos ? sload_i32(p.q_pos + cc.b) : cc.L - 1;
      const LT* qr = (const LT*)&qst[cc.n % 3][w][0];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int f = 16 * j + 4 * kq + e;
          float cs, sn;
          sincos_turns((double)pos, theta[f], &cs, &sn);
          const float a = to_f32(qr[f]), bq = to_f32(qr[f + C::DH / 2]);
          qlo[j][e] = (a * cs - bq * sn) * p.qscale;
          qhi[j][e] = (a * sn + bq * cs) * p.qscale;
        }
      }
    }
    if (had) softmax_prev();
    if (cd.n < n_end) { issue(cd); advance(cd); }
    if (do_ang) { angles(ca, ain, true); advance(ca); }

    const uint8_t* zk = (const uint8_t*)zkb + (cc.n % C::NKB) * C::TILEB;
    const uint8_t* zv = (const uint8_t*)zvb + (prev.n % C::NVB) * C::TILEB;
    const f32x4* tc = angc + (cc.n & 1) * (C::TT * C::AP) + s * C::AP + kq;
    const f32x4* ts = angs + (cc.n & 1) * (C::TT * C::AP) + s * C::AP + kq;
    f32x4 k0[C::NMT], k1[C::NMT];
    // window A: keys of tokens 0-15 on MFMA beside P z_v of the previous tile;
    // the operands of window B and the angles of tokens 0-15 are fetched here
    op_t bopb[C::NKC];
    auto prefetch_b = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc)
        bopb[kc] = *(const op_t*)(zk + kaddr[kc & 3] + 256 * (kc >> 2) + 16 * C::ROWB);
    };
    auto window_a = [&](bool with_pv) __attribute__((always_inline)) {
      op_t bop[C::NKC];
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) bop[kc] = *(const op_t*)(zk + kaddr[kc & 3] + 256 * (kc >> 2));
      prefetch_b();
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) {
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt)
          k0[mt] = mfma16x16x32(breg[kc][mt], bop[kc], kc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : k0[mt]);
        if (with_pv) pv_part(zv, *(const f32x4*)(pb_w + 4 * kc), kc);
      }
      // issue pattern: every MFMA followed by two VALU (the P z_v FMAs)
#pragma unroll
      for (int i = 0; i < C::NKC * C::NMT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    };
    if (have && had) {
      window_a(true);
    } else if (have) {
      window_a(false);
    } else if (had) {
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) pv_part(zv, *(const f32x4*)(pb_w + 4 * kc), kc);
    }
    if (had && seg_end(prev)) record_prev();
    if (have) {
      // window B: keys of tokens 16-31 on MFMA beside RoPE + dot of tokens 0-15;
      // the angles of tokens 16-31 are fetched here
      f32x4 ca0[4], sa0[4], ca1[4], sa1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ca0[j] = tc[4 * j];
        sa0[j] = ts[4 * j];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ca1[j] = tc[16 * C::AP + 4 * j];
        sa1[j] = ts[16 * C::AP + 4 * j];
      }
      float part = 0.f;
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) {
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt)
          k1[mt] = mfma16x16x32(breg[kc][mt], bopb[kc], kc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : k1[mt]);
        if (kc % 2 == 1) part = rope_part(k0, ca0, sa0, kc / 2, kc / 2 + 1, part);
      }
      // issue pattern: every MFMA followed by two VALU (RoPE and dot of tokens 0-15)
#pragma unroll
      for (int i = 0; i < C::NKC * C::NMT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      sc0 = rows4_sum(part);
      sc1 = rows4_sum(rope_part(k1, ca1, sa1, 0, 4, 0.f));
      prev = cc;
      advance(cc);
    }
  }
}

bool mha_supported(const DecodeKey& k, const DecodeParams& p) {
  if (!((k.elt == Elt::F16 || k.elt == Elt::BF16) && k.head_dim == 128 && k.kv_per_group == 4 &&
        k.q_per_kv == 1 && k.rope && k.rk_max <= 256 && k.rv_max <= 256))
    return false;
  for (int j = 0; j < p.G; ++j)
    if (p.rk[j] % 32 != 0) return false;   // B_k is staged in whole 32-row chunks
  return true;
}

hipError_t launch_decode_mha(const DecodeKey& k, const DecodeParams& p, hipStream_t stream, hipEvent_t t0,
                             hipEvent_t t1) {
  const dim3 grid(p.G * p.P), block(256);
  if (k.elt == Elt::F16) {
    if (t0 && t1)
      hipExtLaunchKernelGGL(palu_decode_mha_kernel<_Float16>, grid, block, 0, stream, t0, t1, 0, p);
    else
      hipLaunchKernelGGL(palu_decode_mha_kernel<_Float16>, grid, block, 0, stream, p);
  } else {
    if (t0 && t1)
      hipExtLaunchKernelGGL(palu_decode_mha_kernel<__bf16>, grid, block, 0, stream, t0, t1, 0, p);
    else
      hipLaunchKernelGGL(palu_decode_mha_kernel<__bf16>, grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace palu
