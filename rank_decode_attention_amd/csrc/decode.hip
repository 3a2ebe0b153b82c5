// Fused decode attention over the low-rank latent cache (gfx950).
//
// Method: PALU page, section "Low-rank projection decomposition" (formula
// block: K = z_k B_k, V = z_v B_v) and section "Inference flow" (decode:
// read the latents, rebuild or fuse, attend); arXiv 2407.21118v2 abstract
// (keys and values rebuilt on the fly; RoPE-based attention; fused kernels).
//
// Design (ours; the pages give no kernel):
//  * Work is the flattened list of 32-token tiles of all sequences (each
//    sequence padded to a whole tile).  Block (g, p) takes the p-th equal
//    share of the tiles of head-group g, so ragged batches balance exactly.
//    Where a share crosses a sequence boundary the block closes a split
//    record (m, l, acc) and opens the next; record index p + b is unique.
//  * B_k^g stays in VGPRs for the whole block (loaded once through LDS with
//    transpose reads); each wave owns 16 frequency rows of PPW heads in both
//    RoPE halves, so the pair (i, i + d/2) of a rebuilt key sits in one lane.
//  * Latent tiles stream HBM -> LDS with LDS DMA (global_load_lds_dwordx4),
//    three buffers deep, XOR-swizzled for conflict-free MFMA operand reads.
//  * K^T tile = B_k^T z_k^T on MFMA (16x16x32 for 16-bit, 16x16x4 for fp32),
//    RoPE on the fp32 accumulator with angle recurrences seeded in fp64,
//    scores by in-lane dots + a 4-lane reduction, online softmax in the log2
//    domain, and acc += P z_v on MFMA with P split into hi + lo 16-bit parts
//    (exact to ~2^-22) and z_v read through ds_read_b64_tr_b16.
//  * Without RoPE the score is the absorbed query (q B_k^T, pre-computed per
//    call, hi/lo split) against z_k on MFMA; K is never rebuilt.
//  * A second kernel merges the split records and applies B_v per head.
#include "common.h"
#include "decode.h"

#include <hip/hip_ext.h>
#include <mutex>
#include <type_traits>

namespace palu {

template <class LT_, int DH_, int NG_, int QPK_, int NKC_, int RKMAX_, int RVMAX_, bool ROPE_, int NW_>
struct DecCfg {
  typedef LT_ LT;
  static constexpr bool F32 = std::is_same<LT, float>::value;
  static constexpr int ESZ = sizeof(LT);
  static constexpr int DH = DH_, NG = NG_, QPK = QPK_, NKC = NKC_;
  static constexpr int RKMAX = RKMAX_, RVMAX = RVMAX_;
  static constexpr bool ROPE = ROPE_;
  static constexpr int TT = kDecTile, NW = NW_, NT = 64 * NW_;
  static constexpr int NJ = DH / 32;                    // 16-row frequency blocks per head half
  static constexpr int PPW = ROPE ? NG * NJ / NW : 0;   // kv heads per wave
  static constexpr int RT = 2 * PPW;                    // 16-row MFMA tiles per wave
  static constexpr int NQ = NG * QPK;                   // query heads per group
  static constexpr int KC = F32 ? 16 : 32;              // k per operand chunk
  static constexpr int W = NG * DH;                     // group width
  static constexpr int CPRK = RKMAX * ESZ / 16, CPRV = RVMAX * ESZ / 16;
  // LDS rows are padded so that consecutive token rows start 4 banks apart
  // (keys, 16-byte MFMA operand reads) or 8 banks apart (values, 8-byte
  // transpose reads); the pitch is fixed per instantiation so every operand
  // address is one per-lane base plus a compile-time offset.
  static constexpr int PITK = cdiv(CPRK, 8) * 8 + 1;    // key row pitch in 16-byte slots
  static constexpr int PITV = cdiv(CPRV, 8) * 8 + 2;    // value row pitch in 16-byte slots
  static constexpr int SLK = cdiv(TT * PITK, 64) * 64;  // 16-byte slots of the key region
  static constexpr int SLV = cdiv(TT * PITV, 64) * 64;
  static constexpr int NIK = cdiv(SLK, 64 * NW), NIV = cdiv(SLV, 64 * NW);
  static constexpr int NDMA = NIK + NIV;                // DMA instructions per wave per tile
  // each buffer ends with one instruction's worth of overflow slots: DMA
  // instructions of waves past a region's end land there (never read), so
  // every DMA destination stays inside its own buffer object
  static constexpr int PADS = 64;
  static constexpr int BUFB = (SLK + SLV + PADS) * 16;  // bytes per pipeline buffer
  static constexpr int NNT = RVMAX / 16;                // value n-tiles
  static constexpr int NNTW = cdiv(NNT, NW);
  // partial scores per (head, token): RoPE one per (frequency block, row
  // group); absorbed query one per (wave, hi|lo part)
  // (with several query heads per kv head the row groups are pre-summed in
  // registers to keep the LDS footprint down)
  static constexpr bool PRESUM = ROPE && QPK > 1;
  static constexpr int NP = ROPE ? NJ * (PRESUM ? 1 : 4) : NW;
  static constexpr int NPP = (NP % 8 == 0) ? NP + 4 : cdiv(NP, 4) * 4;   // padded, 16-byte rows
  static constexpr int SMW = cdiv(NQ * TT, 64);         // waves computing the softmax
  static constexpr int PTP = F32 ? TT + 4 : TT + 8;     // P tile row pitch (elements, 16 B padding)
  static constexpr int STG_ROWS = KC;                   // B_k rows staged per pass
  static constexpr int NSI = cdiv(STG_ROWS * W * ESZ / 16, 64 * NW);  // DMA instr per wave per pass

  static_assert(RKMAX % KC == 0 && RVMAX % 16 == 0, "rank caps");
  static_assert(NKC * KC == RKMAX, "register chunks");
  static_assert(!ROPE || (NG * NJ) % NW == 0, "wave mapping needs NG*DH/32 divisible by 8");
  static_assert(!ROPE || NW % NJ == 0, "wave mapping");
  static_assert(F32 ? NQ <= 16 : NQ <= 8, "query heads per group");
  static_assert(STG_ROWS * W * ESZ <= BUFB, "B_k staging must fit one buffer");
  static_assert(DH % 32 == 0, "head_dim");
  static_assert(SMW <= NW && TT == 32, "softmax lanes");
};

// Operand registers of one 16x16xK MFMA input: 8 x 16-bit or 4 x fp32.
template <class LT> struct Op { typedef typename Vec8<LT>::type type; };
template <> struct Op<float> { typedef f32x4 type; };

template <class LT>
__device__ __forceinline__ f32x4 mma(const typename Op<LT>::type& a, const typename Op<LT>::type& b, f32x4 c) {
  if constexpr (std::is_same<LT, float>::value) {
    c = mfma16x16x4(a[0], b[0], c);
    c = mfma16x16x4(a[1], b[1], c);
    c = mfma16x16x4(a[2], b[2], c);
    c = mfma16x16x4(a[3], b[3], c);
    return c;
  } else {
    return mfma16x16x32(a, b, c);
  }
}

// cos/sin of the angle t*theta: the product and its reduction to one turn are
// done in fp64 (exact enough for t up to 2^31), then the hardware sin/cos,
// which take their argument in turns, evaluate the reduced angle.
__device__ __forceinline__ void sincos_angle(double t, double theta_turns, float* c, float* s) {
  double rev = t * theta_turns;
  rev -= rint(rev);
  const float r = (float)rev;
  *c = __builtin_amdgcn_cosf(r);
  *s = __builtin_amdgcn_sinf(r);
}

template <class C>
struct DecState {
  typedef typename C::LT LT;
  typedef typename Op<LT>::type op_t;
  op_t breg[C::ROPE ? C::RT : 1][C::ROPE ? C::NKC : 1];   // B_k^T operand (RoPE path)
  op_t aq[C::ROPE ? 1 : C::NKC];                          // absorbed query operand (no-RoPE path)
  float cs[4], sn[4];                                     // angle at the current tile (u = 0)
  // rotated, pre-scaled query of the lane's rows (one kv head per wave)
  f32x4 qr[C::ROPE && C::PPW * C::QPK <= 4 ? C::PPW * C::QPK * 2 : 1];
  f32x4 acc[C::NNTW];                                     // P z_v accumulators
  float m_run, l_run;
  int L;                                                  // history length of the current sequence
};

template <class C>
__global__ void __launch_bounds__(C::NT, 1) palu_decode_kernel(const DecodeParams p) {
  typedef typename C::LT LT;
  typedef typename Op<LT>::type op_t;
  __shared__ uint4 buf0[C::BUFB / 16];
  __shared__ uint4 buf1[C::BUFB / 16];
  __shared__ uint4 buf2[C::BUFB / 16];
  __shared__ float spart[C::NQ * C::TT * C::NPP];
  __shared__ uint4 ptile[(16 * C::PTP * (C::F32 ? 4 : 2) + 15) / 16];   // P operand: [16 rows][PTP]
  __shared__ float arow[16];                                             // rescale factor per P row
  __shared__ int tstart[kMaxBatch + 1];
  __shared__ int slen[kMaxBatch];
  __shared__ int wsum[C::NW];
  // rotated, pre-scaled query values of each wave: [wave][lane row group][x][qq][half] x 4 rows
  __shared__ f32x4 qtab[C::ROPE ? C::NW * 4 * C::PPW * C::QPK * 2 : 1];
  // cos / sin of the 16-token rotation of each wave's frequency rows: [wave][row group][cos|sin]
  __shared__ f32x4 steptab[C::ROPE ? C::NW * 4 * 2 : 1];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lane = l;
  const int g = blockIdx.x % p.G, pb = blockIdx.x / p.G;
  const int batch = p.batch;
  LT* ptile_h = (LT*)ptile;          // 16-bit P operand rows (hi rows 0-7, lo rows 8-15)
  float* ptile_f = (float*)ptile;    // fp32 P operand rows
  // P rows of absent heads stay zero; their rescale factor stays one
  for (int i = tid; i < (int)(sizeof(ptile) / 16); i += C::NT) ptile[i] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < 16) arow[tid] = 1.f;

  // ---------------------------------------------------------------- tile prefix sums
  {
    // each thread scans up to 4 consecutive sequences, then a block scan
    constexpr int MAXPER = kMaxBatch / C::NT;
    const int per = cdiv(batch, C::NT);
    int loc[MAXPER];
    int s = 0;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      int bb = tid * per + i;
      int v = 0;
      if (i < per && bb < batch) {
        int L = p.seq_lens[bb];
        L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
        slen[bb] = L;
        v = cdiv(L, C::TT);
      }
      loc[i] = v;
      s += v;
    }
    // inclusive wave scan of s
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int o = __shfl_up(incl, d, 64);
      if (l >= d) incl += o;
    }
    if (l == 63) wsum[w] = incl;
    __syncthreads();
    int wbase = 0;
    for (int i = 0; i < w; ++i) wbase += wsum[i];
    int run = wbase + incl - s;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      int bb = tid * per + i;
      if (i < per && bb < batch) tstart[bb] = run;
      run += loc[i];
    }
    if (tid == C::NT - 1) tstart[batch] = run;
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

  const int rk = p.rk[g], rv = p.rv[g];
  const int pk = p.pk[g], pv = p.pv[g];
  const int cprk = pk >> 4, cprv = pv >> 4;
  const int nkc = cdiv(rk, C::KC);
  const int nnt = cdiv(rv, 16);

  DecState<C> st;

  // ---------------------------------------------------------------- per-lane DMA slot geometry
  // slot (row, pos) of each DMA instruction is fixed for the block; only the
  // sequence base and tile start change per tile.
  // Slot q of a region holds chunk (q % PIT) of token row (q / PIT); slots
  // past the row's data (padding) load a valid chunk that is never read.
  int dk_geo[C::NIK], dv_geo[C::NIV];   // (row << 16) | byte offset inside the row
#pragma unroll
  for (int m = 0; m < C::NIK; ++m) {
    const int slot = (m * C::NW + w) * 64 + l;
    int row = slot / C::PITK, pos = slot - row * C::PITK;
    row = row < C::TT ? row : C::TT - 1;
    pos = pos < cprk ? pos : 0;
    dk_geo[m] = (row << 16) | (pos * 16);
  }
#pragma unroll
  for (int m = 0; m < C::NIV; ++m) {
    const int slot = (m * C::NW + w) * 64 + l;
    int row = slot / C::PITV, pos = slot - row * C::PITV;
    row = row < C::TT ? row : C::TT - 1;
    pos = pos < cprv ? pos : 0;
    dv_geo[m] = (row << 16) | (pos * 16);
  }
  const uint8_t* zk_seq = p.zk + p.goff_k[g];
  const uint8_t* zv_seq = p.zv + p.goff_v[g];
  const int64_t sbk = p.seq_bytes_k, sbv = p.seq_bytes_v;

  // locate the sequence holding tile n (n >= tstart[b0]); returns b
  auto seq_of = [&](int n, int b0) __attribute__((always_inline)) {
    int b = b0;
    while (tstart[b + 1] <= n) ++b;
    return b;
  };
  auto seq_len = [&](int b) { return slen[b]; };

  auto issue_tile = [&](uint4* bufp, int b, int t0, int L) __attribute__((always_inline)) {
    // wave-uniform 64-bit bases, per-lane 32-bit offsets (rows past the
    // history are clamped to its last row: valid memory, masked later).
    // Paged caches: the tile's 32 rows lie in one page (pages hold a power
    // of two >= 32 rows); block = page index, rows counted inside the page.
    int blk = b, tin = t0;
    if (p.block_table) {
      blk = sload_i32(p.block_table + (int64_t)b * p.max_pages + (t0 >> p.page_shift));
      tin = t0 & ((1 << p.page_shift) - 1);
    }
    const uint8_t* kb = zk_seq + (int64_t)blk * sbk + (uint32_t)tin * (uint32_t)pk;
    const uint8_t* vb = zv_seq + (int64_t)blk * sbv + (uint32_t)tin * (uint32_t)pv;
    const int lim = L - 1 - t0;
#pragma unroll
    for (int m = 0; m < C::NIK; ++m) {
      const int sbase = (m * C::NW + w) * 64;
      const uint32_t off = (uint32_t)min(dk_geo[m] >> 16, lim) * (uint32_t)pk + (uint32_t)(dk_geo[m] & 0xFFFF);
      const unsigned dst = lds_addr(bufp) + 16u * (sbase < C::SLK ? sbase : C::SLK + C::SLV);
      dma16(kb + off, dst);
    }
#pragma unroll
    for (int m = 0; m < C::NIV; ++m) {
      const int sbase = (m * C::NW + w) * 64;
      const uint32_t off = (uint32_t)min(dv_geo[m] >> 16, lim) * (uint32_t)pv + (uint32_t)(dv_geo[m] & 0xFFFF);
      const unsigned dst = lds_addr(bufp) + 16u * (sbase < C::SLV ? C::SLK + sbase : C::SLK + C::SLV);
      dma16(vb + off, dst);
    }
  };

  // rotation frequencies theta_f = base^(-2f/DH), stored in turns per token
  __shared__ double theta_lds[C::DH / 2];
  if (tid < C::DH / 2) theta_lds[tid] = exp2(-(2.0 * tid / C::DH) * log2(p.rope_base)) * 0.15915494309189535;
  __syncthreads();
  auto rope_theta = [&](int f) __attribute__((always_inline)) { return theta_lds[f]; };

  // ---------------------------------------------------------------- B_k^g into registers (RoPE path)
  const int jf = w % C::NJ;                       // frequency block of this wave
  const int cbase = C::ROPE ? (w / C::NJ) * C::PPW : 0;   // first local kv head of this wave
  if constexpr (C::ROPE) {
    const LT* Bg = (const LT*)p.Bk + p.boff_k[g];
    constexpr int STG_SLOTS = C::STG_ROWS * C::W * C::ESZ / 16;
    auto stage = [&](uint4* bufp, int kc) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < C::NSI; ++m) {
        int sbase = (m * C::NW + w) * 64;
        int slot = sbase + l;
        slot = slot < STG_SLOTS ? slot : STG_SLOTS - 1;
        int e0 = slot * (16 / C::ESZ);              // element index in the staged block
        int row = e0 / C::W, col = e0 - row * C::W;
        int kr = kc * C::KC + row;
        kr = kr < rk ? kr : rk - 1;
        const unsigned dst = lds_addr(bufp) + 16u * (sbase < STG_SLOTS ? sbase : C::SLK + C::SLV);
        dma16(Bg + (int64_t)kr * C::W + col, dst);
      }
    };
    auto gather = [&](const uint4* bufp, int kc) __attribute__((always_inline)) {
      const LT* sb = (const LT*)bufp;
      const int kq = l >> 4, s = l & 15;
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) {
        const int x = rt >> 1, half = rt & 1;
        const int i0 = (cbase + x) * C::DH + half * (C::DH / 2) + 16 * jf;
        op_t v;
        if constexpr (C::F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            int krow = 4 * kq + e;
            float val = sb[krow * C::W + i0 + s];
            v[e] = (kc * C::KC + krow) < rk ? val : 0.f;
          }
        } else {
          i16x4 lo = ds_read_tr16(sb + (8 * kq + (s >> 2)) * C::W + i0 + 4 * (s & 3));
          i16x4 hi = ds_read_tr16(sb + (8 * kq + 4 + (s >> 2)) * C::W + i0 + 4 * (s & 3));
          typedef short s8 __attribute__((ext_vector_type(8)));
          s8 both;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            both[e] = (kc * C::KC + 8 * kq + e) < rk ? lo[e] : (short)0;
            both[e + 4] = (kc * C::KC + 8 * kq + 4 + e) < rk ? hi[e] : (short)0;
          }
          v = __builtin_bit_cast(op_t, both);
        }
        st.breg[rt][kc] = v;
      }
    };
    // three-deep staging pipeline over the NKC chunks of B_k rows
    stage(buf0, 0);
    if (1 < nkc) stage(buf1, 1);
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc) {
      if (kc < nkc) {
        if (kc + 1 < nkc) wait_vmcnt<C::NSI>(); else wait_vmcnt<0>();
        barrier();
        if (kc + 2 < nkc) {
          if ((kc + 2) % 3 == 0) stage(buf0, kc + 2);
          else if ((kc + 2) % 3 == 1) stage(buf1, kc + 2);
          else stage(buf2, kc + 2);
        }
        if (kc % 3 == 0) gather(buf0, kc);
        else if (kc % 3 == 1) gather(buf1, kc);
        else gather(buf2, kc);
      } else {
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) st.breg[rt][kc] = op_t{};
      }
    }
    wait_lgkm0();
    barrier();   // staging buffers free before tile DMA overwrites them

    // frequencies of this lane's 4 rows and the 16/32-token rotation steps
    if ((l & 15) == 0) {
      f32x4 c4, s4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 16 * jf + 4 * (l >> 4) + e;
        float ce, se;
        sincos_angle(16.0, rope_theta(f), &ce, &se);
        c4[e] = ce;
        s4[e] = se;
      }
      steptab[(w * 4 + (l >> 4)) * 2] = c4;
      steptab[(w * 4 + (l >> 4)) * 2 + 1] = s4;
    }
  }

  // ---------------------------------------------------------------- pipeline
  int b_dma = seq_of(n_begin, 0);
  auto issue_n = [&](uint4* bufp, int n) __attribute__((always_inline)) {
    b_dma = seq_of(n, b_dma);
    issue_tile(bufp, b_dma, (n - tstart[b_dma]) * C::TT, seq_len(b_dma));
  };
  issue_n(buf0, n_begin);
  if (n_begin + 1 < n_end) issue_n(buf1, n_begin + 1);

  st.L = 0;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
#pragma unroll
  for (int i = 0; i < C::NNTW; ++i) st.acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  int bcur = seq_of(n_begin, 0);

  auto step = [&](const uint4* bufp, int n) __attribute__((always_inline)) {
    // Lane-derived offsets are recomputed from an opaque copy of the lane id
    // every tile: cheaper than keeping dozens of hoisted addresses alive in
    // registers across the tile loop.
    int l = lane;
    asm volatile("" : "+v"(l));
    // ---- segment bookkeeping
    bcur = seq_of(n, bcur);
    const int b = bcur;
    const bool seg_start = (n == n_begin) || (n == tstart[b]);
    const bool seg_end = (n == n_end - 1) || (n + 1 == tstart[b + 1]);
    const int t0 = (n - tstart[b]) * C::TT;
    if (seg_start) {
      st.L = seq_len(b);
      const int pos = p.q_pos ? p.q_pos[b] : st.L - 1;
      if constexpr (C::ROPE) {
        const LT* qb = (const LT*)p.q + (int64_t)b * p.H * C::DH;
        float qc[4], qs[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sincos_angle((double)pos, rope_theta(16 * jf + 4 * (l >> 4) + e), &qc[e], &qs[e]);
        if constexpr (C::PPW * C::QPK <= 4) {
          // every lane keeps its rows' rotated query in registers for the segment
#pragma unroll
          for (int x = 0; x < C::PPW; ++x)
#pragma unroll
            for (int qq = 0; qq < C::QPK; ++qq) {
              const int h = (g * C::NG + cbase + x) * C::QPK + qq;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int f = 16 * jf + 4 * (l >> 4) + e;
                float qlo = to_f32(qb[h * C::DH + f]);
                float qhi = to_f32(qb[h * C::DH + f + C::DH / 2]);
                st.qr[(x * C::QPK + qq) * 2][e] = (qlo * qc[e] - qhi * qs[e]) * p.qscale;
                st.qr[(x * C::QPK + qq) * 2 + 1][e] = (qlo * qs[e] + qhi * qc[e]) * p.qscale;
              }
            }
        } else if ((l & 15) == 0) {
          // lanes of one row group share their frequency rows: lane 16*kq writes them
#pragma unroll
          for (int x = 0; x < C::PPW; ++x)
#pragma unroll
            for (int qq = 0; qq < C::QPK; ++qq) {
              const int h = (g * C::NG + cbase + x) * C::QPK + qq;
              f32x4 lo4, hi4;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int f = 16 * jf + 4 * (l >> 4) + e;
                float qlo = to_f32(qb[h * C::DH + f]);
                float qhi = to_f32(qb[h * C::DH + f + C::DH / 2]);
                lo4[e] = (qlo * qc[e] - qhi * qs[e]) * p.qscale;
                hi4[e] = (qlo * qs[e] + qhi * qc[e]) * p.qscale;
              }
              f32x4* qt = qtab + ((w * 4 + (l >> 4)) * C::PPW * C::QPK + x * C::QPK + qq) * 2;
              qt[0] = lo4;
              qt[1] = hi4;
            }
        }
      } else {
        const int kq = l >> 4, row = l & 15;
        const int hq = C::F32 ? row : (row & 7);
        const bool lo_part = !C::F32 && row >= 8;
        const bool valid = hq < C::NQ;
        const float* qa = p.qabs + ((int64_t)b * p.H + g * C::NQ + (valid ? hq : 0)) * p.qabs_stride;
#pragma unroll
        for (int kc = 0; kc < C::NKC; ++kc) {
          op_t v;
          if constexpr (C::F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              int k = kc * C::KC + 4 * kq + e;
              v[e] = (valid && k < rk) ? qa[k] : 0.f;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              int k = kc * C::KC + 8 * kq + e;
              float val = (valid && k < rk) ? qa[k] : 0.f;
              LT hi = from_f32<LT>(val);
              LT lo = from_f32<LT>(val - to_f32(hi));
              v[e] = lo_part ? lo : hi;
            }
          }
          st.aq[kc] = v;
        }
      }
      // The segment's global loads finish here (a pipeline drain once per
      // segment); otherwise the compiler keeps them pending and drains the
      // whole prefetch pipeline at later register reuses in every tile.
      wait_vmcnt<0>();
    }
    if constexpr (C::ROPE) {
      if (seg_start || ((n - n_begin) & 63) == 0) {
        // exact seeding of the angle recurrence at this tile's first token
#pragma unroll
        for (int e = 0; e < 4; ++e) sincos_angle((double)(t0 + (l & 15)), rope_theta(16 * jf + 4 * (l >> 4) + e), &st.cs[e], &st.sn[e]);
      }
    }

    const uint8_t* zkt = (const uint8_t*)bufp;
    const uint8_t* zvt = (const uint8_t*)(bufp + C::SLK);
    const int kq = l >> 4, tl = l & 15;

    // ---- partial scores -> spart[hq][t][slot], one slot per (wave part, row group)
    if constexpr (C::ROPE) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4 cacc[C::RT];
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) cacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int t = 16 * u + tl;
        // All NKC chunks run: rows of B_k past the group's rank are zero in
        // registers and the LDS slots they meet hold finite latent data.
#pragma unroll
        for (int kc = 0; kc < C::NKC; ++kc) {
          const op_t bop = *(const op_t*)(zkt + (t * C::PITK + 4 * kc + kq) * 16);
#pragma unroll
          for (int rt = 0; rt < C::RT; ++rt) cacc[rt] = mma<LT>(st.breg[rt][kc], bop, cacc[rt]);
        }
        // RoPE on the accumulator: lane holds token t, rows f_e of both halves
        float c[4], s[4];
        if (u == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) { c[e] = st.cs[e]; s[e] = st.sn[e]; }
        } else {
          const f32x4 c16 = steptab[(w * 4 + kq) * 2], s16 = steptab[(w * 4 + kq) * 2 + 1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            c[e] = st.cs[e] * c16[e] - st.sn[e] * s16[e];
            s[e] = st.sn[e] * c16[e] + st.cs[e] * s16[e];
          }
        }
#pragma unroll
        for (int x = 0; x < C::PPW; ++x) {
          float klo[4], khi[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float a = cacc[2 * x][e], bb = cacc[2 * x + 1][e];
            klo[e] = a * c[e] - bb * s[e];
            khi[e] = a * s[e] + bb * c[e];
          }
#pragma unroll
          for (int qq = 0; qq < C::QPK; ++qq) {
            f32x4 qlo, qhi;
            if constexpr (C::PPW * C::QPK <= 4) {
              qlo = st.qr[(x * C::QPK + qq) * 2];
              qhi = st.qr[(x * C::QPK + qq) * 2 + 1];
            } else {
              const f32x4* qt = qtab + ((w * 4 + kq) * C::PPW * C::QPK + x * C::QPK + qq) * 2;
              qlo = qt[0];
              qhi = qt[1];
            }
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              part = fmaf(qlo[e], klo[e], part);
              part = fmaf(qhi[e], khi[e], part);
            }
            const int hq = (cbase + x) * C::QPK + qq;
            if constexpr (C::PRESUM) {
              part = rows4_sum(part);   // identical in the four row groups
              spart[(hq * C::TT + t) * C::NPP + jf] = part;
            } else {
              spart[(hq * C::TT + t) * C::NPP + jf * 4 + kq] = part;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // advance the angle recurrence by one tile
      const f32x4 c16 = steptab[(w * 4 + kq) * 2], s16 = steptab[(w * 4 + kq) * 2 + 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // rotation by 32 tokens = the 16-token rotation applied twice
        const float c32 = c16[e] * c16[e] - s16[e] * s16[e];
        const float s32 = 2.f * c16[e] * s16[e];
        float c2 = st.cs[e] * c32 - st.sn[e] * s32;
        float s2 = st.sn[e] * c32 + st.cs[e] * s32;
        st.cs[e] = c2; st.sn[e] = s2;
      }
    } else {
      // absorbed query: wave w sums chunks w, w + NW, ...; C rows are query
      // heads (16-bit: rows 0-7 hi parts, 8-15 lo parts)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4 cacc = f32x4{0.f, 0.f, 0.f, 0.f};
        const int t = 16 * u + tl;
#pragma unroll
        for (int kc = 0; kc < C::NKC; ++kc) {
          if ((kc % C::NW) == w) {   // wave-uniform; chunks past the rank have zero query
            const op_t bop = *(const op_t*)(zkt + (t * C::PITK + 4 * kc + kq) * 16);
            cacc = mma<LT>(st.aq[kc], bop, cacc);
          }
        }
        if constexpr (!C::F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) cacc[e] = halves_sum(cacc[e]);   // hi + lo rows
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int hq = 4 * kq + e;
          const bool wr = C::F32 ? (hq < C::NQ) : (kq < 2 && hq < C::NQ);
          if (wr) spart[(hq * C::TT + t) * C::NPP + w] = cacc[e];
        }
      }
    }
    wait_lgkm0();
    barrier();

    // ---- online softmax, once per tile: wave w < SMW, lane -> (head, token)
    if (w < C::SMW) {
      const int hq = (w * 64 + l) / C::TT, t = (w * 64 + l) % C::TT;
      const bool hvalid = hq < C::NQ;
      float sc = 0.f;
      if (hvalid) {
        const float* sp = spart + (hq * C::TT + t) * C::NPP;
#pragma unroll
        for (int j = 0; j < C::NP / 4; ++j) {
          const f32x4 v = *(const f32x4*)(sp + 4 * j);
          sc += (v[0] + v[1]) + (v[2] + v[3]);
        }
#pragma unroll
        for (int j = (C::NP / 4) * 4; j < C::NP; ++j) sc += sp[j];
      }
      sc = (hvalid && t0 + t < st.L) ? sc : -INFINITY;
      const float tmax = max32(sc);
      const float m_new = hvalid ? fmaxf(st.m_run, tmax) : 0.f;
      const float alpha = hvalid ? __builtin_amdgcn_exp2f(st.m_run - m_new) : 1.f;
      const float pr = hvalid ? __builtin_amdgcn_exp2f(sc - m_new) : 0.f;
      const float psum = sum32(pr);
      st.l_run = st.l_run * alpha + psum;
      st.m_run = m_new;
      if (hvalid) {
        if constexpr (C::F32) {
          ptile_f[hq * C::PTP + t] = pr;
        } else {
          const LT hi = from_f32<LT>(pr);
          const LT lo = from_f32<LT>(pr - to_f32(hi));
          ptile_h[hq * C::PTP + t] = hi;
          ptile_h[(8 + hq) * C::PTP + t] = lo;
        }
        if (t == 0) {
          arow[hq] = alpha;
          if constexpr (!C::F32) arow[8 + hq] = alpha;
          if (seg_end) {
            float* rec = p.rec + ((int64_t)g * (p.P + batch) + pb + b) * p.rec_stride;
            rec[2 * hq] = st.m_run;
            rec[2 * hq + 1] = st.l_run;
          }
        }
      }
      if (seg_end) {
        st.m_run = -INFINITY;
        st.l_run = 0.f;
      }
    }
    wait_lgkm0();
    barrier();

    // ---- acc += P z_v (every wave, its value n-tiles)
    const f32x4 ar = *(const f32x4*)(arow + 4 * kq);
    const int row = l & 15;
    if constexpr (C::F32) {
      float pf[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) pf[x] = ptile_f[row * C::PTP + kq + 4 * x];
#pragma unroll
      for (int i = 0; i < C::NNTW; ++i) {
        const int nt = w + i * C::NW;
        if (nt < nnt) {
          f32x4 a = st.acc[i];
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] *= ar[e];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int tt = kq + 4 * x;
            const int col = 16 * nt + row;
            float zvv = *(const float*)(zvt + tt * C::PITV * 16 + col * 4);
            a = mfma16x16x4(pf[x], zvv, a);
          }
          st.acc[i] = a;
        }
      }
    } else {
      const op_t pop = *(const op_t*)(ptile_h + row * C::PTP + 8 * kq);
      const int s = l & 15;
#pragma unroll
      for (int i = 0; i < C::NNTW; ++i) {
        const int nt = w + i * C::NW;
        if (nt < nnt) {
          f32x4 a = st.acc[i];
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] *= ar[e];
          // rows (tokens) 8kq + s/4 (+4), columns 16 nt + 4 (s%4) .. +3
          const int ta = 8 * kq + (s >> 2), tb = ta + 4;
          const int colb = (16 * nt + 4 * (s & 3)) * 2;
          i16x4 va = ds_read_tr16(zvt + ta * C::PITV * 16 + colb);
          i16x4 vb = ds_read_tr16(zvt + tb * C::PITV * 16 + colb);
          typedef short s8 __attribute__((ext_vector_type(8)));
          s8 both = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
          a = mfma16x16x32(pop, __builtin_bit_cast(op_t, both), a);
          st.acc[i] = a;
        }
      }
    }

    // ---- close the split record at the end of a segment
    if (seg_end) {
      const int k = pb + b;
      float* racc = p.rec + ((int64_t)g * (p.P + batch) + k) * p.rec_stride + 2 * C::NQ;   // wave-uniform
#pragma unroll
      for (int i = 0; i < C::NNTW; ++i) {
        const int nt = w + i * C::NW;
        if (nt < nnt) {
          f32x4 a = st.acc[i];
          if constexpr (!C::F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = halves_sum(a[e]);   // hi + lo rows
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int hrow = 4 * kq + e;
            const bool wr = C::F32 ? (hrow < C::NQ) : (kq < 2 && hrow < C::NQ);
            if (wr) racc[(uint32_t)(hrow * p.rvp + 16 * nt + (l & 15))] = a[e];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < C::NNTW; ++i) st.acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Each step: wait for this wave's DMA of tile n, barrier (everyone's data
  // landed, everyone finished the previous tile), prefetch tile n + 2 into the
  // buffer freed by tile n - 1, then compute tile n.
  for (int n = n_begin; n < n_end; n += 3) {
#pragma unroll
    for (int ph = 0; ph < 3; ++ph) {
      const int nn = n + ph;
      if (nn < n_end) {
        if (nn + 1 < n_end) wait_vmcnt<C::NDMA>(); else wait_vmcnt<0>();
        barrier();
        if (nn + 2 < n_end) {
          if (ph == 0) issue_n(buf2, nn + 2);
          else if (ph == 1) issue_n(buf0, nn + 2);
          else issue_n(buf1, nn + 2);
        }
        if (ph == 0) step(buf0, nn);
        else if (ph == 1) step(buf1, nn);
        else step(buf2, nn);
      }
    }
  }
}

// ------------------------------------------------------------------ absorbed query
// qabs[b][h][k] = qscale * sum_d B_k^g[k][c*DH + d] q[b][h][d]   (k < r_k, else 0)
// A small product per (group g, kv head c): rows of B_k^g (ranks, d
// contiguous) times the queries of kv head c of every sequence (columns
// (b, qq), d contiguous), on MFMA with both operands read as 16-byte runs
// straight from global memory.  One wave per (g, c, 16 ranks, 128 columns):
// its B_k rows are loaded once, then every column tile's operands are
// requested before the first product.
constexpr int kQabsColTiles = 8;   // 16-column tiles per wave

template <class LT, int DH>
__global__ void __launch_bounds__(64) palu_qabs_kernel(const DecodeParams p, int qpk, int ng, int nmt) {
  typedef typename Op<LT>::type op_t;
  constexpr int KC = std::is_same<LT, float>::value ? 16 : 32;   // k per MFMA call
  constexpr int NKS = DH / KC;
  constexpr int EPC = 16 / (int)sizeof(LT);                     // elements per 16-byte run
  const int mt = blockIdx.x % nmt, gc = blockIdx.x / nmt;
  const int g = gc / ng, c = gc % ng;
  const int l = threadIdx.x, s = l & 15, kq = l >> 4;
  const int rk = p.rk[g];
  const int k0 = 16 * mt;
  const int w = ng * DH;
  // A: rank k0 + s, d = KC ks + EPC kq .. (zero rows past the rank)
  const LT* Bg = (const LT*)p.Bk + p.boff_k[g] + c * DH;
  op_t a[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    a[ks] = k0 + s < rk ? *(const op_t*)(Bg + (int64_t)(k0 + s) * w + KC * ks + EPC * kq) : op_t{};
  // B: column n = b * qpk + qq (query head h = (g ng + c) qpk + qq)
  const int ncol = p.batch * qpk;
  const int n0 = blockIdx.y * (16 * kQabsColTiles);
  op_t bq[kQabsColTiles][NKS];
#pragma unroll
  for (int t = 0; t < kQabsColTiles; ++t) {
    const int n = n0 + 16 * t + s;
    const int b = n / qpk, h = (g * ng + c) * qpk + n % qpk;
    const LT* qb = (const LT*)p.q + ((int64_t)b * p.H + h) * DH;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) bq[t][ks] = n < ncol ? *(const op_t*)(qb + KC * ks + EPC * kq) : op_t{};
  }
#pragma unroll
  for (int t = 0; t < kQabsColTiles; ++t) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = mma<LT>(a[ks], bq[t][ks], acc);
    // D lane (s, kq): ranks k0 + 4 kq .. +3 of column n0 + 16 t + s
    const int n = n0 + 16 * t + s;
    if (n < ncol && k0 + 4 * kq < p.qabs_stride) {
      const int b = n / qpk, h = (g * ng + c) * qpk + n % qpk;
      float* out = (float*)p.qabs + ((int64_t)b * p.H + h) * p.qabs_stride + k0 + 4 * kq;
      *(f32x4*)out = acc * p.qscale;
    }
  }
}

// ------------------------------------------------------------------ merge + B_v
// Block = (group g, kv head c of the group, 32 output columns of that head,
// 16 rows of (sequence, query head of kv head c)).  For every row the split
// records of its sequence are combined,
//   m* = max m_i, l* = sum l_i 2^(m_i - m*), a = sum acc_i 2^(m_i - m*) / l*,
// then out[b][h][cols] = a . B_v^g[:, c*DH + cols] (16-bit: MFMA with a split
// into hi + lo parts, one wave per 16 columns; fp32: VALU).  The kernel is
// latency-bound: every phase issues all of a thread's global loads before
// using any of them.
constexpr int kMergeRows = 16;
constexpr int kMergeCols = 32;
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxRank = 320;

template <class LT, int DH>
__global__ void __launch_bounds__(kMergeThreads) palu_merge_kernel(const DecodeParams p, int nq, int qpk, int ng) {
  constexpr bool F32 = std::is_same<LT, float>::value;
  constexpr int NCB = DH / kMergeCols;
  constexpr int NT = kMergeThreads;
  const int g = blockIdx.x / (ng * NCB), c = (blockIdx.x / NCB) % ng, cb = blockIdx.x % NCB;
  const int bpc = kMergeRows / qpk;                  // sequences per block
  const int b0 = blockIdx.y * bpc;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int rv = p.rv[g];
  const int rvk = (rv + 31) / 32 * 32;               // rank padded to whole k-steps
  const int w_grp = ng * DH;
  const int wpitch = p.P + 1;
  // (uint4-typed so that the dynamic region starts 16-byte aligned after the
  // static arrays below: the a rows and the B_v slice take 16-byte accesses)
  extern __shared__ uint4 smem_u4[];
  float* smem = (float*)smem_u4;
  float* wts = smem;                                 // [16][P + 1] record weights
  float* a = wts + kMergeRows * wpitch;              // [16][rvk + 4]
  const int apitch = rvk + 4;
  constexpr int BP = kMergeCols + (F32 ? 4 : 16);    // B_v slice row pitch (elements)
  LT* bs = (LT*)(a + kMergeRows * apitch);           // [rvk][BP]
  float* part = (float*)(bs + rvk * BP);             // [NT][8] partial merges of shared items
  __shared__ int rinfo[kMergeRows][2];               // first record index, record count (0: empty row)
  __shared__ int maxrec;

  // stage B_v^g[:, c*DH + cb*32 .. +32], zero rows past the rank
  {
    const LT* Bv = (const LT*)p.Bv + p.boff_v[g] + c * DH + cb * kMergeCols;
    constexpr int EPC = 16 / sizeof(LT);             // elements per 16-byte chunk
    constexpr int CPRW = kMergeCols / EPC;           // chunks per staged row
    constexpr int SPT = cdiv(kMergeMaxRank * CPRW, NT);
    uint4 v[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int i = tid + NT * k, r = i / CPRW, cc = i - r * CPRW;
      v[k] = make_uint4(0u, 0u, 0u, 0u);
      if (r < rv) v[k] = *(const uint4*)(Bv + (int64_t)r * w_grp + cc * EPC);
    }
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int i = tid + NT * k, r = i / CPRW, cc = i - r * CPRW;
      if (r < rvk) *(uint4*)(bs + r * BP + cc * EPC) = v[k];
    }
  }

  // Record phase.  Many valid rows: per-row record weights
  // 2^(m_i - m*) / l* (16 lanes per row) in LDS, then a[row][r] =
  // sum_i w_i acc_i over 4 consecutive ranks per item, the loads of every
  // item of a record issued together.  At most one valid item per thread
  // (small batches, whose sequences are split over many records): nsub
  // threads share an item, each merging every nsub-th record online (four
  // per round), and their partials are combined through LDS.
  const int rows_valid = min(kMergeRows, (p.batch - b0) * qpk);
  const int niv = rows_valid * (rvk / 4);
  if (niv > NT) {
    // per-row record weights: 16 lanes per row
    const int total = p.hdr[p.batch];
    const int tpb = cdiv(total, p.Pg[g]);
    if (tid == 0) maxrec = 0;
    __syncthreads();
    {
      const int row = tid >> 4, sub = tid & 15;
      const int b = b0 + row / qpk, qq = row % qpk;
      const int hq = c * qpk + qq;
      int nrec = 0, k0 = 0;
      if (b < p.batch) {
        int L = p.seq_lens[b];
        L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
        const int ts = p.hdr[b], te = p.hdr[b + 1];
        if (L > 0 && te > ts) {
          const int p0 = ts / tpb, p1 = (te - 1) / tpb;
          nrec = p1 - p0 + 1;
          k0 = p0 + b;
        }
      }
      const float* recs = p.rec + ((int64_t)g * (p.P + p.batch) + k0) * p.rec_stride;
      float m = -INFINITY;
      for (int i = sub; i < nrec; i += 16) m = fmaxf(m, recs[(int64_t)i * p.rec_stride + 2 * hq]);
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
      float ls = 0.f;
      for (int i = sub; i < nrec; i += 16) {
        const float* rr = recs + (int64_t)i * p.rec_stride;
        const float e = exp2f(rr[2 * hq] - m);
        wts[row * wpitch + i] = e;
        ls = fmaf(rr[2 * hq + 1], e, ls);
      }
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) ls += __shfl_xor(ls, d, 64);
      const float inv = nrec > 0 ? 1.f / ls : 0.f;
      for (int i = sub; i < nrec; i += 16) wts[row * wpitch + i] *= inv;
      if (sub == 0) {
        rinfo[row][0] = k0;
        rinfo[row][1] = nrec;
        atomicMax(&maxrec, nrec);
      }
    }
    __syncthreads();

    // a[row][r] = sum_i w_i acc_i[r]: 4 consecutive ranks per item, consecutive
    // threads on consecutive items; per record all of a thread's loads go out
    // before any is used
    {
      constexpr int IPT = cdiv(kMergeRows * kMergeMaxRank / 4, NT);
      const int rq = rvk / 4;                          // items per row
      const int ni = kMergeRows * rq;
      const int nmax = maxrec;
      f32x4 acc4[IPT];
      const float* base[IPT];
      int nr[IPT];
      int rowi[IPT];
#pragma unroll
      for (int k = 0; k < IPT; ++k) {
        const int q = tid + NT * k;
        const int row = q < ni ? q / rq : 0, r4 = q - row * rq;
        const int qq = row % qpk, hq = c * qpk + qq;
        rowi[k] = row;
        nr[k] = (q < ni && 4 * r4 < rv) ? rinfo[row][1] : 0;
        base[k] = p.rec + ((int64_t)g * (p.P + p.batch) + rinfo[row][0]) * p.rec_stride + 2 * nq + hq * p.rvp + 4 * r4;
        acc4[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      for (int i = 0; i < nmax; ++i) {
        f32x4 v[IPT];
#pragma unroll
        for (int k = 0; k < IPT; ++k)
          v[k] = i < nr[k] ? *(const f32x4*)(base[k] + (int64_t)i * p.rec_stride) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
          const float wi = i < nr[k] ? wts[rowi[k] * wpitch + i] : 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc4[k][e] = fmaf(v[k][e], wi, acc4[k][e]);
        }
      }
#pragma unroll
      for (int k = 0; k < IPT; ++k) {
        const int q = tid + NT * k;
        if (q < ni) {
          const int row = q / rq, r4 = q - row * rq;
          *(f32x4*)(a + row * apitch + 4 * r4) = acc4[k];
        }
      }
    }
  } else {
    const int rq = rvk / 4;                          // items per row
    const int ni = kMergeRows * rq;
    const int total = p.hdr[p.batch];
    const int tpb = cdiv(total, p.Pg[g]);
    int nsub = 1;
    while (nsub < 16 && 2 * nsub * niv <= NT) nsub *= 2;
    // record range of the sequence of item q (nrec = 0: no record, a = 0)
    auto range = [&](int q, int& nrec, const float*& base) __attribute__((always_inline)) {
      const int row = q < ni ? q / rq : 0, r4 = q - row * rq;
      const int b = b0 + row / qpk;
      int k0 = 0;
      nrec = 0;
      if (q < ni && 4 * r4 < rv && b < p.batch) {
        int L = p.seq_lens[b];
        L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
        const int ts = p.hdr[b], te = p.hdr[b + 1];
        if (L > 0 && te > ts) {
          const int p0 = ts / tpb, p1 = (te - 1) / tpb;
          nrec = p1 - p0 + 1;
          k0 = p0 + b;
        }
      }
      // (m, l) of head hq at base[2 hq], accumulator ranks at base[2 nq + hq rvp + 4 r4]
      base = p.rec + ((int64_t)g * (p.P + p.batch) + k0) * p.rec_stride;
    };
    // online merge of one record into (m, l, acc)
    auto fold = [&](float& m, float& ls, f32x4& acc, float2 ml, const f32x4& v) __attribute__((always_inline)) {
      const float mn = fmaxf(m, ml.x);
      const float al = exp2f(m - mn), be = exp2f(ml.x - mn);
      ls = fmaf(ls, al, ml.y * be);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(acc[e], al, v[e] * be);
      m = mn;
    };
    auto store_a = [&](int q, float ls, const f32x4& acc, int nrec) __attribute__((always_inline)) {
      const int row = q / rq, r4 = q - row * rq;
      const float inv = nrec > 0 ? 1.f / ls : 0.f;
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[e] * inv;
      *(f32x4*)(a + row * apitch + 4 * r4) = o;
    };
    // thread tid: item tid % niv, records sub, sub + nsub, ... (four per
    // round; nsub = 1 when the valid items fill the block)
    const int q = tid % niv, sub = tid / niv;
    const bool act = sub < nsub;
    int nrec = 0;
    const float* base;
    range(q, nrec, base);
    const int row = q / rq, r4 = q - row * rq;
    const int hq = c * qpk + row % qpk;
    float m = -INFINITY, ls = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (act) {
      for (int i = sub; i < nrec; i += 4 * nsub) {
        float2 ml[4];
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ii = i + u * nsub;
          const float* rr = base + (int64_t)ii * p.rec_stride;
          const bool ok = ii < nrec;
          ml[u] = ok ? *(const float2*)(rr + 2 * hq) : float2{-INFINITY, 0.f};
          v[u] = ok ? *(const f32x4*)(rr + 2 * nq + hq * p.rvp + 4 * r4) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (i + u * nsub < nrec) fold(m, ls, acc, ml[u], v[u]);
      }
      float* pp = part + 8 * (sub * niv + q);
      pp[0] = m;
      pp[1] = ls;
      *(f32x4*)(pp + 4) = acc;
    }
    __syncthreads();
    if (tid < niv) {
      // combine the nsub partials in subset order (a subset without a
      // record has m = -inf and contributes nothing)
      float mc = -INFINITY, lc = 0.f;
      f32x4 ac = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int u = 0; u < nsub && u < nrec; ++u) {
        const float* pp = part + 8 * (u * niv + tid);
        fold(mc, lc, ac, float2{pp[0], pp[1]}, *(const f32x4*)(pp + 4));
      }
      store_a(tid, lc, ac, nrec);
    }
    // rows past the valid ones are zero
    for (int qq = niv + tid; qq < ni; qq += NT) store_a(qq, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}, 0);
  }
  __syncthreads();

  LT* out = (LT*)p.out;
  if constexpr (F32) {
    for (int o = tid; o < kMergeRows * kMergeCols; o += NT) {
      const int row = o / kMergeCols, d = o - row * kMergeCols;
      const int b = b0 + row / qpk, qq = row % qpk;
      if (b >= p.batch) continue;
      const float* ar = a + row * apitch;
      float sacc = 0.f;
      for (int r = 0; r < rv; ++r) sacc = fmaf(ar[r], to_f32(bs[r * BP + d]), sacc);
      const int h = (g * ng + c) * qpk + qq;
      out[((int64_t)b * p.H + h) * DH + cb * kMergeCols + d] = from_f32<LT>(sacc);
    }
  } else {
    typedef typename Vec8<LT>::type op_t;
    if (w >= kMergeCols / 16) return;                 // one wave per 16 columns
    const int kq = l >> 4, s = l & 15;
    const int nt = w;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < rvk / 32; ++ks) {
      const float* ap = a + s * apitch + 32 * ks + 8 * kq;     // A: row s, k = 8 kq .. +7
      op_t ahi, alo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = ap[e];
        const LT hi = from_f32<LT>(v);
        ahi[e] = hi;
        alo[e] = from_f32<LT>(v - to_f32(hi));
      }
      // B: rows (ranks) 32 ks + 8 kq + s/4 (+4), columns 16 nt + 4 (s%4) .. +3
      const int ra = 32 * ks + 8 * kq + (s >> 2), rb = ra + 4;
      const int col = 16 * nt + 4 * (s & 3);
      i16x4 va = ds_read_tr16(bs + ra * BP + col);
      i16x4 vb = ds_read_tr16(bs + rb * BP + col);
      typedef short s8 __attribute__((ext_vector_type(8)));
      s8 both = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
      const op_t bop = __builtin_bit_cast(op_t, both);
      acc = mfma16x16x32(ahi, bop, acc);
      acc = mfma16x16x32(alo, bop, acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * kq + e;
      const int b = b0 + row / qpk, qq = row % qpk;
      if (b < p.batch) {
        const int h = (g * ng + c) * qpk + qq;
        out[((int64_t)b * p.H + h) * DH + cb * kMergeCols + 16 * nt + s] = from_f32<LT>(acc[e]);
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch
template <class C>
hipError_t launch_cfg(const DecodeParams& p, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (t0 && t1)  // events stamped by the dispatch itself: the kernel's own start and end
    hipExtLaunchKernelGGL(palu_decode_kernel<C>, dim3(p.G * p.P), dim3(C::NT), 0, stream, t0, t1, 0, p);
  else
    hipLaunchKernelGGL(palu_decode_kernel<C>, dim3(p.G * p.P), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

struct Entry {
  DecodeKey key;
  hipError_t (*decode)(const DecodeParams&, hipStream_t, hipEvent_t, hipEvent_t);
};

#define PALU_DEC(LTT, ELT, DH, NG, QPK, NKC, RK, RV, ROPE) \
  Entry{DecodeKey{ELT, DH, NG, QPK, RK, RV, ROPE}, &launch_cfg<DecCfg<LTT, DH, NG, QPK, NKC, RK, RV, ROPE, kDecWaves>>}

static const Entry kEntries[] = {
    // fp32 latents: 16-k chunks (head_dim 64, groups of 4 kv heads)
    PALU_DEC(float, Elt::F32, 64, 4, 1, 8, 128, 128, true),
    PALU_DEC(float, Elt::F32, 64, 4, 1, 8, 128, 128, false),
    // 16-bit latents, head_dim 128, groups of 4 kv heads, MHA
    PALU_DEC(_Float16, Elt::F16, 128, 4, 1, 8, 256, 256, true),
    PALU_DEC(_Float16, Elt::F16, 128, 4, 1, 8, 256, 256, false),
    PALU_DEC(__bf16, Elt::BF16, 128, 4, 1, 8, 256, 256, true),
    PALU_DEC(__bf16, Elt::BF16, 128, 4, 1, 8, 256, 256, false),
    // GQA: groups of 2 kv heads, 4 query heads per kv head, ranks up to 320
    PALU_DEC(__bf16, Elt::BF16, 128, 2, 4, 10, 320, 320, true),
    PALU_DEC(__bf16, Elt::BF16, 128, 2, 4, 10, 320, 320, false),
    PALU_DEC(_Float16, Elt::F16, 128, 2, 4, 10, 320, 320, true),
    PALU_DEC(_Float16, Elt::F16, 128, 2, 4, 10, 320, 320, false),
};

static const Entry* find_entry(const DecodeKey& k) {
  const Entry* best = nullptr;
  for (const Entry& e : kEntries) {
    const DecodeKey& c = e.key;
    if (c.elt != k.elt || c.head_dim != k.head_dim || c.kv_per_group != k.kv_per_group ||
        c.q_per_kv != k.q_per_kv || c.rope != k.rope)
      continue;
    if (c.rk_max < k.rk_max || c.rv_max < k.rv_max) continue;
    if (!best || c.rk_max + c.rv_max < best->key.rk_max + best->key.rv_max) best = &e;
  }
  return best;
}

// 16-bit latents without RoPE that no split-kernel instance covers (ranks
// up to 320 with groups of 4 kv heads) are left to the absorbed-query kernel
// alone (at most 8 query heads per group; the absorbed query and the merge
// take head_dim 64 or 128).
static bool abs_only(const DecodeKey& k) {
  return !k.rope && (k.elt == Elt::F16 || k.elt == Elt::BF16) && k.kv_per_group * k.q_per_kv <= 8 &&
         k.rk_max <= 320 && k.rv_max <= 320 && (k.head_dim == 64 || k.head_dim == 128);
}

bool decode_supported(const DecodeKey& k, int* rk_cap, int* rv_cap) {
  const Entry* e = find_entry(k);
  if (!e) {
    if (!abs_only(k)) return false;
    if (rk_cap) *rk_cap = 320;
    if (rv_cap) *rv_cap = 320;
    return true;
  }
  if (rk_cap) *rk_cap = e->key.rk_max;
  if (rv_cap) *rv_cap = e->key.rv_max;
  return true;
}

hipError_t launch_decode(const DecodeKey& k, const DecodeParams& p, hipStream_t stream, hipEvent_t t0,
                         hipEvent_t t1) {
  if (mha_supported(k, p)) return launch_decode_mha(k, p, stream, t0, t1);
  if (abs_supported(k, p)) return launch_decode_abs(k, p, stream, t0, t1);
  const Entry* e = find_entry(k);
  if (!e) return hipErrorInvalidValue;
  return e->decode(p, stream, t0, t1);
}

template <class LT>
static hipError_t launch_qabs_t(const DecodeKey& k, const DecodeParams& p, hipStream_t stream) {
  // (16-byte f32x4 stores of 4 ranks: the row stride is a multiple of 4)
  if (p.qabs_stride % 4 != 0) return hipErrorInvalidValue;
  const int nmt = (p.qabs_stride + 15) / 16;
  const int ncol = p.batch * k.q_per_kv;
  const dim3 grid(p.G * k.kv_per_group * nmt, (ncol + 16 * kQabsColTiles - 1) / (16 * kQabsColTiles));
  if (k.head_dim == 64)
    hipLaunchKernelGGL((palu_qabs_kernel<LT, 64>), grid, dim3(64), 0, stream, p, k.q_per_kv, k.kv_per_group, nmt);
  else if (k.head_dim == 128)
    hipLaunchKernelGGL((palu_qabs_kernel<LT, 128>), grid, dim3(64), 0, stream, p, k.q_per_kv, k.kv_per_group, nmt);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_qabs(const DecodeKey& k, const DecodeParams& p, hipStream_t stream) {
  switch (k.elt) {
    case Elt::F32: return launch_qabs_t<float>(k, p, stream);
    case Elt::F16: return launch_qabs_t<_Float16>(k, p, stream);
    case Elt::BF16: return launch_qabs_t<__bf16>(k, p, stream);
  }
  return hipErrorInvalidValue;
}

template <class LT>
static hipError_t launch_merge_t(const DecodeKey& k, const DecodeParams& p, hipStream_t stream) {
  const int nq = k.kv_per_group * k.q_per_kv;
  if (kMergeRows % k.q_per_kv != 0) return hipErrorInvalidValue;
  if (k.head_dim != 64 && k.head_dim != 128) return hipErrorInvalidValue;
  // 16-byte record loads: the value part of a record starts at 2 * nq floats
  // and records are nq * (2 + rvp) floats apart (rvp is a multiple of 16)
  if (nq % 2 != 0 || k.rv_max > kMergeMaxRank) return hipErrorInvalidValue;
  const int bpc = kMergeRows / k.q_per_kv;
  const int rvk = (k.rv_max + 31) / 32 * 32;
  const size_t smem = (size_t)kMergeRows * (p.P + 1) * sizeof(float) +
                      (size_t)kMergeRows * (rvk + 4) * sizeof(float) +
                      (size_t)rvk * (kMergeCols + (sizeof(LT) == 4 ? 4 : 16)) * sizeof(LT) +
                      (size_t)kMergeThreads * 8 * sizeof(float);   // partial merges of shared items
  if (smem > 160 * 1024) return hipErrorInvalidValue;
  dim3 grid(p.G * k.kv_per_group * (k.head_dim / kMergeCols), (p.batch + bpc - 1) / bpc);
  auto kern = k.head_dim == 64 ? palu_merge_kernel<LT, 64> : palu_merge_kernel<LT, 128>;
  if (smem > 64 * 1024) {
    // raise the dynamic-LDS limit once per instantiation (to the largest size
    // this kernel can ask for)
    static std::once_flag once64, once128;
    static hipError_t err64 = hipSuccess, err128 = hipSuccess;
    const int lim = 160 * 1024;
    if (k.head_dim == 64)
      std::call_once(once64, [&] { err64 = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lim); });
    else
      std::call_once(once128, [&] { err128 = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lim); });
    const hipError_t e = k.head_dim == 64 ? err64 : err128;
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(kMergeThreads), smem, stream, p, nq, k.q_per_kv, k.kv_per_group);
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeKey& k, const DecodeParams& p, hipStream_t stream) {
  switch (k.elt) {
    case Elt::F32: return launch_merge_t<float>(k, p, stream);
    case Elt::F16: return launch_merge_t<_Float16>(k, p, stream);
    case Elt::BF16: return launch_merge_t<__bf16>(k, p, stream);
  }
  return hipErrorInvalidValue;
}

// Multi-query (chunk) attention as decode over virtual sequences: query i
// of sequence b (v = b q_len + i) sits at position L_b - q_len + i and sees
// the history up to and including it; its latent rows are sequence b's
// (the block-table row of b, or block b of a contiguous cache).
__global__ void __launch_bounds__(256) palu_chunk_expand_kernel(const int* seq_lens, const int* block_table, int batch,
                                                                 int q_len, int max_len, int max_pages, int* vlens,
                                                                 int* vqpos, int* vtable) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= batch * q_len) return;
  const int b = v / q_len, i = v - b * q_len;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  const int pos = L - q_len + i;
  vlens[v] = pos >= 0 ? pos + 1 : 0;
  vqpos[v] = pos >= 0 ? pos : 0;
  for (int k = 0; k < max_pages; ++k)
    vtable[(int64_t)v * max_pages + k] = block_table ? block_table[(int64_t)b * max_pages + k] : b;
}

hipError_t launch_chunk_expand(const int* seq_lens, const int* block_table, int batch, int q_len, int max_len,
                               int max_pages, int* vlens, int* vqpos, int* vtable, hipStream_t stream) {
  const int n = batch * q_len;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(palu_chunk_expand_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream, seq_lens,
                     block_table, batch, q_len, max_len, max_pages, vlens, vqpos, vtable);
  return hipGetLastError();
}

}  // namespace palu
