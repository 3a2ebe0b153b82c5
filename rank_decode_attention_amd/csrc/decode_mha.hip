// Fused decode attention for MHA head-groups on gfx950: two waves per kv head.
//
// Method: PALU page, section "Low-rank projection decomposition" (K = z_k B_k,
// V = z_v B_v) and section "Inference flow" (decode: read the latents,
// rebuild, attend); arXiv 2407.21118v2 abstract (keys rebuilt on the fly,
// RoPE-based attention, fused kernels).  Same results and split records as
// palu_decode_kernel; this kernel covers head-groups of 4 kv heads with one
// query head each, head_dim 128, ranks <= 256, 16-bit latents, RoPE.  It is
// instantiated for 4..8 key chunks of 32 ranks (NKC); ranks that are not a
// multiple of 32 need rows that are zero up to the next multiple (the int4
// expansion writes such rows).
//
// Design (ours):
//  * Block = 8 waves, two per SIMD; wave w owns kv head c = w % 4 and the
//    frequency half w / 4 (32 rotation frequencies, both RoPE halves: 64 of
//    the head's 128 dims).  Its B_k^T rows (64 dims x 32 NKC ranks) stay in
//    AGPRs for the whole block, feeding the MFMA A operand directly.
//  * 32-token tiles stream HBM -> LDS through LDS DMA, two tiles ahead, the
//    four DMA pieces of a wave spread over the MFMA window of a step.  Key
//    rows are XOR-swizzled in 16-byte chunks (conflict-free MFMA operand
//    reads), value rows in 32-byte pairs (conflict-free transposed reads).
//    Key tiles use a ring of 3 buffers, value tiles a ring of 4: the value
//    tile of step n is consumed in step n + 1.
//  * Per step n (one barrier): window A = the key rebuild of tokens 0-15 of
//    tile n on MFMA, with the online softmax of tile n-1 (all four heads in
//    every wave, from the half-head partial scores in LDS, summed in a fixed
//    order so that all waves hold identical P) and the rotation of the next
//    angle table laid between the MFMAs; window B = the rebuild of tokens
//    16-31 with RoPE and the query dot of tokens 0-15 between the MFMAs;
//    then P z_v of tile n-1 on MFMA (P split into hi + lo 16-bit parts, each
//    wave 32 value ranks of all four heads, value tile read transposed), RoPE
//    and the dot of tokens 16-31, and the partial scores go to LDS.
//  * RoPE angles (64 frequencies x 32 positions per tile) are formed once
//    per block into a shared table, one step ahead, by rotating the previous
//    tile's entries by 32 positions (re-seeded exactly in fp64 at every
//    segment start and every 64 tiles).
//  * The running maximum is raised only when a tile's maximum exceeds it by
//    more than 2^8, so the accumulator rescale is rare.
#include "common.h"
#include "decode.h"
#include "int4.h"

#include <hip/hip_ext.h>
#include <type_traits>

namespace palu {
namespace {

template <class LT_, int NKC_, bool Q4_>
struct MhaCfg {
  typedef LT_ LT;
  static constexpr bool Q4 = Q4_;              // int4 codes in HBM, expanded into the LDS tiles
  static constexpr int DH = 128, NH = 4, NW = 8, NT = 512, TT = 32;
  static constexpr int RK = 256, RV = 256;     // rank capacity of an LDS latent row
  static constexpr int NKC = NKC_;             // 32-deep k-chunks of the key rebuild (rank <= 32 NKC)
  static_assert(NKC >= 4 && NKC <= RK / 32, "key chunks");
  static constexpr int NMT = DH / 32;          // 16-row M-tiles per wave (half a head: 4)
  static constexpr int ROWB = RK * 2;          // bytes per LDS latent row (512)
  static constexpr int TILEB = TT * ROWB;      // 16 KB per latent tile
  static constexpr int NDT = TILEB / (16 * NT);   // DMA instructions per wave per latent tile (2)
  static constexpr int NDMA = 2 * NDT;         // per tile step: keys, values (+ a query at segment starts)
  // key / value buffer rings: tiles arrive by LDS DMA two steps ahead, or
  // (int4) are expanded into the ring one step ahead
  static constexpr int NKB = Q4 ? 2 : 3, NVB = Q4 ? 3 : 4;
  static constexpr int NSTG = Q4 ? 2 : 3;      // B_k staging slots
  // B_k^T operands in VGPRs (int4 instances up to 5 key chunks, whose other
  // registers fit beside them) or in AGPRs (everything else)
  static constexpr bool BREG_V = Q4 && NKC <= 5;
  static constexpr int AP = 17;                // angle-table row pitch in 16-byte units (68 floats)
  // int4: per-token scales of a tile's 32-rank chunks, fp32, [slot][row][SCP]
  // (an odd pitch puts the rows that 32 consecutive lanes write, and the 16
  // rows a half-wave reads, on distinct banks)
  static constexpr int SCP = 9;
  static constexpr int NSK = Q4 ? NKB : 1, NSV = Q4 ? NVB : 1;
  static constexpr int STGB = 32 * DH * NH * 2;   // bytes of one staged B_k chunk (32 ranks x 512 columns)
  static_assert(NDT * 16 * NT == TILEB, "tile DMA");
  static_assert(NT / 32 == 16, "one DMA instruction covers 16 rows");
  static_assert(STGB <= NKB * TILEB && (NSTG - 1) * STGB <= NVB * TILEB, "B_k staging");
};

constexpr float kTau = 8.0f;   // lazy-rescale threshold (log2 domain)

// Value-tile swizzle (in 32-byte pairs): a transposed operand read touches
// rows 8 kq + e (e < 4, plus the +4 rows in a second read), half a wave
// covering kq = 0, 1; the pair index is XORed with bits 0, 1 and 3 of the row
// so that those eight rows land in eight distinct 32-byte bank groups.
__device__ __forceinline__ int vswz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }

__device__ __forceinline__ void sincos_turns(double t, double theta_turns, float* c, float* s) {
  double rev = t * theta_turns;
  rev -= rint(rev);
  const float r = (float)rev;
  *c = __builtin_amdgcn_cosf(r);
  *s = __builtin_amdgcn_sinf(r);
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

template <class LT, int NKC, bool Q4, bool PAGED>
__global__ void __launch_bounds__(512, 1) palu_decode_mha_kernel(const DecodeParams p) {
  typedef MhaCfg<LT, NKC, Q4> C;
  typedef typename Vec8<LT>::type op_t;
  typedef short s8 __attribute__((ext_vector_type(8)));
  __shared__ uint4 zkb[C::NKB * C::TILEB / 16];
  __shared__ uint4 zvb[C::NVB * C::TILEB / 16];
  __shared__ f32x4 angc[2 * C::TT * C::AP];       // [table][position][frequency / 4]
  __shared__ f32x4 angs[2 * C::TT * C::AP];
  __shared__ uint4 qst[3][C::NW][16];             // raw query of each wave, one per tile step in flight
  __shared__ float sp[2][C::NH][2][C::TT];        // partial scores [tile parity][head][frequency half][token]
  __shared__ uint4 pst[C::NW][2 * C::NH * C::TT * 2 / 16];   // per wave: P (hi, lo) of the previous tile, [part][head][token]
  __shared__ uint4 pzero[C::TT * 2 / 16];          // zero rows of the P operand
  __shared__ f32x4 sck[C::NSK * C::TT * C::SCP / 4];   // int4: key scales [slot][row][chunk]
  __shared__ f32x4 scv[C::NSV * C::TT * C::SCP / 4];   // int4: value scales [slot][row][chunk]
  __shared__ double theta[C::DH / 2];             // rotation frequencies in turns per token
  __shared__ f32x4 stpc[C::DH / 8], stps[C::DH / 8];   // rotation by 32 tokens per frequency
  __shared__ int wsum[C::NW];
  __shared__ int start_info[2];                   // sequence and first token of the block's first tile

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = w & 3, hf = w >> 2;               // kv head, frequency half
  const int kq = l >> 4, s = l & 15;
  const int g = blockIdx.x % p.G, pb = blockIdx.x / p.G;
  const int batch = p.batch;
  // 16-bit latents: the first B_k chunks and the first tile's keys are
  // requested before the tile prefix sums and the rest of the B_k staging,
  // so that their latency overlaps that work (int4 tiles arrive through
  // registers and keep the plain order)
  constexpr bool EARLY = !C::Q4;
  const int rk = p.rk[g];

  // ---------------------------------------------------------------- B_k^T staging (LDS DMA) and gather into AGPRs
  // M-tile mt = 2j + half: dims half*64 + 32*hf + 16j + (0..15), i.e. rotation
  // frequencies 32*hf + 16j + (0..15) in both RoPE halves
  op_t breg[C::NKC][C::NMT];
  const LT* Bg = (const LT*)p.Bk + p.boff_k[g];   // [rk][4 * DH]
  constexpr int W = C::NH * C::DH;
  constexpr int NSI = C::STGB / (16 * C::NT);     // DMA instructions per wave per staged chunk (4)
  uint8_t* const slots[3] = {(uint8_t*)zkb, (uint8_t*)zvb, (uint8_t*)zvb + C::STGB};
  auto stage = [&](int slot, int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NSI; ++m) {
      const int q = (m * C::NW + w) * 64 + l;     // 16-byte slot of the staged chunk
      // (row R's 16-byte chunk c lands at chunk position c ^ 2 (R & 3): the
      // transposed reads below take 32 bytes from each of 4 consecutive rows
      // of 1 KB, which the swizzle puts on 4 distinct 32-byte bank groups)
      const int row = q >> 6, col = ((q & 63) ^ (2 * (row & 3))) * 8;
      const int kr = min(kc * 32 + row, rk - 1);
      dma16(Bg + (int64_t)kr * W + col, lds_addr(slots[slot]) + 16u * ((m * C::NW + w) * 64));
    }
  };
  auto gather = [&](int slot, int kc) __attribute__((always_inline)) {
    const LT* sb = (const LT*)slots[slot];
#pragma unroll
    for (int mt = 0; mt < C::NMT; ++mt) {
      const int j = mt >> 1, half = mt & 1;
      const int i0 = c * C::DH + half * (C::DH / 2) + 32 * hf + 16 * j;
      // (16-bit latents: the rank is a multiple of 32, every staged row is a
      // real row of B_k; int4: element i is rank 32 kc + 8 kq + i, set to
      // zero past the rank, so that the codes the cache holds there, which
      // the tiles carry unmasked, meet zero rows)
      // (element el of rows 8 kq + s / 4 and 8 kq + 4 + s / 4, in the
      // swizzled chunk positions of the staging)
      const int el = i0 + 4 * (s & 3), pel = (((el >> 3) ^ (2 * (s >> 2))) << 3) | (el & 7);
      const i16x4 lo = ds_read_tr16(sb + (8 * kq + (s >> 2)) * W + pel);
      const i16x4 hi = ds_read_tr16(sb + (8 * kq + 4 + (s >> 2)) * W + pel);
      s8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if constexpr (C::Q4) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (32 * kc + 8 * kq + i >= rk) both[i] = 0;
      }
      // move the operand into the AGPR file once; it stays there
      op_t v = __builtin_bit_cast(op_t, both), av;
      if constexpr (C::BREG_V) av = v; else asm volatile("" : "=a"(av) : "0"(v));
      breg[kc][mt] = av;
    }
  };
  const int nkc = cdiv(rk, 32);

  // ---------------------------------------------------------------- tile prefix sums
  // (no table is kept: block (0, 0) writes the tile starts of every sequence
  // to the workspace header, every block notes where its first tile lies)
  int total;
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
    if constexpr (EARLY) {
      stage(0, 0);
      if (1 < nkc) stage(1, 1);
    }
    // (barriers that leave the B_k DMA in flight: LDS writes only)
    auto sync_lds = [&]() __attribute__((always_inline)) {
      if constexpr (EARLY) {
        asm volatile("" ::: "memory");
        wait_lgkm0();
        barrier();
        asm volatile("" ::: "memory");
      } else {
        __syncthreads();
      }
    };
    int incl = sacc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (l >= d) incl += o;
    }
    if (l == 63) wsum[w] = incl;
    if (tid < C::TT * 2 / 16) pzero[tid] = uint4{0u, 0u, 0u, 0u};
    if (tid < C::DH / 2) {
      const double th = exp2(-(2.0 * tid / C::DH) * log2(p.rope_base)) * 0.15915494309189535;
      theta[tid] = th;
      float cv, sv;
      sincos_turns(32.0, th, &cv, &sv);
      ((float*)stpc)[tid] = cv;
      ((float*)stps)[tid] = sv;
    }
    sync_lds();
    int all = 0, before = 0;
    for (int i = 0; i < C::NW; ++i) {
      all += wsum[i];
      before += i < w ? wsum[i] : 0;
    }
    total = all;
    const int tpb0 = cdiv(total, p.P);
    const int nb0 = pb * tpb0;
    int run = before + incl - sacc;
    const bool hdr = (g == 0 && pb == 0);
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int bb = tid * per + i;
      if (i < per && bb < batch) {
        if (hdr) p.hdr[bb] = run;
        // the sequence holding tile nb0 (non-empty: it owns tiles [run, run + loc))
        if (nb0 >= run && nb0 < run + loc[i]) {
          start_info[0] = bb;
          start_info[1] = (nb0 - run) * C::TT;
        }
      }
      run += loc[i];
    }
    if (hdr && tid == C::NT - 1) p.hdr[batch] = total;
    sync_lds();
  }
  const int tpb = cdiv(total, p.P);
  const int n_begin = pb * tpb;
  const int n_end = min(total, n_begin + tpb);
  if (n_begin >= n_end) {
    if constexpr (EARLY) wait_vmcnt<0>();   // (no LDS DMA outlives the block)
    return;
  }

  const int pk = p.pk[g], pv = p.pv[g];
  const int cprk = pk >> 4, cprv = pv >> 4;
  const uint8_t* zk_seq = p.zk + p.goff_k[g];
  const uint8_t* zv_seq = p.zv + p.goff_v[g];
  // int4 caches: zk / zv hold the codes (16 bytes per 32 ranks, pitch pk / pv),
  // sk / sv the binary16 scales (pitch pk / 8, pv / 8)
  const uint8_t* sk_seq = Q4 ? p.sk + p.soff_k[g] : nullptr;
  const uint8_t* sv_seq = Q4 ? p.sv + p.soff_v[g] : nullptr;
  const int64_t sbk = p.seq_bytes_k, sbv = p.seq_bytes_v;
  const int h = g * C::NH + c;                    // query head of this wave (one per kv head)

  // key ring slot of tile m (16-bit latents: the block's first tile takes
  // slot 2, the one slot the B_k staging leaves free)
  const int koff = EARLY ? (2 - n_begin % C::NKB + C::NKB) % C::NKB : 0;
  auto kslot = [&](int m) __attribute__((always_inline)) { return (m + koff) % C::NKB; };

  // ---------------------------------------------------------------- per-lane constants
  // DMA slots: instruction m of wave w fills 16-byte slots (m*NW + w)*64 + l of
  // a tile = row q >> 5, physical chunk q & 31.  Key rows hold logical chunk
  // (physical ^ (row & 15)), so that the 16 token rows of an MFMA operand
  // read fall in distinct banks; value rows hold logical chunk
  // (physical ^ 2 vswz(row)), so that the 16 rows of a transposed read do.
  // Chunks past a row's data load chunk 0 (finite, and multiplied by zero
  // rows of B_k or ignored by the merge).
  auto dslot = [&](int m, int ln, int& row, int& ck, int& cv) __attribute__((always_inline)) {
    const int q = (m * C::NW + w) * 64 + ln;
    const int pc = q & 31;
    row = q >> 5;
    const int lck = pc ^ (row & 15);
    const int lcv = pc ^ (2 * vswz(row));
    ck = 16 * (lck < cprk ? lck : 0);
    cv = 16 * (lcv < cprv ? lcv : 0);
  };
  // Per-lane indices and LDS addresses are re-derived inside the tile loop
  // from an opaque copy of the thread index, where they are used: kept alive
  // across the loop, a dozen of them would not fit beside the MFMA
  // accumulators, and a spilled one costs a scratch reload whose wait would
  // also drain the tile DMA in flight.
  struct Lane { int t, l, s, kq; };
  auto lane = [&]() __attribute__((always_inline)) {
    int t = tid;
    asm volatile("" : "+v"(t));
    Lane r;
    r.t = t;
    r.l = t & 63;
    r.s = t & 15;
    r.kq = (t >> 4) & 3;
    return r;
  };
  // key operand reads: token row 16u + s, logical chunk 4 kc + kq; chunk quad
  // b4 of the row sits at 64 * (b4 ^ (s >> 2)): one base, XORed per use
  auto kbase_of = [&](const Lane& ln) __attribute__((always_inline)) {
    return ln.s * C::ROWB + 16 * (ln.kq ^ (ln.s & 3)) + 64 * (ln.s >> 2);
  };

  // ---------------------------------------------------------------- tile cursors (wave-uniform)
  // The DMA cursor names tile m of the block's range: sequence b, first
  // token t0 of a history of L tokens (empty sequences hold no tiles), and
  // the HBM addresses of its latent rows.  It runs two tiles ahead of the
  // tile being rebuilt.  The tiles behind it are carried as info words
  // (sequence, valid tokens, segment flags), shifted along each step, so
  // that the per-step scalar work stays small: the scalar unit is shared by
  // all waves of a compute unit, and every wave runs this control.
  constexpr int F_START = 1 << 24, F_END = 1 << 25;
  auto len_of = [&](int b) __attribute__((always_inline)) {
    int L = sload_i32(p.seq_lens + b);
    return L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
  };
  struct DCur { int b, t0, L, st; const uint8_t* kb; const uint8_t* vb; const uint8_t* skb; const uint8_t* svb; };
  // (paged caches: the block is the page holding token t0, rows are counted
  // inside it; a page holds a power of two >= 32 rows, so a tile never
  // straddles two pages)
  auto dma_addr = [&](DCur& d) __attribute__((always_inline)) {
    int blk = d.b, tin = d.t0;
    if constexpr (PAGED) {
      blk = sload_i32(p.block_table + (int64_t)d.b * p.max_pages + (d.t0 >> p.page_shift));
      tin = d.t0 & ((1 << p.page_shift) - 1);
    }
    d.kb = zk_seq + (int64_t)blk * sbk + (int64_t)tin * pk;
    d.vb = zv_seq + (int64_t)blk * sbv + (int64_t)tin * pv;
    if constexpr (C::Q4) {
      d.skb = sk_seq + (int64_t)blk * p.seq_sbytes_k + (int64_t)tin * (pk >> 3);
      d.svb = sv_seq + (int64_t)blk * p.seq_sbytes_v + (int64_t)tin * (pv >> 3);
    }
  };
  DCur cd;
  cd.b = __builtin_amdgcn_readfirstlane(start_info[0]);
  cd.t0 = __builtin_amdgcn_readfirstlane(start_info[1]);
  cd.L = len_of(cd.b);
  cd.st = F_START;   // (the block's first tile starts a segment)
  dma_addr(cd);
  // info word of the cursor's tile: b | valid tokens << 16 | F_START (the
  // first tile of a segment: its query is loaded) | F_END (the last tile of
  // its history: its record is written; the block's last tile, handled by
  // the drain step, is the other segment end)
  auto info_of = [&](const DCur& d) __attribute__((always_inline)) {
    const int rem = d.L - d.t0;
    return d.b | (min(rem, C::TT) << 16) | d.st | (rem <= C::TT ? F_END : 0);
  };
  // to the next tile (only called while there is one in the range)
  auto advance = [&](DCur& d) __attribute__((always_inline)) {
    d.t0 += C::TT;
    d.kb += C::TT * pk;
    d.vb += C::TT * pv;
    if constexpr (C::Q4) {
      d.skb += C::TT * (pk >> 3);
      d.svb += C::TT * (pv >> 3);
    }
    d.st = 0;
    if (d.t0 >= d.L) {
      int b = d.b + 1, L = len_of(b);
      while (L == 0) L = len_of(++b);
      d.b = b;
      d.L = L;
      d.t0 = 0;
      d.st = F_START;
      dma_addr(d);
    } else if (PAGED && (d.t0 & ((1 << p.page_shift) - 1)) == 0) {
      dma_addr(d);   // next page of the same history
    }
  };

  // Tile and value tile m of the DMA cursor into their ring slots: four DMA
  // instructions per wave (keys, values; two each), issued one at a time
  // between the MFMAs of a window so that the eight waves do not queue them
  // all at once.  Instruction i covers rows 16i + (2w + l/32); in the last
  // tile of a history, rows past it repeat its last row.
  struct DmaPlan { const uint8_t* kb; const uint8_t* vb; unsigned kdst, vdst, koff[2], voff[2]; };
  auto dma_plan = [&](const DCur& d, int m, const Lane& ln) __attribute__((always_inline)) {
    DmaPlan q;
    q.kb = d.kb;
    q.vb = d.vb;
    q.kdst = lds_addr(zkb) + (unsigned)(kslot(m) * C::TILEB) + 16u * (w * 64);
    q.vdst = lds_addr(zvb) + (unsigned)((m % C::NVB) * C::TILEB) + 16u * (w * 64);
    const int lim = d.L - 1 - d.t0;
    int row, ck, cv;
    dslot(0, ln.l, row, ck, cv);   // (the swizzles of row + 16 are those of row)
#pragma unroll
    for (int i = 0; i < C::NDT; ++i) {
      const int r = min(row + 16 * i, lim);
      q.koff[i] = (unsigned)(r * pk + ck);
      q.voff[i] = (unsigned)(r * pv + cv);
    }
    return q;
  };
  auto dma_piece = [&](const DmaPlan& q, int i) __attribute__((always_inline)) {
    if (i < C::NDT) dma16s(q.kb, q.koff[i], q.kdst + 16u * (i * C::NW * 64));
    else dma16s(q.vb, q.voff[i - C::NDT], q.vdst + 16u * ((i - C::NDT) * C::NW * 64));
  };
  // the query of a segment's first tile m (256 bytes, lanes 0-15), with its tile
  auto dma_query = [&](const DCur& d, int m, const Lane& ln) __attribute__((always_inline)) {
    const uint8_t* qb = (const uint8_t*)p.q + ((int64_t)d.b * p.H + h) * (C::DH * 2);
    if (ln.l < 16) dma16s(qb, 16u * ln.l, lds_addr(&qst[m % 3][w][0]));
  };
  // ---- int4 tiles: lane tid expands one 32-rank chunk of a tile row, keys
  // for tid < 32 nchk (row tid % 32, chunk tid / 32), values for the next
  // 32 nchv lanes (chunk-major, so that the 8 lanes of an LDS write phase
  // hold 8 rows of one chunk, whose swizzled positions differ).
  // Its 16 bytes of codes and its scale are loaded into registers one step
  // ahead (rows past the history repeat its last row); the expansion writes
  // the chunk's codes, as exact 16-bit integers, in four 16-byte pieces into
  // the tile ring in the swizzled layout the DMA would have produced, and its
  // scale, as fp32, into the ring's scale array (zero on rows past the
  // history).  The scale is applied after the matrix products: to each
  // 32-deep partial of the key rebuild, and to P before P z_v, so the latent
  // code * scale enters the attention exactly.  No code is masked: past the
  // rank the keys' codes meet zero rows of B_k and the values' land in
  // accumulator ranks the merge never reads; on rows past the history the
  // key scale is zero and P is zero.
  const int nchk = pk >> 4, nchv = pv >> 4;
  struct Q4It { int row, ch; bool isv, ok; };
  auto q4_item = [&](const Lane& ln) __attribute__((always_inline)) {
    Q4It it;
    int u = ln.t;
    it.isv = u >= 32 * nchk;
    if (it.isv) u -= 32 * nchk;
    it.row = u & 31;
    it.ch = u >> 5;
    it.ok = !it.isv || u < 32 * nchv;
    return it;
  };
  struct Q4Plan { const uint8_t* kb; const uint8_t* vb; const uint8_t* skb; const uint8_t* svb; int lim; };
  auto q4_plan = [&](const DCur& d) __attribute__((always_inline)) {
    return Q4Plan{d.kb, d.vb, d.skb, d.svb, d.L - 1 - d.t0};
  };
  typedef const __attribute__((address_space(1))) u32x4* gq4;
  typedef const __attribute__((address_space(1))) unsigned short* gs16;
  u32x4 q4c = u32x4{0u, 0u, 0u, 0u};   // this lane's codes and scale of the next tile
  unsigned q4s = 0;
  auto q4_load = [&](const Q4Plan& q, const Lane& ln) __attribute__((always_inline)) {
    const Q4It it = q4_item(ln);
    if (it.ok) {
      const int r = min(it.row, q.lim);
      const int pitch = it.isv ? pv : pk;
      const uint8_t* cb = (it.isv ? q.vb : q.kb) + r * pitch + 16 * it.ch;
      const uint8_t* sb = (it.isv ? q.svb : q.skb) + r * (pitch >> 3) + 2 * it.ch;
      q4c = *(gq4)cb;
      q4s = *(gs16)sb;
    }
  };
  auto q4_expand = [&](int m, int nvalid, const Lane& ln) __attribute__((always_inline)) {
    const Q4It it = q4_item(ln);
    if (!it.ok) return;
    uint8_t* rowp = it.isv ? (uint8_t*)zvb + (m % C::NVB) * C::TILEB + it.row * C::ROWB
                           : (uint8_t*)zkb + (m % C::NKB) * C::TILEB + it.row * C::ROWB;
    const int swz = it.isv ? 2 * vswz(it.row) : (it.row & 15);
    const float sf = it.row < nvalid ? (float)__builtin_bit_cast(_Float16, (unsigned short)q4s) : 0.f;
    float* scrow = it.isv ? (float*)scv + ((m % C::NVB) * C::TT + it.row) * C::SCP
                          : (float*)sck + ((m % C::NKB) * C::TT + it.row) * C::SCP;
    scrow[it.ch] = sf;
    const unsigned cw[4] = {q4c[0], q4c[1], q4c[2], q4c[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(uint4*)(rowp + 16 * ((4 * it.ch + i) ^ swz)) = codes8<LT>(cw[i]);
    }
  };

  auto issue = [&](const DCur& d, int m, int info) __attribute__((always_inline)) {
    const Lane ln = lane();
    if (info & F_START) dma_query(d, m, ln);
    if constexpr (C::Q4) {
      q4_load(q4_plan(d), ln);
    } else {
      const DmaPlan q = dma_plan(d, m, ln);
#pragma unroll
      for (int i = 0; i < 2 * C::NDT; ++i) dma_piece(q, i);
    }
  };

  // Angle table of tile cr.n: entries (position t & 31, frequencies
  // 4 (t >> 5) .. +3) rotated by 32 positions from the same entries of the
  // previous table, or seeded exactly in fp64.
  auto ang_rotate = [&](int m, const Lane& ln) __attribute__((always_inline)) {
    const int e = (ln.t & 31) * C::AP + (ln.t >> 5);
    const f32x4 pc = angc[((m - 1) & 1) * (C::TT * C::AP) + e];
    const f32x4 ps = angs[((m - 1) & 1) * (C::TT * C::AP) + e];
    const f32x4 rc = stpc[ln.t >> 5], rs = stps[ln.t >> 5];
    f32x4 oc, os;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      oc[i] = pc[i] * rc[i] - ps[i] * rs[i];
      os[i] = ps[i] * rc[i] + pc[i] * rs[i];
    }
    angc[(m & 1) * (C::TT * C::AP) + e] = oc;
    angs[(m & 1) * (C::TT * C::AP) + e] = os;
  };
  auto ang_seed = [&](int m, int t0) __attribute__((always_inline)) {
    const Lane ln = lane();
    const int tau = ln.t & 31, f4 = ln.t >> 5;
    const int e = tau * C::AP + f4;
    f32x4 oc, os;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float cv, sv;
      sincos_turns((double)(t0 + tau), theta[4 * f4 + i], &cv, &sv);
      oc[i] = cv;
      os[i] = sv;
    }
    angc[(m & 1) * (C::TT * C::AP) + e] = oc;
    angs[(m & 1) * (C::TT * C::AP) + e] = os;
  };

  // ---------------------------------------------------------------- the first tile's keys, B_k^T into AGPRs
  if constexpr (EARLY) {
    const Lane ln = lane();
    dma_query(cd, n_begin, ln);   // (the block's first tile starts a segment)
    const DmaPlan q = dma_plan(cd, n_begin, ln);
#pragma unroll
    for (int i = 0; i < C::NDT; ++i) dma_piece(q, i);
  }
  {
    if constexpr (!EARLY) {
      stage(0, 0);
      if (1 < nkc) stage(1, 1);
    }
    // requests issued between chunk 1 and chunk 2: the first tile's query and keys
    constexpr int NK = EARLY ? 1 + C::NDT : 0;
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc) {
      if (kc < nkc) {
        // chunk kc is in once at most the requests issued after it are outstanding
        if (kc == 0) {
          if (1 < nkc) wait_vmcnt<NSI + NK>(); else wait_vmcnt<NK>();
        } else if (kc == 1) {
          if (2 < nkc) wait_vmcnt<NK + NSI>(); else wait_vmcnt<NK>();
        } else {
          if (kc + 1 < nkc) wait_vmcnt<NSI>(); else wait_vmcnt<0>();
        }
        barrier();
        if constexpr (C::NSTG == 3) {
          if (kc + 2 < nkc) stage((kc + 2) % 3, kc + 2);
          gather(kc % 3, kc);
        } else {
          // two slots: chunk kc + 2 goes into kc's slot once every wave has read it
          gather(kc % 2, kc);
          if (kc + 2 < nkc) {
            wait_lgkm0();
            barrier();
            stage(kc % 2, kc + 2);
          }
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt) {
          op_t z = op_t{}, az;
          if constexpr (C::BREG_V) az = z; else asm volatile("" : "=a"(az) : "0"(z));
          breg[kc][mt] = az;
        }
      }
    }
    wait_lgkm0();
    barrier();   // staging buffers are free before the tile DMA overwrites them
    if constexpr (C::Q4) {
      // ring rows past a group's ranks are read by the MFMAs but never
      // written by the expansion: they must hold finite values (zeros)
      constexpr int NZ = (C::NKB + C::NVB) * C::TILEB / 16;
      for (int i = tid; i < NZ; i += C::NT) {
        uint4* dst = i < C::NKB * C::TILEB / 16 ? zkb + i : zvb + (i - C::NKB * C::TILEB / 16);
        *dst = uint4{0u, 0u, 0u, 0u};
      }
      // (and the scales of chunks past a group's ranks: zero codes times a
      // zero scale)
      constexpr int NZS = (C::NSK + C::NSV) * C::TT * C::SCP / 4;
      for (int i = tid; i < NZS; i += C::NT) {
        f32x4* dst = i < C::NSK * C::TT * C::SCP / 4 ? sck + i : scv + (i - C::NSK * C::TT * C::SCP / 4);
        *dst = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      wait_lgkm0();
      barrier();
    }
  }

  // ---------------------------------------------------------------- running state
  // Softmax state and the P z_v accumulators cover all four heads in every
  // wave: the softmax lane layout is (head l / 16, tokens l % 16 and
  // 16 + l % 16); the P z_v accumulators hold D[head][rank] of the 16x16 MFMA
  // tiles of ranks 32 w + 16 nt + (0..15), rows 0-3 (lanes 0-15) being the
  // heads.  The softmax denominator is kept as per-lane partial sums, reduced
  // over the head's 16 lanes when a record is written.
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  float m_run = -INFINITY, l_lane = 0.f;
  float qlo[2][4], qhi[2][4];
  uint8_t* const pw = (uint8_t*)&pst[w][0];       // this wave's P (hi, lo) of the previous tile

  // P as a 16-bit (hi, lo) pair for the MFMA: hi + lo carries P to about 2^-17
  auto store_p = [&](const Lane& ln, float p0, float p1) __attribute__((always_inline)) {
    const LT h0 = (LT)p0, h1 = (LT)p1;
    const LT g0 = (LT)(p0 - (float)h0), g1 = (LT)(p1 - (float)h1);
    LT* pt = (LT*)pw + ln.kq * C::TT;
    pt[ln.s] = h0;
    pt[16 + ln.s] = h1;
    pt[C::NH * C::TT + ln.s] = g0;
    pt[C::NH * C::TT + 16 + ln.s] = g1;
  };
  // Online softmax of the previous tile for the four heads.  A head's score
  // is the sum of both half-head partials (fixed order).  The running maximum
  // of a head is raised only when the tile holds a score above it by more
  // than kTau: the common path forms P with the current maximum and flags
  // such lanes; softmax_fix (rare) then raises the maxima, rescales and forms
  // P again.
  // (int4: v0, v1 = the value scales of this wave's 32-rank chunk at the
  // lane's two tokens; P enters P z_v multiplied by them)
  struct Sm { float x0, x1, p0, p1, v0, v1; bool up; };
  auto vscales = [&](int m, Sm& sm, const Lane& ln) __attribute__((always_inline)) {
    const float* sv = (const float*)scv + ((m % C::NVB) * C::TT + ln.s) * C::SCP + w;
    sm.v0 = sv[0];
    sm.v1 = sv[16 * C::SCP];
  };
  auto softmax_fast = [&](int m, int info, Sm& sm, const Lane& ln) __attribute__((always_inline)) {
    const int s = ln.s;
    if constexpr (C::Q4) vscales(m, sm, ln);
    const float* sq = &sp[m & 1][ln.kq][0][0];
    const float x0 = sq[s] + sq[C::TT + s];
    const float x1 = sq[16 + s] + sq[C::TT + 16 + s];
    const int nv = (info >> 16) & 63;              // valid tokens of the tile (1..32)
    sm.x0 = s < nv ? x0 : -INFINITY;
    sm.x1 = 16 + s < nv ? x1 : -INFINITY;
    sm.up = fmaxf(sm.x0, sm.x1) > m_run + kTau;
    sm.p0 = __builtin_amdgcn_exp2f(sm.x0 - m_run);
    sm.p1 = __builtin_amdgcn_exp2f(sm.x1 - m_run);
    if constexpr (C::Q4) store_p(ln, sm.p0 * sm.v0, sm.p1 * sm.v1); else store_p(ln, sm.p0, sm.p1);
  };
  auto softmax_fix = [&](Sm& sm, const Lane& ln) __attribute__((always_inline)) {
    const float tmax = max16(fmaxf(sm.x0, sm.x1));
    const float mnew = tmax > m_run + kTau ? tmax : m_run;
    // (alpha is exactly 1 for a head whose maximum stays; 0 on a segment's first tile)
    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
    m_run = mnew;
    l_lane *= alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ae = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(alpha), 16 * e));
      acc[0][e] *= ae;
      acc[1][e] *= ae;
    }
    sm.p0 = __builtin_amdgcn_exp2f(sm.x0 - mnew);
    sm.p1 = __builtin_amdgcn_exp2f(sm.x1 - mnew);
    if constexpr (C::Q4) store_p(ln, sm.p0 * sm.v0, sm.p1 * sm.v1); else store_p(ln, sm.p0, sm.p1);
  };

  // P z_v of the previous tile on MFMA: A = P (rows 0-3 = heads, rows 4-15
  // zero), B = value tile columns 32 w + 16 nt + (0..15) read transposed.
  auto pv_mfma = [&](const uint8_t* zv, const Lane& ln) __attribute__((always_inline)) {
    const int r = ln.s;
    const uint8_t* ah = r < C::NH ? pw + r * (2 * C::TT) + 16 * ln.kq : (const uint8_t*)pzero + 16 * ln.kq;
    const uint8_t* al = r < C::NH ? ah + C::NH * C::TT * 2 : ah;
    const op_t phi = *(const op_t*)ah;
    const op_t plo = *(const op_t*)al;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      // rows 8 kq + r / 4 (+ 4), ranks 32 w + 16 nt + 4 (r & 3) .. +3: the
      // 32-byte pair 2 w + nt of the row, swizzled
      const int r0 = 8 * ln.kq + (r >> 2);
      const int pair = 2 * w + nt;
      const uint8_t* zb0 = zv + r0 * C::ROWB + 32 * (pair ^ vswz(r0)) + 8 * (r & 3);
      const uint8_t* zb1 = zv + (r0 + 4) * C::ROWB + 32 * (pair ^ vswz(r0 + 4)) + 8 * (r & 3);
      const i16x4 lo = ds_read_tr16(zb0);
      const i16x4 hi = ds_read_tr16(zb1);
      const s8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const op_t bz = __builtin_bit_cast(op_t, both);
      acc[nt] = mfma16x16x32(phi, bz, acc[nt]);
      acc[nt] = mfma16x16x32(plo, bz, acc[nt]);
    }
  };

  auto record_prev = [&](int info) __attribute__((always_inline)) {
    const Lane ln = lane();
    const float lsum = sum16(l_lane);
    float* rec = p.rec + ((int64_t)g * (p.P + batch) + pb + (info & 0xFFFF)) * p.rec_stride;
    if (ln.l < 16) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int e = 0; e < C::NH; ++e) rec[2 * C::NH + e * p.rvp + 32 * w + 16 * nt + ln.s] = acc[nt][e];
    }
    if (w == 0 && ln.s == 0) {
      rec[2 * ln.kq] = m_run;
      rec[2 * ln.kq + 1] = lsum;
    }
    acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_lane = 0.f;
  };

  // RoPE on the rebuilt keys of one 16-token half and the query dot
  auto rope_part = [&](const f32x4 (&kt)[C::NMT], const f32x4 (&cj)[2], const f32x4 (&sj)[2], int j0, int j1,
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

  // segment start: rotate this wave's query to its position, pre-scaled
  auto load_query = [&](int m, int info) __attribute__((always_inline)) {
    const int b = info & 0xFFFF;
    const int pos = p.q_pos ? sload_i32(p.q_pos + b) : len_of(b) - 1;
    const LT* qr = (const LT*)&qst[m % 3][w][0];
    const Lane ln = lane();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 32 * hf + 16 * j + 4 * ln.kq + e;
        float cs, sn;
        sincos_turns((double)pos, theta[f], &cs, &sn);
        const float a = to_f32(qr[f]), bq = to_f32(qr[f + C::DH / 2]);
        qlo[j][e] = (a * cs - bq * sn) * p.qscale;
        qhi[j][e] = (a * sn + bq * cs) * p.qscale;
      }
    }
  };

  // ---------------------------------------------------------------- pipeline
  // Step n: tile n's keys are rebuilt and scored, tile n - 1 goes through
  // the softmax and P z_v, tile n + 1's angle table is formed and tile n + 2
  // is loaded.  One barrier per step.  Within a step: window A = keys of
  // tokens 0-15 on MFMA beside the softmax and the next angle table; window
  // B = keys of tokens 16-31 beside RoPE + dot of tokens 0-15; then P z_v on
  // MFMA beside RoPE + dot of tokens 16-31.
  // tiles n_begin and n_begin + 1 (info words of the current and next tile)
  int i_c = info_of(cd), i_a = 0, i_p = 0, t0_a = 0;
  if constexpr (EARLY) {
    // its query and keys are in (waited for with the last B_k chunk, or
    // here); its values go out now
    wait_vmcnt<0>();
    const Lane ln = lane();
    const DmaPlan q = dma_plan(cd, n_begin, ln);
#pragma unroll
    for (int i = C::NDT; i < 2 * C::NDT; ++i) dma_piece(q, i);
  } else {
    issue(cd, n_begin, i_c);
  }
  if constexpr (C::Q4) q4_expand(n_begin, (i_c >> 16) & 63, lane());   // (waits for its loads)
  ang_seed(n_begin, cd.t0);
  if (n_begin + 1 < n_end) {
    advance(cd);
    i_a = info_of(cd);
    t0_a = cd.t0;
    issue(cd, n_begin + 1, i_a);
    if (n_begin + 2 < n_end) advance(cd);
  }

  // lane indices of the tile loop (the addresses derived from them stay in
  // registers across it)
  const Lane lnk = {tid, l, s, kq};
  // (ALL2: tile n + 2 exists, known at compile time in the steady state)
  auto step = [&](int n, auto have_t, auto had_t, auto all2_t) __attribute__((always_inline)) {
    constexpr bool HAVE = decltype(have_t)::value, HAD = decltype(had_t)::value, ALL2 = decltype(all2_t)::value;
    if constexpr (C::Q4) {
      wait_vmcnt<0>();   // the query of tile n; this lane's chunk of tile n + 1
      wait_lgkm0();      // the expansion of tile n (last step) is in LDS
    } else if (HAVE) {
      // (16-bit latents, the first of several steps: its tile's query and keys
      // were waited for before its values were requested, and the values are
      // used one step later)
      if (n + 1 >= n_end) wait_vmcnt<0>();
      else if (HAD || !EARLY) wait_vmcnt<C::NDMA>();
    }
    barrier();   // tile n, angle table n and the partial scores of tile n - 1 are visible
    // tile n + 1 (if any) gets an exact angle table at a segment start and
    // every 64 tiles
    const bool seed = n + 1 < n_end && ((i_a & F_START) || ((n + 1 - n_begin) & 63) == 0);
    if (HAVE && (i_c & F_START)) load_query(n, i_c);
    const Lane ln = lnk;
    // int4: tile n + 1 into its ring slots (its slots held tiles n - 1 and
    // n - 2, consumed before this step's barrier)
    if constexpr (C::Q4) {
      if (n + 1 < n_end) q4_expand(n + 1, (i_a >> 16) & 63, ln);
    }
    // tile n + 2: its DMA instructions go out between the MFMAs of window A
    // (where there is no window A, here); a waiting count of NDMA at the next
    // step stays safe with a query load in front of them
    const bool load2 = ALL2 || n + 2 < n_end;
    DmaPlan dq;
    Q4Plan q4p;
    int i_d = 0, t0_d = 0;
    if (load2) {
      i_d = info_of(cd);
      t0_d = cd.t0;
      if (i_d & F_START) dma_query(cd, n + 2, ln);
      if constexpr (C::Q4) q4p = q4_plan(cd); else dq = dma_plan(cd, n + 2, ln);
      if (n + 3 < n_end) advance(cd);   // (the cursor never walks past the range)
      if (!HAVE) {
        if constexpr (C::Q4) {
          q4_load(q4p, ln);
        } else {
#pragma unroll
          for (int i = 0; i < 2 * C::NDT; ++i) dma_piece(dq, i);
        }
      }
    }
    Sm sm;
    f32x4 k0[C::NMT], k1[C::NMT];
    float part0 = 0.f;    // int4: partial score of tokens 0-15 (window A)
    // int4: the key of token t is sum_c s_c(t) T_c(t), T_c the 32-deep MFMA
    // partial of chunk c over the integer codes.  RoPE and the query dot are
    // linear in the key, so the query is rotated back to the token instead,
    // u = R(t)^T q (per lane: its eight frequency pairs), each partial T_c is
    // dotted with u as soon as it is ready, and the dot is scaled by s_c(t):
    // no key is held, and code * scale enters exactly.
    f32x4 kt[C::NMT];
    float ks[2];          // scales of chunks kc - 1 and kc at this lane's token
    f32x4 qu[C::NMT];     // rotated query: M-tile 2j pairs with 2j + 1
    const float* ksrow = (const float*)sck + (n % C::NKB) * C::TT * C::SCP + ln.s * C::SCP;
    auto qrot = [&](const f32x4 (&cj)[2], const f32x4 (&sj)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float cv = cj[j][e], sv = sj[j][e];
          qu[2 * j][e] = fmaf(qlo[j][e], cv, qhi[j][e] * sv);
          qu[2 * j + 1][e] = fmaf(qhi[j][e], cv, -(qlo[j][e] * sv));
        }
    };
    // the dot of chunk kc's partial (M-tile mt) with the rotated query; after
    // the last M-tile of a chunk, scaled into the half-tile's partial score
    float dc = 0.f;
    auto kdot = [&](float& part, int kc, int mt) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dc = fmaf(qu[mt][e], kt[mt][e], dc);
      if (mt == C::NMT - 1) {
        part = kc == 0 ? ks[0] * dc : fmaf(ks[kc & 1], dc, part);
        dc = 0.f;
      }
    };
    // The partials' MFMAs do not depend on each other: an empty asm that
    // takes the running dot and hands on the next MFMA's B_k operand keeps
    // each MFMA after the dot of the partial whose registers it reuses (else
    // they are all issued first and their results pile up in registers).
    auto kord = [&](int kc, int mt, float part) __attribute__((always_inline)) {
      if constexpr (C::BREG_V)
        asm volatile("" : "+v"(breg[kc][mt]) : "v"(dc), "v"(part));
      else
        asm volatile("" : "+a"(breg[kc][mt]) : "v"(dc), "v"(part));
    };
    const uint8_t* zk = (const uint8_t*)zkb + kslot(n) * C::TILEB;
    const int kbase = kbase_of(ln);
    // key operand of chunk kc of token half u (read two chunks ahead)
    auto bload = [&](int u, int kc) __attribute__((always_inline)) {
      return *(const op_t*)(zk + (kbase ^ (64 * (kc & 3))) + 256 * (kc >> 2) + u * 16 * C::ROWB);
    };
    // angle entries of this lane's token, frequency quads 8 hf + kq + 4 j
    const f32x4* tc = angc + (n & 1) * (C::TT * C::AP) + ln.s * C::AP + 8 * hf + ln.kq;
    const f32x4* ts = angs + (n & 1) * (C::TT * C::AP) + ln.s * C::AP + 8 * hf + ln.kq;
    f32x4 ca0[2], sa0[2], ca1[2], sa1[2];
    // The windows are laid out by hand: after every MFMA a small, fixed
    // piece of the other work, with scheduling fences between the pieces so
    // that the VALU and LDS work stays spread between the MFMAs of its wave.
    if (HAVE) {
      // window A: keys of tokens 0-15 beside the softmax of the previous tile
      // and the angle table of the next one
      float ra0, rb0, ra1, rb1, ps0, ps1;
      f32x4 apc, aps, arc, ars, oc, os;
      LT h0, h1, g0, g1;
      const float* sq = &sp[(n - 1) & 1][ln.kq][0][0];
      const int nv = (i_p >> 16) & 63;                 // valid tokens of the previous tile
      const int ae = (ln.t & 31) * C::AP + (ln.t >> 5);
      LT* pt = (LT*)pw + ln.kq * C::TT;
      auto work = [&](int slot) __attribute__((always_inline)) {
        if (HAD) {
          if (slot == 0) {
            ra0 = sq[ln.s];
            rb0 = sq[C::TT + ln.s];
            ra1 = sq[16 + ln.s];
            rb1 = sq[C::TT + 16 + ln.s];
          }
          if constexpr (C::Q4) {
            if (slot == 2) vscales(n - 1, sm, ln);
          }
          if (slot == 8) { sm.x0 = ra0 + rb0; sm.x1 = ra1 + rb1; }
          if (slot == 9) {
            sm.x0 = ln.s < nv ? sm.x0 : -INFINITY;
            sm.x1 = 16 + ln.s < nv ? sm.x1 : -INFINITY;
          }
          if (slot == 10) sm.up = fmaxf(sm.x0, sm.x1) > m_run + kTau;
          if (slot == 11) sm.p0 = __builtin_amdgcn_exp2f(sm.x0 - m_run);
          if (slot == 12) sm.p1 = __builtin_amdgcn_exp2f(sm.x1 - m_run);
          if (slot == 13) {
            if constexpr (C::Q4) {
              ps0 = sm.p0 * sm.v0;
              ps1 = sm.p1 * sm.v1;
            } else {
              ps0 = sm.p0;
              ps1 = sm.p1;
            }
            h0 = (LT)ps0;
            h1 = (LT)ps1;
          }
          if (slot == 14) g0 = (LT)(ps0 - (float)h0);
          if (slot == 15) g1 = (LT)(ps1 - (float)h1);
          if (slot == 16) {
            pt[ln.s] = h0;
            pt[16 + ln.s] = h1;
            pt[C::NH * C::TT + ln.s] = g0;
            pt[C::NH * C::TT + 16 + ln.s] = g1;
          }
        }
        // angle table of tile n + 1 by rotation (where that tile is seeded or
        // does not exist, the seed overwrites these entries or nobody reads
        // them: table (n + 1) & 1 is not read in this step)
        if (slot == 1) {
          apc = angc[(n & 1) * (C::TT * C::AP) + ae];
          aps = angs[(n & 1) * (C::TT * C::AP) + ae];
          arc = stpc[ln.t >> 5];
          ars = stps[ln.t >> 5];
        }
        if (slot >= 18 && slot < 22) {
          const int i = slot - 18;
          oc[i] = apc[i] * arc[i] - aps[i] * ars[i];
          os[i] = aps[i] * arc[i] + apc[i] * ars[i];
        }
        if (slot == 22) {
          angc[((n + 1) & 1) * (C::TT * C::AP) + ae] = oc;
          angs[((n + 1) & 1) * (C::TT * C::AP) + ae] = os;
        }
        if constexpr (C::Q4) {
          if (slot == 3 && load2) q4_load(q4p, ln);
        } else {
          if (slot % 6 == 3 && slot / 6 < 2 * C::NDT && load2) dma_piece(dq, slot / 6);
        }
        // angles of tokens 0-15 for window B (int4: of tokens 16-31, window
        // A took its own before the chunks)
        if constexpr (C::Q4) {
          if (slot == 24) ca1[0] = tc[16 * C::AP];
          if (slot == 25) sa1[0] = ts[16 * C::AP];
          if (slot == 26) ca1[1] = tc[16 * C::AP + 4];
          if (slot == 27) sa1[1] = ts[16 * C::AP + 4];
        } else {
          if (slot == 24) ca0[0] = tc[0];
          if (slot == 25) sa0[0] = ts[0];
          if (slot == 26) ca0[1] = tc[4];
          if (slot == 27) sa0[1] = ts[4];
        }
      };
      op_t bq[3];
      bq[0] = bload(0, 0);
      bq[1] = bload(0, 1);
      if constexpr (C::Q4) {
        ca0[0] = tc[0];
        sa0[0] = ts[0];
        ca0[1] = tc[4];
        sa0[1] = ts[4];
        qrot(ca0, sa0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) {
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt) {
          if constexpr (C::Q4) {
            if (kc > 0) kdot(part0, kc - 1, mt);
            kord(kc, mt, part0);
            kt[mt] = mfma16x16x32(breg[kc][mt], bq[kc % 3], f32x4{0.f, 0.f, 0.f, 0.f});
            if (mt == 0) ks[kc & 1] = ksrow[0 * C::SCP + kc];
          } else {
            k0[mt] = mfma16x16x32(breg[kc][mt], bq[kc % 3], kc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : k0[mt]);
          }
          if (mt == 0 && kc + 2 < C::NKC) bq[(kc + 2) % 3] = bload(0, kc + 2);
          work(4 * kc + mt);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // (ranks below 256: the pieces laid out for chunks NKC..7 follow)
#pragma unroll
      for (int slot = 4 * C::NKC; slot < 32; ++slot) work(slot);
      if constexpr (C::Q4) {
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt) kdot(part0, C::NKC - 1, mt);
      }
    } else if (HAD) {
      softmax_fast(n - 1, i_p, sm, ln);
    }
    if (HAD) {
      if (__builtin_amdgcn_ballot_w64(sm.up)) softmax_fix(sm, ln);
      l_lane += sm.p0 + sm.p1;
    }
    if (HAVE) {
      // window B: keys of tokens 16-31 beside RoPE + dot of tokens 0-15
      // (int4: tokens 0-15 were scored in window A; the query is rotated to
      // tokens 16-31 and their chunk partials are scored here)
      float part = 0.f;
      float klo, khi;
      op_t bq[3];
      bq[0] = bload(1, 0);
      bq[1] = bload(1, 1);
      if constexpr (C::Q4) qrot(ca1, sa1);
      // piece (kc, mt): RoPE and query dot of rotation pair kc of tokens
      // 0-15 (eight pairs per lane), and the angles of tokens 16-31
      auto wb = [&](int kc, int mt) __attribute__((always_inline)) {
        const int j = kc >> 2, e = kc & 3;
        if constexpr (!C::Q4) {
          const float ka = k0[2 * j][e], kb = k0[2 * j + 1][e];
          if (mt == 0) klo = ka * ca0[j][e] - kb * sa0[j][e];
          if (mt == 1) khi = ka * sa0[j][e] + kb * ca0[j][e];
          if (mt == 2) part = fmaf(qhi[j][e], khi, fmaf(qlo[j][e], klo, part));
        }
        if (!C::Q4 && mt == 3 && kc >= 4) {
          if (kc == 4) ca1[0] = tc[16 * C::AP];
          if (kc == 5) sa1[0] = ts[16 * C::AP];
          if (kc == 6) ca1[1] = tc[16 * C::AP + 4];
          if (kc == 7) sa1[1] = ts[16 * C::AP + 4];
        }
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) {
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt) {
          if constexpr (C::Q4) {
            if (kc > 0) kdot(part, kc - 1, mt);
            kord(kc, mt, part);
            kt[mt] = mfma16x16x32(breg[kc][mt], bq[kc % 3], f32x4{0.f, 0.f, 0.f, 0.f});
            if (mt == 0) ks[kc & 1] = ksrow[16 * C::SCP + kc];
          } else {
            k1[mt] = mfma16x16x32(breg[kc][mt], bq[kc % 3], kc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : k1[mt]);
          }
          wb(kc, mt);
          if (mt == 3 && kc + 2 < C::NKC) bq[(kc + 2) % 3] = bload(1, kc + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int kc = C::NKC; kc < 8; ++kc) {
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt) wb(kc, mt);
      }
      float sc0, sc1;
      if constexpr (C::Q4) {
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt) kdot(part, C::NKC - 1, mt);
        sc0 = rows4_sum(part0);
        if (HAD) pv_mfma((const uint8_t*)zvb + ((n - 1) % C::NVB) * C::TILEB, ln);
        sc1 = rows4_sum(part);
      } else {
        sc0 = rows4_sum(part);
        if (HAD) pv_mfma((const uint8_t*)zvb + ((n - 1) % C::NVB) * C::TILEB, ln);
        sc1 = rows4_sum(rope_part(k1, ca1, sa1, 0, 2, 0.f));
      }
      if (ln.kq == 0) {
        sp[n & 1][c][hf][ln.s] = sc0;
        sp[n & 1][c][hf][16 + ln.s] = sc1;
      }
    } else if (HAD) {
      pv_mfma((const uint8_t*)zvb + ((n - 1) % C::NVB) * C::TILEB, ln);
    }
    if (HAD && (!HAVE || (i_p & F_END))) record_prev(i_p);
    if (seed) ang_seed(n + 1, t0_a);
    i_p = i_c;
    i_c = i_a;
    i_a = i_d;
    t0_a = t0_d;
  };

  const std::true_type yes{};
  const std::false_type no{};
  step(n_begin, yes, no, no);
  int n = n_begin + 1;
  for (; n + 2 < n_end; ++n) step(n, yes, yes, yes);
  for (; n < n_end; ++n) step(n, yes, yes, no);
  step(n_end, no, yes, no);
}

bool mha_supported(const DecodeKey& k, const DecodeParams& p) {
  if (!((k.elt == Elt::F16 || k.elt == Elt::BF16) && k.head_dim == 128 && k.kv_per_group == 4 &&
        k.q_per_kv == 1 && k.rope && k.rk_max <= 256 && k.rv_max <= 256))
    return false;
  // B_k is staged in whole 32-row chunks: rows past the rank (the last row
  // repeated) must meet zero latents (int4 tiles are expanded that way)
  for (int j = 0; j < p.G; ++j)
    if (p.rk[j] % 32 != 0 && !p.zero_padded && !p.q4) return false;
  if (p.q4)
    for (int j = 0; j < p.G; ++j)
      if (p.pk[j] != 16 * ((p.rk[j] + 31) / 32) || p.pv[j] != 16 * ((p.rv[j] + 31) / 32)) return false;
  return p.rvp >= 256;                     // every wave writes its 32 value ranks of the record
}

template <class LT, int NKC, bool Q4, bool PAGED>
static void launch_mha_qp(const DecodeParams& p, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const dim3 grid(p.G * p.P), block(512);
  if (t0 && t1)
    hipExtLaunchKernelGGL((palu_decode_mha_kernel<LT, NKC, Q4, PAGED>), grid, block, 0, stream, t0, t1, 0, p);
  else
    hipLaunchKernelGGL((palu_decode_mha_kernel<LT, NKC, Q4, PAGED>), grid, block, 0, stream, p);
}

template <class LT, int NKC, bool Q4>
static void launch_mha_q(const DecodeParams& p, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (p.block_table)
    launch_mha_qp<LT, NKC, Q4, true>(p, stream, t0, t1);
  else
    launch_mha_qp<LT, NKC, Q4, false>(p, stream, t0, t1);
}

template <class LT, int NKC>
static void launch_mha_inst(const DecodeParams& p, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (p.q4)
    launch_mha_q<LT, NKC, true>(p, stream, t0, t1);
  else
    launch_mha_q<LT, NKC, false>(p, stream, t0, t1);
}

template <class LT>
static void launch_mha_t(int nkc, const DecodeParams& p, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  switch (nkc) {
    case 4: launch_mha_inst<LT, 4>(p, stream, t0, t1); break;
    case 5: launch_mha_inst<LT, 5>(p, stream, t0, t1); break;
    case 6: launch_mha_inst<LT, 6>(p, stream, t0, t1); break;
    case 7: launch_mha_inst<LT, 7>(p, stream, t0, t1); break;
    default: launch_mha_inst<LT, 8>(p, stream, t0, t1); break;
  }
}

hipError_t launch_decode_mha(const DecodeKey& k, const DecodeParams& p, hipStream_t stream, hipEvent_t t0,
                             hipEvent_t t1) {
  // the instance with the fewest 32-deep key chunks that covers every rank
  // (at least 4)
  int nkc = (k.rk_max + 31) / 32;
  nkc = nkc < 4 ? 4 : nkc;
  if (nkc > 8) return hipErrorInvalidValue;
  if (k.elt == Elt::F16)
    launch_mha_t<_Float16>(nkc, p, stream, t0, t1);
  else
    launch_mha_t<__bf16>(nkc, p, stream, t0, t1);
  return hipGetLastError();
}

}  // namespace palu
