// Decode attention without RoPE on gfx950: scores from the absorbed query.
//
// Method: PALU page, section "Low-rank projection decomposition" (K = z_k B_k,
// V = z_v B_v) and section "Inference flow" (decode reads the latents);
// arXiv 2407.21118v2 abstract (fused low-rank attention).  Without RoPE the
// score of query head h against token t is q_h . (z_k[t] B_k^c) =
// (q_h B_k^cT) . z_k[t]: the absorbed query (palu_qabs_kernel, pre-scaled,
// r_k values per head) meets the latent rows directly, keys are never
// rebuilt, and the values accumulate as P z_v in latent space (the merge
// kernel applies B_v).  Nothing here depends on head_dim.
//
// Design (ours):
//  * Block = 8 waves; block (g, p) takes the p-th equal share of the 32-token
//    tiles of group g (the split records of palu_decode_kernel), with one
//    barrier per tile.  Each group's blocks form one range of block ids, as
//    many as the host gives it (in proportion to its time per tile, so that
//    groups of mixed ranks end together).
//  * Key and value rows of a tile stream HBM -> LDS through LDS DMA into a
//    ring of three buffers, two tiles ahead.  Rows are padded (key rows 4
//    banks apart, value rows 8) so that the MFMA operand reads and the
//    transposed value reads are bank-conflict-free.
//  * Waves 0-3 take tokens 0-15 of every tile, waves 4-7 tokens 16-31; each
//    wave runs its own online softmax over its half, so no wave waits for
//    another's scores.  Scores S^T = Z_k Q^T on MFMA (A = the 16 token rows,
//    B = the absorbed query of up to 8 heads split into hi + lo 16-bit
//    rows); after adding the hi and lo rows, lane l holds head row l % 16 at
//    tokens 4q + i (q = l / 16, i < 4), which with P rounded to hi (rows 0-7)
//    and lo (rows 8-15) parts is the A operand of a 16-deep value MFMA.
//  * Online softmax in registers, log2 domain; the running maximum is raised
//    only when a score exceeds it by more than 2^8, so rescales are rare.
//  * acc += P z_v on MFMA; wave w owns the value n-tiles w % 4 + 4 i of its
//    half.  Where a split record is written the two halves meet in LDS.
#include "common.h"
#include "decode.h"

#include <hip/hip_ext.h>
#include <type_traits>

namespace palu {
namespace {

template <class LT_, int RCAP_>
struct AbsCfg {
  typedef LT_ LT;
  static constexpr int NW = 8, NT = 512, TT = 32;
  static constexpr int NB = 3;                          // ring buffers (tiles n, n + 1, n + 2)
  static constexpr int RCAP = RCAP_;                    // rank capacity of an LDS row
  static constexpr int NKC = RCAP / 32;                 // 32-deep chunks of the score contraction
  static constexpr int CPR = RCAP / 8;                  // 16-byte chunks of a row at capacity
  static constexpr int PITK = cdiv(CPR, 8) * 8 + 1;     // key row pitch in 16-byte slots
  static constexpr int PITV = cdiv(CPR, 8) * 8 + 2;     // value row pitch
  static constexpr int SLK = cdiv(TT * PITK, 64) * 64;  // 16-byte slots of the key region
  static constexpr int SLV = cdiv(TT * PITV, 64) * 64;
  static constexpr int NIK = cdiv(SLK, 64 * NW), NIV = cdiv(SLV, 64 * NW);
  static constexpr int NDMA = NIK + NIV;                // DMA instructions per wave per tile
  // DMA instructions of waves past a region's end land in the pad (never read)
  static constexpr int PADS = 64;
  static constexpr int BUFB = (SLK + SLV + PADS) * 16;
  static constexpr int NNT4 = cdiv(RCAP / 16, 4);       // value n-tiles per wave (four waves per half)
  static constexpr int XB = 4 * NNT4 * 64 * 16 + 4 * 2 * 16 * 4;   // segment-end exchange
  static_assert(RCAP % 64 == 0, "rank capacity");
  static_assert(NB * BUFB + XB + 64 <= 160 * 1024, "LDS");
};

constexpr float kAbsTau = 8.0f;       // lazy-rescale threshold (log2 domain)
constexpr float kAbsFloor = -1e30f;   // starting running maximum (below any score)

template <class LT> struct Vec4;
template <> struct Vec4<_Float16> { typedef _Float16 type __attribute__((ext_vector_type(4))); };
template <> struct Vec4<__bf16> { typedef short type __attribute__((ext_vector_type(4))); };

// 16x16x16 MFMA (A: lane l holds row l % 16, k = 4 (l / 16) .. +3)
__device__ __forceinline__ f32x4 mfma16x16x16(Vec4<_Float16>::type a, Vec4<_Float16>::type b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(Vec4<__bf16>::type a, Vec4<__bf16>::type b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 16-byte global -> LDS copy from a wave-uniform base plus a per-lane 32-bit
// byte offset; lane l lands at LDS byte `lds_wave_base` + 16*l.
__device__ __forceinline__ void dma16o(const void* base, unsigned voff, unsigned lds_wave_base) {
  const uint64_t a = (uint64_t)base;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  const unsigned lds = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sb)
               : "memory", "m0");
}

// f(integral_constant<N>) for the smallest N in [N0, MAX] with n <= N (MAX if
// none): a wave-uniform choice between fully unrolled, branch-free bodies.
template <int N0, int MAX, class F>
__device__ __forceinline__ void with_count(int n, F&& f) {
  if constexpr (N0 >= MAX) {
    f(std::integral_constant<int, MAX>{});
  } else {
    if (n <= N0) f(std::integral_constant<int, N0>{});
    else with_count<N0 + 1, MAX>(n, f);
  }
}

// x + the value of lane (l + 8) mod 16 of the same 16-lane row (DPP row_ror:8)
__device__ __forceinline__ float add_ror8(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

}  // namespace

template <class LT, int RCAP, bool PAGED>
__global__ void __launch_bounds__(512, 1) palu_decode_abs_kernel(const DecodeParams p, int nq) {
  typedef AbsCfg<LT, RCAP> C;
  typedef typename Vec8<LT>::type op_t;
  typedef typename Vec4<LT>::type op4_t;
  typedef LT lt4_t __attribute__((ext_vector_type(4)));
  __shared__ uint4 ring[C::NB][C::BUFB / 16];
  __shared__ f32x4 xacc[4][C::NNT4 * 64];   // segment end: value accumulators of half 1
  __shared__ float xml[4][2][16];           // and its maxima and denominators
  __shared__ int wsum[C::NW];
  __shared__ int start_info[2];   // sequence and first token of the block's first tile

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = l & 15, q = l >> 4;
  // block -> (group g, share pb): each group's blocks form one range of
  // block ids, as many as its share of the latent bytes
  int g = 0;
  for (int j = 1; j < p.G; ++j) g = (int)blockIdx.x >= p.gblk[j] ? j : g;
  const int Pg = p.Pg[g], pb = (int)blockIdx.x - p.gblk[g];
  const int batch = p.batch;

  // ---------------------------------------------------------------- tile prefix sums
  // (block (0, 0) writes the tile starts of every sequence to the workspace
  // header for the merge; every block notes where its first tile lies)
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
    int incl = sacc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (l >= d) incl += o;
    }
    if (l == 63) wsum[w] = incl;
    __syncthreads();
    int all = 0, before = 0;
    for (int i = 0; i < C::NW; ++i) {
      all += wsum[i];
      before += i < w ? wsum[i] : 0;
    }
    total = all;
    const int nb0 = pb * cdiv(total, Pg);
    int run = before + incl - sacc;
    const bool hdr = (g == 0 && pb == 0);
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int bb = tid * per + i;
      if (i < per && bb < batch) {
        if (hdr) p.hdr[bb] = run;
        if (nb0 >= run && nb0 < run + loc[i]) {
          start_info[0] = bb;
          start_info[1] = (nb0 - run) * C::TT;
        }
      }
      run += loc[i];
    }
    if (hdr && tid == C::NT - 1) p.hdr[batch] = total;
    __syncthreads();
  }
  const int tpb = cdiv(total, Pg);
  const int n_begin = pb * tpb;
  const int n_end = min(total, n_begin + tpb);
  if (n_begin >= n_end) return;

  const int rv = p.rv[g];
  const int nkc = cdiv(p.rk[g], 32);              // 32-deep chunks of the group's keys
  const int pk = p.pk[g], pv = p.pv[g];
  const int cprk = pk >> 4, cprv = pv >> 4;
  const int nnt = cdiv(rv, 16);
  const uint8_t* zk_seq = p.zk + p.goff_k[g];
  const uint8_t* zv_seq = p.zv + p.goff_v[g];
  const int64_t sbk = p.seq_bytes_k, sbv = p.seq_bytes_v;

  // ---------------------------------------------------------------- DMA slot geometry
  // Slot q of a region holds chunk (q % pitch) of token row (q / pitch);
  // padding slots load a chunk of a real row (finite, never used).
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

  // ---------------------------------------------------------------- tile cursor (wave-uniform)
  // The DMA cursor names a tile of the block's range: sequence b, first token
  // t0 of a history of L tokens, and the HBM addresses of its rows; it runs
  // two tiles ahead of the tile being scored.  The tiles behind it travel as
  // info words: b | valid tokens << 16 | F_START (first tile of a segment:
  // its query is loaded) | F_END (last tile of its history: its record is
  // written; the block's last tile is the other segment end).
  constexpr int F_START = 1 << 24, F_END = 1 << 25;
  auto len_of = [&](int b) __attribute__((always_inline)) {
    const int L = sload_i32(p.seq_lens + b);
    return L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
  };
  struct DCur { int b, t0, L, st; const uint8_t* kb; const uint8_t* vb; };
  // (paged caches: the block is the page holding token t0; a page holds a
  // power of two >= 32 rows, so a tile never straddles two pages)
  auto dma_addr = [&](DCur& d) __attribute__((always_inline)) {
    int blk = d.b, tin = d.t0;
    if constexpr (PAGED) {
      blk = sload_i32(p.block_table + (int64_t)d.b * p.max_pages + (d.t0 >> p.page_shift));
      tin = d.t0 & ((1 << p.page_shift) - 1);
    }
    d.kb = zk_seq + (int64_t)blk * sbk + (int64_t)tin * pk;
    d.vb = zv_seq + (int64_t)blk * sbv + (int64_t)tin * pv;
  };
  auto info_of = [&](const DCur& d) __attribute__((always_inline)) {
    const int rem = d.L - d.t0;
    return d.b | (min(rem, C::TT) << 16) | d.st | (rem <= C::TT ? F_END : 0);
  };
  auto advance = [&](DCur& d) __attribute__((always_inline)) {
    d.t0 += C::TT;
    d.kb += C::TT * pk;
    d.vb += C::TT * pv;
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
  // tile m of the cursor into ring buffer m % 3 (rows past the history
  // repeat its last row)
  auto issue = [&](const DCur& d, int m) __attribute__((always_inline)) {
    const unsigned base = lds_addr(&ring[m % C::NB][0]);
    const int lim = d.L - 1 - d.t0;
#pragma unroll
    for (int i = 0; i < C::NIK; ++i) {
      const int sbase = (i * C::NW + w) * 64;
      const unsigned off = (unsigned)min(dk_geo[i] >> 16, lim) * (unsigned)pk + (unsigned)(dk_geo[i] & 0xFFFF);
      dma16o(d.kb, off, base + 16u * (sbase < C::SLK ? sbase : C::SLK + C::SLV));
    }
#pragma unroll
    for (int i = 0; i < C::NIV; ++i) {
      const int sbase = (i * C::NW + w) * 64;
      const unsigned off = (unsigned)min(dv_geo[i] >> 16, lim) * (unsigned)pv + (unsigned)(dv_geo[i] & 0xFFFF);
      dma16o(d.vb, off, base + 16u * (sbase < C::SLV ? C::SLK + sbase : C::SLK + C::SLV));
    }
  };

  // ---------------------------------------------------------------- running state
  // Absorbed query as the B operand of the score MFMA: lane l holds head row
  // s = l % 16 (head s % 8; rows 8-15 the lo parts), ranks 32 kc + 8 q .. +7.
  op_t aq[C::NKC];
  auto load_query = [&](int b) __attribute__((always_inline)) {
    const int hh = s & 7;
    const bool valid = hh < nq;
    const float* qa = p.qabs + ((int64_t)b * p.H + g * nq + (valid ? hh : 0)) * p.qabs_stride + 8 * q;
    // (every chunk up to the capacity: the absorbed query is zero past the rank)
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc) {
      const f32x4 a0 = *(const f32x4*)(qa + 32 * kc);
      const f32x4 a1 = *(const f32x4*)(qa + 32 * kc + 4);
      op_t v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = valid ? (e < 4 ? a0[e] : a1[e - 4]) : 0.f;
        const LT hi = (LT)x;
        const LT lo = (LT)(x - (float)hi);
        v[e] = s < 8 ? hi : lo;
      }
      aq[kc] = v;
    }
  };
  // Wave w keeps its own online softmax over token half u = w / 4 of every
  // tile (tokens 16 u .. 16 u + 15) and accumulates the value n-tiles
  // grp + 4 i (grp = w % 4): D[head row][rank], rows 0-7 from the hi parts
  // of P, rows 8-15 from the lo parts.  Softmax state per lane for head
  // s % 8; the denominator as per-lane partial sums over the lane's tokens.
  // The maximum starts at a finite floor so that a half that has seen only
  // masked tokens yields p = 0 (not exp2(-inf + inf)).
  const int u = w >> 2, grp = w & 3;
  f32x4 acc[C::NNT4];
#pragma unroll
  for (int i = 0; i < C::NNT4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kAbsFloor, l_lane = 0.f;

  // Segment end: the two halves of each n-tile group meet through LDS
  // (half 1 writes, half 0 combines and writes the split record).  Called by
  // every wave (the segment ends are the same for the whole block).
  auto record = [&](int info) __attribute__((always_inline)) {
    const int b = info & 0xFFFF;
    const float lsum = rows4_sum(l_lane);   // over q: lanes s, s + 16, s + 32, s + 48
    f32x4* xa = &xacc[grp][0];
    if (u == 1) {
#pragma unroll
      for (int i = 0; i < C::NNT4; ++i) xa[i * 64 + l] = acc[i];
      if (l < 16) {
        xml[grp][0][l] = m_run;
        xml[grp][1][l] = lsum;
      }
    }
    wait_lgkm0();
    barrier();
    if (u == 0) {
      const float m1 = xml[grp][0][s], l1 = xml[grp][1][s];
      const float mm = fmaxf(m_run, m1);
      const float a0 = __builtin_amdgcn_exp2f(m_run - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
      float* rec = p.rec + ((int64_t)g * (p.P + batch) + pb + b) * p.rec_stride;
      if (grp == 0 && l < nq) {
        rec[2 * l] = mm;
        rec[2 * l + 1] = lsum * a0 + l1 * a1;
      }
      float* racc = rec + 2 * nq;
      // accumulator row 4 q + e belongs to head (4 q + e) % 8, whose factors
      // lane 4 q + e holds
      float r0[4], r1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r0[e] = shfl(a0, 4 * q + e);
        r1[e] = shfl(a1, 4 * q + e);
      }
#pragma unroll
      for (int i = 0; i < C::NNT4; ++i) {
        const int nt = grp + 4 * i;
        const f32x4 o = xa[i * 64 + l];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = halves_sum(acc[i][e] * r0[e] + o[e] * r1[e]);   // hi + lo rows (lanes l, l ^ 32)
          const int hrow = 4 * q + e;
          if (nt < nnt && q < 2 && hrow < nq) racc[hrow * p.rvp + 16 * nt + s] = c;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::NNT4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kAbsFloor;
    l_lane = 0.f;
  };

  // ---------------------------------------------------------------- pipeline
  DCur cd;
  cd.b = __builtin_amdgcn_readfirstlane(start_info[0]);
  cd.t0 = __builtin_amdgcn_readfirstlane(start_info[1]);
  cd.L = len_of(cd.b);
  cd.st = F_START;   // (the block's first tile starts a segment)
  dma_addr(cd);
  int i_c = info_of(cd), i_a = 0;
  issue(cd, n_begin);
  if (n_begin + 1 < n_end) {
    advance(cd);
    i_a = info_of(cd);
    issue(cd, n_begin + 1);
    if (n_begin + 2 < n_end) advance(cd);
  }

  // The tile loop is instantiated per chunk count NK (the group's 32-deep
  // key chunks, rounded up to even), chosen once per block: inside, every
  // loop is fully unrolled and branch-free (a runtime bound inside the loop
  // puts each operand read and its MFMA in a block of its own).  NR = the
  // value n-tile rounds of a wave at capacity (rounds past the rank repeat
  // the last n-tile and are never recorded).
  auto tile_loop = [&](auto nk_t, auto nr_t) __attribute__((always_inline)) {
    constexpr int NK = decltype(nk_t)::value, NR = decltype(nr_t)::value;
    for (int n = n_begin; n < n_end; ++n) {
      if (n + 1 < n_end) wait_vmcnt<C::NDMA>(); else wait_vmcnt<0>();
      barrier();   // tile n landed for every wave; tile n - 1's buffer is free
      int i_d = 0;
      if (n + 2 < n_end) {
        i_d = info_of(cd);
        issue(cd, n + 2);
        if (n + 3 < n_end) advance(cd);
      }
      // a segment's first tile: its absorbed query (loaded after this step's
      // DMA went out)
      if (i_c & F_START) load_query(i_c & 0xFFFF);

      const uint8_t* zkt = (const uint8_t*)&ring[n % C::NB][0];
      const uint8_t* zvt = zkt + C::SLK * 16;

      // ---- scores of this wave's 16 tokens: D[token 16 u + 4 q + i][head
      // row s], two accumulators (even and odd chunks).  The group's chunk
      // count picks one fully unrolled loop (branch-free inside, so the operand
      // reads go out ahead of the MFMAs); past the rank inside the last chunk
      // the query is zero.
      f32x4 sc0 = f32x4{0.f, 0.f, 0.f, 0.f}, sc1 = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint8_t* arow = zkt + ((16 * u + s) * C::PITK + q) * 16;
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) {
        if (kc & 1) sc1 = mfma16x16x32(*(const op_t*)(arow + 64 * kc), aq[kc], sc1);
        else sc0 = mfma16x16x32(*(const op_t*)(arow + 64 * kc), aq[kc], sc0);
      }
      // hi + lo rows (lanes s and s ^ 8 of a row hold the same sum); tokens
      // past the history masked
      float x[4];
      const int nv = (i_c >> 16) & 63;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = add_ror8(sc0[i] + sc1[i]);
      if (nv < C::TT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = 16 * u + 4 * q + i < nv ? x[i] : -INFINITY;
      }

      // ---- online softmax (lazy maximum)
      bool up = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) up |= x[i] > m_run + kAbsTau;
      if (__builtin_amdgcn_ballot_w64(up)) {
        const float tmax = rows4_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const float mnew = tmax > m_run + kAbsTau ? tmax : m_run;
        // (alpha is exactly 1 for a head whose maximum stays)
        const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
        m_run = mnew;
        l_lane *= alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ae = shfl(alpha, 4 * q + e);   // accumulator row 4 q + e
#pragma unroll
          for (int i = 0; i < C::NNT4; ++i) acc[i][e] *= ae;
        }
      }
      lt4_t pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pj = __builtin_amdgcn_exp2f(x[i] - m_run);
        l_lane += pj;
        const LT hi = (LT)pj;
        const LT lo = (LT)(pj - (float)hi);
        pl[i] = s < 8 ? hi : lo;
      }
      const op4_t pa = __builtin_bit_cast(op4_t, pl);

      // ---- acc += P z_v over the wave's 16 tokens: B[k = 4 q + j][rank
      // 16 nt + s] = z_v[16 u + 4 q + j] (one transposed read), for the wave's
      // n-tiles grp + 4 i below the group's rank (one unrolled loop per count)
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int nt = min(grp + 4 * i, C::RCAP / 16 - 1);
        const int row = 16 * u + 4 * q + (s >> 2);
        const i16x4 vb = ds_read_tr16(zvt + row * C::PITV * 16 + (16 * nt + 4 * (s & 3)) * 2);
        acc[i] = mfma16x16x16(pa, __builtin_bit_cast(op4_t, vb), acc[i]);
      }

      if ((i_c & F_END) || n + 1 == n_end) record(i_c);
      i_c = i_a;
      i_a = i_d;
    }
  };
  // (chunk counts rounded up to even: the extra chunk meets a zero query)
  with_count<1, C::NKC / 2>(cdiv(nkc, 2), [&](auto nk2_t) __attribute__((always_inline)) {
    tile_loop(std::integral_constant<int, 2 * decltype(nk2_t)::value>{}, std::integral_constant<int, C::NNT4>{});
  });
}

bool abs_supported(const DecodeKey& k, const DecodeParams& p) {
  if (k.rope || !(k.elt == Elt::F16 || k.elt == Elt::BF16) || p.q4) return false;
  if (k.kv_per_group * k.q_per_kv > 8 || k.rk_max > 320 || k.rv_max > 320) return false;
  const int cap = (k.rk_max <= 256 && k.rv_max <= 256) ? 256 : 320;
  for (int j = 0; j < p.G; ++j)
    if (p.pk[j] > 2 * cap || p.pv[j] > 2 * cap || p.pk[j] % 16 != 0 || p.pv[j] % 16 != 0) return false;
  // every absorbed-query row holds the capacity's values (zeros past the rank)
  return p.qabs_stride >= cap;
}

template <class LT, int RCAP, bool PAGED>
static void launch_abs_t(const DecodeParams& p, int nq, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const dim3 grid(p.gblk[p.G - 1] + p.Pg[p.G - 1]), block(512);
  if (t0 && t1)
    hipExtLaunchKernelGGL((palu_decode_abs_kernel<LT, RCAP, PAGED>), grid, block, 0, stream, t0, t1, 0, p, nq);
  else
    hipLaunchKernelGGL((palu_decode_abs_kernel<LT, RCAP, PAGED>), grid, block, 0, stream, p, nq);
}

template <class LT, int RCAP>
static void launch_abs_c(const DecodeParams& p, int nq, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (p.block_table)
    launch_abs_t<LT, RCAP, true>(p, nq, stream, t0, t1);
  else
    launch_abs_t<LT, RCAP, false>(p, nq, stream, t0, t1);
}

hipError_t launch_decode_abs(const DecodeKey& k, const DecodeParams& p, hipStream_t stream, hipEvent_t t0,
                             hipEvent_t t1) {
  const int nq = k.kv_per_group * k.q_per_kv;
  const bool small = k.rk_max <= 256 && k.rv_max <= 256;
  if (k.elt == Elt::F16) {
    if (small) launch_abs_c<_Float16, 256>(p, nq, stream, t0, t1);
    else launch_abs_c<_Float16, 320>(p, nq, stream, t0, t1);
  } else {
    if (small) launch_abs_c<__bf16, 256>(p, nq, stream, t0, t1);
    else launch_abs_c<__bf16, 320>(p, nq, stream, t0, t1);
  }
  return hipGetLastError();
}

}  // namespace palu
