// C ABI of the Palu latent-cache library: argument validation, the latent
// cache layout, launch planning and dispatch.  Every argument error is found
// here, on the host, before anything is enqueued.
#include "palu.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "decode.h"
#include "project.h"
#include "quant.h"

using namespace palu;

namespace {

thread_local char g_err[512];
thread_local hipEvent_t g_prof_before = nullptr, g_prof_after = nullptr;

palu_status fail(palu_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

palu_status ok() {
  g_err[0] = 0;
  return PALU_OK;
}

palu_status hip_fail(hipError_t e, const char* what) {
  return fail(PALU_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t roundup(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Row pitch (bytes) of a latent row of rank r.
int64_t row_pitch(palu_dtype dt, int r) {
  switch (dt) {
    case PALU_F32: return 4 * roundup(r, 4);
    case PALU_F16:
    case PALU_BF16: return 2 * roundup(r, 8);
    case PALU_I4: return 16 * ((r + 31) / 32);
  }
  return -1;
}
int64_t scale_pitch(int r) { return 2 * ((r + 31) / 32); }

bool valid_dtype(palu_dtype d) { return d == PALU_F32 || d == PALU_F16 || d == PALU_BF16 || d == PALU_I4; }

palu_status check_desc(const palu_attn_desc* d) {
  if (!d) return fail(PALU_ERR_INVALID_ARG, "desc is NULL");
  if (d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 || d->n_groups <= 0)
    return fail(PALU_ERR_INVALID_ARG, "head counts, head_dim and n_groups must be positive");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(PALU_ERR_INVALID_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", d->n_q_heads,
                d->n_kv_heads);
  if (d->n_kv_heads % d->n_groups != 0)
    return fail(PALU_ERR_INVALID_ARG, "n_kv_heads (%d) must be a multiple of n_groups (%d)", d->n_kv_heads,
                d->n_groups);
  if (d->head_dim % 2 != 0) return fail(PALU_ERR_INVALID_ARG, "head_dim must be even");
  if (d->n_groups > kMaxGroups) return fail(PALU_ERR_UNSUPPORTED, "at most %d groups", kMaxGroups);
  if (!d->rank_k || !d->rank_v) return fail(PALU_ERR_INVALID_ARG, "rank_k / rank_v is NULL");
  for (int j = 0; j < d->n_groups; ++j)
    if (d->rank_k[j] <= 0 || d->rank_v[j] <= 0) return fail(PALU_ERR_INVALID_ARG, "rank of group %d is not positive", j);
  if (!valid_dtype(d->latent_dtype) || !valid_dtype(d->act_dtype) || d->act_dtype == PALU_I4)
    return fail(PALU_ERR_INVALID_ARG, "invalid dtype");
  if (d->use_rope && !(std::isfinite(d->rope_base) && d->rope_base > 0))
    return fail(PALU_ERR_INVALID_ARG, "rope_base must be positive and finite");
  return PALU_OK;
}

struct Layout {
  int64_t pk[kMaxGroups], pv[kMaxGroups], spk[kMaxGroups], spv[kMaxGroups];
  int64_t goff_k[kMaxGroups], goff_v[kMaxGroups], soff_k[kMaxGroups], soff_v[kMaxGroups];
  int64_t seq_k, seq_v, seq_sk, seq_sv;   // bytes of one sequence block
};

void make_layout(const palu_attn_desc* d, int64_t max_len, Layout* L) {
  int64_t ok_ = 0, ov = 0, osk = 0, osv = 0;
  for (int j = 0; j < d->n_groups; ++j) {
    L->pk[j] = row_pitch(d->latent_dtype, d->rank_k[j]);
    L->pv[j] = row_pitch(d->latent_dtype, d->rank_v[j]);
    L->spk[j] = d->latent_dtype == PALU_I4 ? scale_pitch(d->rank_k[j]) : 0;
    L->spv[j] = d->latent_dtype == PALU_I4 ? scale_pitch(d->rank_v[j]) : 0;
    L->goff_k[j] = ok_; L->goff_v[j] = ov; L->soff_k[j] = osk; L->soff_v[j] = osv;
    ok_ += max_len * L->pk[j]; ov += max_len * L->pv[j];
    osk += max_len * L->spk[j]; osv += max_len * L->spv[j];
  }
  L->seq_k = ok_; L->seq_v = ov; L->seq_sk = osk; L->seq_sv = osv;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device (cached per device).
std::atomic<int> g_cu[64];

palu_status device_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev >= 0 && dev < 64) {
    int c = g_cu[dev].load(std::memory_order_relaxed);
    if (c > 0) { *out = c; return PALU_OK; }
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  if (dev >= 0 && dev < 64) g_cu[dev].store(cus, std::memory_order_relaxed);
  *out = cus;
  return PALU_OK;
}

struct DecodePlan {
  DecodeKey key;
  int P, rvp, qabs_stride, nq;
  int Pg[kMaxGroups], gblk[kMaxGroups];   // blocks of each group and the first block id of its range
  size_t hdr_bytes, rec_bytes, qabs_bytes, total;
  // int4 latents: the MHA kernel reads the codes itself (fused4); on other
  // shapes the decode runs on an exact 16-bit copy of the cache in the
  // workspace, every 32-element chunk expanded to hi and lo chunks (rank
  // r' = 64 ceil(r/32)), against factors whose rows are duplicated to match
  bool q4, fused4;
  size_t dense_k_bytes, dense_v_bytes, dup_k_bytes, dup_v_bytes;
  int64_t dk_pitch[kMaxGroups], dv_pitch[kMaxGroups], dk_goff[kMaxGroups], dv_goff[kMaxGroups];
  int64_t dk_seq, dv_seq;
  int drk[kMaxGroups], drv[kMaxGroups];   // ranks the decode kernels see
};

Elt elt_of(palu_dtype d) { return d == PALU_F32 ? Elt::F32 : d == PALU_F16 ? Elt::F16 : Elt::BF16; }

// Fixed time per tile of the absorbed-query kernel, in ranks of row bytes.
// Measured on MI355X at the GQA 8B shape (ranks 320/192/192/128): 0 (byte
// weighting) 235 us, 256: 166 us, 384: 164 us, 512: 167 us, 1024: 174 us,
// uniform split 177 us.
constexpr int kAbsTileRanks = 384;

palu_status plan_decode(const palu_attn_desc* d, int batch, int max_len, DecodePlan* pl) {
  palu_status s = check_desc(d);
  if (s != PALU_OK) return s;
  if (batch < 0) return fail(PALU_ERR_INVALID_ARG, "batch must be >= 0");
  if (max_len <= 0) return fail(PALU_ERR_INVALID_ARG, "max_len must be positive");
  if (batch > kMaxBatch) return fail(PALU_ERR_UNSUPPORTED, "batch above %d", kMaxBatch);
  pl->q4 = d->latent_dtype == PALU_I4;
  if (pl->q4 && d->act_dtype == PALU_F32)
    return fail(PALU_ERR_UNSUPPORTED, "int4 latents need act_dtype F16 or BF16");
  if (!pl->q4 && d->latent_dtype != d->act_dtype)
    return fail(PALU_ERR_UNSUPPORTED, "latent_dtype must equal act_dtype for float latents");
  const int ng = d->n_kv_heads / d->n_groups, qpk = d->n_q_heads / d->n_kv_heads;
  // int4: the MHA kernel reads the codes (ranks rounded up to 32) where it
  // applies; elsewhere the kernels see hi/lo rows of twice that rank
  pl->fused4 = false;
  if (pl->q4) {
    int r32k = 0, r32v = 0;
    for (int j = 0; j < d->n_groups; ++j) {
      r32k = (int)std::max<int64_t>(r32k, roundup(d->rank_k[j], 32));
      r32v = (int)std::max<int64_t>(r32v, roundup(d->rank_v[j], 32));
    }
    if (r32k > 1024 || r32v > 1024) return fail(PALU_ERR_UNSUPPORTED, "int4 latents: rank above 1024");
    const DecodeKey k32{elt_of(d->act_dtype), d->head_dim, ng, qpk, r32k, r32v, d->use_rope != 0};
    int ck = 0, cv = 0;
    if (decode_supported(k32, &ck, &cv)) {
      DecodeParams t;
      memset(&t, 0, sizeof(t));
      t.G = d->n_groups;
      t.q4 = 1;
      t.rvp = (int)roundup(cv, 16);
      for (int j = 0; j < d->n_groups; ++j) {
        t.rk[j] = d->rank_k[j];
        t.rv[j] = d->rank_v[j];
        t.pk[j] = (int)row_pitch(PALU_I4, d->rank_k[j]);
        t.pv[j] = (int)row_pitch(PALU_I4, d->rank_v[j]);
      }
      pl->fused4 = mha_supported(k32, t);
    }
  }
  auto dense_rank = [&](int r) {
    return pl->q4 ? (int)(pl->fused4 ? roundup(r, 32) : 2 * roundup(r, 32)) : r;
  };
  int rk_max = 0, rv_max = 0;
  for (int j = 0; j < d->n_groups; ++j) {
    pl->drk[j] = dense_rank(d->rank_k[j]);
    pl->drv[j] = dense_rank(d->rank_v[j]);
    rk_max = pl->drk[j] > rk_max ? pl->drk[j] : rk_max;
    rv_max = pl->drv[j] > rv_max ? pl->drv[j] : rv_max;
  }
  pl->key = DecodeKey{elt_of(d->act_dtype), d->head_dim, ng, qpk, rk_max, rv_max, d->use_rope != 0};
  int rk_cap = 0, rv_cap = 0;
  if (pl->q4 && !pl->fused4 && !decode_supported(pl->key, &rk_cap, &rv_cap))
    return fail(PALU_ERR_UNSUPPORTED,
                "int4 latents on this shape are attended as exact hi/lo 16-bit rows of twice the rank rounded "
                "up to 32 (%d, %d), which no decode kernel covers; the MHA head-group shape (4 kv heads per "
                "group, one query head each, head_dim 128, RoPE, ranks <= 256) reads int4 codes directly",
                rk_max, rv_max);
  if (!decode_supported(pl->key, &rk_cap, &rv_cap))
    return fail(PALU_ERR_UNSUPPORTED,
                "no decode kernel for dtype %d, head_dim %d, %d kv heads per group, %d query heads per kv head, "
                "ranks <= (%d, %d), rope %d",
                (int)d->latent_dtype, d->head_dim, ng, qpk, rk_max, rv_max, d->use_rope);
  int cus = 0;
  s = device_cus(&cus);
  if (s != PALU_OK) return s;
  const int64_t tiles_bound = (int64_t)batch * ((max_len + kDecTile - 1) / kDecTile);
  int64_t P = (cus + d->n_groups - 1) / d->n_groups;
  if (P > tiles_bound) P = tiles_bound;
  if (P < 1) P = 1;
  pl->nq = ng * qpk;
  pl->rvp = (int)roundup(rv_cap, 16);
  pl->qabs_stride = (int)roundup(rk_cap, 4);
  for (int j = 0; j < d->n_groups; ++j) pl->Pg[j] = (int)P;
  if (!d->use_rope) {
    // The absorbed-query kernel's time per 32-token tile is a fixed part plus
    // a part that grows with the row bytes, so the same total of blocks goes
    // to the groups in proportion to r_k + r_v + kAbsTileRanks, and groups of
    // mixed ranks end together.
    DecodeParams t;
    memset(&t, 0, sizeof(t));
    t.G = d->n_groups;
    t.qabs_stride = pl->qabs_stride;
    for (int j = 0; j < d->n_groups; ++j) {
      t.rk[j] = pl->drk[j];
      t.rv[j] = pl->drv[j];
      t.pk[j] = pl->q4 ? 2 * t.rk[j] : (int)row_pitch(d->latent_dtype, d->rank_k[j]);
      t.pv[j] = pl->q4 ? 2 * t.rv[j] : (int)row_pitch(d->latent_dtype, d->rank_v[j]);
    }
    if (abs_supported(pl->key, t)) {
      int64_t wsum = 0;
      for (int j = 0; j < d->n_groups; ++j) wsum += t.rk[j] + t.rv[j] + kAbsTileRanks;
      const int64_t tot = P * d->n_groups;
      double frac[kMaxGroups];
      int64_t given = 0;
      for (int j = 0; j < d->n_groups; ++j) {
        const double share = (double)tot * (double)(t.rk[j] + t.rv[j] + kAbsTileRanks) / (double)wsum;
        int64_t n = (int64_t)share;
        n = n < 1 ? 1 : n;
        pl->Pg[j] = (int)n;
        frac[j] = share - (double)n;
        given += n;
      }
      for (; given < tot; ++given) {   // the remaining blocks by largest remainder
        int best = 0;
        for (int j = 1; j < d->n_groups; ++j) best = frac[j] > frac[best] ? j : best;
        ++pl->Pg[best];
        frac[best] -= 1.0;
      }
      P = 1;
      for (int j = 0; j < d->n_groups; ++j) {
        if (pl->Pg[j] > tiles_bound) pl->Pg[j] = (int)(tiles_bound > 1 ? tiles_bound : 1);
        P = pl->Pg[j] > P ? pl->Pg[j] : P;
      }
    }
  }
  pl->gblk[0] = 0;
  for (int j = 1; j < d->n_groups; ++j) pl->gblk[j] = pl->gblk[j - 1] + pl->Pg[j - 1];
  pl->P = (int)P;
  pl->hdr_bytes = (size_t)roundup((int64_t)(batch + 1) * 4, 256);
  pl->rec_bytes = (size_t)roundup((int64_t)d->n_groups * (P + batch) * pl->nq * (2 + pl->rvp) * 4, 256);
  pl->qabs_bytes = d->use_rope ? 0 : (size_t)roundup((int64_t)batch * d->n_q_heads * pl->qabs_stride * 4, 256);
  pl->dense_k_bytes = pl->dense_v_bytes = pl->dup_k_bytes = pl->dup_v_bytes = 0;
  pl->dk_seq = pl->dv_seq = 0;
  if (pl->q4 && !pl->fused4) {
    const int64_t w = (int64_t)ng * d->head_dim;
    int64_t bk = 0, bv = 0;
    for (int j = 0; j < d->n_groups; ++j) {
      pl->dk_pitch[j] = 2 * (int64_t)pl->drk[j];
      pl->dv_pitch[j] = 2 * (int64_t)pl->drv[j];
      pl->dk_goff[j] = pl->dk_seq;
      pl->dv_goff[j] = pl->dv_seq;
      pl->dk_seq += (int64_t)max_len * pl->dk_pitch[j];
      pl->dv_seq += (int64_t)max_len * pl->dv_pitch[j];
      bk += (int64_t)pl->drk[j] * w * 2;
      bv += (int64_t)pl->drv[j] * w * 2;
    }
    pl->dense_k_bytes = (size_t)roundup((int64_t)batch * pl->dk_seq, 256);
    pl->dense_v_bytes = (size_t)roundup((int64_t)batch * pl->dv_seq, 256);
    pl->dup_k_bytes = (size_t)roundup(bk, 256);
    pl->dup_v_bytes = (size_t)roundup(bv, 256);
  }
  pl->total = pl->hdr_bytes + pl->rec_bytes + pl->qabs_bytes + pl->dense_k_bytes + pl->dense_v_bytes +
              pl->dup_k_bytes + pl->dup_v_bytes;
  return PALU_OK;
}
// Latent storage one prefill writes (contiguous, or paged through a block table).
struct WriteView {
  void* zk; void* zv; void* sk; void* sv;
  int32_t layout_len, max_len;
  const int32_t* block_table;
  int32_t page_shift, max_pages;
};

palu_status project_impl(const palu_attn_desc* desc, const void* x, int32_t d_model, int64_t n_tok, const void* A_kv,
                         const WriteView* cache, int32_t seq, int32_t pos0, hipStream_t stream) {
  palu_status s = check_desc(desc);
  if (s != PALU_OK) return s;
  if (!x || !A_kv || !cache->zk || !cache->zv) return fail(PALU_ERR_INVALID_ARG, "null pointer");
  if (d_model <= 0 || n_tok < 0 || seq < 0 || pos0 < 0) return fail(PALU_ERR_INVALID_ARG, "bad d_model/n_tok/seq/pos0");
  if (cache->max_len <= 0) return fail(PALU_ERR_INVALID_ARG, "max_len must be positive");
  if ((int64_t)pos0 + n_tok > cache->max_len) return fail(PALU_ERR_INVALID_ARG, "pos0 + n_tok exceeds max_len");
  const bool quant = desc->latent_dtype == PALU_I4;
  if (!quant && desc->latent_dtype != desc->act_dtype)
    return fail(PALU_ERR_UNSUPPORTED, "latent_dtype must equal act_dtype or be I4");
  if (quant && (!cache->sk || !cache->sv)) return fail(PALU_ERR_INVALID_ARG, "I4 scales are NULL");
  if (d_model % 64 != 0) return fail(PALU_ERR_UNSUPPORTED, "d_model must be a multiple of 64");
  if (!aligned16(x) || !aligned16(A_kv) || !aligned16(cache->zk) || !aligned16(cache->zv))
    return fail(PALU_ERR_INVALID_ARG, "x, A_kv and latent buffers must be 16-byte aligned");
  if (2 * desc->n_groups > kMaxLatentRows) return fail(PALU_ERR_UNSUPPORTED, "too many groups");
  if (n_tok == 0) return ok();
  Layout L;
  make_layout(desc, cache->layout_len, &L);
  ProjectParams p;
  memset(&p, 0, sizeof(p));
  p.block_table = cache->block_table; p.page_shift = cache->page_shift; p.max_pages = cache->max_pages;
  p.x = x; p.A = A_kv;
  p.zk = (uint8_t*)cache->zk; p.zv = (uint8_t*)cache->zv;
  p.sk = (uint8_t*)cache->sk; p.sv = (uint8_t*)cache->sv;
  p.n_tok = n_tok; p.d_model = d_model; p.pos0 = pos0;
  p.G = desc->n_groups; p.seq = seq; p.quant = quant ? 1 : 0;
  int64_t col = 0;
  for (int j = 0; j < desc->n_groups; ++j) {
    p.rank[j] = desc->rank_k[j]; p.col_off[j] = col; col += desc->rank_k[j];
  }
  for (int j = 0; j < desc->n_groups; ++j) {
    p.rank[desc->n_groups + j] = desc->rank_v[j]; p.col_off[desc->n_groups + j] = col; col += desc->rank_v[j];
  }
  p.seq_bytes_k = L.seq_k; p.seq_bytes_v = L.seq_v; p.seq_sbytes_k = L.seq_sk; p.seq_sbytes_v = L.seq_sv;
  for (int j = 0; j < desc->n_groups; ++j) {
    p.goff_k[j] = L.goff_k[j]; p.goff_v[j] = L.goff_v[j];
    p.soff_k[j] = L.soff_k[j]; p.soff_v[j] = L.soff_v[j];
    p.pk[j] = (int)L.pk[j]; p.pv[j] = (int)L.pv[j];
  }
  int64_t ntiles = 0;
  for (int j = 0; j < desc->n_groups; ++j) ntiles += (desc->rank_k[j] + kColTile - 1) / kColTile + (desc->rank_v[j] + kColTile - 1) / kColTile;
  if (ntiles > kMaxColTiles) return fail(PALU_ERR_UNSUPPORTED, "more than %d column tiles of %d latent channels", kMaxColTiles, kColTile);
  // (the kernel addresses A_kv and a 256-token slice of x with 32-bit byte offsets)
  const int64_t esz = desc->act_dtype == PALU_F32 ? 4 : 2;
  if (col * d_model * esz > (int64_t)UINT32_MAX || 256 * (int64_t)d_model * esz > (int64_t)UINT32_MAX)
    return fail(PALU_ERR_UNSUPPORTED, "A_kv larger than 4 GiB");
  const bool prof = g_prof_before && g_prof_after;
  hipError_t e = launch_project((int)desc->act_dtype, p, stream, prof ? g_prof_before : nullptr,
                                prof ? g_prof_after : nullptr);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return ok();
}

// page_size / max_pages / n_pages checks shared by the paged entry points
palu_status check_paged(const palu_paged_cache* cache, int* shift) {
  const int ps = cache->page_size;
  if (ps < 32 || (ps & (ps - 1)) != 0) return fail(PALU_ERR_INVALID_ARG, "page_size must be a power of two >= 32");
  if (cache->max_pages <= 0 || cache->n_pages <= 0) return fail(PALU_ERR_INVALID_ARG, "max_pages and n_pages must be positive");
  if ((int64_t)cache->max_pages * ps > INT32_MAX / 2) return fail(PALU_ERR_UNSUPPORTED, "max_pages * page_size too large");
  int sh = 0;
  while ((1 << sh) < ps) ++sh;
  *shift = sh;
  return PALU_OK;
}
// The latent storage one decode call reads: a contiguous cache (rows per
// block = history bound = max_len) or a paged one (rows per block = page
// size; rows of sequence b found through the block table).
struct CacheView {
  void* zk; void* zv; void* sk; void* sv;
  int32_t layout_len;            // rows of one (block, group) in the layout
  int32_t max_len;               // longest history
  const int32_t* block_table;    // paged: [batch][max_pages], else NULL
  int32_t page_shift, max_pages;
};

palu_status decode_impl(const palu_attn_desc* desc, const void* q, const CacheView* cache, const void* B_k,
                        const void* B_v, const int32_t* seq_lens, const int32_t* q_pos, int32_t batch,
                        float sm_scale, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodePlan pl;
  palu_status s = plan_decode(desc, batch, cache->max_len, &pl);
  if (s != PALU_OK) return s;
  if (cache->block_table && pl.q4 && !pl.fused4)
    return fail(PALU_ERR_UNSUPPORTED, "paged int4 pools need the MHA head-group kernel shape "
                                      "(4 kv heads per group, one query head each, head_dim 128, RoPE)");
  if (batch == 0) return ok();   // nothing is read or written
  if (!q || !B_k || !B_v || !seq_lens || !out || !cache->zk || !cache->zv)
    return fail(PALU_ERR_INVALID_ARG, "null pointer");
  if (!std::isfinite(sm_scale)) return fail(PALU_ERR_INVALID_ARG, "sm_scale must be finite");
  if (!aligned16(cache->zk) || !aligned16(cache->zv))
    return fail(PALU_ERR_INVALID_ARG, "latent buffers must be 16-byte aligned");
  if (!workspace) return fail(PALU_ERR_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(PALU_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < pl.total)
    return fail(PALU_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", pl.total, workspace_bytes);

  if (pl.q4) {
    if (!cache->sk || !cache->sv) return fail(PALU_ERR_INVALID_ARG, "I4 scales are NULL");
    if (((uintptr_t)cache->sk & 1u) != 0 || ((uintptr_t)cache->sv & 1u) != 0)
      return fail(PALU_ERR_INVALID_ARG, "I4 scale buffers must be 2-byte aligned");
  }
  Layout L;
  make_layout(desc, cache->layout_len, &L);
  uint8_t* const dense_k = (uint8_t*)workspace + pl.hdr_bytes + pl.rec_bytes + pl.qabs_bytes;
  uint8_t* const dense_v = dense_k + pl.dense_k_bytes;
  uint8_t* const dup_k = dense_v + pl.dense_v_bytes;
  uint8_t* const dup_v = dup_k + pl.dup_k_bytes;
  const int w = (desc->n_kv_heads / desc->n_groups) * desc->head_dim;
  if (pl.q4 && !pl.fused4) {
    // int4 latents -> exact hi/lo 16-bit rows (the history of every sequence,
    // keys and values), and the factors with every row duplicated to match
    static_assert(kDqMaxGroups >= kMaxGroups, "group arrays");
    DequantParams dp;
    memset(&dp, 0, sizeof(dp));
    dp.seq_lens = seq_lens;
    dp.batch = batch; dp.G = desc->n_groups; dp.max_len = cache->max_len;
    for (int which = 0; which < 2; ++which) {
      DequantSide& sd = dp.side[which];
      sd.codes = (const uint8_t*)(which ? cache->zv : cache->zk);
      sd.scales = (const uint8_t*)(which ? cache->sv : cache->sk);
      sd.out = which ? dense_v : dense_k;
      sd.seq_c = which ? L.seq_v : L.seq_k;
      sd.seq_s = which ? L.seq_sv : L.seq_sk;
      sd.seq_o = which ? pl.dv_seq : pl.dk_seq;
      for (int j = 0; j < desc->n_groups; ++j) {
        sd.goff_c[j] = which ? L.goff_v[j] : L.goff_k[j];
        sd.goff_s[j] = which ? L.soff_v[j] : L.soff_k[j];
        sd.goff_o[j] = which ? pl.dv_goff[j] : pl.dk_goff[j];
        sd.rank[j] = which ? desc->rank_v[j] : desc->rank_k[j];
        sd.nch[j] = (sd.rank[j] + 31) / 32;
        sd.magic[j] = (unsigned)(((1ull << 32) + (uint64_t)sd.nch[j] - 1) / (uint64_t)sd.nch[j]);
        dp.max_nch = sd.nch[j] > dp.max_nch ? sd.nch[j] : dp.max_nch;
      }
    }
    dp.n_sides = 2;
    dp.split = 1;
    hipError_t e = launch_dequant(desc->act_dtype == PALU_F16 ? 1 : 2, dp, stream);
    if (e != hipSuccess) return hip_fail(e, "int4 expansion launch");
    DupParams up;
    memset(&up, 0, sizeof(up));
    up.src[0] = B_k; up.src[1] = B_v; up.dst[0] = dup_k; up.dst[1] = dup_v;
    up.G = desc->n_groups; up.w = w;
    int64_t so[2] = {0, 0}, dof[2] = {0, 0};
    for (int j = 0; j < desc->n_groups; ++j) {
      const int r[2] = {desc->rank_k[j], desc->rank_v[j]}, rr[2] = {pl.drk[j], pl.drv[j]};
      for (int side = 0; side < 2; ++side) {
        up.soff[side][j] = so[side]; up.doff[side][j] = dof[side]; up.rank[side][j] = r[side];
        so[side] += (int64_t)r[side] * w; dof[side] += (int64_t)rr[side] * w;
        up.max_rows = rr[side] > up.max_rows ? rr[side] : up.max_rows;
      }
    }
    e = launch_dup_factor(up, stream);
    if (e != hipSuccess) return hip_fail(e, "factor duplication launch");
  }
  DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.q = q; p.zk = (const uint8_t*)cache->zk; p.zv = (const uint8_t*)cache->zv;
  p.Bk = B_k; p.Bv = B_v; p.seq_lens = seq_lens; p.q_pos = q_pos;
  uint8_t* ws = (uint8_t*)workspace;
  p.hdr = (int*)ws;
  p.rec = (float*)(ws + pl.hdr_bytes);
  p.qabs = desc->use_rope ? nullptr : (const float*)(ws + pl.hdr_bytes + pl.rec_bytes);
  p.out = out;
  p.batch = batch; p.max_len = cache->max_len; p.H = desc->n_q_heads; p.G = desc->n_groups; p.P = pl.P;
  p.block_table = cache->block_table; p.page_shift = cache->page_shift; p.max_pages = cache->max_pages;
  p.rvp = pl.rvp; p.rec_stride = pl.nq * (2 + pl.rvp); p.qabs_stride = pl.qabs_stride;
  p.qscale = sm_scale * 1.4426950408889634f;
  p.rope_base = desc->rope_base;
  p.seq_bytes_k = L.seq_k; p.seq_bytes_v = L.seq_v;
  int64_t bk = 0, bv = 0;
  for (int j = 0; j < desc->n_groups; ++j) {
    p.goff_k[j] = L.goff_k[j]; p.goff_v[j] = L.goff_v[j];
    p.boff_k[j] = bk; p.boff_v[j] = bv;
    bk += (int64_t)desc->rank_k[j] * w; bv += (int64_t)desc->rank_v[j] * w;
    p.rk[j] = desc->rank_k[j]; p.rv[j] = desc->rank_v[j];
    p.pk[j] = (int)L.pk[j]; p.pv[j] = (int)L.pv[j];
  }
  if (pl.fused4) {
    // the MHA kernel expands the int4 tiles itself
    p.q4 = 1;
    p.sk = (const uint8_t*)cache->sk; p.sv = (const uint8_t*)cache->sv;
    p.seq_sbytes_k = L.seq_sk; p.seq_sbytes_v = L.seq_sv;
    for (int j = 0; j < desc->n_groups; ++j) {
      p.soff_k[j] = L.soff_k[j]; p.soff_v[j] = L.soff_v[j];
    }
  } else if (pl.q4) {
    p.zk = dense_k; p.zv = dense_v;
    p.Bk = dup_k; p.Bv = dup_v;
    p.seq_bytes_k = pl.dk_seq; p.seq_bytes_v = pl.dv_seq;
    int64_t dk = 0, dv = 0;
    for (int j = 0; j < desc->n_groups; ++j) {
      p.goff_k[j] = pl.dk_goff[j]; p.goff_v[j] = pl.dv_goff[j];
      p.pk[j] = (int)pl.dk_pitch[j]; p.pv[j] = (int)pl.dv_pitch[j];
      p.rk[j] = pl.drk[j]; p.rv[j] = pl.drv[j];
      p.boff_k[j] = dk; p.boff_v[j] = dv;
      dk += (int64_t)pl.drk[j] * w; dv += (int64_t)pl.drv[j] * w;
    }
    p.zero_padded = 1;
  }
  // blocks per group: the plan's weighted counts where the absorbed-query
  // kernel runs (the same test launch_decode applies), else P for every group
  // (the kernels that take block id = p * G + g); the merge reads them
  const bool weighted = !desc->use_rope && abs_supported(pl.key, p);
  for (int j = 0; j < desc->n_groups; ++j) {
    p.Pg[j] = weighted ? pl.Pg[j] : pl.P;
    p.gblk[j] = weighted ? pl.gblk[j] : j * pl.P;
  }
  hipError_t e;
  if (!desc->use_rope) {
    e = launch_qabs(pl.key, p, stream);
    if (e != hipSuccess) return hip_fail(e, "absorbed-query launch");
  }
  const bool prof = g_prof_before && g_prof_after;
  e = launch_decode(pl.key, p, stream, prof ? g_prof_before : nullptr, prof ? g_prof_after : nullptr);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  e = launch_merge(pl.key, p, stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}
// Scratch of palu_decode_attn_noalloc: one array per GPU, held by the loaded
// code object until the process ends.  Host code never uses the array's
// name as a device address: each device's address is resolved once with
// hipGetSymbolAddress (with that device current) and kept here.
static __device__ __align__(256) uint8_t scratch[PALU_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

palu_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PALU_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(PALU_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PALU_OK;
}

// workspace of a chunk call: virtual lengths, positions and block-table rows,
// then the decode workspace of the virtual batch
size_t chunk_front_bytes(int64_t vbatch, int max_pages) {
  return (size_t)roundup(vbatch * (2 + (int64_t)max_pages) * 4, 256);
}

palu_status chunk_impl(const palu_attn_desc* desc, const void* q, int32_t q_len, const CacheView* base,
                       const void* B_k, const void* B_v, const int32_t* seq_lens, int32_t batch, float sm_scale,
                       void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (q_len <= 0) return fail(PALU_ERR_INVALID_ARG, "q_len must be positive");
  if (batch < 0) return fail(PALU_ERR_INVALID_ARG, "batch < 0");
  const int64_t vbatch = (int64_t)batch * q_len;
  if (vbatch > kMaxBatch) return fail(PALU_ERR_UNSUPPORTED, "batch * q_len above %d", kMaxBatch);
  if (batch == 0) return decode_impl(desc, q, base, B_k, B_v, seq_lens, nullptr, 0, sm_scale, out, workspace,
                                     workspace_bytes, stream);
  if (!seq_lens || !workspace) return fail(PALU_ERR_INVALID_ARG, "null pointer");
  if (((uintptr_t)workspace & 255u) != 0) return fail(PALU_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t front = chunk_front_bytes(vbatch, base->max_pages);
  if (workspace_bytes < front) return fail(PALU_ERR_WORKSPACE_TOO_SMALL, "workspace too small for the chunk");
  int* vlens = (int*)workspace;
  int* vqpos = vlens + vbatch;
  int* vtable = vqpos + vbatch;
  hipError_t e = launch_chunk_expand(seq_lens, base->block_table, batch, q_len, base->max_len, base->max_pages,
                                     vlens, vqpos, vtable, stream);
  if (e != hipSuccess) return hip_fail(e, "chunk expansion launch");
  CacheView v = *base;
  v.block_table = vtable;
  return decode_impl(desc, q, &v, B_k, B_v, vlens, vqpos, (int32_t)vbatch, sm_scale, out, (uint8_t*)workspace + front,
                     workspace_bytes - front, stream);
}

}  // namespace

extern "C" {

const char* palu_status_string(palu_status s) {
  switch (s) {
    case PALU_OK: return "PALU_OK";
    case PALU_ERR_INVALID_ARG: return "PALU_ERR_INVALID_ARG";
    case PALU_ERR_UNSUPPORTED: return "PALU_ERR_UNSUPPORTED";
    case PALU_ERR_WORKSPACE_TOO_SMALL: return "PALU_ERR_WORKSPACE_TOO_SMALL";
    case PALU_ERR_HIP: return "PALU_ERR_HIP";
  }
  return "PALU_ERR_UNKNOWN";
}

const char* palu_last_error(void) { return g_err; }

palu_status palu_profile_events(hipEvent_t before_main, hipEvent_t after_main) {
  g_prof_before = before_main;
  g_prof_after = after_main;
  return ok();
}

size_t palu_latent_bytes(const palu_attn_desc* desc, int32_t batch, int32_t max_len, int32_t which,
                         int32_t scales) {
  if (check_desc(desc) != PALU_OK || batch < 0 || max_len <= 0 || (which != 0 && which != 1)) return 0;
  if (scales && desc->latent_dtype != PALU_I4) return 0;
  Layout L;
  make_layout(desc, max_len, &L);
  const int64_t per = scales ? (which ? L.seq_sv : L.seq_sk) : (which ? L.seq_v : L.seq_k);
  return (size_t)(per * batch);
}

int64_t palu_latent_offset(const palu_attn_desc* desc, int32_t max_len, int32_t which, int32_t scales, int32_t b,
                           int32_t j, int32_t t) {
  if (check_desc(desc) != PALU_OK || max_len <= 0 || (which != 0 && which != 1)) return -1;
  if (b < 0 || j < 0 || j >= desc->n_groups || t < 0 || t >= max_len) return -1;
  if (scales && desc->latent_dtype != PALU_I4) return -1;
  Layout L;
  make_layout(desc, max_len, &L);
  if (scales)
    return which ? b * L.seq_sv + L.soff_v[j] + t * L.spv[j] : b * L.seq_sk + L.soff_k[j] + t * L.spk[j];
  return which ? b * L.seq_v + L.goff_v[j] + t * L.pv[j] : b * L.seq_k + L.goff_k[j] + t * L.pk[j];
}

palu_status palu_quant_latent(const void* z, palu_dtype z_dtype, int64_t n_rows, int32_t r, int64_t z_row_stride,
                              void* codes, void* scales, hipStream_t stream) {
  if (n_rows < 0 || r <= 0 || z_row_stride < r) return fail(PALU_ERR_INVALID_ARG, "bad n_rows / r / z_row_stride");
  if (z_dtype == PALU_I4) return fail(PALU_ERR_UNSUPPORTED, "input must be F32, F16 or BF16");
  if (!valid_dtype(z_dtype)) return fail(PALU_ERR_INVALID_ARG, "invalid dtype");
  if (n_rows == 0) return ok();
  if (!z || !codes || !scales) return fail(PALU_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(codes)) return fail(PALU_ERR_INVALID_ARG, "codes must be 16-byte aligned");
  if (z_row_stride > (int64_t)kQuantMaxStrideBytes / (z_dtype == PALU_F32 ? 4 : 2))
    return fail(PALU_ERR_UNSUPPORTED, "z_row_stride above %u bytes", kQuantMaxStrideBytes);
  hipError_t e = launch_quant((int)z_dtype, z, n_rows, r, z_row_stride, codes, scales, stream);
  if (e != hipSuccess) return hip_fail(e, "quantiser launch");
  return ok();
}

palu_status palu_quant_latent_rotated(const void* z, palu_dtype z_dtype, int64_t n_rows, int32_t r,
                                      int64_t z_row_stride, void* codes, void* scales, hipStream_t stream) {
  if (n_rows < 0 || r <= 0 || z_row_stride < r) return fail(PALU_ERR_INVALID_ARG, "bad n_rows / r / z_row_stride");
  if (z_dtype == PALU_I4) return fail(PALU_ERR_UNSUPPORTED, "input must be F32, F16 or BF16");
  if (!valid_dtype(z_dtype)) return fail(PALU_ERR_INVALID_ARG, "invalid dtype");
  if (n_rows == 0) return ok();
  if (!z || !codes || !scales) return fail(PALU_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(codes)) return fail(PALU_ERR_INVALID_ARG, "codes must be 16-byte aligned");
  if (z_row_stride > (int64_t)kQuantMaxStrideBytes / (z_dtype == PALU_F32 ? 4 : 2))
    return fail(PALU_ERR_UNSUPPORTED, "z_row_stride above %u bytes", kQuantMaxStrideBytes);
  hipError_t e = launch_quant((int)z_dtype, z, n_rows, r, z_row_stride, codes, scales, stream, true);
  if (e != hipSuccess) return hip_fail(e, "quantiser launch");
  return ok();
}

palu_status palu_dequant_latent(const void* codes, const void* scales, int64_t n_rows, int32_t r,
                                palu_dtype out_dtype, void* out, hipStream_t stream) {
  if (n_rows < 0 || r <= 0) return fail(PALU_ERR_INVALID_ARG, "bad n_rows / r");
  if (out_dtype != PALU_F16 && out_dtype != PALU_BF16) return fail(PALU_ERR_UNSUPPORTED, "out_dtype must be F16 or BF16");
  if (n_rows == 0) return ok();
  if (!codes || !scales || !out) return fail(PALU_ERR_INVALID_ARG, "null pointer");
  if (((uintptr_t)codes & 3u) != 0 || ((uintptr_t)scales & 1u) != 0 || !aligned16(out))
    return fail(PALU_ERR_INVALID_ARG, "codes must be 4-byte, scales 2-byte and out 16-byte aligned");
  const int nch = (r + 31) / 32;
  if (n_rows > INT32_MAX || (uint64_t)n_rows * (uint64_t)nch * (uint64_t)nch >= (1ull << 32))
    return fail(PALU_ERR_UNSUPPORTED, "too many rows for one call");
  DequantParams dp;
  memset(&dp, 0, sizeof(dp));
  DequantSide& sd = dp.side[0];
  sd.codes = (const uint8_t*)codes;
  sd.scales = (const uint8_t*)scales;
  sd.out = (uint8_t*)out;
  sd.nch[0] = nch;
  sd.rank[0] = r;
  sd.magic[0] = (unsigned)(((1ull << 32) + (uint64_t)nch - 1) / (uint64_t)nch);
  dp.seq_lens = nullptr;
  dp.batch = 1; dp.G = 1; dp.max_len = (int)n_rows; dp.max_nch = nch; dp.n_sides = 1;
  hipError_t e = launch_dequant(out_dtype == PALU_F16 ? 1 : 2, dp, stream);
  if (e != hipSuccess) return hip_fail(e, "int4 expansion launch");
  return ok();
}

palu_status palu_project(const palu_attn_desc* desc, const void* x, int32_t d_model, int64_t n_tok, const void* A_kv,
                         const palu_latent_cache* cache, int32_t seq, int32_t pos0, hipStream_t stream) {
  if (!cache) return fail(PALU_ERR_INVALID_ARG, "null pointer");
  const WriteView v{cache->zk, cache->zv, cache->sk, cache->sv, cache->max_len, cache->max_len, nullptr, 0, 0};
  return project_impl(desc, x, d_model, n_tok, A_kv, &v, seq, pos0, stream);
}

palu_status palu_project_paged(const palu_attn_desc* desc, const void* x, int32_t d_model, int64_t n_tok,
                               const void* A_kv, const palu_paged_cache* cache, int32_t seq, int32_t pos0,
                               hipStream_t stream) {
  if (!cache) return fail(PALU_ERR_INVALID_ARG, "null pointer");
  int shift = 0;
  palu_status s = check_paged(cache, &shift);
  if (s != PALU_OK) return s;
  if (n_tok > 0 && !cache->block_table) return fail(PALU_ERR_INVALID_ARG, "block_table is NULL");
  const WriteView v{cache->zk, cache->zv, cache->sk, cache->sv, cache->page_size, cache->max_pages * cache->page_size,
                    cache->block_table, shift, cache->max_pages};
  return project_impl(desc, x, d_model, n_tok, A_kv, &v, seq, pos0, stream);
}

size_t palu_decode_workspace_bytes(const palu_attn_desc* desc, int32_t batch, int32_t max_len) {
  DecodePlan pl;
  if (plan_decode(desc, batch, max_len, &pl) != PALU_OK) return 0;
  return pl.total;
}

palu_status palu_decode_attn(const palu_attn_desc* desc, const void* q, const palu_latent_cache* cache,
                             const void* B_k, const void* B_v, const int32_t* seq_lens, const int32_t* q_pos,
                             int32_t batch, float sm_scale, void* out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (!cache) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
  const CacheView v{cache->zk, cache->zv, cache->sk, cache->sv, cache->max_len, cache->max_len, nullptr, 0, 0};
  return decode_impl(desc, q, &v, B_k, B_v, seq_lens, q_pos, batch, sm_scale, out, workspace, workspace_bytes,
                     stream);
}

palu_status palu_decode_attn_noalloc(const palu_attn_desc* desc, const void* q, const palu_latent_cache* cache,
                                     const void* B_k, const void* B_v, const int32_t* seq_lens, const int32_t* q_pos,
                                     int32_t batch, float sm_scale, void* out, hipStream_t stream) {
  if (!cache) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
  DecodePlan pl;
  palu_status s = plan_decode(desc, batch, cache->max_len, &pl);
  if (s != PALU_OK) return s;
  if (pl.total > PALU_NOALLOC_SCRATCH_BYTES)
    return fail(PALU_ERR_UNSUPPORTED, "this call needs %zu bytes of scratch, above the %zu bytes of the no-alloc entry point",
                pl.total, (size_t)PALU_NOALLOC_SCRATCH_BYTES);
  if (batch == 0) return ok();   // nothing is read or written
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != PALU_OK) return s;
  const CacheView v{cache->zk, cache->zv, cache->sk, cache->sv, cache->max_len, cache->max_len, nullptr, 0, 0};
  return decode_impl(desc, q, &v, B_k, B_v, seq_lens, q_pos, batch, sm_scale, out, ws, PALU_NOALLOC_SCRATCH_BYTES,
                     stream);
}

palu_status palu_decode_attn_paged(const palu_attn_desc* desc, const void* q, const palu_paged_cache* cache,
                                   const void* B_k, const void* B_v, const int32_t* seq_lens,
                                   const int32_t* q_pos, int32_t batch, float sm_scale, void* out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!cache) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
  int shift = 0;
  palu_status s = check_paged(cache, &shift);
  if (s != PALU_OK) return s;
  if (batch > 0 && !cache->block_table) return fail(PALU_ERR_INVALID_ARG, "block_table is NULL");
  const int ps = cache->page_size;
  const CacheView v{cache->zk, cache->zv, cache->sk, cache->sv, ps, cache->max_pages * ps,
                    cache->block_table, shift, cache->max_pages};
  return decode_impl(desc, q, &v, B_k, B_v, seq_lens, q_pos, batch, sm_scale, out, workspace, workspace_bytes,
                     stream);
}

size_t palu_decode_chunk_workspace_bytes(const palu_attn_desc* desc, int32_t batch, int32_t q_len, int32_t max_len,
                                         int32_t max_pages) {
  if (batch < 0 || q_len <= 0 || max_pages < 0) return 0;
  const int64_t vbatch = (int64_t)batch * q_len;
  if (vbatch > kMaxBatch) return 0;
  const size_t d = palu_decode_workspace_bytes(desc, (int32_t)vbatch, max_len);
  return d == 0 ? 0 : d + chunk_front_bytes(vbatch, max_pages > 0 ? max_pages : 1);
}

palu_status palu_decode_attn_chunk(const palu_attn_desc* desc, const void* q, int32_t q_len,
                                   const palu_latent_cache* cache, const void* B_k, const void* B_v,
                                   const int32_t* seq_lens, int32_t batch, float sm_scale, void* out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!cache) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
  if (cache->max_len <= 0) return fail(PALU_ERR_INVALID_ARG, "max_len must be positive");
  // a contiguous cache is a pool of one block per sequence: block b, rows
  // counted from 0 (the shift only has to exceed every row index)
  int shift = 0;
  while ((1 << shift) < cache->max_len) ++shift;
  const CacheView v{cache->zk, cache->zv, cache->sk, cache->sv, cache->max_len, cache->max_len, nullptr, shift, 1};
  return chunk_impl(desc, q, q_len, &v, B_k, B_v, seq_lens, batch, sm_scale, out, workspace, workspace_bytes, stream);
}

palu_status palu_decode_attn_chunk_paged(const palu_attn_desc* desc, const void* q, int32_t q_len,
                                         const palu_paged_cache* cache, const void* B_k, const void* B_v,
                                         const int32_t* seq_lens, int32_t batch, float sm_scale, void* out,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!cache) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
  int shift = 0;
  palu_status s = check_paged(cache, &shift);
  if (s != PALU_OK) return s;
  if (batch > 0 && !cache->block_table) return fail(PALU_ERR_INVALID_ARG, "block_table is NULL");
  const int ps = cache->page_size;
  const CacheView v{cache->zk, cache->zv, cache->sk, cache->sv, ps, cache->max_pages * ps, cache->block_table, shift,
                    cache->max_pages};
  return chunk_impl(desc, q, q_len, &v, B_k, B_v, seq_lens, batch, sm_scale, out, workspace, workspace_bytes, stream);
}

}  // extern "C"
