/*
 * palu.h - C ABI of the Palu latent-cache attention library for MI355X (gfx950).
 *
 * The method (Palu, "KV-Cache Compression with Low-Rank Projection",
 * arXiv 2407.21118; explained on the page "PALU low-rank projection
 * decomposition", section "Low-rank projection decomposition", formula
 * block) factors the key/value projections as W_k ~ A_k B_k, W_v ~ A_v B_v
 * with A in R^{d_model x r} and B in R^{r x d}.  Only the latents
 * z_k = x A_k and z_v = x A_v are cached; keys and values are rebuilt on the
 * fly as K = z_k B_k and V = z_v B_v.  The same page (section "Rollout",
 * engine integration) places the method at three points of a serving engine:
 * the model runner produces the latents (palu_project), the cache manager
 * stores them (the caller-owned buffers described by palu_latent_cache) and
 * the attention kernel consumes them (palu_decode_attn).  Quantization of
 * the latents composes with the low-rank cache (abstract; page section
 * "Rollout", route C): palu_quant_latent.
 *
 * Conventions for every entry point
 *  - Pointers marked "device" point to GPU memory of the current HIP device;
 *    pointers marked "host" point to CPU memory that is read during the call
 *    only and not retained.  The caller allocates and frees every buffer; the
 *    library never allocates device memory.
 *  - Work is enqueued asynchronously on `stream` (NULL = the legacy default
 *    stream).  Argument errors are detected on the host, before anything is
 *    enqueued, and reported synchronously; a failed launch is reported as
 *    PALU_ERR_HIP.  Faults during execution surface at the caller's next
 *    synchronisation.
 *  - Calls are thread-safe; the library keeps no mutable global state other
 *    than a per-thread error message (palu_last_error).
 *  - Device-side preconditions that the host cannot check (values inside
 *    device arrays) are stated per argument; out-of-range sequence lengths
 *    are clamped to [0, max_len] by the kernels.
 *
 * Data formats
 *  - PALU_F32 / PALU_F16 / PALU_BF16: IEEE binary32, binary16, bfloat16.
 *  - PALU_I4 (latents only): symmetric 4-bit codes in [-7, 7] (4-bit two's
 *    complement; element 2i in the low nibble of byte i) with one binary16
 *    scale per 32 consecutive elements of a token's latent row; a latent
 *    value is code * scale.  Rows are padded with zero nibbles to a multiple
 *    of 32 elements.
 *
 * Latent cache layout (one attention layer; keys and values in separate
 * buffers).  For head-group j with rank r_j the row pitch is
 *     F32: 4 * roundup(r_j, 4) bytes, F16/BF16: 2 * roundup(r_j, 8) bytes,
 *     I4: 16 * ceil(r_j / 32) bytes,
 * and the scale-row pitch (I4 only) is 2 * ceil(r_j / 32) bytes.  Buffers are
 * [batch][group j][max_len][pitch_j] with groups of one sequence stored one
 * after another:  offset(b, j, t) = b * max_len * sum_j pitch_j
 *                                 + max_len * sum_{j' < j} pitch_j' + t * pitch_j.
 * palu_latent_bytes / palu_latent_offset compute these.  Pad bytes of a row
 * are not data but must hold finite values (palu_project writes zeros).
 *
 * Factor matrices (row-major):
 *  - A_kv  [sum_j r_k,j + sum_j r_v,j][d_model]: the transpose of
 *    [A_k^0 | .. | A_k^{G-1} | A_v^0 | .. | A_v^{G-1}] (key ranks first), i.e.
 *    the weight layout of a Linear(d_model -> n_lat): row c holds column c of A;
 *  - B_k   concatenation over j of B_k^j [r_k,j][n_g * head_dim] (the
 *    formula's own orientation);
 *  - B_v   concatenation over j of B_v^j [r_v,j][n_g * head_dim];
 *    column block c of B^j belongs to kv head j * n_g + c (n_g = kv heads per
 *    group), i.e. groups hold contiguous kv heads.
 */
#ifndef PALU_H_
#define PALU_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PALU_OK = 0,
  PALU_ERR_INVALID_ARG = 1,          /* null pointer, inconsistent shape, bad value */
  PALU_ERR_UNSUPPORTED = 2,          /* valid but not implemented (shape/dtype combination) */
  PALU_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below palu_decode_workspace_bytes() */
  PALU_ERR_HIP = 4                   /* HIP runtime error while querying the device or launching */
} palu_status;

typedef enum { PALU_F32 = 0, PALU_F16 = 1, PALU_BF16 = 2, PALU_I4 = 3 } palu_dtype;

/* One attention layer.  Host memory; read during a call only. */
typedef struct {
  int32_t n_q_heads;       /* H */
  int32_t n_kv_heads;      /* H_kv; H % H_kv == 0 (query head h reads kv head h / (H/H_kv)) */
  int32_t head_dim;        /* d_h, even */
  int32_t n_groups;        /* G; H_kv % G == 0; group j holds kv heads [j*n_g, (j+1)*n_g) */
  const int32_t* rank_k;   /* host [G]: rank of the key latent of each group, > 0 */
  const int32_t* rank_v;   /* host [G]: rank of the value latent of each group, > 0 */
  int32_t use_rope;        /* 1: rotary embedding on rebuilt keys and on the query; 0: none */
  double rope_base;        /* theta_i = rope_base^(-2i/d_h); pairs (i, i + d_h/2) */
  palu_dtype latent_dtype; /* F32 | F16 | BF16 | I4 */
  palu_dtype act_dtype;    /* q, B_k, B_v, x, A_kv, out: F32 | F16 | BF16 */
} palu_attn_desc;

/* Caller-owned latent cache of one layer.  zk/zv (and sk/sv for I4) are
 * device pointers laid out as described above. */
typedef struct {
  void* zk;                /* device: key latents (codes for I4) */
  void* zv;                /* device: value latents (codes for I4) */
  void* sk;                /* device: I4 key scales (binary16), else NULL */
  void* sv;                /* device: I4 value scales (binary16), else NULL */
  int32_t max_len;         /* tokens per (sequence, group) block, > 0 */
} palu_latent_cache;

/* Caller-owned paged latent cache of one layer (the cache manager's block
 * tables: PALU page, section "Rollout", engine integration - the cache
 * manager stores the latents; paged KV and continuous batching compose with
 * the method).  Each pool is a set of n_pages pages; a page holds page_size
 * consecutive tokens of one sequence for every group, laid out exactly as
 * the contiguous cache above with max_len = page_size and "sequence" = page
 * (so palu_latent_bytes / palu_latent_offset with max_len = page_size give
 * the pool size and the row offsets inside a page).  Token t of sequence b
 * lives in page block_table[b * max_pages + t / page_size], row
 * t % page_size.  Pages may be shared between sequences (read only). */
typedef struct {
  void* zk;                     /* device: key latent page pool (codes for I4) */
  void* zv;                     /* device: value latent page pool */
  void* sk;                     /* device: I4 key scale page pool, else NULL */
  void* sv;                     /* device: I4 value scale page pool, else NULL */
  const int32_t* block_table;   /* device int32 [batch][max_pages]: page index, in [0, n_pages) for
                                   every page a sequence's history reaches */
  int32_t page_size;            /* tokens per page: a power of two, >= 32 */
  int32_t max_pages;            /* block_table row length; histories are at most max_pages * page_size */
  int32_t n_pages;              /* pages in each pool */
} palu_paged_cache;

/* Human-readable name of a status code (static string). */
const char* palu_status_string(palu_status s);

/* Detail of the last error returned on the calling thread (static per-thread
 * buffer; empty string if none). */
const char* palu_last_error(void);

/* Bytes of one latent buffer of the layout above.  which: 0 = keys, 1 = values.
 * scales: 0 = the latent (code) buffer, 1 = the I4 scale buffer.
 * Returns 0 for an invalid descriptor. */
size_t palu_latent_bytes(const palu_attn_desc* desc, int32_t batch, int32_t max_len,
                         int32_t which, int32_t scales);

/* Byte offset of row t of (sequence b, group j) in a latent (scales = 0) or
 * scale (scales = 1) buffer.  Returns -1 for invalid arguments. */
int64_t palu_latent_offset(const palu_attn_desc* desc, int32_t max_len, int32_t which,
                           int32_t scales, int32_t b, int32_t j, int32_t t);

/*
 * palu_quant_latent - symmetric int4 quantisation of latent rows
 * (quantization composing with the low-rank cache: arXiv 2407.21118v2
 * abstract; PALU page, section "Rollout", route C).
 *   z        device [n_rows] rows of r values of z_dtype (F32 | F16 | BF16),
 *            row i starting at element i * z_row_stride (z_row_stride >= r)
 *   codes    device [n_rows][16 * ceil(r/32)] bytes (output)
 *   scales   device [n_rows][ceil(r/32)] binary16 (output)
 * Per 32-element chunk: s = fp16(amax / 7) (binary32 divide, round to
 * nearest even), code = clamp(rint(z / s), -7, 7) in binary32 with ties to
 * even, code = 0 where s == 0.  Pad nibbles are written as zero.
 * n_rows == 0 is a no-op after the argument checks (pointers may be NULL).
 * Errors: INVALID_ARG for null pointers, n_rows < 0, r <= 0, z_row_stride < r,
 * codes not 16-byte aligned; UNSUPPORTED for z_dtype == I4 and for rows
 * more than 64 MiB apart (z_row_stride times the element size).
 */
palu_status palu_quant_latent(const void* z, palu_dtype z_dtype, int64_t n_rows, int32_t r,
                              int64_t z_row_stride, void* codes, void* scales, hipStream_t stream);

/*
 * palu_quant_latent_rotated - low-rank-aware int4 quantisation (arXiv
 * 2407.21118v2 abstract: a low-rank-aware quantization enhancement; PALU
 * page, section "Rollout", route C: quantization on top of the low-rank
 * cache).  The pages do not define the enhancement; this library's reading:
 * latents of an SVD-style factorisation carry very unequal energy per
 * channel, and a chunk's amax/7 step is set by its largest channel, so
 * every full 32-element chunk is first rotated by the Sylvester Hadamard
 * matrix H of order 32 (entries +-1, H H^T = 32 I), which spreads a chunk's
 * energy over all its elements: the row z becomes z' = z H chunk by chunk
 * (a trailing partial chunk is left as is), and z' is quantised exactly as
 * by palu_quant_latent.  The rotation is undone in the factors, not in the
 * decode: with A' = A H and B' = H B / 32 per full 32-row block (identity
 * on a partial block), z' B' = z B, so palu_decode_attn over the rotated
 * int4 cache with B_k', B_v' attends as over the unrotated latents; a prefill
 * through palu_project with A' writes z' directly (then use
 * palu_quant_latent, or an I4 cache, on it).  z H is formed in binary32 by
 * the fast Walsh-Hadamard butterflies (stages h = 1, 2, 4, 8, 16; the pair
 * (i, i + h) becomes (a + b, a - b)); codes and scales are then decided as in
 * palu_quant_latent.
 * Arguments, layouts and errors: as palu_quant_latent.
 */
palu_status palu_quant_latent_rotated(const void* z, palu_dtype z_dtype, int64_t n_rows, int32_t r,
                                      int64_t z_row_stride, void* codes, void* scales, hipStream_t stream);

/*
 * palu_dequant_latent - int4 latent rows to 16-bit rows (quantization on top
 * of the low-rank cache: PALU page, section "Rollout", route C), for callers
 * that want a 16-bit copy of an int4 cache.  The values are rounded to the
 * 16-bit format; palu_decode_attn does not use this rounding (it attends over
 * the exact code * scale).
 *   codes    device [n_rows][16 * ceil(r/32)] bytes (layout of PALU_I4 above)
 *   scales   device [n_rows][ceil(r/32)] binary16
 *   out      device [n_rows][32 * ceil(r/32)] out_dtype (output): element e of
 *            row i is code * scale of its 32-element chunk, formed exactly in
 *            binary32 and rounded to nearest even into out_dtype, for e < r;
 *            0 for r <= e < 32 * ceil(r/32) (pad nibbles are not read as data)
 * n_rows == 0 is a no-op after the argument checks (pointers may be NULL).
 * Errors: INVALID_ARG for null pointers, n_rows < 0, r <= 0, codes not
 * 4-byte, scales not 2-byte or out not 16-byte aligned; UNSUPPORTED for
 * out_dtype other than F16 / BF16, or n_rows * ceil(r/32)^2 >= 2^32.
 */
palu_status palu_dequant_latent(const void* codes, const void* scales, int64_t n_rows, int32_t r,
                                palu_dtype out_dtype, void* out, hipStream_t stream);

/*
 * palu_project - prefill: write the latents of n_tok new tokens of sequence
 * `seq` (PALU page, section "Inference flow", prefill steps 3-4: compute
 * z_k = x A_k, z_v = x A_v and cache them instead of K/V).
 *   x        device [n_tok][d_model] act_dtype
 *   A_kv     device [sum r_k + sum r_v][d_model] act_dtype (layout above)
 *   cache    latent buffers (host struct, device pointers); rows
 *            pos0 .. pos0 + n_tok - 1 of every group of sequence `seq` are
 *            written (int4 quantised when latent_dtype == I4, else rounded to
 *            nearest even from the fp32 accumulation).
 * Row padding of F32/F16/BF16 latents is written as zero; I4 pad nibbles are
 * zero.  Rows of other sequences or positions are not touched.
 * Errors: INVALID_ARG for null pointers, d_model <= 0, n_tok < 0, seq < 0,
 * pos0 < 0, pos0 + n_tok > max_len, misaligned buffers (x, A_kv and latent
 * buffers must be 16-byte aligned); UNSUPPORTED when latent_dtype is neither
 * act_dtype nor I4, d_model is not a multiple of 64, the latent rows need more
 * than 256 column tiles of 160 channels (sum over rows of ceil(rank / 160)),
 * or A_kv exceeds 4 GiB.
 */
palu_status palu_project(const palu_attn_desc* desc, const void* x, int32_t d_model, int64_t n_tok,
                         const void* A_kv, const palu_latent_cache* cache, int32_t seq, int32_t pos0,
                         hipStream_t stream);

/*
 * palu_project_paged - palu_project into a paged cache: the latents of the
 * n_tok tokens pos0 .. pos0 + n_tok - 1 of sequence `seq` are written to row
 * t % page_size of page block_table[seq * max_pages + t / page_size]; every
 * page these positions reach must be assigned (seq indexes the block table's
 * rows).  Same arithmetic and row contents as palu_project.
 * Errors: as palu_project (with max_len = max_pages * page_size), plus
 * INVALID_ARG for a NULL block_table (n_tok > 0), page_size not a power of
 * two >= 32, max_pages <= 0 or n_pages <= 0.
 */
palu_status palu_project_paged(const palu_attn_desc* desc, const void* x, int32_t d_model, int64_t n_tok,
                               const void* A_kv, const palu_paged_cache* cache, int32_t seq, int32_t pos0,
                               hipStream_t stream);

/* Workspace bytes palu_decode_attn needs for `batch` sequences on the
 * current device (0 for an invalid descriptor). */
size_t palu_decode_workspace_bytes(const palu_attn_desc* desc, int32_t batch, int32_t max_len);

/*
 * palu_decode_attn - one decode step of attention over the latent cache
 * (PALU page, section "Inference flow", decode steps 1-3; section "Why the
 * GPU kernel matters": the rebuild is fused into the attention kernel so that
 * full K and V are never materialised).  For every sequence b and query head
 * h (kv head c = h / (H/H_kv), group j = c / n_g):
 *   K = z_k^j[0:L_b] B_k^j, V = z_v^j[0:L_b] B_v^j (columns of kv head c);
 *   with use_rope, K rows are rotated by their cache index t and q_h by p_b;
 *   out[b][h] = softmax(sm_scale * K q_h) V.
 * Without RoPE the score uses the absorbed query (q_h B_k^T) against z_k and,
 * in all cases, values enter as (softmax . z_v) . B_v; both equal the formula
 * up to rounding.  Arithmetic is binary32 throughout.
 * I4 latents (act_dtype F16 or BF16): the decode attends over the
 * dequantised latent code * scale (PALU page, section "Rollout", route C:
 * quantization on top of the low-rank cache) exactly, never rounded to a
 * 16-bit format.  On MHA head-group shapes (4 kv heads per group, one query
 * head each, head_dim 128, RoPE, ranks <= 256) the decode kernel feeds the
 * codes to the matrix units as exact integers and applies each 32-element
 * chunk's scale afterwards (to the chunk's partial key product, and to the
 * attention weights before they meet the value codes); with F16 activations
 * the scaled weights must stay in the binary16 range, which holds for scales
 * up to 255 (latent magnitudes up to ~1785).  On other shapes the rows
 * [0, L_b) of every sequence are first expanded into the workspace as exact
 * hi + lo pairs of 16-bit values (each 32-element chunk becomes 64 values,
 * rank r -> 64 ceil(r/32)) and attended against B_k / B_v with every row
 * duplicated to match; that doubled rank must fit a decode kernel (no RoPE:
 * up to 320; GQA groups of 2 kv heads with RoPE: up to 320; else UNSUPPORTED).
 *   q          device [batch][H][d_h] act_dtype
 *   cache      latent buffers; rows [0, L_b) of each (b, j) are read
 *   B_k, B_v   device, layout above, act_dtype
 *   seq_lens   device int32 [batch]: L_b (clamped to [0, max_len]); L_b == 0
 *              gives a zero output row
 *   q_pos      device int32 [batch]: RoPE position of the query, or NULL for
 *              L_b - 1 (the new token's latent already appended)
 *   sm_scale   score scale, typically 1/sqrt(d_h); finite
 *   out        device [batch][H][d_h] act_dtype
 *   workspace  device, at least palu_decode_workspace_bytes(desc, batch,
 *              cache->max_len) bytes, 256-byte aligned; contents are scratch
 *              (for I4 on shapes expanded into the workspace it includes
 *              batch * max_len * sum_j 4 * (ceil32(r_k^j) + ceil32(r_v^j))
 *              bytes of hi/lo latents and the duplicated factors)
 * batch == 0 is a no-op after the descriptor checks (pointers may be NULL).
 * Errors: INVALID_ARG for null pointers, batch < 0, head counts that do not
 * divide, odd head_dim, rank <= 0, max_len <= 0, non-finite sm_scale,
 * I4 scales missing or not 2-byte aligned; WORKSPACE_TOO_SMALL; UNSUPPORTED for shapes without a
 * compiled kernel (palu_last_error names the reason).
 */
palu_status palu_decode_attn(const palu_attn_desc* desc, const void* q, const palu_latent_cache* cache,
                             const void* B_k, const void* B_v, const int32_t* seq_lens,
                             const int32_t* q_pos, int32_t batch, float sm_scale, void* out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the device scratch array behind palu_decode_attn_noalloc (one
 * per GPU the library runs on, held until the process ends). */
#define PALU_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * palu_decode_attn_noalloc - palu_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation, kernels and
 * results as palu_decode_attn on a contiguous cache, with the workspace
 * taken from a library-owned static device array of
 * PALU_NOALLOC_SCRATCH_BYTES instead of an argument.  It calls no hipMalloc,
 * hipFree or other allocating routine; its first call on a device resolves
 * that device's copy of the array (hipGetSymbolAddress).
 *   arguments  as palu_decode_attn, without workspace / workspace_bytes
 * No part of the scratch needs to start at zero: every call writes what it
 * reads.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind, so calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 * Errors: as palu_decode_attn, plus UNSUPPORTED when the call needs more
 * than PALU_NOALLOC_SCRATCH_BYTES of workspace (palu_decode_workspace_bytes
 * tells; e.g. I4 caches on shapes that are expanded into the workspace).
 */
palu_status palu_decode_attn_noalloc(const palu_attn_desc* desc, const void* q, const palu_latent_cache* cache,
                                     const void* B_k, const void* B_v, const int32_t* seq_lens,
                                     const int32_t* q_pos, int32_t batch, float sm_scale, void* out,
                                     hipStream_t stream);

/*
 * palu_decode_attn_paged - palu_decode_attn over a paged latent cache: the
 * same computation and results, with row t of sequence b read from page
 * block_table[b * max_pages + t / page_size] (see palu_paged_cache).
 * seq_lens are clamped to [0, max_pages * page_size]; the workspace is
 * palu_decode_workspace_bytes(desc, batch, max_pages * page_size) bytes.
 * Errors: as palu_decode_attn, plus INVALID_ARG for a NULL block_table,
 * page_size not a power of two >= 32, max_pages <= 0 or n_pages <= 0;
 * UNSUPPORTED for I4 pools on shapes other than MHA head-groups of 4 kv
 * heads with head_dim 128 and RoPE.
 */
palu_status palu_decode_attn_paged(const palu_attn_desc* desc, const void* q, const palu_paged_cache* cache,
                                   const void* B_k, const void* B_v, const int32_t* seq_lens,
                                   const int32_t* q_pos, int32_t batch, float sm_scale, void* out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * palu_decode_attn_chunk - attention of q_len new tokens per sequence (a
 * prefill chunk, or tokens to verify) over the latent cache, causal within
 * the chunk: the same computation as palu_decode_attn for every query, with
 * query i of sequence b at position p = L_b - q_len + i attending to the
 * cached tokens 0 .. p (their latents, including the chunk's own, already
 * written; RoPE position p).  p < 0 gives a zero output row.
 *   q, out     device [batch][q_len][H][d_h] act_dtype
 *   seq_lens   device int32 [batch]: L_b, clamped to [0, max_len]
 *   workspace  palu_decode_chunk_workspace_bytes(desc, batch, q_len, max_len, 1) bytes
 * The queries run as batch * q_len decode sequences that share their
 * sequence's latents (batch * q_len <= 2048).  Errors: as palu_decode_attn,
 * plus INVALID_ARG for q_len <= 0; UNSUPPORTED for batch * q_len > 2048 and
 * for I4 caches on shapes other than MHA head-groups of 4 kv heads with
 * head_dim 128 and RoPE.
 */
palu_status palu_decode_attn_chunk(const palu_attn_desc* desc, const void* q, int32_t q_len,
                                   const palu_latent_cache* cache, const void* B_k, const void* B_v,
                                   const int32_t* seq_lens, int32_t batch, float sm_scale, void* out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same over a paged cache; workspace:
 * palu_decode_chunk_workspace_bytes(desc, batch, q_len, max_pages * page_size, max_pages). */
palu_status palu_decode_attn_chunk_paged(const palu_attn_desc* desc, const void* q, int32_t q_len,
                                         const palu_paged_cache* cache, const void* B_k, const void* B_v,
                                         const int32_t* seq_lens, int32_t batch, float sm_scale, void* out,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of a chunk call (max_pages: 1 for a contiguous cache);
 * 0 for invalid arguments. */
size_t palu_decode_chunk_workspace_bytes(const palu_attn_desc* desc, int32_t batch, int32_t q_len, int32_t max_len,
                                         int32_t max_pages);

/*
 * palu_profile_events - timing hook for benchmark harnesses (not part of the
 * method).  When both are set (non-NULL), every later palu_decode_attn call
 * on the calling thread launches its main decode kernel (the one that reads
 * the latent cache, before the merge), and every later palu_project call its
 * projection kernel, with
 * hipExtLaunchKernel, which stamps `before_main` at the kernel's start and
 * `after_main` at its end, so that hipEventElapsedTime gives that kernel's
 * duration.  The caller owns the events (hipEventCreate) and must keep them
 * alive while set; pass NULL, NULL to stop.  Thread-local; never fails.
 */
palu_status palu_profile_events(hipEvent_t before_main, hipEvent_t after_main);

#ifdef __cplusplus
}
#endif
#endif /* PALU_H_ */
