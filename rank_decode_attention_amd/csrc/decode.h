// Host/device interface of the decode kernels (internal to the library).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace palu {

constexpr int kMaxGroups = 16;
constexpr int kMaxBatch = 2048;  // sequences per call (tile prefix sums live in LDS)
constexpr int kDecTile = 32;     // tokens per pipeline tile
constexpr int kDecWaves = 8;     // waves per decode block (2 per SIMD)

// Element types of a decode instantiation.
enum class Elt : int { F32 = 0, F16 = 1, BF16 = 2 };

struct DecodeParams {
  const void* q;            // [batch][H][DH]
  const uint8_t* zk;        // latent buffers (cache layout)
  const uint8_t* zv;
  const void* Bk;           // concatenated B_k^j [r][w]
  const void* Bv;
  const int* seq_lens;      // [batch]
  const int* q_pos;         // [batch] or null
  const float* qabs;        // no-RoPE: [batch][H][qabs_stride] pre-scaled absorbed queries
  int* hdr;                 // workspace: tile_start[batch + 1]
  float* rec;               // workspace: split records
  void* out;                // [batch][H][DH]
  int batch, max_len, H, G;
  int P;                    // blocks per group (the largest Pg: split records are [G][P + batch])
  // blocks of group g and the first block id of its range (the absorbed-query
  // kernel weights them by the group's row bytes; the other kernels use P
  // blocks per group, block id = p * G + g)
  int Pg[kMaxGroups], gblk[kMaxGroups];
  int rec_stride;           // floats per record = NQ * (2 + rvp)
  int rvp;                  // record row length (max value rank rounded up to 16)
  int qabs_stride;
  float qscale;             // sm_scale * log2(e)
  double rope_base;
  int64_t seq_bytes_k, seq_bytes_v;
  int64_t goff_k[kMaxGroups], goff_v[kMaxGroups];   // byte offset of group block inside a sequence block
  int64_t boff_k[kMaxGroups], boff_v[kMaxGroups];   // element offset of B^j inside B_k / B_v
  int rk[kMaxGroups], rv[kMaxGroups];               // ranks
  int pk[kMaxGroups], pv[kMaxGroups];               // row pitches in bytes
  int zero_padded;          // rows hold zeros from the rank up to the next multiple of 32 (int4 copies)
  // int4 caches read directly (MHA kernel): zk / zv hold the codes (pitch
  // pk / pv = 16 bytes per 32 ranks), sk / sv the binary16 scales
  int q4;
  const uint8_t* sk;
  const uint8_t* sv;
  int64_t seq_sbytes_k, seq_sbytes_v;
  int64_t soff_k[kMaxGroups], soff_v[kMaxGroups];
  // paged caches: row t of sequence b lies in page block_table[b * max_pages +
  // (t >> page_shift)] (seq_bytes_* / seq_sbytes_* are then the page sizes and
  // goff_* / soff_* offsets inside a page); NULL for a contiguous cache
  const int* block_table;
  int page_shift, max_pages;
};

// Key of a compiled decode-attention instantiation.
struct DecodeKey {
  Elt elt; int head_dim; int kv_per_group; int q_per_kv; int rk_max; int rv_max; bool rope;
};

// Returns false if no compiled instantiation covers the key (rk_max / rv_max
// are upper bounds that the chosen kernel must reach).
bool decode_supported(const DecodeKey& k, int* rk_cap, int* rv_cap);
// With both events set, the dispatch itself stamps them at the kernel's start and end.
hipError_t launch_decode(const DecodeKey& k, const DecodeParams& p, hipStream_t stream,
                         hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_qabs(const DecodeKey& k, const DecodeParams& p, hipStream_t stream);
// Eight-wave kernel for MHA head-groups of 4 kv heads (head_dim 128, ranks
// <= 256, 16-bit or int4 latents, RoPE; contiguous or paged caches);
// launch_decode uses it where it applies.
bool mha_supported(const DecodeKey& k, const DecodeParams& p);
hipError_t launch_decode_mha(const DecodeKey& k, const DecodeParams& p, hipStream_t stream, hipEvent_t t0,
                             hipEvent_t t1);
// Eight-wave kernel for 16-bit latents without RoPE (absorbed query against
// the latent rows; at most 8 query heads per group, ranks <= 320);
// launch_decode uses it where it applies.
bool abs_supported(const DecodeKey& k, const DecodeParams& p);
hipError_t launch_decode_abs(const DecodeKey& k, const DecodeParams& p, hipStream_t stream, hipEvent_t t0,
                             hipEvent_t t1);
hipError_t launch_merge(const DecodeKey& k, const DecodeParams& p, hipStream_t stream);
// Virtual sequences of a multi-query chunk (see decode.hip): lengths, query
// positions and block-table rows (block_table NULL: row b is block b).
hipError_t launch_chunk_expand(const int* seq_lens, const int* block_table, int batch, int q_len, int max_len,
                               int max_pages, int* vlens, int* vqpos, int* vtable, hipStream_t stream);

}  // namespace palu
