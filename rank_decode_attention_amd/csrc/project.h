// Host interface of the prefill projection kernel (internal to the library).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace palu {

constexpr int kMaxLatentRows = 32;   // 2 * max groups
constexpr int kMaxColTiles = 256;    // column tiles of <= 160 channels (e.g. 32 latent rows of rank <= 1280)
constexpr int kColTile = 160;        // channels per column tile

struct ProjectParams {
  const void* x;          // [n_tok][D]
  const void* A;          // [n_lat][D]  (A transposed)
  uint8_t* zk; uint8_t* zv; uint8_t* sk; uint8_t* sv;
  int64_t n_tok, d_model, pos0;
  int G, seq, quant;
  int rank[kMaxLatentRows];       // keys of groups 0..G-1 then values
  int64_t col_off[kMaxLatentRows];
  int64_t seq_bytes_k, seq_bytes_v, seq_sbytes_k, seq_sbytes_v;
  int64_t goff_k[kMaxLatentRows / 2], goff_v[kMaxLatentRows / 2];
  int64_t soff_k[kMaxLatentRows / 2], soff_v[kMaxLatentRows / 2];
  int pk[kMaxLatentRows / 2], pv[kMaxLatentRows / 2];
  // paged caches: row t of sequence seq lies in page block_table[seq *
  // max_pages + (t >> page_shift)] (seq_bytes_* are then page sizes and
  // goff_* / soff_* offsets inside a page); NULL for a contiguous cache
  const int* block_table;
  int page_shift, max_pages;
  // column tiles (filled by launch_project): latent row << 16 | first channel
  int ntiles;
  int tile[kMaxColTiles];
};

// dtype: 0 = fp32, 1 = fp16, 2 = bf16 (x, A and non-quantised latents)
// (fills p's column-tile list).  With t0 and t1 set the kernel is launched by
// hipExtLaunchKernel, which records them at its start and end.
hipError_t launch_project(int dtype, ProjectParams& p, hipStream_t stream, hipEvent_t t0 = nullptr,
                          hipEvent_t t1 = nullptr);

}  // namespace palu
