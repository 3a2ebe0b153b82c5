// Host interface of the int4 latent quantiser (internal to the library).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace palu {
// dtype: 0 = fp32, 1 = fp16, 2 = bf16 input rows
hipError_t launch_quant(int dtype, const void* z, int64_t n_rows, int r, int64_t stride, void* codes,
                        void* scales, hipStream_t stream);

// Expansion of one layer's int4 latent cache (keys and values) into 16-bit
// rows for the decode kernels: row t of (sequence b, group j) becomes
// 32 * nch[j] values code * scale (exact in fp32, then rounded to the
// activation format), zero from the rank on; rows at or past the sequence's
// history length are not written.  Layouts: [batch][group][max_len][row],
// group blocks at goff_*.
constexpr int kDqMaxGroups = 16;
struct DequantSide {
  const uint8_t* codes;     // int4 rows (16 bytes per 32 elements)
  const uint8_t* scales;    // binary16 rows (2 bytes per 32 elements)
  uint8_t* out;             // 16-bit rows (64 bytes per 32 elements)
  int64_t seq_c, seq_s, seq_o;   // bytes of one sequence block
  int64_t goff_c[kDqMaxGroups], goff_s[kDqMaxGroups], goff_o[kDqMaxGroups];
  int nch[kDqMaxGroups];    // 32-element chunks per row
  int rank[kDqMaxGroups];   // elements past the rank are written as zero
  unsigned magic[kDqMaxGroups];   // ceil(2^32 / nch): c / nch = umulhi(c, magic) for c < max_len * nch
};
struct DequantParams {
  DequantSide side[2];      // keys, values
  const int* seq_lens;      // device [batch], clamped to [0, max_len]; NULL: every length is max_len
  int batch, G, max_len, max_nch;   // (max_len * max_nch^2 < 2^32)
  int n_sides;              // 2: keys and values; 1: side[0] only
};
// out_dtype: 1 = fp16, 2 = bf16
hipError_t launch_dequant(int out_dtype, const DequantParams& p, hipStream_t stream);
}  // namespace palu
