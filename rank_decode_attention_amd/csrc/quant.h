// Host interface of the int4 latent quantiser (internal to the library).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace palu {
// dtype: 0 = fp32, 1 = fp16, 2 = bf16 input rows
hipError_t launch_quant(int dtype, const void* z, int64_t n_rows, int r, int64_t stride, void* codes,
                        void* scales, hipStream_t stream);
}  // namespace palu
