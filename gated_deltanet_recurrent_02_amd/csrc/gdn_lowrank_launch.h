// Internal interface between the C-ABI layer (gdn_api.cpp) and the sliding-window low-rank
// kernel (gdn_lowrank.hip). Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_launch.h"

namespace gdn {

// At most D / 32 wave64s per (sequence, head) (one below D = 64, at most four): at most 2 * D
// work-items per head, within the decode bound of 8 * D threads per head that the caller
// checks.

struct LowrankArgs {
    int64_t B;
    int32_t T, H, D;          // D = dk = dv
    int32_t R;                // window length (slots): 8, 16 or 32
    const void* q;            // act [B][T][H][D]
    const void* k;
    const void* v;
    DType act;
    const float* alpha;       // [B][T][H]
    const float* beta;
    void* U;                  // state dtype [B][H][R][D]  write vectors
    void* K;                  // state dtype [B][H][R][D]  keys
    DType state_dtype;
    float* c;                 // [B][H][R] weights
    int32_t* pos;             // [B][H] next slot (taken modulo R)
    void* o;                  // act [B][T][H][D]
    float scale;
};

inline bool lowrank_supported_r(int32_t r) { return r == 8 || r == 16 || r == 32; }

hipError_t launch_lowrank(const LowrankArgs& a, hipStream_t stream);

}  // namespace gdn
