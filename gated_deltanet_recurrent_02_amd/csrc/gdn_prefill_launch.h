// Internal interface between the C-ABI layer (gdn_api.cpp) and the chunked prefill kernels
// (gdn_prefill.hip). Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_launch.h"

namespace gdn {

// Tokens per chunk, and floats per chunk record in the workspace:
//   [0, 256)   T diag(beta): T = (I + A)^-1 of the chunk, columns scaled by beta   [t][s]
//   [256, 512) P: scale * Gam_ts * (q_t . k_s) for s <= t, 0 above the diagonal     [t][s]
//              (bf16 activations: scale * Gam_ts only; the state kernel applies q_t . k_s)
//   [512, 528) gamma_t: alpha_0 ... alpha_t (alpha = 1 past the end of the sequence)
//   [528, 544) Gam_end,t: alpha_{t+1} ... alpha_15
constexpr int kPrefillChunk = 16;
constexpr int kPrefillRecordFloats = 544;

struct PrefillArgs {
    int64_t B;
    int32_t T, H, D;          // D = dk = dv
    const void* q;            // act [B][T][H][D]
    const void* k;
    const void* v;
    DType act;
    const float* alpha;       // [B][T][H]
    const float* beta;
    void* state;              // state dtype [B][H][D][D]
    DType state_dtype;
    void* o;                  // act [B][T][H][D]
    float scale;
    float* ws;                // [B][H][ceil(T/16)][kPrefillRecordFloats]
};

// Chunks per sequence. The prep kernel launches one 64-thread workgroup per (sequence, head,
// chunk), which the caller keeps below 2^32 work-items; the state kernel runs at most 4
// workgroups of 64 threads per head (D / 32 at D >= 32, one at D = 16), within the decode
// bound of 8 D threads per head that the caller checks too.
constexpr int64_t kPrefillWaveThreads = 64;
inline int64_t prefill_chunks(int32_t T) { return (T + kPrefillChunk - 1) / kPrefillChunk; }

// Enqueues the prep kernel, then the state kernel; nothing is synchronised.
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Size of the fixed device scratch of gdn_prefill_noalloc: 64 MiB, i.e. records for
// B * H * ceil(T / 16) <= 30840 (head, chunk) pairs (one 48-head sequence of 10,280 tokens).
constexpr size_t kPrefillScratchBytes = size_t(64) << 20;

// Device address of the current device's copy of that scratch (looked up on the first call on
// each device, cached afterwards; thread-safe). Allocates nothing.
hipError_t prefill_scratch_address(float** out);

}  // namespace gdn
