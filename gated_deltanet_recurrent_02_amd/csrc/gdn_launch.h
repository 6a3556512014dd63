// Internal interface between the C-ABI layer (gdn_api.cpp) and the kernels (gdn_kernels.hip).
// Arguments are validated by the caller; the launchers only select a kernel instance and
// enqueue it on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

enum class DType : int { F32 = 0, BF16 = 1, F16 = 2 };

// A dispatch covers fewer than 2^32 work-items. Every decode, verify and fused launch runs at
// most kThreadsPerHeadPerDim * D threads per head (checked where each kernel is instantiated),
// so B * H * 8 * D < 2^32 makes every launch fit.
constexpr int64_t kThreadsPerHeadPerDim = 8;
constexpr int64_t kMaxWorkItems = int64_t(1) << 32;

struct DecodeArgs {
    int64_t B;
    int32_t T, H, D;          // D = dk = dv
    const void* q;            // act [B][T][H][D]
    const void* k;            // act [B][T][H][D]
    const void* v;            // act [B][T][H][D]
    DType act;
    const float* alpha;       // [B][T][H]
    const float* beta;        // [B][T][H]
    void* state;              // state dtype [B][H][D][D]
    DType state_dtype;
    void* o;                  // act [B][T][H][D]
    float scale;
};

struct FusedArgs {
    int64_t B;
    int32_t T, H, D;
    const void* qkv;          // bf16 [B][T][3*H*D]
    void* conv_state;         // bf16 [B][3*H*D][3]
    const float* conv_w;      // [3*H*D][4]
    const float* conv_b;      // [3*H*D] or nullptr
    const float* a_logit;     // [B][T][H]
    const float* b_logit;     // [B][T][H]
    void* state;              // state dtype [B][H][D][D]
    DType state_dtype;
    void* o;                  // bf16 [B][T][H][D]
    float scale;
    float l2_eps;
};

struct VerifyArgs {
    int64_t B;
    int32_t T, H, D;          // T new tokens (may be 0: commit only)
    const void* q;            // act [B][T][H][D]
    const void* k;
    const void* v;
    DType act;
    const float* alpha;       // [B][T][H]
    const float* beta;
    void* state;              // state dtype [B][H][D][D]
    DType state_dtype;
    int32_t Tp;               // tokens of the previous call (0: nothing to commit)
    const int32_t* n_prev;    // [B] accepted prefix of the previous call (device)
    const void* k_prev;       // act [B][Tp][H][D]
    const float* alpha_prev;  // [B][Tp][H]
    const float* dk_prev;     // [B][Tp][H][D] write coefficients emitted by the previous call
    void* o;                  // act [B][T][H][D]
    float* dk_out;            // [B][T][H][D]
    float scale;
};

// All return hipSuccess or the launch error; nothing is synchronised.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
hipError_t launch_conv_gate_decode(const FusedArgs& a, hipStream_t stream);

}  // namespace gdn
