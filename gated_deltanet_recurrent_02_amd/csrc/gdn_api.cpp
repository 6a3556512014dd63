// C-ABI entry points of libgdn.so (declared in include/gdn.h): host-side validation, then a
// kernel launch on the caller's stream. Nothing here synchronises or allocates except
// gdn_state_alloc / gdn_state_free.

#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "gdn_launch.h"
#include "gdn_lowrank_launch.h"
#include "gdn_prefill_launch.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

gdn_status fail_hip(const char* what, hipError_t e) {
    g_last_error = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
    return GDN_ERR_HIP;
}

bool supported_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool valid_dtype(gdn_dtype t) { return t == GDN_F32 || t == GDN_BF16 || t == GDN_F16; }
size_t dtype_bytes(gdn_dtype t) { return t == GDN_F32 ? 4 : 2; }
gdn::DType to_dtype(gdn_dtype t) {
    return t == GDN_F32 ? gdn::DType::F32 : (t == GDN_BF16 ? gdn::DType::BF16 : gdn::DType::F16);
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b with overflow detection on size_t.
bool mul_ok(size_t a, size_t b, size_t* out) { return !__builtin_mul_overflow(a, b, out); }

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* p, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, lo + bytes};
}

bool overlaps(const Range& a, const Range& b) {
    return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

// Shape checks shared by the two step functions. Returns GDN_OK, or a failure with message.
gdn_status check_shape(const char* fn, int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv) {
    if (B < 0 || T < 0) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": B and T must be >= 0");
    if (H < 1) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": H must be >= 1");
    if (dk < 1 || dv < 1) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": dk and dv must be >= 1");
    if (dk != dv || !supported_dim(dk))
        return fail(GDN_ERR_UNSUPPORTED,
                    std::string(fn) + ": supported head dims are dk == dv in {16, 32, 64, 128}, got dk=" +
                        std::to_string(dk) + " dv=" + std::to_string(dv));
    if (B * (int64_t)H >= (int64_t(1) << 31))
        return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": B * H must be < 2^31");
    if (B * (int64_t)H * gdn::kThreadsPerHeadPerDim * dk >= gdn::kMaxWorkItems)
        return fail(GDN_ERR_UNSUPPORTED, std::string(fn) + ": B * H * 8 * dk must be < 2^32 (one dispatch)");
    return GDN_OK;
}

gdn_status check_ptrs(const char* fn, std::initializer_list<std::pair<const char*, const void*>> ps) {
    for (auto& p : ps) {
        if (p.second == nullptr)
            return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": " + p.first + " is NULL");
        if (!aligned16(p.second))
            return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": " + p.first + " is not 16-byte aligned");
    }
    return GDN_OK;
}

gdn_status check_disjoint(const char* fn, const Range& out, std::initializer_list<Range> others) {
    for (auto& r : others)
        if (overlaps(out, r))
            return fail(GDN_ERR_INVALID_ARGUMENT,
                        std::string(fn) + ": " + out.name + " overlaps " + r.name);
    return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
        case GDN_ERR_OUT_OF_MEMORY: return "GDN_ERR_OUT_OF_MEMORY";
        case GDN_ERR_HIP: return "GDN_ERR_HIP";
    }
    return "unknown";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

gdn_status gdn_state_alloc(int64_t B, int32_t H, int32_t dk, int32_t dv, gdn_dtype state_dtype,
                           void** state_out, size_t* bytes_out) {
    g_last_error.clear();
    if (!state_out) return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_state_alloc: state_out is NULL");
    *state_out = nullptr;
    if (B < 1 || H < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_state_alloc: B and H must be >= 1");
    if (!valid_dtype(state_dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_state_alloc: bad state_dtype");
    if (dk != dv || !supported_dim(dk))
        return fail(GDN_ERR_UNSUPPORTED, "gdn_state_alloc: supported head dims are dk == dv in {16, 32, 64, 128}");
    size_t bytes = 0;
    if (!mul_ok((size_t)B, (size_t)H, &bytes) || !mul_ok(bytes, (size_t)dk * dv, &bytes) ||
        !mul_ok(bytes, dtype_bytes(state_dtype), &bytes))
        return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_state_alloc: size overflows");
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, bytes);
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) {
        (void)hipGetLastError();
        return fail(GDN_ERR_OUT_OF_MEMORY, "gdn_state_alloc: hipMalloc of " + std::to_string(bytes) +
                                               " bytes failed: " + hipGetErrorString(e));
    }
    if (e != hipSuccess) return fail_hip("gdn_state_alloc: hipMalloc", e);
    e = hipMemset(p, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(p);
        return fail_hip("gdn_state_alloc: zero fill", e);
    }
    *state_out = p;
    if (bytes_out) *bytes_out = bytes;
    return GDN_OK;
}

gdn_status gdn_state_free(void* state) {
    g_last_error.clear();
    if (!state) return GDN_OK;
    hipError_t e = hipFree(state);
    if (e != hipSuccess) return fail_hip("gdn_state_free: hipFree", e);
    return GDN_OK;
}

gdn_status gdn_decode_step(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                           const void* q, const void* k, const void* v, gdn_dtype act_dtype,
                           const float* alpha, const float* beta,
                           void* state, gdn_dtype state_dtype,
                           void* o, float scale, void* stream) {
    static const char* fn = "gdn_decode_step";
    g_last_error.clear();
    gdn_status s = check_shape(fn, B, T, H, dk, dv);
    if (s != GDN_OK) return s;
    if (!valid_dtype(act_dtype) || !valid_dtype(state_dtype))
        return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": bad dtype");
    if (B == 0 || T == 0) return GDN_OK;
    s = check_ptrs(fn, {{"q", q}, {"k", k}, {"v", v}, {"alpha", alpha}, {"beta", beta},
                        {"state", state}, {"o", o}});
    if (s != GDN_OK) return s;
    const size_t tokens = (size_t)B * T * H;
    const size_t ab = dtype_bytes(act_dtype);
    const size_t state_bytes = (size_t)B * H * dk * dv * dtype_bytes(state_dtype);
    Range ro = range("o", o, tokens * dv * ab);
    s = check_disjoint(fn, ro, {range("q", q, tokens * dk * ab), range("k", k, tokens * dk * ab),
                                range("v", v, tokens * dv * ab), range("alpha", alpha, tokens * 4),
                                range("beta", beta, tokens * 4), range("state", state, state_bytes)});
    if (s != GDN_OK) return s;
    Range rs = range("state", state, state_bytes);
    s = check_disjoint(fn, rs, {range("q", q, tokens * dk * ab), range("k", k, tokens * dk * ab),
                                range("v", v, tokens * dv * ab), range("alpha", alpha, tokens * 4),
                                range("beta", beta, tokens * 4)});
    if (s != GDN_OK) return s;

    gdn::DecodeArgs a;
    a.B = B; a.T = T; a.H = H; a.D = dk;
    a.q = q; a.k = k; a.v = v;
    a.act = to_dtype(act_dtype);
    a.alpha = alpha; a.beta = beta;
    a.state = state;
    a.state_dtype = to_dtype(state_dtype);
    a.o = o; a.scale = scale;
    hipError_t e = gdn::launch_decode(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip("gdn_decode_step: kernel launch", e);
    return GDN_OK;
}

gdn_status gdn_decode_verify(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                             const void* q, const void* k, const void* v, gdn_dtype act_dtype,
                             const float* alpha, const float* beta,
                             void* state, gdn_dtype state_dtype,
                             int32_t Tp, const int32_t* n_prev, const void* k_prev,
                             const float* alpha_prev, const float* dk_prev,
                             void* o, float* dk_out, float scale, void* stream) {
    static const char* fn = "gdn_decode_verify";
    g_last_error.clear();
    gdn_status s = check_shape(fn, B, T, H, dk, dv);
    if (s != GDN_OK) return s;
    if (Tp < 0) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": Tp must be >= 0");
    if (!valid_dtype(act_dtype) || !valid_dtype(state_dtype))
        return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": bad dtype");
    if (B == 0 || (T == 0 && Tp == 0)) return GDN_OK;
    s = check_ptrs(fn, {{"state", state}});
    if (s != GDN_OK) return s;
    if (T > 0) {
        s = check_ptrs(fn, {{"q", q}, {"k", k}, {"v", v}, {"alpha", alpha}, {"beta", beta},
                            {"o", o}, {"dk_out", dk_out}});
        if (s != GDN_OK) return s;
    }
    if (Tp > 0) {
        s = check_ptrs(fn, {{"n_prev", n_prev}, {"k_prev", k_prev}, {"alpha_prev", alpha_prev},
                            {"dk_prev", dk_prev}});
        if (s != GDN_OK) return s;
    }
    const size_t ab = dtype_bytes(act_dtype);
    const size_t tok = (size_t)B * T * H, tokp = (size_t)B * Tp * H;
    const size_t state_bytes = (size_t)B * H * dk * dv * dtype_bytes(state_dtype);
    const Range r_s = range("state", state, state_bytes);
    const Range r_q = range("q", q, tok * dk * ab), r_k = range("k", k, tok * dk * ab);
    const Range r_v = range("v", v, tok * dv * ab), r_a = range("alpha", alpha, tok * 4);
    const Range r_b = range("beta", beta, tok * 4), r_o = range("o", o, tok * dv * ab);
    const Range r_d = range("dk_out", dk_out, tok * dv * 4);
    const Range r_n = range("n_prev", n_prev, Tp > 0 ? (size_t)B * 4 : 0);
    const Range r_kp = range("k_prev", k_prev, tokp * dk * ab);
    const Range r_ap = range("alpha_prev", alpha_prev, tokp * 4);
    const Range r_dp = range("dk_prev", dk_prev, tokp * dv * 4);
    s = check_disjoint(fn, r_o, {r_s, r_q, r_k, r_v, r_a, r_b, r_d, r_n, r_kp, r_ap, r_dp});
    if (s != GDN_OK) return s;
    s = check_disjoint(fn, r_d, {r_s, r_q, r_k, r_v, r_a, r_b, r_n, r_kp, r_ap, r_dp});
    if (s != GDN_OK) return s;
    s = check_disjoint(fn, r_s, {r_q, r_k, r_v, r_a, r_b, r_n, r_kp, r_ap, r_dp});
    if (s != GDN_OK) return s;

    gdn::VerifyArgs a;
    a.B = B; a.T = T; a.H = H; a.D = dk;
    a.q = q; a.k = k; a.v = v; a.act = to_dtype(act_dtype);
    a.alpha = alpha; a.beta = beta;
    a.state = state; a.state_dtype = to_dtype(state_dtype);
    a.Tp = Tp; a.n_prev = n_prev; a.k_prev = k_prev; a.alpha_prev = alpha_prev; a.dk_prev = dk_prev;
    a.o = o; a.dk_out = dk_out; a.scale = scale;
    hipError_t e = gdn::launch_verify(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip("gdn_decode_verify: kernel launch", e);
    return GDN_OK;
}

gdn_status gdn_conv_gate_decode(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                const void* qkv, void* conv_state,
                                const float* conv_w, const float* conv_b,
                                const float* a_logit, const float* b_logit,
                                void* state, gdn_dtype state_dtype,
                                void* o, float scale, float l2_eps, void* stream) {
    static const char* fn = "gdn_conv_gate_decode";
    g_last_error.clear();
    gdn_status s = check_shape(fn, B, T, H, dk, dv);
    if (s != GDN_OK) return s;
    if (!valid_dtype(state_dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": bad dtype");
    if (!(l2_eps >= 0.0f)) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": l2_eps must be >= 0");
    if (B == 0 || T == 0) return GDN_OK;
    s = check_ptrs(fn, {{"qkv", qkv}, {"conv_state", conv_state}, {"conv_w", conv_w},
                        {"a_logit", a_logit}, {"b_logit", b_logit}, {"state", state}, {"o", o}});
    if (s != GDN_OK) return s;
    if (conv_b && !aligned16(conv_b))
        return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": conv_b is not 16-byte aligned");
    const size_t C = (size_t)H * (dk + dk + dv);
    const size_t tokens = (size_t)B * T * H;
    const size_t state_bytes = (size_t)B * H * dk * dv * dtype_bytes(state_dtype);
    const Range r_qkv = range("qkv", qkv, (size_t)B * T * C * 2);
    const Range r_cs = range("conv_state", conv_state, (size_t)B * C * 3 * 2);
    const Range r_w = range("conv_w", conv_w, C * 16);
    const Range r_b = range("conv_b", conv_b, conv_b ? C * 4 : 0);
    const Range r_a = range("a_logit", a_logit, tokens * 4);
    const Range r_bl = range("b_logit", b_logit, tokens * 4);
    const Range r_s = range("state", state, state_bytes);
    const Range r_o = range("o", o, tokens * dv * 2);
    s = check_disjoint(fn, r_o, {r_qkv, r_cs, r_w, r_b, r_a, r_bl, r_s});
    if (s != GDN_OK) return s;
    s = check_disjoint(fn, r_cs, {r_qkv, r_w, r_b, r_a, r_bl, r_s});
    if (s != GDN_OK) return s;
    s = check_disjoint(fn, r_s, {r_qkv, r_w, r_b, r_a, r_bl});
    if (s != GDN_OK) return s;

    gdn::FusedArgs a;
    a.B = B; a.T = T; a.H = H; a.D = dk;
    a.qkv = qkv; a.conv_state = conv_state; a.conv_w = conv_w; a.conv_b = conv_b;
    a.a_logit = a_logit; a.b_logit = b_logit;
    a.state = state;
    a.state_dtype = to_dtype(state_dtype);
    a.o = o; a.scale = scale; a.l2_eps = l2_eps;
    hipError_t e = gdn::launch_conv_gate_decode(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip("gdn_conv_gate_decode: kernel launch", e);
    return GDN_OK;
}

}  // extern "C"

namespace {

// Workspace bytes of gdn_prefill; false if the size overflows size_t.
bool prefill_ws_bytes(int64_t B, int32_t T, int32_t H, size_t* out) {
    size_t n = 0;
    return mul_ok((size_t)B, (size_t)H, &n) && mul_ok(n, (size_t)gdn::prefill_chunks(T), &n) &&
           mul_ok(n, (size_t)gdn::kPrefillRecordFloats * sizeof(float), out);
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_workspace_size(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                      size_t* bytes) {
    static const char* fn = "gdn_prefill_workspace_size";
    g_last_error.clear();
    if (!bytes) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": bytes is NULL");
    *bytes = 0;
    gdn_status s = check_shape(fn, B, T, H, dk, dv);
    if (s != GDN_OK) return s;
    if (!prefill_ws_bytes(B, T, H, bytes)) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": size overflows");
    return GDN_OK;
}

}  // extern "C"

namespace {

// gdn_prefill and gdn_prefill_noalloc: validation, then the launch with the given workspace.
// `workspace` NULL means the library's fixed device scratch (no allocation, no caller buffer).
// Prompts of fewer tokens than this take the token-by-token decode kernel instead of the
// chunked form (measured faster for T <= 12 at B = 1, 32 and 256 with fp32 and bf16 states,
// slower from T = 16 on except where the two are within 5%).
constexpr int32_t kPrefillMinTokens = 16;

gdn_status prefill_impl(const char* fn, int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                        const void* q, const void* k, const void* v, gdn_dtype act_dtype,
                        const float* alpha, const float* beta, void* state, gdn_dtype state_dtype,
                        void* o, float scale, void* workspace, size_t workspace_bytes,
                        bool fixed_scratch, void* stream) {
    g_last_error.clear();
    gdn_status s = check_shape(fn, B, T, H, dk, dv);
    if (s != GDN_OK) return s;
    if (!valid_dtype(act_dtype) || !valid_dtype(state_dtype))
        return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": bad dtype");
    if (B == 0 || T == 0) return GDN_OK;
    if (B * (int64_t)H * gdn::prefill_chunks(T) * gdn::kPrefillWaveThreads >= gdn::kMaxWorkItems)
        return fail(GDN_ERR_UNSUPPORTED, std::string(fn) + ": B * H * ceil(T / 16) must be < 2^26 (one dispatch)");
    s = check_ptrs(fn, {{"q", q}, {"k", k}, {"v", v}, {"alpha", alpha}, {"beta", beta},
                        {"state", state}, {"o", o}});
    if (s != GDN_OK) return s;
    size_t need = 0;
    if (!prefill_ws_bytes(B, T, H, &need)) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": size overflows");
    if (fixed_scratch) {
        if (need > gdn::kPrefillScratchBytes)
            return fail(GDN_ERR_UNSUPPORTED,
                        std::string(fn) + ": B * H * ceil(T / 16) * 2176 = " + std::to_string(need) +
                            " bytes of chunk records exceed the fixed scratch of " +
                            std::to_string(gdn::kPrefillScratchBytes) +
                            " bytes (use gdn_prefill with a workspace)");
    } else {
        s = check_ptrs(fn, {{"workspace", workspace}});
        if (s != GDN_OK) return s;
        if (workspace_bytes < need)
            return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": workspace has " +
                                                      std::to_string(workspace_bytes) + " bytes, " +
                                                      std::to_string(need) + " needed");
    }
    const size_t tokens = (size_t)B * T * H;
    const size_t ab = dtype_bytes(act_dtype);
    const size_t state_bytes = (size_t)B * H * dk * dv * dtype_bytes(state_dtype);
    const Range r_q = range("q", q, tokens * dk * ab), r_k = range("k", k, tokens * dk * ab);
    const Range r_v = range("v", v, tokens * dv * ab), r_a = range("alpha", alpha, tokens * 4);
    const Range r_b = range("beta", beta, tokens * 4), r_s = range("state", state, state_bytes);
    const Range r_o = range("o", o, tokens * dv * ab);
    if (fixed_scratch) {
        s = check_disjoint(fn, r_o, {r_q, r_k, r_v, r_a, r_b, r_s});
        if (s != GDN_OK) return s;
        s = check_disjoint(fn, r_s, {r_q, r_k, r_v, r_a, r_b});
        if (s != GDN_OK) return s;
    } else {
        const Range r_w = range("workspace", workspace, need);
        s = check_disjoint(fn, r_o, {r_q, r_k, r_v, r_a, r_b, r_s, r_w});
        if (s != GDN_OK) return s;
        s = check_disjoint(fn, r_s, {r_q, r_k, r_v, r_a, r_b, r_w});
        if (s != GDN_OK) return s;
        s = check_disjoint(fn, r_w, {r_q, r_k, r_v, r_a, r_b});
        if (s != GDN_OK) return s;
    }

    // Prompts shorter than kPrefillMinTokens run token by token on the decode kernel: the same
    // result (the recurrence itself; no chunk records), and faster there at every batch size
    // and state type measured on MI355X (e.g. B = 256, T = 8, fp32 state: 333 vs 509 us).
    if (T < kPrefillMinTokens) {
        gdn::DecodeArgs d;
        d.B = B; d.T = T; d.H = H; d.D = dk;
        d.q = q; d.k = k; d.v = v;
        d.act = to_dtype(act_dtype);
        d.alpha = alpha; d.beta = beta;
        d.state = state;
        d.state_dtype = to_dtype(state_dtype);
        d.o = o; d.scale = scale;
        hipError_t e = gdn::launch_decode(d, reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail_hip((std::string(fn) + ": kernel launch").c_str(), e);
        return GDN_OK;
    }

    gdn::PrefillArgs a;
    a.B = B; a.T = T; a.H = H; a.D = dk;
    a.q = q; a.k = k; a.v = v; a.act = to_dtype(act_dtype);
    a.alpha = alpha; a.beta = beta;
    a.state = state; a.state_dtype = to_dtype(state_dtype);
    a.o = o; a.scale = scale;
    if (fixed_scratch) {
        float* p = nullptr;
        hipError_t e = gdn::prefill_scratch_address(&p);
        if (e != hipSuccess) return fail_hip((std::string(fn) + ": scratch address").c_str(), e);
        a.ws = p;
    } else {
        a.ws = static_cast<float*>(workspace);
    }
    hipError_t e = gdn::launch_prefill(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip((std::string(fn) + ": kernel launch").c_str(), e);
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                       const void* q, const void* k, const void* v, gdn_dtype act_dtype,
                       const float* alpha, const float* beta,
                       void* state, gdn_dtype state_dtype,
                       void* o, float scale, void* workspace, size_t workspace_bytes,
                       void* stream) {
    return prefill_impl("gdn_prefill", B, T, H, dk, dv, q, k, v, act_dtype, alpha, beta, state,
                        state_dtype, o, scale, workspace, workspace_bytes, false, stream);
}

gdn_status gdn_prefill_noalloc(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                               const void* q, const void* k, const void* v, gdn_dtype act_dtype,
                               const float* alpha, const float* beta,
                               void* state, gdn_dtype state_dtype,
                               void* o, float scale, void* stream) {
    return prefill_impl("gdn_prefill_noalloc", B, T, H, dk, dv, q, k, v, act_dtype, alpha, beta,
                        state, state_dtype, o, scale, nullptr, 0, true, stream);
}

gdn_status gdn_lowrank_decode_step(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                   int32_t r, const void* q, const void* k, const void* v,
                                   gdn_dtype act_dtype, const float* alpha, const float* beta,
                                   void* U, void* K, gdn_dtype state_dtype, float* c,
                                   int32_t* pos, void* o, float scale, void* stream) {
    static const char* fn = "gdn_lowrank_decode_step";
    g_last_error.clear();
    gdn_status s = check_shape(fn, B, T, H, dk, dv);
    if (s != GDN_OK) return s;
    if (!valid_dtype(act_dtype) || !valid_dtype(state_dtype))
        return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": bad dtype");
    if (r < 1) return fail(GDN_ERR_INVALID_ARGUMENT, std::string(fn) + ": r must be >= 1");
    if (!gdn::lowrank_supported_r(r))
        return fail(GDN_ERR_UNSUPPORTED, std::string(fn) + ": supported windows are r in {8, 16, 32}, got " +
                                             std::to_string(r));
    if (B == 0 || T == 0) return GDN_OK;
    s = check_ptrs(fn, {{"q", q}, {"k", k}, {"v", v}, {"alpha", alpha}, {"beta", beta},
                        {"U", U}, {"K", K}, {"c", c}, {"pos", pos}, {"o", o}});
    if (s != GDN_OK) return s;
    const size_t tokens = (size_t)B * T * H;
    const size_t heads = (size_t)B * H;
    const size_t ab = dtype_bytes(act_dtype), sb = dtype_bytes(state_dtype);
    const Range r_q = range("q", q, tokens * dk * ab), r_k = range("k", k, tokens * dk * ab);
    const Range r_v = range("v", v, tokens * dv * ab), r_a = range("alpha", alpha, tokens * 4);
    const Range r_b = range("beta", beta, tokens * 4), r_o = range("o", o, tokens * dv * ab);
    const Range r_U = range("U", U, heads * r * dv * sb), r_K = range("K", K, heads * r * dk * sb);
    const Range r_c = range("c", c, heads * r * 4), r_p = range("pos", pos, heads * 4);
    s = check_disjoint(fn, r_o, {r_q, r_k, r_v, r_a, r_b, r_U, r_K, r_c, r_p});
    if (s != GDN_OK) return s;
    s = check_disjoint(fn, r_U, {r_q, r_k, r_v, r_a, r_b, r_K, r_c, r_p});
    if (s != GDN_OK) return s;
    s = check_disjoint(fn, r_K, {r_q, r_k, r_v, r_a, r_b, r_c, r_p});
    if (s != GDN_OK) return s;
    s = check_disjoint(fn, r_c, {r_q, r_k, r_v, r_a, r_b, r_p});
    if (s != GDN_OK) return s;
    s = check_disjoint(fn, r_p, {r_q, r_k, r_v, r_a, r_b});
    if (s != GDN_OK) return s;

    gdn::LowrankArgs a;
    a.B = B; a.T = T; a.H = H; a.D = dk; a.R = r;
    a.q = q; a.k = k; a.v = v; a.act = to_dtype(act_dtype);
    a.alpha = alpha; a.beta = beta;
    a.U = U; a.K = K; a.state_dtype = to_dtype(state_dtype);
    a.c = c; a.pos = pos;
    a.o = o; a.scale = scale;
    hipError_t e = gdn::launch_lowrank(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip("gdn_lowrank_decode_step: kernel launch", e);
    return GDN_OK;
}

}  // extern "C"
