// HIP kernel for the sliding-window low-rank GDN state on gfx950 (CDNA4).
//
// "GDN tuning limits on Kunlun XPU", section 三.3, runs GDN decode on a low-rank state with
// r = 16 or 32 and states that this state caches the most recent r rank-1 updates (it is not
// a factorisation of the full state). Reading used here: a head's state is the sum of the
// last r writes of the gated delta rule, each decayed by every gate since it was written.
// Slot i holds a write vector U_i (dv values), its key K_i (dk values) and a weight c_i, so
// S = sum_i c_i U_i K_i^T; pos is the slot the next token writes (the oldest once full).
// Per token, with p = pos and every product taken over the window before the token:
//     a_i = K_i . k,  g_i = K_i . q      u = sum_i c_i a_i U_i  (= S k)
//     delta = beta (v - alpha u)         y = sum_{i != p} c_i g_i U_i
//     o = scale (alpha y + (k . q) delta)   (= S_t (scale q): the evicted write drops out,
//                                            the others decay by alpha, delta k^T joins)
//     c_i <- alpha c_i for every slot;  slot p <- (delta, k, 1);  pos <- p + 1 (mod r)
// so one pass over the registers serves the write and the readout.
// The dv x dk state is never formed: a token costs O(r D) instead of O(D^2) and the HBM
// traffic is the window read once plus the slots written, the weights and pos.
//
// Mapping: one wave64 per head, four heads per workgroup; the wave keeps the whole window in
// registers for all T tokens of the call:
//   * keys: slot i lives in lanes [i LPK, (i+1) LPK), LPK = 64 / r, each lane a contiguous
//     run of EK = D / LPK columns; K_i . k and K_i . q reduce across those lanes with DPP and
//     lane i LPK's total is read into a scalar register, so every per-slot coefficient is
//     uniform across the wave (k . q reduces the same way: each key group holds the same
//     columns of k and q);
//   * writes: lane l holds EU = D / 64 consecutive columns of every slot's U (for D < 64,
//     column l mod D; lanes >= D repeat that work and store nothing), so u, delta and o are
//     lane-local sums over the slots with scalar coefficients;
//   * weights and pos are uniform across the wave.
// Only the slots the call wrote (one per token; all of them once T >= r) are stored back.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_lowrank_launch.h"

namespace gdn {
namespace {

typedef uint32_t lr_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t lr_u32x2 __attribute__((ext_vector_type(2)));
typedef float lr_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 lr_bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 lr_f16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ element conversions

// Storage types: float (fp32), uint16_t (bf16 bits), _Float16 (fp16). Widening is exact;
// narrowing rounds to nearest even (gfx950's v_cvt_pk_bf16_f32 and v_cvt_pk_f16_f32).
template <typename T> struct Elt;
template <> struct Elt<float> {
    static __device__ __forceinline__ float get(uint32_t w, int) { return __uint_as_float(w); }
    static __device__ __forceinline__ uint32_t put(float lo, float) { return __float_as_uint(lo); }
    static constexpr int per_word = 1;
};
template <> struct Elt<uint16_t> {
    static __device__ __forceinline__ float get(uint32_t w, int e) {
        return e ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
    static __device__ __forceinline__ uint32_t put(float lo, float hi) {
        const lr_f32x2 v = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, lr_bf16x2));
    }
    static constexpr int per_word = 2;
};
template <> struct Elt<_Float16> {
    static __device__ __forceinline__ float get(uint32_t w, int e) {
        const lr_f32x2 f = __builtin_convertvector(__builtin_bit_cast(lr_f16x2, w), lr_f32x2);
        return e ? f.y : f.x;
    }
    static __device__ __forceinline__ uint32_t put(float lo, float hi) {
        const lr_f32x2 v = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, lr_f16x2));
    }
    static constexpr int per_word = 2;
};

// ------------------------------------------------------------------ vector memory

// N consecutive elements of T at p (aligned to their total size, a power of two) into
// floats, with the widest accesses that fit (16, 8, 4 or 2 bytes).
template <typename T, int N>
__device__ __forceinline__ void load_run(const T* p, float (&x)[N]) {
    constexpr int BYTES = N * (int)sizeof(T);
    if constexpr (BYTES == 2) {
        const uint32_t w = *(const uint16_t*)p;
        x[0] = Elt<T>::get(w, 0);
    } else {
        constexpr int W = BYTES / 4;
        uint32_t w[W];
        if constexpr (BYTES % 16 == 0) {
#pragma unroll
            for (int i = 0; i < W / 4; ++i) {
                const lr_u32x4 v = ((const lr_u32x4*)p)[i];
                w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
            }
        } else if constexpr (BYTES == 8) {
            const lr_u32x2 v = *(const lr_u32x2*)p;
            w[0] = v.x; w[1] = v.y;
        } else {
            static_assert(BYTES == 4, "run size");
            w[0] = *(const uint32_t*)p;
        }
#pragma unroll
        for (int e = 0; e < N; ++e) x[e] = Elt<T>::get(w[e / Elt<T>::per_word], e % Elt<T>::per_word);
    }
}

template <typename T, int N>
__device__ __forceinline__ void store_run(T* p, const float (&x)[N]) {
    constexpr int BYTES = N * (int)sizeof(T);
    if constexpr (BYTES == 2) {
        *(uint16_t*)p = (uint16_t)(Elt<T>::put(x[0], 0.0f) & 0xffffu);
    } else {
        constexpr int W = BYTES / 4;
        constexpr int PW = Elt<T>::per_word;
        uint32_t w[W];
#pragma unroll
        for (int i = 0; i < W; ++i) w[i] = Elt<T>::put(x[PW * i], PW == 2 ? x[PW * i + 1] : 0.0f);
        if constexpr (BYTES % 16 == 0) {
#pragma unroll
            for (int i = 0; i < W / 4; ++i)
                ((lr_u32x4*)p)[i] = lr_u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
        } else if constexpr (BYTES == 8) {
            *(lr_u32x2*)p = lr_u32x2{w[0], w[1]};
        } else {
            static_assert(BYTES == 4, "run size");
            *(uint32_t*)p = w[0];
        }
    }
}

// ------------------------------------------------------------------ reductions

template <int CTRL>
__device__ __forceinline__ float lr_dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (2, 4 or 8); every lane of a group gets the same total.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 2 || G == 4 || G == 8, "groups of 2, 4 or 8 lanes");
    x += lr_dpp<0xB1>(x);                         // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 4) x += lr_dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 8) x += lr_dpp<0x141>(x);  // row_half_mirror: the other quad of 8
    return x;
}

// A value every lane holds identically, kept in a scalar register.
__device__ __forceinline__ float uniform_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float lane_value(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// ------------------------------------------------------------------ the kernel

template <int D, int R, typename AT, typename ST>
__global__ __launch_bounds__(64 * kLowrankHeadsPerGroup) void gdn_lowrank_kernel(LowrankArgs a) {
    constexpr int LPK = 64 / R;                 // lanes per key slot
    constexpr int EK = D / LPK;                 // key columns per lane
    constexpr int EU = D >= 64 ? D / 64 : 1;    // write columns per lane
    constexpr int KCH = (16 / (int)sizeof(AT)) < EK ? (16 / (int)sizeof(AT)) : EK;  // per load
    static_assert(EK % KCH == 0, "key run");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t head = (int64_t)blockIdx.x * kLowrankHeadsPerGroup + wave;  // b * H + h
    if (head >= a.B * a.H) return;
    const int64_t b = head / a.H;
    const int h = (int)(head - b * a.H);

    const int ks = lane / LPK;                        // this lane's key slot
    const int kc = (lane % LPK) * EK;                 // its first key column
    const int uc = D >= 64 ? lane * EU : lane % D;    // its first write column
    const bool u_owner = D >= 64 || lane < D;

    ST* Uh = (ST*)a.U + head * (R * D);
    ST* Kh = (ST*)a.K + head * (R * D);
    float* ch = a.c + head * R;

    float Kr[EK];
    load_run<ST, EK>(Kh + ks * D + kc, Kr);
    float Ur[R][EU];
#pragma unroll
    for (int i = 0; i < R; ++i) load_run<ST, EU>(Uh + i * D + uc, Ur[i]);
    float cw[R];
#pragma unroll
    for (int i = 0; i < R; ++i) cw[i] = uniform_f(ch[i]);
    const uint32_t p0 = (uint32_t)a.pos[head] & (uint32_t)(R - 1);
    uint32_t p = p0;

    for (int t = 0; t < a.T; ++t) {
        const int64_t g = (b * a.T + t) * a.H + h;     // (b, t, h)
        const AT* kp = (const AT*)a.k + g * D + kc;
        const AT* qp = (const AT*)a.q + g * D + kc;
        float vt[EU];
        load_run<AT, EU>((const AT*)a.v + g * D + uc, vt);
        const float al = a.alpha[g], be = a.beta[g];

        // One pass over the window before this token: K_i . k, K_i . q and k . q (every key
        // group holds the same columns of k and q, so its k . q total is the whole product).
        float pa = 0.0f, pg = 0.0f, pkq = 0.0f;
#pragma unroll
        for (int c0 = 0; c0 < EK; c0 += KCH) {
            float xk[KCH], xq[KCH];
            load_run<AT, KCH>(kp + c0, xk);
            load_run<AT, KCH>(qp + c0, xq);
#pragma unroll
            for (int e = 0; e < KCH; ++e) {
                pa = fmaf(Kr[c0 + e], xk[e], pa);
                pg = fmaf(Kr[c0 + e], xq[e], pg);
                pkq = fmaf(xk[e], xq[e], pkq);
            }
        }
        pa = group_sum<LPK>(pa);
        pg = group_sum<LPK>(pg);
        const float kq = lane_value(group_sum<LPK>(pkq), 0);

        // u = S k, and y = S q without the slot this token evicts; then
        //   delta = beta (v - alpha u),  o = scale (alpha y + (k . q) delta) = S_t (scale q).
        float u[EU], y[EU];
#pragma unroll
        for (int e = 0; e < EU; ++e) u[e] = y[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float wu = cw[i] * lane_value(pa, i * LPK);
            const float wy = (uint32_t)i == p ? 0.0f : cw[i] * lane_value(pg, i * LPK);
#pragma unroll
            for (int e = 0; e < EU; ++e) {
                u[e] = fmaf(wu, Ur[i][e], u[e]);
                y[e] = fmaf(wy, Ur[i][e], y[e]);
            }
        }
        float o[EU];
#pragma unroll
        for (int e = 0; e < EU; ++e) {
            const float d = be * fmaf(-al, u[e], vt[e]);
            o[e] = a.scale * fmaf(al, y[e], kq * d);
#pragma unroll
            for (int i = 0; i < R; ++i) Ur[i][e] = (uint32_t)i == p ? d : Ur[i][e];
        }
        if (u_owner) store_run<AT, EU>((AT*)a.o + g * D + uc, o);

        // The decay of every stored write; the oldest slot takes (delta, k, 1).
#pragma unroll
        for (int i = 0; i < R; ++i) cw[i] = uniform_f((uint32_t)i == p ? 1.0f : cw[i] * al);
        if ((uint32_t)ks == p) load_run<AT, EK>(kp, Kr);
        p = (p + 1) & (uint32_t)(R - 1);
    }

    // Store the slots this call wrote, every weight, and the next slot.
    const uint32_t written = (uint32_t)(a.T < R ? a.T : R);
    if (u_owner) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            if ((((uint32_t)i - p0) & (uint32_t)(R - 1)) < written) store_run<ST, EU>(Uh + i * D + uc, Ur[i]);
    }
    if ((((uint32_t)ks - p0) & (uint32_t)(R - 1)) < written) store_run<ST, EK>(Kh + ks * D + kc, Kr);
    float mine = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) mine = lane == i ? cw[i] : mine;
    if (lane < R) ch[lane] = mine;
    if (lane == 0) a.pos[head] = (int32_t)p;
}

template <int D, int R, typename AT, typename ST>
hipError_t launch_typed(const LowrankArgs& a, hipStream_t stream) {
    const int64_t heads = a.B * a.H;
    const int64_t groups = (heads + kLowrankHeadsPerGroup - 1) / kLowrankHeadsPerGroup;
    hipLaunchKernelGGL((gdn_lowrank_kernel<D, R, AT, ST>), dim3((uint32_t)groups),
                       dim3(64 * kLowrankHeadsPerGroup), 0, stream, a);
    return hipGetLastError();
}

template <int D, typename AT, typename ST>
hipError_t launch_r(const LowrankArgs& a, hipStream_t stream) {
    switch (a.R) {
        case 8: return launch_typed<D, 8, AT, ST>(a, stream);
        case 16: return launch_typed<D, 16, AT, ST>(a, stream);
        case 32: return launch_typed<D, 32, AT, ST>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int D, typename AT>
hipError_t launch_st(const LowrankArgs& a, hipStream_t stream) {
    switch (a.state_dtype) {
        case DType::F32: return launch_r<D, AT, float>(a, stream);
        case DType::BF16: return launch_r<D, AT, uint16_t>(a, stream);
        case DType::F16: return launch_r<D, AT, _Float16>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_at(const LowrankArgs& a, hipStream_t stream) {
    switch (a.act) {
        case DType::F32: return launch_st<D, float>(a, stream);
        case DType::BF16: return launch_st<D, uint16_t>(a, stream);
        case DType::F16: return launch_st<D, _Float16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_lowrank(const LowrankArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 16: return launch_at<16>(a, stream);
        case 32: return launch_at<32>(a, stream);
        case 64: return launch_at<64>(a, stream);
        case 128: return launch_at<128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
