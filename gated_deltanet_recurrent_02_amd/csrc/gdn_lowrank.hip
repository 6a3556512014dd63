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
// Mapping (see LrGeo and gdn_lowrank_kernel): at D = 128 two wave64s share a head (four for a
// 32-slot fp32 window), each holding its share of the key slots and of the write columns
// (8 KiB of a 16-slot fp32 window), and trade their per-slot key products through LDS once
// per token; at D = 64 two waves share a head; below, one wave holds a whole head. Every wave
// keeps its share of the window in registers for all T tokens of the call.
// Only the slots the call wrote (one per token; all of them once T >= r) are stored back.
// Multi-token calls with bf16 activations at D = 128 on a bf16 window (and on a 16-slot fp32
// window from 4 tokens on) run gdn_lowrank_mm_kernel instead, which forms each round's key
// products on the matrix cores, or, on a bf16 window whose rounds are full or nearly so
// (lr_round_form), gdn_lowrank_round_kernel, which takes each round of tokens in matrix form on
// the matrix cores (see there).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
// floats, with the widest accesses that fit (16, 8, 4 or 2 bytes); NT marks the loads
// nontemporal (streamed past the caches' retention).
template <typename T, int N, bool NT = false>
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
                const lr_u32x4 v = NT ? __builtin_nontemporal_load((const lr_u32x4*)p + i)
                                      : ((const lr_u32x4*)p)[i];
                w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
            }
        } else if constexpr (BYTES == 8) {
            const lr_u32x2 v = NT ? __builtin_nontemporal_load((const lr_u32x2*)p) : *(const lr_u32x2*)p;
            w[0] = v.x; w[1] = v.y;
        } else {
            static_assert(BYTES == 4, "run size");
            w[0] = NT ? __builtin_nontemporal_load((const uint32_t*)p) : *(const uint32_t*)p;
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

// Sum over aligned groups of 16 lanes (one DPP row); every lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float x) {
    x = group_sum<8>(x);
    return x + lr_dpp<0x140>(x);                  // row_mirror: the other half of the row
}

// With U (true) a value every lane of the wave holds identically, kept in a scalar register.
template <bool U>
__device__ __forceinline__ float wave_uniform(float x) {
    if constexpr (U)
        return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
    else
        return x;
}

__device__ __forceinline__ float lane_value(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// ------------------------------------------------------------------ the kernel

// Most waves that share one head at D = 128, chosen by measurement on MI355X (B = 256, H = 48):
// four for a 32-slot fp32 window (88.5 -> 78.6 us per call against two), two otherwise (four
// waves lose 2-22% on 16-slot and 16-bit windows and on multi-token calls). The window is
// read once per call, so its loads are nontemporal (16-slot fp32: 44.7 -> 39.2 us).
template <int R, typename ST>
constexpr int lr_max_waves() { return sizeof(ST) == 4 && R >= 32 ? 4 : 2; }
constexpr bool kLrStateNT = true;
// Tokens per staged round of a multi-token call.
constexpr int kLrRound = 8;
// Multi-token calls on a bf16 window (D = 128, bf16 activations) run each round in matrix form
// (gdn_lowrank_round_kernel) when every round is full or nearly so (a partial last round costs
// what a full one does), else one token at a time over the write columns
// (gdn_lowrank_mm_kernel). Measured on MI355X at B = 256, H = 48 (per-token / round form, us):
// 16 slots T = 4 42.3 / 54.9, T = 8 64.3 / 60.6, T = 10 82.6 / 92.6, T = 12 92.0 / 95.1,
// T = 16 113.0 / 99.7, T = 24 150.4 / 132.7; 32 slots T = 4 65.2 / 84.8, T = 6 83.7 / 87.3,
// T = 8 96.6 / 88.2, T = 10 124.6 / 140.7, T = 16 171.5 / 145.5, T = 24 241.7 / 201.2.
__host__ __device__ constexpr bool lr_round_form(int T) {
    return T >= kLrRound && (T % kLrRound == 0 || T % kLrRound >= kLrRound - 2);
}

// Geometry of one instance: head dim D, window R, storage types AT (activations), ST (state).
template <int D, int R, typename AT, typename ST>
struct LrGeo {
    // waves per head: D / 32 (one wave below D = 64), at most lr_max_waves, and few enough that
    // every wave owns at least 4 key slots
    static constexpr int W0 = D / 32 < lr_max_waves<R, ST>() ? D / 32 : lr_max_waves<R, ST>();
    static constexpr int W1 = W0 < R / 4 ? W0 : R / 4;
    static constexpr int W = W1 < 1 ? 1 : W1;
    static constexpr int RW = R / W;                      // key slots per wave
    static constexpr int LPK = 64 / RW;                   // lanes per key slot
    static constexpr int EK = D / LPK;                    // key columns per lane
    static constexpr int CHE = (16 / (int)sizeof(ST)) < EK ? (16 / (int)sizeof(ST)) : EK;
    static constexpr int NCH = EK / CHE;                  // key chunks per lane
    static constexpr int DW = D / W;                      // write columns per wave
    // write columns per lane: two for 16-bit windows (4-byte loads), else one
    static constexpr int EU = sizeof(ST) == 2 && DW >= 64 ? 2 : 1;
    static constexpr int CL = DW / EU;                    // lanes that cover the wave's columns
    static constexpr int SG = 64 / CL;                    // lanes per write column
    static constexpr int RS = R / SG;                     // write slots per lane
    static_assert(LPK >= 2 && LPK <= 16 && EK * LPK == D && NCH * CHE == EK, "key layout");
    static_assert(CL <= 64 && SG * CL == 64 && (SG == 1 || SG == 2 || SG == 4) && RS >= 1,
                  "write layout");
};

template <int G>
__device__ __forceinline__ float slot_sum(float x) {
    if constexpr (G == 16) return row_sum16(x);
    else return group_sum<G>(x);
}

// Sum over the SG lanes that hold one write column (lanes l, l ^ DW, ...).
template <int SG, int DW>
__device__ __forceinline__ float column_sum(float x) {
    if constexpr (SG >= 2) x += __shfl_xor(x, DW, 64);
    if constexpr (SG == 4) x += __shfl_xor(x, 2 * DW, 64);
    return x;
}

// W wave64s per (sequence, head); every wave keeps its share of the window in registers for
// all T tokens of the call:
//   * keys: the wave owns slots [w RW, (w+1) RW); slot i lives in LPK lanes, lane j of them
//     holding the 16-byte column chunks j, j + LPK, j + 2 LPK, ... (one load instruction covers
//     LPK * 16 contiguous bytes of each of RW rows). K_i . k and K_i . q reduce across the
//     slot's lanes with DPP, and the slot totals go through LDS (one barrier per token) to
//     the lanes that hold that slot's writes;
//   * writes: the wave owns columns [w DW, (w+1) DW) of every slot's U; lane l holds the EU
//     adjacent columns starting at w DW + (l mod CL) EU (EU = 2 for 16-bit windows, so each
//     load is 4 bytes; else 1) of the RS slots of its slot group l / CL, with those slots'
//     weights, so u, y, delta and o are lane-local sums over slots plus one cross-lane sum
//     over the SG groups of a column;
//   * pos is uniform across the workgroup; wave 0 stores the weights and pos.
// One head per workgroup.
// ONE: the call has one token (a separate instance: with the token count known, the keys are
// dead after the key products and the other writes after the sums, which frees registers).
template <int D, int R, typename AT, typename ST, bool ONE>
__global__ __launch_bounds__((64 * LrGeo<D, R, AT, ST>::W))
void gdn_lowrank_kernel(LowrankArgs a) {
    using G = LrGeo<D, R, AT, ST>;
    constexpr int RW = G::RW, LPK = G::LPK, CHE = G::CHE, NCH = G::NCH;
    constexpr int DW = G::DW, SG = G::SG, RS = G::RS, EU = G::EU, CL = G::CL;
    __shared__ float xchg[2][2][R];   // [token parity][K.k, K.q][slot]
    // multi-token calls: the tokens of a round of up to kLrRound, staged once per round
    constexpr int TS = ONE ? 1 : kLrRound;
    __shared__ alignas(16) float tok[ONE ? 1 : 3][TS][ONE ? 4 : D];   // [k, q, v][token][column]
    __shared__ float tok_ab[ONE ? 1 : 2][TS];                           // [alpha, beta][token]

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave within the head
    const int64_t head = blockIdx.x;                                   // b * H + h
    const int64_t b = head / a.H;
    const int h = (int)(head - b * a.H);

    const int ks = w * RW + lane / LPK;               // this lane's key slot
    const int kj = lane % LPK;                        // its chunk phase
    const int uc = w * DW + (lane % CL) * EU;         // its first write column
    const int sg = lane / CL;                         // its slot group: slots [sg RS, (sg+1) RS)

    ST* Uh = (ST*)a.U + head * (R * D);
    ST* Kh = (ST*)a.K + head * (R * D);
    float* ch = a.c + head * R;

    float Kr[NCH][CHE];
#pragma unroll
    for (int m = 0; m < NCH; ++m)
        load_run<ST, CHE, kLrStateNT>(Kh + ks * D + (m * LPK + kj) * CHE, Kr[m]);
    float Ur[RS][EU];
#pragma unroll
    for (int i = 0; i < RS; ++i) load_run<ST, EU, kLrStateNT>(Uh + (sg * RS + i) * D + uc, Ur[i]);
    float cl[RS];   // weights of this lane's write slots (scalar registers when SG == 1)
#pragma unroll
    for (int i = 0; i < RS; ++i) cl[i] = wave_uniform<SG == 1>(ch[sg * RS + i]);
    const uint32_t p0 = (uint32_t)a.pos[head] & (uint32_t)(R - 1);
    uint32_t p = p0;

    const int T = ONE ? 1 : a.T;
    for (int t = 0; t < T; ++t) {
        const int64_t g = (b * a.T + t) * a.H + h;     // (b, t, h)
        const AT* kp = (const AT*)a.k + g * D;
        const AT* qp = (const AT*)a.q + g * D;
        const int tt = ONE ? 0 : t % kLrRound;        // the token's place in its round
        if constexpr (!ONE) {
            if (tt == 0) {
                // stage the round's k, q and v rows (16-byte chunks over the workgroup) and
                // gates; the barrier also ends the previous round's reads of the buffer
                constexpr int CK = 16 / (int)sizeof(AT), NCR = D / CK;
                const int nt = min(kLrRound, T - t);
                __syncthreads();
                for (int c = threadIdx.x; c < nt * 3 * NCR; c += 64 * G::W) {
                    const int j = c / NCR, col = (c - j * NCR) * CK, which = j / nt, u = j - which * nt;
                    const AT* src = which == 0 ? (const AT*)a.k : which == 1 ? (const AT*)a.q
                                                                            : (const AT*)a.v;
                    float x[CK];
                    load_run<AT, CK>(src + ((b * a.T + t + u) * a.H + h) * D + col, x);
#pragma unroll
                    for (int e = 0; e < CK; ++e) tok[which][u][col + e] = x[e];
                }
                if ((int)threadIdx.x < nt) {
                    const int64_t gu = (b * a.T + t + threadIdx.x) * a.H + h;
                    tok_ab[0][threadIdx.x] = a.alpha[gu];
                    tok_ab[1][threadIdx.x] = a.beta[gu];
                }
                __syncthreads();
            }
        }
        float vt[EU];
        float al, be;
        if constexpr (ONE) {
            load_run<AT, EU>((const AT*)a.v + g * D + uc, vt);
            al = a.alpha[g];
            be = a.beta[g];
        } else {
#pragma unroll
            for (int e = 0; e < EU; ++e) vt[e] = tok[2][tt][uc + e];
            al = wave_uniform<true>(tok_ab[0][tt]);
            be = wave_uniform<true>(tok_ab[1][tt]);
        }

        // One pass over this wave's keys before the token: K_i . k, K_i . q and k . q (every
        // slot's lanes cover all D columns of k and q, so a slot's k . q total is the whole
        // product).
        float pa = 0.0f, pg = 0.0f, pkq = 0.0f;
#pragma unroll
        for (int m = 0; m < NCH; ++m) {
            float xk[CHE], xq[CHE];
            if constexpr (ONE) {
                load_run<AT, CHE>(kp + (m * LPK + kj) * CHE, xk);
                load_run<AT, CHE>(qp + (m * LPK + kj) * CHE, xq);
            } else {
#pragma unroll
                for (int e = 0; e < CHE; ++e) {
                    xk[e] = tok[0][tt][(m * LPK + kj) * CHE + e];
                    xq[e] = tok[1][tt][(m * LPK + kj) * CHE + e];
                }
            }
#pragma unroll
            for (int e = 0; e < CHE; ++e) {
                pa = fmaf(Kr[m][e], xk[e], pa);
                pg = fmaf(Kr[m][e], xq[e], pg);
                pkq = fmaf(xk[e], xq[e], pkq);
            }
        }
        pa = slot_sum<LPK>(pa);
        pg = slot_sum<LPK>(pg);
        const float kq = lane_value(slot_sum<LPK>(pkq), 0);
        // the lanes that hold a slot's writes need its totals: trade them through LDS (two
        // buffers by token parity, so one barrier per token keeps every read before the
        // buffer's next write)
        if (kj == 0) {
            xchg[t & 1][0][ks] = pa;
            xchg[t & 1][1][ks] = pg;
        }
        __syncthreads();

        // u = S k, and y = S q without the slot this token evicts, over this lane's slots and
        // then over the column's lanes; then
        //   delta = beta (v - alpha u),  o = scale (alpha y + (k . q) delta) = S_t (scale q).
        float u[EU], y[EU];
#pragma unroll
        for (int e = 0; e < EU; ++e) u[e] = y[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < RS; ++i) {
            const int slot = sg * RS + i;
            // both products unconditionally, then a select: a conditional product would be
            // compiled as a branch around its LDS read, one wait per slot
            const float wu = cl[i] * xchg[t & 1][0][slot];
            const float wg = cl[i] * xchg[t & 1][1][slot];
            const float wy = (uint32_t)slot == p ? 0.0f : wg;
#pragma unroll
            for (int e = 0; e < EU; ++e) {
                u[e] = fmaf(wu, Ur[i][e], u[e]);
                y[e] = fmaf(wy, Ur[i][e], y[e]);
            }
        }
        float d[EU], o[EU];
#pragma unroll
        for (int e = 0; e < EU; ++e) {
            u[e] = column_sum<SG, CL>(u[e]);
            y[e] = column_sum<SG, CL>(y[e]);
            d[e] = be * fmaf(-al, u[e], vt[e]);
            o[e] = a.scale * fmaf(al, y[e], kq * d[e]);
        }
        if (sg == 0) store_run<AT, EU>((AT*)a.o + g * D + uc, o);

        // The decay of every stored write; the oldest slot takes (delta, k, 1).
#pragma unroll
        for (int i = 0; i < RS; ++i) {
            const bool mine = (uint32_t)(sg * RS + i) == p;
#pragma unroll
            for (int e = 0; e < EU; ++e) Ur[i][e] = mine ? d[e] : Ur[i][e];
            cl[i] = wave_uniform<SG == 1>(mine ? 1.0f : cl[i] * al);
        }
        if ((uint32_t)ks == p) {
#pragma unroll
            for (int m = 0; m < NCH; ++m) {
                if constexpr (ONE) {
                    load_run<AT, CHE>(kp + (m * LPK + kj) * CHE, Kr[m]);
                } else {
#pragma unroll
                    for (int e = 0; e < CHE; ++e) Kr[m][e] = tok[0][tt][(m * LPK + kj) * CHE + e];
                }
            }
        }
        p = (p + 1) & (uint32_t)(R - 1);
    }

    // Store the slots this call wrote, every weight, and the next slot.
    const uint32_t written = (uint32_t)(T < R ? T : R);
#pragma unroll
    for (int i = 0; i < RS; ++i)
        if ((((uint32_t)(sg * RS + i) - p0) & (uint32_t)(R - 1)) < written)
            store_run<ST, EU>(Uh + (sg * RS + i) * D + uc, Ur[i]);
    if ((((uint32_t)ks - p0) & (uint32_t)(R - 1)) < written) {
#pragma unroll
        for (int m = 0; m < NCH; ++m) store_run<ST, CHE>(Kh + ks * D + (m * LPK + kj) * CHE, Kr[m]);
    }
    if (w == 0 && lane % CL == 0) {
#pragma unroll
        for (int i = 0; i < RS; ++i) ch[sg * RS + i] = cl[i];
        if (lane == 0) a.pos[head] = (int32_t)p;
    }
}

// ------------------------------------------------------------------ bf16 multi-token form

typedef __bf16 lr_bf16x8 __attribute__((ext_vector_type(8)));
typedef float lr_f32x4 __attribute__((ext_vector_type(4)));

// Two floats as three bf16 parts each (hi, mid, lo: truncations of the value and of the two
// remainders), packed in pairs (x in the low half); hi + mid + lo is exactly the value (24
// significant bits in three runs of 8), so products of exact bf16 operands with the three
// parts sum to the fp32 product.
__device__ __forceinline__ void lr_split3(float x, float y, uint32_t& h, uint32_t& m, uint32_t& l) {
    constexpr uint32_t HI = 0xffff0000u;
    const uint32_t ux = __float_as_uint(x), uy = __float_as_uint(y);
    const float rx = x - __uint_as_float(ux & HI), ry = y - __uint_as_float(uy & HI);
    const uint32_t vx = __float_as_uint(rx), vy = __float_as_uint(ry);
    const float sx = rx - __uint_as_float(vx & HI), sy = ry - __uint_as_float(vy & HI);
    h = __builtin_amdgcn_perm(uy, ux, 0x07060302u);
    m = __builtin_amdgcn_perm(vy, vx, 0x07060302u);
    l = __builtin_amdgcn_perm(__float_as_uint(sy), __float_as_uint(sx), 0x07060302u);
}

// C += A B over a 16 x 16 x 32 slice, bf16 operands (lane l holds k = 8 (l/16) .. + 7 of its
// row / column l % 16), fp32 accumulation into C[4 (l/16) + i][l % 16].
__device__ __forceinline__ lr_f32x4 lr_mfma_k32(lr_u32x4 a, lr_u32x4 b, lr_f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(lr_bf16x8, a),
                                                   __builtin_bit_cast(lr_bf16x8, b), c, 0, 0, 0);
}
// C += A B over a 16 x 16 x 4 slice in fp32: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; same accumulator layout.
__device__ __forceinline__ lr_f32x4 lr_mfma4(float a, float b, lr_f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Multi-token calls with bf16 activations at D = 128 on a bf16 window (r = 16 or 32) or a
// 16-slot fp32 window: the key products of a whole round run on the matrix cores instead of
// per token on the vector ALUs (an fp32 window's keys as three exact bf16 parts each).
// Both operands are exact bf16 and the products accumulate in fp32, as in the vector form
// (summation order differs). Per round of up to kLrRound tokens t0 .. t0+nt-1 (window slot p_r
// the next to be written at the round's start):
//   C[i][n]  = K_i . w_n   for every slot i,    C'[s][n] = k_{t0+s} . w_n,
// with w_n = k_{t0+n} for n < 8 and q_{t0+n-8} for n >= 8, both on 16 x 16 x 32 bf16 products.
// Token t0 + tn sees slot i's key as written at the round's start unless the round has already
// rewritten it: slot i is written by round token s_i = (i - p_r) mod r, so for s_i < tn its key
// is k_{t0+s_i} and its products are C'[s_i][.]. The merged products go to LDS once per round,
// each wave computing them for every slot (the waves need every slot's totals for their write
// columns), which removes the per-token key FMAs, slot sums and the per-token exchange and
// barrier of the vector form. The per-token pass over the write columns is the vector form's.
template <int R, typename ST>
__global__ __launch_bounds__(128) void gdn_lowrank_mm_kernel(LowrankArgs a) {
    constexpr int D = 128;
    using AT = uint16_t;
    using G = LrGeo<D, R, AT, ST>;
    constexpr bool F32 = std::is_same<ST, float>::value;
    static_assert(G::W == 2 && (R == 16 || R == 32) && (F32 || std::is_same<ST, uint16_t>::value),
                  "layout");
    constexpr int DW = G::DW, SG = G::SG, RS = G::RS, EU = G::EU, CL = G::CL;
    constexpr int NTL = R / 16;     // 16-slot tiles of the key products
    constexpr int TS = kLrRound;    // tokens per round
    static_assert(TS == 8, "a round's k and q fill the 16 product columns");
    constexpr int KST = D / 2 + 4;  // row stride (words) of staged bf16 rows: rows in other banks
    // The window's keys: a bf16 window's as raw bf16 pairs, an fp32 window's as floats (split
    // exactly into three bf16 parts where they enter the products).
    constexpr int KW = F32 ? D + 4 : KST;                    // words per key row
    constexpr int KCR = D * (int)sizeof(ST) / 16;            // 16-byte chunks per key row
    __shared__ alignas(16) uint32_t ks[R][KW];
    __shared__ alignas(16) uint32_t kq_raw[2][TS][KST];      // the round's k and q (bf16 pairs)
    __shared__ alignas(16) float vs[TS][D];                  // the round's v
    __shared__ float tok_ab[2][TS];                          // [alpha, beta][token]
    __shared__ alignas(16) float gram[2][TS][16];            // per wave: C'[s][n]
    __shared__ alignas(16) float prod[2][2][TS][R];          // per wave: [K.k, K.q][token][slot]
    __shared__ float kqd[2][TS];                             // per wave: k_t . q_t

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t head = blockIdx.x;
    const int64_t b = head / a.H;
    const int h = (int)(head - b * a.H);
    const int gq = lane >> 4, mq = lane & 15;           // matrix-core lane coordinates
    const int uc = w * DW + (lane % CL) * EU;           // first write column of this lane
    const int sg = lane / CL;                           // slot group: slots [sg RS, (sg+1) RS)

    ST* Uh = (ST*)a.U + head * (R * D);
    ST* Kh = (ST*)a.K + head * (R * D);
    float* ch = a.c + head * R;

    // Staging: thread tid moves token su = tid / 16, columns 8 (tid % 16) .. + 7 of k, q and v;
    // tokens past the round are staged as zeros (their products are never read).
    const int su = tid >> 4, scol = (tid & 15) * 8;
    const int64_t tok_stride = (int64_t)a.H * D;
    const int T = a.T;
    lr_u32x4 rk, rq, rv;
    float gab;
    auto stage_loads = [&](int t0) {
        const int nt = min(TS, T - t0);
        rk = rq = rv = lr_u32x4{0u, 0u, 0u, 0u};
        if (su < nt) {
            const int64_t off = ((b * T + t0) * a.H + h) * D + su * tok_stride + scol;
            rk = *(const lr_u32x4*)((const AT*)a.k + off);
            rq = *(const lr_u32x4*)((const AT*)a.q + off);
            rv = *(const lr_u32x4*)((const AT*)a.v + off);
        }
        gab = 0.0f;
        if (tid < 2 * TS && (tid & 7) < nt) {
            const int64_t gu = (b * T + t0 + (tid & 7)) * a.H + h;
            gab = tid < TS ? a.alpha[gu] : a.beta[gu];
        }
    };
    stage_loads(0);
    // The window's keys in LDS, one copy per head (thread tid moves 16-byte chunks
    // tid + 128 j: slot chunk / KCR, words 4 (chunk % KCR) .. + 3 of the row).
    constexpr int KCT = R * KCR / 128;                       // chunks per thread
    lr_u32x4 kc[KCT];
#pragma unroll
    for (int j = 0; j < KCT; ++j) {
        const int chunk = tid + 128 * j, row = chunk / KCR, cw = (chunk % KCR) * 4;
        kc[j] = __builtin_nontemporal_load((const lr_u32x4*)((const uint32_t*)(Kh + row * D) + cw));
    }
    float Ur[RS][EU];
#pragma unroll
    for (int i = 0; i < RS; ++i) load_run<ST, EU, kLrStateNT>(Uh + (sg * RS + i) * D + uc, Ur[i]);
    float cl[RS];
#pragma unroll
    for (int i = 0; i < RS; ++i) cl[i] = ch[sg * RS + i];
    const uint32_t p0 = (uint32_t)a.pos[head] & (uint32_t)(R - 1);
    uint32_t p = p0;
#pragma unroll
    for (int j = 0; j < KCT; ++j) {
        const int chunk = tid + 128 * j, row = chunk / KCR, cw = (chunk % KCR) * 4;
        *(lr_u32x4*)&ks[row][cw] = kc[j];
    }

    for (int t0 = 0; t0 < T; t0 += TS) {
        const int nt = min(TS, T - t0);
        const uint32_t pr = p;   // slot of the round's first token
        __syncthreads();         // the previous round's readers are done with the buffers
        *(lr_u32x4*)&kq_raw[0][su][scol / 2] = rk;   // (the first round's barrier also covers ks)
        *(lr_u32x4*)&kq_raw[1][su][scol / 2] = rq;
        {
            const uint32_t wv[4] = {rv.x, rv.y, rv.z, rv.w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = Elt<AT>::get(wv[e >> 1], e & 1);
            *(lr_f32x4*)&vs[su][scol] = lr_f32x4{f[0], f[1], f[2], f[3]};
            *(lr_f32x4*)&vs[su][scol + 4] = lr_f32x4{f[4], f[5], f[6], f[7]};
        }
        if (tid < 2 * TS) tok_ab[tid >> 3][tid & 7] = gab;
        if (t0 + TS < T) stage_loads(t0 + TS);
        __syncthreads();

        // C (every slot) and C' (the round's keys) against the round's k | q columns.
        lr_f32x4 C[NTL], Cp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NTL; ++t) C[t] = lr_f32x4{0.f, 0.f, 0.f, 0.f};
        const int vn = mq & 7;                 // the token of product column mq
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int wo = (8 * gq + 32 * s) / 2;
            const lr_u32x4 bv = *(const lr_u32x4*)&kq_raw[mq >> 3][vn][wo];
            const lr_u32x4 av = *(const lr_u32x4*)&kq_raw[0][vn][wo];   // rows >= 8 unused
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                if constexpr (F32) {
                    // columns 8 gq + 32 s .. + 7 as floats, in three exact bf16 parts
                    const lr_u32x4 x0 = *(const lr_u32x4*)&ks[16 * t + mq][2 * wo];
                    const lr_u32x4 x1 = *(const lr_u32x4*)&ks[16 * t + mq][2 * wo + 4];
                    const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    uint32_t hh[4], mm[4], ll[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        lr_split3(__uint_as_float(xs[2 * e]), __uint_as_float(xs[2 * e + 1]),
                                  hh[e], mm[e], ll[e]);
                    const lr_u32x4 ph = {hh[0], hh[1], hh[2], hh[3]};
                    const lr_u32x4 pm = {mm[0], mm[1], mm[2], mm[3]};
                    const lr_u32x4 pl = {ll[0], ll[1], ll[2], ll[3]};
                    C[t] = lr_mfma_k32(ph, bv, C[t]);
                    C[t] = lr_mfma_k32(pm, bv, C[t]);
                    C[t] = lr_mfma_k32(pl, bv, C[t]);
                } else {
                    C[t] = lr_mfma_k32(*(const lr_u32x4*)&ks[16 * t + mq][wo], bv, C[t]);
                }
            }
            Cp = lr_mfma_k32(av, bv, Cp);
        }
        // lane (gq, n = mq) holds C[t][e] = K_{16t + 4gq + e} . w_n and Cp[e] = k_{t0+4gq+e} . w_n
        if (gq < 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) gram[w][4 * gq + e][mq] = Cp[e];
            if (mq >= 8 && ((mq - 8) >> 2) == gq) kqd[w][mq - 8] = Cp[(mq - 8) & 3];
        }
        __syncthreads();
        // Merge: slot i rewritten by round token s_i < vn takes C'[s_i][n].
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            lr_f32x4 m;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t si = ((uint32_t)(16 * t + 4 * gq + e) - pr) & (uint32_t)(R - 1);
                const float gv = gram[w][si < TS ? si : TS - 1][mq];
                m[e] = si < (uint32_t)vn ? gv : C[t][e];
            }
            *(lr_f32x4*)&prod[w][mq >> 3][vn][16 * t + 4 * gq] = m;
        }
        __syncthreads();

        for (int tt = 0; tt < nt; ++tt) {
            const int64_t g = (b * T + t0 + tt) * a.H + h;
            float vt[EU];
#pragma unroll
            for (int e = 0; e < EU; ++e) vt[e] = vs[tt][uc + e];
            const float al = wave_uniform<true>(tok_ab[0][tt]);
            const float be = wave_uniform<true>(tok_ab[1][tt]);
            const float kq = wave_uniform<true>(kqd[w][tt]);
            float u[EU], y[EU];
#pragma unroll
            for (int e = 0; e < EU; ++e) u[e] = y[e] = 0.0f;
#pragma unroll
            for (int i = 0; i < RS; ++i) {
                const int slot = sg * RS + i;
                const float wu = cl[i] * prod[w][0][tt][slot];
                const float wg = cl[i] * prod[w][1][tt][slot];
                const float wy = (uint32_t)slot == p ? 0.0f : wg;
#pragma unroll
                for (int e = 0; e < EU; ++e) {
                    u[e] = fmaf(wu, Ur[i][e], u[e]);
                    y[e] = fmaf(wy, Ur[i][e], y[e]);
                }
            }
            float d[EU], o[EU];
#pragma unroll
            for (int e = 0; e < EU; ++e) {
                u[e] = column_sum<SG, CL>(u[e]);
                y[e] = column_sum<SG, CL>(y[e]);
                d[e] = be * fmaf(-al, u[e], vt[e]);
                o[e] = a.scale * fmaf(al, y[e], kq * d[e]);
            }
            if (sg == 0) store_run<AT, EU>((AT*)a.o + g * D + uc, o);
#pragma unroll
            for (int i = 0; i < RS; ++i) {
                const bool mine = (uint32_t)(sg * RS + i) == p;
#pragma unroll
                for (int e = 0; e < EU; ++e) Ur[i][e] = mine ? d[e] : Ur[i][e];
                cl[i] = mine ? 1.0f : cl[i] * al;
            }
            p = (p + 1) & (uint32_t)(R - 1);
        }
        // The round's keys replace the slots it wrote (every key product of the round was
        // formed before the barrier that precedes the per-token pass).
        if (su < nt) {
            const lr_u32x4 kr = *(const lr_u32x4*)&kq_raw[0][su][scol / 2];
            uint32_t* dst = &ks[(pr + (uint32_t)su) & (uint32_t)(R - 1)][0];
            if constexpr (F32) {
                // the bf16 keys widen exactly
                *(lr_u32x4*)(dst + scol) = lr_u32x4{kr.x << 16, kr.x & 0xffff0000u,
                                                    kr.y << 16, kr.y & 0xffff0000u};
                *(lr_u32x4*)(dst + scol + 4) = lr_u32x4{kr.z << 16, kr.z & 0xffff0000u,
                                                        kr.w << 16, kr.w & 0xffff0000u};
            } else {
                *(lr_u32x4*)(dst + scol / 2) = kr;
            }
        }
    }

    // Store the slots this call wrote, every weight, and the next slot.
    const uint32_t written = (uint32_t)(T < R ? T : R);
#pragma unroll
    for (int i = 0; i < RS; ++i)
        if ((((uint32_t)(sg * RS + i) - p0) & (uint32_t)(R - 1)) < written)
            store_run<ST, EU>(Uh + (sg * RS + i) * D + uc, Ur[i]);
    __syncthreads();   // the last round's keys are in ks
#pragma unroll
    for (int j = 0; j < KCT; ++j) {
        const int chunk = tid + 128 * j, row = chunk / KCR, cw = (chunk % KCR) * 4;
        if ((((uint32_t)row - p0) & (uint32_t)(R - 1)) < written)
            *(lr_u32x4*)((uint32_t*)(Kh + row * D) + cw) = *(const lr_u32x4*)&ks[row][cw];
    }
    if (w == 0) {
        if (lane % CL == 0) {
#pragma unroll
            for (int i = 0; i < RS; ++i) ch[sg * RS + i] = cl[i];
            if (lane == 0) a.pos[head] = (int32_t)p;
        }
    }
}

// Multi-token calls on a bf16 window with bf16 activations at D = 128 (r = 16 or 32) run each
// round of up to kLrRound tokens in matrix form on the matrix cores. Round tokens n = 0..nt-1
// (window slot p_r the next to be written at the round's start) write slots p_r + n, so slot i
// is rewritten by round token s_i = (i - p_r) mod r if s_i < nt. With A_n = alpha_0 ...
// alpha_{n-1} (the decay of the window's old slots at token n) and G_ns = alpha_{s+1} ...
// alpha_{n-1} (that of the round's own write s), the window before token n is the old slots
// with s_i >= n, weights c_i A_n, plus the round's writes s < n, weights G_ns, so
//     u_n = X_n + sum_{s<n} G_ns (k_s . k_n) delta_s,   X_n = sum_{s_i >= n} c_i A_n (K_i . k_n) U_i
// and delta_n = beta_n (v_n - alpha_n u_n) gives, over the round,
//     Delta = T Z,  T = (I + L)^-1,  Z = diag(beta) V - diag(alpha beta) X,
//     L_ns = beta_n alpha_n G_ns (k_s . k_n) (s < n, strictly lower triangular).
// The readout (the slot token n evicts drops out of y_n; the others decay, delta_n joins) is
//     O = scale (diag(alpha) Y + diag(k . q) Delta) = Y' + M Z,   M = L' T,
//     Y'_n = scale alpha_n sum_{s_i > n} c_i A_n (K_i . q_n) U_i,
//     L'_ns = scale alpha_n G_ns (k_s . q_n) (s < n),  L'_nn = scale (k_n . q_n).
// Per round: the key products K_i . [k | q] and the round's Gram (bf16 16 x 16 x 32, as exact
// bf16 operands into fp32), then on fp32 16 x 16 x 4 products over the lane's write columns
// one product of the [X; Y'] weights (16 x r, the key products times c_i, the decays and the
// masks) with the window's writes (r x 128), and one of [T; M] (16 x 8, formed by forward
// substitution on eight lanes) with Z. Rows 0..7 of the results are Delta, rows 8..15 the
// outputs; the rewritten slots take their rows of Delta. Both waves of a head form every
// product over their own 64 write columns.
template <int R>
__global__ __launch_bounds__(128) void gdn_lowrank_round_kernel(LowrankArgs a) {
    constexpr int D = 128;
    using AT = uint16_t;
    using ST = uint16_t;
    static_assert(R == 16 || R == 32, "16- or 32-slot windows");
    constexpr int NTL = R / 16;     // 16-slot tiles of the key products
    constexpr int NS = R / 4;       // window slots per lane in the write products
    constexpr int TS = kLrRound;    // tokens per round
    static_assert(TS == 8, "a round's k and q fill the 16 product columns");
    constexpr int VST = D + 4;      // row stride of the staged v (rows 4 apart in other banks)
    constexpr int KST = D / 2 + 4;  // row stride (words) of staged keys: rows in other banks
    __shared__ alignas(16) uint32_t ks[R][KST];              // the window's keys (bf16 pairs)
    __shared__ alignas(16) uint32_t kq_raw[2][TS][KST];      // the round's k and q (bf16 pairs)
    __shared__ alignas(16) float vs[TS][VST];                // the round's v
    __shared__ float tok_ab[2][TS];                          // [alpha, beta][token]
    __shared__ float dec[2][TS + 1];                         // prefix / suffix decay products
    __shared__ float gram[2][16][TS + 1];                    // per wave: [k | q]_n . k_s at [n][s]
    __shared__ float lmat[2][2][TS][TS];                     // per wave: L, L'
    __shared__ alignas(16) float tm[2][16][TS];              // per wave: [T; M]
    // Per wave: Delta on its columns. It shares the staged k and q's storage: every read of
    // those in a round (key products, key replacement) is behind the barrier that precedes the
    // first write of Delta, and the next round stages after its own barrier.
    static_assert(sizeof(float) * 2 * TS * 64 <= sizeof(kq_raw), "Delta fits the staging");
    float (*dl)[TS][64] = reinterpret_cast<float (*)[TS][64]>(&kq_raw[0][0][0]);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t head = blockIdx.x;
    const int64_t b = head / a.H;
    const int h = (int)(head - b * a.H);
    const int gq = lane >> 4, mq = lane & 15;           // matrix-core lane coordinates
    const int col0 = 64 * w + 4 * mq;                    // this lane's four write columns

    ST* Uh = (ST*)a.U + head * (R * D);
    ST* Kh = (ST*)a.K + head * (R * D);
    float* ch = a.c + head * R;

    // Staging: thread tid moves token su = tid / 16, columns 8 (tid % 16) .. + 7 of k, q and v;
    // tokens past the round are staged as zeros with alpha = beta = 0, which makes their rows
    // and columns of every product below exactly zero. A round's loads are issued one round
    // ahead (the first with the window's), so they land while the previous round computes.
    const int su = tid >> 4, scol = (tid & 15) * 8;
    const int64_t tok_stride = (int64_t)a.H * D;
    const int T = a.T;
    lr_u32x4 rk, rq, rv;
    float gab;
    auto stage_loads = [&](int t0) {
        const int nt = min(TS, T - t0);
        rk = rq = rv = lr_u32x4{0u, 0u, 0u, 0u};
        if (su < nt) {
            const int64_t off = ((b * T + t0) * a.H + h) * D + su * tok_stride + scol;
            rk = *(const lr_u32x4*)((const AT*)a.k + off);
            rq = *(const lr_u32x4*)((const AT*)a.q + off);
            rv = *(const lr_u32x4*)((const AT*)a.v + off);
        }
        gab = 0.0f;
        if (tid < 2 * TS && (tid & 7) < nt) {
            const int64_t gu = (b * T + t0 + (tid & 7)) * a.H + h;
            gab = tid < TS ? a.alpha[gu] : a.beta[gu];
        }
    };
    stage_loads(0);

    // The window's keys in LDS, one copy per head (thread tid moves 16-byte chunks
    // tid + 128 j: slot chunk / 16, columns 8 (chunk % 16) .. + 7).
    lr_u32x4 kc[R / 8];
#pragma unroll
    for (int j = 0; j < R / 8; ++j) {
        const int chunk = tid + 128 * j, row = chunk >> 4, cw8 = (chunk & 15) * 8;
        kc[j] = __builtin_nontemporal_load((const lr_u32x4*)(Kh + row * D + cw8));
    }
    // Writes and weights: lane (gq, mq) holds slot slot_of(s) = 16 (s / 4) + 4 gq + s % 4 (the
    // slot whose key products it holds as C[s / 4][s % 4]), columns col0 .. col0 + 3.
    auto slot_of = [&](int s) { return 16 * (s >> 2) + 4 * gq + (s & 3); };
    float Uw[NS][4], cw[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        load_run<ST, 4, kLrStateNT>(Uh + slot_of(s) * D + col0, Uw[s]);
        cw[s] = ch[slot_of(s)];
    }
    const uint32_t p0 = (uint32_t)a.pos[head] & (uint32_t)(R - 1);
    uint32_t p = p0;
#pragma unroll
    for (int j = 0; j < R / 8; ++j) {
        const int chunk = tid + 128 * j, row = chunk >> 4, cw8 = (chunk & 15) * 8;
        *(lr_u32x4*)&ks[row][cw8 / 2] = kc[j];
    }

    for (int t0 = 0; t0 < T; t0 += TS) {
        const int nt = min(TS, T - t0);
        const uint32_t pr = p;   // slot of the round's first token
        __syncthreads();         // the previous round's readers are done with the buffers
        *(lr_u32x4*)&kq_raw[0][su][scol / 2] = rk;   // (the first round's barrier also covers ks)
        *(lr_u32x4*)&kq_raw[1][su][scol / 2] = rq;
        {
            const uint32_t wv[4] = {rv.x, rv.y, rv.z, rv.w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = Elt<AT>::get(wv[e >> 1], e & 1);
            *(lr_f32x4*)&vs[su][scol] = lr_f32x4{f[0], f[1], f[2], f[3]};
            *(lr_f32x4*)&vs[su][scol + 4] = lr_f32x4{f[4], f[5], f[6], f[7]};
        }
        if (tid < 2 * TS) tok_ab[tid >> 3][tid & 7] = gab;
        if (t0 + TS < T) stage_loads(t0 + TS);
        __syncthreads();
        // Decays: dec[0][j] = alpha_0 ... alpha_{j-1} (A_j), dec[1][j] = alpha_j ... alpha_{nt-1}.
        if (tid < 2 * (TS + 1)) {
            const int j = tid % (TS + 1);
            const bool suffix = tid > TS;
            float pd = 1.0f;
#pragma unroll
            for (int m = 0; m < TS; ++m) {
                const bool in = suffix ? (m >= j && m < nt) : m < j;
                pd = in ? pd * tok_ab[0][m] : pd;
            }
            dec[suffix ? 1 : 0][j] = pd;
        }

        // Key products: C[t][e] = K_{16t + 4gq + e} . w_mq for every slot, and the round's Gram
        // Cp[e] = k_{4gq + e} . w_mq, with w_n = k_n for n < 8 and q_{n-8} for n >= 8.
        lr_f32x4 C[NTL], Cp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NTL; ++t) C[t] = lr_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int wo = (8 * gq + 32 * s) / 2;
            const lr_u32x4 bv = *(const lr_u32x4*)&kq_raw[mq >> 3][mq & 7][wo];
            const lr_u32x4 av = *(const lr_u32x4*)&kq_raw[0][mq & 7][wo];   // rows >= 8 unused
#pragma unroll
            for (int t = 0; t < NTL; ++t)
                C[t] = lr_mfma_k32(*(const lr_u32x4*)&ks[16 * t + mq][wo], bv, C[t]);
            Cp = lr_mfma_k32(av, bv, Cp);
        }
        if (gq < 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) gram[w][mq][4 * gq + e] = Cp[e];
        }
        __syncthreads();

        // Row factors of this lane's product row mq: token m = mq % 8 of X (mq < 8) or Y'
        // (mq >= 8); X rows take the old slots with s_i >= m, Y' rows those with s_i > m.
        const int tokr = mq & 7;
        const float am = dec[0][tokr], alr = tok_ab[0][tokr], ber = tok_ab[1][tokr];
        const float rf = mq < 8 ? alr * ber * am : a.scale * alr * am;
        const uint32_t thr = mq < 8 ? (uint32_t)mq : (uint32_t)(mq - 7);
        // [alpha beta X; Y'] over the window's old slots: 16 x r weights times r x 128 writes
        // (issued before the solve below, which runs on the vector ALUs meanwhile).
        lr_f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = lr_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint32_t si = ((uint32_t)slot_of(s) - pr) & (uint32_t)(R - 1);
            const float wgt = si >= thr ? rf * cw[s] * C[s >> 2][s & 3] : 0.0f;
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] = lr_mfma4(wgt, Uw[s][t], acc[t]);
        }

        // Every key product of the round is formed: the round's keys replace the slots it
        // writes (read again by the next round's products, after its barriers).
        if (su < nt)
            *(lr_u32x4*)&ks[(pr + (uint32_t)su) & (uint32_t)(R - 1)][scol / 2] =
                *(const lr_u32x4*)&kq_raw[0][su][scol / 2];

        // L and L': lane (n, s) = (lane / 8, lane % 8), decays as running products (never
        // ratios). Tokens past the round have zero gates and keys, so their entries are zero.
        {
            const int nn = lane >> 3, ss = lane & 7;
            float gm = 1.0f;
#pragma unroll
            for (int m = 1; m < TS - 1; ++m) gm = (m > ss && m < nn) ? gm * tok_ab[0][m] : gm;
            const float an = tok_ab[0][nn], bn = tok_ab[1][nn];
            const float gkk = gram[w][nn][ss], gkq = gram[w][8 + nn][ss];
            lmat[w][0][nn][ss] = ss < nn ? bn * an * gm * gkk : 0.0f;
            lmat[w][1][nn][ss] = ss < nn ? a.scale * an * gm * gkq : ss == nn ? a.scale * gkq : 0.0f;
        }
        __syncthreads();
        // T = (I + L)^-1 by forward substitution and M = L' T, column c = lane % 8 (lanes 0..7
        // store it).
        {
            const int cc = lane & 7;
            float x[TS];
#pragma unroll
            for (int nn = 0; nn < TS; ++nn) {
                float acc1 = nn == cc ? 1.0f : 0.0f;
#pragma unroll
                for (int ss = 0; ss < nn; ++ss) acc1 = fmaf(-lmat[w][0][nn][ss], x[ss], acc1);
                x[nn] = acc1;
            }
            if (lane < TS) {
#pragma unroll
                for (int nn = 0; nn < TS; ++nn) {
                    float acc1 = 0.0f;
#pragma unroll
                    for (int ss = 0; ss <= nn; ++ss) acc1 = fmaf(lmat[w][1][nn][ss], x[ss], acc1);
                    tm[w][nn][cc] = x[nn];
                    tm[w][TS + nn][cc] = acc1;
                }
            }
        }
        __syncthreads();   // [T; M] is in LDS

        // Per tile: Z = diag(beta) V - alpha beta X on rows 0..7 (lanes gq < 2, rows 4 gq + i),
        // zero elsewhere; the accumulator keeps Y' on rows 8..15 and restarts rows 0..7 at zero;
        // then [Delta; O] += [T; M] Z with the contraction index 4 gq + s in step s (each lane's
        // own Z rows are its b operand).
        {
            const lr_f32x4 tv = *(const lr_f32x4*)&tm[w][mq][4 * (gq & 1)];
            const int r0 = 4 * (gq & 1);
            float av[4], bz[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = gq < 2 ? tv[i] : 0.0f;
                bz[i] = tok_ab[1][r0 + i];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float z[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    z[i] = gq < 2 ? fmaf(bz[i], vs[r0 + i][col0 + t], -acc[t][i]) : 0.0f;
                acc[t] = gq < 2 ? lr_f32x4{0.f, 0.f, 0.f, 0.f} : acc[t];
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[t] = lr_mfma4(av[s], z[s], acc[t]);
            }
        }
        if (gq >= 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (gq - 2) + i;
                if (m < nt) {
                    const float ov[4] = {acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
                    store_run<AT, 4>((AT*)a.o + ((b * T + t0 + m) * a.H + h) * D + col0, ov);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(lr_f32x4*)&dl[w][4 * gq + i][4 * mq] =
                    lr_f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
        }
        __syncthreads();
        // The slots the round wrote take their rows of Delta and weight alpha_{s+1} ...
        // alpha_{nt-1}; the others decay by A_nt.
        const float anl = dec[0][nt];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint32_t si = ((uint32_t)slot_of(s) - pr) & (uint32_t)(R - 1);
            if (si < (uint32_t)nt) {
                const lr_f32x4 d = *(const lr_f32x4*)&dl[w][si][4 * mq];
#pragma unroll
                for (int t = 0; t < 4; ++t) Uw[s][t] = d[t];
                cw[s] = dec[1][si + 1];
            } else {
                cw[s] *= anl;
            }
        }
        p = (pr + (uint32_t)nt) & (uint32_t)(R - 1);
    }

    // Store the slots this call wrote, every weight, and the next slot.
    const uint32_t written = (uint32_t)(T < R ? T : R);
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if ((((uint32_t)slot_of(s) - p0) & (uint32_t)(R - 1)) < written)
            store_run<ST, 4>(Uh + slot_of(s) * D + col0, Uw[s]);
    __syncthreads();   // the last round's keys are in ks
#pragma unroll
    for (int j = 0; j < R / 8; ++j) {
        const int chunk = tid + 128 * j, row = chunk >> 4, cw8 = (chunk & 15) * 8;
        if ((((uint32_t)row - p0) & (uint32_t)(R - 1)) < written)
            *(lr_u32x4*)(Kh + row * D + cw8) = *(const lr_u32x4*)&ks[row][cw8 / 2];
    }
    if (w == 0) {
        if (mq == 0) {
#pragma unroll
            for (int s = 0; s < NS; ++s) ch[slot_of(s)] = cw[s];
            if (lane == 0) a.pos[head] = (int32_t)p;
        }
    }
}

template <int D, int R, typename AT, typename ST>
hipError_t launch_typed(const LowrankArgs& a, hipStream_t stream) {
    using G = LrGeo<D, R, AT, ST>;
    const int64_t heads = a.B * a.H;
    // The launch's own status (not hipGetLastError, which would also report, and clear, an
    // error left on this thread by an earlier, unrelated HIP call).
    LowrankArgs args = a;
    void* argv[] = {&args};
    const void* fn = a.T == 1 ? (const void*)gdn_lowrank_kernel<D, R, AT, ST, true>
                              : (const void*)gdn_lowrank_kernel<D, R, AT, ST, false>;
    if constexpr (D == 128 && (R == 16 || R == 32) && std::is_same<AT, uint16_t>::value &&
                  std::is_same<ST, uint16_t>::value) {
        // bf16 window and activations: several tokens take the matrix-core key products, and
        // rounds that are full or nearly so run in matrix form
        if (lr_round_form(a.T)) fn = (const void*)gdn_lowrank_round_kernel<R>;
        else if (a.T > 1) fn = (const void*)gdn_lowrank_mm_kernel<R, ST>;
    }
    if constexpr (D == 128 && R == 16 && std::is_same<AT, uint16_t>::value &&
                  std::is_same<ST, float>::value) {
        // 16-slot fp32 window, bf16 activations: from 4 tokens on, the matrix-core key
        // products (the keys in three exact bf16 parts). B = 256, H = 48, against the vector
        // form: T = 2 41.3 -> 43.5 us (kept on the vector form), T = 4 56.2 -> 53.6, T = 6
        // 79.2 -> 72.3.
        if (a.T >= 4) fn = (const void*)gdn_lowrank_mm_kernel<R, ST>;
    }
    return hipLaunchKernel(fn, dim3((uint32_t)heads), dim3(64 * G::W), argv, 0, stream);
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
