// HIP kernels for the Gated DeltaNet (GDN) recurrent decode step on gfx950 (CDNA4).
//
// The step, per (sequence b, head h) and token t ("GDN tuning limits on Kunlun XPU", section
// 二 背景: a rank-1 update of the per-head state with a decay, after conv and gating):
//     u = S k,   delta = beta (v - alpha u),   S <- alpha S + delta k^T,
//     o = S_new (scale q) = alpha (S q) + delta (k . q)
// which is S_t = alpha S_{t-1}(I - beta k k^T) + beta v k^T, o_t = S_t q_t regrouped so that the
// state is read once and written once.
//
// The work is a stream: per token a head moves its 64 KiB fp32 state (32 KiB bf16/fp16) through
// ~6 flop per element, far below the chip's flop:byte ridge, so no matrix cores are used and
// the layout exists to keep every HBM access a full, coalesced line:
//   * state [B][H][D][D], row i (value dim) contiguous over the key dim;
//   * SPLIT workgroups of WAVES wave64s per (b, h); each wave owns consecutive rows and visits
//     them RPP = 64/LPR at a time ("passes"); LPR lanes hold one state row, every lane a fixed
//     slice of E = D/LPR columns loaded as 16-byte vectors, so a load instruction covers RPP
//     row segments of LPR*16 bytes each (whole 128-byte lines or more);
//   * the whole state tile of a wave is loaded into registers before anything else, kept there
//     across all T tokens of the call, and stored once at the end;
//   * the per-token vectors (q, k, v, alpha, beta) are staged in LDS once per workgroup, up to
//     TCH tokens at a time, while the state loads are in flight;
//   * row dot products S k and S q reduce across the LPR lanes of a row with DPP steps
//     (quad_perm 1032, quad_perm 2301, then row_half_mirror and row_mirror as LPR needs):
//     every lane ends with the same total, bit for bit, and no LDS is touched.
// Per-head scalars are folded instead of scaling vectors: k and q stay raw in LDS and their
// factors (1/|k|, scale/|q| in the fused path) multiply the row totals. For several tokens the
// registers hold S' = S / c with c the running product of alpha over the call's tokens, which
// turns the update into one FMA per element (S' += (delta / c) k); c is folded back before the
// store, or earlier if it leaves [2^-64, 2^64] (see recur_tokens). With several tokens per
// staged round the wave also forms each token's k . q once instead of once per row.
// The fused kernel replaces the staging by the conv (kernel 4) + SiLU + L2-norm + gate
// prologue of the same chain, computed by the workgroup for the 3*D channels its head owns; it
// is also the only reader and writer of those channels' conv state.
// A few tokens (up to 8) on a bf16 state with bf16 activations take the chunk form instead
// (gdn_decode_chunk_kernel, gdn_verify_chunk_kernel): products with the stored state as packed
// bf16 dots on the loaded words, and the state updated once; see there.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_launch.h"

namespace gdn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------ bf16 <-> fp32

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to two bf16 (lo in bits 0-15), round to nearest even, NaN stays NaN: gfx950's
// v_cvt_pk_bf16_f32, whose results were checked against the bit-level definition
// (u + 0x7fff + ((u >> 16) & 1)) >> 16, with NaN -> (u >> 16) | 0x40, on all 2^32 inputs.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return f32x2_to_bf16x2(f, 0.0f) & 0xffffu; }

// fp16 (IEEE binary16) storage: _Float16. Stores round to nearest even (v_cvt_pk_f16_f32; not
// the round-toward-zero pkrtz form); loads widen exactly.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f32x2_to_f16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

__device__ __forceinline__ f32x2_t f16x2_to_f32x2(uint32_t bits) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2_t, bits), f32x2_t);
}

// Storage element types: float (fp32), uint16_t (bf16 bits), _Float16 (fp16).
template <typename T> struct is_f16 { static constexpr bool value = false; };
template <> struct is_f16<_Float16> { static constexpr bool value = true; };

// Two floats packed into one 32-bit word of the 2-byte storage type ST.
template <typename ST>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if constexpr (is_f16<ST>::value) return f32x2_to_f16x2(lo, hi);
    else return f32x2_to_bf16x2(lo, hi);
}

// Element e (0 = low half, 1 = high half) of a 32-bit word of the 2-byte storage type ST.
template <typename ST>
__device__ __forceinline__ float unpack(uint32_t word, int e) {
    if constexpr (is_f16<ST>::value) {
        const f32x2_t f = f16x2_to_f32x2(word);
        return e ? f.y : f.x;
    } else {
        return e ? __uint_as_float(word & 0xffff0000u) : bf16_to_f32(word & 0xffffu);
    }
}

// A value every lane of the wave holds identically, moved to a scalar register.
__device__ __forceinline__ float uniform(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float act_to_f32(float x) { return x; }
__device__ __forceinline__ float act_to_f32(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float act_to_f32(_Float16 x) { return (float)x; }
template <typename AT> __device__ __forceinline__ AT act_from_f32(float x);
template <> __device__ __forceinline__ float act_from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t act_from_f32<uint16_t>(float x) {
    return (uint16_t)f32_to_bf16(x);
}
template <> __device__ __forceinline__ _Float16 act_from_f32<_Float16>(float x) {
    return __builtin_bit_cast(_Float16, (uint16_t)(f32x2_to_f16x2(x, 0.0f) & 0xffffu));
}

// ------------------------------------------------------------------------ DPP reductions

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR lanes (4, 8 or 16); every lane of a group receives the same
// value.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    static_assert(LPR == 4 || LPR == 8 || LPR == 16, "groups of 4, 8 or 16 lanes");
    x += dpp_mov<0xB1>(x);                           // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_mov<0x4E>(x);                           // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LPR >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror: i <- 7 - i in 8 lanes
    if constexpr (LPR >= 16) x += dpp_mov<0x140>(x); // row_mirror: i <- 15 - i in 16 lanes
    return x;
}

// Sum over a whole wave64; the result is wave-uniform.
__device__ __forceinline__ float wave_sum64(float x) {
    x = row_sum<16>(x);
    const int xi = __builtin_bit_cast(int, x);
    float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
    float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
    float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
    float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
    return (r0 + r1) + (r2 + r3);
}

// ------------------------------------------------------------------------ vector memory

template <int NBYTES> struct Words { uint32_t w[(NBYTES + 3) / 4]; };

template <int NBYTES, bool NT>
__device__ __forceinline__ Words<NBYTES> gload(const void* p) {
    Words<NBYTES> r;
    if constexpr (NBYTES == 16) {
        const u32x4* a = (const u32x4*)p;
        u32x4 x = NT ? __builtin_nontemporal_load(a) : *a;
        r.w[0] = x.x; r.w[1] = x.y; r.w[2] = x.z; r.w[3] = x.w;
    } else if constexpr (NBYTES == 8) {
        const u32x2* a = (const u32x2*)p;
        u32x2 x = NT ? __builtin_nontemporal_load(a) : *a;
        r.w[0] = x.x; r.w[1] = x.y;
    } else if constexpr (NBYTES == 4) {
        const uint32_t* a = (const uint32_t*)p;
        r.w[0] = NT ? __builtin_nontemporal_load(a) : *a;
    } else {
        static_assert(NBYTES == 2, "unsupported access width");
        r.w[0] = *(const uint16_t*)p;
    }
    return r;
}

template <int NBYTES, bool NT>
__device__ __forceinline__ void gstore(void* p, const Words<NBYTES>& r) {
    if constexpr (NBYTES == 16) {
        u32x4 x = {r.w[0], r.w[1], r.w[2], r.w[3]};
        if (NT) __builtin_nontemporal_store(x, (u32x4*)p); else *(u32x4*)p = x;
    } else if constexpr (NBYTES == 8) {
        u32x2 x = {r.w[0], r.w[1]};
        if (NT) __builtin_nontemporal_store(x, (u32x2*)p); else *(u32x2*)p = x;
    } else if constexpr (NBYTES == 4) {
        if (NT) __builtin_nontemporal_store(r.w[0], (uint32_t*)p); else *(uint32_t*)p = r.w[0];
    } else {
        static_assert(NBYTES == 2, "unsupported access width");
        *(uint16_t*)p = (uint16_t)r.w[0];
    }
}

// ------------------------------------------------------------------------ tile geometry

// A kernel instance: head dim D, state type ST, WAVES wave64s per workgroup, SPLIT workgroups
// per head (each owning D/SPLIT consecutive rows), TCH tokens staged in LDS per round,
// nontemporal state loads (NTL) / stores (NTS), the tile order over XCDs (GRP consecutive
// tiles per XCD, see tile_index), and LPR lanes per state row.
template <int D_, typename ST_, int WAVES_, int SPLIT_, int TCH_, bool NTL_, bool NTS_,
          int GRP_ = 1, int LPR_ = 16>
struct Geo {
    static constexpr int D = D_;
    using ST = ST_;
    static constexpr int WAVES = WAVES_, SPLIT = SPLIT_, TCH = TCH_, GRP = GRP_, LPR = LPR_;
    static constexpr bool NTL = NTL_, NTS = NTS_;
    static constexpr int E = D / LPR;                        // state columns per lane
    static constexpr int ES = (int)sizeof(ST);               // bytes per state element
    static constexpr int VW = (E * ES >= 16) ? 16 / ES : E;  // elements per vector access
    static constexpr int NCH = E / VW;                       // vector accesses per row per lane
    static constexpr int VB = VW * ES;                       // bytes per vector access
    static constexpr int NT = 64 * WAVES;                    // threads per workgroup
    static constexpr int RPP = 64 / LPR;                     // rows per pass of a wave
    static constexpr int RPG = D / SPLIT;                    // rows per workgroup
    static constexpr int RPW = RPG / WAVES;                  // rows per wave
    static constexpr int P = RPW / RPP;                      // passes per wave
    static_assert(LPR == 4 || LPR == 8 || LPR == 16, "lanes per row");
    static_assert(D % LPR == 0 && E >= 1 && E % VW == 0, "bad head dim");
    static_assert(D % SPLIT == 0 && RPG % WAVES == 0, "bad split");
    static_assert(RPW % RPP == 0 && P >= 1 && P <= LPR, "bad wave count");
    static_assert(TCH >= 1, "bad token chunk");
    static_assert(GRP >= 1, "bad tile group");
    // Column held by lane l (0..LPR-1 within its row group) as its element e.
    static __device__ __forceinline__ int col(int l, int e) {
        return (e / VW) * (LPR * VW) + l * VW + (e % VW);
    }
};

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup i runs on XCD i % 8), and
// each XCD has its own L2. The tile order decides which tiles share an L2: runs of GRP
// consecutive tiles go to one XCD, consecutive runs to consecutive XCDs. GRP = 1 is the plain
// order (consecutive tiles on different XCDs); GRP = SPLIT keeps all tiles of a head on one XCD
// (its q, k and v are fetched into one L2). Tiles past the last multiple of 8 * GRP keep the
// plain order. The map is a bijection of [0, n) for n = gridDim.x.
template <int GRP>
__device__ __forceinline__ uint32_t tile_index(uint32_t bid, uint32_t n) {
    if constexpr (GRP == 1) {
        return bid;
    } else {
        const uint32_t grouped = (n / (8u * GRP)) * (8u * GRP);
        if (bid >= grouped) return bid;
        const uint32_t x = bid & 7u, i = bid >> 3;
        return ((i / GRP) * 8u + x) * GRP + (i % GRP);
    }
}

// Per-token vectors of one head, raw (k and q unscaled), and the per-token scalars.
template <int D, int TCH>
struct TokLds {
    alignas(16) float q[TCH][D];
    alignas(16) float k[TCH][D];
    alignas(16) float v[TCH][D];
    float alpha[TCH];
    float beta[TCH];
    float qf[TCH];  // factor of q in the readout: scale (times 1/|q| in the fused path)
    float kf[TCH];  // factor of k: 1 (or 1/|k| in the fused path)
};

// Load the wave's state rows into registers: S[p][e] = state[row0 + p*RPP][col(l, e)].
template <class G>
__device__ __forceinline__ void load_state(const typename G::ST* __restrict__ Sg, int row0, int l,
                                           float (&S)[G::P][G::E]) {
    using ST = typename G::ST;
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
        const ST* rowp = Sg + (size_t)(row0 + p * G::RPP) * G::D;
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) {
            Words<G::VB> w = gload<G::VB, G::NTL>(rowp + c * G::LPR * G::VW + l * G::VW);
#pragma unroll
            for (int e = 0; e < G::VW; ++e) {
                float x;
                if constexpr (sizeof(ST) == 4) {
                    x = __uint_as_float(w.w[e]);
                } else {
                    x = unpack<ST>(w.w[e >> 1], e & 1);
                }
                S[p][c * G::VW + e] = x;
            }
        }
    }
}

template <class G>
__device__ __forceinline__ void store_state(typename G::ST* __restrict__ Sg, int row0, int l,
                                            const float (&S)[G::P][G::E]) {
    using ST = typename G::ST;
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
        ST* rowp = Sg + (size_t)(row0 + p * G::RPP) * G::D;
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) {
            Words<G::VB> w;
            if constexpr (sizeof(ST) == 4) {
#pragma unroll
                for (int e = 0; e < G::VW; ++e) w.w[e] = __float_as_uint(S[p][c * G::VW + e]);
            } else {
#pragma unroll
                for (int e = 0; e < G::VW; e += 2) {
                    const float hi = (e + 1 < G::VW) ? S[p][c * G::VW + e + 1] : 0.0f;
                    w.w[e >> 1] = pack2<ST>(S[p][c * G::VW + e], hi);
                }
            }
            gstore<G::VB, G::NTS>(rowp + c * G::LPR * G::VW + l * G::VW, w);
        }
    }
}

// ------------------------------------------------------------------------ one token

// kq = k_raw . q_raw of one token from the lane's E columns, reduced over the row's lanes.
template <class G>
__device__ __forceinline__ float row_kq(const float (&kk)[G::E], const float (&qq)[G::E]) {
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < G::E; ++e) kq = fmaf(kk[e], qq[e], kq);
    return row_sum<G::LPR>(kq);
}

// Row totals shared by both token forms: per pass, u = S k_raw and w = S q_raw (S as held in
// registers), reduced over the row's lanes.
template <class G>
__device__ __forceinline__ void row_dots(const float (&S)[G::P][G::E], const float (&kk)[G::E],
                                         const float (&qq)[G::E], float (&u)[G::P],
                                         float (&w)[G::P]) {
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
        float su = 0.f, sw = 0.f;
#pragma unroll
        for (int e = 0; e < G::E; ++e) {
            su = fmaf(S[p][e], kk[e], su);
            sw = fmaf(S[p][e], qq[e], sw);
        }
        u[p] = su;
        w[p] = sw;
    }
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
        u[p] = row_sum<G::LPR>(u[p]);
        w[p] = row_sum<G::LPR>(w[p]);
    }
}

// What a token step returns on the lane with l == p of each row group, for the row of pass p:
// its readout o and its write coefficient dk (the new state is alpha S + dk k_raw^T).
struct RowOut {
    float o, dk;
};

// One token with S held as is. k = kf k_raw, q = qf q_raw, kq = k_raw . q_raw:
//   u = kf (S k_raw);  delta = beta (v - alpha u);  S <- alpha S + (delta kf) k_raw;
//   o = qf (alpha (S q_raw) + (delta kf) kq).
template <class G>
__device__ __forceinline__ RowOut token_plain(float (&S)[G::P][G::E], const float (&kk)[G::E],
                                             const float (&qq)[G::E], const float (&vr)[G::P],
                                             float a, float bt, float kf, float qf, float kq,
                                             int l) {
    float u[G::P], w[G::P];
    row_dots<G>(S, kk, qq, u, w);
    RowOut r = {0.f, 0.f};
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
        const float delta = bt * (vr[p] - a * (kf * u[p]));
        const float dk = delta * kf;
#pragma unroll
        for (int e = 0; e < G::E; ++e) S[p][e] = fmaf(dk, kk[e], a * S[p][e]);
        const float op = qf * fmaf(a, w[p], dk * kq);
        r.o = (l == p) ? op : r.o;
        r.dk = (l == p) ? dk : r.dk;
    }
    return r;
}

// One token with registers holding S' = S / c; cn = c alpha (in [2^-64, 2^64]) is the new
// scale. With u' = S' k_raw, w' = S' q_raw:
//   delta = beta (v - alpha kf c u');  S' <- S' + (delta kf / cn) k_raw;
//   o = qf (cn w' + (delta kf) (k_raw . q_raw)),
// since alpha S + dk k = cn (S' + dk k / cn) and alpha S q = cn S' q: one FMA per element.
template <class G>
__device__ __forceinline__ RowOut token_scaled(float (&S)[G::P][G::E], const float (&kk)[G::E],
                                              const float (&qq)[G::E], const float (&vr)[G::P],
                                              float a, float bt, float kf, float qf, float kq,
                                              float c, float cn, int l) {
    float u[G::P], w[G::P];
    row_dots<G>(S, kk, qq, u, w);
    const float kc = kf * c, inv_cn = __builtin_amdgcn_rcpf(cn);
    RowOut r = {0.f, 0.f};
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
        const float delta = bt * (vr[p] - a * (kc * u[p]));
        const float dk = delta * kf;
        const float coef = dk * inv_cn;
#pragma unroll
        for (int e = 0; e < G::E; ++e) S[p][e] = fmaf(coef, kk[e], S[p][e]);
        const float op = qf * fmaf(cn, w[p], dk * kq);
        r.o = (l == p) ? op : r.o;
        r.dk = (l == p) ? dk : r.dk;
    }
    return r;
}

template <class G>
__device__ __forceinline__ void scale_state(float (&S)[G::P][G::E], float c) {
#pragma unroll
    for (int p = 0; p < G::P; ++p)
#pragma unroll
        for (int e = 0; e < G::E; ++e) S[p][e] *= c;
}

// Per-token operands of a lane: its E columns of raw k and q, the v entries of its rows, and
// the token's scalars (wave-uniform, moved to scalar registers).
template <class G>
struct TokenOperands {
    float kk[G::E], qq[G::E], vr[G::P];
    float a, bt, kf, qf;
    __device__ __forceinline__ void load(const TokLds<G::D, G::TCH>& L, int tt, int row0, int l) {
        if constexpr (G::VW % 4 == 0) {
            // columns e..e+3 of a lane are contiguous and 16-byte aligned: ds_read_b128
#pragma unroll
            for (int e = 0; e < G::E; e += 4) {
                const float4 k4 = *(const float4*)&L.k[tt][G::col(l, e)];
                const float4 q4 = *(const float4*)&L.q[tt][G::col(l, e)];
                kk[e] = k4.x; kk[e + 1] = k4.y; kk[e + 2] = k4.z; kk[e + 3] = k4.w;
                qq[e] = q4.x; qq[e + 1] = q4.y; qq[e + 2] = q4.z; qq[e + 3] = q4.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < G::E; ++e) {
                kk[e] = L.k[tt][G::col(l, e)];
                qq[e] = L.q[tt][G::col(l, e)];
            }
        }
#pragma unroll
        for (int p = 0; p < G::P; ++p) vr[p] = L.v[tt][row0 + p * G::RPP];
        a = uniform(L.alpha[tt]);
        bt = uniform(L.beta[tt]);
        kf = uniform(L.kf[tt]);
        qf = uniform(L.qf[tt]);
    }
};

// k_raw . q_raw of every token of a round, formed once per wave (with several tokens per round):
// the 64 / TCH lanes of group j sum token j's products, so token tt reads its value from lane
// tt * (64 / TCH). Lanes of tokens past the round's count read stale LDS and are never used.
template <class G>
__device__ __forceinline__ float round_kq(const TokLds<G::D, G::TCH>& L, int lane) {
    constexpr int LT = 64 / G::TCH, EL = G::D / LT, VK = EL < 4 ? EL : 4;
    static_assert(LT == 4 || LT == 8 || LT == 16, "token groups of 4, 8 or 16 lanes");
    static_assert(EL % VK == 0 && (VK == 2 || VK == 4), "columns per lane");
    const int tt = lane / LT, j = lane % LT;
    float kq = 0.f;
    // lane j sums the VK-column blocks j, j + LT, j + 2 LT, ... of its token
#pragma unroll
    for (int e = 0; e < EL; e += VK) {
        const int at = e * LT + VK * j;
        if constexpr (VK == 4) {
            const float4 k4 = *(const float4*)&L.k[tt][at];
            const float4 q4 = *(const float4*)&L.q[tt][at];
            kq = fmaf(k4.x, q4.x, kq);
            kq = fmaf(k4.y, q4.y, kq);
            kq = fmaf(k4.z, q4.z, kq);
            kq = fmaf(k4.w, q4.w, kq);
        } else {
            const float2 k2 = *(const float2*)&L.k[tt][at];
            const float2 q2 = *(const float2*)&L.q[tt][at];
            kq = fmaf(k2.x, q2.x, kq);
            kq = fmaf(k2.y, q2.y, kq);
        }
    }
    return row_sum<LT>(kq);
}

// The recurrence for `nt` staged tokens. `obase` points at o[b][t0][h][0]; consecutive tokens
// are `ostride` elements apart. The row of pass p is row0 + p*RPP with row0 = rbase + g, rbase
// the wave's first row; the lane with l == p of row group g writes o for that row, so one
// store covers all the wave's rows.
// With MULTI the registers hold S / c and `c` carries the scale across rounds; every token
// runs the scaled form. A token whose c alpha would leave [2^-64, 2^64] (alpha = 0, very small
// or large, NaN) first multiplies the registers by c and then by its alpha, and runs with
// c = alpha = 1 (exactly the plain form's update). One loop body with the state defined only
// by the update's FMAs lets the compiler keep the state registers in place across tokens (two
// inlined token forms made it copy them every token and raised the register count).
// With DELTA, each token's write coefficients dk (one per row) also go to `dbase`, laid out
// like o but in fp32.
template <class G, bool MULTI, typename AT, bool DELTA = false>
__device__ __forceinline__ void recur_tokens(float (&S)[G::P][G::E],
                                             const TokLds<G::D, G::TCH>& L, int nt, int rbase,
                                             int g, int l, AT* __restrict__ obase, size_t ostride,
                                             float& c, float* __restrict__ dbase = nullptr) {
    const int row0 = rbase + g;
    auto put_o = [&](int tt, RowOut r) {
        if (l < G::P) {
            const size_t at = (size_t)tt * ostride + rbase + l * G::RPP + g;
            obase[at] = act_from_f32<AT>(r.o);
            if constexpr (DELTA) dbase[at] = r.dk;
        }
    };
    constexpr bool kRoundKq = G::TCH >= 4;
    float kqv = 0.f;
    if constexpr (kRoundKq) kqv = round_kq<G>(L, g * G::LPR + l);
    auto kq_of = [&](int tt, const TokenOperands<G>& t) {
        if constexpr (kRoundKq) {
            return __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                __builtin_bit_cast(int, kqv), tt * (64 / G::TCH)));
        } else {
            return row_kq<G>(t.kk, t.qq);
        }
    };
    if constexpr (!MULTI) {
        for (int tt = 0; tt < nt; ++tt) {
            TokenOperands<G> t;
            t.load(L, tt, row0, l);
            put_o(tt, token_plain<G>(S, t.kk, t.qq, t.vr, t.a, t.bt, t.kf, t.qf, kq_of(tt, t), l));
        }
    } else {
        for (int tt = 0; tt < nt; ++tt) {
            TokenOperands<G> t;
            t.load(L, tt, row0, l);
            float a = t.a, cn = c * a;
            if (!(cn >= 0x1p-64f && cn <= 0x1p64f)) {
                // Fold c and then this token's alpha into the registers (two roundings, as
                // the plain form takes them); the token then runs with c = alpha = 1.
                scale_state<G>(S, c);
                scale_state<G>(S, a);
                a = 1.0f;
                c = 1.0f;
                cn = 1.0f;
            }
            put_o(tt, token_scaled<G>(S, t.kk, t.qq, t.vr, a, t.bt, t.kf, t.qf, kq_of(tt, t), c,
                                      cn, l));
            c = cn;
        }
    }
}

// ------------------------------------------------------------------------ token staging

// The per-token vectors a workgroup needs -- q and k in full, v for its own rows -- moved to
// LDS in 16-byte chunks. fetch() issues the global loads into registers and commit() converts
// and writes them, so the first round's loads can be issued before the state loads (the wait
// for them then does not wait for the state) and each lane waits once, not once per element.
template <class G, typename AT>
struct TokenStage {
    static constexpr int D = G::D;
    static constexpr int CHK = 16 / (int)sizeof(AT);          // elements per 16-byte chunk
    static constexpr int NQ = D / CHK, NV = G::RPG / CHK;     // chunks of q (= of k), of v
    static constexpr int NCH = 2 * NQ + NV;                   // chunks per token
    static constexpr int CPL = (G::TCH * NCH + G::NT - 1) / G::NT;  // chunks per lane, max
    static_assert(D % CHK == 0 && G::RPG % CHK == 0, "rows must fill whole 16-byte chunks");
    u32x4 raw[CPL];
    float al = 0.f, be = 0.f;

    __device__ __forceinline__ void fetch(const AT* __restrict__ q, const AT* __restrict__ k,
                                          const AT* __restrict__ v, const float* __restrict__ alpha,
                                          const float* __restrict__ beta, int64_t b, int T, int H,
                                          int h, int part, int t0, int nt, int tid) {
#pragma unroll
        for (int s = 0; s < CPL; ++s) {
            const int c = tid + s * G::NT;
            if (c < nt * NCH) {
                const int tt = c / NCH, r = c - tt * NCH;
                const size_t tok = ((size_t)b * T + t0 + tt) * H + h;
                const AT* src = r < NQ ? q + tok * D + r * CHK
                              : r < 2 * NQ ? k + tok * D + (r - NQ) * CHK
                                           : v + tok * D + part * G::RPG + (r - 2 * NQ) * CHK;
                raw[s] = *(const u32x4*)src;
            }
        }
        if (tid < nt) {
            const size_t tok = ((size_t)b * T + t0 + tid) * H + h;
            al = alpha[tok];
            be = beta[tok];
        }
    }

    __device__ __forceinline__ void commit(TokLds<D, G::TCH>& L, int part, int nt, int tid,
                                           float scale) const {
#pragma unroll
        for (int s = 0; s < CPL; ++s) {
            const int c = tid + s * G::NT;
            if (c < nt * NCH) {
                const int tt = c / NCH, r = c - tt * NCH;
                float* dst = r < NQ ? &L.q[tt][r * CHK]
                           : r < 2 * NQ ? &L.k[tt][(r - NQ) * CHK]
                                        : &L.v[tt][part * G::RPG + (r - 2 * NQ) * CHK];
                float f[CHK];
                const uint32_t wv[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
                for (int e = 0; e < CHK; ++e) {
                    if constexpr (sizeof(AT) == 4) f[e] = __uint_as_float(wv[e]);
                    else f[e] = unpack<AT>(wv[e >> 1], e & 1);
                }
#pragma unroll
                for (int e = 0; e < CHK; e += 4) *(float4*)&dst[e] = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
            }
        }
        if (tid < nt) {
            L.alpha[tid] = al;
            L.beta[tid] = be;
            L.qf[tid] = scale;
            L.kf[tid] = 1.0f;
        }
    }
};

// ------------------------------------------------------------------------ decode kernel

template <class G, bool MULTI, typename AT>
__global__ __launch_bounds__(G::NT) void gdn_decode_kernel(
    int T, int H, const AT* __restrict__ q, const AT* __restrict__ k, const AT* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    typename G::ST* __restrict__ state, AT* __restrict__ o, float scale) {
    constexpr int D = G::D;
    __shared__ TokLds<D, G::TCH> L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / G::LPR, l = lane % G::LPR;
    const uint32_t tile = tile_index<G::GRP>(blockIdx.x, gridDim.x);
    const int64_t n = tile / G::SPLIT;  // b * H + h
    const int part = (int)(tile - n * G::SPLIT);
    const int64_t b = n / H;
    const int h = (int)(n - b * H);
    typename G::ST* Sg = state + (size_t)n * D * D;
    const int rbase = part * G::RPG + wave * G::RPW;

    float S[G::P][G::E];
    float c = 1.0f;
    if constexpr (G::TCH == 1) {
        // One token per round (the one-token launch shape): stage q, k and the workgroup's own
        // v rows element by element after the state loads are issued. Measured on MI355X at
        // B=256 H=48 D=128 T=1, this form (vector loads of alpha and beta by the lanes below
        // nt) beats a 16-byte fetch issued before or after the state loads, and a scalar-load
        // variant, by 1-3%; staging only the own v rows instead of all of v: 256.3 -> 253.2 us.
        load_state<G>(Sg, rbase + g, l, S);
        for (int t0 = 0; t0 < T; t0 += G::TCH) {
            const int nt = min(G::TCH, T - t0);
            if (t0 > 0) __syncthreads();  // the previous round's readers are done with L
            // q and k in full, v for the workgroup's own rows only
            constexpr int NE = 2 * D + G::RPG;  // elements staged per token
            for (int i = tid; i < nt * NE; i += G::NT) {
                const int tt = i / NE, r = i - tt * NE;
                const int which = r < D ? 0 : (r < 2 * D ? 1 : 2);
                const int j = which == 2 ? part * G::RPG + (r - 2 * D) : r - which * D;
                const size_t tok = ((size_t)b * T + t0 + tt) * H + h;
                const AT* src = which == 0 ? q : (which == 1 ? k : v);
                const float x = act_to_f32(src[tok * D + j]);
                if (which == 0) L.q[tt][j] = x; else if (which == 1) L.k[tt][j] = x; else L.v[tt][j] = x;
            }
            if (tid < nt) {
                const size_t tok = ((size_t)b * T + t0 + tid) * H + h;
                L.alpha[tid] = alpha[tok];
                L.beta[tid] = beta[tok];
                L.qf[tid] = scale;
                L.kf[tid] = 1.0f;
            }
            __syncthreads();
            recur_tokens<G, MULTI, AT>(S, L, nt, rbase, g, l,
                                       o + (((size_t)b * T + t0) * H + h) * D, (size_t)H * D, c);
        }
    } else {
        TokenStage<G, AT> st;
        st.fetch(q, k, v, alpha, beta, b, T, H, h, part, 0, min(G::TCH, T), tid);
        load_state<G>(Sg, rbase + g, l, S);
        for (int t0 = 0; t0 < T; t0 += G::TCH) {
            const int nt = min(G::TCH, T - t0);
            if (t0 > 0) {
                __syncthreads();  // the previous round's readers are done with L
                st.fetch(q, k, v, alpha, beta, b, T, H, h, part, t0, nt, tid);
            }
            st.commit(L, part, nt, tid, scale);
            __syncthreads();
            recur_tokens<G, MULTI, AT>(S, L, nt, rbase, g, l,
                                       o + (((size_t)b * T + t0) * H + h) * D, (size_t)H * D, c);
        }
    }
    if (MULTI && c != 1.0f) scale_state<G>(S, c);
    store_state<G>(Sg, rbase + g, l, S);
}

// ------------------------------------------------------------------------ chunk-form decode

// A few tokens (3 .. TCH for decode, 1 .. TCH for verify) on a bf16 state with bf16
// activations. The token-by-token form needs S_{t-1} k_t and S_t q_t, two FMAs per state
// element and token on the current fp32 state. Over one call they unroll to products with the
// stored state S0 (the chunk form of the same
// recurrence; "GDN tuning limits on Kunlun XPU", section 三.3 names it):
//     gamma_t = alpha_0 ... alpha_t,  d(t, s) = alpha_{s+1} ... alpha_t  (d(t, t) = 1),
//     S_{t-1} k_t = gamma_{t-1} S0 k_t + sum_{s<t} d(t-1, s) (k_s . k_t) delta_s,
//     delta_t = beta_t (v_t - alpha_t S_{t-1} k_t),
//     o_t = scale (gamma_t S0 q_t + sum_{s<=t} d(t, s) (k_s . q_t) delta_s),
//     S_T = gamma_{T-1} S0 + sum_s d(T-1, s) delta_s k_s^T.
// S0 is the loaded bf16 state and k, q are bf16, so S0 k_t and S0 q_t take one packed bf16 dot
// (v_dot2c_f32_bf16: two products, fp32 accumulation) per two elements on the raw words, with
// no widening; the Gram products k_s . k_t, k_s . q_t are shared by the workgroup through LDS,
// the decays are running products of alpha, and the per-row part is a few scalar operations
// per token; the state is widened, updated and rounded once at the end.

template <int D, int TCH>
struct ChunkLds {
    alignas(16) uint16_t kb[TCH][D];  // k, q as stored (bf16 bits)
    alignas(16) uint16_t qb[TCH][D];
    alignas(16) float k[TCH][D];      // k widened (the final update)
    alignas(16) float v[TCH][D];      // v widened (the workgroup's rows)
    float alpha[TCH], beta[TCH];
    float kk[TCH][TCH];               // k_s . k_t
    float kq[TCH][TCH];               // k_s . q_t
};

typedef __bf16 bf16x2_dot_t __attribute__((ext_vector_type(2)));

// acc + x.lo y.lo + x.hi y.hi for two packed bf16 pairs (fp32 accumulation).
__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_dot_t, x),
                                           __builtin_bit_cast(bf16x2_dot_t, y), acc, false);
}

// The per-token vectors of the workgroup's head moved to LDS: k and q as stored, k and v
// widened, the gates. fetch() issues the global loads into registers (before the state loads)
// and commit() writes them, as TokenStage does for the token-by-token kernels.
template <class G>
struct ChunkStage {
    static constexpr int D = G::D, TCH = G::TCH;
    static constexpr int CHK = 8;             // bf16 per 16-byte chunk
    static constexpr int NQ = D / CHK;        // chunks of q (= of k, = of v)
    static constexpr int NCHK = 3 * NQ;       // chunks per token
    static constexpr int CPL = (TCH * NCHK + G::NT - 1) / G::NT;
    static_assert(D % CHK == 0 && G::SPLIT == 1, "whole 16-byte chunks, whole heads");
    u32x4 raw[CPL];
    float al = 0.f, be = 0.f;

    __device__ __forceinline__ void fetch(const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k,
                                          const uint16_t* __restrict__ v,
                                          const float* __restrict__ alpha,
                                          const float* __restrict__ beta, int64_t b, int T, int H,
                                          int h, int nt, int tid) {
#pragma unroll
        for (int s = 0; s < CPL; ++s) {
            const int c = tid + s * G::NT;
            if (c < nt * NCHK) {
                const int tt = c / NCHK, r = c - tt * NCHK;
                const size_t tok = ((size_t)b * T + tt) * H + h;
                const uint16_t* src = r < NQ ? q + tok * D + r * CHK
                                    : r < 2 * NQ ? k + tok * D + (r - NQ) * CHK
                                                 : v + tok * D + (r - 2 * NQ) * CHK;
                raw[s] = *(const u32x4*)src;
            }
        }
        if (tid < nt) {
            const size_t tok = ((size_t)b * T + tid) * H + h;
            al = alpha[tok];
            be = beta[tok];
        }
    }

    __device__ __forceinline__ void commit(ChunkLds<D, TCH>& L, int nt, int tid) const {
#pragma unroll
        for (int s = 0; s < CPL; ++s) {
            const int c = tid + s * G::NT;
            if (c < nt * NCHK) {
                const int tt = c / NCHK, r = c - tt * NCHK;
                const uint32_t wv[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
                if (r < 2 * NQ) {
                    uint16_t* dst = r < NQ ? &L.qb[tt][r * CHK] : &L.kb[tt][(r - NQ) * CHK];
                    *(u32x4*)dst = raw[s];
                }
                if (r >= NQ) {
                    float* dst = r < 2 * NQ ? &L.k[tt][(r - NQ) * CHK] : &L.v[tt][(r - 2 * NQ) * CHK];
                    *(float4*)dst = make_float4(unpack<uint16_t>(wv[0], 0), unpack<uint16_t>(wv[0], 1),
                                                unpack<uint16_t>(wv[1], 0), unpack<uint16_t>(wv[1], 1));
                    *(float4*)(dst + 4) = make_float4(unpack<uint16_t>(wv[2], 0), unpack<uint16_t>(wv[2], 1),
                                                      unpack<uint16_t>(wv[3], 0), unpack<uint16_t>(wv[3], 1));
                }
            }
        }
        if (tid < nt) {
            L.alpha[tid] = al;
            L.beta[tid] = be;
        }
    }
};

// The state rows of the lane as stored: Sw[p][w] holds columns col(l, 2w), col(l, 2w + 1) of
// row row0 + p RPP.
template <class G>
__device__ __forceinline__ void load_state_words(const uint16_t* __restrict__ Sg, int row0, int l,
                                                 uint32_t (&Sw)[G::P][G::E / 2]) {
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
        const uint16_t* rowp = Sg + (size_t)(row0 + p * G::RPP) * G::D;
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) {
            Words<G::VB> w = gload<G::VB, G::NTL>(rowp + c * G::LPR * G::VW + l * G::VW);
#pragma unroll
            for (int i = 0; i < G::VW / 2; ++i) Sw[p][c * (G::VW / 2) + i] = w.w[i];
        }
    }
}

template <class G>
__device__ __forceinline__ void store_state_words(uint16_t* __restrict__ Sg, int row0, int l,
                                                  const uint32_t (&Sw)[G::P][G::E / 2]) {
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
        uint16_t* rowp = Sg + (size_t)(row0 + p * G::RPP) * G::D;
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) {
            Words<G::VB> w;
#pragma unroll
            for (int i = 0; i < G::VW / 2; ++i) w.w[i] = Sw[p][c * (G::VW / 2) + i];
            gstore<G::VB, G::NTS>(rowp + c * G::LPR * G::VW + l * G::VW, w);
        }
    }
}

// Gram products k_s . k_t and k_s . q_t of the staged tokens, over the workgroup: token pair
// (s, t) = (pi / TCH, pi % TCH) on the LG lanes of group pi = tid / LG, each lane summing
// D / LG columns; the pairs reach LDS for every wave (after a barrier).
template <class G>
__device__ __forceinline__ void chunk_gram(ChunkLds<G::D, G::TCH>& L, int nt, int tid) {
    constexpr int D = G::D, TCH = G::TCH;
    constexpr int LG = G::NT / (TCH * TCH);  // lanes per pair
    constexpr int CW = D / LG / 2;           // words per lane
    static_assert(G::NT % (TCH * TCH) == 0 &&
                  (LG == 1 || LG == 2 || LG == 4 || LG == 8 || LG == 16) && CW % 4 == 0,
                  "Gram lanes");
    const int pi = tid / LG, j = tid % LG;
    const int gs = pi / TCH, gt = pi % TCH;
    const u32x4* ks = (const u32x4*)&L.kb[gs][2 * CW * j];
    const u32x4* kt = (const u32x4*)&L.kb[gt][2 * CW * j];
    const u32x4* qt = (const u32x4*)&L.qb[gt][2 * CW * j];
    float a = 0.f, c = 0.f;
    if (gs < nt && gt < nt) {
#pragma unroll
        for (int w = 0; w < CW / 4; ++w) {
            const u32x4 x = ks[w], y = kt[w], z = qt[w];
            a = dot2_bf16(x.x, y.x, a); a = dot2_bf16(x.y, y.y, a);
            a = dot2_bf16(x.z, y.z, a); a = dot2_bf16(x.w, y.w, a);
            c = dot2_bf16(x.x, z.x, c); c = dot2_bf16(x.y, z.y, c);
            c = dot2_bf16(x.z, z.z, c); c = dot2_bf16(x.w, z.w, c);
        }
    }
    if constexpr (LG >= 2) {
        a += dpp_mov<0xB1>(a);
        c += dpp_mov<0xB1>(c);
    }
    if constexpr (LG >= 4) {
        a += dpp_mov<0x4E>(a);
        c += dpp_mov<0x4E>(c);
    }
    if constexpr (LG >= 8) {
        a += dpp_mov<0x141>(a);
        c += dpp_mov<0x141>(c);
    }
    if constexpr (LG >= 16) {
        a += dpp_mov<0x140>(a);
        c += dpp_mov<0x140>(c);
    }
    if (j == 0) {
        L.kk[gs][gt] = a;
        L.kq[gs][gt] = c;
    }
}

// The staged tokens from the stored state words: S0 k_t and S0 q_t on the words, then the
// per-row recurrence; o_t (and with DELTA the write coefficient delta_t, in fp32) goes to
// obase (dbase) + t ostride + row on the lane with l == p of each row group. The per-head
// coefficients are formed inline (wave-uniform values): dc[s] = d(t, s) and dp[s] = d(t-1, s)
// as running products, gam = gamma_t. On return dl holds delta_s of the lane's rows, dc[s] =
// d(nt-1, s) and gam = gamma_{nt-1}.
template <class G, bool DELTA>
__device__ __forceinline__ void chunk_tokens(const uint32_t (&Sw)[G::P][G::E / 2],
                                             const ChunkLds<G::D, G::TCH>& L, int nt, int rbase,
                                             int g, int l, uint16_t* __restrict__ obase,
                                             float* __restrict__ dbase, size_t ostride,
                                             float scale, float (&dl)[G::P][G::TCH],
                                             float (&dc)[G::TCH], float& gam) {
    constexpr int TCH = G::TCH, P = G::P, W = G::E / 2;
    gam = 1.0f;
#pragma unroll
    for (int t = 0; t < TCH; ++t) {
        if (t >= nt) break;
        const float at = L.alpha[t], bt = L.beta[t];
        const float gprev = gam;
        gam *= at;
        float dp[TCH];
#pragma unroll
        for (int s = 0; s < TCH; ++s) {
            if (s < t) {
                dp[s] = dc[s];
                dc[s] = s < t - 1 ? dc[s] * at : at;
            }
        }
        dc[t] = 1.0f;
        if (t > 0) dp[t - 1] = 1.0f;
        uint32_t kw[W], qw[W];
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) {
            const int col = c * G::LPR * G::VW + l * G::VW;
            Words<G::VB> a = gload<G::VB, false>(&L.kb[t][col]);
            Words<G::VB> bq = gload<G::VB, false>(&L.qb[t][col]);
#pragma unroll
            for (int i = 0; i < G::VW / 2; ++i) {
                kw[c * (G::VW / 2) + i] = a.w[i];
                qw[c * (G::VW / 2) + i] = bq.w[i];
            }
        }
        float u0[P], w0[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            float su = 0.f, sw = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                su = dot2_bf16(Sw[p][w], kw[w], su);
                sw = dot2_bf16(Sw[p][w], qw[w], sw);
            }
            u0[p] = su;
            w0[p] = sw;
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            u0[p] = row_sum<G::LPR>(u0[p]);
            w0[p] = row_sum<G::LPR>(w0[p]);
        }
        float cu[TCH], co[TCH];
#pragma unroll
        for (int s = 0; s < TCH; ++s) {
            if (s < t) cu[s] = dp[s] * L.kk[s][t];
            if (s <= t) co[s] = dc[s] * L.kq[s][t];
        }
        float ov = 0.f, dv = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int row = rbase + g + p * G::RPP;
            float u = gprev * u0[p];
#pragma unroll
            for (int s = 0; s < TCH; ++s)
                if (s < t) u = fmaf(cu[s], dl[p][s], u);
            dl[p][t] = bt * (L.v[t][row] - at * u);
            float op = gam * w0[p];
#pragma unroll
            for (int s = 0; s < TCH; ++s)
                if (s <= t) op = fmaf(co[s], dl[p][s], op);
            ov = (l == p) ? scale * op : ov;
            dv = (l == p) ? dl[p][t] : dv;
        }
        if (l < P) {
            const size_t at_o = (size_t)t * ostride + rbase + l * G::RPP + g;
            obase[at_o] = act_from_f32<uint16_t>(ov);
            if constexpr (DELTA) dbase[at_o] = dv;
        }
    }
}

template <class G>
__global__ __launch_bounds__(G::NT) void gdn_decode_chunk_kernel(
    int T, int H, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, uint16_t* __restrict__ state, uint16_t* __restrict__ o,
    float scale) {
    constexpr int D = G::D, TCH = G::TCH, P = G::P;
    static_assert(sizeof(typename G::ST) == 2 && G::E % 2 == 0, "bf16 rows");
    __shared__ ChunkLds<D, TCH> L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / G::LPR, l = lane % G::LPR;
    const int64_t n = tile_index<G::GRP>(blockIdx.x, gridDim.x);  // b * H + h
    const int64_t b = n / H;
    const int h = (int)(n - b * H);
    uint16_t* Sg = state + (size_t)n * D * D;
    const int rbase = wave * G::RPW;
    const int nt = T;  // 3 .. TCH, checked by the launcher

    ChunkStage<G> st;
    st.fetch(q, k, v, alpha, beta, b, T, H, h, nt, tid);
    uint32_t Sw[P][G::E / 2];
    load_state_words<G>(Sg, rbase + g, l, Sw);
    st.commit(L, nt, tid);
    __syncthreads();
    chunk_gram<G>(L, nt, tid);
    __syncthreads();

    float dl[P][TCH], dc[TCH], gam;
    chunk_tokens<G, false>(Sw, L, nt, rbase, g, l, o + ((size_t)b * T * H + h) * D, nullptr,
                           (size_t)H * D, scale, dl, dc, gam);

    // ---- S_T = gamma_{T-1} S0 + sum_s d(T-1, s) delta_s k_s^T, rounded once, stored
    const float gT = gam;
    float cs[P][TCH];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int s = 0; s < TCH; ++s) cs[p][s] = s < nt ? dc[s] * dl[p][s] : 0.0f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        uint16_t* rowp = Sg + (size_t)(rbase + g + p * G::RPP) * D;
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) {
            const int col = c * G::LPR * G::VW + l * G::VW;
            float acc[G::VW];
#pragma unroll
            for (int i = 0; i < G::VW; i += 2) {
                const uint32_t wd = Sw[p][c * (G::VW / 2) + i / 2];
                acc[i] = gT * unpack<uint16_t>(wd, 0);
                acc[i + 1] = gT * unpack<uint16_t>(wd, 1);
            }
#pragma unroll
            for (int s = 0; s < TCH; ++s) {
                if (s >= nt) break;
                if constexpr (G::VW % 4 == 0) {
#pragma unroll
                    for (int i = 0; i < G::VW; i += 4) {
                        const float4 k4 = *(const float4*)&L.k[s][col + i];
                        acc[i] = fmaf(cs[p][s], k4.x, acc[i]);
                        acc[i + 1] = fmaf(cs[p][s], k4.y, acc[i + 1]);
                        acc[i + 2] = fmaf(cs[p][s], k4.z, acc[i + 2]);
                        acc[i + 3] = fmaf(cs[p][s], k4.w, acc[i + 3]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < G::VW; i += 2) {
                        const float2 k2 = *(const float2*)&L.k[s][col + i];
                        acc[i] = fmaf(cs[p][s], k2.x, acc[i]);
                        acc[i + 1] = fmaf(cs[p][s], k2.y, acc[i + 1]);
                    }
                }
            }
            Words<G::VB> w;
#pragma unroll
            for (int i = 0; i < G::VW; i += 2) w.w[i / 2] = f32x2_to_bf16x2(acc[i], acc[i + 1]);
            gstore<G::VB, G::NTS>(rowp + col, w);
        }
    }
}

// ------------------------------------------------------------------------ verify kernel

// The accepted prefix of the previous call for sequence b: n_prev[b] clamped to [0, Tp]
// (0 when there was no previous call), wave-uniform.
__device__ __forceinline__ int accepted_prefix(int64_t b, int Tp, const int32_t* __restrict__ n_prev) {
    if (Tp <= 0) return 0;
    const int np = __builtin_amdgcn_readfirstlane(n_prev[b]);
    return np < 0 ? 0 : (np > Tp ? Tp : np);
}

// Replay the previous call's first np tokens onto the lane's state rows S (fp32 registers):
//     S <- alpha_t S + dk_t k_t^T      for t < np,
// from the write coefficients dk that call emitted. The registers hold S / cc with cc the
// product of the alphas replayed so far, so each replayed token costs one FMA per element
// (S' <- S' + (dk / cc') k, cc' = cc alpha); cc is folded back when it would leave
// [2^-64, 2^64] and at the end. The next token's operands are loaded before this token's
// update (the index is clamped, so the loads are unconditional).
template <class G, typename AT>
__device__ __forceinline__ void commit_prefix(float (&S)[G::P][G::E], int np, int64_t b, int H,
                                              int h, int row0, int l, int Tp,
                                              const AT* __restrict__ k_prev,
                                              const float* __restrict__ alpha_prev,
                                              const float* __restrict__ dk_prev) {
    constexpr int D = G::D;
    struct Replay {
        float kk[G::E], dl[G::P], a;
    };
    auto load_replay = [&](int t, Replay& r) {
        const size_t tok = ((size_t)b * Tp + t) * H + h;
#pragma unroll
        for (int e = 0; e < G::E; ++e) r.kk[e] = act_to_f32(k_prev[tok * D + G::col(l, e)]);
#pragma unroll
        for (int p = 0; p < G::P; ++p) r.dl[p] = dk_prev[tok * D + row0 + p * G::RPP];
        r.a = uniform(alpha_prev[tok]);
    };
    float cc = 1.0f;
    Replay cur;
    load_replay(0, cur);
    for (int t = 0; t < np; ++t) {
        Replay nxt;
        load_replay(min(t + 1, np - 1), nxt);
        float cn = cc * cur.a;
        if (!(cn >= 0x1p-64f && cn <= 0x1p64f)) {
            scale_state<G>(S, cc);
            scale_state<G>(S, cur.a);
            cn = 1.0f;
        }
        const float inv_cn = __builtin_amdgcn_rcpf(cn);
#pragma unroll
        for (int p = 0; p < G::P; ++p) {
            const float coef = cur.dl[p] * inv_cn;
#pragma unroll
            for (int e = 0; e < G::E; ++e) S[p][e] = fmaf(coef, cur.kk[e], S[p][e]);
        }
        cc = cn;
        cur = nxt;
    }
    if (cc != 1.0f) scale_state<G>(S, cc);
}


// Speculative verify with a deferred commit. The stored state is the committed state as of the
// start of the previous call; that call's accepted prefix (n_prev[b] of its Tp tokens, clamped
// to [0, Tp]) is folded in first by replaying its updates from the write coefficients it
// emitted,
//     S <- alpha_t S + dk_t k_t^T      for t < n_prev[b],
// and the result is stored (nothing is stored when the prefix is empty). The T new tokens then
// run from it in registers, emitting o and dk for every token; the state after them is not
// stored: the next call commits whichever prefix was accepted. One state read and at most one
// state write per call, as for a plain step.
template <class G, typename AT>
__global__ __launch_bounds__(G::NT) void gdn_verify_kernel(
    int T, int H, const AT* __restrict__ q, const AT* __restrict__ k, const AT* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    typename G::ST* __restrict__ state, int Tp, const int32_t* __restrict__ n_prev,
    const AT* __restrict__ k_prev, const float* __restrict__ alpha_prev,
    const float* __restrict__ dk_prev, AT* __restrict__ o, float* __restrict__ dk_out,
    float scale) {
    constexpr int D = G::D;
    __shared__ TokLds<D, G::TCH> L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / G::LPR, l = lane % G::LPR;
    const uint32_t tile = tile_index<G::GRP>(blockIdx.x, gridDim.x);
    const int64_t n = tile / G::SPLIT;  // b * H + h
    const int part = (int)(tile - n * G::SPLIT);
    const int64_t b = n / H;
    const int h = (int)(n - b * H);
    typename G::ST* Sg = state + (size_t)n * D * D;
    const int rbase = part * G::RPG + wave * G::RPW;
    const int row0 = rbase + g;

    TokenStage<G, AT> st;
    if (T > 0) st.fetch(q, k, v, alpha, beta, b, T, H, h, part, 0, min(G::TCH, T), tid);

    float S[G::P][G::E];
    load_state<G>(Sg, row0, l, S);

    // Commit the previous call's accepted prefix.
    const int np = accepted_prefix(b, Tp, n_prev);
    if (np > 0) commit_prefix<G, AT>(S, np, b, H, h, row0, l, Tp, k_prev, alpha_prev, dk_prev);
    if (np > 0) {
        store_state<G>(Sg, row0, l, S);
        // the new tokens run from the committed state as stored (the state the next call
        // loads, to which it applies their write coefficients)
        if constexpr (sizeof(typename G::ST) == 2) {
#pragma unroll
            for (int p = 0; p < G::P; ++p)
#pragma unroll
                for (int e = 0; e < G::E; e += 2) {
                    const uint32_t w = pack2<typename G::ST>(S[p][e], S[p][e + 1]);
                    S[p][e] = unpack<typename G::ST>(w, 0);
                    S[p][e + 1] = unpack<typename G::ST>(w, 1);
                }
        }
    }

    // Verify the new tokens from the committed state.
    float c = 1.0f;
    for (int t0 = 0; t0 < T; t0 += G::TCH) {
        const int nt = min(G::TCH, T - t0);
        if (t0 > 0) {
            __syncthreads();  // the previous round's readers are done with L
            st.fetch(q, k, v, alpha, beta, b, T, H, h, part, t0, nt, tid);
        }
        st.commit(L, part, nt, tid, scale);
        __syncthreads();
        const size_t ob = (((size_t)b * T + t0) * H + h) * D;
        recur_tokens<G, true, AT, true>(S, L, nt, rbase, g, l, o + ob, (size_t)H * D, c,
                                        dk_out + ob);
    }
}

// ------------------------------------------------------------------------ fused kernel

// One workgroup per head (SPLIT == 1): it is then the only reader and writer of the head's
// conv-state channels.
template <class G, bool MULTI>
__global__ __launch_bounds__(G::NT) void gdn_conv_gate_decode_kernel(
    int T, int H, const uint16_t* __restrict__ qkv, uint16_t* __restrict__ conv_state,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    const float* __restrict__ a_logit, const float* __restrict__ b_logit,
    typename G::ST* __restrict__ state, uint16_t* __restrict__ o, float scale, float l2_eps) {
    static_assert(G::SPLIT == 1, "the fused kernel needs one workgroup per head");
    constexpr int D = G::D;
    constexpr int CH = 3 * D;                        // channels owned by this head
    constexpr int CPT = (CH + G::NT - 1) / G::NT;    // channels per thread
    __shared__ TokLds<D, G::TCH> L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / G::LPR, l = lane % G::LPR;
    const uint32_t tile = tile_index<G::GRP>(blockIdx.x, gridDim.x);
    const int64_t n = tile;
    const int64_t b = n / H;
    const int h = (int)(n - b * H);
    const size_t C = (size_t)3 * H * D;
    typename G::ST* Sg = state + (size_t)n * D * D;
    const int rbase = wave * G::RPW;

    // Per owned channel: taps, bias, the rolling window of raw inputs (bf16 bits), and the
    // round's new raw inputs. The first round's loads are all issued before the state loads.
    float tap[CPT][4], bias[CPT];
    uint32_t win[CPT][3], xr[CPT][G::TCH];
    size_t chan[CPT];
    float av = 0.f, bv = 0.f;
    const int nt0 = min(G::TCH, T);
    auto fetch_round = [&](int t0, int nt) {
#pragma unroll
        for (int s = 0; s < CPT; ++s) {
            if (tid + s * G::NT < CH) {
#pragma unroll
                for (int tt = 0; tt < G::TCH; ++tt)
                    if (tt < nt) xr[s][tt] = qkv[((size_t)b * T + t0 + tt) * C + chan[s]];
            }
        }
        if (tid < nt) {
            const size_t tok = ((size_t)b * T + t0 + tid) * H + h;
            av = a_logit[tok];
            bv = b_logit[tok];
        }
    };
#pragma unroll
    for (int s = 0; s < CPT; ++s) {
        const int ci = tid + s * G::NT;
        if (ci < CH) {
            const int blk = ci / D, j = ci - blk * D;
            const size_t c = (size_t)blk * H * D + (size_t)h * D + j;
            chan[s] = c;
            const float4 w4 = *(const float4*)(conv_w + c * 4);
            tap[s][0] = w4.x; tap[s][1] = w4.y; tap[s][2] = w4.z; tap[s][3] = w4.w;
            bias[s] = conv_b ? conv_b[c] : 0.0f;
            const uint16_t* cs = conv_state + ((size_t)b * C + c) * 3;
            win[s][0] = cs[0]; win[s][1] = cs[1]; win[s][2] = cs[2];
        }
    }
    fetch_round(0, nt0);

    float S[G::P][G::E];
    load_state<G>(Sg, rbase + g, l, S);

    float c = 1.0f;
    for (int t0 = 0; t0 < T; t0 += G::TCH) {
        const int nt = min(G::TCH, T - t0);
        if (t0 > 0) {
            __syncthreads();
            fetch_round(t0, nt);
        }
        // Conv (kernel 4, tap 3 on the current input) + SiLU, into LDS.
#pragma unroll
        for (int s = 0; s < CPT; ++s) {
            const int ci = tid + s * G::NT;
            if (ci < CH) {
                const int blk = ci / D, j = ci - blk * D;
                float* dst = blk == 0 ? &L.q[0][j] : (blk == 1 ? &L.k[0][j] : &L.v[0][j]);
#pragma unroll
                for (int tt = 0; tt < G::TCH; ++tt) {
                    if (tt < nt) {
                        const uint32_t x = xr[s][tt];
                        float y = tap[s][0] * bf16_to_f32(win[s][0]);
                        y = fmaf(tap[s][1], bf16_to_f32(win[s][1]), y);
                        y = fmaf(tap[s][2], bf16_to_f32(win[s][2]), y);
                        y = fmaf(tap[s][3], bf16_to_f32(x), y);
                        y += bias[s];
                        win[s][0] = win[s][1]; win[s][1] = win[s][2]; win[s][2] = x;
                        // SiLU with the hardware exp2 and reciprocal (about 1 ulp each)
                        dst[tt * D] = y * __builtin_amdgcn_rcpf(
                                              1.0f + __builtin_amdgcn_exp2f(-y * 1.44269504f));
                    }
                }
            }
        }
        // Gates: beta = sigma(b), alpha = exp(-softplus(a)).
        if (tid < nt) {
            L.beta[tid] = 1.0f / (1.0f + expf(-bv));
            L.alpha[tid] = expf(-(fmaxf(av, 0.0f) + log1pf(expf(-fabsf(av)))));
        }
        __syncthreads();
        // L2 norms of q and k per token: one wave per (token, q|k) reduction.
        for (int r = wave; r < 2 * nt; r += G::WAVES) {
            const int tt = r >> 1;
            const float* src = (r & 1) ? L.k[tt] : L.q[tt];
            float ss = 0.f;
            for (int j = lane; j < D; j += 64) ss = fmaf(src[j], src[j], ss);
            ss = wave_sum64(ss);
            if (lane == 0) {
                const float inv = 1.0f / sqrtf(ss + l2_eps);
                if (r & 1) L.kf[tt] = inv; else L.qf[tt] = inv * scale;
            }
        }
        __syncthreads();
        recur_tokens<G, MULTI, uint16_t>(S, L, nt, rbase, g, l,
                                         o + (((size_t)b * T + t0) * H + h) * D, (size_t)H * D, c);
    }

    // The conv state keeps the last three raw inputs, oldest first (a byte-exact move).
#pragma unroll
    for (int s = 0; s < CPT; ++s) {
        const int ci = tid + s * G::NT;
        if (ci < CH) {
            uint16_t* cs = conv_state + ((size_t)b * C + chan[s]) * 3;
            cs[0] = (uint16_t)win[s][0]; cs[1] = (uint16_t)win[s][1]; cs[2] = (uint16_t)win[s][2];
        }
    }
    if (MULTI && c != 1.0f) scale_state<G>(S, c);
    store_state<G>(Sg, rbase + g, l, S);
}

// The verify kernel for a bf16 state with bf16 activations and 1 .. TCH new tokens, in the
// chunk form: the committed state as stored is the S0 of the new tokens, whose o and write
// coefficients come from packed bf16 dots on its words (as in gdn_decode_chunk_kernel); the
// state after them is never formed (nothing is stored for it).
template <class G>
__global__ __launch_bounds__(G::NT) void gdn_verify_chunk_kernel(
    int T, int H, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, uint16_t* __restrict__ state, int Tp,
    const int32_t* __restrict__ n_prev, const uint16_t* __restrict__ k_prev,
    const float* __restrict__ alpha_prev, const float* __restrict__ dk_prev,
    uint16_t* __restrict__ o, float* __restrict__ dk_out, float scale) {
    constexpr int D = G::D, TCH = G::TCH, P = G::P, E = G::E;
    static_assert(sizeof(typename G::ST) == 2 && E % 2 == 0, "bf16 rows");
    __shared__ ChunkLds<D, TCH> L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / G::LPR, l = lane % G::LPR;
    const int64_t n = tile_index<G::GRP>(blockIdx.x, gridDim.x);  // b * H + h
    const int64_t b = n / H;
    const int h = (int)(n - b * H);
    uint16_t* Sg = state + (size_t)n * D * D;
    const int rbase = wave * G::RPW;
    const int nt = T;  // 1 .. TCH, checked by the launcher

    ChunkStage<G> st;
    st.fetch(q, k, v, alpha, beta, b, T, H, h, nt, tid);
    uint32_t Sw[P][E / 2];
    load_state_words<G>(Sg, rbase + g, l, Sw);

    const int np = accepted_prefix(b, Tp, n_prev);
    if (np > 0) {
        float S[P][E];
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int e = 0; e < E; e += 2) {
                S[p][e] = unpack<uint16_t>(Sw[p][e / 2], 0);
                S[p][e + 1] = unpack<uint16_t>(Sw[p][e / 2], 1);
            }
        commit_prefix<G, uint16_t>(S, np, b, H, h, rbase + g, l, Tp, k_prev, alpha_prev, dk_prev);
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int e = 0; e < E; e += 2) Sw[p][e / 2] = f32x2_to_bf16x2(S[p][e], S[p][e + 1]);
        store_state_words<G>(Sg, rbase + g, l, Sw);
    }

    st.commit(L, nt, tid);
    __syncthreads();
    chunk_gram<G>(L, nt, tid);
    __syncthreads();
    float dl[P][TCH], dc[TCH], gam;
    const size_t ob = ((size_t)b * T * H + h) * D;
    chunk_tokens<G, true>(Sw, L, nt, rbase, g, l, o + ob, dk_out + ob, (size_t)H * D, scale, dl,
                          dc, gam);
}

// ------------------------------------------------------------------------ dispatch

template <class G, bool MULTI, typename AT>
hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
    int T = a.T, H = a.H;
    const AT* q = (const AT*)a.q;
    const AT* k = (const AT*)a.k;
    const AT* v = (const AT*)a.v;
    const float* alpha = a.alpha;
    const float* beta = a.beta;
    typename G::ST* state = (typename G::ST*)a.state;
    AT* o = (AT*)a.o;
    float scale = a.scale;
    void* args[] = {&T, &H, &q, &k, &v, &alpha, &beta, &state, &o, &scale};
    static_assert((int64_t)G::NT * G::SPLIT <= kThreadsPerHeadPerDim * G::D, "threads per head");
    return hipLaunchKernel((const void*)gdn_decode_kernel<G, MULTI, AT>,
                           dim3((unsigned)(a.B * a.H * G::SPLIT)), dim3(G::NT), args, 0, s);
}

template <class G>
hipError_t launch_chunk_g(const DecodeArgs& a, hipStream_t s) {
    int T = a.T, H = a.H;
    const uint16_t* q = (const uint16_t*)a.q;
    const uint16_t* k = (const uint16_t*)a.k;
    const uint16_t* v = (const uint16_t*)a.v;
    const float* alpha = a.alpha;
    const float* beta = a.beta;
    uint16_t* state = (uint16_t*)a.state;
    uint16_t* o = (uint16_t*)a.o;
    float scale = a.scale;
    void* args[] = {&T, &H, &q, &k, &v, &alpha, &beta, &state, &o, &scale};
    static_assert((int64_t)G::NT <= kThreadsPerHeadPerDim * G::D, "threads per head");
    return hipLaunchKernel((const void*)gdn_decode_chunk_kernel<G>, dim3((unsigned)(a.B * a.H)),
                           dim3(G::NT), args, 0, s);
}

template <class G>
hipError_t launch_verify_chunk_g(const VerifyArgs& a, hipStream_t s) {
    int T = a.T, H = a.H, Tp = a.Tp;
    const uint16_t* q = (const uint16_t*)a.q;
    const uint16_t* k = (const uint16_t*)a.k;
    const uint16_t* v = (const uint16_t*)a.v;
    const float* alpha = a.alpha;
    const float* beta = a.beta;
    uint16_t* state = (uint16_t*)a.state;
    const int32_t* n_prev = a.n_prev;
    const uint16_t* k_prev = (const uint16_t*)a.k_prev;
    const float* alpha_prev = a.alpha_prev;
    const float* dk_prev = a.dk_prev;
    uint16_t* o = (uint16_t*)a.o;
    float* dk_out = a.dk_out;
    float scale = a.scale;
    void* args[] = {&T, &H, &q, &k, &v, &alpha, &beta, &state, &Tp, &n_prev, &k_prev,
                    &alpha_prev, &dk_prev, &o, &dk_out, &scale};
    static_assert((int64_t)G::NT <= kThreadsPerHeadPerDim * G::D, "threads per head");
    return hipLaunchKernel((const void*)gdn_verify_chunk_kernel<G>, dim3((unsigned)(a.B * a.H)),
                           dim3(G::NT), args, 0, s);
}

template <class G, typename AT>
hipError_t launch_verify_g(const VerifyArgs& a, hipStream_t s) {
    int T = a.T, H = a.H, Tp = a.Tp;
    const AT* q = (const AT*)a.q;
    const AT* k = (const AT*)a.k;
    const AT* v = (const AT*)a.v;
    const float* alpha = a.alpha;
    const float* beta = a.beta;
    typename G::ST* state = (typename G::ST*)a.state;
    const int32_t* n_prev = a.n_prev;
    const AT* k_prev = (const AT*)a.k_prev;
    const float* alpha_prev = a.alpha_prev;
    const float* dk_prev = a.dk_prev;
    AT* o = (AT*)a.o;
    float* dk_out = a.dk_out;
    float scale = a.scale;
    void* args[] = {&T, &H, &q, &k, &v, &alpha, &beta, &state, &Tp, &n_prev, &k_prev,
                    &alpha_prev, &dk_prev, &o, &dk_out, &scale};
    static_assert((int64_t)G::NT * G::SPLIT <= kThreadsPerHeadPerDim * G::D, "threads per head");
    return hipLaunchKernel((const void*)gdn_verify_kernel<G, AT>,
                           dim3((unsigned)(a.B * a.H * G::SPLIT)), dim3(G::NT), args, 0, s);
}

template <class G, bool MULTI>
hipError_t launch_fused_g(const FusedArgs& a, hipStream_t s) {
    int T = a.T, H = a.H;
    const uint16_t* qkv = (const uint16_t*)a.qkv;
    uint16_t* cs = (uint16_t*)a.conv_state;
    const float* w = a.conv_w;
    const float* cb = a.conv_b;
    const float* al = a.a_logit;
    const float* bl = a.b_logit;
    typename G::ST* state = (typename G::ST*)a.state;
    uint16_t* o = (uint16_t*)a.o;
    float scale = a.scale, eps = a.l2_eps;
    void* args[] = {&T, &H, &qkv, &cs, &w, &cb, &al, &bl, &state, &o, &scale, &eps};
    static_assert((int64_t)G::NT * 1 <= kThreadsPerHeadPerDim * G::D, "threads per head");
    return hipLaunchKernel((const void*)gdn_conv_gate_decode_kernel<G, MULTI>,
                           dim3((unsigned)(a.B * a.H)), dim3(G::NT), args, 0, s);
}

constexpr int max_int(int a, int b) { return a > b ? a : b; }

// Head count from which one-token fp32-state calls spread a head's tiles over the XCDs.
constexpr int64_t kOneTokenSpreadHeads = 8192;

// Launch geometry, chosen by sweeping variants on MI355X at B=256, H=48, D=128 (variants with
// the same lanes per row reproduce each other bit for bit; only the schedule differs):
//  * one token, fp32 state: one wave per workgroup, 8 rows (4 KiB) per wave, nontemporal
//    state loads and stores -- 79% of HBM peak; larger workgroups synchronise their waves'
//    load/store phases and lose 5-15%; 16 rows per wave (256 -> 278 us at B = 256) and 4 rows
//    per wave (-> 294 us) lose too;
//    From 8192 heads, runs of 4 consecutive tiles share an XCD (a head's 16 tiles on 4 XCDs):
//    at B = 256 H = 48, 253.1 -> 251.6 us against consecutive tiles on different XCDs, and
//    runs of 2, 8 and 16 tiles measured 260.4, 263.4 and 259.5 us (an in-place stream with
//    the same tiles and no arithmetic shows the same order: the state stream's placement over
//    the XCDs decides, not the q, k, v fetches the grouping saves).
//    Below 8192 heads the 16 tiles of a head stay on one XCD (its q, k and v are fetched into
//    one L2): B = 8 .. 128 at H = 48 run 3-8% faster that way (B = 64: 70.4 -> 65.8 us),
//    B = 160 and 192 tie;
//  * one token, bf16 state: all rows of a head in one workgroup, 8 rows per wave, 8 lanes per
//    row (two 16-byte loads per lane and row): 140 -> 130 us at B=256 H=48 D=128 against 16
//    lanes per row (fp32 states show no difference); runs of 4 heads per XCD: 128.2 -> 124.9
//    us (2: 126.5 us); the multi-token 16-bit calls take the same order (decode T = 4 156.4 ->
//    154.4 us, verify 184.4 -> 183.4, fused unchanged);
//  * several tokens (and the fused path): the per-token arithmetic is repeated on registers,
//    so occupancy and instruction count decide: 16 rows per wave, one workgroup per head,
//    8 lanes per row where it saves reduction steps (bf16 state, fused prologue);
//  * several tokens, fp32 state, decode: one wave per workgroup again (16 rows): 2% faster
//    than a workgroup per head at B=256 H=48 D=128 T=4, where the verify kernel is 3% slower
//    with it; 8 rows per wave (16 tiles per head) is slower (277 -> 302 us); runs of 2 tiles
//    per XCD: 273.4 -> 266.2 us against a head's 8 tiles on one XCD (runs of 1 and 4: 277.8,
//    275.0 us);
//  * verify, fp32 state: a workgroup per head, runs of 2 heads per XCD (272.0 -> 267.8 us
//    against 1; 4: 269.0 us);
//  * fused path, fp32 state: 4 waves of 32 rows per head (190 VGPRs, two workgroups per CU):
//    2.5% faster than 8 waves of 16 rows at B=256 H=48 D=128 T=4; 16-bit states lose 9% with
//    it; runs of 4 heads per XCD: 277.6 -> 263.8 us against 1 (2: 267.8 us). The fused kernel
//    needs the whole head in one workgroup (the conv state of the q and k channels is read and
//    rewritten by it).
template <int D, typename ST> struct DecodeOneToken {  // 2-byte states
    using G = Geo<D, ST, D / 8, 1, 1, true, true, 4, 8>;
};
template <int D> struct DecodeOneToken<D, float> {
    using G = Geo<D, float, 1, D / 8, 1, true, true, 4>;
    using G_small = Geo<D, float, 1, D / 8, 1, true, true, D / 8>;  // fewer than 8192 heads
};

template <int D, typename ST> struct DecodeTokens {  // 2-byte states
    using G = Geo<D, ST, max_int(1, D / 16), 1, 8, true, true, 4, 8>;
};
template <int D> struct DecodeTokens<D, float> {
    using G = Geo<D, float, 1, max_int(1, D / 16), 8, true, true, 2, 16>;
};

// Chunk form (bf16 state and activations, up to TCH tokens): the multi-token geometry.
template <int D> struct DecodeChunk {
    using G = Geo<D, uint16_t, max_int(1, D / 16), 1, 8, true, true, 4, 8>;
};

template <int D, typename ST> struct VerifyTokens {  // 2-byte states
    using G = Geo<D, ST, max_int(1, D / 16), 1, 8, true, true, 4, 8>;
};
template <int D> struct VerifyTokens<D, float> {
    using G = Geo<D, float, max_int(1, D / 16), 1, 8, true, true, 2, 16>;
};

template <int D, typename ST> struct FusedTokens {  // 2-byte states
    using G = Geo<D, ST, max_int(1, D / 16), 1, 8, true, true, 4, 8>;
};
template <int D> struct FusedTokens<D, float> {
    using G = Geo<D, float, max_int(1, D / 32), 1, 8, true, true, 4, 8>;
};

template <int D, typename ST, typename AT>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
    if constexpr (sizeof(ST) == 4) {
        if (a.T == 1 && a.B * a.H < kOneTokenSpreadHeads)
            return launch_decode_g<typename DecodeOneToken<D, ST>::G_small, false, AT>(a, s);
    }
    if (a.T == 1) return launch_decode_g<typename DecodeOneToken<D, ST>::G, false, AT>(a, s);
    // The chunk form from 3 tokens: at 2 its per-call Gram products and barriers cost more than
    // the dots it saves (B = 256, H = 48, D = 128: 134.6 against 128.4 us; 3 tokens 132.8
    // against 137.0, 8 tokens 216.2 against 224.2).
    if constexpr (sizeof(ST) == 2 && !is_f16<ST>::value && sizeof(AT) == 2 && !is_f16<AT>::value) {
        if (a.T >= 3 && a.T <= DecodeChunk<D>::G::TCH)
            return launch_chunk_g<typename DecodeChunk<D>::G>(a, s);
    }
    return launch_decode_g<typename DecodeTokens<D, ST>::G, true, AT>(a, s);
}

template <int D, typename ST>
hipError_t launch_decode_s(const DecodeArgs& a, hipStream_t s) {
    switch (a.act) {
        case DType::F32: return launch_decode_t<D, ST, float>(a, s);
        case DType::BF16: return launch_decode_t<D, ST, uint16_t>(a, s);
        default: return launch_decode_t<D, ST, _Float16>(a, s);
    }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
    switch (a.state_dtype) {
        case DType::F32: return launch_decode_s<D, float>(a, s);
        case DType::BF16: return launch_decode_s<D, uint16_t>(a, s);
        default: return launch_decode_s<D, _Float16>(a, s);
    }
}

template <int D, typename ST>
hipError_t launch_verify_s(const VerifyArgs& a, hipStream_t s) {
    using G = typename VerifyTokens<D, ST>::G;
    if constexpr (sizeof(ST) == 2 && !is_f16<ST>::value) {
        if (a.act == DType::BF16 && a.T >= 1 && a.T <= DecodeChunk<D>::G::TCH)
            return launch_verify_chunk_g<typename DecodeChunk<D>::G>(a, s);
    }
    switch (a.act) {
        case DType::F32: return launch_verify_g<G, float>(a, s);
        case DType::BF16: return launch_verify_g<G, uint16_t>(a, s);
        default: return launch_verify_g<G, _Float16>(a, s);
    }
}

template <int D>
hipError_t launch_verify_d(const VerifyArgs& a, hipStream_t s) {
    switch (a.state_dtype) {
        case DType::F32: return launch_verify_s<D, float>(a, s);
        case DType::BF16: return launch_verify_s<D, uint16_t>(a, s);
        default: return launch_verify_s<D, _Float16>(a, s);
    }
}

template <int D, typename ST>
hipError_t launch_fused_t(const FusedArgs& a, hipStream_t s) {
    if (a.T == 1) return launch_fused_g<typename FusedTokens<D, ST>::G, false>(a, s);
    return launch_fused_g<typename FusedTokens<D, ST>::G, true>(a, s);
}

template <int D>
hipError_t launch_fused_d(const FusedArgs& a, hipStream_t s) {
    switch (a.state_dtype) {
        case DType::F32: return launch_fused_t<D, float>(a, s);
        case DType::BF16: return launch_fused_t<D, uint16_t>(a, s);
        default: return launch_fused_t<D, _Float16>(a, s);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    switch (a.D) {
        case 16: return launch_decode_d<16>(a, s);
        case 32: return launch_decode_d<32>(a, s);
        case 64: return launch_decode_d<64>(a, s);
        case 128: return launch_decode_d<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t s) {
    switch (a.D) {
        case 16: return launch_verify_d<16>(a, s);
        case 32: return launch_verify_d<32>(a, s);
        case 64: return launch_verify_d<64>(a, s);
        case 128: return launch_verify_d<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_conv_gate_decode(const FusedArgs& a, hipStream_t s) {
    switch (a.D) {
        case 16: return launch_fused_d<16>(a, s);
        case 32: return launch_fused_d<32>(a, s);
        case 64: return launch_fused_d<64>(a, s);
        case 128: return launch_fused_d<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
