// Chunked (prefill) form of the gated delta rule on gfx950 (CDNA4): T sequential tokens per
// head with the state-touching work done as dense products on the matrix cores.
//
// The result is that of T steps of the recurrence ("GDN tuning limits on Kunlun XPU", section
// 二: S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t (scale q_t)); the
// same page (section 三.3) runs long prompts through a chunked form of it. Regrouping over a chunk
// of 16 tokens t = 0..15 with S the state before the chunk and
//     gamma_t = alpha_0 alpha_1 ... alpha_t,   Gam_ts = alpha_{s+1} ... alpha_t  (Gam_tt = 1),
// and the kernel form delta_t = beta_t (v_t - alpha_t S_{t-1} k_t), S_t = alpha_t S_{t-1} + delta_t k_t^T:
//     S_t = gamma_t S + sum_{s<=t} Gam_ts delta_s k_s^T, so (I + A) Delta = diag(beta) (V - gamma . K S^T)
// with A_ts = beta_t Gam_ts (k_t . k_s) for s < t (strictly lower triangular), Delta the 16 x dv
// matrix of the delta_t, and
//     Delta = T diag(beta) (V - gamma . X),   X = K S^T,            T = (I + A)^-1
//     O     = scale gamma . (Q S^T) + P Delta,   P_ts = scale Gam_ts (q_t . k_s), s <= t
//     S_end = gamma_15 S + Delta^T diag(Gam_end) K,   Gam_end,t = alpha_{t+1} ... alpha_15
// (". " scales row t by the per-token factor). All decays are products of alphas, never ratios,
// so alpha = 0 is exact. Tokens past the end of the sequence enter with alpha = 1, beta = 0 and
// zero vectors, which makes their delta exactly 0.
//
// Two kernels:
//   * prep (one wave per (b, h, chunk); all chunks in parallel): the chunk's Gram product K K^T
//     on MFMA, the decays, T by forward substitution, and P (for bf16 activations only its
//     factor scale Gam; see below), written as one record of 544 floats to the caller's
//     workspace;
//   * state (one wave per (b, h, 32 state rows: two tiles of 16), sequential over the chunks):
//     the rows' state stays in registers for the whole call as S' = S / c (c a running product of
//     chunk decays); per chunk the products X = K S'^T and Y = Q S'^T, Delta = T diag(beta) Z,
//     O = Y + P Delta and the update, with the next chunk's operands loaded while the current
//     one computes.
// Matrix-core layout (lane l = 16 g + n; checked on the device against a CPU product): for
// v_mfma_f32_16x16x4f32 operand a is A[l%16][l/16], operand b is B[l/16][l%16]; the 16 x 16 x 32
// and 16 x 16 x 16 bf16 forms hold 8 and 4 consecutive k per lane (k = 8 (l/16) + e, 4 (l/16)
// + e); all accumulate into C[4 g + i][n], i = 0..3. The state's accumulator tiles of the update
// are arranged so that the same registers are the b operand of the next chunk's K S'^T and
// Q S'^T: tile mt, element i of lane (g, n) is S[row n][column (D/4) g + (D/16) i + mt], so each
// lane holds one state row's contiguous run of D/4 columns and every load is a contiguous vector.
// For bf16 activations (D >= 32) k and q are exact bf16 operands of the bf16 matrix cores and
// the fp32 state enters as three bf16 parts whose sum is exact (two for Q S'^T, whose result is
// rounded to bf16); other activation types use the fp32 form. A NaN or infinity in a token's k,
// q or v also reaches the earlier outputs of its own chunk (products with the structural zeros
// of T diag(beta) and P); finite inputs are exact to fp32 rounding.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "gdn_prefill_launch.h"

namespace gdn {
namespace {

constexpr int CH = kPrefillChunk;
constexpr int REC = kPrefillRecordFloats;
constexpr int REC_T = 0, REC_P = 256, REC_G = 512, REC_GE = 528;
static_assert(REC == REC_GE + CH, "record layout");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// D += A B over one 4-wide slice of the contraction (16 x 16 x 4, fp32 in and out).
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// D += A B with bf16 operands and fp32 accumulation: 16 x 16 x 32 (a, b: 8 bf16 per lane,
// lane l holding k = 8 (l/16) .. + 7) and 16 x 16 x 16 (4 bf16 per lane, k = 4 (l/16) .. + 3);
// the accumulator layout is that of mfma4 (checked on the device against a CPU product).
__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// Two floats as three packed pairs of bf16 (first value in the low half) whose sum is exact:
// x = hi + mid + lo with hi the top 8 significant bits of x (truncation), mid the top 8 of the
// exact remainder x - hi, and lo the rest, which has at most 8 significant bits left. A
// product with a bf16 operand is then an fp32-exact product split over three bf16 products
// (an fp32 value carries 24 significant bits). Non-finite values stay non-finite.
struct Split3 { uint32_t h, m, l; };

// The high halves of two words packed into one, x's in the low half: (x >> 16) | (y & 0xffff0000)
// in one byte permute (v_perm_b32 picks bytes 2, 3 of x and 2, 3 of y).
__device__ __forceinline__ uint32_t hi_halves(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x07060302u);
}
// The low halves likewise: (x & 0xffff) | (y << 16).
__device__ __forceinline__ uint32_t lo_halves(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x05040100u);
}

__device__ __forceinline__ Split3 split3(float a, float b) {
    constexpr uint32_t HI = 0xffff0000u;
    const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    const float ra = a - __uint_as_float(ua & HI), rb = b - __uint_as_float(ub & HI);
    const uint32_t va = __float_as_uint(ra), vb = __float_as_uint(rb);
    const float sa = ra - __uint_as_float(va & HI), sb = rb - __uint_as_float(vb & HI);
    return Split3{hi_halves(ua, ub), hi_halves(va, vb),
                  hi_halves(__float_as_uint(sa), __float_as_uint(sb))};
}

// bf16 activations of head dim >= 32 take the bf16 matrix-core path (k and q are exact bf16
// operands); other types and D = 16 take fp32 MFMA (16 x 16 x 4).
template <int D, typename AT>
constexpr bool kBf16Mma = std::is_same<AT, uint16_t>::value && D >= 32;

__device__ __forceinline__ float lane_value(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Element types of activations and state: float, uint16_t (bf16 bits), _Float16.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float get(const uint32_t* w, int e) { return __uint_as_float(w[e]); }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float get(const uint32_t* w, int e) {
        const uint32_t x = w[e >> 1];
        return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
    }
    // Round to nearest even (gfx950's v_cvt_pk_bf16_f32), NaN stays NaN.
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        const f32x2_t v = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    }
};
template <> struct Elem<_Float16> {
    static __device__ __forceinline__ float get(const uint32_t* w, int e) {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, w[e >> 1]);
        return (float)((e & 1) ? h.y : h.x);
    }
    // Round to nearest even (v_cvt_pk_f16_f32).
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        const f32x2_t v = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    }
};

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) {
    return (uint16_t)(Elem<uint16_t>::pack(x, 0.0f) & 0xffffu);
}
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) {
    return __builtin_bit_cast(_Float16, (uint16_t)(Elem<_Float16>::pack(x, 0.0f) & 0xffffu));
}
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
template <> __device__ __forceinline__ float to_f32<_Float16>(_Float16 x) { return (float)x; }

// N contiguous elements of type T held as raw 32-bit words, loaded with the widest vector
// accesses their alignment allows (a run of N elements starts at a multiple of min(16, bytes)).
template <typename T, int N>
struct Run {
    static constexpr int BYTES = N * (int)sizeof(T);
    static constexpr int WORDS = (BYTES + 3) / 4;
    uint32_t w[WORDS];

    template <bool NT = false>
    __device__ __forceinline__ void load(const T* p) {
        if constexpr (BYTES >= 16) {
            static_assert(BYTES % 16 == 0, "run length");
#pragma unroll
            for (int i = 0; i < BYTES / 16; ++i) {
                const u32x4* a = (const u32x4*)p + i;
                const u32x4 x = NT ? __builtin_nontemporal_load(a) : *a;
                w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
            }
        } else if constexpr (BYTES == 8) {
            const u32x2 x = *(const u32x2*)p;
            w[0] = x.x; w[1] = x.y;
        } else if constexpr (BYTES == 4) {
            w[0] = *(const uint32_t*)p;
        } else {
            static_assert(BYTES == 2, "run length");
            w[0] = *(const uint16_t*)p;
        }
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < WORDS; ++i) w[i] = 0u;
    }
    __device__ __forceinline__ float get(int e) const { return Elem<T>::get(w, e); }
};

// Stores N floats as N contiguous elements of T (rounded to nearest even for 2-byte types).
template <typename T, int N, bool NT>
__device__ __forceinline__ void store_run(T* p, const float* x) {
    constexpr int BYTES = N * (int)sizeof(T);
    uint32_t w[(BYTES + 3) / 4];
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < N; ++e) w[e] = __float_as_uint(x[e]);
    } else {
        static_assert(N % 2 == 0, "run length");
#pragma unroll
        for (int e = 0; e < N; e += 2) w[e / 2] = Elem<T>::pack(x[e], x[e + 1]);
    }
    static_assert(BYTES % 16 == 0 || BYTES == 8, "run length");
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
        for (int i = 0; i < BYTES / 16; ++i) {
            const u32x4 v = {w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
            if (NT) __builtin_nontemporal_store(v, (u32x4*)p + i); else ((u32x4*)p)[i] = v;
        }
    } else {
        const u32x2 v = {w[0], w[1]};
        *(u32x2*)p = v;
    }
}

// ------------------------------------------------------------------------ prep kernel

// One wave per (b, h, chunk c); workgroup id = (b H + h) nch + c, which is also the record's
// index in the workspace. Lane (g, n) = (lane / 16, lane % 16) holds token n's k (and q) over
// the columns (D/4) g .. (D/4) g + D/4 - 1, so that the same registers are the a and b operands
// of the Gram products (the contraction runs over the key dim in any order).
// With bf16 activations the record's P slot holds scale Gam_ts (s <= t, 0 above) and the state
// kernel multiplies it by q_t . k_s, which it forms from registers it holds anyway, so this
// kernel never reads q; for other activation types it stores P itself.
template <int D, typename AT>
__global__ __launch_bounds__(64) void gdn_prefill_prep_kernel(
    int T, int H, int nch, const AT* __restrict__ q, const AT* __restrict__ k,
    const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ ws,
    float scale) {
    constexpr int R = D / 4;
    constexpr bool kFormsP = !kBf16Mma<D, AT>;
    __shared__ float sA[CH][CH];
    const int lane = threadIdx.x, g = lane >> 4, n = lane & 15;
    const uint32_t wid = blockIdx.x;
    const int c = (int)(wid % (uint32_t)nch);
    const int64_t bh = wid / (uint32_t)nch;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    const int t0 = c * CH;
    const int nv = min(CH, T - t0);

    Run<AT, R> kx, qx;
    if (n < nv) {
        const int64_t off = ((b * T + t0 + n) * H + h) * D + R * g;
        kx.load(k + off);
        if constexpr (kFormsP) qx.load(q + off);
    } else {
        kx.zero();
        if constexpr (kFormsP) qx.zero();
    }
    // Lane t < 16 holds token t's gates; past the end alpha = 1, beta = 0.
    float al = 1.0f, be = 0.0f;
    if (lane < nv) {
        const int64_t ti = (b * T + t0 + lane) * H + h;
        al = alpha[ti];
        be = beta[ti];
    }

    // G[t][s] = k_t . k_s (and QK[t][s] = q_t . k_s); lane (g, n) holds rows t = 4g + j, column
    // s = n.
    f32x4 G = {0.f, 0.f, 0.f, 0.f}, QK = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kBf16Mma<D, AT>) {
        // 8 key columns per lane and step: words 4s .. 4s+3 of the lane's run.
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            const u32x4 ka = {kx.w[4 * s], kx.w[4 * s + 1], kx.w[4 * s + 2], kx.w[4 * s + 3]};
            G = mfma_k32(ka, ka, G);
        }
    } else {
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const float ke = kx.get(e);
            G = mfma4(ke, ke, G);
            QK = mfma4(qx.get(e), ke, QK);
        }
    }

    // Decays of column s = n: a running product over t, Gam_{t,n} = alpha_{n+1} ... alpha_t for
    // t > n (1 for t <= n), multiplied in increasing t; the lane keeps rows t = 4g + j. After
    // the last token it holds Gam_end,n = Gam_{15,n}, and on the lanes of column 0,
    // gamma_t = alpha_0 Gam_{t,0}.
    float run = 1.0f;
    float gam[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int t = 0; t < CH; ++t) {
        const float at = lane_value(al, t);
        run = (t > n) ? run * at : 1.0f;
        if (g == t / 4) gam[t % 4] = run;
    }

    float* rec = ws + (size_t)wid * REC;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 4 * g + j;
        const float bt = __shfl(be, t);
        sA[t][n] = (n < t) ? bt * gam[j] * G[j] : 0.0f;
        const float p = kFormsP ? scale * gam[j] * QK[j] : scale * gam[j];
        rec[REC_P + t * CH + n] = (n <= t) ? p : 0.0f;
    }
    const float a0 = lane_value(al, 0);
    if (n == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) rec[REC_G + 4 * g + j] = a0 * gam[j];
    }
    if (g == 0) rec[REC_GE + n] = run;
    __syncthreads();

    // T = (I + A)^-1 by forward substitution: lane c < 16 computes column c,
    // T[t][c] = [t == c] - sum_{s<t} A[t][s] T[s][c]; stored with column c scaled by beta_c.
    if (lane < CH) {
        float x[CH];
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            float acc = (t == lane) ? 1.0f : 0.0f;
#pragma unroll
            for (int s = 0; s < t; ++s) acc = fmaf(-sA[t][s], x[s], acc);
            x[t] = acc;
        }
#pragma unroll
        for (int t = 0; t < CH; ++t) rec[REC_T + t * CH + lane] = x[t] * be;
    }
}

// ------------------------------------------------------------------------ state kernel

// One lane's operands of one chunk: lane (g, m) = (lane / 16, lane % 16). Loads never branch:
// past the end of the sequence they read the last token again (always in bounds). Those
// tokens then contribute exact zeros: their rows and columns of T diag(beta) are zero (beta = 0
// in the record), so only their entries of Z are cleared, which also keeps a non-finite value
// in the last token from reaching earlier tokens through 0 * inf. Branch-free loads let the
// next chunk's loads stay in flight while the current chunk computes.
template <int D, int RT, typename AT>
struct ChunkOps {
    static constexpr int R = D / 4, NMT = D / 16;
    Run<AT, R> kx, qx;   // a operands of K S^T and Q S^T: token m, columns R g .. R g + R - 1
    Run<AT, NMT> ku[4];  // a operand of the update, step s: token 4g + s, columns NMT m .. + NMT
    AT v[RT][4];         // v[token 4g + j][state row of tile r], raw
    f32x4 tb, pm;        // T diag(beta)[m][4g .. 4g+3], P (bf16 path: scale Gam)[m][4g .. 4g+3]
    f32x4 gm, ge;        // gamma and Gam_end of tokens 4g .. 4g+3
    float gend;          // gamma_15: decay of the whole chunk
    int nv;              // tokens of the chunk inside the sequence (1..16)
};

template <int D, int RT, typename AT>
__device__ __forceinline__ void load_chunk(ChunkOps<D, RT, AT>& x, int c, int T, int H, int64_t b,
                                           int h, int row0, const AT* __restrict__ q,
                                           const AT* __restrict__ k, const AT* __restrict__ v,
                                           const float* __restrict__ wsh, int g, int m) {
    constexpr int R = D / 4, NMT = D / 16;
    const int t0 = c * CH;
    const int nv = min(CH, T - t0);
    x.nv = nv;
    const int64_t tok0 = (b * T + t0) * H + h;  // index of (b, t0, h) in [B][T][H]
    const int last = nv - 1;
    {
        const int64_t off = (tok0 + (int64_t)min(m, last) * H) * D + R * g;
        x.kx.load(k + off);
        x.qx.load(q + off);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
        x.ku[s].load(k + (tok0 + (int64_t)min(4 * g + s, last) * H) * D + NMT * m);
    // v: the 16 lanes of a lane group read 32 or 64 contiguous bytes of one token's v, the rest
    // of each line by other waves; cached loads let the L2 serve those (the nontemporal hint
    // cost 1.6% on the prompt workload and 5-9% on short prompts).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const AT* vt = v + (tok0 + (int64_t)min(4 * g + j, last) * H) * D + row0;
#pragma unroll
        for (int r = 0; r < RT; ++r) x.v[r][j] = vt[16 * r];
    }
    const float* rec = wsh + (size_t)c * REC;
    x.tb = *(const f32x4*)(rec + REC_T + CH * m + 4 * g);
    x.pm = *(const f32x4*)(rec + REC_P + CH * m + 4 * g);
    x.gm = *(const f32x4*)(rec + REC_G + 4 * g);
    x.ge = *(const f32x4*)(rec + REC_GE + 4 * g);
    x.gend = rec[REC_G + CH - 1];
}

// One chunk for the wave's RT tiles of 16 state rows; tile r holds rows row0 + 16 r (lane's
// row n of the tile). Tiles are interleaved innermost so that consecutive products are
// independent. The registers hold S' = S / c with c a wave-uniform running product of the
// chunk decays, so the decay of the state costs per-token factors instead of a multiply per
// state element: X = c K S'^T, and S_end = gamma_15 c (S' + K^T diag(Gam_end) Delta / (gamma_15 c)).
// When gamma_15 c leaves [2^-64, 2^64] (alpha = 0, long strong decay, or alpha > 1 or < 0) the
// product is folded into S' first and c restarts at 1.
template <int D, int RT, typename AT>
__device__ __forceinline__ void chunk_step(f32x4 (&S)[RT][D / 16], float& c,
                                           const ChunkOps<D, RT, AT>& x, int ci, int T, int H,
                                           int64_t b, int h, int row0, AT* __restrict__ o,
                                           float scale, int g) {
    constexpr int R = D / 4, NMT = D / 16;
    const int nv = x.nv;
    // X' = K S'^T and Y' = Q S'^T; lane (g, n) ends with rows (tokens) 4g + j of state row n.
    f32x4 X[RT], Y[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) X[r] = Y[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    // bf16 path: the record holds scale Gam for P; K Q^T (lane (g, m) ends with k_{4g+s} . q_m,
    // exactly the a operand P[m][4g + s] needs) completes it.
    f32x4 QKt = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kBf16Mma<D, AT>) {
        // Step s contracts over the lane's columns t = 8s .. 8s+7 of its run (state elements
        // (mt, i) = (t % NMT, t / NMT)); S' enters as three bf16 parts for X (which feeds the
        // state) and two for Y (o is rounded to the activation type; the dropped part is below
        // 2^-16 of each element).
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            const u32x4 ka = {x.kx.w[4 * s], x.kx.w[4 * s + 1], x.kx.w[4 * s + 2], x.kx.w[4 * s + 3]};
            const u32x4 qa = {x.qx.w[4 * s], x.qx.w[4 * s + 1], x.qx.w[4 * s + 2], x.qx.w[4 * s + 3]};
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                Split3 p[4];
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const int t = 8 * s + 2 * pp;
                    p[pp] = split3(S[r][t % NMT][t / NMT], S[r][t % NMT + 1][t / NMT]);
                }
                const u32x4 bh = {p[0].h, p[1].h, p[2].h, p[3].h};
                const u32x4 bm = {p[0].m, p[1].m, p[2].m, p[3].m};
                const u32x4 bl = {p[0].l, p[1].l, p[2].l, p[3].l};
                X[r] = mfma_k32(ka, bh, X[r]);
                Y[r] = mfma_k32(qa, bh, Y[r]);
                X[r] = mfma_k32(ka, bm, X[r]);
                Y[r] = mfma_k32(qa, bm, Y[r]);
                X[r] = mfma_k32(ka, bl, X[r]);
            }
            QKt = mfma_k32(ka, qa, QKt);
        }
    } else {
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const float ke = x.kx.get(e), qe = x.qx.get(e);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const float s = S[r][e % NMT][e / NMT];
                X[r] = mfma4(ke, s, X[r]);
                Y[r] = mfma4(qe, s, Y[r]);
            }
        }
    }
    // Z = V - gamma c . X', then Delta = T diag(beta) Z (step s contracts over tokens 4g + s).
    f32x4 gx, gy;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gx[j] = x.gm[j] * c;
        gy[j] = gx[j] * scale;
    }
    f32x4 Z[RT], Dl[RT], O[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        Dl[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Z[r][j] = (4 * g + j < nv) ? fmaf(-gx[j], X[r][j], to_f32<AT>(x.v[r][j])) : 0.0f;
            O[r][j] = gy[j] * Y[r][j];
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) Dl[r] = mfma4(x.tb[s], Z[r][s], Dl[r]);
    // O = scale gamma c . Y' + P Delta.
    f32x4 pm = x.pm;
    if constexpr (kBf16Mma<D, AT>) pm *= QKt;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) O[r] = mfma4(pm[s], Dl[r][s], O[r]);
    // S' <- S' + K^T diag(Gam_end / c_new) Delta with c_new = gamma_15 c, tile by tile of 16 key
    // columns (after folding c_new into S' when it is out of range).
    float cn = x.gend * c;
    if (!(fabsf(cn) >= 0x1p-64f && fabsf(cn) <= 0x1p64f)) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) S[r][mt] *= cn;
        cn = 1.0f;
    }
    c = cn;
    const float rc = 1.0f / cn;
    f32x4 Dt[RT];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float f = x.ge[j] * rc;
#pragma unroll
        for (int r = 0; r < RT; ++r) Dt[r][j] = f * Dl[r][j];
    }
    if constexpr (kBf16Mma<D, AT>) {
        // 16 x 16 x 16 over the chunk's tokens 4g .. 4g+3 (lane group g): K^T as packed pairs of
        // tokens (4g, 4g+1), (4g+2, 4g+3) of column NMT m + mt; Delta' as three bf16 parts.
        u32x2 dh[RT], dm[RT], dl[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const Split3 p0 = split3(Dt[r][0], Dt[r][1]), p1 = split3(Dt[r][2], Dt[r][3]);
            dh[r] = u32x2{p0.h, p1.h};
            dm[r] = u32x2{p0.m, p1.m};
            dl[r] = u32x2{p0.l, p1.l};
        }
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            const int wi = mt >> 1;
            const uint32_t k0 = x.ku[0].w[wi], k1 = x.ku[1].w[wi], k2 = x.ku[2].w[wi], k3 = x.ku[3].w[wi];
            const u32x2 ka = (mt & 1) ? u32x2{hi_halves(k0, k1), hi_halves(k2, k3)}
                                      : u32x2{lo_halves(k0, k1), lo_halves(k2, k3)};
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                S[r][mt] = mfma_k16(ka, dh[r], S[r][mt]);
                S[r][mt] = mfma_k16(ka, dm[r], S[r][mt]);
                S[r][mt] = mfma_k16(ka, dl[r], S[r][mt]);
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                const float ks = x.ku[s].get(mt);
#pragma unroll
                for (int r = 0; r < RT; ++r) S[r][mt] = mfma4(ks, Dt[r][s], S[r][mt]);
            }
    }

    const int64_t tok0 = (b * T + ci * CH) * H + h;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (4 * g + j < nv) {
            AT* ot = o + (tok0 + (int64_t)(4 * g + j) * H) * D + row0;
#pragma unroll
            for (int r = 0; r < RT; ++r) ot[16 * r] = from_f32<AT>(O[r][j]);
        }
}

// Two consecutive chunks (x0 = chunk ci, x1 = chunk ci + 1) from one split of S', for the
// bf16 matrix-core path. With S_mid = gamma0_15 c S' + K0^T diag(Gam_end0) Delta0 the state
// between the chunks (never formed) and M = K1 K0^T, N = Q1 K0^T (16 x 16), the second chunk's
// products are
//     K1 S_mid^T = c_mid K1 S'^T + (M diag(Gam_end0)) Delta0,   c_mid = gamma0_15 c,
//     Q1 S_mid^T = c_mid Q1 S'^T + (N diag(Gam_end0)) Delta0,
// so both chunks take their products from the same three bf16 parts of S' and the second adds
// a 16 x 16 correction on the matrix cores. The state update then runs once for both chunks,
// contracting over their 32 tokens on the 16 x 16 x 32 form:
//     S'_end = S' + K0^T diag(Gam_end0 gamma1_15 / c_end) Delta0 + K1^T diag(Gam_end1 / c_end) Delta1,
// c_end = gamma1_15 c_mid (folded into S' when out of [2^-64, 2^64], as in chunk_step). Same
// algebra as two chunk_step calls; fp32 rounding differs. `prefetch` issues the next pair's
// loads before anything else (prompt workload 622 -> 593 us against issuing them after the S'
// products: the longer the loads have, the fewer of the head's four waves miss in the L2).
template <int D, int RT, typename AT, typename F>
__device__ __forceinline__ void pair_step(f32x4 (&S)[RT][D / 16], float& c,
                                          const ChunkOps<D, RT, AT>& x0,
                                          const ChunkOps<D, RT, AT>& x1, int ci, int T, int H,
                                          int64_t b, int h, int row0, AT* __restrict__ o,
                                          float scale, int g, F&& prefetch) {
    static_assert(kBf16Mma<D, AT>, "the paired form runs on the bf16 matrix cores");
    constexpr int NMT = D / 16;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    prefetch();
    __builtin_amdgcn_sched_barrier(0);
    f32x4 X0[RT], Y0[RT], X1[RT], Y1[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) X0[r] = Y0[r] = X1[r] = Y1[r] = zero4;
    // QKj: lane (g, m) ends with k_{4g+s} . q_m of chunk j (P's a operand); M and N: lane
    // (g, n) ends with k0_{4g+s} . k1_n and k0_{4g+s} . q1_n, i.e. M[n][4g+s], N[n][4g+s], the
    // a operands of the corrections.
    f32x4 QK0 = zero4, QK1 = zero4, M = zero4, N = zero4;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        const u32x4 ka0 = {x0.kx.w[4 * s], x0.kx.w[4 * s + 1], x0.kx.w[4 * s + 2], x0.kx.w[4 * s + 3]};
        const u32x4 qa0 = {x0.qx.w[4 * s], x0.qx.w[4 * s + 1], x0.qx.w[4 * s + 2], x0.qx.w[4 * s + 3]};
        const u32x4 ka1 = {x1.kx.w[4 * s], x1.kx.w[4 * s + 1], x1.kx.w[4 * s + 2], x1.kx.w[4 * s + 3]};
        const u32x4 qa1 = {x1.qx.w[4 * s], x1.qx.w[4 * s + 1], x1.qx.w[4 * s + 2], x1.qx.w[4 * s + 3]};
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            Split3 p[4];
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const int t = 8 * s + 2 * pp;
                p[pp] = split3(S[r][t % NMT][t / NMT], S[r][t % NMT + 1][t / NMT]);
            }
            const u32x4 bh = {p[0].h, p[1].h, p[2].h, p[3].h};
            const u32x4 bm = {p[0].m, p[1].m, p[2].m, p[3].m};
            const u32x4 bl = {p[0].l, p[1].l, p[2].l, p[3].l};
            X0[r] = mfma_k32(ka0, bh, X0[r]);
            X1[r] = mfma_k32(ka1, bh, X1[r]);
            Y0[r] = mfma_k32(qa0, bh, Y0[r]);
            Y1[r] = mfma_k32(qa1, bh, Y1[r]);
            X0[r] = mfma_k32(ka0, bm, X0[r]);
            X1[r] = mfma_k32(ka1, bm, X1[r]);
            Y0[r] = mfma_k32(qa0, bm, Y0[r]);
            Y1[r] = mfma_k32(qa1, bm, Y1[r]);
            X0[r] = mfma_k32(ka0, bl, X0[r]);
            X1[r] = mfma_k32(ka1, bl, X1[r]);
        }
        QK0 = mfma_k32(ka0, qa0, QK0);
        QK1 = mfma_k32(ka1, qa1, QK1);
        M = mfma_k32(ka0, ka1, M);
        N = mfma_k32(ka0, qa1, N);
    }
    // First chunk, as in chunk_step.
    f32x4 Z0[RT], D0[RT], O0[RT];
    f32x4 gx0, gy0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gx0[j] = x0.gm[j] * c;
        gy0[j] = gx0[j] * scale;
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        D0[r] = zero4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Z0[r][j] = (4 * g + j < x0.nv) ? fmaf(-gx0[j], X0[r][j], to_f32<AT>(x0.v[r][j])) : 0.0f;
            O0[r][j] = gy0[j] * Y0[r][j];
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) D0[r] = mfma4(x0.tb[s], Z0[r][s], D0[r]);
    const f32x4 pm0 = x0.pm * QK0;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) O0[r] = mfma4(pm0[s], D0[r][s], O0[r]);

    // Second chunk: its products with S_mid, the corrections through Delta0.
    const float cm = x0.gend * c;
    const f32x4 Mg = M * x0.ge, Ng = N * x0.ge;
    f32x4 Xc[RT], Yc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) Xc[r] = Yc[r] = zero4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            Xc[r] = mfma4(Mg[s], D0[r][s], Xc[r]);
            Yc[r] = mfma4(Ng[s], D0[r][s], Yc[r]);
        }
    f32x4 Z1[RT], D1[RT], O1[RT];
    f32x4 gx1, gy1, sg1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gx1[j] = x1.gm[j] * cm;
        gy1[j] = gx1[j] * scale;
        sg1[j] = x1.gm[j] * scale;
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        D1[r] = zero4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float z = fmaf(-gx1[j], X1[r][j], to_f32<AT>(x1.v[r][j]));
            Z1[r][j] = (4 * g + j < x1.nv) ? fmaf(-x1.gm[j], Xc[r][j], z) : 0.0f;
            O1[r][j] = fmaf(gy1[j], Y1[r][j], sg1[j] * Yc[r][j]);
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) D1[r] = mfma4(x1.tb[s], Z1[r][s], D1[r]);
    const f32x4 pm1 = x1.pm * QK1;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) O1[r] = mfma4(pm1[s], D1[r][s], O1[r]);

    // The update over both chunks' 32 tokens.
    float cn = x1.gend * cm;
    if (!(fabsf(cn) >= 0x1p-64f && fabsf(cn) <= 0x1p64f)) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) S[r][mt] *= cn;
        cn = 1.0f;
    }
    c = cn;
    const float rc = 1.0f / cn;
    const float r0 = x1.gend * rc;
    u32x4 dh[RT], dm[RT], dl[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        f32x4 t0, t1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            t0[j] = (x0.ge[j] * r0) * D0[r][j];
            t1[j] = (x1.ge[j] * rc) * D1[r][j];
        }
        const Split3 p0 = split3(t0[0], t0[1]), p1 = split3(t0[2], t0[3]);
        const Split3 p2 = split3(t1[0], t1[1]), p3 = split3(t1[2], t1[3]);
        dh[r] = u32x4{p0.h, p1.h, p2.h, p3.h};
        dm[r] = u32x4{p0.m, p1.m, p2.m, p3.m};
        dl[r] = u32x4{p0.l, p1.l, p2.l, p3.l};
    }
    // 16 x 16 x 32: lane group g holds contraction slots 8g .. 8g+7 = tokens 4g .. 4g+3 of the
    // first chunk, then of the second; K^T as packed pairs of those tokens of column NMT m + mt.
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const int wi = mt >> 1;
        const uint32_t a0 = x0.ku[0].w[wi], a1 = x0.ku[1].w[wi], a2 = x0.ku[2].w[wi], a3 = x0.ku[3].w[wi];
        const uint32_t b0 = x1.ku[0].w[wi], b1 = x1.ku[1].w[wi], b2 = x1.ku[2].w[wi], b3 = x1.ku[3].w[wi];
        const u32x4 ka = (mt & 1)
            ? u32x4{hi_halves(a0, a1), hi_halves(a2, a3), hi_halves(b0, b1), hi_halves(b2, b3)}
            : u32x4{lo_halves(a0, a1), lo_halves(a2, a3), lo_halves(b0, b1), lo_halves(b2, b3)};
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            S[r][mt] = mfma_k32(ka, dh[r], S[r][mt]);
            S[r][mt] = mfma_k32(ka, dm[r], S[r][mt]);
            S[r][mt] = mfma_k32(ka, dl[r], S[r][mt]);
        }
    }

    const int64_t tok0 = (b * T + ci * CH) * H + h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        AT* ot = o + (tok0 + (int64_t)(4 * g + j) * H) * D + row0;
#pragma unroll
        for (int r = 0; r < RT; ++r) ot[16 * r] = from_f32<AT>(O0[r][j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (4 * g + j < x1.nv) {
            AT* ot = o + (tok0 + (int64_t)(CH + 4 * g + j) * H) * D + row0;
#pragma unroll
            for (int r = 0; r < RT; ++r) ot[16 * r] = from_f32<AT>(O1[r][j]);
        }
}

// One wave per (b, h, RT tiles of 16 state rows). With `remap`, workgroup ids are regrouped so
// the waves of a head run on one XCD (workgroup i runs on XCD i % 8) and share its L2 for the
// head's k, q and chunk records.
template <int D, int RT, typename AT, typename ST>
__global__ __launch_bounds__(64) void gdn_prefill_state_kernel(
    int T, int H, int nch, const AT* __restrict__ q, const AT* __restrict__ k,
    const AT* __restrict__ v, const float* __restrict__ ws, ST* __restrict__ state,
    AT* __restrict__ o, float scale, int remap) {
    constexpr int R = D / 4, NMT = D / 16, NW = D / (16 * RT);
    static_assert(NW * 16 * RT == D, "tiles per wave");
    const int lane = threadIdx.x, g = lane >> 4, n = lane & 15;
    uint32_t w = blockIdx.x;
    if (remap) w = (w & 7u) * (gridDim.x >> 3) + (w >> 3);
    const int wt = (int)(w % NW);
    const int64_t bh = w / NW;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    const int row0 = 16 * RT * wt + n;

    // State rows: each lane reads its D/4 contiguous columns, so one load instruction touches
    // 16 bytes of each of 64 lines and the lines fill over the run's instructions. Ordinary
    // (cached) loads and stores let the L2 merge those partial lines; with the nontemporal
    // hint a short-prompt call (B=256, T=16, fp32 state) took 1159 instead of 534 us.
    f32x4 S[RT][NMT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        Run<ST, R> sr;
        sr.template load<false>(state + ((size_t)bh * D + row0 + 16 * r) * D + R * g);
#pragma unroll
        for (int e = 0; e < R; ++e) S[r][e % NMT][e / NMT] = sr.get(e);
    }

    const float* wsh = ws + (size_t)bh * nch * REC;
    float cs = 1.0f;  // S = cs S' (wave-uniform)
    if constexpr (kBf16Mma<D, AT>) {
        // Chunks in pairs (pair_step); the next pair's operands load while the current pair
        // computes. An odd last chunk runs alone.
        ChunkOps<D, RT, AT> A0, A1, B0, B1;
        load_chunk<D, RT, AT>(A0, 0, T, H, b, h, row0, q, k, v, wsh, g, n);
        load_chunk<D, RT, AT>(A1, min(1, nch - 1), T, H, b, h, row0, q, k, v, wsh, g, n);
        for (int c = 0; c + 1 < nch; c += 4) {
            pair_step<D, RT, AT>(S, cs, A0, A1, c, T, H, b, h, row0, o, scale, g, [&]() {
                load_chunk<D, RT, AT>(B0, min(c + 2, nch - 1), T, H, b, h, row0, q, k, v, wsh, g, n);
                load_chunk<D, RT, AT>(B1, min(c + 3, nch - 1), T, H, b, h, row0, q, k, v, wsh, g, n);
            });
            if (c + 3 >= nch) break;
            pair_step<D, RT, AT>(S, cs, B0, B1, c + 2, T, H, b, h, row0, o, scale, g, [&]() {
                load_chunk<D, RT, AT>(A0, min(c + 4, nch - 1), T, H, b, h, row0, q, k, v, wsh, g, n);
                load_chunk<D, RT, AT>(A1, min(c + 5, nch - 1), T, H, b, h, row0, q, k, v, wsh, g, n);
            });
        }
        if (nch & 1) {
            load_chunk<D, RT, AT>(A0, nch - 1, T, H, b, h, row0, q, k, v, wsh, g, n);
            chunk_step<D, RT, AT>(S, cs, A0, nch - 1, T, H, b, h, row0, o, scale, g);
        }
    } else {
        ChunkOps<D, RT, AT> A, Bo;
        load_chunk<D, RT, AT>(A, 0, T, H, b, h, row0, q, k, v, wsh, g, n);
        // The prefetches are unconditional (the last chunk is read again at the end): a load
        // that only some paths issue would make the compiler wait for every load in flight. The
        // scheduling barriers keep them ahead of the chunk's products instead of sunk to its end.
        for (int c = 0; c < nch; c += 2) {
            load_chunk<D, RT, AT>(Bo, min(c + 1, nch - 1), T, H, b, h, row0, q, k, v, wsh, g, n);
            __builtin_amdgcn_sched_barrier(0);
            chunk_step<D, RT, AT>(S, cs, A, c, T, H, b, h, row0, o, scale, g);
            if (c + 1 >= nch) break;
            load_chunk<D, RT, AT>(A, min(c + 2, nch - 1), T, H, b, h, row0, q, k, v, wsh, g, n);
            __builtin_amdgcn_sched_barrier(0);
            chunk_step<D, RT, AT>(S, cs, Bo, c + 1, T, H, b, h, row0, o, scale, g);
        }
    }

#pragma unroll
    for (int r = 0; r < RT; ++r) {
        float out[R];
#pragma unroll
        for (int e = 0; e < R; ++e) out[e] = S[r][e % NMT][e / NMT] * cs;
        store_run<ST, R, false>(state + ((size_t)bh * D + row0 + 16 * r) * D + R * g, out);
    }
}

// ------------------------------------------------------------------------ dispatch

template <int D, typename AT, typename ST>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
    int T = a.T, H = a.H;
    int nch = (int)prefill_chunks(a.T);
    const AT* q = (const AT*)a.q;
    const AT* k = (const AT*)a.k;
    const AT* v = (const AT*)a.v;
    const float* alpha = a.alpha;
    const float* beta = a.beta;
    float* ws = a.ws;
    const float* wsc = a.ws;
    ST* state = (ST*)a.state;
    AT* o = (AT*)a.o;
    float scale = a.scale;
    const int64_t heads = a.B * a.H;
    void* pargs[] = {&T, &H, &nch, &q, &k, &alpha, &beta, &ws, &scale};
    hipError_t e = hipLaunchKernel((const void*)gdn_prefill_prep_kernel<D, AT>,
                                   dim3((unsigned)(heads * nch)), dim3(64), pargs, 0, s);
    if (e != hipSuccess) return e;
    constexpr int RT = (D >= 32) ? 2 : 1;  // 16-row tiles per wave
    static_assert(D / (16 * RT) * 64 <= kThreadsPerHeadPerDim * D, "threads per head");
    const unsigned grid = (unsigned)(heads * (D / (16 * RT)));
    int remap = (grid % 8u == 0u) ? 1 : 0;
    void* sargs[] = {&T, &H, &nch, &q, &k, &v, &wsc, &state, &o, &scale, &remap};
    return hipLaunchKernel((const void*)gdn_prefill_state_kernel<D, RT, AT, ST>, dim3(grid),
                           dim3(64), sargs, 0, s);
}

template <int D, typename ST>
hipError_t launch_prefill_s(const PrefillArgs& a, hipStream_t s) {
    switch (a.act) {
        case DType::F32: return launch_prefill_t<D, float, ST>(a, s);
        case DType::BF16: return launch_prefill_t<D, uint16_t, ST>(a, s);
        default: return launch_prefill_t<D, _Float16, ST>(a, s);
    }
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t s) {
    switch (a.state_dtype) {
        case DType::F32: return launch_prefill_s<D, float>(a, s);
        case DType::BF16: return launch_prefill_s<D, uint16_t>(a, s);
        default: return launch_prefill_s<D, _Float16>(a, s);
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    switch (a.D) {
        case 16: return launch_prefill_d<16>(a, s);
        case 32: return launch_prefill_d<32>(a, s);
        case 64: return launch_prefill_d<64>(a, s);
        default: return launch_prefill_d<128>(a, s);
    }
}

// ------------------------------------------------------------------------ fixed scratch

// The chunk records of gdn_prefill_noalloc live in this file-scope device array instead of a
// caller's workspace. Every GPU the library runs on holds its own copy until the process ends;
// in host code `scratch` is only a host-side stand-in for it, so its device address is
// looked up once per device (hipGetSymbolAddress, with that device current) and only that
// address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[kPrefillScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t prefill_scratch_address(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = static_cast<float*>(p);
    return hipSuccess;
}

}  // namespace gdn
