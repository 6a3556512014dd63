// In-place stream probe: a calibration kernel for the benchmark, not part of the GDN library.
//
// It reads a [heads][128][128] state buffer and writes every word back to where it came from,
// with the same tile geometry, lane mapping, 16-byte vector width, cache hints and workgroup
// order as the decode kernels' state load and store, and no arithmetic (each word is XORed
// with a runtime zero so the compiler cannot drop the store). Its time is the practical
// ceiling of the decode kernels' in-place read-modify-write stream on this GPU: what a decode
// launch would take if the recurrence cost nothing. The per-head vectors (q, k, v, gates, o)
// are not touched; they are under 1% of a decode launch's bytes.
//
// Variants (`variant` argument), all for a 128 x 128 state per head:
//   0  4-byte state, one-token decode geometry: one wave per workgroup, 16 workgroups per
//      head of 8 rows each, 16 lanes per row, nontemporal loads and stores
//   1  4-byte state, multi-token decode geometry: one wave per workgroup, 8 workgroups per
//      head of 16 rows each, 16 lanes per row, nontemporal
//   2  2-byte state, one-token decode geometry: 16 waves per workgroup (one per head), 8 rows
//      per wave, 8 lanes per row, nontemporal
//   3  as 0 with ordinary cached loads and stores
//   4  4-byte state, one wave per workgroup, 4 rows per wave (32 workgroups per head)
//   5  4-byte state, 4 waves per workgroup of 8 rows each (4 workgroups per head)
//   6  4-byte state, 16 waves per workgroup of 8 rows each (one workgroup per head)
//   7  4-byte state, one wave of 8 rows per workgroup, 32 lanes per row (2 whole rows, 1 KiB
//      contiguous, per load instruction)
//   8  4-byte state, one wave of 8 rows per workgroup, 8 lanes per row
//   9  4-byte state, one wave of 16 rows per workgroup, 32 lanes per row
//  10  4-byte state, one wave of 32 rows per workgroup, 16 lanes per row
// `group` sets the workgroup order over the 8 XCDs (workgroup i runs on XCD i % 8): runs of
// `group` consecutive tiles share an XCD (1 = consecutive tiles on different XCDs; 16 with
// variant 0 = every tile of a head on one XCD). Tiles past the last multiple of 8 * group keep
// the plain order.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int ES, int LPR, int RPW, int WAVES, int SPLIT, bool NT>
__global__ __launch_bounds__(64 * WAVES) void gdn_stream_probe_kernel(uint8_t* __restrict__ state,
                                                                     uint32_t group, uint32_t x) {
    constexpr int D = 128;
    constexpr int VW = 16 / ES;        // elements per 16-byte vector
    constexpr int E = D / LPR;         // elements per lane and row
    constexpr int NCH = E / VW;        // vectors per lane and row
    constexpr int RPP = 64 / LPR;      // rows per pass of a wave
    constexpr int P = RPW / RPP;       // passes per wave
    constexpr int RPG = RPW * WAVES;   // rows per workgroup
    static_assert(RPG * SPLIT == D && P >= 1 && NCH >= 1, "geometry");
    const uint32_t bid = blockIdx.x, n = gridDim.x;
    uint32_t tile = bid;
    const uint32_t grouped = (n / (8u * group)) * (8u * group);
    if (bid < grouped) {
        const uint32_t xcd = bid & 7u, i = bid >> 3;
        tile = ((i / group) * 8u + xcd) * group + (i % group);
    }
    const uint32_t head = tile / SPLIT, part = tile - head * SPLIT;
    uint8_t* base = state + (size_t)head * D * D * ES;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, l = lane % LPR;
    const int row0 = part * RPG + wave * RPW + g;
    u32x4 r[P][NCH];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const u32x4* a = (const u32x4*)(base + ((size_t)(row0 + p * RPP) * D + c * LPR * VW + l * VW) * ES);
            r[p][c] = NT ? __builtin_nontemporal_load(a) : *a;
        }
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            u32x4* a = (u32x4*)(base + ((size_t)(row0 + p * RPP) * D + c * LPR * VW + l * VW) * ES);
            const u32x4 w = r[p][c] ^ x;
            if (NT) __builtin_nontemporal_store(w, a); else *a = w;
        }
}

template <int ES, int LPR, int RPW, int WAVES, int SPLIT, bool NT>
hipError_t launch(void* state, int64_t heads, uint32_t group, hipStream_t s) {
    uint8_t* p = (uint8_t*)state;
    uint32_t x = 0;
    void* args[] = {&p, &group, &x};
    return hipLaunchKernel((const void*)gdn_stream_probe_kernel<ES, LPR, RPW, WAVES, SPLIT, NT>,
                           dim3((uint32_t)(heads * SPLIT)), dim3(64 * WAVES), args, 0, s);
}

}  // namespace

// `bytes` is the size of the buffer at `state`; a variant whose heads x 128 x 128 elements do
// not fit in it is refused. Returns 0 on success, 1 for bad arguments (nothing launched), 2 if
// the launch failed.
extern "C" int gdn_stream_probe(void* state, size_t bytes, int64_t heads, int variant,
                                uint32_t group, void* stream) {
    if (state == nullptr || heads < 1 || heads * 32 >= (int64_t(1) << 31) || group < 1 ||
        ((uintptr_t)state & 15u) != 0)
        return 1;
    const size_t elem = variant == 2 ? 2 : 4;
    if (variant < 0 || variant > 10 || (size_t)heads * 128 * 128 * elem > bytes) return 1;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (variant) {
        case 0: e = launch<4, 16, 8, 1, 16, true>(state, heads, group, s); break;
        case 1: e = launch<4, 16, 16, 1, 8, true>(state, heads, group, s); break;
        case 2: e = launch<2, 8, 8, 16, 1, true>(state, heads, group, s); break;
        case 3: e = launch<4, 16, 8, 1, 16, false>(state, heads, group, s); break;
        case 4: e = launch<4, 16, 4, 1, 32, true>(state, heads, group, s); break;
        case 5: e = launch<4, 16, 8, 4, 4, true>(state, heads, group, s); break;
        case 6: e = launch<4, 16, 8, 16, 1, true>(state, heads, group, s); break;
        case 7: e = launch<4, 32, 8, 1, 16, true>(state, heads, group, s); break;
        case 8: e = launch<4, 8, 8, 1, 16, true>(state, heads, group, s); break;
        case 9: e = launch<4, 32, 16, 1, 8, true>(state, heads, group, s); break;
        case 10: e = launch<4, 16, 32, 1, 4, true>(state, heads, group, s); break;
        default: return 1;
    }
    return e == hipSuccess ? 0 : 2;
}
