// Axis-1 trellis kernels for gfx950: the fused decode + bf16 MFMA kernel that
// serves both the M = 1 GEMV and the M <= 32 prefill, and the diagnostic
// expand kernel. Both decode through the same fragment builder.
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0,
// page 60: tiled-prefill.ts (axis-1 tile decode + matrix multiply, bf16
// rounding of each weight), wide-prefill.ts (axis-1 multi-vector GEMV),
// vector-expand.ts (whole-matrix decode).
//
// Work mapping (one 64-lane wavefront):
//   lane l -> stored row n0 + (l % 16), run c = l / 16 of the current block.
//   Run c holds weights t in [64c, 64c + 64) of a 256-weight block. Weight t
//   sits at bit (255 - t) * k, so the run is the contiguous bit range
//   [64 (3 - c) k, 64 (4 - c) k) -- exactly 2k words -- plus the 11 window
//   bits that spill into the next word (the block's word 0 for the last run:
//   the tail-biting wrap). Each lane therefore loads 2k + 1 words, coalesced
//   across the 4 runs of a row.
//   The 64 weights of a run become eight 8-weight B fragments of
//   v_mfma_f32_16x16x32_bf16 (B[k][n], k = 8 c + e within the instruction);
//   the A fragment is the matching 8 activations of row m = l % 16. Because
//   A and B index k identically, the hardware's k order inside the
//   instruction does not matter.
//   A workgroup (4 waves) owns 16 output rows; wave w takes blocks
//   w, w + 4, ... and the four partial tiles are summed in LDS in a fixed
//   order, so results are deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace trellis {
namespace {

constexpr int kThreads = 256;

// One block of a wave: 8 B fragments, each multiplied against MT A fragments
// (x rows m = 16 mt + j). Row m of A only feeds row m of D, so lanes whose m
// is at or past M may carry any finite row of x: their D rows are never
// stored, and no masking is needed.
template <int K, int MT>
__device__ __forceinline__ void block_mma(const uint32_t (&w)[2 * K + 1],
                                          const float* __restrict__ lut_s, float scale,
                                          const uint16_t* __restrict__ xrow0,
                                          const uint16_t* __restrict__ xrow1,
                                          floatx4 (&acc)[MT]) {
    static_for<0, 8>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        const bf16x8 bfrag = as_bf16x8(run64_fragment<K, S, false>(w, lut_s, scale));
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(xrow0 + 8 * S);
        acc[0] = mfma16x16x32(as_bf16x8(a0), bfrag, acc[0]);
        if constexpr (MT == 2) {
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(xrow1 + 8 * S);
            acc[1] = mfma16x16x32(as_bf16x8(a1), bfrag, acc[1]);
        }
    });
}

template <int K, int MT>
__global__ __launch_bounds__(kThreads) void axis1_mma_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
    const float* __restrict__ scales, const float* __restrict__ lut,
    uint16_t* __restrict__ y, int N, int nb, int M) {
    constexpr int wpb = Bits<K>::wpb;
    __shared__ __attribute__((aligned(16))) float lut_s[kLutEntries];
    __shared__ float red[4][MT * 16][16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, c = lane >> 4, cp = 3 - c;
    const int n0 = blockIdx.x * 16;
    const int n = n0 + j;
    const int row = n < N ? n : N - 1;  // ragged tail: valid address, result dropped
    const long in = static_cast<long>(nb) * kT;
    const uint32_t* __restrict__ rowp = codes + static_cast<size_t>(row) * nb * wpb;
    const float scale = scales[row];
    // A-fragment rows: m = j (and 16 + j); rows past M read row 0 (see block_mma).
    const uint16_t* __restrict__ xr0 = x + (j < M ? j : 0) * in + 64 * c;
    const uint16_t* __restrict__ xr1 = x + (16 + j < M ? 16 + j : 0) * in + 64 * c;

    uint32_t wa[2 * K + 1], wb[2 * K + 1];
    if (wave < nb) load_run64<K>(rowp + static_cast<size_t>(wave) * wpb, cp, wa);
    stage_lut<kThreads>(lut_s, lut);
    __syncthreads();

    floatx4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Blocks wave, wave + 4, ...; two register sets ping-pong so the next
    // block's words are in flight while the current one is decoded.
    for (int b = wave; b < nb; b += 8) {
        if (b + 4 < nb) load_run64<K>(rowp + static_cast<size_t>(b + 4) * wpb, cp, wb);
        block_mma<K, MT>(wa, lut_s, scale, xr0 + static_cast<long>(b) * kT,
                         xr1 + static_cast<long>(b) * kT, acc);
        if (b + 4 >= nb) break;
        if (b + 8 < nb) load_run64<K>(rowp + static_cast<size_t>(b + 8) * wpb, cp, wa);
        block_mma<K, MT>(wb, lut_s, scale, xr0 + static_cast<long>(b + 4) * kT,
                         xr1 + static_cast<long>(b + 4) * kT, acc);
    }

    // D layout: lane holds D[m = 4c + v][n = j] of each 16x16 tile.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][mt * 16 + 4 * c + v][j] = acc[mt][v];
    __syncthreads();
    for (int idx = tid; idx < MT * 16 * 16; idx += kThreads) {
        const int m = idx >> 4, jj = idx & 15;
        const float sum = ((red[0][m][jj] + red[1][m][jj]) + red[2][m][jj]) + red[3][m][jj];
        const int nn = n0 + jj;
        if (m < M && nn < N) y[static_cast<size_t>(m) * N + nn] = round_bf16(sum);
    }
}

// Whole-matrix decode: one lane per 64-weight run, same fragment builder as
// the fused kernel, 16-byte stores of 8 bf16 weights.
template <int K>
__global__ __launch_bounds__(kThreads) void expand_kernel(
    const uint32_t* __restrict__ codes, const float* __restrict__ scales,
    const float* __restrict__ lut, uint16_t* __restrict__ w, long rows, int nb) {
    constexpr int wpb = Bits<K>::wpb;
    __shared__ __attribute__((aligned(16))) float lut_s[kLutEntries];
    stage_lut<kThreads>(lut_s, lut);
    __syncthreads();
    const long run = static_cast<long>(blockIdx.x) * kThreads + threadIdx.x;
    const long runs = rows * nb * 4;
    if (run >= runs) return;
    const long row = run / (static_cast<long>(nb) * 4);
    const int rem = static_cast<int>(run - row * nb * 4);
    const int b = rem >> 2, cp = rem & 3, c = 3 - cp;
    uint32_t wr[2 * K + 1];
    load_run64<K>(codes + (static_cast<size_t>(row) * nb + b) * wpb, cp, wr);
    const float scale = scales[row];
    uint16_t* dst = w + static_cast<size_t>(row) * nb * kT + b * kT + 64 * c;
    static_for<0, 8>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        *reinterpret_cast<u32x4*>(dst + 8 * S) = run64_fragment<K, S, false>(wr, lut_s, scale);
    });
}

template <int K, int MT>
hipError_t launch_axis1_k(const uint16_t* x, int M, const uint32_t* codes, const float* scales,
                          const float* lut, uint16_t* y, int N, int nb, hipStream_t st) {
    const dim3 grid((N + 15) / 16);
    return launch_kernel(axis1_mma_kernel<K, MT>, grid, dim3(kThreads), st, x, codes, scales, lut, y,
                         N, nb, M);
}

template <int K>
hipError_t launch_expand_k(const uint32_t* codes, const float* scales, const float* lut,
                           uint16_t* w, long rows, int nb, hipStream_t st) {
    const long runs = rows * nb * 4;
    const dim3 grid(static_cast<unsigned>((runs + kThreads - 1) / kThreads));
    return launch_kernel(expand_kernel<K>, grid, dim3(kThreads), st, codes, scales, lut, w, rows, nb);
}

}  // namespace

hipError_t launch_axis1(const uint16_t* x, int M, const uint32_t* codes, const float* scales,
                        const float* lut, uint16_t* y, int N, int nb, int k, hipStream_t st) {
    const bool two = M > 16;
    switch (k) {
    case 2: return two ? launch_axis1_k<2, 2>(x, M, codes, scales, lut, y, N, nb, st)
                       : launch_axis1_k<2, 1>(x, M, codes, scales, lut, y, N, nb, st);
    case 3: return two ? launch_axis1_k<3, 2>(x, M, codes, scales, lut, y, N, nb, st)
                       : launch_axis1_k<3, 1>(x, M, codes, scales, lut, y, N, nb, st);
    case 4: return two ? launch_axis1_k<4, 2>(x, M, codes, scales, lut, y, N, nb, st)
                       : launch_axis1_k<4, 1>(x, M, codes, scales, lut, y, N, nb, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_expand(const uint32_t* codes, const float* scales, const float* lut,
                         uint16_t* w, long rows, int nb, int k, hipStream_t st) {
    switch (k) {
    case 2: return launch_expand_k<2>(codes, scales, lut, w, rows, nb, st);
    case 3: return launch_expand_k<3>(codes, scales, lut, w, rows, nb, st);
    case 4: return launch_expand_k<4>(codes, scales, lut, w, rows, nb, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace trellis
