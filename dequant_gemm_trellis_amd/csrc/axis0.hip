// Axis-0 trellis kernels for gfx950: split-K decode + bf16 MFMA partials and
// the ordered split reduction. They serve the M = 1 "scatter" GEMV and the
// axis-0 prefill.
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0,
// page 59: scatter.ts (axis-0 GEMV: 128 row splits of ceil(rows/128) rows,
// float32 partials [M][128][cols], then a sum over the split axis and a cast)
// and splitk-prefill.ts (axis-0 prefill: split-K float32 partials and an
// ordered accumulate kernel).
//
// On axis 0 the contraction runs over stored rows r, and the MFMA B fragment
// of a lane holds 8 consecutive contraction indices of one output column. So
// a lane decodes an 8 x 8 patch: 8 stored rows x 8 adjacent columns. For each
// row it loads the two words that hold the 8 windows (always enough: at most
// 7k + 12 bits starting anywhere inside a word), funnels them to a 64-bit
// value, and reads the windows at compile-time offsets. Column e of the patch
// over the 8 rows is the B fragment of MFMA number e, whose accumulator
// collects output column 8j + e. The A fragment is x[m][the same 8 rows].
//
// Mapping: a wave owns 128 output columns (lane j = l % 16 -> columns
// 8j..8j+7, row chunk c = l / 16 -> rows 8c..8c+7 of each 32-row step) and one
// split of rows. A workgroup holds the 4 consecutive splits of one column
// tile; their partials are summed in LDS in wave order, then written as one
// partial per split group. The reduce kernel sums split groups in ascending
// order. Every order is fixed, so repeated calls give identical bits.
#include "common.hpp"
#include "launch.hpp"

namespace trellis {
namespace {

constexpr int kThreads = 256;  // split reduce
constexpr int kTileCols = 128;
// Splits per workgroup, one wave each; their partials are summed in LDS in
// wave order. (8 or 16 per workgroup measured 15% and 3x slower.)
constexpr int kA0Waves = 4;
constexpr int kA0Threads = kA0Waves * kWave;

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    floatx2 p = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}

template <int K, int MT>
__global__ __launch_bounds__(kA0Threads) void axis0_mma_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
    const float* __restrict__ scales, const float* __restrict__ lut,
    float* __restrict__ partial, int R, int C, int M, int S, int rows_per_split) {
    constexpr int wpb = Bits<K>::wpb;
    __shared__ __attribute__((aligned(16))) float lut_s[kLutEntries];
    __shared__ float red[8][MT * 16][16];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, c = lane >> 4;
    const int groups = (S + kA0Waves - 1) / kA0Waves;
    const int tile = blockIdx.x / groups;
    const int sgroup = blockIdx.x - tile * groups;
    const int split = sgroup * kA0Waves + wave;
    const int col0 = tile * kTileCols;
    const int blk = col0 / kT;
    const int t0 = (col0 % kT) + 8 * j;         // first weight of this lane's 8 columns
    const int lo = (kT - 8 - t0) * K;           // bit of weight t0 + 7
    const int w0 = lo >> 5, sh = lo & 31;
    const int w1 = (w0 + 1 == wpb) ? 0 : w0 + 1;  // tail-biting wrap to word 0
    const size_t row_words = static_cast<size_t>(C) / kT * wpb;
    const uint32_t* __restrict__ cbase = codes + static_cast<size_t>(blk) * wpb;

    int r_begin = split * rows_per_split;
    int r_end = r_begin + rows_per_split;
    if (split >= S) r_begin = r_end = 0;
    if (r_end > R) r_end = R;
    if (r_begin > r_end) r_begin = r_end;

    stage_lut<kA0Threads>(lut_s, lut);
    __syncthreads();

    floatx4 acc[8][MT];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[e][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // A-fragment rows m = 16 mt + j; rows at or past M read row 0 (their D
    // rows are never stored). Contraction rows past the split end are real
    // terms and are zeroed in x.
    const uint16_t* __restrict__ xr0 = x + static_cast<size_t>(j < M ? j : 0) * R;
    const uint16_t* __restrict__ xr1 = x + static_cast<size_t>(16 + j < M ? 16 + j : 0) * R;

    for (int rs = r_begin; rs < r_end; rs += 32) {
        const int rc = rs + 8 * c;  // first row of this lane's chunk
        uint32_t g[8][2];
        float sc[8];
        static_for<0, 8>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int r = rc + i < r_end ? rc + i : r_end - 1;  // masked rows: valid address
            const uint32_t* p = cbase + static_cast<size_t>(r) * row_words;
            const uint32_t a = p[w0], bw = p[w1];
            g[i][0] = __builtin_amdgcn_alignbit(bw, a, sh);
            g[i][1] = bw >> sh;
            sc[i] = scales[r];
        });
        bf16x8 afrag[MT];
        static_for<0, MT>([&](auto mc) {
            constexpr int mt = decltype(mc)::value;
            const uint16_t* xp = (mt == 0 ? xr0 : xr1) + rc;
            u32x4 a;
            if (rc + 8 <= r_end && ((reinterpret_cast<uintptr_t>(xp) & 15) == 0)) {
                a = *reinterpret_cast<const u32x4*>(xp);
            } else {
                static_for<0, 4>([&](auto dc) {
                    constexpr int d = decltype(dc)::value;
                    const uint32_t lo16 = rc + 2 * d < r_end ? xp[2 * d] : 0u;
                    const uint32_t hi16 = rc + 2 * d + 1 < r_end ? xp[2 * d + 1] : 0u;
                    a[d] = lo16 | (hi16 << 16);
                });
            }
            afrag[mt] = as_bf16x8(a);
        });
        static_for<0, 8>([&](auto ec) {
            // weight t0 + e starts (7 - e) * k bits above `lo`
            constexpr int e = decltype(ec)::value;
            constexpr int o = (7 - e) * K;
            u32x4 bq;
            static_for<0, 4>([&](auto dc) {
                constexpr int d = decltype(dc)::value;
                const float v0 = lds_lut(lut_s, lut_byte_offset<o>(g[2 * d]));
                const float v1 = lds_lut(lut_s, lut_byte_offset<o>(g[2 * d + 1]));
                bq[d] = pack2(v0 * sc[2 * d], v1 * sc[2 * d + 1]);
            });
            const bf16x8 bfrag = as_bf16x8(bq);
            static_for<0, MT>([&](auto mc) {
                constexpr int mt = decltype(mc)::value;
                acc[e][mt] = mfma16x16x32(afrag[mt], bfrag, acc[e][mt]);
            });
        });
    }

    // Sum the waves' tiles in wave order through LDS; the last wave stores.
    // D layout: lane holds D[m = 4c + v][n = j] of each 16x16 tile.
    for (int w = 0; w < kA0Waves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int m = mt * 16 + 4 * c + v;
                        const float prev = w == 0 ? 0.f : red[e][m][j];
                        const float sum = w == 0 ? acc[e][mt][v] : prev + acc[e][mt][v];
                        if (w < kA0Waves - 1) {
                            red[e][m][j] = sum;
                        } else if (m < M) {
                            partial[(static_cast<size_t>(sgroup) * M + m) * C + col0 + 8 * j + e] = sum;
                        }
                    }
        }
        __syncthreads();
    }
}

// y[i] = bf16( sum over split groups g ascending of partial[g][i] ), i < M*C.
// Four waves each sum a contiguous quarter of the groups; the quarters are
// then added in order.
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(
    const float* __restrict__ partial, uint16_t* __restrict__ y, int MC, int G) {
    __shared__ float red[4][64];
    const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = blockIdx.x * 64 + lane;
    const int per = (G + 3) / 4;
    const int g0 = q * per, g1 = min(G, g0 + per);
    float s = 0.f;
    if (i < MC) {
        int g = g0;
        for (; g + 8 <= g1; g += 8) {  // loads issued together, added in order
            float v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = partial[static_cast<size_t>(g + t) * MC + i];
#pragma unroll
            for (int t = 0; t < 8; ++t) s += v[t];
        }
        if (g + 4 <= g1) {
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = partial[static_cast<size_t>(g + t) * MC + i];
#pragma unroll
            for (int t = 0; t < 4; ++t) s += v[t];
            g += 4;
        }
        for (; g < g1; ++g) s += partial[static_cast<size_t>(g) * MC + i];
    }
    red[q][lane] = s;
    __syncthreads();
    if (q == 0 && i < MC) y[i] = round_bf16(((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]);
}

template <int K, int MT>
hipError_t launch_axis0_k(const uint16_t* x, int M, const uint32_t* codes, const float* scales,
                          const float* lut, float* partial, int R, int C, int S,
                          hipStream_t st) {
    const int rows_per_split = (R + S - 1) / S;
    const int groups = axis0_split_groups(S);
    const dim3 grid(static_cast<unsigned>((C / kTileCols) * groups));
    return launch_kernel(axis0_mma_kernel<K, MT>, grid, dim3(kA0Threads), st, x, codes, scales, lut,
                         partial, R, C, M, S, rows_per_split);
}

}  // namespace

int axis0_split_groups(int S) { return (S + kA0Waves - 1) / kA0Waves; }

hipError_t launch_axis0(const uint16_t* x, int M, const uint32_t* codes, const float* scales,
                        const float* lut, float* partial, uint16_t* y, int R, int C, int S, int k,
                        hipStream_t st) {
    const bool two = M > 16;
    hipError_t e;
    switch (k) {
    case 2: e = two ? launch_axis0_k<2, 2>(x, M, codes, scales, lut, partial, R, C, S, st)
                    : launch_axis0_k<2, 1>(x, M, codes, scales, lut, partial, R, C, S, st); break;
    case 3: e = two ? launch_axis0_k<3, 2>(x, M, codes, scales, lut, partial, R, C, S, st)
                    : launch_axis0_k<3, 1>(x, M, codes, scales, lut, partial, R, C, S, st); break;
    case 4: e = two ? launch_axis0_k<4, 2>(x, M, codes, scales, lut, partial, R, C, S, st)
                    : launch_axis0_k<4, 1>(x, M, codes, scales, lut, partial, R, C, S, st); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int MC = M * C;
    return launch_kernel(split_reduce_kernel, dim3((MC + 63) / 64), dim3(kThreads), st, partial, y,
                         MC, axis0_split_groups(S));
}

}  // namespace trellis
