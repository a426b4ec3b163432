// Axis-0 trellis kernels for gfx950: split-K decode + bf16 MFMA partials and
// the ordered reduction over the splits. They serve the M = 1 "scatter" GEMV
// and the axis-0 prefill.
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0,
// page 59: scatter.ts (axis-0 GEMV: the stored rows split into ranges, one
// float32 partial per range and output column, then a sum over the ranges and
// a cast) and splitk-prefill.ts (axis-0 prefill: split-K float32 partials and
// an ordered accumulate kernel).
//
// On axis 0 the contraction runs over stored rows r, and the MFMA B fragment
// of a lane holds 8 consecutive contraction indices of one output column. So
// a lane decodes an 8 x 8 patch: 8 stored rows x 8 adjacent columns. For each
// row it loads the two words that hold the 8 windows (always enough: at most
// 7k + 12 bits starting anywhere inside a word), funnels them to a 64-bit
// value, and reads the windows at compile-time offsets (for k = 2 as four
// adjacent-column pairs from the pair table). Column e of the patch over the 8
// rows is the B fragment of MFMA number e, whose accumulator collects output
// column 8j + e. The A fragment is x[m][the same 8 rows].
//
// Mapping: a workgroup of 8 waves owns one 128-column tile and one of P
// contiguous row ranges of it ("parts"; P = 256 / tiles, at least 1, a fixed
// count so that results do not depend on the device). Each wave takes a
// contiguous share of the part's 32-row steps (lane j = l % 16 -> columns
// 8j..8j+7, c = l / 16 -> rows 8c..8c+7 of a step) and accumulates in
// registers; the waves' tiles are summed in LDS in wave order, one partial per
// part, and the reduce kernel sums the parts in a fixed order. Every order is
// fixed, so repeated calls give identical bits.
//
// The decode table (the k = 2 pair table, or eight bank-partitioned copies of
// the codebook for k = 3, 4) is staged once per workgroup, and the next
// step's words, scales and activations are in flight in registers while one
// step is decoded (the first-generation kernel, one wave per split, four per
// workgroup, restaged the codebook in 1280 workgroups and waited on every
// step's loads).
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace trellis {

// Partials of the scatter variant that allocates nothing: one array per
// device, held until the process ends. Host code never passes this name to a
// kernel (on the host it is only a stand-in for the symbol); it uses the
// device address static_scratch() looked up for the current device.
__device__ __align__(256) float scratch[kStaticScratchFloats];

namespace {

constexpr int kThreads = 256;       // split reduce
constexpr int kTileCols = 128;
constexpr int kA0Threads = 512;     // 8 waves, two per SIMD
constexpr int kA0Waves = kA0Threads / kWave;
constexpr int kA0TargetGroups = 256;  // tiles x parts is about this
constexpr int kXcds = 8;              // accelerator dies, each with its own L2

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    floatx2 p = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}

// Decode table: the k = 2 pair table, or for k = 3, 4 the bank-partitioned
// codebook copies (both 128 KB).
template <int K>
struct A0Lds {
    static constexpr bool pair = K == 2;
    static constexpr bool rep = !pair;
    using Table = DecodeTable<kA0Threads, pair, rep>;
    static constexpr int tab_floats = Table::floats;
    static constexpr int red_floats = kA0Waves * 16 * kTileCols;  // one M tile of wave partials
    static constexpr int floats = tab_floats > red_floats ? tab_floats : red_floats;
};

// One 32-row step of a lane: the raw words w0, w1 of its 8 rows (the funnel
// shift waits until decode, so the loads can be in flight meanwhile), the
// rows' scales, and its A fragment per M tile.
template <int MT>
struct A0Step {
    uint32_t a[8], b[8];
    float sc[8];
    u32x4 x[MT];
    int rc;  // first row of the lane's 8-row chunk
};

struct A0Ctx {
    const uint32_t* cbase;  // word 0 of the tile's block in stored row 0
    const float* scales;
    const uint16_t* xr[2];  // A rows m = j and 16 + j (rows past M read row 0)
    size_t row_words;
    int w0, w1, R, c;
    // Buffer-addressed loads (BUF): raw buffer resources over the tile's
    // codes and the scales, and 32-bit byte offsets into them.
    __amdgpu_buffer_rsrc_t rcodes, rscales;
    uint32_t row_bytes;     // stored-row stride of the codes
    uint32_t wb0, wb1;      // byte offsets of words w0, w1 within a row
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
    // dword 3 of a raw (untyped, unswizzled) buffer resource on this family
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             0x00020000);
}

// Issue step s's loads; every address is valid whatever s is (rows clamp to
// the last stored row), so the loads are unconditional. With VEC (R % 8 == 0,
// scales 16-byte aligned) a lane's 8 rows are all stored rows or all past the
// end: its A fragment is one aligned 16-byte load and, with VSC, its 8 scales
// two (VSC is off for two M tiles, where the kernels then spill registers);
// otherwise x is read element by element with the row count applied.
//
// With BUF (VEC, and every byte offset below 2^31) the same loads go through
// raw buffer resources: one 32-bit lane offset per step, the row stride as
// the uniform scalar offset, so no 64-bit address arithmetic per row (the
// scales always as eight 4-byte loads, which the compiler merges; x as in VEC).
template <int MT, bool VEC, bool VSC, bool BUF>
__device__ __forceinline__ void a0_load(A0Step<MT>& st, const A0Ctx& cx, int s) {
    const int rc = 32 * s + 8 * cx.c;
    st.rc = rc;
    if constexpr (BUF) {
        static_assert(VEC, "buffer loads take whole 8-row chunks");
        const uint32_t rcc = static_cast<uint32_t>(rc < cx.R ? rc : cx.R - 8);
        const uint32_t vo = rcc * cx.row_bytes;
        static_for<0, 8>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int so = static_cast<int>(i * cx.row_bytes);
            st.a[i] = __builtin_amdgcn_raw_buffer_load_b32(cx.rcodes, static_cast<int>(vo + cx.wb0), so, 0);
            st.b[i] = __builtin_amdgcn_raw_buffer_load_b32(cx.rcodes, static_cast<int>(vo + cx.wb1), so, 0);
        });
        // 4-byte loads only (adjacent ones are merged into wide loads); this
        // compiler lowers the 16-byte raw buffer load builtin to one dword.
        static_for<0, 8>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            st.sc[i] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(cx.rscales, static_cast<int>(4 * rcc + 4 * i), 0, 0));
        });
        static_for<0, MT>([&](auto mc) {  // one 16-byte global load
            constexpr int mt = decltype(mc)::value;
            st.x[mt] = *reinterpret_cast<const u32x4*>(cx.xr[mt] + rcc);
        });
        return;
    }
    static_for<0, 8>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int r = rc + i < cx.R ? rc + i : cx.R - 1;
        const uint32_t* p = cx.cbase + static_cast<size_t>(r) * cx.row_words;
        st.a[i] = p[cx.w0];
        st.b[i] = p[cx.w1];
        if constexpr (!VSC) st.sc[i] = cx.scales[r];
    });
    if constexpr (VSC) {
        static_assert(VEC, "vector scales need whole 8-row chunks");
        const int rs = rc < cx.R ? rc : cx.R - 8;
        const floatx4 lo = *reinterpret_cast<const floatx4*>(cx.scales + rs);
        const floatx4 hi = *reinterpret_cast<const floatx4*>(cx.scales + rs + 4);
        st.sc[0] = lo.x; st.sc[1] = lo.y; st.sc[2] = lo.z; st.sc[3] = lo.w;
        st.sc[4] = hi.x; st.sc[5] = hi.y; st.sc[6] = hi.z; st.sc[7] = hi.w;
    }
    static_for<0, MT>([&](auto mc) {
        constexpr int mt = decltype(mc)::value;
        if constexpr (VEC) {
            const int rx = rc < cx.R ? rc : cx.R - 8;
            st.x[mt] = *reinterpret_cast<const u32x4*>(cx.xr[mt] + rx);
        } else {
            const uint16_t* xp = cx.xr[mt] + rc;
            static_for<0, 4>([&](auto dc) {
                constexpr int d = decltype(dc)::value;
                const uint32_t lo16 = rc + 2 * d < cx.R ? xp[2 * d] : 0u;
                const uint32_t hi16 = rc + 2 * d + 1 < cx.R ? xp[2 * d + 1] : 0u;
                st.x[mt][d] = lo16 | (hi16 << 16);
            });
        }
    });
}

// Decode a step's 8 x 8 patch and multiply, column by column (k = 3, 4; the
// next two columns' gathers in flight while one is packed and multiplied) or
// column pair by column pair (k = 2, the next pair's gathers in flight).
template <int K, int MT, bool VEC>
__device__ __forceinline__ void a0_decode(const A0Step<MT>& st, const A0Ctx& cx, int sh,
                                          const float* __restrict__ tab, uint32_t cofs,
                                          floatx4 (&acc)[8][MT]) {
    uint32_t g[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        g[i][0] = __builtin_amdgcn_alignbit(st.b[i], st.a[i], sh);
        g[i][1] = st.b[i] >> sh;
    }
    bf16x8 afrag[MT];
    const bool live = !VEC || st.rc < cx.R;  // VEC: a chunk past the end contributes nothing
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        afrag[mt] = as_bf16x8(live ? st.x[mt] : u32x4{0u, 0u, 0u, 0u});
    if constexpr (A0Lds<K>::pair) {
        // columns 2p (earlier weight) and 2p + 1: the pair field starts at the
        // later weight, (6 - 2p) k bits above the lane's lowest window
        auto gather = [&](auto pc, floatx2 (&v)[8]) {
            constexpr int O = (6 - 2 * decltype(pc)::value) * K;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = lds_pair(tab, field_offset<O, 14, 3>(g[i]));
        };
        floatx2 va[8], vb[8];
        gather(std::integral_constant<int, 0>{}, va);
        static_for<0, 4>([&](auto pc) {
            constexpr int p = decltype(pc)::value;
            floatx2 (&cur)[8] = (p & 1) ? vb : va;
            floatx2 (&nxt)[8] = (p & 1) ? va : vb;
            __builtin_amdgcn_s_setprio(2);
            if constexpr (p + 1 < 4) gather(std::integral_constant<int, p + 1>{}, nxt);
            __builtin_amdgcn_s_setprio(0);
            u32x4 b0, b1;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                b0[d] = pack2(cur[2 * d].x * st.sc[2 * d], cur[2 * d + 1].x * st.sc[2 * d + 1]);
                b1[d] = pack2(cur[2 * d].y * st.sc[2 * d], cur[2 * d + 1].y * st.sc[2 * d + 1]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[2 * p][mt] = mfma16x16x32(afrag[mt], as_bf16x8(b0), acc[2 * p][mt]);
                acc[2 * p + 1][mt] = mfma16x16x32(afrag[mt], as_bf16x8(b1), acc[2 * p + 1][mt]);
            }
        });
    } else {
        // weight t0 + e starts (7 - e) k bits above the lane's lowest window;
        // the lane reads its own codebook copy (byte offset cofs)
        auto gather = [&](auto ec, float (&v)[8]) {
            constexpr int o = (7 - decltype(ec)::value) * K;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = lds_lut(tab, field_offset<o, kL, 5>(g[i]) | cofs);
        };
        float v3[3][8];
        gather(std::integral_constant<int, 0>{}, v3[0]);
        gather(std::integral_constant<int, 1>{}, v3[1]);
        static_for<0, 8>([&](auto ec) {
            constexpr int e = decltype(ec)::value;
            float (&cur)[8] = v3[e % 3];
            __builtin_amdgcn_s_setprio(2);  // the gathers issue at raised priority
            if constexpr (e + 2 < 8) gather(std::integral_constant<int, e + 2>{}, v3[(e + 2) % 3]);
            __builtin_amdgcn_s_setprio(0);
            u32x4 bq;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                bq[d] = pack2(cur[2 * d] * st.sc[2 * d], cur[2 * d + 1] * st.sc[2 * d + 1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[e][mt] = mfma16x16x32(afrag[mt], as_bf16x8(bq), acc[e][mt]);
        });
    }
}

template <int K, int MT, bool VEC, bool BUF>
__global__ __launch_bounds__(kA0Threads) void axis0_mma_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
    const float* __restrict__ scales, const float* __restrict__ lut,
    float* __restrict__ partial, CodeLayout lay, int R, int C, int M, int P) {
    constexpr int wpb = Bits<K>::wpb;
    __shared__ __attribute__((aligned(16))) float lds[A0Lds<K>::floats];
    float* const tab = lds;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, c = lane >> 4;
    // Workgroup b runs on XCD b % 8 (round-robin dispatch). The (part, tile)
    // pairs are numbered part-major and each XCD takes a contiguous range of
    // them, so that neighbouring tiles of a part, whose code rows share cache
    // lines (a k = 3 tile reads 48 bytes of each row), meet in one L2.
    const int G = static_cast<int>(gridDim.x), tiles = G / P;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int L = xcd * (G / kXcds) + min(xcd, G % kXcds) + slot;
    const int part = L / tiles;
    const int tile = L - part * tiles;
    const int col0 = tile * kTileCols;
    const int blk = col0 / kT;
    const int t0 = (col0 % kT) + 8 * j;         // first weight of this lane's 8 columns
    const int lo = (kT - 8 - t0) * K;           // bit of weight t0 + 7
    const int w0 = lo >> 5, sh = lo & 31;
    const int w1 = (w0 + 1 == wpb) ? 0 : w0 + 1;  // tail-biting wrap to word 0

    // This part's 32-row steps, and this wave's contiguous share of them.
    const int RS = (R + 31) / 32;
    const int p0 = static_cast<int>(static_cast<long>(part) * RS / P);
    const int p1 = static_cast<int>(static_cast<long>(part + 1) * RS / P);
    const int s0 = p0 + wave * (p1 - p0) / kA0Waves;
    const int s1 = p0 + (wave + 1) * (p1 - p0) / kA0Waves;

    A0Ctx cx;
    cx.cbase = codes + block_word<K>(lay, 0, blk);
    cx.scales = scales;
    cx.xr[0] = x + static_cast<size_t>(j < M ? j : 0) * R;
    cx.xr[1] = x + static_cast<size_t>(16 + j < M ? 16 + j : 0) * R;
    cx.row_words = lay.row_words;
    cx.w0 = w0;
    cx.w1 = w1;
    cx.R = R;
    cx.c = c;
    if constexpr (BUF) {
        // the launcher checked that R rows of codes span less than 2^31 bytes
        cx.row_bytes = static_cast<uint32_t>(lay.row_words * 4);
        cx.rcodes = raw_rsrc(cx.cbase, static_cast<uint32_t>(R) * cx.row_bytes);
        cx.rscales = raw_rsrc(scales, 4u * static_cast<uint32_t>(R));
        cx.wb0 = 4u * static_cast<uint32_t>(w0);
        cx.wb1 = 4u * static_cast<uint32_t>(w1);
    }

    floatx4 acc[8][MT];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[e][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // The table sources first, then the first step's loads (unconditional; a
    // wave without steps reads a valid clamped step), so the table stores do
    // not wait for them.
    typename A0Lds<K>::Table::Src tsrc;
    A0Lds<K>::Table::fetch(tsrc, lut);
    asm volatile("" ::: "memory");
    A0Step<MT> sa, sb;
    constexpr bool kVsc = VEC && MT == 1;
    a0_load<MT, VEC, kVsc, BUF>(sa, cx, s0);
    A0Lds<K>::Table::store(tsrc, tab);
    __syncthreads();

    // Two register sets alternate: the next step's loads are in flight while
    // one is decoded. Inside the loop every load feeds an unconditional decode
    // (a load used only under a branch gets sunk into it, behind the waits);
    // an odd last step is decoded after the loop.
    const uint32_t cofs = rep_lane_offset();  // the lane's codebook copy (k = 3, 4)
    int s = s0;
    for (; s + 1 < s1; s += 2) {
        a0_load<MT, VEC, kVsc, BUF>(sb, cx, s + 1);
        a0_decode<K, MT, VEC>(sa, cx, sh, tab, cofs, acc);
        a0_load<MT, VEC, kVsc, BUF>(sa, cx, s + 2);
        a0_decode<K, MT, VEC>(sb, cx, sh, tab, cofs, acc);
    }
    if (s < s1) a0_decode<K, MT, VEC>(sa, cx, sh, tab, cofs, acc);
    __syncthreads();  // the table is dead from here on; its space takes the wave partials

    // Sum the waves' tiles in wave order, one M tile at a time.
    // D layout: lane holds D[m = 4c + v][n = j] of the tile of column 8j + e.
    float* const red = lds;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[(wave * 16 + 4 * c + v) * kTileCols + 8 * j + e] = acc[e][mt][v];
        __syncthreads();
        for (int idx = tid; idx < 16 * kTileCols; idx += kA0Threads) {
            const int m = idx / kTileCols, col = idx % kTileCols;
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < kA0Waves; ++w) sum += red[(w * 16 + m) * kTileCols + col];
            const int mm = 16 * mt + m;
            if (mm < M) partial[(static_cast<size_t>(part) * M + mm) * C + col0 + col] = sum;
        }
        __syncthreads();
    }
}

// y[i] = bf16( sum over parts g ascending of partial[g][i] ), i < M*C.
// Four waves each sum a contiguous quarter of the parts; the quarters are
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

template <int K, int MT, bool VEC, bool BUF>
hipError_t launch_axis0_k(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                          const float* scales, const float* lut, float* partial, int R, int C, int P,
                          hipStream_t st) {
    const dim3 grid(static_cast<unsigned>((C / kTileCols) * P));
    return launch_kernel(axis0_mma_kernel<K, MT, VEC, BUF>, grid, dim3(kA0Threads), st, x, codes,
                         scales, lut, partial, lay, R, C, M, P);
}

template <int K, int MT>
hipError_t launch_axis0_v(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                          const float* scales, const float* lut, float* partial, int R, int C, int P,
                          hipStream_t st) {
    if (R % 8 == 0 && reinterpret_cast<uintptr_t>(scales) % 16 == 0) {
        // buffer loads when every byte offset they form fits in 31 bits
        const uint64_t lim = 1ull << 31;
        if (static_cast<uint64_t>(R) * lay.row_words * 4 < lim)
            return launch_axis0_k<K, MT, true, true>(x, M, codes, lay, scales, lut, partial, R, C, P, st);
        return launch_axis0_k<K, MT, true, false>(x, M, codes, lay, scales, lut, partial, R, C, P, st);
    }
    return launch_axis0_k<K, MT, false, false>(x, M, codes, lay, scales, lut, partial, R, C, P, st);
}

}  // namespace

hipError_t static_scratch(float** ptr) {
    static std::mutex mu;
    static float* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = static_cast<float*>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

int axis0_parts(int R, int C) {
    const int tiles = C / kTileCols, steps = (R + 31) / 32;
    int P = kA0TargetGroups / tiles;
    if (P > steps) P = steps;
    return P > 1 ? P : 1;
}

hipError_t launch_axis0(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                        const float* scales, const float* lut, float* partial, uint16_t* y, int R,
                        int C, int k, hipStream_t st) {
    const bool two = M > 16;
    const int P = axis0_parts(R, C);
    hipError_t e;
    switch (k) {
    case 2: e = two ? launch_axis0_v<2, 2>(x, M, codes, lay, scales, lut, partial, R, C, P, st)
                    : launch_axis0_v<2, 1>(x, M, codes, lay, scales, lut, partial, R, C, P, st); break;
    case 3: e = two ? launch_axis0_v<3, 2>(x, M, codes, lay, scales, lut, partial, R, C, P, st)
                    : launch_axis0_v<3, 1>(x, M, codes, lay, scales, lut, partial, R, C, P, st); break;
    case 4: e = two ? launch_axis0_v<4, 2>(x, M, codes, lay, scales, lut, partial, R, C, P, st)
                    : launch_axis0_v<4, 1>(x, M, codes, lay, scales, lut, partial, R, C, P, st); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int MC = M * C;
    return launch_kernel(split_reduce_kernel, dim3((MC + 63) / 64), dim3(kThreads), st, partial, y,
                         MC, P);
}

}  // namespace trellis
