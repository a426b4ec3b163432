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
// Mapping: the 32-row steps of every 128-column tile are cut into the same nr
// contiguous ranges, one per wave (a lane j = l % 16 takes columns 8j..8j+7,
// c = l / 16 rows 8c..8c+7 of a step), and the wave accumulates its range in
// registers. Waves are numbered band-major: band b holds ranges nv b .. nv b +
// nv - 1 of tile 0, then of tile 1, and so on, and workgroup L takes waves nv
// L .. nv L + nv - 1. Usually nr = 8 P with P = 256 / tiles bands (at most the
// step count) and nv = 8, so a workgroup owns one band of one tile. Where that
// leaves a quarter or more of the compute units idle (e.g. 136 tiles: 136
// workgroups), nr = 2048 / tiles (256 compute units x 8 waves), nv = 8 (fewer
// when there are fewer than 2048 ranges), and the last band's nr mod nv ranges
// of several tiles share workgroups, a tile's spanning at most two. The plan
// depends on R and C only, not on the device. All tiles have the same ranges,
// so neighbouring tiles, whose code rows share cache lines, read the same rows
// at the same time. A workgroup sums its waves' tiles in LDS in wave order, one
// partial per run of waves on one tile, and the reduce kernel sums a tile's
// partials in range order; at M <= 8 with whole bands the partial kernel does
// that sum itself (FUSED: the bands meet as call-tagged words in the
// workspace). Every order is fixed, so repeated calls give identical bits.
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

// The wave plan: nr ranges per tile, nv waves used per workgroup, nf = nr / nv
// whole bands first (nf nv tiles waves), then the partial band of rr = nr -
// nf nv waves per tile. Partial slots: one per whole-band workgroup
// (band-major), then tw per tile for its partial-band run: with rr > 1 a run
// can be cut by a workgroup end, and its second piece takes the tile's
// second slot (a run that is not cut writes zeros there).
struct A0Bands {
    int nr, nv, nf, tiles;
    int rr, full, tw;
    __host__ __device__ A0Bands(int nr_, int nv_, int nf_, int tiles_)
        : nr(nr_), nv(nv_), nf(nf_), tiles(tiles_) {
        rr = nr - nf * nv;
        full = nf * nv * tiles;
        tw = rr > 1 ? 2 : 1;
    }
    __host__ __device__ int slots() const { return nf * tiles + (rr ? tw * tiles : 0); }
    __host__ __device__ int band_slot(int kb, int t) const { return kb * tiles + t; }
    __host__ __device__ int tail_slot(int t) const { return nf * tiles + tw * t; }
};

constexpr int kFusedMaxBands = 8;  // bands per tile of the fused sum, at most

// TAIL: the plan has a partial band (nr % nv != 0); without it every
// workgroup is a whole band's.
template <int K, int MT, bool VEC, bool BUF, bool TAIL, bool FUSED>
__global__ __launch_bounds__(kA0Threads) void axis0_mma_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
    const float* __restrict__ scales, const float* __restrict__ lut,
    float* __restrict__ partial, CodeLayout lay, int R, int C, int M, int nr, int nv, int nf,
    uint16_t* __restrict__ y, unsigned int tag) {
    static_assert(!FUSED || !TAIL, "the fused sum serves whole-band plans");
    constexpr int wpb = Bits<K>::wpb;
    __shared__ __attribute__((aligned(16))) float lds[A0Lds<K>::floats];
    float* const tab = lds;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, c = lane >> 4;
    // Workgroup b runs on XCD b % 8 (round-robin dispatch), and each XCD
    // takes a contiguous range of the workgroups: a band's neighbouring tiles,
    // whose code rows share cache lines (a k = 3 tile reads 48 bytes of each
    // row), meet in one L2.
    const int G = static_cast<int>(gridDim.x), tiles = C / kTileCols, RS = (R + 31) / 32;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int L = xcd * (G / kXcds) + min(xcd, G % kXcds) + slot;
    const A0Bands bd(nr, nv, nf, tiles);
    const int gw = L * nv + wave;                          // this wave's number
    const bool live = wave < nv && gw < nr * tiles;
    const bool band = !TAIL || L * nv < bd.full;           // a whole-band workgroup
    const int kb = L / tiles;                              // its band
    int tile = 0, k = 0;                                   // this wave's tile and range
    if (live) {
        if (band) {
            tile = L - kb * tiles;
            k = kb * nv + wave;
        } else {
            const int rem = gw - bd.full;
            tile = rem / bd.rr;
            k = nf * nv + (rem - tile * bd.rr);
        }
    }
    const int col0 = tile * kTileCols;
    const int blk = col0 / kT;
    const int t0 = (col0 % kT) + 8 * j;         // first weight of this lane's 8 columns
    const int lo = (kT - 8 - t0) * K;           // bit of weight t0 + 7
    const int w0 = lo >> 5, sh = lo & 31;
    const int w1 = (w0 + 1 == wpb) ? 0 : w0 + 1;  // tail-biting wrap to word 0

    // This wave's 32-row steps (none for a wave past the last range; nr x RS
    // fits in 31 bits: nr <= 2048, RS <= 2^14).
    const int s0 = k * RS / nr;
    const int s1 = live ? (k + 1) * RS / nr : s0;

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

    // Sum the waves' tiles in wave order, one M tile at a time: all of them
    // into one partial in a whole-band workgroup, else one partial per run of
    // waves on one tile (waves past the last range hold zeros and end no run,
    // so adding them changes nothing). The slot each wave's run of a tile
    // ends in (-1: its run goes on) is uniform and fixed before the sums, and
    // each sum's LDS reads are all issued before its first add.
    int end_slot[kA0Waves] = {-1, -1, -1, -1, -1, -1, -1, -1};
    int zero_slot[kA0Waves] = {-1, -1, -1, -1, -1, -1, -1, -1};
    const int bslot = bd.band_slot(kb, L - kb * tiles);  // a whole-band workgroup's slot
    if (!band) {
        const int nlive = min(nv, nr * tiles - L * nv);
        const int rem = L * nv - bd.full;
        int t = rem / bd.rr, in = rem - t * bd.rr;  // the first wave's tile and place in its run
        bool second = in > 0;                       // the run began in the previous workgroup
#pragma unroll
        for (int w = 0; w < kA0Waves; ++w) {
            if (w < nlive) {
                const bool whole = in + 1 == bd.rr;  // the tile's last wave
                if (whole || w + 1 == nlive) {
                    end_slot[w] = bd.tail_slot(t) + (second ? 1 : 0);
                    if (whole && !second && bd.tw == 2) zero_slot[w] = bd.tail_slot(t) + 1;
                    ++t;
                    in = 0;
                    second = false;
                } else {
                    ++in;
                }
            }
        }
    }
    const size_t mstride = static_cast<size_t>(M) * kTileCols;
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
            const int mm = 16 * mt + m;
            float* const dst = partial + static_cast<size_t>(mm) * kTileCols + col;
            float pv[kA0Waves];  // all reads issued before the first add
#pragma unroll
            for (int w = 0; w < kA0Waves; ++w) pv[w] = red[(w * 16 + m) * kTileCols + col];
            float sum = 0.f;
            if (band) {
#pragma unroll
                for (int w = 0; w < kA0Waves; ++w) sum += pv[w];
                if constexpr (FUSED) {
                    if (mm < M)
                        __hip_atomic_store(reinterpret_cast<unsigned long long*>(partial) +
                                               static_cast<size_t>(bslot) * mstride +
                                               static_cast<size_t>(mm) * kTileCols + col,
                                           tagged_word(slot_tag(tag, bslot), sum),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    if (mm < M) dst[static_cast<size_t>(bslot) * mstride] = sum;
                }
            } else {
#pragma unroll
                for (int w = 0; w < kA0Waves; ++w) {
                    sum += pv[w];
                    if (end_slot[w] >= 0) {
                        if (mm < M) {
                            dst[static_cast<size_t>(end_slot[w]) * mstride] = sum;
                            if (zero_slot[w] >= 0) dst[static_cast<size_t>(zero_slot[w]) * mstride] = 0.f;
                        }
                        sum = 0.f;
                    }
                }
            }
        }
        __syncthreads();
    }
    if constexpr (FUSED) {
        // Every band's partial of this tile, as tagged words: where all carry
        // this call's tag, sum them in band order. The workgroup that checks
        // last sees every band's store (each completed before its writer's
        // own check), so every output is written at least once; workgroups
        // that find all current at once write the same bits. A wave sums only
        // when all its outputs are current (the writers are the same for all
        // of a tile's outputs), so a stale word could pass only if a whole
        // wave's words matched this call's tags.
        __builtin_amdgcn_s_waitcnt(0);
        const unsigned long long* const pw = reinterpret_cast<const unsigned long long*>(partial);
        const int t = L - kb * tiles;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int it = 0; it < 16 * kTileCols / kA0Threads; ++it) {
                const int idx = tid + it * kA0Threads;
                const int m = idx / kTileCols, col = idx % kTileCols;  // m uniform in a wave
                const int mm = 16 * mt + m;
                if (mm >= M) continue;
                unsigned long long wv[kFusedMaxBands];
#pragma unroll
                for (int b = 0; b < kFusedMaxBands; ++b)
                    wv[b] = __hip_atomic_load(pw + static_cast<size_t>(bd.band_slot(b < nf ? b : kb, t)) * mstride +
                                                  static_cast<size_t>(mm) * kTileCols + col,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                bool stale = false;
#pragma unroll
                for (int b = 0; b < kFusedMaxBands; ++b)
                    stale |= b < nf && static_cast<unsigned int>(wv[b] >> 32) != slot_tag(tag, bd.band_slot(b, t));
                if (__builtin_amdgcn_ballot_w64(stale) != 0) continue;  // a later workgroup sums
                float sum = 0.f;
#pragma unroll
                for (int b = 0; b < kFusedMaxBands; ++b)
                    if (b < nf) sum += __uint_as_float(static_cast<unsigned int>(wv[b]));
                y[static_cast<size_t>(mm) * C + t * kTileCols + col] = round_bf16(sum);
            }
    }
}

// y[m][col] = bf16( the partials of col's tile t summed in range order: the
// whole bands' slots b tiles + t, b ascending, then the tile's partial-band
// slots ). A block takes 64 outputs of one row m and one tile; four waves
// each sum a contiguous quarter of the bands (the last also the partial
// band), then the quarters are added in order.
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(
    const float* __restrict__ partial, uint16_t* __restrict__ y, int M, int C, int nr, int nv,
    int nf) {
    __shared__ float red[4][64];
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int i0 = blockIdx.x * 64;
    const int m = i0 / C, col0 = i0 - m * C;
    const int tiles = C / kTileCols, t = col0 / kTileCols;
    const A0Bands bd(nr, nv, nf, tiles);
    const size_t mstride = static_cast<size_t>(M) * kTileCols;
    const float* const src = partial + static_cast<size_t>(m) * kTileCols + col0 % kTileCols + lane;
    const int per = (bd.nf + 3) / 4;
    const int b0 = q * per, b1 = min(bd.nf, b0 + per);
    float s = 0.f;
    int b = b0;
    for (; b + 4 <= b1; b += 4) {  // loads issued together, added in order
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = src[static_cast<size_t>(bd.band_slot(b + u, t)) * mstride];
#pragma unroll
        for (int u = 0; u < 4; ++u) s += v[u];
    }
    for (; b < b1; ++b) s += src[static_cast<size_t>(bd.band_slot(b, t)) * mstride];
    if (q == 3 && bd.rr) {
        s += src[static_cast<size_t>(bd.tail_slot(t)) * mstride];
        if (bd.tw == 2) s += src[static_cast<size_t>(bd.tail_slot(t) + 1) * mstride];
    }
    red[q][lane] = s;
    __syncthreads();
    if (q == 0) y[i0 + lane] = round_bf16(((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane]);
}

// The same sum with one wave per 64 outputs, for plans of at most
// kReduceOneWave partials per tile: the loads issued together, then added in
// range order, with no LDS round and no barrier.
constexpr int kReduceOneWave = 16;
__global__ __launch_bounds__(kWave) void split_reduce_wave_kernel(
    const float* __restrict__ partial, uint16_t* __restrict__ y, int M, int C, int nr, int nv,
    int nf) {
    const int lane = threadIdx.x;
    const int i0 = blockIdx.x * 64;
    const int m = i0 / C, col0 = i0 - m * C;
    const int tiles = C / kTileCols, t = col0 / kTileCols;
    const A0Bands bd(nr, nv, nf, tiles);
    const size_t mstride = static_cast<size_t>(M) * kTileCols;
    const float* const src = partial + static_cast<size_t>(m) * kTileCols + col0 % kTileCols + lane;
    const int n = bd.nf + (bd.rr ? bd.tw : 0);  // <= kReduceOneWave
    float v[kReduceOneWave];
#pragma unroll
    for (int u = 0; u < kReduceOneWave; ++u) {
        const int sl = u < bd.nf ? bd.band_slot(u, t) : bd.tail_slot(t) + (u - bd.nf);
        v[u] = u < n ? src[static_cast<size_t>(sl) * mstride] : 0.f;
    }
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < kReduceOneWave; ++u)
        if (u < n) s += v[u];
    y[i0 + lane] = round_bf16(s);
}

// The same sum with four adjacent outputs per lane (16-byte partial loads,
// 8-byte stores): one wave per 256 outputs of one activation row, i.e. two
// column tiles, C a multiple of 256.
__global__ __launch_bounds__(kWave) void split_reduce_wave4_kernel(
    const float* __restrict__ partial, uint16_t* __restrict__ y, int M, int C, int nr, int nv,
    int nf) {
    const int lane = threadIdx.x;
    const int i0 = blockIdx.x * 256;
    const int m = i0 / C, col = i0 - m * C + 4 * lane;
    const int tiles = C / kTileCols, t = col / kTileCols;
    const A0Bands bd(nr, nv, nf, tiles);
    const size_t mstride = static_cast<size_t>(M) * kTileCols;
    const float* const src = partial + static_cast<size_t>(m) * kTileCols + col % kTileCols;
    const int n = bd.nf + (bd.rr ? bd.tw : 0);  // <= kReduceOneWave
    floatx4 v[kReduceOneWave];
#pragma unroll
    for (int u = 0; u < kReduceOneWave; ++u) {
        const int sl = u < bd.nf ? bd.band_slot(u, t) : bd.tail_slot(t) + (u - bd.nf);
        v[u] = u < n ? *reinterpret_cast<const floatx4*>(src + static_cast<size_t>(sl) * mstride)
                     : floatx4{0.f, 0.f, 0.f, 0.f};
    }
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kReduceOneWave; ++u)
        if (u < n) s += v[u];
    const uint32_t lo = round_bf16(s[0]) | (static_cast<uint32_t>(round_bf16(s[1])) << 16);
    const uint32_t hi = round_bf16(s[2]) | (static_cast<uint32_t>(round_bf16(s[3])) << 16);
    *reinterpret_cast<uint2*>(y + i0 + 4 * lane) = make_uint2(lo, hi);
}

template <int K, int MT, bool VEC, bool BUF>
hipError_t launch_axis0_k(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                          const float* scales, const float* lut, float* partial, int R, int C,
                          A0Plan pl, uint16_t* y, unsigned int tag, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(pl.G)), block(kA0Threads);
    const int nf = pl.ranges / pl.waves;
    if (pl.ranges % pl.waves)
        return launch_kernel(axis0_mma_kernel<K, MT, VEC, BUF, true, false>, grid, block, st, x, codes,
                             scales, lut, partial, lay, R, C, M, pl.ranges, pl.waves, nf, y, 0u);
    if (tag)
        return launch_kernel(axis0_mma_kernel<K, MT, VEC, BUF, false, true>, grid, block, st, x, codes,
                             scales, lut, partial, lay, R, C, M, pl.ranges, pl.waves, nf, y, tag);
    return launch_kernel(axis0_mma_kernel<K, MT, VEC, BUF, false, false>, grid, block, st, x, codes, scales,
                         lut, partial, lay, R, C, M, pl.ranges, pl.waves, nf, y, 0u);
}

template <int K, int MT>
hipError_t launch_axis0_v(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                          const float* scales, const float* lut, float* partial, int R, int C,
                          A0Plan pl, uint16_t* y, unsigned int tag, hipStream_t st) {
    if (R % 8 == 0 && reinterpret_cast<uintptr_t>(scales) % 16 == 0) {
        // buffer loads when every byte offset they form fits in 31 bits
        const uint64_t lim = 1ull << 31;
        if (static_cast<uint64_t>(R) * lay.row_words * 4 < lim)
            return launch_axis0_k<K, MT, true, true>(x, M, codes, lay, scales, lut, partial, R, C, pl, y, tag, st);
        return launch_axis0_k<K, MT, true, false>(x, M, codes, lay, scales, lut, partial, R, C, pl, y, tag, st);
    }
    return launch_axis0_k<K, MT, false, false>(x, M, codes, lay, scales, lut, partial, R, C, pl, y, tag, st);
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

A0Plan axis0_plan(int R, int C) {
    const int tiles = C / kTileCols, RS = (R + 31) / 32;
    // Whole bands only: P = 256 / tiles bands (at most the step count) of 8
    // ranges per tile (some empty when a band has fewer than 8 steps), one
    // workgroup per (band, tile).
    int P = kA0TargetGroups / tiles;
    if (P > RS) P = RS;
    if (P < 1) P = 1;
    const int groups = P * tiles;
    const int rounds = (groups + kA0TargetGroups - 1) / kA0TargetGroups;
    if (4 * groups >= 3 * rounds * kA0TargetGroups)  // fills at least 3/4 of its rounds
        return A0Plan{groups, kA0Waves * P, kA0Waves};
    // Otherwise the finer plan: 2048 / tiles ranges per tile (the chip's 256
    // compute units x 8 waves), at most the step count, with a partial band.
    int nr = kA0Waves * kA0TargetGroups / tiles;
    if (nr > RS) nr = RS;
    if (nr < 1) nr = 1;
    const int waves = nr * tiles;  // at most max(2048, tiles)
    int v = (waves + kA0TargetGroups - 1) / kA0TargetGroups;
    if (v > kA0Waves) v = kA0Waves;
    return A0Plan{(waves + v - 1) / v, nr, v};
}

// Whether the partial kernel sums its partials itself (M <= 8; whole bands
// only, at most kFusedMaxBands per tile, and at most half the static array's
// partials, so that the scatter's 8-byte tagged words still fit there). The
// plan depends on R, C and M only.
bool axis0_fused(int R, int C, int M) {
    // measured at 17408 x 5120: M = 2 / 4 / 8 1.2 / 1.3 / 0.5 us faster than
    // the reduce launch, M = 16 0.8 us and M = 32 3 us slower
    if (M > 8) return false;
    const A0Plan pl = axis0_plan(R, C);
    const A0Bands bd(pl.ranges, pl.waves, pl.ranges / pl.waves, C / kTileCols);
    return pl.ranges % pl.waves == 0 && pl.ranges / pl.waves <= kFusedMaxBands &&
           static_cast<size_t>(bd.slots()) * kTileCols * 2 <= kStaticScratchFloats;
}

size_t axis0_partial_floats(int R, int C, int M) {
    const A0Plan pl = axis0_plan(R, C);
    const A0Bands bd(pl.ranges, pl.waves, pl.ranges / pl.waves, C / kTileCols);
    const size_t n = static_cast<size_t>(bd.slots()) * static_cast<size_t>(M) * kTileCols;
    return axis0_fused(R, C, M) ? 2 * n : n;
}

hipError_t launch_axis0(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                        const float* scales, const float* lut, float* partial, uint16_t* y, int R,
                        int C, int k, hipStream_t st) {
    const bool two = M > 16;
    const A0Plan pl = axis0_plan(R, C);
    const unsigned int tag = axis0_fused(R, C, M) && !stream_capturing(st) ? next_call_tag() : 0u;
    hipError_t e;
    switch (k) {
    case 2: e = two ? launch_axis0_v<2, 2>(x, M, codes, lay, scales, lut, partial, R, C, pl, y, tag, st)
                    : launch_axis0_v<2, 1>(x, M, codes, lay, scales, lut, partial, R, C, pl, y, tag, st); break;
    case 3: e = two ? launch_axis0_v<3, 2>(x, M, codes, lay, scales, lut, partial, R, C, pl, y, tag, st)
                    : launch_axis0_v<3, 1>(x, M, codes, lay, scales, lut, partial, R, C, pl, y, tag, st); break;
    case 4: e = two ? launch_axis0_v<4, 2>(x, M, codes, lay, scales, lut, partial, R, C, pl, y, tag, st)
                    : launch_axis0_v<4, 1>(x, M, codes, lay, scales, lut, partial, R, C, pl, y, tag, st); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || tag) return e;
    const int MC = M * C;  // a multiple of 128
    const int nf = pl.ranges / pl.waves;
    const int terms = nf + (pl.ranges % pl.waves ? (pl.ranges % pl.waves > 1 ? 2 : 1) : 0);
    // a fused plan under stream capture: the same sum in band order as the
    // fused kernel's (bit-identical to an uncaptured call)
    if (axis0_fused(R, C, M))
        return launch_kernel(split_reduce_wave_kernel, dim3(MC / 64), dim3(kWave), st, partial, y, M,
                             C, pl.ranges, pl.waves, nf);
    // One wave per 64 outputs where there are enough of them to fill the chip
    // several times over (measured: M = 32 at 5120 outputs 0.7 us faster per
    // MLP layer), four adjacent outputs per lane where a wave's 256 stay in
    // one activation row (a further 0.1-0.2 us there); below that, four waves
    // per 64 outputs keep fewer dependent loads per lane (M = 1: the one-wave
    // form was 0.2 us slower).
    if (terms <= kReduceOneWave && MC / 64 >= 1024 && C % 256 == 0)
        return launch_kernel(split_reduce_wave4_kernel, dim3(MC / 256), dim3(kWave), st, partial, y,
                             M, C, pl.ranges, pl.waves, nf);
    if (terms <= kReduceOneWave && MC / 64 >= 1024)
        return launch_kernel(split_reduce_wave_kernel, dim3(MC / 64), dim3(kWave), st, partial, y, M,
                             C, pl.ranges, pl.waves, nf);
    return launch_kernel(split_reduce_kernel, dim3(MC / 64), dim3(kThreads), st, partial, y, M, C,
                         pl.ranges, pl.waves, nf);
}

}  // namespace trellis
