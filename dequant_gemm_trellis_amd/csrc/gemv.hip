// Axis-1 trellis GEMV (one activation row) for gfx950:
//   y[n] = bf16( sum_k x[k] * bf16( fl32( LUT[window(n, k)] * scales[n] ) ) ).
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0,
// page 60: wide-prefill.ts (axis-1 GEMV: decode each weight, round it to bf16,
// dot with the activations, float accumulation, bf16 store) and the
// tiled-prefill.ts weight-tile decode (window of weight t at bit (T-1-t)*k,
// wrapping inside the block).
//
// What bounds this kernel on MI355X is the codebook gather, not HBM: every
// weight needs one random read of the 4096-entry table, and random LDS reads
// bank-conflict. A wave-wide random ds_read costs about the same whether it
// moves 4 or 8 bytes per lane, so for k = 2 the kernel reads a pair table
// instead (one gather per two weights; see stage_pair_table). For k = 3 and 4
// the pair index would be 15/16 bits (256/512 KB) and does not fit in LDS, so
// those read the codebook itself, from eight bank-partitioned copies that cut
// the bank conflicts (see kRepCopies).
//
// Work mapping. The grid is persistent: one 512-thread workgroup (8 waves)
// per compute unit, workgroup g owning rows [g N / G, (g+1) N / G), so every CU gets the
// same number of rows. A unit of work is one 256-weight block of one row;
// units are numbered block-major inside a row chunk (all rows of block 0,
// then block 1, ...) and wave w takes the contiguous range
// [w U / 8, (w + 1) U / 8), 16 units per step. The 16 units of a step are
// thus 16 rows of one block (two where the range crosses a block edge), and a
// lane's block changes only once or twice over the wave's whole range.
// Lane l = 16 c + j takes the 64-weight run c of the unit in its column j.
// The run's 64 weights form eight 8-weight B fragments of
// v_mfma_f32_16x16x32_bf16 and the A fragment of the same lane carries the 8
// matching activations. Then D[j][j] sums exactly the four lanes of column j
// -- that unit's dot product -- while the off-diagonal entries mix units and
// are ignored: the matrix core does the multiply-adds and the 4-lane
// reduction, leaving the VALU to the decode. Unit partials go to LDS and each
// row is summed over its blocks in ascending order, so the result does not
// depend on timing.
//
// The activations are staged in LDS once per workgroup (served from the cache
// hierarchy instead, they cost several times the code traffic) and a lane
// keeps its unit's A fragments in registers until its block changes. Block b
// starts at byte 528 b, a stride of 132 words (4 mod 64), which keeps the
// reads of lanes on two different blocks on disjoint banks.
//
// Code words are prefetched two steps ahead into registers: measured under
// load, a memory round trip takes longer than one step of decode.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace trellis {
namespace {

// 8 waves per CU: measured 6-8% faster than 16 (less contention in the LDS
// queue); 4 or 6 were slower.
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kPartialCap = 2048;    // LDS for unit partials beyond the activation staging
constexpr int kXStride = 528;        // bytes per staged activation block (512 + 16)

// Decode table: the k = 2 pair table, or for k = 3, 4 the codebook in
// bank-partitioned copies (kRepCopies, 128 KB); both leave 32 KB of LDS.
// SINGLE: the plain 16 KB codebook, for launches whose workgroups decode too
// few units to repay building a 128 KB table (kSmallUnits).
template <int K, bool SINGLE = false>
struct GemvLds {
    static constexpr bool pair = K == 2 && !SINGLE;
    static constexpr bool rep = K != 2 && !SINGLE;
    static constexpr int tab_floats = pair ? 2 * kPairEntries : rep ? kRepFloats : kLutEntries;
    // activation bytes that fit beside the table and the partials in 160 KB
    static constexpr int x_bytes = 24576;
    static constexpr int max_blocks = x_bytes / kXStride;
    // fragments whose gathers are in flight ahead of the one being packed
    // (3 and 4 measured no faster)
    static constexpr int depth = 2;
};

// Below this many units (row x block) per workgroup the GEMV stages the plain
// codebook: writing a 128 KB table costs about as much LDS time as the faster
// gathers save over some 75 units.
constexpr int kSmallUnits = 64;

// Fragment S's gathers from the kernel's decode table.
template <int K, int S, bool SINGLE>
__device__ __forceinline__ Gathered<GemvLds<K, SINGLE>::pair> gemv_gather(
    const uint32_t (&w)[2 * K + 1], const float* __restrict__ tab) {
    return gather_tab<K, S, GemvLds<K, SINGLE>::pair, GemvLds<K, SINGLE>::rep>(w, tab);
}

template <int K, bool SINGLE>
using GemvTable = DecodeTable<kThreads, GemvLds<K, SINGLE>::pair, GemvLds<K, SINGLE>::rep>;

// Code words of one step for one lane, plus the unit's block and the
// row-major index (row * nb + block) of its partial.
template <int K>
struct Step {
    uint32_t w[2 * K + 1];
    float scale;
    uint32_t b;
    uint32_t slot;
};

struct XFrag {
    u32x4 v[8];
};

struct Ctx {
    const uint32_t* codes;   // word 0 of block 0 of the row chunk's first row
    CodeLayout lay;          // where a (row, block)'s words sit
    const float* scales;     // scale of the chunk's first row
    int nb;                  // blocks per row
    int cr;                  // rows in the chunk
    uint32_t magic;          // ceil(2^31 / cr): u / cr == mulhi(2u, magic) for u < 2^11
    int cp;                  // 3 - c: bit-position order of this lane's run
};

__device__ __forceinline__ uint32_t div_magic(int d) {
    // u / d == mulhi(2u, ceil(2^31 / d)) exactly while u * d < 2^31 (u < 2048 here)
    return static_cast<uint32_t>(((1ull << 31) + d - 1) / d);
}

// Unit u of the chunk (block-major): block u / cr, chunk row u % cr. Units at
// or past the wave's end re-read its last unit. Row-major codes (PAIRS false)
// sit at the unit's row-major index times wpb, a 32-bit product within the
// chunk; block-interleaved codes take the general 64-bit offset.
template <int K, bool PAIRS>
__device__ __forceinline__ void load_step(Step<K>& st, const Ctx& cx, int u, int u_end) {
    const uint32_t uu = static_cast<uint32_t>(u < u_end ? u : u_end - 1);
    const uint32_t b = __umulhi(uu << 1, cx.magic);
    const uint32_t rl = uu - b * static_cast<uint32_t>(cx.cr);
    st.b = b;
    st.slot = rl * static_cast<uint32_t>(cx.nb) + b;
    if constexpr (PAIRS)
        load_run64_words<K>(cx.codes + block_word<K>(cx.lay, rl, b), cx.cp, st.w);
    else
        load_run64_words<K>(cx.codes + st.slot * Bits<K>::wpb, cx.cp, st.w);
    st.scale = cx.scales[rl];
}

__device__ __forceinline__ XFrag load_x(const char* __restrict__ xs, uint32_t b, int c) {
    XFrag xf;
    const u32x4* p = reinterpret_cast<const u32x4*>(xs + b * kXStride + 128 * c);
#pragma unroll
    for (int s = 0; s < 8; ++s) xf.v[s] = p[s];
    return xf;
}

// One unit: eight fragments, software-pipelined so the LDS gathers of the next
// two fragments are in flight while one is packed and multiplied.
// D[j][j] of the 16x16 MFMA tile sits in lane 16 (j / 4) + j, register j % 4.
// The word after the run is not loaded but taken from the lane that holds the
// next run (next_run_word): one vector-memory instruction less per step
// measurably helps, since cache-missing loads slow the LDS-bound decode.
// The A fragments stay in registers while the lane's unit stays in the same
// block (xb), which with contiguous unit ranges per wave is all but one or two
// steps; re-reading them every step would cost about a quarter of the LDS time.
template <int K, bool SINGLE>
__device__ __forceinline__ void run_step(Step<K> st, XFrag& xf, uint32_t& xb,
                                         const char* __restrict__ xs,
                                         const float* __restrict__ tab, float* __restrict__ part,
                                         int u, int u_end, int j, int c) {
    constexpr bool P = GemvLds<K, SINGLE>::pair;
    st.w[2 * K] = next_run_word(st.w[0]);
    if (st.b != xb) {
        xb = st.b;
        xf = load_x(xs, st.b, c);
    }
    // Fragments in the order 7 .. 0: only the run's first weights (fragment 0)
    // have windows reaching into the next run's word, so its exchange has the
    // whole step to arrive.
    constexpr int D = GemvLds<K>::depth;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    Gathered<P> g[8];
    static_for<0, D>([&](auto ic) {
        constexpr int S = 7 - decltype(ic)::value;
        g[S] = gemv_gather<K, S, SINGLE>(st.w, tab);
    });
    static_for<0, 8>([&](auto ic) {
        constexpr int S = 7 - decltype(ic)::value;
        // Raised wave priority while a fragment's gathers issue, so the other
        // wave of the SIMD does not hold them back with its packing work and
        // the LDS queue stays fed (1-2% faster; around the packing instead,
        // no faster).
        __builtin_amdgcn_s_setprio(2);
        if constexpr (S >= D) g[S - D] = gemv_gather<K, S - D, SINGLE>(st.w, tab);
        __builtin_amdgcn_s_setprio(0);
        const bf16x8 bfrag = as_bf16x8(pack_fragment<P>(g[S], st.scale));
        acc = mfma16x16x32(as_bf16x8(xf.v[S]), bfrag, acc);
    });
    if (c == (j >> 2) && u < u_end) {
        const int v = j & 3;
        part[st.slot] = v == 0 ? acc[0] : v == 1 ? acc[1] : v == 2 ? acc[2] : acc[3];
    }
}

// silu(v) = v / (1 + e^-v) in float32: the gate nonlinearity of SwiGLU.
__device__ __forceinline__ float silu_f32(float v) { return v / (1.0f + expf(-v)); }

// Two projections of the same shape and the same activations (the gate and
// up projections of an MLP) can share one launch.
//   Without SWIGLU, workgroups below G0 compute y_a from (codes_a, scales_a,
//   lut_a), the others y_b from the b operands, each set of workgroups
//   splitting the N rows evenly; a single projection passes G0 = gridDim.x.
//   With SWIGLU (G0 = gridDim.x) every workgroup owns a row range of both: it
//   decodes the range's gate rows (a operands) from the gate codebook, restages
//   its table from the up codebook, decodes the same rows of the up projection
//   (b operands), and writes y_a[n] = bf16(silu(g_n) * u_n) from the two row
//   sums, float32 throughout. The unit partials of both phases stay in LDS.
template <int K, bool PAIRS, bool SINGLE, bool SWIGLU>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes_a,
    const float* __restrict__ scales_a, const float* __restrict__ lut_a,
    uint16_t* __restrict__ y_a, const uint32_t* __restrict__ codes_b,
    const float* __restrict__ scales_b, const float* __restrict__ lut_b,
    uint16_t* __restrict__ y_b, int G0, CodeLayout lay, int N, int nb) {
    // One LDS array with the table first: a gather address then needs no base
    // added (the table at 64 KB, past the 16-bit instruction offset, costs a
    // VALU op per weight). The unit partials take what the nb staged
    // activation blocks leave of the rest.
    __shared__ __attribute__((aligned(16)))
    float lds[GemvLds<K, SINGLE>::tab_floats + GemvLds<K>::x_bytes / 4 + kPartialCap];
    float* const tab = lds;
    char* const xs = reinterpret_cast<char*>(lds + GemvLds<K, SINGLE>::tab_floats);
    float* const part = reinterpret_cast<float*>(xs + nb * kXStride);
    const int part_cap = (GemvLds<K>::x_bytes - nb * kXStride) / 4 + kPartialCap;
    constexpr int kPhases = SWIGLU ? 2 : 1;

    const bool second = !SWIGLU && static_cast<int>(blockIdx.x) >= G0;
    const uint32_t* const codes = second ? codes_b : codes_a;
    const float* const scales = second ? scales_b : scales_a;
    const float* const lut = second ? lut_b : lut_a;
    uint16_t* const y = second ? y_b : y_a;
    const int G = second ? static_cast<int>(gridDim.x) - G0 : G0;
    const int g = second ? static_cast<int>(blockIdx.x) - G0 : static_cast<int>(blockIdx.x);
    const int r0 = static_cast<int>(static_cast<long>(g) * N / G);
    const int r1 = static_cast<int>(static_cast<long>(g + 1) * N / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, c = lane >> 4;
    const int chunk_rows = part_cap / (kPhases * nb);

    Ctx cx{codes + static_cast<size_t>(r0) * lay.row_words, lay, scales + r0, nb, 1, 0u, 3 - c};
    Step<K> sa, sb, sc;
    XFrag xf;
    uint32_t xb = ~0u;
    // Prologue: the codebook and the activations are fetched first, then the
    // first two steps' code words; the table and activation stores then wait
    // only for their own data (memory-counter waits retire in issue order),
    // while the code words are still on their way from HBM.
    constexpr int kXChunks = (GemvLds<K>::max_blocks * 32 + kThreads - 1) / kThreads;
    typename GemvTable<K, SINGLE>::Src tsrc;
    GemvTable<K, SINGLE>::fetch(tsrc, lut);
    u32x4 xv[kXChunks];
#pragma unroll
    for (int q = 0; q < kXChunks; ++q) {  // 16-byte chunks of x, 32 per block
        const int i = tid + q * kThreads;   // past the end: re-read the last chunk
        xv[q] = reinterpret_cast<const u32x4*>(x)[i < nb * 32 ? i : nb * 32 - 1];
    }
    asm volatile("" ::: "memory");  // keep the table and activation loads ahead of the code words
    // Wave w takes units [w U / W, (w + 1) U / W) of the chunk, 16 per step.
    // Every workgroup owns at least one row (G <= N), so CR >= 1, and the
    // first two steps are loaded unconditionally (a wave without units
    // re-reads a valid one): a load under a branch would make the table
    // stores below wait for the code words too.
    int CR = min(r1 - r0, chunk_rows), U = CR * nb;
    int ub = wave * U / kWaves, ue = (wave + 1) * U / kWaves;
    cx.cr = CR;
    cx.magic = div_magic(CR);
    load_step<K, PAIRS>(sa, cx, ub + j, ue > 1 ? ue : 1);
    load_step<K, PAIRS>(sb, cx, ub + 16 + j, ue > 1 ? ue : 1);
    GemvTable<K, SINGLE>::store(tsrc, tab);
#pragma unroll
    for (int q = 0; q < kXChunks; ++q) {
        const int i = tid + q * kThreads;
        if (i < nb * 32) *reinterpret_cast<u32x4*>(xs + (i >> 5) * kXStride + (i & 31) * 16) = xv[q];
    }
    __syncthreads();

    for (int cr0 = r0; cr0 < r1; cr0 += chunk_rows) {
        CR = min(r1 - cr0, chunk_rows);
        U = CR * nb;
        ub = wave * U / kWaves;
        ue = (wave + 1) * U / kWaves;
        for (int ph = 0; ph < kPhases; ++ph) {
            if constexpr (SWIGLU) {
                // Every phase but the first of the launch switches projection:
                // the other codebook is fetched and the phase's first two steps
                // loaded while the waves finish with the old table, which is
                // then rewritten.
                if (cr0 != r0 || ph != 0) {
                    cx.codes = (ph ? codes_b : codes_a) + static_cast<size_t>(cr0) * lay.row_words;
                    cx.scales = (ph ? scales_b : scales_a) + cr0;
                    cx.cr = CR;
                    cx.magic = div_magic(CR);
                    typename GemvTable<K, SINGLE>::Src ts;
                    GemvTable<K, SINGLE>::fetch(ts, ph ? lut_b : lut_a);
                    asm volatile("" ::: "memory");
                    load_step<K, PAIRS>(sa, cx, ub + j, ue > 1 ? ue : 1);
                    load_step<K, PAIRS>(sb, cx, ub + 16 + j, ue > 1 ? ue : 1);
                    __syncthreads();
                    GemvTable<K, SINGLE>::store(ts, tab);
                    __syncthreads();
                }
            } else if (cr0 != r0 && ue > ub) {
                cx.codes = codes + static_cast<size_t>(cr0) * lay.row_words;
                cx.scales = scales + cr0;
                cx.cr = CR;
                cx.magic = div_magic(CR);
                load_step<K, PAIRS>(sa, cx, ub + j, ue);
                load_step<K, PAIRS>(sb, cx, ub + 16 + j, ue);
            }
            float* const pp = part + ph * U;  // this phase's unit partials
            // Three register sets rotate, so the code words of the next two
            // steps are in flight while one step is decoded. Every load is
            // unconditional (past the end it re-reads a valid unit) and only
            // the decode steps are guarded: the memory-counter waits the
            // compiler places must hold on every path, so a conditional load,
            // or a loop exit between loads, makes it wait for the prefetch too.
            for (int u0 = ub; u0 < ue; u0 += 48) {
                const int ua = u0 + j;
                load_step<K, PAIRS>(sc, cx, ua + 32, ue);
                run_step<K, SINGLE>(sa, xf, xb, xs, tab, pp, ua, ue, j, c);
                load_step<K, PAIRS>(sa, cx, ua + 48, ue);
                if (u0 + 16 < ue) run_step<K, SINGLE>(sb, xf, xb, xs, tab, pp, ua + 16, ue, j, c);
                load_step<K, PAIRS>(sb, cx, ua + 64, ue);
                if (u0 + 32 < ue) run_step<K, SINGLE>(sc, xf, xb, xs, tab, pp, ua + 32, ue, j, c);
            }
        }
        __syncthreads();
        // Each row: its block partials added in ascending block order (for
        // SWIGLU once per projection).
        auto row_sum = [&](const float* pr) {
            float s = 0.f;
            int q = 0;
            for (; q + 8 <= nb; q += 8) {  // reads issued together, added in order
                float v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = pr[q + i];
#pragma unroll
                for (int i = 0; i < 8; ++i) s += v[i];
            }
            for (; q < nb; ++q) s += pr[q];
            return s;
        };
        for (int r = tid; r < CR; r += kThreads) {
            const float s = row_sum(part + r * nb);
            if constexpr (SWIGLU) y[cr0 + r] = round_bf16(silu_f32(s) * row_sum(part + U + r * nb));
            else y[cr0 + r] = round_bf16(s);
        }
        __syncthreads();
    }
}

// One projection on min(N, CUs) workgroups, or two (the b operands non-null)
// on min(N, CUs / 2) workgroups each, so that every CU runs one workgroup.
template <int K>
hipError_t launch_gemv_k(const uint16_t* x, const uint32_t* codes, const float* scales,
                         const float* lut, uint16_t* y, const uint32_t* codes_b,
                         const float* scales_b, const float* lut_b, uint16_t* y_b, CodeLayout lay,
                         int N, int nb, hipStream_t st) {
    const bool dual = codes_b != nullptr;
    int G0 = dual ? cu_count() / 2 : cu_count();
    if (G0 < 1) G0 = 1;
    if (G0 > N) G0 = N;
    const int G = dual ? 2 * G0 : G0;
    if (!dual) {
        codes_b = codes;
        scales_b = scales;
        lut_b = lut;
        y_b = y;
    }
    // Row-major iff a row's blocks are contiguous (with two blocks per row the
    // two layouts coincide). Workgroups own ceil(N / G0) rows at most.
    const bool rowmajor = lay.row_words == static_cast<uint64_t>(nb) * Bits<K>::wpb;
    const bool small = static_cast<long>((N + G0 - 1) / G0) * nb < kSmallUnits;
    auto kern = small ? (rowmajor ? gemv_kernel<K, false, true, false> : gemv_kernel<K, true, true, false>)
                      : (rowmajor ? gemv_kernel<K, false, false, false> : gemv_kernel<K, true, false, false>);
    return launch_kernel(kern, dim3(G), dim3(kThreads), st, x, codes, scales, lut, y, codes_b,
                         scales_b, lut_b, y_b, G0, lay, N, nb);
}

// Gate and up with the SwiGLU epilogue: min(N, CUs) workgroups, each owning a
// row range of both projections.
template <int K>
hipError_t launch_gemv_swiglu_k(const uint16_t* x, const uint32_t* codes_g, const float* scales_g,
                                const float* lut_g, const uint32_t* codes_u,
                                const float* scales_u, const float* lut_u, uint16_t* h,
                                CodeLayout lay, int N, int nb, hipStream_t st) {
    int G = cu_count();
    if (G > N) G = N;
    if (G < 1) G = 1;
    const bool rowmajor = lay.row_words == static_cast<uint64_t>(nb) * Bits<K>::wpb;
    const bool small = 2l * ((N + G - 1) / G) * nb < kSmallUnits;
    auto kern = small ? (rowmajor ? gemv_kernel<K, false, true, true> : gemv_kernel<K, true, true, true>)
                      : (rowmajor ? gemv_kernel<K, false, false, true> : gemv_kernel<K, true, false, true>);
    return launch_kernel(kern, dim3(G), dim3(kThreads), st, x, codes_g, scales_g, lut_g, h, codes_u,
                         scales_u, lut_u, h, G, lay, N, nb);
}

// ---------------------------------------------------------------------------
// Several activation rows, 1 <= M <= 8, in the GEMV's work mapping (the
// M-row counterpart of wide-prefill.ts's multi-vector GEMV on page 60).
//
// Units, steps, the code prefetch and the decode are those of gemv_kernel;
// only the multiply differs. Lane l = 16 c + j still decodes run c of the
// step's unit j into B fragments, but the A fragment of lane (c, m = j) now
// holds activation row m (rows m >= M repeat row M - 1) at the run-c
// positions of a block, so D[m][j] of the 16x16 tile is row m against unit j:
// the MFMA yields M outputs per unit instead of one diagonal entry. A holds
// one block, so a step whose 16 units straddle a block edge (workgroups own
// at least 16 rows, so at most two blocks) multiplies again with the next
// block's fragments and each lane keeps the product of its own unit's block.
// Unlike tiled-prefill.ts-style 16-row tasks, no row slots are left empty
// when a workgroup's row count is not a multiple of 16.
//
// Each unit's M partials go to LDS in unit order, M rounded up to 4 or 8
// (lane (c, j) stores D[4c .. 4c + 3][j], one 16-byte write); each output is
// the sum of its row's block partials in ascending block order. Rows are
// split into equal chunks whose partials fit beside the table. Activation
// fragments are loaded straight from global memory in A layout (M x 4 cache
// lines per instruction), one block ahead of use: xf holds the step's first
// block, xn the next one.
// Chunks for a workgroup of `rows` rows when at most `max_rows` rows' partials
// fit: the fewest balanced chunks, or 0 if one would hold fewer than 16 rows.
__host__ __device__ inline int rows_chunks(int rows, int max_rows) {
    if (max_rows < 16 || rows < 16) return 0;
    const int n = (rows + max_rows - 1) / max_rows;
    return rows / n >= 16 ? n : 0;
}

// REP (k = 3, 4): the bank-partitioned codebook copies, which leave room for
// the partials of fewer rows (one chunk of 68 rows up to 4 activation rows at
// 5120 inputs); else the 16 KB codebook.
template <int K, bool REP>
struct RowsLds {
    static constexpr bool pair = K == 2;
    static constexpr bool rep = REP;
    using Table = DecodeTable<kThreads, pair, rep>;
    static constexpr int tab_floats = Table::floats;
    static constexpr int part_floats = (pair || rep) ? 7936 : 32768;  // the rest of 160 KB
};

// Activation fragments of block b in A layout from xa (row m = j, column 64 c).
__device__ __forceinline__ void load_xa(XFrag& xn, const uint16_t* xa, uint32_t b) {
    const u32x4* p = reinterpret_cast<const u32x4*>(xa + b * kT);
#pragma unroll
    for (int s = 0; s < 8; ++s) xn.v[s] = p[s];
}

// The same through an opaque global-address-space pointer, for the prologue
// (through the restrict kernel pointer the loads would be sunk to first use).
__device__ __forceinline__ void load_xa_opaque(XFrag& xn, const uint16_t* xa, uint32_t b) {
    using gu32x4 = const __attribute__((address_space(1))) u32x4*;
    gu32x4 p = (gu32x4)(xa + b * kT);
    asm volatile("" : "+v"(p));
#pragma unroll
    for (int s = 0; s < 8; ++s) xn.v[s] = p[s];
}

// One step of 16 units: eight fragments, gathers two ahead as in run_step.
// STRAD: the step's units reach into block blo + 1, multiplied against xn.
template <int K, bool REP, bool STRAD>
__device__ __forceinline__ void run_rows_step(Step<K> st, const XFrag& xf, const XFrag& xn,
                                              uint32_t blo, const float* __restrict__ tab,
                                              float* __restrict__ part, int u, int u_end, int c) {
    constexpr bool P = RowsLds<K, REP>::pair;
    constexpr int D = GemvLds<K>::depth;
    st.w[2 * K] = next_run_word(st.w[0]);
    floatx4 d1 = {0.f, 0.f, 0.f, 0.f}, d2 = {0.f, 0.f, 0.f, 0.f};
    Gathered<P> g[8];
    static_for<0, D>([&](auto ic) {
        constexpr int S = 7 - decltype(ic)::value;
        g[S] = gather_tab<K, S, P, REP>(st.w, tab);
    });
    static_for<0, 8>([&](auto ic) {
        constexpr int S = 7 - decltype(ic)::value;
        __builtin_amdgcn_s_setprio(2);  // as in run_step
        if constexpr (S >= D) g[S - D] = gather_tab<K, S - D, P, REP>(st.w, tab);
        __builtin_amdgcn_s_setprio(0);
        const bf16x8 bfrag = as_bf16x8(pack_fragment<P>(g[S], st.scale));
        d1 = mfma16x16x32(as_bf16x8(xf.v[S]), bfrag, d1);
        if constexpr (STRAD) d2 = mfma16x16x32(as_bf16x8(xn.v[S]), bfrag, d2);
    });
    if constexpr (STRAD) {
        if (st.b != blo) d1 = d2;
    }
    // D rows 4c + v: only c = 0 holds activation rows (M <= kGemvRowsMaxM = 4)
    if (c == 0 && u < u_end) *reinterpret_cast<floatx4*>(part + u * 4) = d1;
}

template <int K, bool PAIRS, bool REP>
__global__ __launch_bounds__(kThreads) void gemv_rows_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
    const float* __restrict__ scales, const float* __restrict__ lut,
    uint16_t* __restrict__ y, CodeLayout lay, int N, int nb, int M) {
    using Lds = RowsLds<K, REP>;
    __shared__ __attribute__((aligned(16))) float lds[Lds::tab_floats + Lds::part_floats];
    float* const tab = lds;
    float* const part = lds + Lds::tab_floats;

    const int G = gridDim.x, g = blockIdx.x;
    const int r0 = static_cast<int>(static_cast<long>(g) * N / G);
    const int r1 = static_cast<int>(static_cast<long>(g + 1) * N / G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, c = lane >> 4;
    constexpr int m4 = 4;  // partial floats per unit (M <= kGemvRowsMaxM = 4)
    // Balanced row chunks whose unit partials fit; chunk q is rows
    // [r0 + q rows / n, r0 + (q + 1) rows / n). The launcher guarantees at
    // least 16 rows per chunk (rows_chunks).
    const int rows = r1 - r0;
    const int nchunks = rows_chunks(rows, Lds::part_floats / (m4 * nb));
    const long in = static_cast<long>(nb) * kT;
    const uint16_t* const xa = x + (j < M ? j : M - 1) * in + 64 * c;

    Ctx cx{codes + static_cast<size_t>(r0) * lay.row_words, lay, scales + r0, nb, 1, 0u, 3 - c};
    Step<K> sa, sb, sc;
    XFrag xf, xn;
    // Prologue: the table sources first, then the first two steps' code words
    // and the first two blocks' activation fragments (all unconditional), so
    // the table stores wait only for their own data.
    typename Lds::Table::Src tsrc;
    Lds::Table::fetch(tsrc, lut);
    asm volatile("" ::: "memory");
    int CR = rows / nchunks, U = CR * nb;
    int ub = wave * U / kWaves, ue = (wave + 1) * U / kWaves;
    cx.cr = CR;
    cx.magic = div_magic(CR);
    uint32_t xb = static_cast<uint32_t>((ub < U ? ub : U - 1) / CR);
    load_step<K, PAIRS>(sa, cx, ub + j, ue > 1 ? ue : 1);
    load_step<K, PAIRS>(sb, cx, ub + 16 + j, ue > 1 ? ue : 1);
    load_xa_opaque(xf, xa, xb);
    load_xa_opaque(xn, xa, xb + 1 < static_cast<uint32_t>(nb) ? xb + 1 : xb);
    asm volatile("" ::: "memory");
    Lds::Table::store(tsrc, tab);
    __syncthreads();

    for (int q = 0; q < nchunks; ++q) {
        const int cr0 = r0 + q * rows / nchunks;
        CR = r0 + (q + 1) * rows / nchunks - cr0;
        U = CR * nb;
        ub = wave * U / kWaves;
        ue = (wave + 1) * U / kWaves;
        if (cr0 != r0 && ue > ub) {
            cx.codes = codes + static_cast<size_t>(cr0) * lay.row_words;
            cx.scales = scales + cr0;
            cx.cr = CR;
            cx.magic = div_magic(CR);
            load_step<K, PAIRS>(sa, cx, ub + j, ue);
            load_step<K, PAIRS>(sb, cx, ub + 16 + j, ue);
            xb = static_cast<uint32_t>(ub / CR);
            load_xa(xf, xa, xb);
            load_xa(xn, xa, xb + 1 < static_cast<uint32_t>(nb) ? xb + 1 : xb);
        }
        // One step: advance the activation blocks when the step starts in the
        // next block (steps move at most one block on: CR >= 16), then decode
        // and multiply, twice if the step reaches into the block after.
        auto step = [&](const Step<K>& st, int u0) {
            const uint32_t blo = static_cast<uint32_t>(u0 / CR);
            const int ulast = (u0 + 15 < ue ? u0 + 15 : ue - 1);
            const bool strad = static_cast<uint32_t>(ulast / CR) != blo;
            if (blo != xb) {
                xb = blo;
                xf = xn;
                load_xa(xn, xa, blo + 1 < static_cast<uint32_t>(nb) ? blo + 1 : blo);
            }
            // k = 3, 4: the second multiply on every step measured 1-2% faster
            // than a branch (the compiler hoists the branch's common gathers
            // and waits for all of them at it); k = 2: the branch.
            if constexpr (K != 2) {
                (void)strad;
                run_rows_step<K, REP, true>(st, xf, xn, blo, tab, part, u0 + j, ue, c);
            } else if (strad) {
                run_rows_step<K, REP, true>(st, xf, xn, blo, tab, part, u0 + j, ue, c);
            } else {
                run_rows_step<K, REP, false>(st, xf, xn, blo, tab, part, u0 + j, ue, c);
            }
        };
        // Three register sets rotate as in gemv_kernel; every load is
        // unconditional, only the steps are guarded.
        for (int u0 = ub; u0 < ue; u0 += 48) {
            load_step<K, PAIRS>(sc, cx, u0 + 32 + j, ue);
            step(sa, u0);
            load_step<K, PAIRS>(sa, cx, u0 + 48 + j, ue);
            if (u0 + 16 < ue) step(sb, u0 + 16);
            load_step<K, PAIRS>(sb, cx, u0 + 64 + j, ue);
            if (u0 + 32 < ue) step(sc, u0 + 32);
        }
        __syncthreads();
        // y[m][row] = sum over blocks, ascending, of the unit partials.
        for (int o = tid; o < CR * M; o += kThreads) {
            const int m = o / CR, rl = o - m * CR;
            const float* pr = part + rl * m4 + m;
            const int bstride = CR * m4;
            float s = 0.f;
            int bq = 0;
            for (; bq + 8 <= nb; bq += 8) {  // reads issued together, added in order
                float v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = pr[(bq + i) * bstride];
#pragma unroll
                for (int i = 0; i < 8; ++i) s += v[i];
            }
            for (; bq < nb; ++bq) s += pr[bq * bstride];
            y[static_cast<size_t>(m) * N + cr0 + rl] = round_bf16(s);
        }
        __syncthreads();
    }
}

// One workgroup per compute unit, but at least 16 rows each, so a step's 16
// units span at most two blocks.
int rows_grid(int N) {
    const int G = N / 16 < cu_count() ? N / 16 : cu_count();
    return G < 1 ? 1 : G;
}

template <int K, bool REP>
hipError_t launch_gemv_rows_kr(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                               const float* scales, const float* lut, uint16_t* y, int N, int nb,
                               hipStream_t st) {
    const int G = rows_grid(N);
    if (lay.row_words == static_cast<uint64_t>(nb) * Bits<K>::wpb)
        return launch_kernel(gemv_rows_kernel<K, false, REP>, dim3(G), dim3(kThreads), st, x,
                             codes, scales, lut, y, lay, N, nb, M);
    return launch_kernel(gemv_rows_kernel<K, true, REP>, dim3(G), dim3(kThreads), st, x, codes,
                         scales, lut, y, lay, N, nb, M);
}

// Every workgroup's partials fit in one chunk beside a RowsLds<K, REP> table.
template <int K, bool REP>
bool rows_one_chunk(int M, int N, int nb) {
    const int max_rows = RowsLds<K, REP>::part_floats / (4 * nb);
    const int G = rows_grid(N);
    // workgroups own floor(N / G) or ceil(N / G) rows
    return rows_chunks(N / G, max_rows) == 1 && rows_chunks((N + G - 1) / G, max_rows) == 1;
}

template <int K>
hipError_t launch_gemv_rows_k(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                              const float* scales, const float* lut, uint16_t* y, int N, int nb,
                              hipStream_t st) {
    // k = 3, 4: the replicated codebook when every workgroup's partials fit in
    // one chunk beside it.
    if constexpr (K != 2) {
        if (rows_one_chunk<K, true>(M, N, nb))
            return launch_gemv_rows_kr<K, true>(x, M, codes, lay, scales, lut, y, N, nb, st);
    }
    return launch_gemv_rows_kr<K, false>(x, M, codes, lay, scales, lut, y, N, nb, st);
}

}  // namespace

// Per-device cache; atomic so that host threads calling the library at the
// same time only ever race to store the same value.
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int gemv_max_blocks(int k) {
    return k == 2 ? GemvLds<2>::max_blocks : GemvLds<4>::max_blocks;
}

hipError_t launch_gemv(const uint16_t* x, const uint32_t* codes, CodeLayout lay, const float* scales,
                       const float* lut, uint16_t* y, int N, int nb, int k, hipStream_t st) {
    switch (k) {
    case 2: return launch_gemv_k<2>(x, codes, scales, lut, y, nullptr, nullptr, nullptr, nullptr, lay, N, nb, st);
    case 3: return launch_gemv_k<3>(x, codes, scales, lut, y, nullptr, nullptr, nullptr, nullptr, lay, N, nb, st);
    case 4: return launch_gemv_k<4>(x, codes, scales, lut, y, nullptr, nullptr, nullptr, nullptr, lay, N, nb, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_dual(const uint16_t* x, const uint32_t* codes_a, const float* scales_a,
                            const float* lut_a, uint16_t* y_a, const uint32_t* codes_b,
                            const float* scales_b, const float* lut_b, uint16_t* y_b,
                            CodeLayout lay, int N, int nb, int k, hipStream_t st) {
    switch (k) {
    case 2: return launch_gemv_k<2>(x, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, lay, N, nb, st);
    case 3: return launch_gemv_k<3>(x, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, lay, N, nb, st);
    case 4: return launch_gemv_k<4>(x, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, lay, N, nb, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_swiglu(const uint16_t* x, const uint32_t* codes_g, const float* scales_g,
                              const float* lut_g, const uint32_t* codes_u, const float* scales_u,
                              const float* lut_u, uint16_t* h, CodeLayout lay, int N, int nb, int k,
                              hipStream_t st) {
    switch (k) {
    case 2: return launch_gemv_swiglu_k<2>(x, codes_g, scales_g, lut_g, codes_u, scales_u, lut_u, h, lay, N, nb, st);
    case 3: return launch_gemv_swiglu_k<3>(x, codes_g, scales_g, lut_g, codes_u, scales_u, lut_u, h, lay, N, nb, st);
    case 4: return launch_gemv_swiglu_k<4>(x, codes_g, scales_g, lut_g, codes_u, scales_u, lut_u, h, lay, N, nb, st);
    default: return hipErrorInvalidValue;
    }
}

bool gemv_rows_supported(int M, int N, int nb, int k) {
    if (M < 1 || M > kGemvRowsMaxM || N < 16 || nb < 1) return false;
    const int max_rows =
        (k == 2 ? RowsLds<2, false>::part_floats : RowsLds<4, false>::part_floats) / (4 * nb);
    const int G = rows_grid(N);
    // workgroups own floor(N / G) or ceil(N / G) rows
    return rows_chunks(N / G, max_rows) > 0 && rows_chunks((N + G - 1) / G, max_rows) > 0;
}

hipError_t launch_gemv_rows(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                            const float* scales, const float* lut, uint16_t* y, int N, int nb,
                            int k, hipStream_t st) {
    switch (k) {
    case 2: return launch_gemv_rows_k<2>(x, M, codes, lay, scales, lut, y, N, nb, st);
    case 3: return launch_gemv_rows_k<3>(x, M, codes, lay, scales, lut, y, N, nb, st);
    case 4: return launch_gemv_rows_k<4>(x, M, codes, lay, scales, lut, y, N, nb, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace trellis
