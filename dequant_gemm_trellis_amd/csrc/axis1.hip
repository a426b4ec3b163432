// Axis-1 trellis kernels for gfx950: the fused decode + bf16 MFMA kernel of
// 16-row groups for several activation rows (1 <= M <= 32; the library sends
// small batches to the GEMV-mapped kernel in gemv.hip when that fits and
// measured faster, and long single rows here when neither GEMV kernel takes
// them), and the diagnostic expand kernel. Both decode through the same
// fragment builder.
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0,
// page 60: tiled-prefill.ts (axis-1 tile decode + matrix multiply, bf16
// rounding of each weight), wide-prefill.ts (axis-1 multi-vector GEMV),
// vector-expand.ts (whole-matrix decode).
//
// Fragment mapping (one 64-lane wavefront, v_mfma_f32_16x16x32_bf16):
//   lane l -> row j = l % 16 of a 16-row group, run c = l / 16 of a block.
//   Run c holds weights t in [64c, 64c + 64) of a 256-weight block. Weight t
//   sits at bit (255 - t) * k, so the run is the contiguous bit range
//   [64 (3 - c) k, 64 (4 - c) k) -- exactly 2k words -- plus the 11 window
//   bits that spill into the next word (the block's word 0 for the last run:
//   the tail-biting wrap), taken from the lane that holds the next run.
//   The 64 weights of a run become eight 8-weight B fragments (B[k][n],
//   k = 8 c + e within the instruction); the A fragment is the matching 8
//   activations of row m = 16 mt + j. Because A and B index k identically,
//   the hardware's k order inside the instruction does not matter.
//
// Work mapping. The grid is persistent (one workgroup per compute unit),
// workgroup g owning rows [g N / G, (g+1) N / G), at most kGroups
// 16-row groups; or, given a workspace, whole groups only plus a block range
// of one leftover group (the balanced plan, SplitArgs). A task is one group x
// one 256-weight block; the workgroup's
// tasks are numbered block-major (all groups of block 0, then block 1, ...)
// and each wave takes a contiguous range of them. A wave thus meets only a
// few blocks and loads their activation fragments once per block, reusing
// them for every group. Each wave keeps one accumulator tile per group; at the
// end the per-wave tiles are summed in LDS in wave order (deterministic),
// reusing the table's space. Lanes of rows past the workgroup's range decode
// all-zero words, so their gathers all hit one LDS address.
//
// Activation fragments reach the lanes one of two ways, chosen by M:
//   - direct (one M tile, M <= 16): each lane loads its own fragments from
//     global memory in A layout, a task ahead of use. Lanes of rows m >= M
//     read row M - 1, so an instruction touches only M x 4 distinct cache
//     lines, and nothing goes through the LDS, which the codebook gathers
//     keep busy;
//   - staged (two M tiles): coalesced loads of 16 rows, transposed through a
//     per-wave LDS slot when the block changes (the two tiles' direct
//     fragments, twice over for the fetch ahead, do not fit in registers).
// At k = 3, 4 both use the bank-partitioned codebook copies (the staged path
// with a one-line slot beside them).
#include <unistd.h>

#include <atomic>
#include <chrono>

#include "common.hpp"
#include "launch.hpp"

namespace trellis {
namespace {

constexpr int kThreads = 256;    // expand kernel
constexpr int kGroups = 5;       // 16-row groups per prefill workgroup (80 rows)
constexpr int kDualGroups = 9;   // the same for the two-projection launch (144 rows)
// Mixed gate/up groups: each projection's codebook in kMixedCopies
// bank-partitioned copies, beside which a one-line activation slot fits.
constexpr int kMixedCopies = 4;
constexpr int kMixedLines = kMixedCopies > 1 ? 1 : 4;
constexpr uint32_t kMixedSpan = kLutEntries * 4 * kMixedCopies;  // bytes per codebook

// Prefill workgroup size: 8 waves, two per SIMD. For one M tile this
// measured 2-7% faster than 16 waves (less contention in the LDS queue); two
// M tiles need the register budget of two waves per SIMD anyway, and 4 waves
// measured much slower.
template <int MT>
struct PrefillShape {
    static constexpr int threads = 512;
    static constexpr int waves = threads / kWave;
};

// Per-wave activation slot (staged path only): `lines` 128-byte lines (8
// chunks of 16 bytes) of each of the 16 rows of each M tile. Beside a 128 KB
// table (the pair table or the codebook copies) only one line fits (2 KB per
// tile); beside the plain 16 KB codebook all four would.
template <int K, int MT, bool DIRECT, int KG = kGroups>
struct PrefillLds {
    static constexpr bool pair = K == 2;
    // k = 3, 4: the bank-partitioned codebook copies (128 KB), beside which a
    // staged launch (two M tiles) has room for the one-line slot only; with two
    // lines of one tile per round that measured 2.5% faster than the 16 KB
    // codebook with the four-line slot. (A staged launch of one M tile does
    // not occur; it would keep the plain codebook.)
    static constexpr bool rep = !pair && (DIRECT || MT == 2);
    using Table = DecodeTable<PrefillShape<MT>::threads, pair, rep>;
    static constexpr int tab_floats = Table::floats;
    static constexpr int waves = PrefillShape<MT>::waves;
    static constexpr int lines = tab_floats > kLutEntries ? 1 : 4;
    static constexpr int slot_chunks = DIRECT ? 0 : MT * lines * 16 * 8;
    // direct activations: a per-wave area for the first block's fragments,
    // fetched coalesced and passed through LDS two lines at a time (at
    // M = 9..16 the per-lane A-layout loads touch 64 cache lines per
    // instruction, which cost the prologue about 1 us)
    static constexpr int pro_chunks = DIRECT ? 2 * 16 * 8 : 0;
    static constexpr int decode_floats = tab_floats + waves * (slot_chunks + pro_chunks) * 4;
    static constexpr int part_floats = waves * KG * 256;  // one M tile of wave partials
    static constexpr int floats = decode_floats > part_floats ? decode_floats : part_floats;
};

struct TaskCtx {
    const uint32_t* codes;
    CodeLayout lay;
    const float* scales;
    int nb, gc, r0, r1, j, cp;
    // Mixed groups (MIXED): virtual row v < rm is row r0 + v of the first
    // projection (codes, scales), v >= rm row r0 + v - rm of the second
    // (codes_b, scales_b), whose codebook sits 16 KB above the first in LDS.
    const uint32_t* codes_b;
    const float* scales_b;
    int rm;
    // Folded last group (gf >= 1; see task_place): the number of full groups
    // before it. -1: no folding.
    int gf = -1;
    // Split leftover group (SPLIT; see SplitArgs): this workgroup's nq tasks
    // of the 16-row group at rows [rs, rs + 16) (rows from rn on are padding),
    // blocks qb0 .. qb0 + nq - 1, numbered first, in accumulator slot gc. The
    // whole groups' blocks follow in block-major order from block bs (then
    // wrapping to 0): with staged activations bs is the last split block, so
    // that wave 0's first whole-group task needs no activation refresh.
    int nq = 0, qb0 = 0, rs = 0, rn = 0, bs = 0;
};

template <int K>
struct Task {
    uint32_t w[2 * K + 1];
    float scale;
    int b, g;      // block and row group: uniform across the wave
    bool valid;    // this lane's row lies in the workgroup's range
    bool fold;     // a folded task (uniform)
    uint32_t sel;  // MIXED: byte offset of this lane's codebook in LDS
};

// Where task tc sits. Without folding, block-major: tc = b gc + g. Folding
// serves a last group of at most 8 rows with one M tile of at most 8
// activation rows: A and B then have 8 spare rows and columns, so a task can
// hold that group's rows for two blocks side by side -- lanes j < 8 block b,
// j >= 8 block b + 1, A rows 0-7 block b's activations, rows 8-15 block
// b + 1's -- and the two diagonal 8x8 quarters of D are the two blocks'
// partials (the other two quarters are ignored). Each pair of blocks (2P,
// 2P + 1) runs the gf full groups of block 2P, the folded task, then the full
// groups of block 2P + 1 (an odd last block: its full groups and a folded task
// with an empty second half), so blocks still change one at a time and the
// last group costs half a task per block instead of a whole one.
//
// A wave loads its tasks in order (tau0, tau0 + 1, ...; past its last task it
// re-reads that one), so a cursor walks the sequence with compares: one
// division when it is set, none per task.
struct TaskCursor {
    int tau;  // the task the next load reads
    int b0;   // its block (no folding) or the pair's first block (folding)
    int rem;  // its position within the block's gc or the pair's 2 gf + 1 tasks
};

template <bool FOLD, bool SPLIT = false>
__device__ __forceinline__ TaskCursor task_cursor(const TaskCtx& cx, int tau0, int tau_end) {
    const int tau = tau0 < tau_end ? tau0 : tau_end - 1;
    if constexpr (SPLIT) {
        if (tau < cx.nq) return {tau, 0, 0};
        const int q = (tau - cx.nq) / cx.gc;
        return {tau, q, tau - cx.nq - q * cx.gc};
    }
    const bool fold = FOLD && cx.gf >= 0;
    const int per = fold ? 2 * cx.gf + 1 : cx.gc;
    const int q = tau / per;
    return {tau, fold ? 2 * q : q, tau - q * per};
}

// The cursor's task (block, group, folded?), then the cursor moves on unless
// that was the last task before tau_end.
template <bool FOLD, bool SPLIT = false>
__device__ __forceinline__ void task_place(const TaskCtx& cx, TaskCursor& k, int tau_end, int& b,
                                           int& g, bool& fold) {
    if constexpr (SPLIT) {
        // the split tasks first, then the full groups block-major; the
        // block-major cursor starts moving past the first full task
        const bool sp = k.tau < cx.nq;
        const int bw = k.b0 + cx.bs;
        b = sp ? cx.qb0 + k.tau : (bw < cx.nb ? bw : bw - cx.nb);
        g = sp ? cx.gc : k.rem;
        fold = false;
        if (k.tau + 1 < tau_end && ++k.tau > cx.nq && ++k.rem == cx.gc) {
            k.rem = 0;
            ++k.b0;
        }
        return;
    }
    const bool folding = FOLD && cx.gf >= 0;
    if (!folding) {
        b = k.b0;
        g = k.rem;
        fold = false;
    } else {
        fold = k.rem == cx.gf;
        b = k.b0 + (k.rem > cx.gf ? 1 : 0);
        g = k.rem < cx.gf ? k.rem : k.rem > cx.gf ? k.rem - cx.gf - 1 : cx.gf;
    }
    if (k.tau + 1 < tau_end) {
        ++k.tau;
        if (++k.rem == (folding ? 2 * cx.gf + 1 : cx.gc)) {
            k.rem = 0;
            k.b0 += folding ? 2 : 1;
        }
    }
}

// A folded task's lane: row r0 + 16 g + (j & 7) of block b + (j >> 3). Lanes
// past the rows or past the last block re-read a valid row and block; their
// scale is zeroed, since their D columns are added into stored rows.
__device__ __forceinline__ void fold_lane(const TaskCtx& cx, int g, int b, int& rc, int& bl,
                                          bool& valid) {
    const int row = cx.r0 + 16 * g + (cx.j & 7);
    const int blk = b + (cx.j >> 3);
    valid = row < cx.r1 && blk < cx.nb;
    rc = row < cx.r1 ? row : cx.r1 - 1;
    bl = blk < cx.nb ? blk : cx.nb - 1;
}

// The stored row, code array and scales of lane row 16 g + j of a task, and
// whether it is a real row (rows past the range re-read the last real one).
template <bool MIXED, bool SPLIT = false>
__device__ __forceinline__ int task_row(const TaskCtx& cx, int g, bool& valid, bool& second) {
    if constexpr (SPLIT) {
        if (g == cx.gc) {  // the split group (a uniform test)
            const int row = cx.rs + cx.j;
            valid = row < cx.rn;
            second = false;
            return valid ? row : cx.rn - 1;
        }
    }
    const int v = 16 * g + cx.j;
    if constexpr (MIXED) {
        valid = v < 2 * cx.rm;
        const int vc = valid ? v : 2 * cx.rm - 1;
        second = vc >= cx.rm;
        return cx.r0 + (second ? vc - cx.rm : vc);
    } else {
        const int row = cx.r0 + v;
        valid = row < cx.r1;
        second = false;
        return valid ? row : cx.r1 - 1;
    }
}

// Word offset of block b of row rc. Row-major codes (PAIRS false) keep the
// plain row-major product; the general layout form measured 1% slower there
// (more scalar work per task).
template <int K, bool PAIRS>
__device__ __forceinline__ uint64_t task_word(const TaskCtx& cx, int rc, int b) {
    if constexpr (PAIRS) return block_word<K>(cx.lay, rc, b);
    else return (static_cast<size_t>(rc) * cx.nb + b) * Bits<K>::wpb;
}

// This lane's copy of its codebook (mixed groups), as a byte offset.
__device__ __forceinline__ uint32_t mixed_copy_offset() {
    return (threadIdx.x & (kMixedCopies - 1)) << 2;
}

// Load the cursor's task: its code words (2k per lane) and scale. Past the
// wave's last task it re-reads that task: every load is unconditional, so the
// compiler's memory-counter waits never have to cover a skipped load.
template <int K, bool PAIRS, bool MIXED = false, bool FOLD = false, bool SPLIT = false>
__device__ __forceinline__ void load_task(Task<K>& t, const TaskCtx& cx, TaskCursor& k, int tau_end) {
    int b, g;
    task_place<FOLD, SPLIT>(cx, k, tau_end, b, g, t.fold);
    bool second;
    int rc = task_row<MIXED, SPLIT>(cx, g, t.valid, second);
    int bl = b;
    if (FOLD && t.fold) fold_lane(cx, g, b, rc, bl, t.valid);
    t.b = b;
    t.g = g;
    if constexpr (MIXED) t.sel = (second ? kMixedSpan : 0u) | mixed_copy_offset();
    const uint32_t* codes = second ? cx.codes_b : cx.codes;
    const float* scales = second ? cx.scales_b : cx.scales;
    load_run64_words<K>(codes + task_word<K, PAIRS>(cx, rc, bl), cx.cp, t.w);
    t.scale = scales[rc];
    if (FOLD && t.fold && !t.valid) t.scale = 0.f;
}

// load_task through opaque global-address-space pointers, for the prologue:
// through the restrict kernel pointers the loads count as invariant and the
// compiler sinks them past the table stores and the barrier to their first
// use, so the table stores and the code words no longer overlap.
template <int K, bool PAIRS, bool MIXED = false, bool FOLD = false, bool SPLIT = false>
__device__ __forceinline__ void load_task_opaque(Task<K>& t, const TaskCtx& cx, TaskCursor& k,
                                                 int tau_end) {
    using gu32 = const __attribute__((address_space(1))) uint32_t*;
    using gu32x4 = const __attribute__((address_space(1))) u32x4*;
    using gf32 = const __attribute__((address_space(1))) float*;
    gu32 codes_a = (gu32)cx.codes;  // generic to global: an address-space cast
    gf32 scales_a = (gf32)cx.scales;
    gu32 codes_b = (gu32)cx.codes_b;
    gf32 scales_b = (gf32)cx.scales_b;
    asm volatile("" : "+s"(codes_a), "+s"(scales_a), "+s"(codes_b), "+s"(scales_b));
    int b, g;
    task_place<FOLD, SPLIT>(cx, k, tau_end, b, g, t.fold);
    bool second;
    int rc = task_row<MIXED, SPLIT>(cx, g, t.valid, second);
    int bl = b;
    if (FOLD && t.fold) fold_lane(cx, g, b, rc, bl, t.valid);
    t.b = b;
    t.g = g;
    if constexpr (MIXED) t.sel = (second ? kMixedSpan : 0u) | mixed_copy_offset();
    const gu32 codes = second ? codes_b : codes_a;
    const gf32 scales = second ? scales_b : scales_a;
    const gu32 p = codes + task_word<K, PAIRS>(cx, rc, bl) + 2 * K * cx.cp;
    if constexpr (K == 2) {
        const u32x4 v = *reinterpret_cast<gu32x4>(p);
        t.w[0] = v.x; t.w[1] = v.y; t.w[2] = v.z; t.w[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < 2 * K; ++i) t.w[i] = p[i];
    }
    t.scale = scales[rc];
    if (FOLD && t.fold && !t.valid) t.scale = 0.f;
}

template <int MT>
struct XFrags {
    u32x4 v[MT][8];
};

// Direct path: activation fragments of block b in A layout. A fragment S of
// lane (j, c) is x[m = 16 mt + j][256 b + 64 c + 8 S .. + 8] (the weights
// 64 c + 8 S + e are the ones that lane decodes); xa[mt] points at row m (row
// M - 1 for m >= M: row m of A only feeds row m of D, which is never stored
// for m >= M), column 64 c.
template <int MT>
__device__ __forceinline__ void load_x_frags(XFrags<MT>& xn, const uint16_t* const (&xa)[MT], int b) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int S = 0; S < 8; ++S)
            xn.v[mt][S] = *reinterpret_cast<const u32x4*>(xa[mt] + b * kT + 8 * S);
}

// The same through an opaque global-address-space pointer, for the prologue
// (see load_task_opaque).
template <int MT>
__device__ __forceinline__ void load_x_frags_opaque(XFrags<MT>& xn, const uint16_t* const (&xa)[MT],
                                                    int b) {
    using gu32x4 = const __attribute__((address_space(1))) u32x4*;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        gu32x4 p = (gu32x4)(xa[mt] + b * kT);
        asm volatile("" : "+v"(p));
#pragma unroll
        for (int S = 0; S < 8; ++S) xn.v[mt][S] = p[S];
    }
}

// Staged path: activation fragments of block b for a wave, the same A layout
// as load_x_frags, i.e. chunk S of 128-byte line c of the row's block. Fetched
// directly, each instruction would touch 64 cache lines (16 rows x 4 lines),
// which measured slower than staging from M = 16 up. Instead instruction
// (c, h) reads line c of rows 8h .. 8h + 7 (8 lanes per line, coalesced) and
// the lines pass through the wave's LDS slot to the lanes of group c: all
// four at once when the slot holds them, else two lines of one M tile at a
// time (half the lanes read per round). Chunk S of row r
// of a line sits at slot chunk 8 r + (S ^ (r & 7)), so the writes are
// conflict-free and the reads at most 2-way.
template <int MT, int LINES>
__device__ __forceinline__ void load_x_block(XFrags<MT>& xf, u32x4* __restrict__ slot,
                                             const uint16_t* const (&xrows)[MT][2], int b,
                                             int lane, int j, int c) {
    const int wr = lane >> 3, ws = lane & 7;  // row within the half and chunk this lane loaded
    if constexpr (LINES == 4) {
        u32x4 raw[MT][4][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int line = 0; line < 4; ++line)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    raw[mt][line][h] =
                        *reinterpret_cast<const u32x4*>(xrows[mt][h] + b * kT + 64 * line);
        wave_lds_sync();  // the previous block's reads of the slot come first
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int line = 0; line < 4; ++line)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 8 * h + wr;
                    slot[((mt * 4 + line) * 16 + r) * 8 + (ws ^ (r & 7))] = raw[mt][line][h];
                }
        wave_lds_sync();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int S = 0; S < 8; ++S)
                xf.v[mt][S] = slot[((mt * 4 + c) * 16 + j) * 8 + (S ^ (j & 7))];
        return;
    }
    // A one-line slot of both M tiles holds two lines of one: two lines are
    // fetched at a time, then pass through the slot one M tile at a time, so
    // that half the lanes (the two lines' groups) read at each round.
    // (the slot holds two lines of 16 rows: the one-line slot of two M tiles,
    // or the prologue area of one)
#pragma unroll
    for (int l0 = 0; l0 < 4; l0 += 2) {
        u32x4 raw[MT][2][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int dl = 0; dl < 2; ++dl)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    raw[mt][dl][h] =
                        *reinterpret_cast<const u32x4*>(xrows[mt][h] + b * kT + 64 * (l0 + dl));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            wave_lds_sync();  // earlier reads of the slot come first
#pragma unroll
            for (int dl = 0; dl < 2; ++dl)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 8 * h + wr;
                    slot[(dl * 16 + r) * 8 + (ws ^ (r & 7))] = raw[mt][dl][h];
                }
            wave_lds_sync();
            if ((c >> 1) == (l0 >> 1)) {
                const int dl = c - l0;
#pragma unroll
                for (int S = 0; S < 8; ++S) xf.v[mt][S] = slot[(dl * 16 + j) * 8 + (S ^ (j & 7))];
            }
        }
    }
}

// A wave's accumulator tiles: per M tile, groups [0, 5) in one array and the
// rest (the nine-group launches) in another, so that a uniform dynamic group
// index into any of them stays in registers (a larger indexed array the
// compiler keeps in scratch memory). Tile 1's arrays are unused with one tile.
template <int KG>
struct AccShape {
    static constexpr int lo = KG < kGroups ? KG : kGroups;
    static constexpr int hi = KG - lo > 0 ? KG - lo : 1;
};
#define TRELLIS_ACC_PARAMS(KG)                                                      \
    floatx4 (&al0)[AccShape<KG>::lo], floatx4 (&al1)[AccShape<KG>::lo],            \
        floatx4 (&ah0)[AccShape<KG>::hi], floatx4 (&ah1)[AccShape<KG>::hi]
// Group g (known at compile time once loops unroll), tile mt.
template <int KG>
__device__ __forceinline__ floatx4& acc_at(TRELLIS_ACC_PARAMS(KG), int g, int mt) {
    constexpr int lo = AccShape<KG>::lo;
    return g < lo ? (mt == 0 ? al0[g] : al1[g]) : (mt == 0 ? ah0[g - lo] : ah1[g - lo]);
}

// Which blocks a wave's fragment sets hold: xf block b, xn block lb (direct
// path).
struct XCursor {
    int b = -1;
    int lb = -1;
};

// Where a wave's activation fragments come from (see the two paths above).
template <int MT>
struct XSource {
    const uint16_t* xrows[MT][2];  // staged: coalesced row pointers
    const uint16_t* xa[MT];        // direct: A-layout row pointers
    u32x4* slot;                   // staged: this wave's LDS slot
    int nb;
    bool hi;                       // folding kernel, lanes j >= 8 (see lane_block)
};

// The block whose activations a lane's direct fragments for block b hold. In
// the folding kernel lanes j >= 8 (A rows 8-15) hold rows 0-7 of block b + 1
// (of b itself at the last block), so a folded task multiplies the fragments
// as they are; every other task leaves D rows 8-15 unused (M <= 8).
template <int MT>
__device__ __forceinline__ int lane_block(const XSource<MT>& xs, int b) {
    return b + (xs.hi && b + 1 < xs.nb ? 1 : 0);
}

// One task: eight fragments, the gathers of the next two in flight while one is
// packed and multiplied against the MT activation tiles. A new block first
// refreshes the activation fragments. Direct path: xf takes xn; xn is fetched
// one task ahead, by the task before one that enters a new block (tn is the
// wave's next task), so the loads have a whole task to arrive. (Fetching the
// next block at the block change itself, the compiler issued the loads ahead
// of the move into temporaries and copied those into xn at once, i.e. waited
// for the loads it had just issued: 6-10% of the kernel.) A block a wave enters
// unannounced (its first) is fetched at once. Staged path: through the LDS
// slot, the one memory wait that covers the prefetched code words.
// MIXED (staged activations, k = 3, 4): each lane reads its copy of the
// codebook of its row's projection (Task::sel), beside a one-line slot.
template <int K, int MT, bool DIRECT, int KG, bool MIXED = false, bool FOLD = false>
__device__ __forceinline__ void run_task(Task<K> t, const Task<K>& tn, XFrags<MT>& xf,
                                         XFrags<MT>& xn, XCursor& xc,
                                         const XSource<MT>& xs, TRELLIS_ACC_PARAMS(KG),
                                         const float* __restrict__ tab, int lane, int j, int c) {
    static_assert(!MIXED || (K != 2 && !DIRECT), "mixed groups read two plain codebooks");
    constexpr bool P = PrefillLds<K, MT, DIRECT>::pair;
    constexpr bool REP = PrefillLds<K, MT, DIRECT>::rep;
    constexpr int kLines = MIXED ? kMixedLines : PrefillLds<K, MT, DIRECT>::lines;
    // (Distinct empty asm statements open and close each fetch, so that the
    // compiler neither hoists its loads above the branch nor merges fetches
    // into one through a selected address.)
    if (t.b != xc.b) {
        if constexpr (DIRECT) {
            if (xc.lb == t.b) {
                xf = xn;
            } else {
                asm volatile("; x fetch now");
                load_x_frags<MT>(xf, xs.xa, lane_block(xs, t.b));
                // wait here, on this path only: after the branches the
                // compiler's wait for xf would also cover a fetch ahead
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int S = 0; S < 8; ++S) asm volatile("; x fetch now done" : : "v"(xf.v[mt][S]));
            }
        } else {
            load_x_block<MT, kLines>(xf, xs.slot, xs.xrows, t.b, lane, j, c);
        }
        xc.b = t.b;
    }
    if constexpr (DIRECT) {
        if (tn.b != t.b && tn.b != xc.lb) {
            asm volatile("; x fetch ahead");
            load_x_frags<MT>(xn, xs.xa, lane_block(xs, tn.b));
            asm volatile("; x fetch ahead done");
            xc.lb = tn.b;
        }
    }
    if (!t.valid) {
#pragma unroll
        for (int i = 0; i < 2 * K; ++i) t.w[i] = 0u;
    }
    t.w[2 * K] = next_run_word(t.w[0]);
    // The group's accumulators move into cur and back by a uniform register
    // index (s_set_gpr_idx moves) into its array; nine groups pick the array
    // under one uniform branch (distinct asm markers keep the two sides from
    // merging into a selected address). One uniform branch per group and
    // direction instead measured 1-5% slower; it remains for nine groups of two
    // M tiles, whose indexed arrays the compiler partly keeps in scratch memory
    // (the empty asm keeps each a branch: as selects they cost 36 VALU per
    // task).
    constexpr int kLo = AccShape<KG>::lo;
    constexpr bool kIndexed = !(MT == 2 && KG > kGroups);
    floatx4 cur[MT];
    if constexpr (!kIndexed) {
        static_for<0, KG>([&](auto gc) {
            constexpr int G = decltype(gc)::value;
            if (t.g == G) {
                asm volatile("");
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) cur[mt] = acc_at<KG>(al0, al1, ah0, ah1, G, mt);
            }
        });
    } else if (KG <= kLo || t.g < kLo) {
        asm volatile("; acc lo in");
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) cur[mt] = mt == 0 ? al0[t.g] : al1[t.g];
        asm volatile("; acc lo in done");
    } else {
        asm volatile("; acc hi in");
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) cur[mt] = mt == 0 ? ah0[t.g - kLo] : ah1[t.g - kLo];
        asm volatile("; acc hi in done");
    }
    // Fragments 7 .. 0: only fragment 0 reads the word from the neighbouring
    // lane, which thus has the whole task to arrive.
    auto gather = [&](auto sc) {
        constexpr int S = decltype(sc)::value;
        if constexpr (MIXED) return gather_run64_sel<K, S, kMixedCopies>(t.w, tab, t.sel);
        else return gather_tab<K, S, P, REP>(t.w, tab);
    };
    Gathered<P> g0 = gather(std::integral_constant<int, 7>{});
    Gathered<P> g1 = gather(std::integral_constant<int, 6>{});
    static_for<0, 8>([&](auto ic) {
        constexpr int S = 7 - decltype(ic)::value;
        Gathered<P> g2;
        __builtin_amdgcn_s_setprio(2);  // the gathers issue at raised priority
        if constexpr (S >= 2) g2 = gather(std::integral_constant<int, S - 2>{});
        __builtin_amdgcn_s_setprio(0);
        const bf16x8 bfrag = as_bf16x8(pack_fragment<P>(g0, t.scale));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            cur[mt] = mfma16x16x32(as_bf16x8(xf.v[mt][S]), bfrag, cur[mt]);
        g0 = g1;
        if constexpr (S >= 2) g1 = g2;
    });
    if constexpr (!kIndexed) {
        static_for<0, KG>([&](auto gc) {
            constexpr int G = decltype(gc)::value;
            if (t.g == G) {
                asm volatile("");
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc_at<KG>(al0, al1, ah0, ah1, G, mt) = cur[mt];
            }
        });
    } else if (KG <= kLo || t.g < kLo) {
        asm volatile("; acc lo out");
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) (mt == 0 ? al0[t.g] : al1[t.g]) = cur[mt];
        asm volatile("; acc lo out done");
    } else {
        asm volatile("; acc hi out");
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) (mt == 0 ? ah0[t.g - kLo] : ah1[t.g - kLo]) = cur[mt];
        asm volatile("; acc hi out done");
    }
}

// Balanced plan of the single-projection launch (SPLIT). With ng 16-row
// groups over G workgroups, each workgroup owns f = ng / G full groups, and
// the L = ng % G leftover groups are each cut into p = G / L block ranges, one
// per workgroup, so every workgroup decodes f nb + nb / p tasks instead of
// (f + 1) nb. The parts of a leftover group meet through the workspace,
// without counters or cache maintenance.
// Each value travels as one 64-bit word, the call's tag above the float's
// bits, stored and loaded with device-scope relaxed atomics (performed at the
// device's coherence point, past the per-XCD L2; a 64-bit atomic is never
// torn). A part stores its tile once its split tasks are done, goes on, and
// at the end of its tasks waits for those stores and loads every part of
// its group: if every word carries the tag, it sums them. The part that
// checks last sees the others' stores, which completed before their own
// checks, so at least one part sums; parts that find all words current at
// the same time write the same bits. Words of another call, or whatever the
// workspace held, carry another tag (tags repeat after 2^32 calls; each
// slot's expected tag differs, see slot_tag). A graph replay would reuse its
// tag, so captured calls take the plan without the split.
constexpr int kSplitMaxParts = 8;  // parts per leftover group, at most

struct SplitArgs {
    unsigned long long* part;  // per workgroup: its part's tile, MT x 64 lanes x 4 tagged words
    unsigned int tag;          // this call's tag (never 0)
    int f;                     // full groups per workgroup
    int p;                     // parts per leftover group
    int pen;                   // tasks wave 0 takes fewer than an equal share
};

// silu(v) = v / (1 + e^-v) in float32: the gate nonlinearity of SwiGLU.
__device__ __forceinline__ float silu_f32(float v) { return v / (1.0f + expf(-v)); }

// Two projections of the same geometry over the same activation rows (an
// MLP's gate and up) can share one launch.
//   Without SWIGLU, workgroups below G0 compute y_a from (codes_a, scales_a,
//   lut_a), the others y_b from the b operands, each half splitting its rows
//   as one launch of its own would; a single projection passes G0 = gridDim.x.
//   With SWIGLU (G0 = gridDim.x) every workgroup owns a row range of both: it
//   runs its tasks on the gate (a operands), reduces the waves' tiles and keeps
//   each output's gate sum in the register of the thread that reduced it,
//   restages the table from the up codebook, runs the same tasks on the up
//   projection (b operands) and writes y_a[m][n] = bf16(silu(g) * u), the same
//   thread reducing the same output in both phases.
template <int K, int MT, bool DIRECT, bool PAIRS, int KG, bool SWIGLU, bool FOLD, bool SPLIT,
          bool STAGE1 = false>
__global__ __launch_bounds__(PrefillShape<MT>::threads) void axis1_prefill_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes_a,
    const float* __restrict__ scales_a, const float* __restrict__ lut_a,
    uint16_t* __restrict__ y_a, const uint32_t* __restrict__ codes_b,
    const float* __restrict__ scales_b, const float* __restrict__ lut_b,
    uint16_t* __restrict__ y_b, int G0, CodeLayout lay, int N, int nb, int M, SplitArgs sp) {
    static_assert(!SPLIT || (!SWIGLU && !FOLD), "the split plan serves the single projection");
    static_assert(!STAGE1 || (DIRECT && !FOLD), "the staged first block serves the direct layout");
    constexpr int kThreadsP = PrefillShape<MT>::threads, kWaves = PrefillShape<MT>::waves;
    using Lds = PrefillLds<K, MT, DIRECT, KG>;
    __shared__ __attribute__((aligned(16))) float lds[Lds::floats];
    float* const tab = lds;

    const bool second = !SWIGLU && static_cast<int>(blockIdx.x) >= G0;
    const uint32_t* const codes = second ? codes_b : codes_a;
    const float* const scales = second ? scales_b : scales_a;
    const float* const lut = second ? lut_b : lut_a;
    uint16_t* const y = second ? y_b : y_a;
    const int G = second ? static_cast<int>(gridDim.x) - G0 : G0;
    const int wg = second ? static_cast<int>(blockIdx.x) - G0 : static_cast<int>(blockIdx.x);
    // Split plan: sp.f full groups per workgroup, then part q of leftover
    // group ell (blocks [q nb / p, (q + 1) nb / p)).
    const int r0 = SPLIT ? 16 * sp.f * wg : static_cast<int>(static_cast<long>(wg) * N / G);
    const int r1 = SPLIT ? r0 + 16 * sp.f : static_cast<int>(static_cast<long>(wg + 1) * N / G);
    const int ell = SPLIT ? wg / sp.p : 0, q = SPLIT ? wg - ell * sp.p : 0;
    const int qb0 = SPLIT ? q * nb / sp.p : 0;
    const int nq = SPLIT ? (q + 1) * nb / sp.p - qb0 : 0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, c = lane >> 4, cp = 3 - c;
    const int gc = (r1 - r0 + 15) >> 4;  // full or own groups in this workgroup, <= KG
    // Folding (task_place): direct fragments, one M tile, M <= 8, a last group
    // of at most 8 rows after at least one full group.
    const bool fold = FOLD && M <= 8 && gc >= 2 && r1 - r0 - 16 * (gc - 1) <= 8;
    const int tasks = SPLIT ? nq + gc * nb : fold ? (nb >> 1) * (2 * gc - 1) + (nb & 1) * gc : gc * nb;
    // Wave w takes tasks [w V / 8, (w + 1) V / 8) - pen, V = tasks + pen: with
    // the split plan wave 0 publishes its part mid-way (memory round trips it
    // waits for), so it takes pen tasks fewer than an equal share.
    const int pen = SPLIT ? sp.pen : 0;
    const int vt = tasks + pen;
    const int tau0 = wave == 0 ? 0 : static_cast<int>(static_cast<long>(wave) * vt / kWaves) - pen;
    const int tau1 = static_cast<int>(static_cast<long>(wave + 1) * vt / kWaves) - pen;
    const long in = static_cast<long>(nb) * kT;

    // Staged path, coalesced activation rows: half h of tile mt is rows
    // 16 mt + 8 h + lane / 8, lane % 8 the 16-byte chunk within a line. Direct
    // path: lane (j, c) reads row 16 mt + j from column 64 c of each block.
    // A rows past M read row M - 1: row m of A only feeds row m of D, which is
    // never stored for m >= M.
    XSource<MT> xs;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = 16 * mt + 8 * h + (lane >> 3);
            xs.xrows[mt][h] = x + (m < M ? m : M - 1) * in + 8 * (lane & 7);
        }
        // (folding kernel: row j & 7 in both halves of A, see lane_block)
        const int m = FOLD ? (j & 7) : 16 * mt + j;
        xs.xa[mt] = x + (m < M ? m : M - 1) * in + 64 * c;
    }
    xs.slot = reinterpret_cast<u32x4*>(lds + Lds::tab_floats) + wave * Lds::slot_chunks;
    xs.nb = nb;
    xs.hi = FOLD && j >= 8;

    TaskCtx cx{codes, lay, scales, nb, gc > 0 ? gc : 1, r0, r1, j, cp, codes, scales, 0,
               fold ? gc - 1 : -1};
    if constexpr (SPLIT) {
        cx.nq = nq;
        cx.qb0 = qb0;
        cx.bs = MT == 2 ? qb0 + nq - 1 : 0;  // measured: staged activations gain, direct ones not
        cx.rs = 16 * (sp.f * G + ell);
        cx.rn = N;
    }
    // the wave whose range holds the split tasks (wave 0; the launcher keeps
    // them within its share) publishes the part after its last one
    const int split_last = SPLIT && tau0 == 0 ? nq - 1 : -1;
    floatx4 al0[AccShape<KG>::lo], al1[AccShape<KG>::lo], ah0[AccShape<KG>::hi], ah1[AccShape<KG>::hi];
#pragma unroll
    for (int g = 0; g < KG; ++g)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc_at<KG>(al0, al1, ah0, ah1, g, mt) = floatx4{0.f, 0.f, 0.f, 0.f};

    // Prologue: the codebook first, then the first two tasks' code words and,
    // on the direct path, the first block's activation fragments
    // (unconditionally: a wave without tasks re-reads a valid one, and a load
    // under a branch would make the table stores wait for the code words too).
    typename Lds::Table::Src tsrc;
    Lds::Table::fetch(tsrc, lut);
    asm volatile("" ::: "memory");
    Task<K> ta, tb, tc;
    const int tend = tau1 > 1 ? tau1 : 1;  // a wave without tasks re-reads a valid one
    TaskCursor cur = task_cursor<FOLD, SPLIT>(cx, tau0, tend);
    load_task_opaque<K, PAIRS, false, FOLD, SPLIT>(ta, cx, cur, tend);
    load_task_opaque<K, PAIRS, false, FOLD, SPLIT>(tb, cx, cur, tend);
    XFrags<MT> xn;
    // The first block's fragments: loaded directly here, or (STAGE1, M > 8,
    // where a direct load touches 64 cache lines per instruction) coalesced
    // through this wave's LDS area after the barrier.
    constexpr bool kStagedFirst = STAGE1;
    if constexpr (DIRECT && !kStagedFirst) load_x_frags_opaque<MT>(xn, xs.xa, lane_block(xs, ta.b));
    asm volatile("" ::: "memory");
    Lds::Table::store(tsrc, tab);
    __syncthreads();
    if constexpr (kStagedFirst) {
        u32x4* const area = reinterpret_cast<u32x4*>(lds + Lds::tab_floats) + wave * Lds::pro_chunks;
        load_x_block<MT, 2>(xn, area, xs.xrows, ta.b, lane, j, c);
    }

    // Three register sets rotate: the words of the next two tasks are in
    // flight while one is decoded. (No branch around the loop: the prologue's
    // loads would be sunk into it, behind the barrier.)
    XFrags<MT> xf;
    XCursor xc;
    xc.lb = ta.b;  // the prologue's fetch
    // Split plan, in two steps of the wave that ran the split tasks (see
    // SplitArgs): after them it stores its part's tile (slot gc) to the
    // workspace, [wg][mt][lane][4] tagged words in D layout, and goes on;
    // after its last task it checks its group's parts and, if all are
    // current, sums them in part order and writes the group's rows of y. The
    // wave takes a task or two fewer than the others (SplitArgs::pen), which
    // covers the round trip.
    auto split_tile = [&](floatx4 (&mine)[MT]) {
        // slot gc by uniform branches on constant indices: a dynamic index
        // would move the accumulator arrays to scratch memory
        static_for<0, KG>([&](auto gi) {
            constexpr int Gs = decltype(gi)::value;
            if (gc == Gs) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) mine[mt] = acc_at<KG>(al0, al1, ah0, ah1, Gs, mt);
            }
        });
    };
    auto split_store = [&]() {
        floatx4 mine[MT];
        split_tile(mine);
        unsigned long long* const own = sp.part + (static_cast<size_t>(wg) * MT * kWave + lane) * 4;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                __hip_atomic_store(own + mt * kWave * 4 + v, tagged_word(slot_tag(sp.tag, wg), mine[mt][v]),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto split_finish = [&]() {
        __builtin_amdgcn_s_waitcnt(0);  // this part's stores complete before the check
        // every part of the group, all loads in flight together (parts past
        // p re-read this one and are not used)
        unsigned long long w[kSplitMaxParts][MT][4];
#pragma unroll
        for (int pq = 0; pq < kSplitMaxParts; ++pq) {
            unsigned long long* src =
                sp.part + (static_cast<size_t>(ell * sp.p + (pq < sp.p ? pq : q)) * MT * kWave + lane) * 4;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    w[pq][mt][v] = __hip_atomic_load(src + mt * kWave * 4 + v, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        }
        bool stale = false;
#pragma unroll
        for (int pq = 0; pq < kSplitMaxParts; ++pq)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    stale |= pq < sp.p &&
                             static_cast<unsigned int>(w[pq][mt][v] >> 32) != slot_tag(sp.tag, ell * sp.p + pq);
        if (__builtin_amdgcn_ballot_w64(stale) != 0) return;  // a later part sums
        floatx4 mine[MT];
        split_tile(mine);
        floatx4 sum[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sum[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pq = 0; pq < kSplitMaxParts; ++pq)
            if (pq < sp.p) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        sum[mt][v] += pq == q ? mine[mt][v]
                                              : __uint_as_float(static_cast<unsigned int>(w[pq][mt][v]));
            }
        // D[4 c + v][j] of tile mt: activation row 16 mt + 4 c + v, weight row rs + j
        const int row = cx.rs + j;
        if (row < N) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 16 * mt + 4 * c + v;
                    if (m < M) y[static_cast<size_t>(m) * N + row] = round_bf16(sum[mt][v]);
                }
        }
    };
    auto run_tasks = [&]() {
        for (int t0 = tau0; t0 < tau1; t0 += 3) {
            load_task<K, PAIRS, false, FOLD, SPLIT>(tc, cx, cur, tend);
            run_task<K, MT, DIRECT, KG, false, FOLD>(ta, tb, xf, xn, xc, xs, al0, al1, ah0, ah1, tab, lane, j, c);
            load_task<K, PAIRS, false, FOLD, SPLIT>(ta, cx, cur, tend);
            if (t0 + 1 < tau1)
                run_task<K, MT, DIRECT, KG, false, FOLD>(tb, tc, xf, xn, xc, xs, al0, al1, ah0, ah1, tab, lane, j, c);
            load_task<K, PAIRS, false, FOLD, SPLIT>(tb, cx, cur, tend);
            if (t0 + 2 < tau1)
                run_task<K, MT, DIRECT, KG, false, FOLD>(tc, ta, xf, xn, xc, xs, al0, al1, ah0, ah1, tab, lane, j, c);
            if constexpr (SPLIT) {
                // once the batch holding the last split task is done
                if (split_last >= t0 && split_last < t0 + 3) split_store();
            }
        }
    };
    run_tasks();
    if constexpr (SPLIT) {
        if (split_last >= 0) split_finish();
    }
    __syncthreads();  // the table is dead from here on; its space takes the partials

    // part[wave][group][m][j]: D[m = 4c + v][j] of each tile; untouched groups
    // add zeros. Output (16 mt + m, row) is reduced by thread idx % 512 in
    // pass idx / 512, idx = (group * 16 + m) * 16 + j, the waves added in order
    // (for a folded group, then the waves' second-block quarter).
    float* const part = lds;
    constexpr int kPasses = (KG * 256 + kThreadsP - 1) / kThreadsP;
    auto reduce = [&](auto&& sink) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int g = 0; g < KG; ++g)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    part[((wave * KG + g) * 16 + 4 * c + v) * 16 + j] = acc_at<KG>(al0, al1, ah0, ah1, g, mt)[v];
            __syncthreads();
#pragma unroll
            for (int it = 0; it < kPasses; ++it) {
                const int idx = tid + it * kThreadsP;
                if (idx < gc * 256) {
                    const int g = idx >> 8, m = (idx >> 4) & 15, jj = idx & 15;
                    float s = 0.f;
                    for (int w = 0; w < kWaves; ++w) s += part[((w * KG + g) * 16 + m) * 16 + jj];
                    // a folded group: block b + 1's quarter of D for the same row
                    if (fold && g == gc - 1 && m < 8 && jj < 8)
                        for (int w = 0; w < kWaves; ++w)
                            s += part[((w * KG + g) * 16 + 8 + m) * 16 + 8 + jj];
                    sink(mt, it, 16 * mt + m, r0 + 16 * g + jj, s);
                }
            }
            __syncthreads();
        }
    };
    if constexpr (SWIGLU) {
        float gsum[MT][kPasses];
        reduce([&](int mt, int it, int, int, float s) { gsum[mt][it] = s; });
        // The up projection: its codebook and first tasks, as in the prologue.
        cx.codes = codes_b;
        cx.scales = scales_b;
        typename Lds::Table::Src ts;
        Lds::Table::fetch(ts, lut_b);
        asm volatile("" ::: "memory");
        cur = task_cursor<FOLD>(cx, tau0, tend);
        load_task_opaque<K, PAIRS, false, FOLD>(ta, cx, cur, tend);
        load_task_opaque<K, PAIRS, false, FOLD>(tb, cx, cur, tend);
        if constexpr (DIRECT) load_x_frags_opaque<MT>(xn, xs.xa, lane_block(xs, ta.b));
        asm volatile("" ::: "memory");
        Lds::Table::store(ts, tab);
#pragma unroll
        for (int g = 0; g < KG; ++g)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc_at<KG>(al0, al1, ah0, ah1, g, mt) = floatx4{0.f, 0.f, 0.f, 0.f};
        xc = XCursor{};
        xc.lb = ta.b;
        __syncthreads();
        run_tasks();
        __syncthreads();
        reduce([&](int mt, int it, int mm, int row, float s) {
            if (mm < M && row < r1)
                y[static_cast<size_t>(mm) * N + row] = round_bf16(silu_f32(gsum[mt][it]) * s);
        });
    } else {
        reduce([&](int, int, int mm, int row, float s) {
            if (mm < M && row < r1) y[static_cast<size_t>(mm) * N + row] = round_bf16(s);
        });
    }
}

// Gate and up with the SwiGLU epilogue at k = 3, 4 and two M tiles (M = 17..32),
// in mixed groups. Both projections read the same activations, so a 16-row
// MFMA group may hold rows of either as long as each lane reads its own row's
// codebook: the two codebooks, each in four bank-partitioned copies (64 KB),
// sit one after the other in LDS and a lane's gather offset carries its
// projection and its copy (Task::sel). A workgroup owns rows [r0, r1) of both,
// rm <= 72 of them, i.e. 2 rm virtual rows in at most kDualGroups groups --
// the slot count of the dual launch, where the two-phase kernel runs two
// rounds of five -- with the one-line activation slots beside the codebooks
// (160 KB). (Two plain codebooks with four-line slots measured 1.2% slower at
// k = 4, M = 32.) The waves' tiles are reduced as in the prefill
// epilogue; output (m, i) is bf16(silu(g) * u) with g the sum of virtual row
// i and u that of virtual row rm + i.
constexpr int kMixedRows = 16 * kDualGroups / 2;  // rows of each projection per workgroup

struct MixedLds {
    static constexpr int threads = 512, waves = threads / kWave, MT = 2;
    static constexpr int tab_floats = 2 * kLutEntries * kMixedCopies;
    static constexpr int slot_chunks = MT * kMixedLines * 16 * 8;
    static constexpr int decode_floats = tab_floats + waves * slot_chunks * 4;
    static constexpr int part_floats = waves * kDualGroups * 256;
    static constexpr int floats = decode_floats > part_floats ? decode_floats : part_floats;
    static_assert(floats * 4 <= 160 * 1024, "fits the CU's LDS");
};

template <int K, bool PAIRS>
__global__ __launch_bounds__(MixedLds::threads) void axis1_swiglu_mixed_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes_g,
    const float* __restrict__ scales_g, const float* __restrict__ lut_g,
    const uint32_t* __restrict__ codes_u, const float* __restrict__ scales_u,
    const float* __restrict__ lut_u, uint16_t* __restrict__ h, CodeLayout lay, int N, int nb,
    int M) {
    constexpr int MT = 2, KG = kDualGroups, kWaves = MixedLds::waves;
    constexpr int kThreadsP = MixedLds::threads;
    __shared__ __attribute__((aligned(16))) float lds[MixedLds::floats];
    float* const tab = lds;

    const int G = static_cast<int>(gridDim.x), wg = static_cast<int>(blockIdx.x);
    const int r0 = static_cast<int>(static_cast<long>(wg) * N / G);
    const int r1 = static_cast<int>(static_cast<long>(wg + 1) * N / G);
    const int rm = r1 - r0;  // 1 <= rm <= kMixedRows (the launcher's grid)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, c = lane >> 4, cp = 3 - c;
    const int gc = (2 * rm + 15) >> 4;
    const int tasks = gc * nb;
    const int tau0 = static_cast<int>(static_cast<long>(wave) * tasks / kWaves);
    const int tau1 = static_cast<int>(static_cast<long>(wave + 1) * tasks / kWaves);
    const long in = static_cast<long>(nb) * kT;

    XSource<MT> xs;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int m = 16 * mt + 8 * hh + (lane >> 3);
            xs.xrows[mt][hh] = x + (m < M ? m : M - 1) * in + 8 * (lane & 7);
        }
        const int m = 16 * mt + j;
        xs.xa[mt] = x + (m < M ? m : M - 1) * in + 64 * c;
    }
    xs.slot = reinterpret_cast<u32x4*>(lds + MixedLds::tab_floats) + wave * MixedLds::slot_chunks;
    xs.nb = nb;
    xs.hi = false;

    TaskCtx cx{codes_g, lay, scales_g, nb, gc, r0, r1, j, cp, codes_u, scales_u, rm};
    floatx4 al0[AccShape<KG>::lo], al1[AccShape<KG>::lo], ah0[AccShape<KG>::hi], ah1[AccShape<KG>::hi];
#pragma unroll
    for (int g = 0; g < KG; ++g)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc_at<KG>(al0, al1, ah0, ah1, g, mt) = floatx4{0.f, 0.f, 0.f, 0.f};

    // Prologue: both codebooks, then the first two tasks' code words; the
    // codebook stores wait only for their own data.
    RepSrc<kThreadsP> src_g, src_u;  // 8 entries of each codebook per thread
    fetch_rep<kThreadsP>(src_g, lut_g);
    fetch_rep<kThreadsP>(src_u, lut_u);
    asm volatile("" ::: "memory");
    Task<K> ta, tb, tc;
    const int tend = tau1 > 1 ? tau1 : 1;
    TaskCursor cur = task_cursor<false>(cx, tau0, tend);
    load_task_opaque<K, PAIRS, true>(ta, cx, cur, tend);
    load_task_opaque<K, PAIRS, true>(tb, cx, cur, tend);
    asm volatile("" ::: "memory");
    {
        constexpr int R = kMixedCopies, span = kMixedSpan / 4;  // floats per codebook
#pragma unroll
        for (int i = 0; i < RepSrc<kThreadsP>::n; ++i) {
            const int e = tid + kThreadsP * i;
            const float a = src_g.a[i], b = src_u.a[i];
            if constexpr (R == 1) {
                tab[e] = a;
                tab[span + e] = b;
            } else if constexpr (R == 4) {
                *reinterpret_cast<float4*>(tab + 4 * e) = float4{a, a, a, a};
                *reinterpret_cast<float4*>(tab + span + 4 * e) = float4{b, b, b, b};
            } else {
                static_assert(R == 1 || R == 4, "staged for one or four copies");
            }
        }
    }
    __syncthreads();

    XFrags<MT> xf, xn;
    XCursor xc;
    for (int t0 = tau0; t0 < tau1; t0 += 3) {
        load_task<K, PAIRS, true>(tc, cx, cur, tend);
        run_task<K, MT, false, KG, true>(ta, tb, xf, xn, xc, xs, al0, al1, ah0, ah1, tab, lane, j, c);
        load_task<K, PAIRS, true>(ta, cx, cur, tend);
        if (t0 + 1 < tau1) run_task<K, MT, false, KG, true>(tb, tc, xf, xn, xc, xs, al0, al1, ah0, ah1, tab, lane, j, c);
        load_task<K, PAIRS, true>(tb, cx, cur, tend);
        if (t0 + 2 < tau1) run_task<K, MT, false, KG, true>(tc, ta, xf, xn, xc, xs, al0, al1, ah0, ah1, tab, lane, j, c);
    }
    __syncthreads();  // the tables and slots are dead from here on

    // part[wave][group][m][j] as in the prefill epilogue; then the thread of
    // output (16 mt + m, i) sums the waves' tiles of gate virtual row i and up
    // virtual row rm + i and writes h.
    float* const part = lds;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int g = 0; g < KG; ++g)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                part[((wave * KG + g) * 16 + 4 * c + v) * 16 + j] = acc_at<KG>(al0, al1, ah0, ah1, g, mt)[v];
        __syncthreads();
        for (int o = tid; o < 16 * rm; o += kThreadsP) {
            const int m = o / rm, i = o - m * rm;
            const int u = rm + i;
            const float* pg = part + ((i >> 4) * 16 + m) * 16 + (i & 15);
            const float* pu = part + ((u >> 4) * 16 + m) * 16 + (u & 15);
            float sg = 0.f, su = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                sg += pg[w * KG * 256];
                su += pu[w * KG * 256];
            }
            if (16 * mt + m < M)
                h[static_cast<size_t>(16 * mt + m) * N + r0 + i] = round_bf16(silu_f32(sg) * su);
        }
        __syncthreads();
    }
}

// Whole-matrix decode: one lane per 64-weight run, same fragment builder as
// the fused kernel, 16-byte stores of 8 bf16 weights.
template <int K>
__global__ __launch_bounds__(kThreads) void expand_kernel(
    const uint32_t* __restrict__ codes, const float* __restrict__ scales,
    const float* __restrict__ lut, uint16_t* __restrict__ w, CodeLayout lay, long rows, int nb) {
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
    load_run64<K>(codes + block_word<K>(lay, static_cast<uint32_t>(row), b), cp, wr);
    const float scale = scales[row];
    uint16_t* dst = w + static_cast<size_t>(row) * nb * kT + b * kT + 64 * c;
    static_for<0, 8>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        *reinterpret_cast<u32x4*>(dst + 8 * S) = run64_fragment<K, S, false>(wr, lut_s, scale);
    });
}

// One workgroup per compute unit while that leaves at most kGroups groups
// each; beyond that, as many workgroups as needed, run in rounds.
int axis1_grid(int N) {
    const int groups = (N + 15) / 16;
    int G = groups < cu_count() ? groups : cu_count();
    if ((N + G - 1) / G > 16 * kGroups) G = (N + 16 * kGroups - 1) / (16 * kGroups);
    return G;
}

// Whether a workgroup of G over N rows ends in a group of at most 8 rows after
// a full one, where folding pays (the row counts differ by at most one).
bool fold_pays(int N, int G) {
    for (int rows = N / G; rows <= (N + G - 1) / G; ++rows) {
        const int gc = (rows + 15) >> 4;
        if (gc >= 2 && rows - 16 * (gc - 1) <= 8) return true;
    }
    return false;
}

// One launch of the 16-row-group kernel: the folding variant when asked for
// (one M tile of directly loaded activations, M <= 8), row-major or
// block-interleaved codes.
template <int K, int MT, bool DIRECT, int KG, bool SWIGLU>
hipError_t launch_prefill(bool fold, int G, int G0, hipStream_t st, const uint16_t* x,
                          const uint32_t* codes_a, const float* scales_a, const float* lut_a,
                          uint16_t* y_a, const uint32_t* codes_b, const float* scales_b,
                          const float* lut_b, uint16_t* y_b, CodeLayout lay, int N, int nb, int M,
                          const SplitArgs* split = nullptr) {
    const SplitArgs sp = split ? *split : SplitArgs{};
    auto go = [&](auto kernel) {
        return launch_kernel(kernel, dim3(G), dim3(PrefillShape<MT>::threads), st, x, codes_a,
                             scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, G0, lay, N, nb, M,
                             sp);
    };
    // Row-major iff a row's blocks are contiguous (with two blocks per row the
    // two layouts coincide).
    const bool rowmajor = lay.row_words == static_cast<uint64_t>(nb) * Bits<K>::wpb;
    // the first block staged (coalesced) with direct activations at M = 9..16:
    // measured 0.2-0.55 us faster there, 0.3-0.8 us slower at M = 5..8
    const bool stage1 = DIRECT && M > 8;
    if constexpr (!SWIGLU && KG == kGroups && !(K == 2 && MT == 2)) {
        if (split) {
            if constexpr (DIRECT) {
                if (stage1)
                    return rowmajor ? go(axis1_prefill_kernel<K, MT, DIRECT, false, KG, false, false, true, true>)
                                    : go(axis1_prefill_kernel<K, MT, DIRECT, true, KG, false, false, true, true>);
            }
            return rowmajor ? go(axis1_prefill_kernel<K, MT, DIRECT, false, KG, false, false, true>)
                            : go(axis1_prefill_kernel<K, MT, DIRECT, true, KG, false, false, true>);
        }
    }
    if constexpr (DIRECT && MT == 1) {
        if (fold && M <= 8)
            return rowmajor ? go(axis1_prefill_kernel<K, MT, DIRECT, false, KG, SWIGLU, true, false>)
                            : go(axis1_prefill_kernel<K, MT, DIRECT, true, KG, SWIGLU, true, false>);
        if (stage1)
            return rowmajor ? go(axis1_prefill_kernel<K, MT, DIRECT, false, KG, SWIGLU, false, false, true>)
                            : go(axis1_prefill_kernel<K, MT, DIRECT, true, KG, SWIGLU, false, false, true>);
    }
    return rowmajor ? go(axis1_prefill_kernel<K, MT, DIRECT, false, KG, SWIGLU, false, false>)
                    : go(axis1_prefill_kernel<K, MT, DIRECT, true, KG, SWIGLU, false, false>);
}

// The balanced plan for N rows of nb blocks over G workgroups at M rows and
// k bits (SplitArgs), or p = 0 where it does not apply: some groups left
// over, cut into at least two and at most kSplitMaxParts (and nb) parts, one
// more accumulator slot free, and the split tasks within wave 0's share of
// every workgroup. Not at k = 2 with two M tiles: there wave 0's split tasks
// (a block each) restage the activations at every task, and the plan measured
// 2% slower (at 5120 -> 17408, M = 32). Wave 0's lighter share: one task at
// M <= 8, two above, as measured best.
struct SplitPlan {
    int f = 0, p = 0, L = 0, pen = 0;
};

SplitPlan split_plan(int N, int nb, int G, int M, int k) {
    const int ng = (N + 15) / 16;
    if (G < 1 || (k == 2 && M > 16)) return {};
    const int f = ng / G, L = ng % G;
    if (L == 0 || f < 1 || f + 1 > kGroups || G % L != 0) return {};
    const int p = G / L;
    if (p < 2 || p > nb || p > kSplitMaxParts) return {};
    const int nq_max = (nb + p - 1) / p, nq_min = nb / p;
    const int waves = PrefillShape<1>::waves;
    // wave 0's share, (tasks + pen) / 8 - pen, holds the split tasks
    auto fits = [&](int pen) { return (f * nb + nq_min + pen) / waves - pen >= nq_max; };
    int pen = M <= 8 ? 1 : 2;
    while (pen > 0 && !fits(pen)) --pen;
    if (!fits(pen)) return {};
    return {f, p, L, pen};
}

// Workspace of the balanced plan: one part's tile per workgroup, 8-byte
// tagged words.
size_t split_bytes(const SplitPlan& sp, int G, int MT) {
    return sp.p ? static_cast<size_t>(G) * MT * kWave * 4 * sizeof(unsigned long long) : 0;
}

template <int K, int MT, bool DIRECT>
hipError_t launch_axis1_k(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                          const float* scales, const float* lut, uint16_t* y, int N, int nb,
                          float* workspace, size_t workspace_bytes, hipStream_t st) {
    const int G = axis1_grid(N);
    const SplitPlan plan = split_plan(N, nb, G, M, K);
    const size_t need = split_bytes(plan, G, MT);
    if (workspace && need && workspace_bytes >= need && !stream_capturing(st)) {
        const SplitArgs sp{reinterpret_cast<unsigned long long*>(workspace), next_call_tag(), plan.f,
                           plan.p, plan.pen};
        return launch_prefill<K, MT, DIRECT, kGroups, false>(false, G, G, st, x, codes, scales,
                                                             lut, y, codes, scales, lut, y, lay, N,
                                                             nb, M, &sp);
    }
    return launch_prefill<K, MT, DIRECT, kGroups, false>(fold_pays(N, G), G, G, st, x, codes,
                                                         scales, lut, y, codes, scales, lut, y,
                                                         lay, N, nb, M);
}

// Gate and up with the SwiGLU epilogue: the single launch's grid, every
// workgroup decoding its rows of both projections.
template <int K, int MT, bool DIRECT>
hipError_t launch_axis1_swiglu_k(const uint16_t* x, int M, const uint32_t* codes_g,
                                 const float* scales_g, const float* lut_g,
                                 const uint32_t* codes_u, const float* scales_u,
                                 const float* lut_u, uint16_t* h, CodeLayout lay, int N, int nb,
                                 hipStream_t st) {
    const int G = axis1_grid(N);
    return launch_prefill<K, MT, DIRECT, kGroups, true>(fold_pays(N, G), G, G, st, x, codes_g,
                                                        scales_g, lut_g, h, codes_u, scales_u,
                                                        lut_u, h, lay, N, nb, M);
}

// Workgroups per projection of the two-projection launch: half the compute
// units each, or one per 16-row group when there are fewer.
int axis1_dual_groups(int N) {
    const int groups = (N + 15) / 16;
    const int half = cu_count() / 2 > 0 ? cu_count() / 2 : 1;
    return groups < half ? groups : half;
}

template <int K, int MT, bool DIRECT>
hipError_t launch_axis1_dual_k(const uint16_t* x, int M, const uint32_t* codes_a,
                               const float* scales_a, const float* lut_a, uint16_t* y_a,
                               const uint32_t* codes_b, const float* scales_b,
                               const float* lut_b, uint16_t* y_b, CodeLayout lay, int N, int nb,
                               hipStream_t st) {
    const int G0 = axis1_dual_groups(N);
    if ((N + G0 - 1) / G0 > 16 * kDualGroups) return hipErrorInvalidValue;  // checked by the caller
    return launch_prefill<K, MT, DIRECT, kDualGroups, false>(fold_pays(N, G0), 2 * G0, G0, st, x,
                                                             codes_a, scales_a, lut_a, y_a, codes_b,
                                                             scales_b, lut_b, y_b, lay, N, nb, M);
}

template <int K>
hipError_t launch_expand_k(const uint32_t* codes, CodeLayout lay, const float* scales,
                           const float* lut, uint16_t* w, long rows, int nb, hipStream_t st) {
    const long runs = rows * nb * 4;
    const dim3 grid(static_cast<unsigned>((runs + kThreads - 1) / kThreads));
    return launch_kernel(expand_kernel<K>, grid, dim3(kThreads), st, codes, scales, lut, w, lay, rows,
                         nb);
}

}  // namespace

unsigned int next_call_tag() {
    static std::atomic<unsigned long long> next{
        (static_cast<unsigned long long>(
             std::chrono::steady_clock::now().time_since_epoch().count()) *
         0x9E3779B97F4A7C15ull) ^
        (static_cast<unsigned long long>(getpid()) << 32)};
    for (;;) {
        const unsigned int t = static_cast<unsigned int>(next.fetch_add(1, std::memory_order_relaxed));
        if (t) return t;
    }
}

bool stream_capturing(hipStream_t st) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    // a query that fails counts as capturing: the plans without tags are safe everywhere
    return hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone;
}

hipError_t launch_axis1(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                        const float* scales, const float* lut, uint16_t* y, int N, int nb, int k,
                        float* workspace, size_t workspace_bytes, hipStream_t st) {
    // One M tile (direct activation fragments) up to M = 16, two (staged) above.
    const int shape = M > 16 ? 2 : 0;
    float* const ws = workspace;
    const size_t wb = workspace_bytes;
    switch (k * 4 + shape) {
    case 8: return launch_axis1_k<2, 1, true>(x, M, codes, lay, scales, lut, y, N, nb, ws, wb, st);
    case 10: return launch_axis1_k<2, 2, false>(x, M, codes, lay, scales, lut, y, N, nb, ws, wb, st);
    case 12: return launch_axis1_k<3, 1, true>(x, M, codes, lay, scales, lut, y, N, nb, ws, wb, st);
    case 14: return launch_axis1_k<3, 2, false>(x, M, codes, lay, scales, lut, y, N, nb, ws, wb, st);
    case 16: return launch_axis1_k<4, 1, true>(x, M, codes, lay, scales, lut, y, N, nb, ws, wb, st);
    case 18: return launch_axis1_k<4, 2, false>(x, M, codes, lay, scales, lut, y, N, nb, ws, wb, st);
    default: return hipErrorInvalidValue;
    }
}

size_t axis1_split_bytes(int M, int N, int nb, int k) {
    const int G = axis1_grid(N);
    return split_bytes(split_plan(N, nb, G, M, k), G, M > 16 ? 2 : 1);
}

bool axis1_dual_supported(int M, int N, int k) {
    if (M < 1 || M > 32 || N < 1 || k < 2 || k > 4) return false;
    const int G0 = axis1_dual_groups(N);
    return (N + G0 - 1) / G0 <= 16 * kDualGroups;
}

hipError_t launch_axis1_dual(const uint16_t* x, int M, const uint32_t* codes_a,
                             const float* scales_a, const float* lut_a, uint16_t* y_a,
                             const uint32_t* codes_b, const float* scales_b, const float* lut_b,
                             uint16_t* y_b, CodeLayout lay, int N, int nb, int k,
                             hipStream_t st) {
    if (!axis1_dual_supported(M, N, k)) return hipErrorInvalidValue;
    // M tiles and activation loads as for the single launch
    const int shape = M > 16 ? 2 : 0;
    switch (k * 4 + shape) {
    case 8: return launch_axis1_dual_k<2, 1, true>(x, M, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, lay, N, nb, st);
    case 10: return launch_axis1_dual_k<2, 2, false>(x, M, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, lay, N, nb, st);
    case 12: return launch_axis1_dual_k<3, 1, true>(x, M, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, lay, N, nb, st);
    case 14: return launch_axis1_dual_k<3, 2, false>(x, M, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, lay, N, nb, st);
    case 16: return launch_axis1_dual_k<4, 1, true>(x, M, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, lay, N, nb, st);
    case 18: return launch_axis1_dual_k<4, 2, false>(x, M, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b, lay, N, nb, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_axis1_swiglu(const uint16_t* x, int M, const uint32_t* codes_g,
                               const float* scales_g, const float* lut_g, const uint32_t* codes_u,
                               const float* scales_u, const float* lut_u, uint16_t* h,
                               CodeLayout lay, int N, int nb, int k, hipStream_t st) {
    // k = 3, 4 with two M tiles: mixed gate/up groups; at most kMixedRows rows
    // of each projection per workgroup.
    if (k != 2 && M > 16) {
        int G = cu_count() < N ? cu_count() : N;
        if ((N + G - 1) / G > kMixedRows) G = (N + kMixedRows - 1) / kMixedRows;
        const bool rowmajor = lay.row_words == static_cast<uint64_t>(nb) * 8 * k;
        if (k == 3)
            return launch_kernel(rowmajor ? axis1_swiglu_mixed_kernel<3, false> : axis1_swiglu_mixed_kernel<3, true>,
                                 dim3(G), dim3(MixedLds::threads), st, x, codes_g, scales_g, lut_g,
                                 codes_u, scales_u, lut_u, h, lay, N, nb, M);
        return launch_kernel(rowmajor ? axis1_swiglu_mixed_kernel<4, false> : axis1_swiglu_mixed_kernel<4, true>,
                             dim3(G), dim3(MixedLds::threads), st, x, codes_g, scales_g, lut_g,
                             codes_u, scales_u, lut_u, h, lay, N, nb, M);
    }
    // M tiles and activation loads as for the single launch
    const int shape = M > 16 ? 2 : 0;
    switch (k * 4 + shape) {
    case 8: return launch_axis1_swiglu_k<2, 1, true>(x, M, codes_g, scales_g, lut_g, codes_u, scales_u, lut_u, h, lay, N, nb, st);
    case 10: return launch_axis1_swiglu_k<2, 2, false>(x, M, codes_g, scales_g, lut_g, codes_u, scales_u, lut_u, h, lay, N, nb, st);
    case 12: return launch_axis1_swiglu_k<3, 1, true>(x, M, codes_g, scales_g, lut_g, codes_u, scales_u, lut_u, h, lay, N, nb, st);
    case 16: return launch_axis1_swiglu_k<4, 1, true>(x, M, codes_g, scales_g, lut_g, codes_u, scales_u, lut_u, h, lay, N, nb, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_expand(const uint32_t* codes, CodeLayout lay, const float* scales,
                         const float* lut, uint16_t* w, long rows, int nb, int k, hipStream_t st) {
    switch (k) {
    case 2: return launch_expand_k<2>(codes, lay, scales, lut, w, rows, nb, st);
    case 3: return launch_expand_k<3>(codes, lay, scales, lut, w, rows, nb, st);
    case 4: return launch_expand_k<4>(codes, lay, scales, lut, w, rows, nb, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace trellis
