// Device-side building blocks shared by the trellis kernels (gfx950).
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0,
// page 60 (tiled-prefill.ts weight-tile decode, vector-expand.ts) and
// page 59 (scatter.ts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.hpp"

namespace trellis {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 256;           // weights per block
constexpr int kL = 12;            // window bits
constexpr int kLutEntries = 4096; // 2^L codebook entries
constexpr int kWave = 64;

// Words per 256-weight block.
template <int K> struct Bits {
    static constexpr int wpb = kT * K / 32;   // 16 / 24 / 32
};

// Orders one wave's LDS stores before, and its loads after, the call, for
// data that lanes of the wave pass to one another through LDS. The hardware
// runs a wave's LDS instructions in order, so no wait is needed (wave-scope
// fences emit none), but the compiler reasons per lane: without the fences it
// may sink a store whose value no later load of the same lane reads into a
// branch, or move it past another lane's load.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Tagged partials: workgroups that meet through a workspace pass each float
// as one 64-bit word, a per-call tag above the float's bits. The tag is mixed
// with the word's slot, so that a workspace filled with one constant never
// carries the expected tag in two slots at once.
__device__ __forceinline__ unsigned int slot_tag(unsigned int tag, int slot) {
    return tag ^ (static_cast<unsigned int>(slot) * 0x9E3779B9u);
}
__device__ __forceinline__ unsigned long long tagged_word(unsigned int tag, float v) {
    return (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(v);
}

// Word offset of block b of stored row r (CodeLayout).
template <int K>
__device__ __forceinline__ uint64_t block_word(const CodeLayout& lay, uint32_t r, uint32_t b) {
    return static_cast<uint64_t>(r) * lay.row_words + static_cast<uint64_t>(b >> 1) * lay.pair_words +
           (b & 1u) * static_cast<uint32_t>(Bits<K>::wpb);
}

// Copy the 16 KB float32 codebook into LDS with 16-byte loads
// (page 59 scatter.ts stages the LUT into threadgroup memory once per group).
template <int NTHREADS>
__device__ __forceinline__ void stage_lut(float* __restrict__ lut_s, const float* __restrict__ lut) {
    const float4* src = reinterpret_cast<const float4*>(lut);
    float4* dst = reinterpret_cast<float4*>(lut_s);
#pragma unroll
    for (int i = threadIdx.x; i < kLutEntries / 4; i += NTHREADS) dst[i] = src[i];
}

// Compile-time loop: f(std::integral_constant<int, I>{}) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Bit field of a little-endian word array, pre-scaled for LDS addressing:
// ((bits >> O) & (2^WIDTH - 1)) << SHIFT, formed as one shift or funnel shift
// plus one mask. O is a template constant, so every word index is known at
// compile time and the array stays in registers.
// field_raw: the same before the mask, i.e. the field at bits [SHIFT, SHIFT +
// WIDTH) of the result with whatever bits surround it.
template <int O, int WIDTH, int SHIFT, int N>
__device__ __forceinline__ uint32_t field_raw(const uint32_t (&w)[N]) {
    if constexpr (O < SHIFT) {
        static_assert(O + WIDTH <= 32, "field must sit in word 0");
        return w[0] << (SHIFT - O);
    } else {
        constexpr int s = O - SHIFT, wi = s >> 5, sh = s & 31;
        if constexpr (sh + WIDTH + SHIFT <= 32) {
            return w[wi] >> sh;
        } else {
            static_assert(wi + 1 < N, "field runs past the loaded words");
            return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
        }
    }
}

template <int O, int WIDTH, int SHIFT, int N>
__device__ __forceinline__ uint32_t field_offset(const uint32_t (&w)[N]) {
    constexpr uint32_t mask = ((1u << WIDTH) - 1u) << SHIFT;
    return field_raw<O, WIDTH, SHIFT>(w) & mask;
}

// (a & mask) | b in one VALU op (v_and_or_b32). Written out because the
// compiler turns an OR of disjoint bits into an add and then re-associates it
// with the LDS base, which costs a separate AND and ADD per gather.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t b) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(b));
    return r;
}

// Byte offset into the LDS codebook (4-byte entries) of the 12-bit window
// that starts at bit O.
template <int O, int N>
__device__ __forceinline__ uint32_t lut_byte_offset(const uint32_t (&w)[N]) {
    return field_offset<O, kL, 2>(w);
}

__device__ __forceinline__ float lds_lut(const float* lut_s, uint32_t byte_off) {
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut_s) + byte_off);
}

__device__ __forceinline__ floatx2 lds_pair(const float* tab, uint32_t byte_off) {
    return *reinterpret_cast<const floatx2*>(reinterpret_cast<const char*>(tab) + byte_off);
}

// Two decoded weights packed as bf16x2 (low half = first): each is the float32
// product value*scale rounded to bf16, nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_weights(float v0, float v1, float scale) {
    floatx2 p = {v0 * scale, v1 * scale};
    bf16x2 h = __builtin_convertvector(p, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------------------
// 64-weight runs. Weight t of a 256-weight block sits at bit (255 - t) k of
// the block's bit string, so the run of weights [64c, 64c + 64) is the
// contiguous bit range [64 (3 - c) k, 64 (4 - c) k) -- exactly 2k words,
// starting at word 2k cp with cp = 3 - c -- plus the up to 11 window bits that
// spill into the next word (word 0 of the same block after the last word: the
// tail-biting wrap). Inside the run, weight 64c + i is local symbol
// q = 63 - i, whose window starts at local bit q k.
// STREAM marks the loads non-temporal: the codes are read exactly once.
template <typename T, bool STREAM>
__device__ __forceinline__ T load_words(const T* p) {
    if constexpr (STREAM) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int K, bool STREAM = false>
__device__ __forceinline__ void load_run64(const uint32_t* __restrict__ block, int cp,
                                           uint32_t (&w)[2 * K + 1]) {
    constexpr int wpb = Bits<K>::wpb;
    const uint32_t* p = block + 2 * K * cp;
    if constexpr (K == 2) {
        const u32x4 v = load_words<u32x4, STREAM>(reinterpret_cast<const u32x4*>(p));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (K == 3) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 a = load_words<u32x2, STREAM>(reinterpret_cast<const u32x2*>(p));
        const u32x2 b = load_words<u32x2, STREAM>(reinterpret_cast<const u32x2*>(p + 2));
        const u32x2 c = load_words<u32x2, STREAM>(reinterpret_cast<const u32x2*>(p + 4));
        w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y; w[4] = c.x; w[5] = c.y;
    } else {
        const u32x4 a = load_words<u32x4, STREAM>(reinterpret_cast<const u32x4*>(p));
        const u32x4 b = load_words<u32x4, STREAM>(reinterpret_cast<const u32x4*>(p + 4));
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
    const int nxt = 2 * K * (cp + 1);
    w[2 * K] = load_words<uint32_t, STREAM>(block + (nxt == wpb ? 0 : nxt));
}

// The 2k run words only; the word after the run comes from the neighbour lane
// (next_run_word) instead of a second load.
template <int K>
__device__ __forceinline__ void load_run64_words(const uint32_t* __restrict__ block, int cp,
                                                 uint32_t (&w)[2 * K + 1]) {
    const uint32_t* p = block + 2 * K * cp;
    if constexpr (K == 2) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (K == 3) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 a = *reinterpret_cast<const u32x2*>(p);
        const u32x2 b = *reinterpret_cast<const u32x2*>(p + 2);
        const u32x2 c = *reinterpret_cast<const u32x2*>(p + 4);
        w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y; w[4] = c.x; w[5] = c.y;
    } else {
        const u32x4 a = *reinterpret_cast<const u32x4*>(p);
        const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
}

// When the four runs of a block sit in lanes l, l + 16, l + 32, l + 48 with
// run cp = 3 - l / 16, the word after run cp is the first word of run cp + 1,
// held 16 lanes below; after the last run (cp = 3) it is word 0 of the block,
// run 0, held 48 lanes above. Both are a rotation of the wave by 16 lanes.
__device__ __forceinline__ uint32_t next_run_word(uint32_t first_word) {
    const int lane = threadIdx.x & 63;
    return static_cast<uint32_t>(
        __builtin_amdgcn_ds_bpermute(((lane - 16) & 63) << 2, static_cast<int>(first_word)));
}

// Entries of the k = 2 pair table: entry F (the 14-bit union of the windows
// of an adjacent pair of weights, which overlap by 10 bits) holds
// (LUT[F >> 2], LUT[F & 0xFFF]), the values of the earlier and the later weight.
constexpr int kPairEntries = 1 << 14;

// B fragment S (0..7) of a 64-weight run: weights 64c + 8S + e, e = 0..7,
// packed two per dword, low half first (the MFMA operand layout). The fetch
// is split from the pack so callers can keep several fragments' gathers in
// flight: gather_run64 issues the LDS reads (4 pair-table reads when PAIR,
// else 8 codebook reads), pack_fragment turns the values into the operand.
// Pair j of the fragment is weights 2j, 2j + 1: local symbols q0 = 63 - 8S - 2j
// (the earlier weight) and q0 - 1.
template <bool PAIR>
struct Gathered {
    floatx2 v[4];  // v[j] = values of the earlier and the later weight of pair j
};

template <int K, int S, bool PAIR>
__device__ __forceinline__ Gathered<PAIR> gather_run64(const uint32_t (&w)[2 * K + 1],
                                                       const float* __restrict__ tab) {
    static_assert(!PAIR || K == 2, "pair table only for k = 2");
    Gathered<PAIR> g;
    static_for<0, 4>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        constexpr int q0 = 63 - 8 * S - 2 * d;
        if constexpr (PAIR) {
            // the 14-bit union starts at the later weight's window, bit 2 (q0 - 1)
            g.v[d] = lds_pair(tab, field_offset<2 * (q0 - 1), 14, 3>(w));
        } else {
            g.v[d].x = lds_lut(tab, lut_byte_offset<q0 * K>(w));
            g.v[d].y = lds_lut(tab, lut_byte_offset<(q0 - 1) * K>(w));
        }
    });
    return g;
}

// Bank-partitioned codebook copies (k = 3, 4). A wave's random 4-byte LDS
// reads are bank-conflict bound: 32 lanes of random 12-bit indices pile up
// several deep on the most loaded bank. With kRepCopies copies of the
// codebook, entry e of copy c at byte (e << 5) | (c << 2), copy c occupies only
// the banks with (bank & 7) == c; lane l reads copy l & 7, so the lanes of one
// read pass spread over disjoint bank groups four at a time. Measured on MI355X
// (uniform random indices, 8 waves per CU): 6.1 instead of 7.6 clocks per
// wave-wide read, 10.4 instead of 8.4 values per clock per CU. The copies fill
// 128 KB of LDS.
constexpr int kRepCopies = 8;
constexpr int kRepFloats = kLutEntries * kRepCopies;

// This lane's copy, as the byte offset OR-ed into every gather address.
__device__ __forceinline__ uint32_t rep_lane_offset() {
    return (threadIdx.x & (kRepCopies - 1)) << 2;
}

// Gathers of fragment S from the replicated codebook (layout above).
template <int K, int S>
__device__ __forceinline__ Gathered<false> gather_run64_rep(const uint32_t (&w)[2 * K + 1],
                                                            const float* __restrict__ tab,
                                                            uint32_t cofs) {
    Gathered<false> g;
    static_for<0, 4>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        constexpr int q0 = 63 - 8 * S - 2 * d;
        g.v[d].x = lds_lut(tab, field_offset<q0 * K, kL, 5>(w) | cofs);
        g.v[d].y = lds_lut(tab, field_offset<(q0 - 1) * K, kL, 5>(w) | cofs);
    });
    return g;
}

// Gathers of fragment S from one of several codebooks laid out one after
// another in LDS, each in R bank-partitioned copies (entry e of copy c at byte
// (e R + c) 4, R a power of two): `sel` is the byte offset of this lane's
// codebook (a multiple of R 16 KB) OR-ed with that of its copy, merged into
// the window's offset as the copy offset is above.
template <int K, int S, int R = 1>
__device__ __forceinline__ Gathered<false> gather_run64_sel(const uint32_t (&w)[2 * K + 1],
                                                            const float* __restrict__ tab,
                                                            uint32_t sel) {
    constexpr int sh = 2 + (R == 1 ? 0 : R == 2 ? 1 : R == 4 ? 2 : 3);
    static_assert(R == 1 || R == 2 || R == 4 || R == 8, "R copies, a power of two");
    Gathered<false> g;
    static_for<0, 4>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        constexpr int q0 = 63 - 8 * S - 2 * d;
        constexpr uint32_t mask = (kLutEntries - 1u) << sh;
        g.v[d].x = lds_lut(tab, and_or(field_raw<q0 * K, kL, sh>(w), mask, sel));
        g.v[d].y = lds_lut(tab, and_or(field_raw<(q0 - 1) * K, kL, sh>(w), mask, sel));
    });
    return g;
}

// Staging of the replicated codebook in two phases as fetch_table/store_table:
// entry e fills the two 16-byte chunks at byte e << 5 (four copies each);
// thread tid stages entries tid + NTHREADS i, one register each.
template <int NTHREADS>
struct RepSrc {
    static_assert(kLutEntries % NTHREADS == 0, "every thread stages the same number of entries");
    static constexpr int n = kLutEntries / NTHREADS;
    float a[n];
};

template <int NTHREADS>
__device__ __forceinline__ void fetch_rep(RepSrc<NTHREADS>& src, const float* lut) {
    using gf32 = const __attribute__((address_space(1))) float*;
    gf32 l = (gf32)lut;
    asm volatile("" : "+s"(l));
#pragma unroll
    for (int i = 0; i < RepSrc<NTHREADS>::n; ++i) src.a[i] = l[threadIdx.x + NTHREADS * i];
}

template <int NTHREADS>
__device__ __forceinline__ void store_rep(const RepSrc<NTHREADS>& src, float* __restrict__ tab) {
    float4* dst = reinterpret_cast<float4*>(tab);
#pragma unroll
    for (int i = 0; i < RepSrc<NTHREADS>::n; ++i) {
        const float a = src.a[i];
        const int e = threadIdx.x + NTHREADS * i;
        dst[2 * e] = float4{a, a, a, a};
        dst[2 * e + 1] = float4{a, a, a, a};
    }
}

template <bool PAIR>
__device__ __forceinline__ u32x4 pack_fragment(const Gathered<PAIR>& g, float scale) {
    u32x4 r;
    static_for<0, 4>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        r[d] = pack_weights(g.v[d].x, g.v[d].y, scale);
    });
    return r;
}

template <int K, int S, bool PAIR>
__device__ __forceinline__ u32x4 run64_fragment(const uint32_t (&w)[2 * K + 1],
                                                const float* __restrict__ tab, float scale) {
    return pack_fragment<PAIR>(gather_run64<K, S, PAIR>(w, tab), scale);
}

// Decode table staging in two phases, so that a kernel can issue its other
// loads in between and wait for all of them once: fetch_table loads this
// thread's share of the codebook into registers, store_table writes the LDS
// table from them. With PAIR the table is the k = 2 pair table: entry F holds
// (LUT[F >> 2], LUT[F & 0xFFF]); the four entries 4 grp + i share F >> 2 = grp
// and take F & 0xFFF = 4 (grp & 1023) + i.
template <int NTHREADS, bool PAIR>
struct TableSrc {
    static constexpr int n = (PAIR ? kPairEntries : kLutEntries) / 4 / NTHREADS;
    float a[n];
    floatx4 b[n];
};

// The loads go through an opaque global-address-space copy of the pointer:
// through a restrict kernel pointer they count as invariant, and the compiler
// sinks them past any barrier to their use in store_table, after whatever the
// kernel issued in between.
template <int NTHREADS, bool PAIR>
__device__ __forceinline__ void fetch_table(TableSrc<NTHREADS, PAIR>& src, const float* lut) {
    using gf32 = const __attribute__((address_space(1))) float*;
    using gf32x4 = const __attribute__((address_space(1))) floatx4*;
    gf32 l = (gf32)lut;  // generic to global: an address-space cast
    asm volatile("" : "+s"(l));
    const gf32x4 l4 = reinterpret_cast<gf32x4>(l);
#pragma unroll
    for (int i = 0; i < TableSrc<NTHREADS, PAIR>::n; ++i) {
        const int grp = threadIdx.x + NTHREADS * i;
        if constexpr (PAIR) {
            src.a[i] = l[grp];
            src.b[i] = l4[grp & 1023];
        } else {
            src.b[i] = l4[grp];
        }
    }
}

template <int NTHREADS, bool PAIR>
__device__ __forceinline__ void store_table(const TableSrc<NTHREADS, PAIR>& src,
                                            float* __restrict__ tab) {
    float4* dst = reinterpret_cast<float4*>(tab);
#pragma unroll
    for (int i = 0; i < TableSrc<NTHREADS, PAIR>::n; ++i) {
        const int grp = threadIdx.x + NTHREADS * i;
        if constexpr (PAIR) {
            const float a = src.a[i];
            const floatx4 b = src.b[i];
            dst[2 * grp] = float4{a, b[0], a, b[1]};
            dst[2 * grp + 1] = float4{a, b[2], a, b[3]};
        } else {
            const floatx4 b = src.b[i];
            dst[grp] = float4{b[0], b[1], b[2], b[3]};
        }
    }
}

// Build the k = 2 pair table in LDS from the codebook in global memory.
template <int NTHREADS>
__device__ __forceinline__ void stage_pair_table(float* __restrict__ tab,
                                                 const float* __restrict__ lut) {
    TableSrc<NTHREADS, true> src;
    fetch_table<NTHREADS, true>(src, lut);
    store_table<NTHREADS, true>(src, tab);
}

// Fragment S's gathers from a kernel's decode table (DecodeTable kinds).
template <int K, int S, bool PAIR, bool REP>
__device__ __forceinline__ Gathered<PAIR> gather_tab(const uint32_t (&w)[2 * K + 1],
                                                     const float* __restrict__ tab) {
    if constexpr (REP) return gather_run64_rep<K, S>(w, tab, rep_lane_offset());
    else return gather_run64<K, S, PAIR>(w, tab);
}

// Staging of a kernel's decode table in two phases (fetch into registers,
// store to LDS): the 16 KB codebook, the k = 2 pair table (PAIR) or the
// bank-partitioned codebook copies (REP).
template <int NTHREADS, bool PAIR, bool REP>
struct DecodeTable {
    static_assert(!(PAIR && REP), "one table kind");
    using Src = std::conditional_t<REP, RepSrc<NTHREADS>, TableSrc<NTHREADS, PAIR>>;
    static constexpr int floats = PAIR ? 2 * kPairEntries : REP ? kRepFloats : kLutEntries;
    static __device__ __forceinline__ void fetch(Src& s, const float* lut) {
        if constexpr (REP) fetch_rep<NTHREADS>(s, lut);
        else fetch_table<NTHREADS, PAIR>(s, lut);
    }
    static __device__ __forceinline__ void store(const Src& s, float* __restrict__ tab) {
        if constexpr (REP) store_rep<NTHREADS>(s, tab);
        else store_table<NTHREADS, PAIR>(s, tab);
    }
};

__device__ __forceinline__ uint16_t round_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace trellis
