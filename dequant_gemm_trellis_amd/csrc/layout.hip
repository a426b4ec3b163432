// Code-array layout conversion for gfx950: rewrites the words of every
// 256-weight block from one block layout into the other (row-major, or block
// interleave 2).
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0,
// page 60 vector-expand.ts and page 59 scatter.ts / splitk-prefill.ts: with
// their INTERLEAVE constant set they find block b of stored row r at word
// (b / 2) * rows * 2 * wpb + r * 2 * wpb + (b % 2) * wpb, i.e. pairs of
// blocks outermost, then rows, then the pair's two blocks.
//
// The copy is a pure permutation of 16-byte chunks (wpb = 16 / 24 / 32 words
// is a multiple of 4). Threads are numbered in the destination's order, so
// the stores are dense and each source block is read as wpb / 4 adjacent
// chunks by adjacent threads.
#include "common.hpp"
#include "launch.hpp"

namespace trellis {
namespace {

constexpr int kRepackThreads = 256;

// Chunk i of the destination: block q = i / cpb in destination order, chunk
// i % cpb of it. In row-major order q = r * nb + b; in interleave-2 order
// q = (b / 2) * rows * 2 + r * 2 + b % 2.
template <int K, bool DST_PAIRS>
__global__ __launch_bounds__(kRepackThreads) void repack_kernel(
    const uint32_t* __restrict__ src, CodeLayout from, uint32_t* __restrict__ dst, int rows,
    int nb, uint64_t chunks) {
    constexpr int cpb = Bits<K>::wpb / 4;
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * kRepackThreads + threadIdx.x;
    if (i >= chunks) return;
    const uint64_t q = i / cpb;
    const uint32_t e = static_cast<uint32_t>(i - q * cpb);
    uint32_t r, b;
    if constexpr (DST_PAIRS) {
        const uint64_t per_pair = 2ull * static_cast<uint64_t>(rows);
        const uint64_t pair = q / per_pair;
        const uint32_t rem = static_cast<uint32_t>(q - pair * per_pair);
        r = rem >> 1;
        b = static_cast<uint32_t>(2 * pair) + (rem & 1u);
    } else {
        r = static_cast<uint32_t>(q / static_cast<uint64_t>(nb));
        b = static_cast<uint32_t>(q - static_cast<uint64_t>(r) * nb);
    }
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + block_word<K>(from, r, b) + 4 * e);
    *reinterpret_cast<u32x4*>(dst + 4 * i) = v;
}

template <int K>
hipError_t launch_repack_k(const uint32_t* src, CodeLayout from, uint32_t* dst, bool dst_pairs,
                           int rows, int nb, hipStream_t st) {
    const uint64_t chunks = static_cast<uint64_t>(rows) * nb * (Bits<K>::wpb / 4);
    if (chunks == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((chunks + kRepackThreads - 1) / kRepackThreads));
    if (dst_pairs)
        return launch_kernel(repack_kernel<K, true>, grid, dim3(kRepackThreads), st, src, from, dst,
                             rows, nb, chunks);
    return launch_kernel(repack_kernel<K, false>, grid, dim3(kRepackThreads), st, src, from, dst,
                         rows, nb, chunks);
}

}  // namespace

hipError_t launch_repack(const uint32_t* src, CodeLayout from, uint32_t* dst, bool dst_pairs,
                         int rows, int nb, int k, hipStream_t st) {
    switch (k) {
    case 2: return launch_repack_k<2>(src, from, dst, dst_pairs, rows, nb, st);
    case 3: return launch_repack_k<3>(src, from, dst, dst_pairs, rows, nb, st);
    case 4: return launch_repack_k<4>(src, from, dst, dst_pairs, rows, nb, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace trellis
