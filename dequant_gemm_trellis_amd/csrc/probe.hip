// Codebook-gather rate probe for gfx950: the ceiling that the decode of every
// trellis kernel here runs against.
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0,
// page 59 scatter.ts (the codebook is staged in threadgroup memory, lutTG,
// and every weight is decoded by one read of it at its window) and page 60
// tiled-prefill.ts (the weight-tile decode reads the table the same way).
//
// Each decoded weight costs one random read of a table in LDS. This kernel
// does nothing but such reads, from the three table layouts the kernels use,
// with the occupancy they run at (one 512-thread workgroup of 8 waves per
// compute unit, the LDS allocation of the GEMV), so that the time per read is
// what the hardware gives a decode that does no other work:
//   kind 0: the k = 2 pair table, 16384 entries of 8 bytes (ds_read_b64,
//           two decoded weights per lane and read);
//   kind 1: the codebook in eight bank-partitioned copies (entry e of copy c at
//           byte 32 e + 4 c, lane l reading copy l % 8; ds_read_b32);
//   kind 2: the plain 16 KB codebook (ds_read_b32).
// Indices are uniform random over the table: a counter-based integer hash
// gives each lane 32 entries, and round r reads entry e XOR m_r with m_r the
// same for the whole wave. XOR by a wave-uniform mask permutes the banks of
// all lanes alike, so every round repeats the bank-conflict pattern of 32
// independent random index vectors per wave (65536 over the device). Timing
// two round counts and taking the difference removes the launch, the table
// fill and the store.
#include <stdint.h>

#include "common.hpp"
#include "launch.hpp"
#include "trellis_probe.h"

namespace trellis {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeReads = 32;            // independent index vectors per lane
constexpr int kProbeLdsFloats = 40960;     // 160 KB: one workgroup per CU, as the GEMV

// Integer hash (xor-shift-multiply, 32-bit avalanche), for the probe's indices.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <int KIND>
struct ProbeKind {
    // byte offset of table entry e for this lane, and the entry-bit mask
    static constexpr int entry_bits = KIND == 0 ? 14 : 12;
    static constexpr int table_floats = KIND == 0 ? 2 * 16384 : KIND == 1 ? 8 * 4096 : 4096;
    static __device__ __forceinline__ uint32_t offset(uint32_t e, int lane) {
        if constexpr (KIND == 0) return e << 3;
        else if constexpr (KIND == 1) return (e << 5) | ((lane & 7) << 2);
        else return e << 2;
    }
    static __device__ __forceinline__ uint32_t round_mask(int r) {
        const uint32_t e = (static_cast<uint32_t>(r) * 0x9E3779B1u) >> (32 - entry_bits);
        return offset(e, 0);
    }
};

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void gather_probe_kernel(float* __restrict__ out,
                                                                     int rounds, uint32_t seed) {
    using PK = ProbeKind<KIND>;
    __shared__ __attribute__((aligned(16))) float lds[kProbeLdsFloats];
    const int tid = threadIdx.x, lane = tid & 63;
    for (int i = tid; i < PK::table_floats; i += kProbeThreads)
        lds[i] = static_cast<float>(i & 1023) * (1.f / 1024.f);
    uint32_t off[kProbeReads];
    const uint32_t gid = blockIdx.x * kProbeThreads + tid;
#pragma unroll
    for (int i = 0; i < kProbeReads; ++i) {
        const uint32_t h = mix32(seed ^ mix32(gid * kProbeReads + i));
        off[i] = PK::offset(h >> (32 - PK::entry_bits), lane);
    }
    __syncthreads();
    const char* base = reinterpret_cast<const char*>(lds);
    float acc = 0.f;
    for (int r = 0; r < rounds; ++r) {
        const uint32_t m = PK::round_mask(r);
#pragma unroll
        for (int i = 0; i < kProbeReads; ++i) {
            if constexpr (KIND == 0) {
                const floatx2 v = *reinterpret_cast<const floatx2*>(base + (off[i] ^ m));
                acc += v.x + v.y;
            } else {
                acc += *reinterpret_cast<const float*>(base + (off[i] ^ m));
            }
        }
    }
    out[gid] = acc;
}

}  // namespace
}  // namespace trellis

extern "C" {

uint64_t trellis_gather_probe_values(int32_t kind, int32_t rounds) {
    if (kind < 0 || kind > 2 || rounds < 0) return 0;
    const uint64_t lanes = static_cast<uint64_t>(trellis::cu_count()) * trellis::kProbeThreads;
    return lanes * trellis::kProbeReads * static_cast<uint64_t>(rounds) * (kind == 0 ? 2u : 1u);
}

size_t trellis_gather_probe_out_floats(void) {
    return static_cast<size_t>(trellis::cu_count()) * trellis::kProbeThreads;
}

int trellis_gather_probe(int32_t kind, int32_t rounds, float* out, size_t out_floats,
                         hipStream_t stream) {
    if (!out) return TRELLIS_PROBE_ERR_ARG;
    if (kind < 0 || kind > 2 || rounds < 0 || rounds > (1 << 20)) return TRELLIS_PROBE_ERR_ARG;
    const int G = trellis::cu_count();
    if (out_floats < static_cast<size_t>(G) * trellis::kProbeThreads) return TRELLIS_PROBE_ERR_ARG;
    const uint32_t seed = 0x5EEDu;
    hipError_t e;
    switch (kind) {
    case 0: e = trellis::launch_kernel(trellis::gather_probe_kernel<0>, dim3(G), dim3(trellis::kProbeThreads), stream, out, rounds, seed); break;
    case 1: e = trellis::launch_kernel(trellis::gather_probe_kernel<1>, dim3(G), dim3(trellis::kProbeThreads), stream, out, rounds, seed); break;
    default: e = trellis::launch_kernel(trellis::gather_probe_kernel<2>, dim3(G), dim3(trellis::kProbeThreads), stream, out, rounds, seed); break;
    }
    return e == hipSuccess ? 0 : TRELLIS_PROBE_ERR_HIP;
}

}  // extern "C"
