// Host-side launchers of the trellis kernels (internal to libtrellis.so).
// Callers have validated every argument; these only enqueue work.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace trellis {

template <typename T> struct non_deduced { using type = T; };

// Launch `kernel` on `st` and return the launch's own status (unlike
// hipGetLastError, not one left behind by an earlier call).
template <typename... P>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t st,
                         typename non_deduced<P>::type... args) {
    void* argv[] = {static_cast<void*>(&args)..., nullptr};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, st);
}

// Compute units of the current device (cached per device).
int cu_count();

// Where the words of block b of stored row r start in the code array:
//   r * row_words + (b / 2) * pair_words + (b % 2) * wpb      (wpb = 8k).
// Row-major layout, [rows][nb][wpb] (block interleave 0):
//   row_words = nb * wpb, pair_words = 2 * wpb.
// Block interleave 2, [nb / 2][rows][2][wpb] (pages: vector-expand.ts and
// scatter.ts with INTERLEAVE set):
//   row_words = 2 * wpb, pair_words = rows * 2 * wpb.
struct CodeLayout {
    uint64_t row_words;
    uint64_t pair_words;
};

inline CodeLayout code_layout(int interleave, int rows, int nb, int k) {
    const uint64_t wpb = 8u * static_cast<uint64_t>(k);
    if (interleave == 2) return {2 * wpb, static_cast<uint64_t>(rows) * 2 * wpb};
    return {static_cast<uint64_t>(nb) * wpb, 2 * wpb};
}

// Axis-1 GEMV (M = 1): persistent kernel, one workgroup per compute unit,
// activations staged in LDS. Needs nb <= gemv_max_blocks(k).
hipError_t launch_gemv(const uint16_t* x, const uint32_t* codes, CodeLayout lay, const float* scales,
                       const float* lut, uint16_t* y, int N, int nb, int k, hipStream_t st);
int gemv_max_blocks(int k);

// Two axis-1 GEMVs of one shape over the same x in one launch (half of the
// compute units each); same conditions as launch_gemv.
hipError_t launch_gemv_dual(const uint16_t* x, const uint32_t* codes_a, const float* scales_a,
                            const float* lut_a, uint16_t* y_a, const uint32_t* codes_b,
                            const float* scales_b, const float* lut_b, uint16_t* y_b,
                            CodeLayout lay, int N, int nb, int k, hipStream_t st);

// Gate and up (one activation row) with the SwiGLU epilogue in one launch:
// h[n] = bf16(silu(g_n) * u_n) from the float32 row sums of both projections;
// same conditions as launch_gemv.
hipError_t launch_gemv_swiglu(const uint16_t* x, const uint32_t* codes_g, const float* scales_g,
                              const float* lut_g, const uint32_t* codes_u, const float* scales_u,
                              const float* lut_u, uint16_t* h, CodeLayout lay, int N, int nb, int k,
                              hipStream_t st);

// Axis 1, 1 <= M <= kGemvRowsMaxM, in the GEMV's unit mapping (one workgroup
// per compute unit, at least 16 rows each); gemv_rows_supported says whether
// the geometry fits it (at least 16 rows, 16 rows' unit partials fit in LDS).
// Beyond 4 rows the 16-row-group kernel measured faster: at k = 2 only about
// 49 rows' partials of 8 floats fit beside the 128 KB pair table at 5120
// inputs, and a second chunk (pipeline restart, a second epilogue, a block
// edge every other step) was 14-21% slower; at k = 3, 4 the 16-row-group
// kernel with directly loaded activations reads the codebook copies and was
// 0.5-4% faster than this kernel on one codebook (M = 5, 8).
constexpr int kGemvRowsMaxM = 4;
bool gemv_rows_supported(int M, int N, int nb, int k);
hipError_t launch_gemv_rows(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                            const float* scales, const float* lut, uint16_t* y, int N, int nb,
                            int k, hipStream_t st);

// Axis 1, 1 <= M <= 32: y[M][N] from x[M][nb*256] and codes [N][nb][8k]
// (16-row groups). Persistent workgroups of at most 80 rows; any nb. Given a
// workspace of at least axis1_split_bytes(M, N, nb, k) > 0 bytes, outside
// stream capture, the balanced plan: whole groups per workgroup, the leftover
// groups cut by blocks, their parts meeting through the workspace (any
// initial contents; calls sharing a workspace must not overlap in time).
hipError_t launch_axis1(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                        const float* scales, const float* lut, uint16_t* y, int N, int nb, int k,
                        float* workspace, size_t workspace_bytes, hipStream_t st);
size_t axis1_split_bytes(int M, int N, int nb, int k);

// Tags of calls whose workgroups meet through tagged words in a workspace:
// a fresh 32-bit value per call (never 0), from a per-process start. Such
// plans are not used under stream capture (a replay would repeat the tag).
unsigned int next_call_tag();
bool stream_capturing(hipStream_t st);

// Two axis-1 projections of one geometry over the same x[M][nb*256], 1 <= M
// <= 32, in one launch of the 16-row-group kernel (half the compute units
// each, at most 144 rows per workgroup); axis1_dual_supported says whether
// the geometry fits.
bool axis1_dual_supported(int M, int N, int k);
hipError_t launch_axis1_dual(const uint16_t* x, int M, const uint32_t* codes_a,
                             const float* scales_a, const float* lut_a, uint16_t* y_a,
                             const uint32_t* codes_b, const float* scales_b, const float* lut_b,
                             uint16_t* y_b, CodeLayout lay, int N, int nb, int k,
                             hipStream_t st);

// Gate and up over the same x[M][nb*256], 1 <= M <= 32, with the SwiGLU
// epilogue, in one launch of a 16-row-group kernel, every workgroup decoding
// its rows of both projections (k = 3, 4 at M > 16: side by side in shared
// groups; otherwise gate, then up, on the grid of launch_axis1):
// h[m][n] = bf16(silu(g[m][n]) * u[m][n]) from the float32 sums.
hipError_t launch_axis1_swiglu(const uint16_t* x, int M, const uint32_t* codes_g,
                               const float* scales_g, const float* lut_g, const uint32_t* codes_u,
                               const float* scales_u, const float* lut_u, uint16_t* h,
                               CodeLayout lay, int N, int nb, int k, hipStream_t st);

// Axis 0, 1 <= M <= 32: split-K partials of 128-column tiles over ranges of
// the stored rows, then the ordered reduce over them into y[M][C]. `partial`
// holds axis0_partial_floats(R, C, M) floats.
hipError_t launch_axis0(const uint16_t* x, int M, const uint32_t* codes, CodeLayout lay,
                        const float* scales, const float* lut, float* partial, uint16_t* y, int R,
                        int C, int k, hipStream_t st);

// The axis-0 split: every 128-column tile's rows cut into `ranges` ranges,
// one per wave, `waves` waves per workgroup, G workgroups. It depends on R
// and C only (not on the device), so results do not either.
struct A0Plan {
    int G;       // workgroups
    int ranges;  // row ranges per tile
    int waves;   // waves used per workgroup
};
A0Plan axis0_plan(int R, int C);
size_t axis0_partial_floats(int R, int C, int M);

// The scatter variant that allocates nothing keeps its split-K partials in a
// file-scope device array of kStaticScratchFloats floats (2 MB), one per
// device. static_scratch returns the current device's address of it, looked
// up with hipGetSymbolAddress on the first call on that device.
constexpr size_t kStaticScratchFloats = size_t(1) << 19;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(float** ptr);

// Decoded weights w[rows][nb*256].
hipError_t launch_expand(const uint32_t* codes, CodeLayout lay, const float* scales,
                         const float* lut, uint16_t* w, long rows, int nb, int k, hipStream_t st);

// Copy every block of a code array from layout `from` into dst, written
// densely in block-interleave-2 order when dst_pairs, else row-major (src and
// dst must not overlap).
hipError_t launch_repack(const uint32_t* src, CodeLayout from, uint32_t* dst, bool dst_pairs,
                         int rows, int nb, int k, hipStream_t st);

}  // namespace trellis
