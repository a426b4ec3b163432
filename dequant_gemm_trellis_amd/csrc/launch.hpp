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

// Axis-1 GEMV (M = 1): persistent kernel, one workgroup per compute unit,
// activations staged in LDS. Needs nb <= gemv_max_blocks(k).
hipError_t launch_gemv(const uint16_t* x, const uint32_t* codes, const float* scales,
                       const float* lut, uint16_t* y, int N, int nb, int k, hipStream_t st);
int gemv_max_blocks(int k);

// Axis 1, 1 <= M <= 32: y[M][N] from x[M][nb*256] and codes [N][nb][8k].
// Persistent workgroups of at most 80 rows; any nb.
hipError_t launch_axis1(const uint16_t* x, int M, const uint32_t* codes, const float* scales,
                        const float* lut, uint16_t* y, int N, int nb, int k, hipStream_t st);

// Axis 0, 1 <= M <= 32: per-part partials, then the ordered reduce over the
// parts into y[M][C]. `partial` holds axis0_parts(R, C) * M * C floats.
hipError_t launch_axis0(const uint16_t* x, int M, const uint32_t* codes, const float* scales,
                        const float* lut, float* partial, uint16_t* y, int R, int C, int k,
                        hipStream_t st);
int axis0_parts(int R, int C);

// Decoded weights w[rows][nb*256].
hipError_t launch_expand(const uint32_t* codes, const float* scales, const float* lut,
                         uint16_t* w, long rows, int nb, int k, hipStream_t st);

}  // namespace trellis
