// C-ABI entry points of libtrellis.so: argument validation on the host, then
// kernel launches on the caller's stream. Nothing is enqueued unless every
// check passes. Semantics of each entry point are documented in trellis.h.
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0;
// page 60 tiled-prefill.ts and wide-prefill.ts reject unsupported geometry
// (T 256, L 12, k 2/3/4, cols a multiple of 256) before any launch; page 60
// vector-expand.ts and page 59 scatter.ts define the block-interleave-2 code
// layout.
#include <math.h>
#include <stdint.h>

#include "launch.hpp"
#include "trellis.h"

namespace {

constexpr int32_t kMaxFeatures = 1 << 19;
constexpr uint64_t kMaxWeights = 1ull << 40;

struct Dims {
    int rows, cols, nb;
    trellis::CodeLayout lay;
};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_geometry(const trellis_geometry* g, Dims* d) {
    if (!g) return TRELLIS_ERR_NULL;
    if (g->axis != 0 && g->axis != 1) return TRELLIS_ERR_GEOMETRY;
    if (g->T != 256 || g->L != 12) return TRELLIS_ERR_GEOMETRY;
    if (g->k < 2 || g->k > 4) return TRELLIS_ERR_GEOMETRY;
    if (g->in_features < 1 || g->out_features < 1) return TRELLIS_ERR_GEOMETRY;
    if (g->in_features > kMaxFeatures || g->out_features > kMaxFeatures) return TRELLIS_ERR_GEOMETRY;
    d->rows = g->axis == 1 ? g->out_features : g->in_features;
    d->cols = g->axis == 1 ? g->in_features : g->out_features;
    if (d->cols % g->T != 0) return TRELLIS_ERR_GEOMETRY;
    if (static_cast<uint64_t>(d->rows) * static_cast<uint64_t>(d->cols) > kMaxWeights)
        return TRELLIS_ERR_GEOMETRY;
    d->nb = d->cols / g->T;
    if (g->block_interleave != 0 && g->block_interleave != 2) return TRELLIS_ERR_GEOMETRY;
    if (g->block_interleave == 2 && d->nb % 2 != 0) return TRELLIS_ERR_GEOMETRY;
    d->lay = trellis::code_layout(g->block_interleave, d->rows, d->nb, g->k);
    return TRELLIS_OK;
}

// Operand checks shared by the compute entry points.
int check_operands(const void* codes, const float* scales, const float* lut) {
    if (!codes || !scales || !lut) return TRELLIS_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(lut, 16) || !aligned(scales, 4)) return TRELLIS_ERR_ALIGN;
    return TRELLIS_OK;
}

int check_io(const void* x, const void* y) {
    if (!x || !y) return TRELLIS_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16)) return TRELLIS_ERR_ALIGN;
    return TRELLIS_OK;
}

// Axis-0 workspace: the float32 partials of the split contraction, one
// M x 128 block per (workgroup, column tile) share.
size_t axis0_workspace(const Dims& d, int M) {
    return trellis::axis0_partial_floats(d.rows, d.cols, M) * sizeof(float);
}

int status_of(hipError_t e) { return e == hipSuccess ? TRELLIS_OK : TRELLIS_ERR_HIP; }

// Axis 1, M activation rows. M = 1: the persistent GEMV kernel, which stages
// the whole activation vector in LDS. Up to 4 rows (and single rows too long
// for that staging): the GEMV's unit mapping with M outputs per unit, when
// the workgroups own at least 16 rows whose partials fit in LDS. Otherwise
// the tiled kernel of 16-row groups.
hipError_t launch_axis1_any(const uint16_t* x, int M, const uint32_t* codes, const float* scales,
                            const float* lut, uint16_t* y, const Dims& d, int k, hipStream_t st,
                            float* workspace = nullptr, size_t workspace_bytes = 0) {
    if (M == 1 && d.nb <= trellis::gemv_max_blocks(k))
        return trellis::launch_gemv(x, codes, d.lay, scales, lut, y, d.rows, d.nb, k, st);
    if (trellis::gemv_rows_supported(M, d.rows, d.nb, k))
        return trellis::launch_gemv_rows(x, M, codes, d.lay, scales, lut, y, d.rows, d.nb, k, st);
    return trellis::launch_axis1(x, M, codes, d.lay, scales, lut, y, d.rows, d.nb, k, workspace,
                                 workspace_bytes, st);
}

// Axis-1 workspace at M rows: the balanced plan's, when the 16-row-group
// kernel serves M and the plan applies; else none.
size_t axis1_workspace(const Dims& d, int M, int k) {
    if (M < 1 || (M == 1 && d.nb <= trellis::gemv_max_blocks(k)) ||
        trellis::gemv_rows_supported(M, d.rows, d.nb, k))
        return 0;
    return trellis::axis1_split_bytes(M, d.rows, d.nb, k);
}

}  // namespace

extern "C" {

int trellis_lut_upload(const float* host_lut, int32_t entries, float* dev_lut, hipStream_t stream) {
    if (!host_lut || !dev_lut) return TRELLIS_ERR_NULL;
    if (entries != 4096) return TRELLIS_ERR_LUT;
    if (!aligned(dev_lut, 16)) return TRELLIS_ERR_ALIGN;
    for (int i = 0; i < entries; ++i)
        if (!isfinite(host_lut[i])) return TRELLIS_ERR_LUT;
    const size_t bytes = static_cast<size_t>(entries) * sizeof(float);
    return status_of(hipMemcpyAsync(dev_lut, host_lut, bytes, hipMemcpyHostToDevice, stream));
}

int trellis_gemv(const uint16_t* x, const uint32_t* codes, const float* scales, const float* lut,
                 const trellis_geometry* g, uint16_t* y, hipStream_t stream) {
    Dims d;
    int st = check_geometry(g, &d);
    if (st) return st;
    if (g->axis != 1) return TRELLIS_ERR_GEOMETRY;
    if ((st = check_operands(codes, scales, lut)) || (st = check_io(x, y))) return st;
    return status_of(launch_axis1_any(x, 1, codes, scales, lut, y, d, g->k, stream));
}

int trellis_gemv_dual(const uint16_t* x, const uint32_t* codes_a, const float* scales_a,
                      const float* lut_a, uint16_t* y_a, const uint32_t* codes_b,
                      const float* scales_b, const float* lut_b, uint16_t* y_b,
                      const trellis_geometry* g, hipStream_t stream) {
    Dims d;
    int st = check_geometry(g, &d);
    if (st) return st;
    if (g->axis != 1) return TRELLIS_ERR_GEOMETRY;
    if ((st = check_operands(codes_a, scales_a, lut_a)) || (st = check_io(x, y_a)) ||
        (st = check_operands(codes_b, scales_b, lut_b)) || (st = check_io(x, y_b)))
        return st;
    const uintptr_t a = reinterpret_cast<uintptr_t>(y_a), b = reinterpret_cast<uintptr_t>(y_b);
    const uintptr_t bytes = static_cast<uintptr_t>(d.rows) * sizeof(uint16_t);
    if (a < b + bytes && b < a + bytes) return TRELLIS_ERR_OVERLAP;
    if (d.nb <= trellis::gemv_max_blocks(g->k))
        return status_of(trellis::launch_gemv_dual(x, codes_a, scales_a, lut_a, y_a, codes_b,
                                                   scales_b, lut_b, y_b, d.lay, d.rows, d.nb,
                                                   g->k, stream));
    // rows too long to stage: the two projections one after the other
    if ((st = status_of(launch_axis1_any(x, 1, codes_a, scales_a, lut_a, y_a, d, g->k, stream))))
        return st;
    return status_of(launch_axis1_any(x, 1, codes_b, scales_b, lut_b, y_b, d, g->k, stream));
}

int trellis_gemv_scatter(const uint16_t* x, const uint32_t* codes, const float* scales,
                         const float* lut, const trellis_geometry* g, float* workspace,
                         size_t workspace_bytes, uint16_t* y, hipStream_t stream) {
    Dims d;
    int st = check_geometry(g, &d);
    if (st) return st;
    if (g->axis != 0) return TRELLIS_ERR_GEOMETRY;
    if ((st = check_operands(codes, scales, lut)) || (st = check_io(x, y))) return st;
    if (!workspace) return TRELLIS_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return TRELLIS_ERR_ALIGN;
    if (workspace_bytes < axis0_workspace(d, 1)) return TRELLIS_ERR_WORKSPACE;
    return status_of(trellis::launch_axis0(x, 1, codes, d.lay, scales, lut, workspace, y, d.rows,
                                           d.cols, g->k, stream));
}

int trellis_gemv_scatter_static(const uint16_t* x, const uint32_t* codes, const float* scales,
                                const float* lut, const trellis_geometry* g, uint16_t* y,
                                hipStream_t stream) {
    Dims d;
    int st = check_geometry(g, &d);
    if (st) return st;
    if (g->axis != 0) return TRELLIS_ERR_GEOMETRY;
    if ((st = check_operands(codes, scales, lut)) || (st = check_io(x, y))) return st;
    if (axis0_workspace(d, 1) > trellis_static_scratch_bytes()) return TRELLIS_ERR_WORKSPACE;
    float* partial = nullptr;
    if (trellis::static_scratch(&partial) != hipSuccess) return TRELLIS_ERR_HIP;
    return status_of(trellis::launch_axis0(x, 1, codes, d.lay, scales, lut, partial, y, d.rows,
                                           d.cols, g->k, stream));
}

size_t trellis_static_scratch_bytes(void) {
    return trellis::kStaticScratchFloats * sizeof(float);
}

int trellis_prefill(const uint16_t* x, int32_t M, const uint32_t* codes, const float* scales,
                    const float* lut, const trellis_geometry* g, float* workspace,
                    size_t workspace_bytes, uint16_t* y, hipStream_t stream) {
    Dims d;
    int st = check_geometry(g, &d);
    if (st) return st;
    if (M < 0 || M > TRELLIS_MAX_M) return TRELLIS_ERR_GEOMETRY;
    if (M == 0) return TRELLIS_OK;
    if ((st = check_operands(codes, scales, lut)) || (st = check_io(x, y))) return st;
    if (g->axis == 1) {
        // the workspace is optional here: without one, the unbalanced plan
        if (workspace) {
            if (!aligned(workspace, 16)) return TRELLIS_ERR_ALIGN;
            if (workspace_bytes < axis1_workspace(d, M, g->k)) return TRELLIS_ERR_WORKSPACE;
        }
        return status_of(launch_axis1_any(x, M, codes, scales, lut, y, d, g->k, stream, workspace,
                                          workspace ? workspace_bytes : 0));
    }
    if (!workspace) return TRELLIS_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return TRELLIS_ERR_ALIGN;
    if (workspace_bytes < axis0_workspace(d, M)) return TRELLIS_ERR_WORKSPACE;
    return status_of(trellis::launch_axis0(x, M, codes, d.lay, scales, lut, workspace, y, d.rows,
                                           d.cols, g->k, stream));
}

int trellis_prefill_dual(const uint16_t* x, int32_t M, const uint32_t* codes_a,
                         const float* scales_a, const float* lut_a, uint16_t* y_a,
                         const uint32_t* codes_b, const float* scales_b, const float* lut_b,
                         uint16_t* y_b, const trellis_geometry* g, hipStream_t stream) {
    Dims d;
    int st = check_geometry(g, &d);
    if (st) return st;
    if (g->axis != 1) return TRELLIS_ERR_GEOMETRY;
    if (M < 0 || M > TRELLIS_MAX_M) return TRELLIS_ERR_GEOMETRY;
    if ((st = check_operands(codes_a, scales_a, lut_a)) || (st = check_io(x, y_a)) ||
        (st = check_operands(codes_b, scales_b, lut_b)) || (st = check_io(x, y_b)))
        return st;
    const uintptr_t a = reinterpret_cast<uintptr_t>(y_a), b = reinterpret_cast<uintptr_t>(y_b);
    const uintptr_t bytes = static_cast<uintptr_t>(M) * static_cast<uintptr_t>(d.rows) * sizeof(uint16_t);
    if (a < b + bytes && b < a + bytes) return TRELLIS_ERR_OVERLAP;
    if (M == 0) return TRELLIS_OK;
    if (M == 1)
        return trellis_gemv_dual(x, codes_a, scales_a, lut_a, y_a, codes_b, scales_b, lut_b, y_b,
                                 g, stream);
    // 2..32 rows: one launch of the 16-row-group kernel over both projections
    // (at 5120 -> 17408 measured 16-24% faster than two launches at 5..16
    // rows, and 10-13% faster than two launches of the small-batch kernel at
    // 2..4). Row ranges too long for one launch take one per projection.
    if (trellis::axis1_dual_supported(M, d.rows, g->k))
        return status_of(trellis::launch_axis1_dual(x, M, codes_a, scales_a, lut_a, y_a, codes_b,
                                                    scales_b, lut_b, y_b, d.lay, d.rows, d.nb,
                                                    g->k, stream));
    if ((st = status_of(launch_axis1_any(x, M, codes_a, scales_a, lut_a, y_a, d, g->k, stream))))
        return st;
    return status_of(launch_axis1_any(x, M, codes_b, scales_b, lut_b, y_b, d, g->k, stream));
}

int trellis_gate_up_swiglu(const uint16_t* x, int32_t M, const uint32_t* codes_g,
                           const float* scales_g, const float* lut_g, const uint32_t* codes_u,
                           const float* scales_u, const float* lut_u, const trellis_geometry* g,
                           uint16_t* h, hipStream_t stream) {
    Dims d;
    int st = check_geometry(g, &d);
    if (st) return st;
    if (g->axis != 1) return TRELLIS_ERR_GEOMETRY;
    if (M < 0 || M > TRELLIS_MAX_M) return TRELLIS_ERR_GEOMETRY;
    if ((st = check_operands(codes_g, scales_g, lut_g)) ||
        (st = check_operands(codes_u, scales_u, lut_u)) || (st = check_io(x, h)))
        return st;
    if (M == 0) return TRELLIS_OK;
    // One row whose activations fit the GEMV's staging: the GEMV mapping;
    // otherwise the 16-row-group kernel (any row length, 1..32 rows).
    if (M == 1 && d.nb <= trellis::gemv_max_blocks(g->k))
        return status_of(trellis::launch_gemv_swiglu(x, codes_g, scales_g, lut_g, codes_u, scales_u,
                                                     lut_u, h, d.lay, d.rows, d.nb, g->k, stream));
    return status_of(trellis::launch_axis1_swiglu(x, M, codes_g, scales_g, lut_g, codes_u, scales_u,
                                                  lut_u, h, d.lay, d.rows, d.nb, g->k, stream));
}

size_t trellis_workspace_bytes(const trellis_geometry* g, int32_t M, int32_t op) {
    Dims d;
    if (check_geometry(g, &d)) return static_cast<size_t>(-1);
    switch (op) {
    case TRELLIS_OP_GEMV:
        return (g->axis == 1 && M == 1) ? 0 : static_cast<size_t>(-1);
    case TRELLIS_OP_GEMV_SCATTER:
        return (g->axis == 0 && M == 1) ? axis0_workspace(d, 1) : static_cast<size_t>(-1);
    case TRELLIS_OP_PREFILL:
        if (M < 0 || M > TRELLIS_MAX_M) return static_cast<size_t>(-1);
        if (M == 0) return 0;
        return g->axis == 1 ? axis1_workspace(d, M, g->k) : axis0_workspace(d, M);
    default:
        return static_cast<size_t>(-1);
    }
}

int trellis_expand(const uint32_t* codes, const float* scales, const float* lut,
                   const trellis_geometry* g, uint16_t* w, hipStream_t stream) {
    Dims d;
    int st = check_geometry(g, &d);
    if (st) return st;
    if ((st = check_operands(codes, scales, lut))) return st;
    if (!w) return TRELLIS_ERR_NULL;
    if (!aligned(w, 16)) return TRELLIS_ERR_ALIGN;
    return status_of(
        trellis::launch_expand(codes, d.lay, scales, lut, w, d.rows, d.nb, g->k, stream));
}

int trellis_repack(const uint32_t* src, uint32_t* dst, const trellis_geometry* g,
                   int32_t to_block_interleave, hipStream_t stream) {
    Dims d;
    int st = check_geometry(g, &d);
    if (st) return st;
    trellis_geometry to = *g;
    to.block_interleave = to_block_interleave;
    Dims dt;
    if ((st = check_geometry(&to, &dt))) return st;
    if (!src || !dst) return TRELLIS_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16)) return TRELLIS_ERR_ALIGN;
    const uint64_t bytes = static_cast<uint64_t>(d.rows) * static_cast<uint64_t>(d.cols) *
                           static_cast<uint64_t>(g->k) / 8;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), t0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < t0 + bytes && t0 < s0 + bytes) return TRELLIS_ERR_OVERLAP;
    return status_of(trellis::launch_repack(src, d.lay, dst, to_block_interleave == 2, d.rows, d.nb,
                                            g->k, stream));
}

const char* trellis_strerror(int status) {
    switch (status) {
    case TRELLIS_OK: return "success";
    case TRELLIS_ERR_NULL: return "a required pointer is null";
    case TRELLIS_ERR_GEOMETRY: return "unsupported geometry, axis or batch size for this operation";
    case TRELLIS_ERR_ALIGN: return "a pointer is not aligned as required (16 bytes; scales 4)";
    case TRELLIS_ERR_LUT: return "codebook must hold 4096 finite float32 entries";
    case TRELLIS_ERR_WORKSPACE: return "workspace missing or too small";
    case TRELLIS_ERR_HIP: return "HIP runtime error while enqueuing work";
    case TRELLIS_ERR_OVERLAP: return "source and destination arrays overlap";
    default: return "unknown trellis status";
    }
}

}  // extern "C"
