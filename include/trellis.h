/*
 * trellis.h -- C ABI of libtrellis.so: fused trellis-dequantize-and-multiply
 * for bitshift-trellis-coded weights on AMD Instinct MI355X (gfx950).
 *
 * The operation (diff views of the npm package "@mlx-bun/inference",
 * 0.0.0-stage -> 1.0.0; page 60: src/kernels/trellis/tiled-prefill.ts,
 * vector-expand.ts, wide-prefill.ts; page 59: scatter.ts, splitk-prefill.ts):
 *
 *   A projection is stored as a matrix [rows][cols] of k-bit codes, cut into
 *   blocks of T = 256 weights along each row. Axis 1 stores [out][in]
 *   (y = x W^T); axis 0 stores [in][out] (y = x W), the storage convention of
 *   tiled-prefill.ts's weight-tile decode.
 *
 *   Codes: uint32 words, T*k/32 per block, in one of two block layouts
 *   (geometry field block_interleave):
 *     0: row-major [rows][cols/T][T*k/32];
 *     2: block pairs outermost, [cols/(2T)][rows][2][T*k/32]: block b of
 *        row r starts at word (b/2)*rows*2*wpb + r*2*wpb + (b%2)*wpb
 *        (page 60 vector-expand.ts and page 59 scatter.ts address a block
 *        so when their INTERLEAVE constant is set); cols/T must be even.
 *   The block is a T*k-bit string, LSB-first within a word, words ascending. Weight t of a
 *   block reads the L = 12 bits starting at bit (T-1-t)*k, wrapping to bit 0
 *   of the same block (tail-biting). That window indexes a 4096-entry float32
 *   codebook; the entry times the row's float32 scale is rounded to float32
 *   and then to bf16 (round-to-nearest-even):
 *       W[r][c] = bf16( fl32( LUT[window(r, c)] * scales[r] ) )
 *   (page 60 tiled-prefill.ts weight-tile decode and wide-prefill.ts; page 59
 *   scatter.ts rounds the scaled value before its multiply-add).
 *   On axis 0 the scale belongs to the stored row, i.e. the input feature.
 *
 *   Outputs are bf16, accumulated in float32. The summation order inside a
 *   call is fixed, so repeated calls give identical bits.
 *
 * Conventions for every compute entry point:
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing and keeps no reference after the call returns.
 *   - x, codes, lut, y and workspace must be 16-byte aligned; scales 4-byte.
 *     Arrays are dense and row-major (no strides).
 *   - Outputs (y, workspace) must not overlap the inputs (x, codes, scales,
 *     lut) or each other: kernels read inputs while other workgroups already
 *     write outputs. Only the overlaps named at an entry point are checked;
 *     any other gives undefined results.
 *   - The arrays and the stream belong to the current HIP device; launch
 *     shapes are sized from its compute-unit count (so bits can differ
 *     between devices with different counts, never between calls on one).
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without waiting. All validation happens on the host before anything is
 *     enqueued: on a negative status nothing was enqueued. A kernel fault
 *     shows up at the caller's next synchronisation.
 *   - Geometry accepted: axis in {0, 1}, T = 256, L = 12, k in {2, 3, 4},
 *     1 <= in_features, out_features <= 2^19, cols % 256 == 0 (cols is
 *     in_features on axis 1, out_features on axis 0), block_interleave in
 *     {0, 2}, and with 2 an even number of blocks per row (cols % 512 == 0).
 *     Every operation gives bit-identical results for either layout.
 */
#ifndef TRELLIS_H
#define TRELLIS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Shape of one coded projection (the pages' TrellisGeometry fields). */
typedef struct trellis_geometry {
    int32_t axis;          /* 1: stored [out][in], y = x W^T; 0: stored [in][out], y = x W */
    int32_t T;             /* weights per block; must be 256 */
    int32_t L;             /* window width in bits; must be 12 */
    int32_t k;             /* bits per weight: 2, 3 or 4 */
    int32_t in_features;
    int32_t out_features;
    int32_t block_interleave;  /* code layout: 0 row-major, 2 block pairs (see above) */
} trellis_geometry;

/* Status codes (0 = success, negative = nothing enqueued). */
enum {
    TRELLIS_OK = 0,
    TRELLIS_ERR_NULL = -1,       /* a required pointer is null */
    TRELLIS_ERR_GEOMETRY = -2,   /* axis, T, L, k, feature counts or M not supported by this op */
    TRELLIS_ERR_ALIGN = -3,      /* a pointer is not aligned as required */
    TRELLIS_ERR_LUT = -4,        /* codebook size is not 2^L, or an entry is not finite */
    TRELLIS_ERR_WORKSPACE = -5,  /* workspace missing or smaller than trellis_workspace_bytes() */
    TRELLIS_ERR_HIP = -6,        /* the HIP runtime reported an error while enqueuing */
    TRELLIS_ERR_OVERLAP = -7     /* source and destination arrays overlap */
};

/* Operation selector for trellis_workspace_bytes(). */
enum {
    TRELLIS_OP_GEMV = 0,
    TRELLIS_OP_GEMV_SCATTER = 1,
    TRELLIS_OP_PREFILL = 2
};

/* Largest activation batch accepted by trellis_prefill (page 60
 * tiled-prefill.ts serves M = 5..32). */
#define TRELLIS_MAX_M 32

/*
 * Copy a host codebook of `entries` float32 values into the caller's device
 * buffer `dev_lut` (4 * entries bytes, 16-byte aligned). The codebook plays
 * the part of the pages' precise host LUT (page 59 scatter.ts stages `lut`
 * into threadgroup memory). entries must be 4096 (2^L with L = 12) and every
 * entry finite, else TRELLIS_ERR_LUT (checked on the host before anything is
 * enqueued). The copy is enqueued on `stream` like any other work and the
 * call returns without waiting: `host_lut` must stay valid and unchanged
 * until the stream has run the copy (synchronise it before freeing or
 * reusing the host array).
 */
int trellis_lut_upload(const float *host_lut, int32_t entries, float *dev_lut,
                       hipStream_t stream);

/*
 * Axis-1 GEMV, one activation row (decode step):
 *   y[n] = bf16( sum_{k < in} x[k] * W[n][k] ),  n < out.
 * x: bf16 [in]; codes: uint32 [out][in*k/32]; scales: float32 [out];
 * lut: float32 [4096] on the device; y: bf16 [out]. g->axis must be 1.
 * Weights as in page 60 wide-prefill.ts (decode, round to bf16, dot, float
 * accumulation, bf16 store).
 */
int trellis_gemv(const uint16_t *x, const uint32_t *codes, const float *scales,
                 const float *lut, const trellis_geometry *g, uint16_t *y,
                 hipStream_t stream);

/*
 * Two axis-1 GEMVs of the same geometry over the same activation row, in one
 * launch: the gate and up projections of a decoder MLP at a decode step.
 *   y_a[n] = bf16( sum_k x[k] * Wa[n][k] ),  y_b[n] = bf16( sum_k x[k] * Wb[n][k] )
 * with Wa from (codes_a, scales_a, lut_a) and Wb from (codes_b, scales_b,
 * lut_b), each laid out as for trellis_gemv; g (axis 1) describes both. The
 * results are bit-identical to two trellis_gemv calls; one launch saves the
 * second launch and its codebook staging. (The pages run each projection on
 * its own, page 60 wide-prefill.ts; the shared launch is this library's.)
 * y_a and y_b must not overlap (TRELLIS_ERR_OVERLAP). For rows too long to
 * stage in one launch the two projections are enqueued one after the other;
 * should the runtime then reject the second launch (TRELLIS_ERR_HIP), the
 * first one stays enqueued.
 */
int trellis_gemv_dual(const uint16_t *x, const uint32_t *codes_a, const float *scales_a,
                      const float *lut_a, uint16_t *y_a, const uint32_t *codes_b,
                      const float *scales_b, const float *lut_b, uint16_t *y_b,
                      const trellis_geometry *g, hipStream_t stream);

/*
 * Axis-0 "scatter" GEMV, one activation row (page 59 scatter.ts: split-K over
 * the stored rows, float32 partials per row range, then their sum and a cast):
 *   partial[s][n] = sum over stored rows r in range s of x[r] * W[r][n]
 *   y[n]          = bf16( sum over s of partial[s][n] ).
 * The stored rows of each 128-column tile are split into the same contiguous
 * ranges, nr of them: 8 P with P = max(1, min(ceil(in / 32), 256 / (out /
 * 128))), or 2048 / (out / 128) (at most ceil(in / 32)) where 8 P ranges
 * would leave a quarter or more of the GPU's 256 compute units idle. The
 * count depends on the geometry only, and every sum runs in a fixed order,
 * so a geometry always gives the same bits. (The pages use 128 ranges; the
 * count only changes the float32 summation order, which is free.)
 * x: bf16 [in]; codes: uint32 [in][out*k/32]; scales: float32 [in];
 * lut: float32 [4096]; y: bf16 [out]. g->axis must be 0.
 * workspace: scratch of at least
 * trellis_workspace_bytes(g, 1, TRELLIS_OP_GEMV_SCATTER) bytes (one 128-wide
 * partial per workgroup and column tile it sums, at most 4096 of them); its
 * contents on entry do not matter and are overwritten. Where every
 * workgroup owns a whole band of ranges of one tile and a tile has at most
 * 8 bands (e.g. 17408 -> 5120), the bands meet in the same launch (here and
 * in the axis-0 prefill up to M = 8): each
 * partial travels as 8-byte words tagged with the call, and a workgroup that
 * finds all of its tile's partials current sums them in range order (the
 * partials take 8 bytes per value then); otherwise, and under stream
 * capture, a second launch sums float32 partials. Calls sharing a workspace
 * must not overlap in time.
 */
int trellis_gemv_scatter(const uint16_t *x, const uint32_t *codes, const float *scales,
                         const float *lut, const trellis_geometry *g, float *workspace,
                         size_t workspace_bytes, uint16_t *y, hipStream_t stream);

/*
 * trellis_gemv_scatter without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the partials go to a static device
 * array of trellis_static_scratch_bytes() bytes (2 MB; one per device, held
 * until the process ends), which covers the scatter of every accepted
 * geometry (at most 4096 partials of 128 floats, or 2048 of 128 tagged
 * words); a geometry needing more would return TRELLIS_ERR_WORKSPACE. The call allocates nothing: the array's device
 * address is looked up once per device on the first call there. Outputs are
 * bit-identical to trellis_gemv_scatter's. Every call on a device shares that
 * device's array, so calls that overlap on one device (concurrent streams,
 * host threads) race and give undefined results; calls ordered on one stream
 * are safe (each overwrites every partial it reads).
 */
int trellis_gemv_scatter_static(const uint16_t *x, const uint32_t *codes, const float *scales,
                                const float *lut, const trellis_geometry *g, uint16_t *y,
                                hipStream_t stream);

/* Bytes of the static partials array of trellis_gemv_scatter_static. */
size_t trellis_static_scratch_bytes(void);

/*
 * Small-batch GEMM (prefill), M activation rows, 0 <= M <= 32 (M = 0 is a
 * no-op that returns TRELLIS_OK):
 *   axis 1: y[m][n] = bf16( sum_k x[m][k] * W[n][k] )   (page 60 tiled-prefill.ts)
 *   axis 0: y[m][n] = bf16( sum_r x[m][r] * W[r][n] )   (page 59 splitk-prefill.ts:
 *           row splits with float32 partials, then an ordered sum)
 * x: bf16 [M][in]; y: bf16 [M][out]; codes/scales/lut as for the GEMVs.
 * workspace: scratch of trellis_workspace_bytes(g, M, TRELLIS_OP_PREFILL)
 * bytes, 16-byte aligned; its contents on entry do not matter. On axis 0 it
 * is required. On axis 1 it is optional: where that size is not 0 (16-row
 * groups left over after whole groups per compute unit, e.g. 17408 output
 * rows), a workspace of it lets the leftover groups be cut by blocks across
 * workgroups, whose parts meet through it (each output still the float32
 * sum of its products, in another order: results within the prefill's
 * tolerance of the call without one, not bit-identical to it); a null
 * workspace keeps whole groups per workgroup; a non-null one that is too
 * small is TRELLIS_ERR_WORKSPACE. A call being captured into a graph does
 * not use it. Calls sharing a workspace must not overlap in time.
 */
int trellis_prefill(const uint16_t *x, int32_t M, const uint32_t *codes, const float *scales,
                    const float *lut, const trellis_geometry *g, float *workspace,
                    size_t workspace_bytes, uint16_t *y, hipStream_t stream);

/*
 * Two axis-1 prefills of the same geometry over the same M activation rows,
 * 0 <= M <= 32: the gate and up projections of a decoder MLP at prefill.
 *   y_a[m][n] = bf16( sum_k x[m][k] * Wa[n][k] ),  y_b likewise with Wb
 * with Wa from (codes_a, scales_a, lut_a) and Wb from (codes_b, scales_b,
 * lut_b), each laid out as for trellis_prefill; g (axis 1) describes both;
 * x: bf16 [M][in]; y_a, y_b: bf16 [M][out], not overlapping
 * (TRELLIS_ERR_OVERLAP). For 2 <= M <= 32 one launch serves both (half the
 * compute units each; the pages run each projection on its own, page 60
 * tiled-prefill.ts, the shared launch is this library's) when each
 * workgroup's rows fit; M = 1 is trellis_gemv_dual; otherwise the two
 * projections are enqueued one after the other, and should the runtime
 * reject the second launch (TRELLIS_ERR_HIP),
 * the first one stays enqueued. Results are within the prefill's tolerance of
 * two trellis_prefill calls, not always bit-identical to them (the shared
 * launch splits rows differently, which changes the float32 summation order).
 */
int trellis_prefill_dual(const uint16_t *x, int32_t M, const uint32_t *codes_a,
                         const float *scales_a, const float *lut_a, uint16_t *y_a,
                         const uint32_t *codes_b, const float *scales_b, const float *lut_b,
                         uint16_t *y_b, const trellis_geometry *g, hipStream_t stream);

/*
 * The gate and up projections of a decoder MLP with their SwiGLU epilogue, in
 * one launch, for 0 <= M <= 32 activation rows (M = 0 is a no-op):
 *   h[m][n] = bf16( silu(g[m][n]) * u[m][n] ),   silu(v) = v / (1 + e^-v),
 *   g[m][n] = sum_k x[m][k] * Wg[n][k],  u[m][n] = sum_k x[m][k] * Wu[n][k]
 * with Wg from (codes_g, scales_g, lut_g) and Wu from (codes_u, scales_u,
 * lut_u), each laid out as for trellis_prefill; g (axis 1) describes both;
 * x: bf16 [M][in]; h: bf16 [M][out], which then feeds the down projection.
 * g and u are the float32 sums (never rounded to bf16), silu is evaluated in
 * float32, and only h is rounded. The pages tune their kernels for the Qwen
 * MLP geometry (page 60 tiled-prefill.ts, its dispatch notes; page 60
 * wide-prefill.ts takes that model's normalised activations) but print no
 * activation function; SwiGLU is that MLP's, and the fused epilogue is this
 * library's. Each workgroup decodes the same row range of both projections
 * (either the gate rows, then the up rows after restaging its codebook table,
 * or, at k = 3, 4 with 17 <= M <= 32, gate and up rows side by side in shared
 * 16-row groups), so both sums of an output meet in one workgroup: no
 * workspace, a fixed summation order (repeated calls give identical bits).
 */
int trellis_gate_up_swiglu(const uint16_t *x, int32_t M, const uint32_t *codes_g,
                           const float *scales_g, const float *lut_g, const uint32_t *codes_u,
                           const float *scales_u, const float *lut_u,
                           const trellis_geometry *g, uint16_t *h, hipStream_t stream);

/*
 * Workspace bytes an operation needs for geometry g and batch M (0 if it
 * needs none). Returns (size_t)-1 if g, M or op is not supported. The
 * workspace holds the split-K float32 partials of the axis-0 operations
 * (page 59 splitk-prefill.ts sizes its workspace as splits x M x N floats
 * and keeps no dense weight buffer): S x M x 128 floats here, S <= 4096 the
 * (workgroup, column tile) partials of trellis_gemv_scatter's split (8-byte
 * tagged words instead of floats where the scatter sums them in one
 * launch). For the
 * axis-1 prefill it is the optional workspace of the leftover 16-row groups'
 * parts (one 16 x 16 or 32 x 16 tile of 8-byte tagged words per compute
 * unit), 0 where there is none to cut or where the cut does not pay.
 */
size_t trellis_workspace_bytes(const trellis_geometry *g, int32_t M, int32_t op);

/*
 * Diagnostic export of the decoded weights (page 60 vector-expand.ts):
 *   w[r][c] = bf16( fl32( LUT[window(r, c)] * scales[r] ) ),  w is bf16 [rows][cols].
 * Uses the same decoder as the fused operations. Not on the hot path.
 */
int trellis_expand(const uint32_t *codes, const float *scales, const float *lut,
                   const trellis_geometry *g, uint16_t *w, hipStream_t stream);

/*
 * Rewrite a code array from one block layout into the other (page 60
 * vector-expand.ts / page 59 scatter.ts INTERLEAVE addressing; a one-time
 * conversion, not on the hot path). g describes the projection and
 * g->block_interleave the layout of `src`; `to_block_interleave` (0 or 2)
 * is the layout written to `dst`, which must then also satisfy the geometry
 * rules (2 needs cols % 512 == 0). src and dst: device uint32 arrays of
 * rows*cols*k/32 words, 16-byte aligned, not overlapping
 * (TRELLIS_ERR_OVERLAP). Equal layouts make a plain copy.
 */
int trellis_repack(const uint32_t *src, uint32_t *dst, const trellis_geometry *g,
                   int32_t to_block_interleave, hipStream_t stream);

/* Static, human-readable text for a status code (the entry points reject
 * unsupported input before any launch, as page 60 tiled-prefill.ts throws
 * before dispatching; this names the reason). */
const char *trellis_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_H */
