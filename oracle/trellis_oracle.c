/*
 * CPU oracle for the trellis dequantize-and-multiply path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it. It shares no code, header, table or constant with
 * the HIP library.
 *
 * It is a plain, slow, single-threaded rendering of the definition:
 *   W[r][c] = bf16_rne( fl32( LUT[window(r, c)] * scale[r] ) )
 *   y       = x . W^T   (axis 1)      y = x . W   (axis 0)
 * with the contraction accumulated in double precision, input index
 * ascending. Build with -O2 -fno-fast-math -ffp-contract=off so the float
 * product is one IEEE round-to-nearest-even multiply, never contracted.
 *
 * Pages cited (diff views of the npm package "@mlx-bun/inference",
 * 0.0.0-stage -> 1.0.0):
 *   [P60] page 60: src/kernels/trellis/tiled-prefill.ts, vector-expand.ts,
 *         wide-prefill.ts
 *   [P59] page 59: src/kernels/trellis/scatter.ts, splitk-prefill.ts
 *
 * Readings taken where the pages are silent (each is listed with its
 * reason in the design notes):
 *   - the bitstream of a block is read LSB-first inside each 32-bit word,
 *     words ascending ([P60] tiled-prefill.ts weight-tile decode, which
 *     forms a window as low word >> off | next word << (32 - off));
 *   - the window wraps inside its own block (tail-biting): bit positions
 *     are taken modulo T*k ([P60] same passage: the word after the last
 *     word of a block is word 0 of that block);
 *   - the codebook is an uploaded 4096-entry float32 table used verbatim;
 *   - the rounding is the float32 product first, then bf16
 *     round-to-nearest-even ([P60] tiled-prefill.ts casts value*scale to
 *     the activation type; [P59] scatter.ts rounds value*scale before the
 *     multiply-add);
 *   - on axis 0 the scale belongs to the stored row, i.e. the input index
 *     ([P59] scatter.ts reads scales[r] inside its row loop);
 *   - the code array is row-major [rows][cols/T][T*k/32] (block interleave
 *     0), or, with block interleave 2, pairs of blocks outermost: the words
 *     of block b of row r start at (b/2)*rows*2*wpb + r*2*wpb + (b%2)*wpb
 *     ([P60] vector-expand.ts and [P59] scatter.ts, splitk-prefill.ts
 *     address a block this way when their INTERLEAVE constant is set). The
 *     pages give no layout for an odd block count under interleave 2, so it
 *     is rejected.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 round-to-nearest-even of a finite float32, textbook bit method: add
 * 0x7FFF plus the lowest kept bit, keep the high half. */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Element-wise form of oracle_bf16_rne over n values. */
void oracle_bf16_rne_n(const float *f, long n, uint16_t *out)
{
    for (long i = 0; i < n; ++i) out[i] = oracle_bf16_rne(f[i]);
}

double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Storage convention ([P60] tiled-prefill.ts: row = n, col = k on axis 1;
 * row = k, col = n on axis 0). Returns 0 on an unsupported geometry. */
static int oracle_dims(int axis, int in_features, int out_features, int *rows, int *cols)
{
    if (axis == 1) { *rows = out_features; *cols = in_features; return 1; }
    if (axis == 0) { *rows = in_features; *cols = out_features; return 1; }
    return 0;
}

/* Word offset of block b of stored row r in the code array, for block
 * interleave 0 or 2 (see the header). Returns -1 for any other layout, or for
 * interleave 2 with an odd block count. */
static long oracle_block_word(long r, long b, long rows, long nb, long wpb, int interleave)
{
    if (interleave == 0) return (r * nb + b) * wpb;
    if (interleave == 2 && nb % 2 == 0) return (b / 2) * rows * 2 * wpb + r * 2 * wpb + (b % 2) * wpb;
    return -1;
}

/* Bit i of a block's bitstring, i in [0, T*k): bit (i mod 32) of word i/32. */
static unsigned oracle_bit(const uint32_t *block, long i)
{
    return (unsigned)((block[i / 32] >> (i % 32)) & 1u);
}

/* Unpack a block into an explicit array of T*k bits. */
void oracle_block_bits(const uint32_t *block, int T, int k, uint8_t *bits)
{
    for (long i = 0; i < (long)T * k; ++i)
        bits[i] = (uint8_t)oracle_bit(block, i);
}

/* Window of weight t: the L bits starting at bit (T-1-t)*k, wrapping around
 * the end of the block's T*k-bit string, bit j of the window = bit p+j of the
 * string ([P60] tiled-prefill.ts, weight-tile decode). */
uint32_t oracle_window_from_bits(const uint8_t *bits, int T, int k, int L, int t)
{
    const long n = (long)T * k;
    const long p = (long)(T - 1 - t) * k;
    uint32_t w = 0;
    for (int j = 0; j < L; ++j)
        w |= (uint32_t)bits[(p + j) % n] << j;
    return w;
}

/* The same window read straight from the words (no unpacked array). */
uint32_t oracle_window(const uint32_t *block, int T, int k, int L, int t)
{
    const long n = (long)T * k;
    const long p = (long)(T - 1 - t) * k;
    uint32_t w = 0;
    for (int j = 0; j < L; ++j)
        w |= (uint32_t)oracle_bit(block, (p + j) % n) << j;
    return w;
}

/* One decoded weight: float32 product of the codebook entry and the row
 * scale, then bf16 round-to-nearest-even. */
uint16_t oracle_weight(float value, float scale)
{
    volatile float product = value * scale;
    return oracle_bf16_rne(product);
}

/* Expand the whole stored matrix to bf16 W[rows][cols] ([P60]
 * vector-expand.ts computes the same matrix). `interleave` is the code
 * array's block interleave (0 or 2). Returns 0 on bad geometry. */
int oracle_expand(const uint32_t *codes, const float *scales, const float *lut,
                  int axis, int T, int L, int k, int in_features, int out_features,
                  int interleave, uint16_t *W)
{
    int rows, cols;
    if (!oracle_dims(axis, in_features, out_features, &rows, &cols)) return 0;
    if (T <= 0 || k <= 0 || cols % T != 0 || ((long)T * k) % 32 != 0) return 0;
    const int nb = cols / T;
    const int wpb = T * k / 32;
    if (oracle_block_word(0, 0, rows, nb, wpb, interleave) < 0) return 0;
    uint8_t *bits = (uint8_t *)malloc((size_t)T * k);
    if (!bits) return 0;
    for (long r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            oracle_block_bits(codes + oracle_block_word(r, b, rows, nb, wpb, interleave), T, k, bits);
            for (int t = 0; t < T; ++t) {
                uint32_t win = oracle_window_from_bits(bits, T, k, L, t);
                W[(size_t)r * cols + (size_t)b * T + t] = oracle_weight(lut[win], scales[r]);
            }
        }
    }
    free(bits);
    return 1;
}

/* y[m][n] = sum_k x[m][k] * W(n, k) in double, k ascending, where W(n, k)
 * is W[n][k] on axis 1 and W[k][n] on axis 0. x and W are bf16 bits. */
int oracle_matmul_f64(const uint16_t *x, int M, const uint16_t *W,
                      int axis, int in_features, int out_features, double *y)
{
    for (long m = 0; m < M; ++m) {
        for (long n = 0; n < out_features; ++n) {
            double acc = 0.0;
            for (long kk = 0; kk < in_features; ++kk) {
                size_t wi = axis == 1 ? (size_t)n * in_features + kk
                                      : (size_t)kk * out_features + n;
                acc += oracle_bf16_to_f64(x[(size_t)m * in_features + kk]) *
                       oracle_bf16_to_f64(W[wi]);
            }
            y[(size_t)m * out_features + n] = acc;
        }
    }
    return 1;
}

/* Fused form: each weight is decoded from the words inside the contraction
 * loop (no materialised W). Same products and the same summation order as
 * oracle_expand followed by oracle_matmul_f64. Rows [n_begin, n_end) of the
 * output (all M of them) are computed; pass 0, out_features for all.
 * `interleave` is the code array's block interleave (0 or 2). */
int oracle_fused_f64(const uint16_t *x, int M, const uint32_t *codes, const float *scales,
                     const float *lut, int axis, int T, int L, int k,
                     int in_features, int out_features, int interleave,
                     int n_begin, int n_end, double *y)
{
    int rows, cols;
    if (!oracle_dims(axis, in_features, out_features, &rows, &cols)) return 0;
    if (T <= 0 || k <= 0 || cols % T != 0 || ((long)T * k) % 32 != 0) return 0;
    if (M < 1 || M > 64) return 0;
    const int nb = cols / T;
    const int wpb = T * k / 32;
    if (oracle_block_word(0, 0, rows, nb, wpb, interleave) < 0) return 0;
    double acc[64];
    for (long n = n_begin; n < n_end; ++n) {
        for (int m = 0; m < M; ++m) acc[m] = 0.0;
        for (long kk = 0; kk < in_features; ++kk) {
            long r = axis == 1 ? n : kk;   /* stored row */
            long c = axis == 1 ? kk : n;   /* stored column */
            const uint32_t *block = codes + oracle_block_word(r, c / T, rows, nb, wpb, interleave);
            uint32_t win = oracle_window(block, T, k, L, (int)(c % T));
            double w = oracle_bf16_to_f64(oracle_weight(lut[win], scales[r]));
            for (int m = 0; m < M; ++m)
                acc[m] += oracle_bf16_to_f64(x[(size_t)m * in_features + kk]) * w;
        }
        for (int m = 0; m < M; ++m) y[(size_t)m * out_features + n] = acc[m];
    }
    return 1;
}

/* ---------------------------------------------------------------------------
 * SwiGLU epilogue of a decoder MLP's gate and up projections.
 *
 * The pages tune their kernels for the Qwen MLP geometry (the prefill's
 * dispatch notes in [P60] tiled-prefill.ts; [P60] wide-prefill.ts takes the
 * RMSNorm output of such a model as its activations) but print no activation
 * function. The plainest reading of that MLP, taken here, is the SwiGLU of
 * the gate and up projections, h = silu(g) * u with silu(v) = v / (1 + e^-v),
 * whose product feeds the down projection. Computed in double from the
 * double contraction results; the GPU's h (bf16) is compared to it within the
 * output tolerance.
 */
#include <math.h>

/* silu(v) = v * sigmoid(v) = v / (1 + exp(-v)), in double. */
double oracle_silu(double v)
{
    return v / (1.0 + exp(-v));
}

/* h[i] = silu(g[i]) * u[i] for i < n, in double. */
void oracle_swiglu_f64(const double *g, const double *u, long n, double *h)
{
    for (long i = 0; i < n; ++i) h[i] = oracle_silu(g[i]) * u[i];
}
