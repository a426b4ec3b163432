/*
 * trellis_probe.h -- measurement support in libtrellis.so: the rate at which
 * an MI355X (gfx950) compute unit serves random reads of a decode table in
 * LDS. It is not part of the dequantize-and-multiply operation; the benchmark
 * uses it as the decode ceiling that the fused kernels are measured against.
 *
 * The operation it prices (diff views of the npm package "@mlx-bun/inference",
 * 0.0.0-stage -> 1.0.0; page 59 scatter.ts stages the codebook in threadgroup
 * memory and decodes each weight by reading it at the weight's window; page 60
 * tiled-prefill.ts's weight-tile decode reads it the same way) is one table read
 * per decoded weight, at a uniformly random index when the codes are uniformly
 * random.
 *
 * Conventions as in trellis.h: `out` is a caller-owned device array, work is
 * enqueued on `stream` and the call returns without waiting; on a nonzero
 * status nothing was enqueued.
 */
#ifndef TRELLIS_PROBE_H
#define TRELLIS_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Table layouts (the decode tables of the kernels). */
enum {
    TRELLIS_PROBE_PAIR_B64 = 0,     /* k = 2 pair table: 16384 x 8 bytes, 8-byte reads, 2 weights each */
    TRELLIS_PROBE_COPIES8_B32 = 1,  /* codebook in 8 bank-partitioned copies, 4-byte reads */
    TRELLIS_PROBE_SINGLE_B32 = 2    /* the plain 4096-entry codebook, 4-byte reads */
};

enum {
    TRELLIS_PROBE_ERR_ARG = -2,  /* kind, rounds or out not valid (out too small or null) */
    TRELLIS_PROBE_ERR_HIP = -6   /* the HIP runtime rejected the launch */
};

/*
 * Enqueue one probe launch: one 512-thread workgroup per compute unit of the
 * current device, each lane reading the table of `kind` 32 * rounds times at
 * uniformly random entries (0 <= rounds <= 2^20), and storing one float (the
 * sum of what it read, to keep the reads live) to out[lane]. `out` is a device
 * float array of at least trellis_gather_probe_out_floats() elements, 4-byte
 * aligned. Time two launches that differ only in `rounds`: the difference
 * divided by the difference of trellis_gather_probe_values() is the time per
 * decoded weight of a gather-only decode.
 */
int trellis_gather_probe(int32_t kind, int32_t rounds, float *out, size_t out_floats,
                         hipStream_t stream);

/* Decoded-weight values one launch reads in its timed loop (two per 8-byte
 * pair-table read), over the whole device; 0 for an invalid kind or rounds. */
uint64_t trellis_gather_probe_values(int32_t kind, int32_t rounds);

/* Elements of `out` that trellis_gather_probe writes on the current device. */
size_t trellis_gather_probe_out_floats(void);

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_PROBE_H */
