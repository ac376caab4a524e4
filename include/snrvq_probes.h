/* snrvq_probes.h -- micro-benchmarks of the part's own rates
 * (libsnrvq_probes.so), the ceilings the decoder's kernels are measured
 * against beside the published peaks: matrix-core throughput with no memory
 * traffic, LDS read bandwidth, Snake throughput on the vector ALU, and MFMA
 * and Snake work issued by the same waves.  Not part of the decoder's
 * boundary (include/snrvq.h); measurement only.
 *
 * Every call runs on the current HIP device and stream 0: one untimed
 * launch, then `reps` timed launches of a grid of (CUs x waves_per_simd)
 * work-groups of 256 threads (one wave per SIMD each), `iters` loop
 * iterations per wave.  It allocates one small device buffer (a record per
 * wave) and frees it before returning.  Return value: 0 on success, 1 for an
 * argument out of range, 2 if the buffer cannot be allocated, 3 for a HIP
 * error while running.
 */
#ifndef SNRVQ_PROBES_H
#define SNRVQ_PROBES_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct probe_result {
    double us;        /* wall time of one launch (HIP events), microseconds */
    double rate;      /* the probe's rate; unit per call below */
    double clock_ghz; /* mean shader clock of the waves (cycle counter against the 100 MHz counter) */
} probe_result;

/* Compute units of the current device. */
int probe_cu_count(void);

/* Independent MFMA chains, accumulators updated in place, no memory traffic:
 * kind 0: 8 chains of v_mfma_f32_16x16x32_f16 per wave; kind 1: 4 chains of
 * v_mfma_f32_32x32x16_f16.  rate: TFLOP/s.  waves_per_simd 1..8. */
int probe_mfma(int kind, int waves_per_simd, int iters, int reps, probe_result *res);

/* Conflict-free 16-byte LDS reads (64 consecutive slots per read, 8 reads
 * per iteration) from a 64 KiB array per work-group (16 KiB above two waves
 * per SIMD).  rate: TB/s over all CUs.  waves_per_simd 1..8. */
int probe_lds(int waves_per_simd, int iters, int reps, probe_result *res);

/* Global -> LDS direct loads (global_load_lds, 16 bytes per lane) from a
 * 256 KiB source resident in L2: 8 KiB per wave per iteration, all waited
 * for before the next.  rate: TB/s over all CUs.  waves_per_simd 1..4. */
int probe_gload(int waves_per_simd, int iters, int reps, probe_result *res);

/* HBM streaming: y = x + 1 over two buffers of `mib` MiB each (64..8192),
 * grid of CUs x blocks_per_cu work-groups (1..32), 16-byte loads and stores.
 * rate: GB/s of reads plus writes.  clock_ghz is not measured (0).  The two
 * buffers are allocated and freed by the call. */
int probe_hbm(int mib, int blocks_per_cu, int reps, probe_result *res);

/* MFMA and Snake chains in the same waves, 8 MFMAs (16x16x32 f16) and 16
 * Snakes (x + sin^2(2 pi frac(x a)) / alpha, 5 VALU instructions) per
 * iteration: mode 0 Snakes only, 1 MFMAs only, 2 both in separate blocks,
 * 3 both interleaved (one MFMA, then two Snakes).  rate: Snakes per second
 * (modes 0, 2, 3) or TFLOP/s (mode 1).  waves_per_simd 1..8. */
int probe_overlap(int mode, int waves_per_simd, int iters, int reps, probe_result *res);

#ifdef __cplusplus
}
#endif

#endif /* SNRVQ_PROBES_H */
