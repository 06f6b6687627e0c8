/*
 * smcsd_bench.h -- measurement helpers exported by libsmcsd.so next to the round itself.
 *
 * The round is a streaming reduction: every logit is read once, so its speed is bounded by
 * HBM bandwidth (the SMC-SD page, section 2, notes that decoding on GPUs is limited by memory
 * bandwidth). These two kernels calibrate that bound on the machine at hand:
 *  - a plain streaming read gives the attainable read bandwidth;
 *  - a plain copy of known size turns hardware byte counters (FETCH_SIZE / WRITE_SIZE) into
 *    bytes.
 * A third runs the round's logits pass alone, many times back to back, so that its kernels
 * can be timed without an event around each launch (an event costs microseconds of queue
 * time, a large share of a short kernel).
 * They are not part of the round.
 */
#ifndef SMCSD_BENCH_H
#define SMCSD_BENCH_H

#include "smcsd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes from `src` with 16-byte non-temporal loads in a grid-stride loop of
 * `grid` workgroups x 256 threads. Each thread XOR-folds what it reads and stores one word
 * to sink[grid*256], so the loads cannot be dropped. `bytes` must be a multiple of 16 and
 * `src` 16-byte aligned. The caller owns both buffers.
 */
smcsd_status smcsd_bench_stream_read(const void *src, size_t bytes, uint32_t *sink,
                                     int32_t grid, smcsd_stream stream);

/* Copy `bytes` (a multiple of 16, both pointers 16-byte aligned) from src to dst. */
smcsd_status smcsd_bench_copy(const void *src, void *dst, size_t bytes, smcsd_stream stream);

/*
 * The logits pass of smcsd_round (the kernels that read the logits; no weights,
 * resampling, bonus choice or page remap), `repeats` >= 1 times back to back on `stream`,
 * with the same arguments and the same checks as smcsd_round (timing events ignored). Each
 * repeat overwrites the pass's partials in the workspace; no output of the round is written.
 */
smcsd_status smcsd_bench_logits_pass(const smcsd_round_args *args, int32_t repeats,
                                     smcsd_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* SMCSD_BENCH_H */
