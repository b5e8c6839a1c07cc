/*
 * commvq_probes.h: measurement probes of libcommvq_probes.so. They are used by the benchmark to place the
 * attention kernels against what this device delivers; they are not part of the attention path.
 *
 *   commvq_probe_read_stream: one streaming read of `bytes` bytes of device memory at `buf` (16-byte loads,
 *     `bytes` a multiple of 16, buf 16-byte aligned), `blocks` workgroups of 256 threads, grid-stride.
 *     The loaded words are folded into a value that is written to `sink` (4 bytes of device memory) only
 *     if it equals a fixed constant, which keeps every load. Timing the call gives the HBM read rate a
 *     plain kernel reaches (bytes / time).
 *   commvq_probe_lds_gather: `blocks` workgroups of 8 waves, one per CU (each holds 160 KiB of LDS, as the
 *     attention kernels do); every wave performs iters x 16 random 16-byte row reads (ds_read_b128) from a
 *     64 KiB table of 16 groups x 256 rows, the access pattern of the attention kernels' codebook gathers
 *     (each lane a random row of the same group). Per call: blocks x 8 x iters x 16 x 1 KiB are gathered,
 *     so bytes / time is the random-gather throughput of LDS. `sink` as above.
 *   commvq_probe_lds_bin_add: `blocks` workgroups of 8 waves, one per CU (160 KiB of LDS each); every wave
 *     performs iters x 42 x 2 random 64-bit LDS atomic adds (ds_add_u64) into bins of 42 units x 2 head
 *     pairs x 64 codewords, the access pattern of the bit-packed attention kernel's value bins (each lane a
 *     random codeword of the same unit, both head pairs). `sink` (8 bytes of device memory, zeroed by the
 *     caller) receives the bins' total, blocks x 8 x iters x 42 x 2 x 64 when every add landed; wave
 *     instructions / time is the throughput of random 64-bit LDS adds.
 * All return 0 or the hipError_t of the launch; pointers are device pointers; work is enqueued on `stream`
 * (a hipStream_t; NULL is the default stream).
 */
#ifndef COMMVQ_PROBES_H
#define COMMVQ_PROBES_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int commvq_probe_read_stream(const void* buf, size_t bytes, int blocks, void* sink, void* stream);
int commvq_probe_lds_gather(int iters, int blocks, void* sink, void* stream);
int commvq_probe_lds_bin_add(int iters, int blocks, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* COMMVQ_PROBES_H */
