/*
 * tgemm_stamps.h -- extra entry points of libtgemm_stamps.so, the tooling build of libtgemm
 * (same sources compiled with TGEMM_STAMPS and TGEMM_SWEEP_CONFIGS; it also exports
 * everything in tgemm.h). Not part of the product library: libtgemm.so does not export
 * these. Besides the stamps, this build compiles every row of the config table, including
 * the variants the product leaves out (tgemm_config_info.built is 1 for all of them), for
 * the offline sweep, the MFMA throughput probe (the measured compute ceiling) and the LDS
 * access probe (bank-conflict cycles of any lane address pattern).
 *
 * In the instrumented build every workgroup of the GEMM kernels (all configs except the
 * generic one) and of the MFMA probe records, at its end, TGEMM_STAMP_WORDS 64-bit words
 * into a device-side table indexed by workgroup id (ids below TGEMM_STAMP_WORKGROUPS; each
 * launch overwrites the rows of its workgroups):
 *   [0] wall clock at kernel start      (s_memrealtime, 100 MHz ticks)
 *   [1] wall clock at main-loop start
 *   [2] wall clock at main-loop end
 *   [3] wall clock after every wave's stores completed
 *   [4] shader-clock ticks from kernel start to main-loop end (s_memtime counts at the
 *       current shader clock, so [4] / ([2] - [0]) * 100 MHz is the clock the workgroup
 *       ran at)
 *   [5] main-loop iterations (k-tiles, or probe rounds)
 *   [6] threads per workgroup
 *   [7] 1 once written
 * The stamps cost a few instructions per workgroup and one extra barrier at its end.
 */
#ifndef TGEMM_STAMPS_H_
#define TGEMM_STAMPS_H_

#include <stdint.h>

#include "tgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define TGEMM_STAMP_WORKGROUPS 4096
#define TGEMM_STAMP_WORDS 8

/* Writes the table's shape; returns TGEMM_OK or TGEMM_ENULL. */
TGEMM_API int tgemm_stamps_capacity(int* workgroups, int* words_per_workgroup);

/* Copies the first `words` words of the table of the current device to host memory
 * (synchronous; words <= TGEMM_STAMP_WORKGROUPS * TGEMM_STAMP_WORDS). Returns TGEMM_OK,
 * TGEMM_ENULL, TGEMM_EINVAL_DIM or TGEMM_ELAUNCH (the copy failed). */
TGEMM_API int tgemm_stamps_read(uint64_t* host, int64_t words);

/* Zeroes the table of the current device (synchronous). Returns TGEMM_OK or
 * TGEMM_ELAUNCH. */
TGEMM_API int tgemm_stamps_clear(void);

/* ---- MFMA throughput probe (the measured compute ceiling of the board) ---- */

/* Enqueues `blocks` workgroups of TGEMM_PROBE_THREADS threads (8 waves). Every wave
 * issues iters x TGEMM_PROBE_MFMA_PER_ITER independent 16x16x32 fp16 MFMAs (16384 FLOP
 * each) on pseudo-random register operands, with no memory traffic, then each thread
 * writes one float to out. out: caller-owned device memory of blocks * TGEMM_PROBE_THREADS
 * floats. FLOP per launch = blocks * TGEMM_PROBE_THREADS / 64 * iters *
 * TGEMM_PROBE_MFMA_PER_ITER * 16384. Returns TGEMM_OK, TGEMM_ENULL (out NULL),
 * TGEMM_EINVAL_DIM (blocks outside [1, 2^20] or iters outside [1, 2^24]), TGEMM_EDEVICE
 * or TGEMM_ELAUNCH. */
#define TGEMM_PROBE_THREADS 512
#define TGEMM_PROBE_MFMA_PER_ITER 16
TGEMM_API int tgemm_mfma_probe(int blocks, int iters, void* out, void* stream);

/* The same probe with a choice of operands and MFMA shape. Every mode does the same FLOP
 * per launch as tgemm_mfma_probe (FLOP = blocks * TGEMM_PROBE_THREADS / 64 * iters *
 * TGEMM_PROBE_MFMA_PER_ITER * 16384):
 *   TGEMM_PROBE_SYNTHETIC   the pseudo-random register operands of tgemm_mfma_probe,
 *                           16x16x32 MFMAs (operands may be NULL);
 *   TGEMM_PROBE_OPERANDS    operands loaded once from `operands`, 16x16x32 MFMAs;
 *   TGEMM_PROBE_OPERANDS_32 operands from `operands`, 32x32x16 MFMAs (8 accumulators of
 *                           16 floats, half as many MFMAs of twice the FLOP);
 *   TGEMM_PROBE_LDS_READS   operands from `operands`, 16x16x32 MFMAs, plus per wave and
 *                           round 6 conflict-free ds_read_b128 from a 64 KiB LDS copy of
 *                           the same values (the read rate of the 256 x 256 ping-pong
 *                           GEMM), whose results are the next round's operands.
 * operands: device memory of TGEMM_PROBE_THREADS * 64 binary16 values (64 KiB), 16-byte
 * aligned; thread t of every workgroup takes values [64 t, 64 t + 64). Their magnitudes
 * and signs set how much the multipliers toggle, so the power the probe draws. Returns
 * TGEMM_OK, TGEMM_ENULL (out NULL, or operands NULL for a mode that reads them),
 * TGEMM_EALIGN (operands not 16-byte aligned), TGEMM_EINVAL_DIM (mode unknown, blocks
 * outside [1, 2^20] or iters outside [1, 2^24]), TGEMM_EDEVICE or TGEMM_ELAUNCH. */
#define TGEMM_PROBE_SYNTHETIC 0
#define TGEMM_PROBE_OPERANDS 1
#define TGEMM_PROBE_OPERANDS_32 2
#define TGEMM_PROBE_LDS_READS 3
TGEMM_API int tgemm_mfma_probe_ex(int mode, int blocks, int iters, const void* operands, void* out,
                                  void* stream);

/* ---- LDS access probe (calibrates the host-side LDS bank model) ---- */

/* Enqueues `blocks` workgroups of one wave (64 lanes) each with a 64 KiB LDS block. Every
 * wave runs `iters` rounds; a round issues ni instructions of kind op (TGEMM_LDS_*) and
 * waits for them; instruction j of a round is issued by the lanes whose bit is set in
 * active[j] and accesses byte address addrs[j * 64 + lane] of the (uninitialised) block.
 * addrs: host memory, ni * 64 int32, each in [0, 65536 - width] and a multiple of the
 * access width (4, 8 or 16 bytes; 8 for TGEMM_LDS_READ_TR16_B64), checked for every lane;
 * active: host memory, ni lane masks. out: caller-owned
 * device memory of `blocks` floats. Returns TGEMM_OK, TGEMM_ENULL, TGEMM_EINVAL_DIM (op,
 * ni outside [1, 8], iters outside [1, 2^20], blocks outside [1, 2^16], or an address out
 * of range or misaligned; checked before anything is enqueued), TGEMM_EDEVICE or
 * TGEMM_ELAUNCH. */
#define TGEMM_LDS_READ_B32 0
#define TGEMM_LDS_READ_B64 1
#define TGEMM_LDS_READ_B128 2
#define TGEMM_LDS_WRITE_B32 3
#define TGEMM_LDS_WRITE_B64 4
#define TGEMM_LDS_WRITE_B128 5
#define TGEMM_LDS_READ_TR16_B64 6
TGEMM_API int tgemm_lds_probe(int op, const int32_t* addrs, const uint64_t* active, int ni, int iters,
                              int blocks, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_STAMPS_H_ */
