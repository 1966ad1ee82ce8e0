/*
 * libselscan_probes: calibration kernels for the benchmark, built beside libselscan
 * for gfx950. They compute nothing of the selective scan; they measure two ceilings of
 * the GPU they run on, so that the scan's kernels can be compared with what this chip
 * reaches rather than with spec-sheet figures alone:
 *
 *  - ssp_rmw: the read-modify-write rate of HBM for a decode-step-sized buffer, with the
 *    access pattern of the decode step's state update (16-byte nontemporal loads and
 *    stores, every load of a lane issued before its stores);
 *  - ssp_issue: the VALU issue rate of fp32 FMAs and of the v_exp_f32 transcendental,
 *    alone and interleaved with FMAs, from which the cost of one exponential in FMA
 *    issue slots follows.
 *
 * Both take device pointers and a hipStream_t (NULL = default stream), enqueue one
 * kernel and return 0, or a nonzero hipError_t code when the launch fails or an
 * argument is unusable (nothing is enqueued then). Asynchronous; they allocate nothing.
 */
#ifndef SELSCAN_PROBES_H
#define SELSCAN_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In place over buf[0 .. n_floats): buf[i] = buf[i] * 0.5f + 1.0f, read and written with
 * 16-byte nontemporal accesses, 64 bytes per lane. buf must be 16-byte aligned and
 * n_floats a positive multiple of 16. Moves 8 * n_floats bytes. */
int ssp_rmw(float* buf, size_t n_floats, void* stream);

/* Issue-rate kernel: 2048 workgroups of 256 lanes (8 waves on each SIMD of a 256-CU
 * GPU), each lane running 8 independent chains for `iters` iterations. Per chain and
 * iteration: mode 0, `kfma` fmas; mode 1, one v_exp_f32; mode 2, one v_exp_f32 and
 * `kfma` fmas (on a separate register, so they can interleave). kfma in {1, 3, 7, 8};
 * iters >= 4, a multiple of 4. One float per lane is written to out (2048 * 256 floats),
 * so the work cannot be optimised away. */
int ssp_issue(float* out, int64_t iters, int mode, int kfma, void* stream);

#define SSP_ISSUE_LANES (2048 * 256)
#define SSP_ISSUE_CHAINS 8

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_PROBES_H */
