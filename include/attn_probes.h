/*
 * attn_probes.h - microbenchmarks of the MI355X (gfx950) units that bound the
 * attention kernels, in their own library (libattn_probes.so).
 *
 * The cost model of "Chapter 33 推理计算优化" §33.1 bounds an execution by
 * its work over the rate of the unit that does it (time >= max(F/R, Q/b)).
 * These entry points measure those rates on the part itself: each launches
 * one kernel on `stream` (a hipStream_t as void*, NULL = null stream) and
 * returns 0, -2 for an invalid argument (nothing launched) or -1 if the
 * launch failed.  The caller times the call (events on the same stream) and
 * owns every pointer, which must be device memory.  `out` receives one
 * element per thread (blocks x 256 of them) so that the work cannot be
 * optimised away; its values carry no meaning.
 */
#ifndef ATTN_PROBES_H
#define ATTN_PROBES_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: every 16-byte word of [src, src + bytes) is read once
 * (bytes rounded down to 16; src 16-byte aligned).  Work: `bytes` of HBM
 * reads. */
int attn_probe_stream_read(const void* src, size_t bytes, unsigned* out, int blocks, void* stream);

/* v_exp_f32 rate: 8 independent chains of `iters` exponentials per thread,
 * i.e. blocks x 256 x 8 x iters exponentials. */
int attn_probe_exp(float* out, int blocks, int iters, void* stream);

/* LDS read rate: every wave of a 4-wave workgroup reads a 64 KB LDS buffer
 * `iters` times, with 16-byte reads (transposed = 0) or 8-byte transposed
 * reads, ds_read_b64_tr_b16 (transposed = 1): blocks x 4 x 64 KB x iters
 * bytes (half that with transposed reads, which move 8 bytes per lane). */
int attn_probe_lds_read(unsigned* out, int blocks, int iters, int transposed, void* stream);

/* bf16 MFMA rate: 4 independent v_mfma_f32_32x32x16_bf16 accumulators per
 * wave, `iters` rounds: blocks x 4 x 4 x iters x 32768 flops. */
int attn_probe_mfma(float* out, int blocks, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBES_H */
