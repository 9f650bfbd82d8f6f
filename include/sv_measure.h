/*
 * libspecverify — measurement aid (not a step of the verification method).
 *
 * The verification kernels are bound by how fast HBM delivers the logit rows.
 * Beside MI355X's 8 TB/s peak, the figure that bounds them in practice is the
 * rate a plain read of the same kind sustains: every byte read once with the
 * 16-byte non-temporal buffer loads the kernels stream logits with, and no
 * arithmetic beyond keeping the loads alive.  sv_stream_read is that read.
 */
#ifndef SV_MEASURE_H
#define SV_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes at device address `src` once, on `stream`.
 *   src      device buffer, 16-byte aligned (owned by the caller)
 *   bytes    a multiple of 16; 0 is a no-op that returns SV_OK
 *   blocks   1024-thread workgroups in [1, 65536]; workgroup i reads the i-th
 *            of `blocks` equal contiguous shares, as a sequence-resident
 *            verification workgroup reads its sequence's rows (each share at
 *            most 2 GiB)
 *   out      device uint32 [blocks]: word i receives the XOR of the 32-bit
 *            words of workgroup i's share (so that the loads are kept); words
 *            of workgroups left without a share (more blocks than 16-byte
 *            chunks) are not written
 * Asynchronous; returns SV_OK, SV_ERR_NULL (src or out NULL, bytes > 0),
 * SV_ERR_SHAPE (misaligned src, bytes not a multiple of 16, blocks out of
 * range, a share above 2 GiB) or SV_ERR_HIP (launch refused), checked on the
 * host before launching.
 */
int sv_stream_read(const void* src, size_t bytes, int blocks, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SV_MEASURE_H */
