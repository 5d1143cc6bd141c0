/*
 * libmla_roofs -- measurement kernels that the benchmark uses to find what
 * this MI355X (gfx950) actually sustains, beside the published peaks, and to
 * run the attention path from a cold cache.  Nothing on the attention path
 * calls them; they live in their own library (libmla_roofs.so).
 *
 * Conventions: device pointers, 16-byte aligned; stream is a hipStream_t
 * passed as void* (NULL = the null stream); every call only enqueues work and
 * returns 0 on success, -1 for an invalid argument (nothing enqueued) or -4
 * when the HIP runtime reports an error.
 */
#ifndef LIBMLA_ROOFS_H
#define LIBMLA_ROOFS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Overwrite bytes of buf (a multiple of 16) with a pattern in 16-byte
 * stores.  With bytes well above the 256 MB last-level cache this evicts the
 * L2s and the memory-side cache, so that the next kernel reads from HBM. */
int mla_roofs_flush(void* buf, size_t bytes, void* stream);

/* Read bytes of buf (a multiple of 16) once, in 16-byte loads spread over
 * the whole chip (every workgroup sweeps the buffer grid-stride, so each
 * sweep is one contiguous span), and fold the data into sink [sink_words]
 * uint32 (one word per workgroup, so that the loads are live); sink_words
 * must be at least mla_roofs_read_grid().  nontemporal != 0 marks the loads
 * non-temporal.  The HBM read rate is bytes / duration. */
int mla_roofs_hbm_read(const void* buf, size_t bytes, int32_t nontemporal, uint32_t* sink, size_t sink_words,
                       void* stream);

/* Workgroups mla_roofs_hbm_read launches on the current device (host only;
 * 0 when the device cannot be queried). */
int mla_roofs_read_grid(void);

/* Dense bf16 matrix-core work with no memory traffic: every SIMD of every
 * compute unit runs two waves, each issuing iters rounds of four independent
 * v_mfma_f32_32x32x16_bf16 (32768 flops each).  *flops receives the flop
 * count of the launch (host-side).  sink [sink_words] uint32, at least
 * mla_roofs_mfma_grid() * 4 words, keeps the results live. */
int mla_roofs_mfma_bf16(int32_t iters, uint32_t* sink, size_t sink_words, double* flops, void* stream);

/* Workgroups (256 threads each) mla_roofs_mfma_bf16 launches (host only). */
int mla_roofs_mfma_grid(void);

/* An empty kernel of one workgroup: times what an event pair around one
 * launch costs beyond the kernel itself. */
int mla_roofs_empty(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_ROOFS_H */
