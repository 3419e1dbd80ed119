/*
 * sss_probe.h -- bandwidth probes of libsss (measurement helpers, not steps
 * of the method).
 *
 * The attention path is bound by reading the paged KV cache once
 * (SparseSpec §2.1 and §3.2: decode attention is memory-bound and its time
 * is linear in the KV bytes; §4.2 reports attention kernels as fractions of
 * bandwidth).  These kernels read bytes and do nothing else, with the same
 * loads the attention kernels use (16-byte non-temporal global loads), so
 * that a kernel's rate can be set against what the memory system delivers
 * for the same bytes, and so that hardware byte counters can be calibrated
 * against a transfer of exactly known size.
 *
 * Both write one 32-bit XOR of what each workgroup read to `sink` (device,
 * SSS_PROBE_SINK_WORDS words, caller-owned), which keeps the loads live; its
 * value has no meaning.  Nothing else is written.  Launches are async on
 * `stream`; the library allocates nothing.
 */
#ifndef SSS_PROBE_H_
#define SSS_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "sss.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Words of `sink` the probes may write (one per workgroup of their grid). */
#define SSS_PROBE_SINK_WORDS 4096

/*
 * Streaming read of `bytes` bytes at `src` (device, 16-byte aligned, bytes a
 * multiple of 16), each byte once: contiguous 32 KiB blocks dealt
 * round-robin over a grid of SSS_PROBE_SINK_WORDS workgroups.  Errors:
 * SSS_ERR_INVALID_ARGUMENT for a NULL or misaligned pointer or a size that
 * is not a multiple of 16.
 */
sss_status sss_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Paged read: every cached token row of K and of V that a verify pass over
 * `batch` requests reads (tokens [0, seq_lens[b]) of every KV head, found
 * through the page table), each once, as (page, head) runs, a workgroup
 * walking the pages of one (request, KV head) at a time with 8 runs of K
 * and of V in flight -- the verify's KV bytes and access pattern without
 * its arithmetic.  kv as for sss_verify_attn (BF16 or F32; page_size *
 * head_dim * element size a multiple of 16 bytes).  Runs of a page id
 * outside [0, num_pages) are not counted.  Errors: SSS_ERR_INVALID_ARGUMENT
 * for NULL or misaligned pointers or invalid sizes, SSS_ERR_UNSUPPORTED for
 * another dtype or a run size that is not a multiple of 16 bytes.
 */
sss_status sss_probe_paged_read(const sss_paged_kv* kv, int32_t batch, uint32_t* sink,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSS_PROBE_H_ */
