/*
 * pa_probe.h -- memory bandwidth probes of libpa (measurement aids).
 *
 * The probes read memory and do nothing else: no arithmetic of the method,
 * no stores except one 32-bit word per workgroup.  They measure what the
 * memory system of the device delivers for an access pattern, which is the
 * achievable reference to set next to the HBM peak when the decode kernels
 * are measured.  Decode is limited by memory bandwidth, prefill by compute
 * ([bicarait] "Blueprint Arsitektur 3: Chunked Prefill"), and the bytes a
 * decode reads are each logical block's K/V rows, reached through the block
 * table ([nalar] "Kernel attention harus mengikuti block table").
 *
 *   pa_probe_read    streams one contiguous buffer
 *   pa_probe_gather  reads exactly the K/V bytes a decode call over the same
 *                    pools, tables and context lengths reads: the (block,
 *                    KV head) chunk of K and of V of every logical block a
 *                    context covers, at the physical block its table names
 *
 * To show that every byte really is read, workgroup i stores the XOR of all
 * 32-bit words it loaded in sink[i]; the XOR of the whole sink is then the
 * XOR of every word loaded, counted once per load (a chunk two sequences
 * share is loaded twice and cancels out), which a test recomputes on the
 * host.
 *
 * Conventions are those of pa.h: device pointers on the current HIP device,
 * caller-owned memory (the library allocates nothing), asynchronous on
 * `stream` (a hipStream_t as void*, NULL = null stream), scalar arguments
 * validated on the host before any HIP call, so a rejected call has no
 * effect.  Loads are non-temporal 16-byte loads.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest sink (= workgroups launched) a probe accepts. */
#define PA_PROBE_MAX_SINK 65536
/* Largest batch pa_probe_gather takes (its per-sequence prefix is in LDS). */
#define PA_PROBE_MAX_SEQS 16384

/* ---------------------------------------------------------------------------
 * pa_probe_read: read `bytes` bytes of `buf` once.
 *   buf       device pointer, 16-byte aligned
 *   bytes     a multiple of 16, >= 0 (0: nothing is launched)
 *   sink      uint32 [sink_len], written (one word per workgroup)
 *   sink_len  workgroups of 256 threads to launch, 1 .. PA_PROBE_MAX_SINK;
 *             they stride over the buffer together, four 16-byte loads in
 *             flight per thread
 * Errors: PA_ERR_NULL (buf or sink NULL with bytes > 0), PA_ERR_SHAPE
 * (bytes < 0 or not a multiple of 16, sink_len out of range),
 * PA_ERR_UNSUPPORTED (buf not 16-byte aligned), PA_ERR_HIP (launch).
 * ------------------------------------------------------------------------- */
pa_status pa_probe_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t sink_len,
                        void* stream);

/* ---------------------------------------------------------------------------
 * pa_probe_gather: read the K/V chunks a decode call would read.
 *   k_cache, v_cache, block_tables, context_lens, num_seqs, num_kv_heads,
 *   head_dim, block_size, num_blocks, max_blocks_per_seq, dtype: as for
 *   pa_decode_attention (pa.h); head_dim 64 or 128, block_size 8/16/32/64.
 *   Work items are the (sequence, KV head, logical block) triples of the
 *   blocks each context covers, in that order; the W = 4 * sink_len waves
 *   (sink_len workgroups of 4) split them into W equal contiguous ranges,
 *   as the decode's stream-K split does, and walk their range one item at
 *   a time, the next item's table entry loaded while the current item's
 *   K and V chunks are read.  A sequence is read when 0 < ctx <=
 *   max_blocks_per_seq * block_size (its first ceil(ctx / block_size)
 *   blocks); a table entry outside [0, num_blocks) is skipped (nothing
 *   faults on bad contents).
 * Errors: as pa_decode_attention for the shared arguments, plus
 * PA_ERR_SHAPE for sink_len out of range, PA_ERR_NULL for a NULL sink and
 * PA_ERR_UNSUPPORTED for num_seqs > PA_PROBE_MAX_SEQS.
 * ------------------------------------------------------------------------- */
pa_status pa_probe_gather(const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, pa_dtype dtype, uint32_t* sink,
                          int32_t sink_len, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
