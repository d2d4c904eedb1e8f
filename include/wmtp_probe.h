/*
 * wmtp_probe.h -- measurement aids exported by libwmtp.so beside the attention calls of wmtp.h.
 *
 * They belong to no operation of the method; they exist to put the attention kernels' bandwidth in
 * context on the machine at hand:
 *   - wmtp_probe_read streams a buffer once with the same 16-byte nontemporal loads the attention
 *     kernels use for K and V, and does nothing else with it, so its GB/s is the read rate a
 *     streaming kernel can reach on this GPU (quoted beside the 8 TB/s published HBM peak);
 *   - wmtp_probe_handoff runs the data movement of a split-K read without its arithmetic (read a
 *     buffer in n workgroups, each writing a partial result, then a second launch reading all the
 *     partials), so its time is a floor for a two-launch attention read of that shape;
 *   - wmtp_llc_flush overwrites a scratch buffer, which evicts from the L2 caches and the 256 MB
 *     Infinity Cache whatever a previous call left there, so the next call's reads come from HBM
 *     ("cold"); the windowed draft reads only S+W rows, which otherwise stay cached between calls.
 *
 * All three follow the conventions of wmtp.h: device pointers owned by the caller, work enqueued on
 * `stream` (NULL = null stream), host-side validation first, no allocation, no global state, a
 * nonzero wmtp_status (wmtp.h) and nothing launched on invalid arguments.
 */
#ifndef WMTP_PROBE_H
#define WMTP_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of a wmtp_probe_read launch, and so the uint32 entries it writes to `out`. */
#define WMTP_PROBE_BLOCKS 512

/*
 * Read `bytes` bytes of `buf` once and write, for each of the WMTP_PROBE_BLOCKS workgroups, the
 * XOR of the 32-bit words it read into out[workgroup]; the XOR of all of out[] is therefore the
 * XOR of every 32-bit word of the buffer (a check that every byte was read exactly once).
 *   buf    device memory, 16-byte aligned, `bytes` a positive multiple of 16 (else INVALID_ARG)
 *   out    device memory of WMTP_PROBE_BLOCKS uint32 entries, all of them written
 */
int wmtp_probe_read(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* Workgroups of the second launch of wmtp_probe_handoff, and so the uint32 entries of its `out`. */
#define WMTP_PROBE_HANDOFF_BLOCKS 256

/*
 * The skeleton of a split-K read with no arithmetic: two dependent launches on `stream`, shaped
 * like a short attention read followed by its merge.
 *   launch 1: n_groups workgroups; workgroup g reads its contiguous share of `buf` once (the same
 *             loads as wmtp_probe_read; shares of ceil(bytes/16 / n_groups) 16-byte words, the
 *             last ones shorter or empty), folds it into c_g = the XOR of its 32-bit words, then
 *             writes part_bytes of partial results at parts + g * part_bytes: 16-byte word i holds
 *             the uint32s (c_g + i, g, i, 0), i taken modulo 2^32.
 *   launch 2: WMTP_PROBE_HANDOFF_BLOCKS workgroups; workgroup w reads its contiguous share of the
 *             n_groups * part_bytes bytes of partials and writes the XOR of their 32-bit words to
 *             out[w] (every entry written; the XOR of all of them is the XOR of every partial word).
 *   buf    device memory, 16-byte aligned, `bytes` a positive multiple of 16
 *   parts  device memory, 16-byte aligned, n_groups * part_bytes bytes; part_bytes a positive
 *          multiple of 16; 1 <= n_groups <= 65535; n_groups * part_bytes < 2^40
 *   out    device memory of WMTP_PROBE_HANDOFF_BLOCKS uint32 entries
 * Errors: INVALID_ARG (anything above violated), HIP.
 */
int wmtp_probe_handoff(const void* buf, size_t bytes, int32_t n_groups, void* parts,
                       size_t part_bytes, uint32_t* out, void* stream);

/*
 * Overwrite `bytes` bytes of `buf` with the byte value `value` using ordinary (cache-allocating)
 * 16-byte stores. For a cold-cache measurement pass at least twice the last-level cache (512 MiB).
 *   buf    device memory, 16-byte aligned, `bytes` a positive multiple of 16 (else INVALID_ARG)
 */
int wmtp_llc_flush(void* buf, size_t bytes, uint8_t value, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WMTP_PROBE_H */
