/*
 * wmtp_probe.h -- measurement aids exported by libwmtp.so beside the attention calls of wmtp.h.
 *
 * They belong to no operation of the method; they exist to put the attention kernels' bandwidth in
 * context on the machine at hand:
 *   - wmtp_probe_read streams a buffer once with the same 16-byte nontemporal loads the attention
 *     kernels use for K and V, and does nothing else with it, so its GB/s is the read rate a
 *     streaming kernel can reach on this GPU (quoted beside the 8 TB/s published HBM peak);
 *   - wmtp_llc_flush overwrites a scratch buffer, which evicts from the L2 caches and the 256 MB
 *     Infinity Cache whatever a previous call left there, so the next call's reads come from HBM
 *     ("cold"); the windowed draft reads only S+W rows, which otherwise stay cached between calls.
 *
 * Both follow the conventions of wmtp.h: device pointers owned by the caller, work enqueued on
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
