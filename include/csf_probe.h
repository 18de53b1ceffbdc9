/*
 * csf_probe.h — measurement kernels that go with the CSF decoder
 * (libcsf_probe.so, gfx950).  They decode nothing: they give the ceilings and
 * floors the decoder's timings are read against, as the pages read theirs
 * against warm and cache-flushed runs ("finegrained-kernels: decode losslessly
 * compressed NVFP4 scales (CSF)", kernels-community PR 1236, measurements
 * paragraph).  Same status codes and stream convention as csf.h; every
 * launch is enqueued on hip_stream and returns without synchronising; the
 * library allocates nothing.
 */
#ifndef CSF_PROBE_H
#define CSF_PROBE_H

#include <stdint.h>

#include "csf.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Flags of csf_probe_mix. */
#define CSF_PROBE_NT_ENTRIES 1u /* non-temporal loads of read stream 1 (the decoder's entry stream) */

/*
 * Stream mix at the decoder's access shape: dst (device, dst_bytes) is cut
 * into tiles of 16 KiB; read stream s (device src[s], src_bytes[s] bytes,
 * 1 <= nsrc <= 3) is cut into as many pieces, on 16-byte boundaries.
 * Workgroups of 256 lanes take tiles grid-stride (grid workgroups); per tile
 * every lane issues, for each stream, the 16-byte loads of its share of the
 * piece (as many as the largest piece needs: at most two for stream 0, three
 * for stream 1, one for stream 2), and stores four 16-byte runs whose bytes
 * depend on every loaded byte, non-temporal; each wave store instruction
 * covers 1 KiB, and the next tile's loads are issued before this tile's
 * stores.  Bytes read = sum of src_bytes, written = dst_bytes.  A larger
 * piece (above 8, 12 or 4 KiB) returns CSF_E_SIZE.
 * Errors: CSF_E_NULL, CSF_E_SIZE, CSF_E_HIP.
 */
csf_status csf_probe_mix(const uint8_t *const *src, const uint64_t *src_bytes, uint32_t nsrc, uint8_t *dst,
                         uint64_t dst_bytes, uint32_t grid, uint32_t flags, void *hip_stream);

/*
 * Launch floor with k dependent round trips: grid workgroups of block lanes
 * (a multiple of 64, at most 1024).  Each workgroup follows hops links of a
 * chain in buf (device u32[words], words < 2^30, every value < words, read
 * with vector buffer loads; the caller fills it,
 * for example with a random permutation), starting at an index set by the
 * workgroup number and seed, each load waiting for the previous one; then,
 * when out is not NULL, every lane stores 16 bytes at out + 16 * (workgroup
 * * block + lane) (out holds grid * block * 16 bytes).  hops = 0 with out
 * NULL is an empty kernel.
 * Errors: CSF_E_NULL (buf with hops > 0), CSF_E_SIZE, CSF_E_HIP.
 */
csf_status csf_probe_chain(const uint32_t *buf, uint64_t words, uint32_t seed, uint32_t hops, uint8_t *out,
                           uint32_t grid, uint32_t block, void *hip_stream);

/*
 * Host cost of the decode entry points: calls back-to-back enqueues of
 * csf_decode (second NULL) or csf_decode_paired with these arguments, timed
 * on the host's steady clock; returns nanoseconds per call (the enqueues
 * only; the GPU runs the decodes afterwards), or a negative value when a call
 * fails (-1 - its status) or calls is 0.
 */
double csf_probe_host_ns(const csf_stack *first, uint8_t *ws_first, const csf_stack *second, uint8_t *ws_second,
                         const int32_t *expert_start, uint32_t calls, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* CSF_PROBE_H */
