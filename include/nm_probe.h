/*
 * nm_probe.h -- measurement utilities of libnmsparse.so (not part of the sparse method).
 *
 * They give the bench two reference points on the same GPU, in the same process:
 *   nm_probe_read  streams `bytes` from `src` and discards them (a pure read of HBM):
 *                  the attainable read bandwidth, i.e. the practical ceiling of a
 *                  kernel that only has to read its operand once.
 *   nm_probe_copy  copies `bytes` from `src` to `dst`: a kernel of known traffic
 *                  (bytes read + bytes written) used to calibrate the FETCH_SIZE and
 *                  WRITE_SIZE hardware counters against real bytes.
 *   nm_probe_read_shaped  the same pure read with the launch shape chosen by the caller:
 *                  `blocks` workgroups (1..2^20) of `threads` lanes (64..1024, a multiple
 *                  of 64), `unroll` (1, 2, 4 or 8) 16-byte loads in flight per lane;
 *                  `blocked` = 0 sweeps the buffer grid-stride, 1 gives each workgroup its
 *                  own contiguous slice. Sweeping these at one byte count gives the
 *                  fastest single launch that only reads that many bytes. Any other
 *                  value of these four returns NM_ERR_SHAPE.
 * Conventions as in nm_sparse.h: device pointers owned by the caller, `stream` is a
 * hipStream_t as void*, asynchronous, validated before any HIP call, status codes
 * from nm_status. `bytes` must be a positive multiple of 16 and the pointers 16-byte
 * aligned; `sink` receives at most one uint32 (written only if the data XOR-reduces
 * to the caller's `magic`, which keeps the reads from being optimised away).
 */
#ifndef NM_PROBE_H
#define NM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int nm_probe_read(const void* src, size_t bytes, uint32_t* sink, uint32_t magic, void* stream);
int nm_probe_read_shaped(const void* src, size_t bytes, uint32_t* sink, uint32_t magic, int blocks, int threads,
                         int unroll, int blocked, void* stream);
int nm_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NM_PROBE_H */
