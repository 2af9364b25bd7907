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
int nm_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NM_PROBE_H */
