/* sdm_probe.h -- measurement aid shipped beside libsdm.so (libsdm_probe.so).
 *
 * Not part of the SDM path. It measures the rate at which the GPU moves
 * random pieces of table rows in place, the access pattern of the scan's
 * table traffic, so that the scan's fraction of the published HBM peak can be
 * read against what this access pattern reaches in practice.
 */
#ifndef SDM_PROBE_H
#define SDM_PROBE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Random in-place row-piece traffic over a device table of rows x 512 bytes
 * (tab, device memory the caller owns, rows <= 2^31 - 1). Access k reads
 * piece_bytes (64, 128, 256 or 512) at a piece of a row, both picked by an
 * integer hash of k; every odd access writes the piece back (first float
 * + 1). naccess accesses over grid (1 .. 65536) workgroups of 256 threads;
 * sink (device, grid * 256 floats) receives one value per thread so the
 * loads are not removed. Asynchronous on stream (a hipStream_t, NULL = the
 * default stream). Bytes moved = naccess * piece_bytes * 1.5.
 * Returns 0, 1 for an invalid argument, 2 for a launch error. */
int sdm_probe_gather(float* tab, int64_t rows, int piece_bytes, int64_t naccess, int grid, float* sink,
                     void* stream);

#ifdef __cplusplus
}
#endif
#endif
