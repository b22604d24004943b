/*
 * kvq_stream.h - streaming probes that measure the HBM bandwidth a kernel of a given launch shape
 * can reach on this device: the practical ceiling that the append's and the decode's achieved
 * bandwidth are compared with, next to the nominal peak.
 *
 * Measurement support only (libkvq_stream.so, built beside libkvq.so); no part of the KV-cache
 * path calls it. The pages make both paths bandwidth-bound (OScaR summary, "Introduction"), so
 * the fraction of a measured streaming rate is the figure that says how much of the achievable
 * bandwidth a kernel leaves unused.
 *
 * One call is one launch of grid_blocks workgroups of block_threads threads over grid-stride loops
 * of 16-byte units, eight units a grid stride apart per thread and iteration. The launch reads
 * src[0 .. rows * read_units) and writes dst[0 .. rows * write_units) (16-byte elements), in one of
 * two layouts:
 *   layout 0  rows of read_units loads followed by write_units stores: row r reads
 *             src[r * read_units ..) and writes dst[r * write_units ..), consecutive threads take
 *             consecutive units, so one wave both reads and writes (as a kernel that loads a token
 *             row and stores its codes does);
 *   layout 1  of every read_units + write_units consecutive workgroups the first read_units only
 *             read and the rest only write, each kind walking its own linear stream; each kind's
 *             share of the workgroups is its share of the bytes, so both streams end together.
 * Loads are non-temporal (they do not displace lines the rest of the launch would reuse); stores
 * are ordinary. Stored values are position stamps: (u, r, k, 0) for unit k of row r at unit index
 * u in layout 0, (r, read_units + k, j, 1) for store j (row r, position k) in layout 1.
 *
 *   read-only   read_units > 0, write_units = 0 (dst unused, may be NULL)
 *   write-only  read_units = 0, write_units > 0 (src unused, may be NULL)
 *   copy        read_units = write_units
 *   mix         e.g. 32 : 9, the append's 512 bytes read per 144 written (INT4 token-head)
 *
 * Arguments: device pointers src (rows * read_units * 16 bytes) and dst (rows * write_units * 16
 * bytes), both 16-byte aligned; sink: one device uint32 that a load result is written to only in
 * the unlikely case it equals `key` (it keeps the loads from being dropped as dead code); stream:
 * the HIP stream (NULL = the default stream). The caller owns all memory.
 *
 * Returns 0 on success, 1 for invalid sizes, layout or alignment (nothing launched; layout 1 needs
 * at least read_units + write_units workgroups), 2 for a HIP launch error.
 */
#ifndef KVQ_STREAM_H
#define KVQ_STREAM_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t kvq_stream_probe(const void* src, void* dst, uint64_t rows, uint32_t read_units, uint32_t write_units,
                         int32_t layout, uint32_t grid_blocks, uint32_t block_threads, uint32_t key,
                         uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif  // KVQ_STREAM_H
