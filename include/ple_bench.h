/*
 * ple_bench.h - measurement kernels of libple_bench, the streaming-copy
 * ceilings the benchmark reports next to the lookup.  Not part of the lookup
 * path: plain 16-byte copies with the same access patterns as the lookup's
 * row traffic, so that the lookup's bandwidth can be compared with what the
 * HBM delivers for those patterns on the same GPU in the same run.
 * Conventions as in ple.h (device pointers 16-byte aligned, stream as void*,
 * PLE_OK or an error code; ple_bench_error_message() describes the last
 * failure on the calling thread).
 */
#ifndef PLE_BENCH_H
#define PLE_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Contiguous copy: dst[i] = src[i] for `bytes` bytes (a multiple of 16),
 * 16-byte chunks, 32 chunks in flight per lane, non-temporal loads and
 * stores (each byte is touched once).
 */
int ple_bench_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * Row gather from caller row indices: dst row k = src row rows[k] for k <
 * nrows, rows of row_bytes bytes (a multiple of 16, at most 16384); 32 rows
 * per wave, one 16-byte chunk per lane per row in flight, non-temporal loads.
 * rows: device int32 [nrows], each in [0, src_rows) (clamped into range).
 */
int ple_bench_copy_rows(const void* src, int64_t src_rows, int32_t row_bytes, const int32_t* rows, int64_t nrows,
                        void* dst, void* stream);

const char* ple_bench_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* PLE_BENCH_H */
