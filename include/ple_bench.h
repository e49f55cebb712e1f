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

/*
 * Row gather with the memory pattern of a quantized table's lookup, without
 * its arithmetic: dst row k (out_row_bytes, a power of two in 32..16384) is
 * src row rows[k] (out_row_bytes / expand bytes; expand 1, 2 or 4) repeated
 * `expand` times, plus the table's side reads: aux_mode 0 none, 1 one 4-byte
 * word per row (aux: [src_rows] words, the fp8 per-row scale), 2 one byte per
 * 16 output elements (aux: [src_rows][out_row_bytes / 32] bytes, the NVFP4
 * block scales).  The side value is XORed into each chunk, so its load
 * counts.  1024 output chunks per wave, non-temporal loads and stores.
 */
int ple_bench_gather_expand(const void* src, int64_t src_rows, int32_t expand, const void* aux, int32_t aux_mode,
                            const int32_t* rows, int64_t nrows, int32_t out_row_bytes, void* dst, void* stream);

const char* ple_bench_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* PLE_BENCH_H */
