// Streaming-copy ceilings for the benchmark (include/ple_bench.h): a
// contiguous copy and a row gather from caller indices, both one pass of
// 16-byte chunks per lane with every load of a wave in flight before its
// stores, the shape that streams fastest on this GPU.  Kept apart from
// libple: they measure the memory system, they are not part of the path.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>

#include "ple.h"
#include "ple_bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;
constexpr int kCopyLoads = 32;  // chunks in flight per lane (contiguous copy)
constexpr int kRowsPerWave = 32;

thread_local char g_msg[256];

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return code;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n) {
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t base = wave * (kCopyLoads * kWave);
    u32x4 v[kCopyLoads];
#pragma unroll
    for (int u = 0; u < kCopyLoads; ++u) {
        const int64_t i = base + u * kWave + lane;
        if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyLoads; ++u) {
        const int64_t i = base + u * kWave + lane;
        if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
}

// Rows of cpr 16-byte chunks; a wave copies kRowsPerWave rows, chunk c of
// every row by lanes c, c+64, ... (ONE_PASS: rows of exactly 64 chunks, one
// load per lane per row, the loop-free body the lookup's 1 KiB rows take).
template <bool ONE_PASS>
__global__ __launch_bounds__(256) void copy_rows_kernel(const u32x4* __restrict__ src, int64_t src_rows, int cpr,
                                                        const int32_t* __restrict__ rows, int64_t nrows,
                                                        u32x4* __restrict__ dst) {
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t r0 = wave * kRowsPerWave;
    if (r0 >= nrows) return;
    int my = 0;
    if (lane < kRowsPerWave && r0 + lane < nrows) {
        my = rows[r0 + lane];
        my = my < 0 ? 0 : (my >= src_rows ? (int)(src_rows - 1) : my);
    }
    if (ONE_PASS) {
        u32x4 v[kRowsPerWave];
#pragma unroll
        for (int u = 0; u < kRowsPerWave; ++u) {
            const int id = __shfl(my, u, kWave);
            if (r0 + u < nrows) v[u] = __builtin_nontemporal_load(src + (int64_t)id * kWave + lane);
        }
#pragma unroll
        for (int u = 0; u < kRowsPerWave; ++u)
            if (r0 + u < nrows) dst[(r0 + u) * kWave + lane] = v[u];
        return;
    }
    for (int c0 = 0; c0 < cpr; c0 += kWave) {
        const int c = c0 + lane;
        u32x4 v[kRowsPerWave];
#pragma unroll
        for (int u = 0; u < kRowsPerWave; ++u) {
            const int id = __shfl(my, u, kWave);
            if (r0 + u < nrows && c < cpr) v[u] = __builtin_nontemporal_load(src + (int64_t)id * cpr + c);
        }
#pragma unroll
        for (int u = 0; u < kRowsPerWave; ++u)
            if (r0 + u < nrows && c < cpr) dst[(r0 + u) * cpr + c] = v[u];
    }
}

}  // namespace

extern "C" {

const char* ple_bench_error_message(void) { return g_msg; }

int ple_bench_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes % 16 != 0) return fail(PLE_ERR_INVALID_ARGUMENT, "bytes must be a multiple of 16");
    if (bytes == 0) return PLE_OK;
    if (src == nullptr || dst == nullptr || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
        return fail(PLE_ERR_INVALID_ARGUMENT, "src and dst must be non-NULL and 16-byte aligned");
    const int64_t n = (int64_t)(bytes / 16);
    const int64_t waves = (n + kCopyLoads * kWave - 1) / (kCopyLoads * kWave);
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)src, (u32x4*)dst, n);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PLE_OK : fail(PLE_ERR_DEVICE, "copy launch: %s", hipGetErrorString(e));
}

int ple_bench_copy_rows(const void* src, int64_t src_rows, int32_t row_bytes, const int32_t* rows, int64_t nrows,
                        void* dst, void* stream) {
    if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > 16384)
        return fail(PLE_ERR_INVALID_ARGUMENT, "row_bytes must be a multiple of 16 in 16..16384");
    if (src_rows < 1 || nrows < 0) return fail(PLE_ERR_INVALID_ARGUMENT, "src_rows >= 1 and nrows >= 0");
    if (nrows == 0) return PLE_OK;
    if (src == nullptr || dst == nullptr || rows == nullptr || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15) ||
        ((uintptr_t)rows & 3))
        return fail(PLE_ERR_INVALID_ARGUMENT, "src, dst and rows must be non-NULL and aligned");
    const int64_t waves = (nrows + kRowsPerWave - 1) / kRowsPerWave;
    if (row_bytes == 16 * kWave)
        hipLaunchKernelGGL(copy_rows_kernel<true>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                           (hipStream_t)stream, (const u32x4*)src, src_rows, row_bytes / 16, rows, nrows, (u32x4*)dst);
    else
        hipLaunchKernelGGL(copy_rows_kernel<false>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                           (hipStream_t)stream, (const u32x4*)src, src_rows, row_bytes / 16, rows, nrows, (u32x4*)dst);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PLE_OK : fail(PLE_ERR_DEVICE, "copy_rows launch: %s", hipGetErrorString(e));
}

}  // extern "C"
