// Streaming-copy ceilings for the benchmark (include/ple_bench.h): a
// contiguous copy, a row gather from caller indices and a widening row
// gather with a quantized table's side reads, all one pass of 16-byte chunks
// per lane with every load of a wave in flight before its stores, the shape
// that streams fastest on this GPU.  Kept apart from
// libple: they measure the memory system, they are not part of the path.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>

#include "ple.h"
#include "ple_bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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

// Row gather that widens, with a quantized table's side reads: output row k
// (out_cpr 16-byte chunks) holds input row rows[k] (16 / E bytes per output
// chunk) repeated E times.  AUX 1 reads one 4-byte word per row (one lane
// per row, shared by shuffle), AUX 2 one byte per 16 output elements (each
// lane its chunk's byte); the side value is XORed into the chunk so that its
// load counts.  A wave covers 1024 output chunks (1024 / out_cpr rows), all
// loads in flight before the stores.
template <int E, int AUX>
__global__ __launch_bounds__(256) void gather_expand_kernel(const char* __restrict__ src, int64_t src_rows,
                                                            const uint8_t* __restrict__ aux,
                                                            const int32_t* __restrict__ rows, int64_t nrows,
                                                            int out_cpr_log2, u32x4* __restrict__ dst) {
    constexpr int IB = 16 / E;  // input bytes per output chunk
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & (kWave - 1);
    const int out_cpr = 1 << out_cpr_log2;
    const int rpw = 1024 >> out_cpr_log2;
    const int64_t r0 = wave * rpw;
    if (r0 >= nrows) return;
    int my = 0;
    uint32_t my_aux = 0;
    if (lane < rpw && r0 + lane < nrows) {
        my = rows[r0 + lane];
        my = my < 0 ? 0 : (my >= src_rows ? (int)(src_rows - 1) : my);
        if (AUX == 1) my_aux = ((const uint32_t*)aux)[my];
    }
    const int64_t in_row_bytes = (int64_t)out_cpr * IB;
    u32x4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int idx = u * kWave + lane;
        const int row = idx >> out_cpr_log2;
        const int ch = idx & (out_cpr - 1);
        const int id = __shfl(my, row, kWave);
        const uint32_t a = AUX == 1 ? __shfl(my_aux, row, kWave) : 0u;
        if (r0 + row < nrows) {
            const char* p = src + (int64_t)id * in_row_bytes + ch * IB;
            if (E == 1) {
                v[u] = __builtin_nontemporal_load((const u32x4*)p);
            } else if (E == 2) {
                const u32x2 q = __builtin_nontemporal_load((const u32x2*)p);
                v[u] = u32x4{q.x, q.y, q.x, q.y};
            } else {
                const uint32_t w = __builtin_nontemporal_load((const uint32_t*)p);
                v[u] = u32x4{w, w, w, w};
            }
            if (AUX == 1) v[u].x ^= a;
            if (AUX == 2) v[u].x ^= aux[(int64_t)id * (out_cpr >> 1) + (ch >> 1)];
        }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int idx = u * kWave + lane;
        if (r0 + (idx >> out_cpr_log2) < nrows) __builtin_nontemporal_store(v[u], dst + r0 * out_cpr + idx);
    }
}

template <int E>
void launch_expand(int aux_mode, unsigned blocks, hipStream_t s, const char* src, int64_t src_rows,
                   const uint8_t* aux, const int32_t* rows, int64_t nrows, int l2, u32x4* dst) {
    if (aux_mode == 1)
        hipLaunchKernelGGL((gather_expand_kernel<E, 1>), dim3(blocks), dim3(256), 0, s, src, src_rows, aux, rows,
                           nrows, l2, dst);
    else if (aux_mode == 2)
        hipLaunchKernelGGL((gather_expand_kernel<E, 2>), dim3(blocks), dim3(256), 0, s, src, src_rows, aux, rows,
                           nrows, l2, dst);
    else
        hipLaunchKernelGGL((gather_expand_kernel<E, 0>), dim3(blocks), dim3(256), 0, s, src, src_rows, aux, rows,
                           nrows, l2, dst);
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

int ple_bench_gather_expand(const void* src, int64_t src_rows, int32_t expand, const void* aux, int32_t aux_mode,
                            const int32_t* rows, int64_t nrows, int32_t out_row_bytes, void* dst, void* stream) {
    if (expand != 1 && expand != 2 && expand != 4) return fail(PLE_ERR_INVALID_ARGUMENT, "expand must be 1, 2 or 4");
    if (aux_mode < 0 || aux_mode > 2) return fail(PLE_ERR_INVALID_ARGUMENT, "aux_mode must be 0, 1 or 2");
    if (out_row_bytes < 32 || out_row_bytes > 16384 || (out_row_bytes & (out_row_bytes - 1)) != 0)
        return fail(PLE_ERR_INVALID_ARGUMENT, "out_row_bytes must be a power of two in 32..16384");
    if (src_rows < 1 || nrows < 0) return fail(PLE_ERR_INVALID_ARGUMENT, "src_rows >= 1 and nrows >= 0");
    if (nrows == 0) return PLE_OK;
    if (src == nullptr || dst == nullptr || rows == nullptr || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15) ||
        ((uintptr_t)rows & 3))
        return fail(PLE_ERR_INVALID_ARGUMENT, "src, dst and rows must be non-NULL and aligned");
    if (aux_mode != 0 && (aux == nullptr || (aux_mode == 1 && ((uintptr_t)aux & 3))))
        return fail(PLE_ERR_INVALID_ARGUMENT, "aux must be non-NULL (and 4-byte aligned for mode 1)");
    const int out_cpr = out_row_bytes / 16;
    if (out_cpr > 1024) return fail(PLE_ERR_INVALID_ARGUMENT, "out_row_bytes at most 16384");
    int l2 = 0;
    while ((1 << l2) < out_cpr) ++l2;
    const int64_t rpw = 1024 / out_cpr;
    const int64_t waves = (nrows + rpw - 1) / rpw;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    hipStream_t s = (hipStream_t)stream;
    const char* sp = (const char*)src;
    const uint8_t* ap = (const uint8_t*)aux;
    if (expand == 1)
        launch_expand<1>(aux_mode, blocks, s, sp, src_rows, ap, rows, nrows, l2, (u32x4*)dst);
    else if (expand == 2)
        launch_expand<2>(aux_mode, blocks, s, sp, src_rows, ap, rows, nrows, l2, (u32x4*)dst);
    else
        launch_expand<4>(aux_mode, blocks, s, sp, src_rows, ap, rows, nrows, l2, (u32x4*)dst);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PLE_OK : fail(PLE_ERR_DEVICE, "gather_expand launch: %s", hipGetErrorString(e));
}

}  // extern "C"
