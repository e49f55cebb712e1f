// Rank-major row selection for a table sharded across data-parallel replicas.
//
// Method: "PR #54371 [Qwen4Exp] Support UVA PLE-offload and Engram tensor
// parallelism" (实现拆解 item 3: the IDs of every replica are gathered into
// equal padded slots and each replica selects its own token window) and
// "PR #56512 [DS V4.1][Engram] async prefetch for offloaded engram lookups
// and engram DP sharding" (实现拆解 items 3-4: head shards in TP-major order,
// and a kernel taking a rank's token window out of the rank-major gathered
// buffer).
//
// gathered [E][E*slot][W] -> out [n][E*W]: each thread moves one 16-byte
// chunk; consecutive threads write consecutive output chunks and read
// consecutive chunks of one shard row.
#include "ple_launch.h"

namespace ple {

__global__ __launch_bounds__(256) void select_rows_kernel(const u32x4* __restrict__ gathered, int E, int64_t slot,
                                                          int rank, int64_t n, int wc, u32x4* __restrict__ out) {
    // wc = 16-byte chunks per shard row; a token's output row is E*wc chunks
    const int64_t total = n * (int64_t)E * wc;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = c / ((int64_t)E * wc);
        const int64_t rem = c - t * E * wc;
        const int64_t k = rem / wc;
        const int64_t j = rem - k * wc;
        out[c] = gathered[((k * E * slot) + (int64_t)rank * slot + t) * wc + j];
    }
}

hipError_t launch_select_rows(const uint16_t* gathered, int E, int64_t slot, int rank, int64_t n, int width,
                              uint16_t* out, hipStream_t s) {
    const int wc = width / 8;
    const int64_t total = n * (int64_t)E * wc;
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    hipLaunchKernelGGL(select_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)gathered, E, slot,
                       rank, n, wc, (u32x4*)out);
    return hipGetLastError();
}

}  // namespace ple
