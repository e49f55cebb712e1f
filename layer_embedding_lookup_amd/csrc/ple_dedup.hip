// Repeated-row elimination before a host-link read.
//
// Method: the host-resident table of "PR #54371 [Qwen4Exp] Support UVA
// PLE-offload and Engram tensor parallelism" (功能与动机: rows read across the
// host link by the GPU) and the prefetch of "PR #56512 [DS V4.1][Engram]
// async prefetch for offloaded engram lookups and engram DP sharding"
// (功能与动机: the host-link time of the lookup is what the prefetch hides).
// Rows that repeat within a batch (the same n-gram in several places) need
// to cross the host link once: the first occurrence is read from the host
// table, the others are copied from it in device memory.
//
// An open-addressing hash set in device memory (capacity a power of two at
// least twice the number of rows, so linear probing ends within a few slots)
// maps each row ID to the position of the row that inserted it first; every
// other position with that ID copies that row.  Which position wins the
// insert race does not matter: all of them hold the same row.
#include "ple_launch.h"

namespace ple {

__device__ __forceinline__ uint32_t dedup_slot(int32_t id, int log2cap) {
    return ((uint32_t)id * 0x9E3779B1u) >> (32 - log2cap);  // Fibonacci hashing
}

__global__ __launch_bounds__(256) void dedup_clear_kernel(int32_t* __restrict__ keys, int64_t cap,
                                                          int32_t* __restrict__ num_unique) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cap; i += (int64_t)gridDim.x * blockDim.x)
        keys[i] = -1;
    if (num_unique != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *num_unique = 0;
}

// keys[s] = the row ID owning slot s, rep[s] = the position that inserted it;
// slot_of[i] = the slot of position i's ID.  Device-wide atomics are slow
// (they are resolved beyond the per-XCD L2), so a wave first elects one lane
// per distinct ID among its 64, and a lane probes with plain loads and only
// tries the compare-and-swap on a free slot.
__global__ __launch_bounds__(256) void dedup_insert_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                           int32_t* __restrict__ keys, int32_t* __restrict__ rep,
                                                           int log2cap, int32_t* __restrict__ slot_of,
                                                           int32_t* __restrict__ num_unique) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    const int32_t id = i < n ? ids[i] : -2 - lane;  // past the end: distinct, never inserted
    int leader = lane;
#pragma unroll 8
    for (int k = 0; k < 64; ++k) {
        const int32_t other = __shfl(id, k, 64);
        if (k < leader && other == id) leader = k;
    }
    const uint32_t mask = (1u << log2cap) - 1u;
    uint32_t s = dedup_slot(id, log2cap);
    bool inserted = false;
    if (i < n && leader == lane) {
        // at most cap probes; with the load factor at most 1/2 a free or
        // matching slot comes long before that
        for (uint32_t probe = 0; probe <= mask; ++probe) {
            int32_t cur = __hip_atomic_load(keys + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (cur == -1) {
                cur = atomicCAS(keys + s, -1, id);
                if (cur == -1) {
                    rep[s] = (int32_t)i;
                    inserted = true;
                    break;
                }
            }
            if (cur == id) break;
            s = (s + 1) & mask;
        }
    }
    s = (uint32_t)__shfl((int)s, leader, 64);
    if (i < n) slot_of[i] = (int32_t)s;
    // one counter update per wave (a single address takes one atomic at a time)
    const int won = __popcll(__ballot(inserted));
    if (num_unique != nullptr && lane == 0 && won > 0) atomicAdd(num_unique, won);
}

// rep_of[i] = the position whose row position i copies (i itself for the first).
// slot_of and rep_of may be the same array: each position reads and then
// writes only its own entry.
__global__ __launch_bounds__(256) void dedup_resolve_kernel(const int32_t* slot_of, int64_t n,
                                                            const int32_t* __restrict__ rep, int32_t* rep_of) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int32_t r = rep[slot_of[i]];
    rep_of[i] = (r >= 0 && r < n) ? r : (int32_t)i;  // every slot_of entry was inserted; the guard only bounds reads
}

// rows[i] = rows[rep_of[i]] for every repeated position (the first
// occurrences were gathered before and are only read here).  A wave walks
// 1024 consecutive 16-byte chunks of the [n][dim] rows.
__global__ __launch_bounds__(256) void dedup_copy_kernel(const int32_t* __restrict__ rep_of, int64_t n, int cpr,
                                                         u32x4* __restrict__ rows) {
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t total = n * (int64_t)cpr;
    // each wave copies 16 chunks per lane: positions [wave*1024, wave*1024+1024) of the chunk space
    for (int u = 0; u < 16; ++u) {
        const int64_t c = wave * 1024 + (int64_t)u * 64 + lane;
        if (c >= total) break;
        const int64_t i = c / cpr;
        const int32_t r = rep_of[i];
        if (r != (int32_t)i) rows[c] = rows[(int64_t)r * cpr + (c - i * cpr)];
    }
}

// n == 0 (keys may then be NULL) only zeroes num_unique.
hipError_t launch_dedup(const int32_t* ids, int64_t n, int32_t* keys, int32_t* rep, int log2cap,
                        int32_t* slot_rep, int32_t* num_unique, hipStream_t s) {
    const int64_t cap = n > 0 ? (int64_t)1 << log2cap : 0;
    int64_t cb = (cap + 255) / 256;
    if (cb < 1) cb = 1;
    if (cb > 4096) cb = 4096;
    hipLaunchKernelGGL(dedup_clear_kernel, dim3((unsigned)cb), dim3(256), 0, s, keys, cap, num_unique);
    if (n == 0) return hipGetLastError();
    const unsigned nb = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(dedup_insert_kernel, dim3(nb), dim3(256), 0, s, ids, n, keys, rep, log2cap, slot_rep,
                       num_unique);
    // resolve in place: slot_of -> rep_of (each position reads only its own entry)
    hipLaunchKernelGGL(dedup_resolve_kernel, dim3(nb), dim3(256), 0, s, slot_rep, n, rep, slot_rep);
    return hipGetLastError();
}

hipError_t launch_dedup_copy(const int32_t* rep_of, int64_t n, int dim, uint16_t* rows, hipStream_t s) {
    const int cpr = dim / 8;
    const int64_t waves = (n * cpr + 1023) / 1024;
    hipLaunchKernelGGL(dedup_copy_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, rep_of, n, cpr,
                       (u32x4*)rows);
    return hipGetLastError();
}

}  // namespace ple
