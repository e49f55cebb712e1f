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
// maps each row ID to the position of the row that inserted it first.  Two
// compact lists follow from the inserts: those positions, one per distinct
// ID, for the gather to read from the table, and every other position, whose
// row is then copied from the first one within the staging rows (the same
// lookup kernel walks both lists).  Which position wins the insert race does
// not matter: all of them hold the same row.  The keys and the lists' counts
// are cleared by the ID launch before.
#include "ple_launch.h"

namespace ple {

__device__ __forceinline__ uint32_t dedup_slot(int32_t id, int log2cap) {
    return ((uint32_t)id * 0x9E3779B1u) >> (32 - log2cap);  // Fibonacci hashing
}

// keys[s] = the row ID owning slot s, rep[s] = the position that inserted it;
// slot_of[i] = the slot of position i's ID; the inserting positions are
// appended to list, the others to repeats.  Device-wide atomics are slow
// (they are resolved beyond the per-XCD L2), so a wave first elects one lane
// per distinct ID among its 64, a lane probes with plain loads and only tries
// the compare-and-swap on a free slot, and the wave reserves its entries of
// each list with one add.
__device__ __forceinline__ void append_wave(bool mine, int lane, int32_t* count, int32_t* out, int32_t value) {
    const uint64_t m = __ballot(mine);
    if (m == 0) return;  // whole wave
    const int first = __ffsll((unsigned long long)m) - 1;
    int base = 0;
    if (lane == first) base = atomicAdd(count, __popcll(m));
    base = __shfl(base, first, 64);
    if (mine) out[base + __popcll(m & ((1ull << lane) - 1ull))] = value;  // rank among the lanes below
}

__global__ __launch_bounds__(256) void dedup_insert_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                           int32_t* __restrict__ keys, int32_t* __restrict__ rep,
                                                           int log2cap, int32_t* __restrict__ slot_of,
                                                           int32_t* __restrict__ list, int32_t* __restrict__ repeats,
                                                           int32_t* __restrict__ counts) {
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
    append_wave(inserted, lane, counts, list, (int32_t)i);
    append_wave(i < n && !inserted, lane, counts + 1, repeats, (int32_t)i);
}

__global__ void dedup_count_kernel(const int32_t* __restrict__ count, int32_t* __restrict__ num_unique) {
    if (threadIdx.x == 0) *num_unique = count != nullptr ? *count : 0;
}

hipError_t launch_dedup_insert(const int32_t* ids, int64_t n, int32_t* keys, int32_t* rep, int log2cap,
                               int32_t* slot_of, int32_t* list, int32_t* repeats, int32_t* counts, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(dedup_insert_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids, n, keys, rep,
                       log2cap, slot_of, list, repeats, counts);
    return hipGetLastError();
}

hipError_t launch_dedup_count(const int32_t* count, int32_t* num_unique, hipStream_t s) {
    hipLaunchKernelGGL(dedup_count_kernel, dim3(1), dim3(64), 0, s, count, num_unique);
    return hipGetLastError();
}

}  // namespace ple
