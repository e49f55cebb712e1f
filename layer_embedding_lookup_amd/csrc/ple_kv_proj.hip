// Merged key/value projection kv = x . W^T on the CDNA4 matrix cores.
//
// Method: "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels", 实现拆解
// item 1 (key and value projections merged into one linear layer producing
// [key | value]).
//
// x [M][K] (gathered rows, K = H*D) and W [O][K] are both K-contiguous, so
// every lane's MFMA operand (8 consecutive bf16 along K) is one 16-byte read
// for both sides.  Problems with at least 256 tiles of 256 x 256 run on
// eight waves of 128 x 64 with 16x16x32 MFMAs (kv_proj_pipe8w, two waves per
// SIMD); smaller ones on one four-wave pipelined body of 32x32x16 MFMAs at
// 128 x 128 tiles (a 1024-token speculative-verify batch) or 64 x 64 tiles
// (decode batches).
// The designs are described above the bodies.  The block tile is the largest
// that still gives 256 blocks, one per CU.  Blocks are numbered so that the blocks resident on one XCD (block id
// mod 8 picks the XCD) work on neighbouring tiles and share their x and W
// panels in that XCD's L2.
#include "ple_launch.h"

#include <type_traits>

namespace ple {

// Tile order: XCD-major then grouped row-major (GROUP_M tile rows share W panels).
template <int GROUP_M>
__device__ __forceinline__ void tile_of_block(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    // Blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous
    // range of tiles (when the count divides evenly).
    int lin = bid;
    if ((total & 7) == 0) {
        const int per = total >> 3;
        lin = (bid & 7) * per + (bid >> 3);
    }
    const int group = lin / (GROUP_M * tiles_n);
    const int first_m = group * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int in_group = lin - group * GROUP_M * tiles_n;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// ---------------------------------------------------------------------------
// Pipelined kernel body for batches too small to give 256 blocks of 256 x
// 256: BT x BT block tile, 4 waves (one per SIMD), each a (BT/2) x (BT/2)
// block held in accumulator tiles of 32 x 32.  For BT = 128 that is 4 tiles
// and LDS stages of 32 KiB; for BT = 64, one tile and stages of 16 KiB.
// K-slices of 64.
//
// Why this shape: the fragment reads of the next 16-deep K-step are spread
// between the current step's MFMAs, so with one wave per SIMD the matrix core
// stays fed without a second wave to cover for it; the narrow tiles give
// blocks: a 1024-token batch gets 256 blocks of 128 x 128, a 256-token decode
// batch 256 blocks of 64 x 64 (there the W panels, read by four blocks each
// from the XCD's L2, bound the kernel, not the matrix cores).
//
// Operands go global -> LDS with buffer loads that write LDS directly
// (buffer_load_dwordx4 ... lds): a scalar buffer resource per operand panel
// and a 32-bit per-lane offset.  Each copy instruction fills 1 KiB = 8 whole
// 128-byte K-slice rows, so every request is a full cache line.  The copies
// of slice kt+2 go into the stage slice kt has just left: they start between
// the last K-step's MFMAs of slice kt (after the barrier that ends every read
// of that stage) and finish between the first K-step's MFMAs of slice kt+1,
// and the barrier at the end of slice kt+1 waits for them.
//
// LDS layout of one operand slice: row r holds 8 chunks of 16 bytes (64
// bf16 of K); chunk kc sits at position r*8 + (kc ^ ((r >> 1) & 7)).  A
// fragment read takes one k-chunk of 32 consecutive rows; the LDS serves 16
// lanes (256 bytes, 64 banks) per cycle and any 16 consecutive rows land on
// distinct 16-byte bank groups.  The MFMA operands are swapped (W fragment
// first) so each lane's accumulators are 4 consecutive output features of one
// token, which the epilogue writes to LDS as 8-byte pairs before coalesced
// 16-byte stores.
//
// The LDS fragment reads are inline assembly with explicit waits: the
// compiler's own waits would drain every read in flight before each MFMA
// group, which exposes the LDS latency on every K-step.  Each wait lists the
// fragment registers it covers as operands, so no MFMA can be scheduled
// above the wait for its inputs.
// ---------------------------------------------------------------------------
constexpr int kBigThreads = 256;
constexpr int kBBK = 64;
constexpr int kNStage = 2;
constexpr int kBigMaxK = 1 << 20;  // keeps 256 rows of K bf16 within a 32-bit buffer offset

// Block tile BT x BT (256, or 128 / 64 for problems too small to fill the
// chip with wider tiles); each of the 4 waves holds a (BT/2) x (BT/2) block
// as NB x NB accumulator tiles of 32 x 32.
template <int BT>
struct PipeShape {
    static constexpr int NB = BT / 64;                    // 32-row blocks per wave and operand
    static constexpr int NCOPY = BT / 32;                 // copy instructions per operand, wave and slice
    static constexpr int COPY_SPLIT = NCOPY / 2;          // of those, issued in a slice's last K-step (2 stages)
    static constexpr int OP_BYTES = BT * kBBK * 2;        // one operand's slice (BT rows of 128 bytes)
    static constexpr int STAGE_BYTES = 2 * OP_BYTES;      // x + W slices
    // LDS stages: the narrower tiles run fewer MFMAs per slice, so more
    // slices are kept in flight to cover the copy latency (128 KiB each way)
    static constexpr int NS = BT == 256 ? kNStage : (128 * 1024) / STAGE_BYTES;
    static constexpr int OUT_ROW = BT + 8;                // epilogue row (elements)
    static constexpr int LDS_BYTES = (NS * STAGE_BYTES > BT * OUT_ROW * 2) ? NS * STAGE_BYTES : BT * OUT_ROW * 2;
    // copy instructions of one slice (both operands) per wave
    static constexpr int SLICE_COPIES = 2 * NCOPY;
    static_assert((NS & (NS - 1)) == 0 && (NS - 1) * SLICE_COPIES <= 63, "stages must fit the vmcnt counter");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait for this wave's copies and LDS reads, then join the workgroup barrier.
// The "memory" clobber keeps the compiler from moving LDS or global accesses
// across it.
#define PLE_WAIT_VM_BARRIER0() asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory")

template <int NB>
struct PipeFrag {
    u32x4 a[NB], b[NB];  // x fragments of the token blocks, W fragments of the feature blocks
};
// A wait names the fragment registers it covers, so no MFMA reading them can
// be scheduled above it.
#define PLE_FRAG_REGS4(f) \
    "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3])
#define PLE_FRAG_REGS2(f) "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.b[0]), "+v"(f.b[1])
#define PLE_FRAG_REGS1(f) "+v"(f.a[0]), "+v"(f.b[0])

template <int BT>
__device__ __forceinline__ void kv_proj_pipe(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int M,
                                             int K, int O, uint16_t* __restrict__ out) {
    using P = PipeShape<BT>;
    constexpr int NB = P::NB;
    constexpr int WT = BT / 2;  // wave block
    using Frag = PipeFrag<NB>;
    extern __shared__ __align__(16) char lds_raw[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves: WT tokens x WT features each

    const int tiles_m = (M + BT - 1) / BT;
    const int tiles_n = (O + BT - 1) / BT;
    int tm, tn;
    tile_of_block<8>(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BT, n0 = tn * BT;

    // Copy instruction i (0..NCOPY-1) of wave `wave` fills rows g*8 .. g*8+7
    // of an operand slice, g = i*4 + wave; lane L lands at position g*64 + L:
    // row g*8 + L/8, chunk kc = (L & 7) ^ ((row >> 1) & 7).  Rows past the end
    // of x or W read the last row (their outputs are never stored).
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + (int64_t)m0 * K), (short)0, min(M - m0, BT) * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w + (int64_t)n0 * K), (short)0, min(O - n0, BT) * K * 2, 0x00020000);
    uint32_t aoff[P::NCOPY], boff[P::NCOPY];
#pragma unroll
    for (int i = 0; i < P::NCOPY; ++i) {
        const int row = (i * 4 + wave) * 8 + (lane >> 3);
        const int kc = (lane & 7) ^ ((row >> 1) & 7);
        aoff[i] = (uint32_t)((min(m0 + row, M - 1) - m0) * K * 2 + kc * 16);
        boff[i] = (uint32_t)((min(n0 + row, O - 1) - n0) * K * 2 + kc * 16);
    }
    const int nk = K / kBBK;
    // copy instruction i of slice kt into stage kt % NS; slices past the end
    // (the loop below is uniform) re-read the last slice into a stage that no
    // later read uses
    auto copy_one = [&](int kt, int i) {
        char* base = lds_raw + (kt & (P::NS - 1)) * P::STAGE_BYTES;
        const int g = i * 4 + wave;
        const int ko = min(kt, nk - 1) * kBBK * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(base + g * 1024), 16, aoff[i], ko, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(base + P::OP_BYTES + g * 1024), 16, boff[i], ko, 0,
                                                 0);
    };

    f32x16 acc[NB][NB];  // [W block j][x block i]
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;

    const int frow = lane & 31;
    const int fk = lane >> 5;
    const int sw = (frow >> 1) & 7;  // the chunk swizzle, the same for every 32-row block
    // LDS byte address of this lane's fragment chunk for K-step kk in stage 0,
    // first 32-row block (the others are +4096 bytes each)
    uint32_t a_addr[4], b_addr[4];
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_raw;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const uint32_t col = (uint32_t)(((kk * 2 + fk) ^ sw) * 16);
        a_addr[kk] = lds_base + (wm * WT + frow) * 128 + col;
        b_addr[kk] = lds_base + P::OP_BYTES + (wn * WT + frow) * 128 + col;
    }
    // fragment read q (0..2*NB-1) of K-step kk of slice kt: x blocks, then W blocks
    auto read_one = [&](int q, int kt, int kk, Frag& f) {
        const uint32_t so = (uint32_t)(kt & (P::NS - 1)) * P::STAGE_BYTES;
        const uint32_t pa = a_addr[kk] + so, pb = b_addr[kk] + so;
        if constexpr (NB == 4) {
            switch (q) {
                case 0: asm volatile("ds_read_b128 %0, %1" : "=v"(f.a[0]) : "v"(pa)); break;
                case 1: asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(f.a[1]) : "v"(pa)); break;
                case 2: asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(f.a[2]) : "v"(pa)); break;
                case 3: asm volatile("ds_read_b128 %0, %1 offset:12288" : "=v"(f.a[3]) : "v"(pa)); break;
                case 4: asm volatile("ds_read_b128 %0, %1" : "=v"(f.b[0]) : "v"(pb)); break;
                case 5: asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(f.b[1]) : "v"(pb)); break;
                case 6: asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(f.b[2]) : "v"(pb)); break;
                default: asm volatile("ds_read_b128 %0, %1 offset:12288" : "=v"(f.b[3]) : "v"(pb)); break;
            }
        } else if constexpr (NB == 2) {
            switch (q) {
                case 0: asm volatile("ds_read_b128 %0, %1" : "=v"(f.a[0]) : "v"(pa)); break;
                case 1: asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(f.a[1]) : "v"(pa)); break;
                case 2: asm volatile("ds_read_b128 %0, %1" : "=v"(f.b[0]) : "v"(pb)); break;
                default: asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(f.b[1]) : "v"(pb)); break;
            }
        } else {
            if (q == 0)
                asm volatile("ds_read_b128 %0, %1" : "=v"(f.a[0]) : "v"(pa));
            else
                asm volatile("ds_read_b128 %0, %1" : "=v"(f.b[0]) : "v"(pb));
        }
    };
    auto wait_frag = [&](Frag& f) {
        if constexpr (NB == 4)
            asm volatile("s_waitcnt lgkmcnt(0)" : PLE_FRAG_REGS4(f));
        else if constexpr (NB == 2)
            asm volatile("s_waitcnt lgkmcnt(0)" : PLE_FRAG_REGS2(f));
        else
            asm volatile("s_waitcnt lgkmcnt(0)" : PLE_FRAG_REGS1(f));
    };
    // the barrier of an NS-stage slice: this wave's copies of every slice but
    // the next NS-2 have landed
    auto wait_barrier_vm = [&](Frag& f) {
        constexpr int V = (P::NS - 2) * P::SLICE_COPIES;
        if constexpr (NB == 2)
            asm volatile("s_waitcnt vmcnt(%4) lgkmcnt(0)\n\ts_barrier" : PLE_FRAG_REGS2(f) : "i"(V) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(%2) lgkmcnt(0)\n\ts_barrier" : PLE_FRAG_REGS1(f) : "i"(V) : "memory");
    };
    auto wait_barrier = [&](Frag& f) {
        if constexpr (NB == 4)
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : PLE_FRAG_REGS4(f) : : "memory");
        else if constexpr (NB == 2)
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : PLE_FRAG_REGS2(f) : : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : PLE_FRAG_REGS1(f) : : "memory");
    };
    // One K-step: NB*NB MFMAs on `cur`.  After MFMA t < 2*NB comes fragment
    // read t of (rkt, rkk) into `nxt`, and copy instructions [c0, c1) of slice
    // ckt are spread over the MFMAs.  The order is pinned.
    auto kstep = [&](const Frag& cur, Frag& nxt, int rkt, int rkk, int ckt, int c0, int c1) {
        constexpr int NT = NB * NB;
        const int nc = c1 - c0;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int j = t / NB, i = t % NB;
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur.b[j]),
                                                                __builtin_bit_cast(bf16x8, cur.a[i]), acc[j][i], 0, 0,
                                                                0);
            if (rkk >= 0) {
                if constexpr (2 * NB <= NT) {
                    if (t < 2 * NB) read_one(t, rkt, rkk, nxt);
                } else {
#pragma unroll
                    for (int q = 0; q < 2 * NB; ++q) read_one(q, rkt, rkk, nxt);  // NT == 1
                }
            }
            if (nc > 0 && nc <= NT && (t * nc) % NT < nc) copy_one(ckt, c0 + (t * nc) / NT);
            if (nc > NT)
#pragma unroll
                for (int c = (t * nc) / NT; c < ((t + 1) * nc) / NT; ++c) copy_one(ckt, c0 + c);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // One slice.  On entry f0 is receiving K-step 0 of slice kt.  LDS reads
    // return in order, so when a K-step starts, the reads issued during the
    // previous one are the only ones in flight and waiting for all of them
    // covers its fragments.  The first K-step finishes the copies of slice
    // kt+1 that slice kt-1 began; the last begins those of slice kt+2, into
    // the stage this slice has just left.  The last slice's look-ahead reads
    // and copies land in the other stage and are never used.
    auto slice = [&](int kt, Frag& f0, Frag& f1) {
        if constexpr (P::NS == 2) {
            wait_frag(f0);
            kstep(f0, f1, kt, 1, kt + 1, P::COPY_SPLIT, P::NCOPY);
            wait_frag(f1);
            kstep(f1, f0, kt, 2, 0, 0, 0);
            wait_frag(f0);
            kstep(f0, f1, kt, 3, 0, 0, 0);
            // every read of this stage is complete (all waves) and slice kt+1 has landed
            __builtin_amdgcn_sched_barrier(0);
            wait_barrier(f1);
            __builtin_amdgcn_sched_barrier(0);
            kstep(f1, f0, kt + 1, 0, kt + 2, 0, P::COPY_SPLIT);
        } else {
            // NS stages: slices kt+1 .. kt+NS-1 are in flight or landed; after
            // the barrier (this wave's copies of slice kt+1 done, every read of
            // slice kt done) the last K-step refills slice kt's stage with
            // slice kt+NS
            wait_frag(f0);
            kstep(f0, f1, kt, 1, 0, 0, 0);
            wait_frag(f1);
            kstep(f1, f0, kt, 2, 0, 0, 0);
            wait_frag(f0);
            kstep(f0, f1, kt, 3, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            wait_barrier_vm(f1);
            __builtin_amdgcn_sched_barrier(0);
            kstep(f1, f0, kt + 1, 0, kt + P::NS, 0, P::NCOPY);
        }
    };

    Frag f0, f1;
    if constexpr (P::NS == 2) {
        // slice 0 whole, then the first part of slice 1
#pragma unroll
        for (int i = 0; i < P::NCOPY; ++i) copy_one(0, i);
        PLE_WAIT_VM_BARRIER0();
#pragma unroll
        for (int i = 0; i < P::COPY_SPLIT; ++i) copy_one(1, i);
    } else {
        // slices 0 .. NS-1, then wait for slice 0
#pragma unroll
        for (int k = 0; k < P::NS; ++k)
#pragma unroll
            for (int i = 0; i < P::NCOPY; ++i) copy_one(k, i);
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "i"((P::NS - 1) * P::SLICE_COPIES) : "memory");
    }
#pragma unroll
    for (int q = 0; q < 2 * NB; ++q) read_one(q, 0, 0, f0);
    for (int kt = 0; kt < nk; ++kt) slice(kt, f0, f1);
    // The last slice's look-ahead reads into f0 are still in flight and
    // opaque to the compiler's own waits: this wait names f0's registers, so
    // no epilogue value is placed in them before the reads have landed.
    if constexpr (NB == 4)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : PLE_FRAG_REGS4(f0) : : "memory");
    else if constexpr (NB == 2)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : PLE_FRAG_REGS2(f0) : : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : PLE_FRAG_REGS1(f0) : : "memory");
    __syncthreads();  // every wave is done with the stages before the epilogue reuses LDS

    // epilogue: acc[j][i][e] is feature n0 + wn*WT + j*32 + 8*(e/4) + 4*(lane/32) + e%4
    // of token m0 + wm*WT + i*32 + lane%32
    uint16_t* Cs = (uint16_t*)lds_raw;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int m = wm * WT + i * 32 + frow;
                const int o = wn * WT + j * 32 + 8 * g + 4 * fk;
                const uint32_t lo = pack_bf16x2(acc[j][i][4 * g], acc[j][i][4 * g + 1]);
                const uint32_t hi = pack_bf16x2(acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]);
                *(uint2*)(Cs + m * P::OUT_ROW + o) = make_uint2(lo, hi);
            }
    __syncthreads();
#pragma unroll 4
    for (int c = tid; c < BT * BT / 8; c += kBigThreads) {
        const int row = c / (BT / 8);  // BT/8 chunks of 8 features per row
        const int col = (c % (BT / 8)) * 8;
        const int gr = m0 + row, gc = n0 + col;
        if (gr < M && gc < O) *(u32x4*)(out + (int64_t)gr * O + gc) = *(const u32x4*)(Cs + row * P::OUT_ROW + col);
    }
}

// ---------------------------------------------------------------------------
// 256-wide tiles with eight waves (two per SIMD) on 16x16x32 MFMAs: wave
// (wm, wn) holds a 128 x 64 block (x rows wm*128.., W rows wn*64..) as 8 x 4
// accumulator tiles of 16 x 16 (128 accumulation registers), so a wave
// waiting on its fragments leaves the matrix core to the other wave of its
// SIMD.  Row layout in LDS and the copy instructions as the four-wave body; a
// slice is two K-steps of 32 with 12 fragment reads each.  Instead of two
// stages of both operands, the LDS holds a ring of five operand slices, which
// gives the W copies a second slice of lead.  The tiles an XCD runs at once
// are grouped four tile rows by eight tile columns, so each W panel is shared
// by four blocks in that XCD's L2 and each x panel by eight: more of the W
// copies wait on the last-level cache.
// ---------------------------------------------------------------------------
constexpr int kWideThreads = 512;
// five operand-slice slots (160 KiB, all of the LDS), which also hold the epilogue's rows
constexpr int kWideLdsBytes = 5 * PipeShape<256>::OP_BYTES;
static_assert(kWideLdsBytes >= PipeShape<256>::LDS_BYTES, "the epilogue's rows fit in the ring");
struct Frag8w {
    u32x4 a[8], b[4];
};
#define PLE_FRAG8W_REGS(f)                                                                                       \
    "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.a[4]), "+v"(f.a[5]), "+v"(f.a[6]), "+v"(f.a[7]), \
        "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3])

__device__ __forceinline__ void kv_proj_pipe8w(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int M,
                                               int K, int O, uint16_t* __restrict__ out) {
    using P = PipeShape<256>;
    constexpr int BT = 256, NC = 4;  // copy instructions per operand, wave and slice
    extern __shared__ __align__(16) char lds_raw[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int tiles_m = (M + BT - 1) / BT;
    const int tiles_n = (O + BT - 1) / BT;
    int tm, tn;
    tile_of_block<4>(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BT, n0 = tn * BT;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + (int64_t)m0 * K), (short)0, min(M - m0, BT) * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w + (int64_t)n0 * K), (short)0, min(O - n0, BT) * K * 2, 0x00020000);
    // copy instruction i of wave `wave` fills rows g*8 .. g*8+7, g = i*8 + wave
    uint32_t aoff[NC], boff[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int row = (i * 8 + wave) * 8 + (lane >> 3);
        const int kc = (lane & 7) ^ ((row >> 1) & 7);
        aoff[i] = (uint32_t)((min(m0 + row, M - 1) - m0) * K * 2 + kc * 16);
        boff[i] = (uint32_t)((min(n0 + row, O - 1) - n0) * K * 2 + kc * 16);
    }
    const int nk = K / kBBK;
    // Operand ring: W slice k in slot k mod 3, x slice k in slot 3 + k mod 2
    // (slots of one operand slice, 32 KiB).  W slices are copied two slices
    // ahead of their use and x slices one ahead, each into the slot its
    // operand's slice three (W) or two (x) back has just left.
    auto copy_x = [&](int k, int i) {  // k uniform
        char* base = lds_raw + (3 + (k & 1)) * P::OP_BYTES + (i * 8 + wave) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)base, 16, aoff[i], min(k, nk - 1) * kBBK * 2, 0, 0);
    };
    auto copy_w = [&](int k, int i) {
        char* base = lds_raw + (k % 3) * P::OP_BYTES + (i * 8 + wave) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)base, 16, boff[i], min(k, nk - 1) * kBBK * 2, 0, 0);
    };

    f32x4 acc[4][8];  // [W block jb][x block ib]
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    const int fk = lane >> 4;
    const int sw = (frow >> 1) & 7;
    uint32_t a_addr[2], b_addr[2];
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_raw;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const uint32_t col = (uint32_t)(((ks * 4 + fk) ^ sw) * 16);
        a_addr[ks] = lds_base + (wm * 128 + frow) * 128 + col;
        b_addr[ks] = lds_base + (wn * 64 + frow) * 128 + col;
    }
    auto read_one = [&](int q, int kt, int ks, Frag8w& f) {
        const uint32_t pa = a_addr[ks] + (uint32_t)(3 + (kt & 1)) * P::OP_BYTES;
        const uint32_t pb = b_addr[ks] + (uint32_t)(kt % 3) * P::OP_BYTES;
        switch (q) {
            case 0: asm volatile("ds_read_b128 %0, %1" : "=v"(f.a[0]) : "v"(pa)); break;
            case 1: asm volatile("ds_read_b128 %0, %1 offset:2048" : "=v"(f.a[1]) : "v"(pa)); break;
            case 2: asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(f.a[2]) : "v"(pa)); break;
            case 3: asm volatile("ds_read_b128 %0, %1 offset:6144" : "=v"(f.a[3]) : "v"(pa)); break;
            case 4: asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(f.a[4]) : "v"(pa)); break;
            case 5: asm volatile("ds_read_b128 %0, %1 offset:10240" : "=v"(f.a[5]) : "v"(pa)); break;
            case 6: asm volatile("ds_read_b128 %0, %1 offset:12288" : "=v"(f.a[6]) : "v"(pa)); break;
            case 7: asm volatile("ds_read_b128 %0, %1 offset:14336" : "=v"(f.a[7]) : "v"(pa)); break;
            case 8: asm volatile("ds_read_b128 %0, %1" : "=v"(f.b[0]) : "v"(pb)); break;
            case 9: asm volatile("ds_read_b128 %0, %1 offset:2048" : "=v"(f.b[1]) : "v"(pb)); break;
            case 10: asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(f.b[2]) : "v"(pb)); break;
            default: asm volatile("ds_read_b128 %0, %1 offset:6144" : "=v"(f.b[3]) : "v"(pb)); break;
        }
    };
    auto wait_frag = [&](Frag8w& f) { asm volatile("s_waitcnt lgkmcnt(0)" : PLE_FRAG8W_REGS(f)); };
    // the wait leaves the NC copies of the newest W slice in flight (copies
    // complete in issue order, so every older one has landed)
    auto wait_barrier = [&](Frag8w& f) {
        asm volatile("s_waitcnt vmcnt(%12) lgkmcnt(0)\n\ts_barrier" : PLE_FRAG8W_REGS(f) : "i"(NC) : "memory");
    };
    // one K-step of 32: 32 MFMAs on cur; after MFMA t < 12, fragment read t of
    // (rkt, rks) into nxt; with ckt >= 0, the NC copies of x slice ckt after
    // MFMAs 2 and 10, then those of W slice ckt + 1 after MFMAs 18 and 26
    auto kstep = [&](const Frag8w& cur, Frag8w& nxt, int rkt, int rks, int ckt) {
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const int j = t / 8, i = t % 8;
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.b[j]),
                                                                __builtin_bit_cast(bf16x8, cur.a[i]), acc[j][i], 0, 0,
                                                                0);
            if (t < 12) read_one(t, rkt, rks, nxt);
            if (ckt >= 0 && t % 8 == 2) {
                if (t < 16) {
                    copy_x(ckt, 2 * (t / 8));
                    copy_x(ckt, 2 * (t / 8) + 1);
                } else {
                    copy_w(ckt + 1, 2 * (t / 8) - 4);
                    copy_w(ckt + 1, 2 * (t / 8) - 3);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    Frag8w f0, f1;
    // x0, W0, x1, W1, W2; slice 0 landed before the first reads
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
        for (int i = 0; i < NC; ++i) copy_x(k, i);
#pragma unroll
        for (int i = 0; i < NC; ++i) copy_w(k, i);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) copy_w(2, i);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "i"(3 * NC) : "memory");
#pragma unroll
    for (int q = 0; q < 12; ++q) read_one(q, 0, 0, f0);
    for (int kt = 0; kt < nk; ++kt) {
        wait_frag(f0);
        kstep(f0, f1, kt, 1, -1);
        __builtin_amdgcn_sched_barrier(0);
        wait_barrier(f1);  // slice kt+1 has landed; every read of slice kt is done
        __builtin_amdgcn_sched_barrier(0);
        kstep(f1, f0, kt + 1, 0, kt + 2);
    }
    // the last look-ahead reads into f0 land before its registers are reused
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : PLE_FRAG8W_REGS(f0) : : "memory");
    __syncthreads();

    // acc[jb][ib][e]: feature n0 + wn*64 + jb*16 + 4*fk + e of token m0 + wm*128 + ib*16 + frow
    uint16_t* Cs = (uint16_t*)lds_raw;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int m = wm * 128 + i * 16 + frow;
            const int o = wn * 64 + j * 16 + 4 * fk;
            *(uint2*)(Cs + m * P::OUT_ROW + o) =
                make_uint2(pack_bf16x2(acc[j][i][0], acc[j][i][1]), pack_bf16x2(acc[j][i][2], acc[j][i][3]));
        }
    __syncthreads();
#pragma unroll 4
    for (int c = tid; c < BT * BT / 8; c += kWideThreads) {
        const int row = c / (BT / 8);
        const int col = (c % (BT / 8)) * 8;
        const int gr = m0 + row, gc = n0 + col;
        if (gr < M && gc < O) *(u32x4*)(out + (int64_t)gr * O + gc) = *(const u32x4*)(Cs + row * P::OUT_ROW + col);
    }
}
#undef PLE_FRAG8W_REGS

#undef PLE_FRAG_REGS4
#undef PLE_FRAG_REGS2
#undef PLE_FRAG_REGS1

// The block tiles as plain kernels (their bodies use device-only
// builtins, which a kernel template would also instantiate for the host).
__global__ __launch_bounds__(kWideThreads, 1) void kv_proj_wide_kernel(const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ w, int M, int K,
                                                                       int O, uint16_t* __restrict__ out) {
    kv_proj_pipe8w(x, w, M, K, O, out);
}
__global__ __launch_bounds__(kBigThreads, 1) void kv_proj_mid_kernel(const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ w, int M, int K,
                                                                     int O, uint16_t* __restrict__ out) {
    kv_proj_pipe<128>(x, w, M, K, O, out);
}
__global__ __launch_bounds__(kBigThreads, 1) void kv_proj_small_kernel(const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ w, int M, int K,
                                                                       int O, uint16_t* __restrict__ out) {
    kv_proj_pipe<64>(x, w, M, K, O, out);
}

template <int BT>
static hipError_t launch_kv_proj_pipe(const uint16_t* x, const uint16_t* w, int64_t M, int K, int O, uint16_t* kv,
                                      hipStream_t s) {
    using P = PipeShape<BT>;
    static_assert(BT == 128 || BT == 64, "256-wide tiles run on the eight-wave body");
    const void* fn = BT == 128 ? (const void*)kv_proj_mid_kernel : (const void*)kv_proj_small_kernel;
    static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, P::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const int tiles = (int)((M + BT - 1) / BT) * ((O + BT - 1) / BT);
    if (BT == 128)
        hipLaunchKernelGGL(kv_proj_mid_kernel, dim3(tiles), dim3(kBigThreads), P::LDS_BYTES, s, x, w, (int)M, K, O,
                           kv);
    else
        hipLaunchKernelGGL(kv_proj_small_kernel, dim3(tiles), dim3(kBigThreads), P::LDS_BYTES, s, x, w, (int)M, K, O,
                           kv);
    return hipGetLastError();
}

hipError_t launch_kv_proj(const uint16_t* x, const uint16_t* w, int64_t M, int K, int O, uint16_t* kv,
                          hipStream_t s) {
    // the widest block tile that still gives 256 blocks
    if (K > kBigMaxK) return hipErrorInvalidValue;  // rejected by the argument checks before this
    const int64_t big_tiles = ((M + 255) / 256) * ((O + 255) / 256);
    if (big_tiles >= 256) {
        static const hipError_t attr = hipFuncSetAttribute((const void*)kv_proj_wide_kernel,
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, kWideLdsBytes);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(kv_proj_wide_kernel, dim3((unsigned)big_tiles), dim3(kWideThreads), kWideLdsBytes, s, x, w,
                           (int)M, K, O, kv);
        return hipGetLastError();
    }
    // (64-wide tiles take 128 KiB of LDS, so only while one block per CU covers them)
    const int64_t mid_tiles = ((M + 127) / 128) * ((O + 127) / 128);
    const int64_t small_tiles = ((M + 63) / 64) * ((O + 63) / 64);
    if (mid_tiles >= 256 || small_tiles > 256) return launch_kv_proj_pipe<128>(x, w, M, K, O, kv, s);
    return launch_kv_proj_pipe<64>(x, w, M, K, O, kv, s);
}

}  // namespace ple
