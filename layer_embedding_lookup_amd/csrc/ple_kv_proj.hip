// Merged key/value projection kv = x . W^T on the CDNA4 matrix cores.
//
// Method: "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels", 实现拆解
// item 1 (key and value projections merged into one linear layer producing
// [key | value]).
//
// x [M][K] (gathered rows, K = H*D) and W [O][K] are both K-contiguous, so
// every lane's MFMA operand (8 consecutive bf16 along K) is one 16-byte read
// for both sides.  Block tile BM x BN x 64, four waves in a 2x2 grid, each wave
// a (BM/2) x (BN/2) grid of v_mfma_f32_32x32x16_bf16 tiles with fp32
// accumulators.  Tiles are staged through double-buffered, row-padded LDS;
// the next K-slice's global loads are in flight while the current one feeds
// the MFMAs.  The epilogue rounds to bf16 through LDS so that the global
// stores are coalesced 16-byte rows.  Blocks are numbered so that the blocks
// resident on one XCD (block id mod 8 picks the XCD) work on neighbouring
// tiles and share their x and W panels in that XCD's L2.
#include "ple_launch.h"

#include <type_traits>

namespace ple {

constexpr int kBK = 64;
constexpr int kLdsPad = 8;             // bf16 elements of padding per LDS row
constexpr int kLdsRow = kBK + kLdsPad;  // 72 elements = 144 bytes

template <int BM, int BN>
struct GemmShape {
    static constexpr int TI = BM / 64;  // 32x32 MFMA tiles per wave along M
    static constexpr int TJ = BN / 64;  // ... along N
    static constexpr int A_CHUNKS = BM * kBK / 8 / 256;  // 16-byte chunks per thread per K-slice
    static constexpr int B_CHUNKS = BN * kBK / 8 / 256;
    static constexpr int LDS_TILE = (BM + BN) * kLdsRow;  // elements per buffer
    static constexpr int OUT_ROW = BN + 8;                // epilogue LDS row (elements)
    static constexpr int LDS_BYTES_MAIN = 2 * LDS_TILE * 2;
    static constexpr int LDS_BYTES_OUT = BM * OUT_ROW * 2;
    static constexpr int LDS_BYTES = LDS_BYTES_MAIN > LDS_BYTES_OUT ? LDS_BYTES_MAIN : LDS_BYTES_OUT;
};

// Tile order: XCD-major then grouped row-major (GROUP_M tile rows share W panels).
__device__ __forceinline__ void tile_of_block(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    // Blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous
    // range of tiles (when the count divides evenly).
    int lin = bid;
    if ((total & 7) == 0) {
        const int per = total >> 3;
        lin = (bid & 7) * per + (bid >> 3);
    }
    constexpr int GROUP_M = 8;
    const int group = lin / (GROUP_M * tiles_n);
    const int first_m = group * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int in_group = lin - group * GROUP_M * tiles_n;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void kv_proj_kernel(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ w, int M, int K, int O,
                                                      uint16_t* __restrict__ out) {
    using S = GemmShape<BM, BN>;
    extern __shared__ __align__(16) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (O + BN - 1) / BN;
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // global -> register staging: chunk c of a K-slice is row c/8, 16-byte column c%8
    const u32x4* ga[S::A_CHUNKS];
    const u32x4* gb[S::B_CHUNKS];
#pragma unroll
    for (int i = 0; i < S::A_CHUNKS; ++i) {
        const int c = tid + 256 * i;
        const int row = min(m0 + (c >> 3), M - 1);  // rows past M read row M-1 (never stored)
        ga[i] = (const u32x4*)(x + (int64_t)row * K) + (c & 7);
    }
#pragma unroll
    for (int i = 0; i < S::B_CHUNKS; ++i) {
        const int c = tid + 256 * i;
        const int row = min(n0 + (c >> 3), O - 1);
        gb[i] = (const u32x4*)(w + (int64_t)row * K) + (c & 7);
    }
    u32x4 ra[S::A_CHUNKS], rb[S::B_CHUNKS];

    auto load_slice = [&](int kt) {
#pragma unroll
        for (int i = 0; i < S::A_CHUNKS; ++i) ra[i] = ga[i][kt * (kBK / 8)];
#pragma unroll
        for (int i = 0; i < S::B_CHUNKS; ++i) rb[i] = gb[i][kt * (kBK / 8)];
    };
    auto store_slice = [&](int buf) {
        uint16_t* As = lds + buf * S::LDS_TILE;
        uint16_t* Bs = As + BM * kLdsRow;
#pragma unroll
        for (int i = 0; i < S::A_CHUNKS; ++i) {
            const int c = tid + 256 * i;
            *(u32x4*)(As + (c >> 3) * kLdsRow + (c & 7) * 8) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < S::B_CHUNKS; ++i) {
            const int c = tid + 256 * i;
            *(u32x4*)(Bs + (c >> 3) * kLdsRow + (c & 7) * 8) = rb[i];
        }
    };

    f32x16 acc[S::TI][S::TJ];
#pragma unroll
    for (int i = 0; i < S::TI; ++i)
#pragma unroll
        for (int j = 0; j < S::TJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nk = K / kBK;
    load_slice(0);
    store_slice(0);
    __syncthreads();

    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_slice(kt + 1);
        const uint16_t* As = lds + cur * S::LDS_TILE;
        const uint16_t* Bs = As + BM * kLdsRow;
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            bf16x8 af[S::TI], bfr[S::TJ];
#pragma unroll
            for (int i = 0; i < S::TI; ++i)
                af[i] = *(const bf16x8*)(As + (wm * (BM / 2) + i * 32 + frag_row) * kLdsRow + kk + frag_k);
#pragma unroll
            for (int j = 0; j < S::TJ; ++j)
                bfr[j] = *(const bf16x8*)(Bs + (wn * (BN / 2) + j * 32 + frag_row) * kLdsRow + kk + frag_k);
#pragma unroll
            for (int i = 0; i < S::TI; ++i)
#pragma unroll
                for (int j = 0; j < S::TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_slice(cur ^ 1);
        __syncthreads();
    }

    // epilogue: fp32 -> bf16 into LDS [BM][BN+8], then coalesced 16-byte stores
    uint16_t* Cs = lds;
    const int col_in = lane & 31;
    const int row_grp = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < S::TI; ++i)
#pragma unroll
        for (int j = 0; j < S::TJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                // element e of a 32x32 tile: row 8*(e/4) + 4*(lane/32) + e%4, column lane%32
                const int r0 = wm * (BM / 2) + i * 32 + 8 * (e >> 2) + row_grp + (e & 3);
                const int c = wn * (BN / 2) + j * 32 + col_in;
                const uint32_t pk = pack_bf16x2(acc[i][j][e], acc[i][j][e + 1]);
                Cs[r0 * S::OUT_ROW + c] = (uint16_t)(pk & 0xFFFFu);
                Cs[(r0 + 1) * S::OUT_ROW + c] = (uint16_t)(pk >> 16);
            }
    __syncthreads();
    constexpr int OUT_CHUNKS = BM * BN / 8 / 256;
#pragma unroll
    for (int i = 0; i < OUT_CHUNKS; ++i) {
        const int c = tid + 256 * i;
        const int row = c / (BN / 8);
        const int col = (c - row * (BN / 8)) * 8;
        const int gr = m0 + row, gc = n0 + col;
        if (gr < M && gc < O) *(u32x4*)(out + (int64_t)gr * O + gc) = *(const u32x4*)(Cs + row * S::OUT_ROW + col);
    }
}

// ---------------------------------------------------------------------------
// Large-problem kernel: 256 x 256 block tile, 4 waves (one per SIMD), each a
// 128 x 128 block held in 16 accumulator tiles of 32 x 32 (256 registers
// per lane, in the accumulation half of the register file).  K-slices of 64
// in two LDS stages of 64 KiB.
//
// Why this shape: a wave's LDS traffic per MFMA falls as its block grows,
// and 128 x 128 is the largest block whose accumulators fit one wave; the
// fragment reads of the next 16-deep K-step are spread between the current
// step's 16 MFMAs, so with one wave per SIMD the matrix core stays fed
// without a second wave to cover for it.
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
constexpr int kBigTile = 256;
constexpr int kBigThreads = 256;
constexpr int kBBK = 64;
constexpr int kNStage = 2;
constexpr int kBigOpBytes = kBigTile * kBBK * 2;  // one operand's slice: 32 KiB
constexpr int kBigStageBytes = 2 * kBigOpBytes;    // x + W slices: 64 KiB
constexpr int kBigOutRow = kBigTile + 8;           // epilogue row (elements)
constexpr int kBigLdsBytes = (kNStage * kBigStageBytes > kBigTile * kBigOutRow * 2) ? kNStage * kBigStageBytes
                                                                                    : kBigTile * kBigOutRow * 2;
constexpr int kBigMaxK = 1 << 20;  // keeps 256 rows of K bf16 within a 32-bit buffer offset
constexpr int kCopySplit = 4;      // copy instructions (of 8 per operand) issued in a slice's last K-step

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait for this wave's copies and LDS reads, then join the workgroup barrier.
// The "memory" clobber keeps the compiler from moving LDS or global accesses
// across it.
#define PLE_WAIT_VM_BARRIER0() asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory")

struct BigFrag {
    u32x4 a[4], b[4];  // x fragments of the 4 token blocks, W fragments of the 4 feature blocks
};
#define PLE_FRAG_REGS(f) \
    "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3])

__global__ __launch_bounds__(kBigThreads, 1) void kv_proj_big_kernel(const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ w, int M, int K,
                                                                     int O, uint16_t* __restrict__ out) {
    extern __shared__ __align__(16) char lds_raw[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves: 128 tokens x 128 features each

    const int tiles_m = (M + kBigTile - 1) / kBigTile;
    const int tiles_n = (O + kBigTile - 1) / kBigTile;
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kBigTile, n0 = tn * kBigTile;

    // Copy instruction i (0..7) of wave `wave` fills rows g*8 .. g*8+7 of an
    // operand slice, g = i*4 + wave; lane L lands at position g*64 + L: row
    // g*8 + L/8, chunk kc = (L & 7) ^ ((row >> 1) & 7).  Rows past the end of
    // x or W read the last row (their outputs are never stored).
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + (int64_t)m0 * K), (short)0, min(M - m0, kBigTile) * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w + (int64_t)n0 * K), (short)0, min(O - n0, kBigTile) * K * 2, 0x00020000);
    uint32_t aoff[8], boff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (i * 4 + wave) * 8 + (lane >> 3);
        const int kc = (lane & 7) ^ ((row >> 1) & 7);
        aoff[i] = (uint32_t)((min(m0 + row, M - 1) - m0) * K * 2 + kc * 16);
        boff[i] = (uint32_t)((min(n0 + row, O - 1) - n0) * K * 2 + kc * 16);
    }
    const int nk = K / kBBK;
    // copy instruction i of slice kt into stage kt % 2; slices past the end
    // (the loop below is uniform) re-read the last slice into a stage that no
    // later read uses
    auto copy_one = [&](int kt, int i) {
        char* base = lds_raw + (kt % kNStage) * kBigStageBytes;
        const int g = i * 4 + wave;
        const int ko = min(kt, nk - 1) * kBBK * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(base + g * 1024), 16, aoff[i], ko, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(base + kBigOpBytes + g * 1024), 16, boff[i], ko, 0, 0);
    };

    f32x16 acc[4][4];  // [W block j][x block i]
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
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
        a_addr[kk] = lds_base + (wm * 128 + frow) * 128 + col;
        b_addr[kk] = lds_base + kBigOpBytes + (wn * 128 + frow) * 128 + col;
    }
    // fragment read q (0..7) of K-step kk of slice kt: x blocks 0..3, then W blocks 0..3
    auto read_one = [&](int q, int kt, int kk, BigFrag& f) {
        const uint32_t so = (uint32_t)(kt & 1) * kBigStageBytes;
        const uint32_t pa = a_addr[kk] + so, pb = b_addr[kk] + so;
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
    };
    // One K-step: 16 MFMAs on `cur`.  After MFMA t < 8 comes fragment read t
    // of (rkt, rkk) into `nxt`, and copy instructions [c0, c1) of slice ckt are
    // spread over the 16.  The order is pinned.
    auto kstep = [&](const BigFrag& cur, BigFrag& nxt, int rkt, int rkk, int ckt, int c0, int c1) {
        const int nc = c1 - c0;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int j = t >> 2, i = t & 3;
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur.b[j]),
                                                                __builtin_bit_cast(bf16x8, cur.a[i]), acc[j][i], 0, 0,
                                                                0);
            if (rkk >= 0 && t < 8) read_one(t, rkt, rkk, nxt);
            if (nc > 0 && (t * nc) % 16 < nc) copy_one(ckt, c0 + (t * nc) / 16);
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
    auto slice = [&](int kt, BigFrag& f0, BigFrag& f1) {
        asm volatile("s_waitcnt lgkmcnt(0)" : PLE_FRAG_REGS(f0));
        kstep(f0, f1, kt, 1, kt + 1, kCopySplit, 8);
        asm volatile("s_waitcnt lgkmcnt(0)" : PLE_FRAG_REGS(f1));
        kstep(f1, f0, kt, 2, 0, 0, 0);
        asm volatile("s_waitcnt lgkmcnt(0)" : PLE_FRAG_REGS(f0));
        kstep(f0, f1, kt, 3, 0, 0, 0);
        // every read of this stage is complete (all waves) and slice kt+1 has landed
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : PLE_FRAG_REGS(f1) : : "memory");
        __builtin_amdgcn_sched_barrier(0);
        kstep(f1, f0, kt + 1, 0, kt + 2, 0, kCopySplit);
    };

    // slice 0 whole, then the first part of slice 1
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_one(0, i);
    PLE_WAIT_VM_BARRIER0();
#pragma unroll
    for (int i = 0; i < kCopySplit; ++i) copy_one(1, i);
    BigFrag f0, f1;
#pragma unroll
    for (int q = 0; q < 8; ++q) read_one(q, 0, 0, f0);
    for (int kt = 0; kt < nk; ++kt) slice(kt, f0, f1);
    // the fragment reads above are opaque to the compiler's own waits
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();  // every wave is done with the stages before the epilogue reuses LDS

    // epilogue: acc[j][i][e] is feature n0 + wn*128 + j*32 + 8*(e/4) + 4*(lane/32) + e%4
    // of token m0 + wm*128 + i*32 + lane%32
    uint16_t* Cs = (uint16_t*)lds_raw;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int m = wm * 128 + i * 32 + frow;
                const int o = wn * 128 + j * 32 + 8 * g + 4 * fk;
                const uint32_t lo = pack_bf16x2(acc[j][i][4 * g], acc[j][i][4 * g + 1]);
                const uint32_t hi = pack_bf16x2(acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]);
                *(uint2*)(Cs + m * kBigOutRow + o) = make_uint2(lo, hi);
            }
    __syncthreads();
#pragma unroll 4
    for (int c = tid; c < kBigTile * kBigTile / 8; c += kBigThreads) {
        const int row = c >> 5;  // 32 chunks of 8 features per row
        const int col = (c & 31) * 8;
        const int gr = m0 + row, gc = n0 + col;
        if (gr < M && gc < O) *(u32x4*)(out + (int64_t)gr * O + gc) = *(const u32x4*)(Cs + row * kBigOutRow + col);
    }
}
#undef PLE_FRAG_REGS

static hipError_t launch_kv_proj_big(const uint16_t* x, const uint16_t* w, int64_t M, int K, int O, uint16_t* kv,
                                     hipStream_t s) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)kv_proj_big_kernel,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kBigLdsBytes);
    if (attr != hipSuccess) return attr;
    const int tiles = (int)((M + kBigTile - 1) / kBigTile) * ((O + kBigTile - 1) / kBigTile);
    hipLaunchKernelGGL(kv_proj_big_kernel, dim3(tiles), dim3(kBigThreads), kBigLdsBytes, s, x, w, (int)M, K, O, kv);
    return hipGetLastError();
}

template <int BM, int BN>
static hipError_t launch_kv_proj_t(const uint16_t* x, const uint16_t* w, int64_t M, int K, int O, uint16_t* kv,
                                   hipStream_t s) {
    using S = GemmShape<BM, BN>;
    static const hipError_t attr = hipFuncSetAttribute((const void*)kv_proj_kernel<BM, BN>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const int tiles = (int)((M + BM - 1) / BM) * ((O + BN - 1) / BN);
    hipLaunchKernelGGL((kv_proj_kernel<BM, BN>), dim3(tiles), dim3(256), S::LDS_BYTES, s, x, w, (int)M, K, O, kv);
    return hipGetLastError();
}

hipError_t launch_kv_proj(const uint16_t* x, const uint16_t* w, int64_t M, int K, int O, uint16_t* kv,
                          hipStream_t s) {
    // 256 x 256 tiles when they alone fill the chip; 128 x 128 otherwise
    const int64_t big_tiles = ((M + kBigTile - 1) / kBigTile) * ((O + kBigTile - 1) / kBigTile);
    if (big_tiles >= 256 && K <= kBigMaxK) return launch_kv_proj_big(x, w, M, K, O, kv, s);
    return launch_kv_proj_t<128, 128>(x, w, M, K, O, kv, s);
}

}  // namespace ple
