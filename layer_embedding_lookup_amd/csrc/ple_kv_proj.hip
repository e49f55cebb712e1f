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
// Large-problem kernel: 256 x 256 block tile, 8 waves (two per SIMD) of
// 128 x 64, K-slices of 32 in a ring of 4 LDS stages.
//
// Operands go global -> LDS with the gfx950 direct-to-LDS 16-byte loads
// (global_load_lds_dwordx4): no register staging.  The copies run three
// slices ahead of the MFMAs (about three slices of compute to arrive from L2,
// the last-level cache or HBM).  Each thread waits only for its own copies of
// the slice it is about to use (vmcnt lets the later slices stay in flight),
// then one barrier makes everyone's copies visible and frees the stage the
// next copy overwrites.  With two waves per SIMD, one wave's MFMAs cover the
// other's LDS fragment reads.
//
// LDS layout of a stage: rows of 32 bf16 = 4 chunks of 16 bytes, chunk
// (row, kc) at position row*4 + (kc ^ ((row >> 2) & 3)).  An MFMA fragment
// read takes one k-chunk of 32 consecutive rows; the LDS serves 16 lanes
// (256 bytes, 64 banks) per cycle, and any 16 consecutive rows land on 16
// distinct 16-byte bank groups.  One wave copy instruction fills 1 KiB =
// 16 rows x 4 chunks, each lane fetching the global chunk that belongs at its
// position.  The MFMA operands are swapped (W fragment first) so each lane's
// accumulators are 4 consecutive output features of one token, which the
// epilogue writes to LDS as 8-byte pairs before coalesced 16-byte stores.
// ---------------------------------------------------------------------------
constexpr int kBigTile = 256;
constexpr int kBigThreads = 512;
constexpr int kBBK = 32;
constexpr int kNStage = 4;
constexpr int kBigStageBytes = 2 * kBigTile * kBBK * 2;  // x + W slices: 32 KiB
constexpr int kBigOutRow = kBigTile + 8;                 // epilogue row (elements)
constexpr int kBigLdsBytes = (kNStage * kBigStageBytes > kBigTile * kBigOutRow * 2) ? kNStage * kBigStageBytes
                                                                                    : kBigTile * kBigOutRow * 2;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz4(int row, int kc) { return row * 4 + (kc ^ ((row >> 2) & 3)); }

// Wait until at most n of this wave's vector-memory operations (the later
// slices' copies) are outstanding and all its LDS reads are complete, then
// join the workgroup barrier.  __syncthreads() would wait for every copy in
// flight (its release fence counts direct-to-LDS copies as pending LDS
// writes), which would serialise the copy pipeline.  The "memory" clobber
// keeps the compiler from moving LDS or global accesses across the barrier.
#define PLE_STR2(x) #x
#define PLE_STR(x) PLE_STR2(x)
#define PLE_WAIT_VM_BARRIER(n) asm volatile("s_waitcnt vmcnt(" PLE_STR(n) ") lgkmcnt(0)\n\ts_barrier" ::: "memory")

__global__ __launch_bounds__(kBigThreads, 1) void kv_proj_big_kernel(const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ w, int M, int K,
                                                                     int O, uint16_t* __restrict__ out) {
    extern __shared__ __align__(16) char lds_raw[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves: 128 tokens x 64 features each

    const int tiles_m = (M + kBigTile - 1) / kBigTile;
    const int tiles_n = (O + kBigTile - 1) / kBigTile;
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kBigTile, n0 = tn * kBigTile;

    // copy instruction i (0..1) of wave `wave` fills rows g*16 .. g*16+15 of
    // each operand, g = i*8 + wave; lane L lands at position g*64 + L:
    // row = g*16 + L/4, chunk kc = (L & 3) ^ ((L >> 4) & 3)
    const int lkc = (lane & 3) ^ ((lane >> 4) & 3);
    const uint16_t* asrc[2];
    const uint16_t* bsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (i * 8 + wave) * 16 + (lane >> 2);
        asrc[i] = x + (int64_t)min(m0 + row, M - 1) * K + lkc * 8;
        bsrc[i] = w + (int64_t)min(n0 + row, O - 1) * K + lkc * 8;
    }
    auto issue_slice = [&](int kt) {
        char* base = lds_raw + (kt % kNStage) * kBigStageBytes;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int g = i * 8 + wave;
            __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + kt * kBBK), (lds_ptr_t)(base + g * 1024), 16, 0,
                                             0);
            __builtin_amdgcn_global_load_lds((const void*)(bsrc[i] + kt * kBBK),
                                             (lds_ptr_t)(base + kBigTile * kBBK * 2 + g * 1024), 16, 0, 0);
        }
    };

    f32x16 acc[2][4];  // [W sub-tile j][x sub-tile i]
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;

    // per thread and slice: 2 x + 2 W copy instructions (the waits below count 4)
    const int nk = K / kBBK;
#pragma unroll
    for (int p = 0; p < kNStage - 1; ++p)
        if (p < nk) issue_slice(p);

    const int frow = lane & 31;
    const int fk = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        // slices <= kt complete: the copies of up to two later slices may remain in flight;
        // after the barrier stage (kt-1) % 4, read in the previous iteration, is free
        const int ahead = min(nk - 1 - kt, kNStage - 2);
        if (ahead >= 2)
            PLE_WAIT_VM_BARRIER(8);
        else if (ahead == 1)
            PLE_WAIT_VM_BARRIER(4);
        else
            PLE_WAIT_VM_BARRIER(0);
        if (kt + kNStage - 1 < nk) issue_slice(kt + kNStage - 1);

        const u32x4* As = (const u32x4*)(lds_raw + (kt % kNStage) * kBigStageBytes);
        const u32x4* Bs = As + kBigTile * 4;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int kc = kk * 2 + fk;
            bf16x8 af[4], bfr[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = __builtin_bit_cast(bf16x8, As[swz4(wm * 128 + i * 32 + frow, kc)]);
#pragma unroll
            for (int j = 0; j < 2; ++j) bfr[j] = __builtin_bit_cast(bf16x8, Bs[swz4(wn * 64 + j * 32 + frow, kc)]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[j][i], 0, 0, 0);
        }
    }
    __syncthreads();  // all reads of the last stage are done before the epilogue reuses LDS

    // epilogue: acc[j][i][e] is feature n0 + wn*64 + j*32 + 8*(e/4) + 4*(lane/32) + e%4
    // of token m0 + wm*128 + i*32 + lane%32
    uint16_t* Cs = (uint16_t*)lds_raw;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int m = wm * 128 + i * 32 + frow;
                const int o = wn * 64 + j * 32 + 8 * g + 4 * fk;
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
    if (big_tiles >= 256) return launch_kv_proj_big(x, w, M, K, O, kv, s);
    return launch_kv_proj_t<128, 128>(x, w, M, K, O, kv, s);
}

}  // namespace ple
