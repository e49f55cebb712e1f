// N-gram IDs, row gather and the fused ids+gather lookup for gfx950.
//
// Method: "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels",
// 实现拆解 item 2 and 关键源码片段 (per-token n-gram IDs over ragged requests
// with EOS replacement, the carried ngram_context and int64 wraparound); the
// row lookup of "PR #54371 [Qwen4Exp] Support UVA PLE-offload and Engram
// tensor parallelism", 关键源码片段 (embedding lookup, also from pinned host
// memory); FP8 e4m3fn tables with a per-row or a global scale, and NVFP4
// tables, from "Support PLE-Offload for Qwen3.8-Flash-Next - #53899".
//
// Design for CDNA4: each wave owns a few consecutive tokens (at most 64
// (token, head) rows).  One lane per row computes the ID in registers: the
// per-head hash constants come from the kernel arguments through a per-wave
// LDS stage filled by one load at entry, the wave finds request boundaries
// with one cooperative load of query_start_loc and ballots, the window tokens
// are loaded in the same round trip, and the modulo is a Barrett reduction
// instead of a 64-bit divide.  The IDs never leave registers: the wave then
// streams its rows with 16-byte loads (one wave instruction moves a whole
// 1 KiB bf16 row), 16 loads in flight per lane, and writes coalesced 16-byte
// chunks into the wave's contiguous [tokens][H*D] slab, either with per-lane
// addresses (row IDs by cross-lane reads) or, for rows of 64 x 2^k chunks,
// from scalar row bases with buffer stores.  Waves never wait for each other.
#include "ple_launch.h"

// Tuning knobs (compile-time): 16-byte output chunks per lane per pass by
// table format, non-temporal row stores by table format (measured: the
// expanding fp8 and NVFP4 stores gain from them, plain bf16 copies do not),
// and which stream bf16 rows take (0: per-lane, 1: scalar-address).
#ifndef PLE_LOOKUP_LOADS
#define PLE_LOOKUP_LOADS 16
#endif
#ifndef PLE_LOOKUP_LOADS_FP8
#define PLE_LOOKUP_LOADS_FP8 16
#endif
#ifndef PLE_LOOKUP_LOADS_FP4
#define PLE_LOOKUP_LOADS_FP4 16
#endif
#ifndef PLE_LOOKUP_NT_STORE_BF16
#define PLE_LOOKUP_NT_STORE_BF16 0
#endif
#ifndef PLE_LOOKUP_NT_LOAD_BF16
#define PLE_LOOKUP_NT_LOAD_BF16 1
#endif
#ifndef PLE_LOOKUP_NT_STORE_QUANT
#define PLE_LOOKUP_NT_STORE_QUANT 1
#endif
#ifndef PLE_LOOKUP_BF16_SCALAR_ROWS
#define PLE_LOOKUP_BF16_SCALAR_ROWS 0
#endif
#ifndef PLE_LOOKUP_QUANT_SCALAR_ROWS
#define PLE_LOOKUP_QUANT_SCALAR_ROWS 1
#endif
#ifndef PLE_LOOKUP_BLOCK
#define PLE_LOOKUP_BLOCK 256  // threads per block; waves are independent
#endif

namespace ple {

// Carried context: out[r][i] = the (C-i)-th most recent raw token of ctx[r] ++ tok[a:b].
__global__ __launch_bounds__(256) void context_out_kernel(const int32_t* __restrict__ tok,
                                                          const int32_t* __restrict__ qsl, int64_t T, int R,
                                                          int C, int32_t eos, const int32_t* __restrict__ ctx,
                                                          int32_t* __restrict__ ctx_out) {
    const int64_t n = (int64_t)R * C;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < n;
         p += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(p / C);
        const int i = (int)(p - (int64_t)r * C);
        int64_t a, b;
        carried_window(qsl, T, r, nullptr, a, b);
        ctx_out[p] = carried_token(tok, ctx, C, eos, r, i, a, b);
    }
}

// fp8 e4m3fn x8 (8 bytes) -> 8 bf16 (one 16-byte chunk), each value
// float(code) * scale in fp32, then round to nearest even.
__device__ __forceinline__ u32x4 dequant8_fp8(uint32_t q0, uint32_t q1, float scale) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q0, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q0, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)q1, false);
    const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)q1, true);
    return u32x4{pack_bf16x2_canon(a.x * scale, a.y * scale), pack_bf16x2_canon(b.x * scale, b.y * scale),
                 pack_bf16x2_canon(c.x * scale, c.y * scale), pack_bf16x2_canon(d.x * scale, d.y * scale)};
}

// NVFP4 x8 (4 bytes of e2m1 codes, element 2i in the low nibble of byte i;
// all 8 in one 16-element block) -> 8 bf16.  Element value:
// (e2m1 * e4m3fn(block scale)) * table scale; the first product is exact in
// fp32 (at most 2 x 4 significant bits), the second is one fp32 multiply.
// v_cvt_scalef32_pk_f32_fp4 with scale 1.0 decodes a byte's two codes
// exactly (low nibble first).
__device__ __forceinline__ u32x4 dequant8_fp4(uint32_t q, uint32_t bcode, float tscale) {
    const f32x2 sv = __builtin_amdgcn_cvt_pk_f32_fp8((int)bcode, false);
    const float s = sv.x;
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
    return u32x4{pack_bf16x2_canon((v0.x * s) * tscale, (v0.y * s) * tscale),
                 pack_bf16x2_canon((v1.x * s) * tscale, (v1.y * s) * tscale),
                 pack_bf16x2_canon((v2.x * s) * tscale, (v2.y * s) * tscale),
                 pack_bf16x2_canon((v3.x * s) * tscale, (v3.y * s) * tscale)};
}

// Everything a lane needs for the ID of its (token t, head h) pair apart from
// the request boundaries: the raw tokens w[j] = tok[max(t-j, 0)] for shifts
// j <= C (a value is used only when t-j lies in the token's request) and
// head h's constants.
struct IdInputs {
    int32_t w[PLE_MAX_CONTEXT + 1];
    uint64_t m[PLE_MAX_CONTEXT + 1];
    uint64_t barrett;
    uint32_t vocab, wrap_mod, offset, order;
};

// The head records reach each lane through LDS.  A wave loads the records of
// heads 0..15 (1 KiB, one 16-byte chunk per lane) straight from the kernel
// argument block at entry: the load needs only the block's address, so it is
// in flight together with the kernel's first scalar argument loads, and the
// records cost no round trip of their own.  Heads 16..31 (more than 16 heads
// in a call) follow once the head count is known.
struct HeadStage {
    u32x4 lo;  // chunk `lane` of head records 0..15
};

__device__ __forceinline__ void head_stage_load(const HashParams& hp, int lane, HeadStage& st) {
    st.lo = ((const u32x4*)&hp.head[0])[lane];
}

// The wave's stage holds 128 chunks (32 records); id_consts_read reads them.
__device__ __forceinline__ void head_stage_store(const HashParams& hp, const HeadStage& st, int H, int lane,
                                                 u32x4* __restrict__ lds) {
    lds[lane] = st.lo;
    if (H > 16) lds[kWave + lane] = ((const u32x4*)&hp.head[0])[kWave + lane];  // wave-uniform
}

// The token window comes from memory (t clamped into the batch, for waves
// past its end), the head record from the wave's LDS stage; the first only
// issues loads, so that they share one round trip with the query_start_loc
// load and the stage's own load.
__device__ __forceinline__ void id_tokens_load(const HashParams& hp, const int32_t* __restrict__ tok, int64_t T,
                                               int64_t t, IdInputs& in) {
    const int C = hp.context_len;
    const int64_t tc = t < T ? t : T - 1;
#pragma unroll
    for (int j = 0; j <= PLE_MAX_CONTEXT; ++j) {
        const int64_t p = tc - (j <= C ? j : C);
        in.w[j] = tok[p >= 0 ? p : 0];
    }
}

__device__ __forceinline__ void id_consts_read(const HashParams& hp, const u32x4* __restrict__ lds, int h,
                                               IdInputs& in) {
    const int C = hp.context_len;
    __builtin_amdgcn_wave_barrier();  // the record reads follow the wave's own LDS writes
    const u32x4 c0 = lds[4 * h], c1 = lds[4 * h + 1], c2 = lds[4 * h + 2], c3 = lds[4 * h + 3];
    in.m[0] = (uint64_t)c0.y << 32 | c0.x;
    in.m[1] = (uint64_t)c0.w << 32 | c0.z;
    in.m[2] = (uint64_t)c1.y << 32 | c1.x;
    in.m[3] = (uint64_t)c1.w << 32 | c1.z;
#pragma unroll
    for (int j = 4; j <= PLE_MAX_CONTEXT; ++j) in.m[j] = C >= 4 ? hp.mult_hi[h][j - 4] : 0u;  // wave-uniform
    in.barrett = (uint64_t)c2.y << 32 | c2.x;
    in.vocab = c2.z;
    in.wrap_mod = c2.w;
    in.offset = c3.x;
    in.order = c3.y;
}

// ID of the lane's (token t, head h) pair in request r starting at a:
// shifts before the request start read the carried context (oldest first)
// or EOS; once a shift reads EOS every older shift reads EOS (the current
// token never masks); the wrapped 64-bit sum of token x multiplier is
// reduced by a signed floor modulo and offset into the head's rows.
__device__ __forceinline__ int32_t window_id(const IdInputs& in, int C, int32_t eos,
                                             const int32_t* __restrict__ ctx, int r, int64_t a, int64_t t) {
    // raw tokens of shifts 1..C first (the context reads all in flight), then the sum
    int32_t raw[PLE_MAX_CONTEXT + 1];
#pragma unroll
    for (int j = 1; j <= PLE_MAX_CONTEXT; ++j) {
        raw[j] = in.w[j];
        if (j <= C && j < (int)in.order) {
            const int64_t p = t - j;
            if (p < a) raw[j] = ctx != nullptr ? ctx[(int64_t)r * C + (C - (a - p))] : eos;
        }
    }
    uint64_t acc = (uint64_t)(int64_t)in.w[0] * in.m[0];
    bool crossed = false;
#pragma unroll
    for (int j = 1; j <= PLE_MAX_CONTEXT; ++j) {
        if (j <= C && j < (int)in.order) {
            crossed |= (raw[j] == eos);
            const int64_t sj = crossed ? (int64_t)eos : (int64_t)raw[j];
            acc += (uint64_t)sj * in.m[j];
        }
    }
    return (int32_t)(in.offset + floor_mod_wrapped(acc, in.vocab, in.barrett, in.wrap_mod));
}

// pointer into global memory (address space 1) from a 64-bit address, so that
// loads through it are global, not flat, instructions
template <typename T>
using gptr = const T __attribute__((address_space(1)))*;

// 64-bit value of lane `l` for every lane
__device__ __forceinline__ uint64_t shfl64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, l, kWave);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), l, kWave);
    return (uint64_t)hi << 32 | lo;
}

// 64-bit value of lane `l` (wave-uniform) as a scalar
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return (uint64_t)hi << 32 | lo;
}

// What both row streams need: every lane produces one 16-byte output chunk
// (8 bf16 elements) per step, so stores are always lane-contiguous; its input
// is the same 8 elements of the stored row: 16 bytes (bf16), 8 (fp8 codes) or
// 4 (NVFP4 codes, plus the block's scale code).
struct StreamArgs {
    const char* table;
    uint16_t* out;  // the wave's [rows][dim] output slab
    int cpr;        // 16-byte output chunks per row
    int shift;      // log2(cpr), or -1
    int nrows;
    int total;      // nrows * cpr
};

__device__ __forceinline__ StreamArgs stream_args(const LookupArgs& g, int64_t t0, int nrows) {
    StreamArgs a;
    a.table = (const char*)g.table;
    a.out = g.rows + t0 * g.num_heads * (int64_t)g.dim;
    a.cpr = g.dim >> 3;
    a.shift = g.cpr_log2;
    a.nrows = nrows;
    a.total = nrows * a.cpr;
    return a;
}

template <int DTYPE>
constexpr int in_bytes() {  // input bytes per output chunk
    return DTYPE == kFmtBF16 ? 16 : (DTYPE == kFmtFP8 ? 8 : 4);
}

__device__ __forceinline__ void store16(u32x4* p, u32x4 v, bool nt) {
    if (nt)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Per-lane stream (any row length): chunk idx = base + u*64 + lane of the
// wave's slab belongs to row idx / cpr, whose ID the lane reads from the
// row's owning lane; up to UNROLL loads per lane in flight, then the stores.
// bf16 tables take this stream by default: for plain row copies it measured
// faster than the scalar-address stream below.
template <int DTYPE, int MODE, int UNROLL>
__device__ __forceinline__ void stream_rows_lane(const LookupArgs& g, const StreamArgs& a, int id, int orow,
                                                 float tscale, int lane) {
    constexpr int IB = in_bytes<DTYPE>();
    const int64_t row_bytes = (int64_t)a.cpr * IB;
    float scale = 0.f;
    if (DTYPE == kFmtFP8) scale = g.scales[(int64_t)id * g.scale_stride];
    u32x4* __restrict__ out = (u32x4*)a.out;
    for (int base = 0; base < a.total; base += kWave * UNROLL) {
        u32x4 v[UNROLL];
        float sc[UNROLL];
        uint32_t bsc[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = base + u * kWave + lane;
            int row = a.shift >= 0 ? (idx >> a.shift) : (idx / a.cpr);
            row = row < a.nrows ? row : a.nrows - 1;
            const int rid = __shfl(id, row, kWave);
            if (DTYPE == kFmtFP8) sc[u] = __shfl(scale, row, kWave);
            if (idx < a.total) {
                const int ch = idx - row * a.cpr;
                const char* src = a.table + (int64_t)rid * row_bytes + (int64_t)ch * IB;
                if (DTYPE == kFmtBF16) {
                    v[u] = PLE_LOOKUP_NT_LOAD_BF16 ? __builtin_nontemporal_load((const u32x4*)src) : *(const u32x4*)src;
                } else if (DTYPE == kFmtFP8) {
                    const u32x2 q = __builtin_nontemporal_load((const u32x2*)src);
                    v[u] = u32x4{q.x, q.y, 0u, 0u};
                } else {
                    v[u] = u32x4{__builtin_nontemporal_load((const uint32_t*)src), 0u, 0u, 0u};
                    bsc[u] = g.block_scales[(int64_t)rid * (g.dim >> 4) + (ch >> 1)];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = base + u * kWave + lane;
            if (idx < a.total) {
                // list mode: each row goes to its own output row (list entry)
                u32x4* dst = out + idx;
                if (MODE == kModeList) {
                    int row = a.shift >= 0 ? (idx >> a.shift) : (idx / a.cpr);
                    row = row < a.nrows ? row : a.nrows - 1;
                    dst = (u32x4*)g.rows + (int64_t)__shfl(orow, row, kWave) * a.cpr + (idx - row * a.cpr);
                }
                if (DTYPE == kFmtBF16)
                    store16(dst, v[u], PLE_LOOKUP_NT_STORE_BF16);
                else if (DTYPE == kFmtFP8)
                    store16(dst, dequant8_fp8(v[u].x, v[u].y, sc[u]), PLE_LOOKUP_NT_STORE_QUANT);
                else
                    store16(dst, dequant8_fp4(v[u].x, bsc[u], tscale), PLE_LOOKUP_NT_STORE_QUANT);
            }
        }
    }
}

// Scalar-address stream, for rows of 64 x 2^k output chunks: every pass of 64
// chunks then lies in one row.  Lane u first works out pass u's source
// address and store offset with a few vector operations for all passes at
// once (the row's base address fetched from the lane that owns the row); each
// load then takes them by lane reads into scalar registers, so the loads go
// out back to back from scalar bases.  The wave's output slab is a buffer
// resource: a store at an offset past its end is dropped by the hardware,
// which masks the ragged tail without a branch (a branch around each store
// lets the compiler sink the loads into it).
template <int DTYPE, int UNROLL>
__device__ __forceinline__ void stream_rows_scalar(const LookupArgs& g, const StreamArgs& a, int id, float tscale,
                                                   int lane) {
    constexpr int IB = in_bytes<DTYPE>();
    const int64_t row_bytes = (int64_t)a.cpr * IB;
    const __amdgpu_buffer_rsrc_t orsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.out, (short)0, a.total * 16, 0x00020000);
    // per lane (one row each): the row's address, its fp8 scale (loaded now,
    // used at the dequant) and its NVFP4 block-scale address
    const uint64_t my_row = (uint64_t)a.table + (uint64_t)(uint32_t)id * (uint64_t)row_bytes;
    float my_scale = 0.f;
    uint64_t my_bs = 0;
    if (DTYPE == kFmtFP8) my_scale = g.scales[(int64_t)id * g.scale_stride];
    if (DTYPE == kFmtNVFP4) my_bs = (uint64_t)g.block_scales + (uint64_t)(uint32_t)id * (uint64_t)(g.dim >> 4);
    const int lppr = a.shift - 6;  // log2(passes per row)
    const bool nt = DTYPE == kFmtBF16 ? PLE_LOOKUP_NT_STORE_BF16 : PLE_LOOKUP_NT_STORE_QUANT;
    for (int base = 0; base < a.total; base += kWave * UNROLL) {
        // pass P = base/64 + lane covers chunks [cp*64, cp*64 + 64) of row P >> lppr
        const int P = (base >> 6) + lane;
        const int prow = P >> lppr;
        const int pcp = P & ((1 << lppr) - 1);
        const int prowc = prow < a.nrows ? prow : a.nrows - 1;
        const uint64_t paddr = shfl64(my_row, prowc) + (uint64_t)(pcp * kWave * IB);
        const int psoff = prow < a.nrows ? (prow * a.cpr + pcp * kWave) * 16 : a.total * 16;
        uint64_t pbs = 0;
        if (DTYPE == kFmtNVFP4) pbs = shfl64(my_bs, prowc) + (uint64_t)(pcp * kWave / 2);
        u32x4 v[UNROLL];
        uint32_t bsc[UNROLL];
        int soff[UNROLL], rsel[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            soff[u] = __builtin_amdgcn_readlane(psoff, u);
            rsel[u] = DTYPE == kFmtFP8 ? __builtin_amdgcn_readlane(prowc, u) : 0;
            {  // every pass loads (the address is a valid row); stores past the slab are dropped
                const uint64_t rb = readlane64(paddr, u);
                if (DTYPE == kFmtBF16) {
                    v[u] = __builtin_nontemporal_load((gptr<u32x4>)rb + lane);
                } else if (DTYPE == kFmtFP8) {
                    const u32x2 q = __builtin_nontemporal_load((gptr<u32x2>)rb + lane);
                    v[u] = u32x4{q.x, q.y, 0u, 0u};
                } else {
                    v[u] = u32x4{__builtin_nontemporal_load((gptr<uint32_t>)rb + lane), 0u, 0u, 0u};
                    bsc[u] = ((gptr<uint8_t>)readlane64(pbs, u))[lane >> 1];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            u32x4 o;
            if (DTYPE == kFmtBF16) {
                o = v[u];
            } else if (DTYPE == kFmtFP8) {
                const float s = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_scale), rsel[u]));
                o = dequant8_fp8(v[u].x, v[u].y, s);
            } else {
                o = dequant8_fp4(v[u].x, bsc[u], tscale);
            }
            // the whole offset in the vector operand, soffset the constant 0:
            // with a register soffset the compiler takes a 128-bit buffer
            // store as free of the store-data hazard and may overwrite the
            // data registers with the very next VALU instruction, which
            // corrupted stored dwords now and then (dequantizing formats)
            __builtin_amdgcn_raw_buffer_store_b128(o, orsrc, lane * 16 + soff[u], 0, nt ? 2 : 0);
        }
    }
}

// One wave: `tokens_per_wave` consecutive tokens x H heads = at most 64 rows,
// one lane per (token, head) pair for the IDs.  No block-level barrier: each
// wave computes its IDs and streams its rows on its own.  MODE_HASH computes
// the IDs, MODE_IDS reads (and clamps) caller IDs.
template <int DTYPE, int MODE, int UNROLL, bool SCALAR_ROWS>
__global__ __launch_bounds__(PLE_LOOKUP_BLOCK) void lookup_kernel(HashParams hp, LookupArgs g) {
    __shared__ u32x4 head_lds[PLE_LOOKUP_BLOCK / kWave][2 * kWave];
    const int lane = threadIdx.x & (kWave - 1);
    HeadStage hst;
    if (MODE == kModeHash) head_stage_load(hp, lane, hst);
    // the wave index is uniform; saying so keeps everything derived from it
    // (token range, row count, output slab) in scalar registers
    const int64_t wave = (int64_t)blockIdx.x * (PLE_LOOKUP_BLOCK / kWave) +
                         __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int TW = g.tokens_per_wave;
    const int64_t t0 = wave * TW;
    const bool live = t0 < g.num_tokens;  // waves past the batch end leave after the IDs
    const int H = g.num_heads;
    const int nt = live ? (int)min((int64_t)TW, g.num_tokens - t0) : 0;
    const int nrows = nt * H;
    const bool active = lane < nrows;
    const int my_k = active ? lane / H : 0;
    const int h = active ? lane - my_k * H : 0;
    const int64_t t = t0 + my_k;

    int32_t id = 0;
    if (MODE == kModeHash) {
        // one round trip: window tokens, query_start_loc and the head records
        IdInputs in;
        id_tokens_load(hp, g.tok, g.num_tokens, t, in);
        QslProbe qp;
        qsl_probe_load(g.qsl, g.num_reqs, lane, qp);
        u32x4* lds = head_lds[threadIdx.x >> 6];
        head_stage_store(hp, hst, H, lane, lds);
        id_consts_read(hp, lds, h, in);
        int r;
        int64_t a;
        wave_find_request_probed(g.qsl, qp, g.num_reqs, t, t0, nt, my_k, lane, r, a);
        id = window_id(in, hp.context_len, hp.eos, g.ctx, r, a, t);
        if (active && g.ids_out != nullptr) g.ids_out[t0 * H + lane] = id;
    } else if (MODE == kModeIds) {
        id = active ? g.ids_in[t0 * H + lane] : 0;
        id = id < 0 ? 0 : (id >= g.num_rows ? (int32_t)(g.num_rows - 1) : id);
    }
    // list mode (one head: a "token" is a list entry): entries at or past the
    // device-side count are left alone
    int orow = 0;
    int nrows_l = nrows;
    if (MODE == kModeList) {
        int cnt = *g.list_count;
        cnt = cnt < 0 ? 0 : (cnt > g.num_tokens ? (int)g.num_tokens : cnt);
        if (g.count_out != nullptr && wave == 0 && lane == 0) *g.count_out = cnt;
        if (t0 >= cnt) return;  // whole wave (no barriers in this mode)
        nrows_l = (int)min((int64_t)nrows, cnt - t0);
        if (lane < nrows_l) {
            orow = g.list[t0 + lane];
            orow = orow < 0 ? 0 : (orow >= g.num_tokens ? (int)(g.num_tokens - 1) : orow);
            id = g.ids_in[orow];
            if (g.rep != nullptr) {
                id = id < 0 ? 0 : (id >= g.rep_len ? (int32_t)(g.rep_len - 1) : id);
                id = g.rep[id];
            }
            id = id < 0 ? 0 : (id >= g.num_rows ? (int32_t)(g.num_rows - 1) : id);
        }
    }
    if (!live) return;  // whole wave
    const float tscale = DTYPE == kFmtNVFP4 ? g.scales[0] : 0.f;

    const StreamArgs sa = stream_args(g, t0, nrows_l);
    if (SCALAR_ROWS)
        stream_rows_scalar<DTYPE, UNROLL>(g, sa, id, tscale, lane);
    else
        stream_rows_lane<DTYPE, MODE, UNROLL>(g, sa, id, orow, tscale, lane);
}

// IDs only: the lookup kernel's first phase.  Each wave takes 64/H
// consecutive tokens (one lane per (token, head)) and writes their IDs as one
// coalesced store.
__global__ __launch_bounds__(256) void ngram_ids_kernel(HashParams hp, const int32_t* __restrict__ tok,
                                                        const int32_t* __restrict__ qsl, int64_t T, int R,
                                                        const int32_t* __restrict__ ctx,
                                                        int32_t* __restrict__ ids, int id_blocks,
                                                        int32_t* __restrict__ clear, int64_t clear_n,
                                                        int32_t* __restrict__ zero, int zero_n) {
    __shared__ u32x4 head_lds[4][2 * kWave];
    if ((int)blockIdx.x >= id_blocks) {  // the clearing blocks (no barriers in this kernel)
        const int64_t nb = (int64_t)gridDim.x - id_blocks;
        for (int64_t i = ((int64_t)blockIdx.x - id_blocks) * blockDim.x + threadIdx.x; i < clear_n;
             i += nb * blockDim.x)
            clear[i] = -1;
        if (zero != nullptr && (int)blockIdx.x == id_blocks && (int)threadIdx.x < zero_n) zero[threadIdx.x] = 0;
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    HeadStage hst;
    head_stage_load(hp, lane, hst);
    u32x4* lds = head_lds[threadIdx.x >> 6];
    const int H = hp.num_heads;
    head_stage_store(hp, hst, H, lane, lds);
    const int TW = kWave / H;
    const int64_t nwaves = (T + TW - 1) / TW;
    for (int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); wave < nwaves;
         wave += (int64_t)id_blocks * 4) {
        const int64_t t0 = wave * TW;
        const int nt = (int)min((int64_t)TW, T - t0);
        const bool active = lane < nt * H;
        const int my_k = active ? lane / H : 0;
        const int h = active ? lane - my_k * H : 0;
        const int64_t t = t0 + my_k;
        IdInputs in;
        id_tokens_load(hp, tok, T, t, in);
        id_consts_read(hp, lds, h, in);
        QslProbe qp;
        qsl_probe_load(qsl, R, lane, qp);
        int r;
        int64_t a;
        wave_find_request_probed(qsl, qp, R, t, t0, nt, my_k, lane, r, a);
        const int32_t id = window_id(in, hp.context_len, hp.eos, ctx, r, a, t);
        if (active) ids[t0 * H + lane] = id;
    }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_ngram_ids(const HashParams& hp, const int32_t* tok, const int32_t* qsl, int64_t T, int R,
                            const int32_t* ctx, int32_t* ids, hipStream_t s, int32_t* clear, int64_t clear_n,
                            int32_t* zero, int zero_n) {
    const int TW = kWave / hp.num_heads;
    const int64_t waves = (T + TW - 1) / TW;
    int64_t blocks = (waves + 3) / 4;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    int64_t clear_blocks = 0;
    if (clear != nullptr || zero != nullptr) {
        clear_blocks = (clear_n + 255) / 256;
        clear_blocks = clear_blocks < 1 ? 1 : (clear_blocks > 1024 ? 1024 : clear_blocks);
    }
    hipLaunchKernelGGL(ngram_ids_kernel, dim3((unsigned)(blocks + clear_blocks)), dim3(256), 0, s, hp, tok, qsl, T, R,
                       ctx, ids, (int)blocks, clear, clear_n, zero, zero_n < 0 ? 0 : (zero_n > 64 ? 64 : zero_n));
    return hipGetLastError();
}

hipError_t launch_context_out(const int32_t* tok, const int32_t* qsl, int64_t T, int R, int C, int32_t eos,
                              const int32_t* ctx, int32_t* ctx_out, hipStream_t s) {
    const int64_t n = (int64_t)R * C;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(context_out_kernel, dim3((unsigned)blocks), dim3(256), 0, s, tok, qsl, T, R, C, eos, ctx,
                       ctx_out);
    return hipGetLastError();
}

static int lookup_loads(int dtype) {
    return dtype == PLE_DTYPE_BF16 ? PLE_LOOKUP_LOADS : (dtype == PLE_DTYPE_NVFP4 ? PLE_LOOKUP_LOADS_FP4 : PLE_LOOKUP_LOADS_FP8);
}

int lookup_tokens_per_wave(int H, int chunks_per_row, int dtype, int64_t num_tokens) {
    // about lookup_loads(dtype) output chunks per lane, at most 64 rows (one
    // lane per row for the IDs); chunks_per_row counts 16-byte output chunks
    const int chunks_per_token = H * chunks_per_row;
    int tw = (lookup_loads(dtype) * kWave) / chunks_per_token;
    if (tw > kWave / H) tw = kWave / H;
    // small batches (decode, speculative verify): fewer tokens per wave so
    // that the grid still gives every SIMD of the 256 CUs a wave
    const int64_t fill = (num_tokens + 1023) / 1024;
    if (tw > fill) tw = (int)fill;
    return tw < 1 ? 1 : tw;
}

template <int DTYPE, int MODE>
static hipError_t launch_lookup_t(const HashParams& hp, const LookupArgs& g, hipStream_t s) {
    constexpr int WPB = PLE_LOOKUP_BLOCK / kWave;  // waves per block
    constexpr int UNROLL = DTYPE == kFmtBF16 ? PLE_LOOKUP_LOADS
                                             : (DTYPE == kFmtNVFP4 ? PLE_LOOKUP_LOADS_FP4 : PLE_LOOKUP_LOADS_FP8);
    const int64_t waves = (g.num_tokens + g.tokens_per_wave - 1) / g.tokens_per_wave;
    const int64_t blocks = (waves + WPB - 1) / WPB;
    // the scalar-address stream needs rows of 64 x 2^k output chunks (list
    // mode writes each row to its own output row: the per-lane stream only)
    if constexpr (MODE != kModeList) {
        const bool scalar_rows =
            g.cpr_log2 >= 6 && (DTYPE == kFmtBF16 ? PLE_LOOKUP_BF16_SCALAR_ROWS : PLE_LOOKUP_QUANT_SCALAR_ROWS);
        if (scalar_rows) {
            hipLaunchKernelGGL((lookup_kernel<DTYPE, MODE, UNROLL, true>), dim3((unsigned)blocks),
                               dim3(PLE_LOOKUP_BLOCK), 0, s, hp, g);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((lookup_kernel<DTYPE, MODE, UNROLL, false>), dim3((unsigned)blocks), dim3(PLE_LOOKUP_BLOCK), 0,
                       s, hp, g);
    return hipGetLastError();
}

template <int DTYPE>
static hipError_t launch_lookup_fmt(const HashParams& hp, const LookupArgs& g, int mode, hipStream_t s) {
    if (mode == kModeHash) return launch_lookup_t<DTYPE, kModeHash>(hp, g, s);
    if (mode == kModeList) return launch_lookup_t<DTYPE, kModeList>(hp, g, s);
    return launch_lookup_t<DTYPE, kModeIds>(hp, g, s);
}

hipError_t launch_lookup(const HashParams& hp, const LookupArgs& g, int dtype, int mode, hipStream_t s) {
    if (dtype == PLE_DTYPE_BF16) return launch_lookup_fmt<kFmtBF16>(hp, g, mode, s);
    if (dtype == PLE_DTYPE_NVFP4) return launch_lookup_fmt<kFmtNVFP4>(hp, g, mode, s);
    // per-row and global-scale fp8 (the scale stride tells them apart)
    return launch_lookup_fmt<kFmtFP8>(hp, g, mode, s);
}

}  // namespace ple
