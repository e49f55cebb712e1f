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
// wave finds request boundaries with one cooperative load of query_start_loc
// and ballots, the window tokens are loaded in the same round trip, and the
// modulo is a Barrett reduction instead of a 64-bit divide.  The IDs never
// leave registers: the wave then streams its rows with 16-byte loads (one wave
// instruction moves a whole 1 KiB bf16 row; the row's ID comes from the
// owning lane by a cross-lane read), 16 loads in flight per lane, and writes
// coalesced 16-byte chunks into the wave's contiguous [tokens][H*D] slab.
// Waves never wait for each other.
#include "ple_launch.h"

// Tuning knobs (compile-time): 16-byte loads in flight per lane, and whether
// table reads / row writes carry the non-temporal hint.
// Output chunks (16 bytes) per lane per pass, by table format.
#ifndef PLE_LOOKUP_LOADS
#define PLE_LOOKUP_LOADS 16
#endif
#ifndef PLE_LOOKUP_LOADS_FP8
#define PLE_LOOKUP_LOADS_FP8 16
#endif
#ifndef PLE_LOOKUP_LOADS_FP4
#define PLE_LOOKUP_LOADS_FP4 16
#endif
#ifndef PLE_LOOKUP_NT_LOAD
#define PLE_LOOKUP_NT_LOAD 1
#endif
#ifndef PLE_LOOKUP_NT_STORE
#define PLE_LOOKUP_NT_STORE 0
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

// ID of head h for token t, given its request (r, a) and the raw tokens
// w[j] = tok[max(t-j, 0)] loaded ahead (the value is used only when t-j >= a).
__device__ __forceinline__ int32_t window_id(const HashParams& hp, const int32_t (&w)[PLE_MAX_CONTEXT + 1],
                                             const int32_t* __restrict__ ctx, int r, int64_t a, int64_t t, int h) {
    const int C = hp.context_len;
    const int32_t eos = hp.eos;
    const int order = hp.order[h];
    uint64_t acc = (uint64_t)(int64_t)w[0] * hp.mult[h][0];
    bool crossed = false;
#pragma unroll
    for (int j = 1; j <= PLE_MAX_CONTEXT; ++j) {
        if (j < order) {
            const int64_t p = t - j;
            int32_t raw;
            if (p >= a)
                raw = w[j];
            else if (ctx != nullptr)
                raw = ctx[(int64_t)r * C + (C - (a - p))];
            else
                raw = eos;
            crossed |= (raw == eos);
            const int64_t sj = crossed ? (int64_t)eos : (int64_t)raw;
            acc += (uint64_t)sj * hp.mult[h][j];
        }
    }
    return (int32_t)(hp.offset[h] + floor_mod_wrapped(acc, hp.vocab[h], hp.barrett[h], hp.wrap_mod[h]));
}

__device__ __forceinline__ void store16(u32x4* p, u32x4 v) {
#if PLE_LOOKUP_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// One wave: `tokens_per_wave` consecutive tokens x H heads = at most 64 rows,
// one lane per (token, head) pair for the IDs.  No block-level barrier: each
// wave computes its IDs and streams its rows on its own.  MODE_HASH computes
// the IDs, MODE_IDS reads (and clamps) caller IDs.
template <int DTYPE, int MODE, int UNROLL>
__global__ __launch_bounds__(PLE_LOOKUP_BLOCK) void lookup_kernel(HashParams hp, LookupArgs g) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = (int64_t)blockIdx.x * (PLE_LOOKUP_BLOCK / kWave) + (threadIdx.x >> 6);
    const int TW = g.tokens_per_wave;
    const int64_t t0 = wave * TW;
    if (t0 >= g.num_tokens) return;  // whole wave
    const int H = g.num_heads;
    const int nt = (int)min((int64_t)TW, g.num_tokens - t0);
    const int nrows = nt * H;
    const bool active = lane < nrows;
    const int my_k = active ? lane / H : 0;
    const int h = active ? lane - my_k * H : 0;
    const int64_t t = t0 + my_k;

    int32_t id = 0;
    if (MODE == kModeHash) {
        int32_t w[PLE_MAX_CONTEXT + 1];
#pragma unroll
        for (int j = 0; j <= PLE_MAX_CONTEXT; ++j)
            w[j] = (j <= hp.context_len) ? g.tok[t - j >= 0 ? t - j : 0] : 0;
        int r;
        int64_t a;
        wave_find_request(g.qsl, g.num_reqs, t, t0, nt, my_k, lane, r, a);
        id = window_id(hp, w, g.ctx, r, a, t, h);
        if (active && g.ids_out != nullptr) g.ids_out[t0 * H + lane] = id;
    } else {
        id = active ? g.ids_in[t0 * H + lane] : 0;
        id = id < 0 ? 0 : (id >= g.num_rows ? (int32_t)(g.num_rows - 1) : id);
    }
    // ids mode with rep_of: a repeated row is left for a later copy
    int skip = 0;
    if (MODE == kModeIds && g.rep_of != nullptr && active) skip = g.rep_of[t0 * H + lane] != (int32_t)(t0 * H + lane);
    float scale = 0.f;
    if (DTYPE == kFmtFP8) scale = g.scales[(int64_t)id * g.scale_stride];
    const float tscale = DTYPE == kFmtNVFP4 ? g.scales[0] : 0.f;

    // Every lane produces one 16-byte output chunk (8 bf16 elements) per
    // step, so stores are always lane-contiguous; its input is the same 8
    // elements of the stored row: 16 bytes (bf16), 8 (fp8 codes) or 4 (NVFP4
    // codes, plus the block's scale code).
    const int cpr = g.dim >> 3;    // output chunks per row
    const int shift = g.cpr_log2;  // >= 0 when cpr is a power of two
    const int total = nrows * cpr;
    const char* __restrict__ table = (const char*)g.table;
    constexpr int IB = DTYPE == kFmtBF16 ? 16 : (DTYPE == kFmtFP8 ? 8 : 4);  // input bytes per chunk
    const int64_t row_bytes = (int64_t)cpr * IB;
    u32x4* __restrict__ out = (u32x4*)(g.rows + t0 * H * (int64_t)g.dim);

    for (int base = 0; base < total; base += kWave * UNROLL) {
        u32x4 v[UNROLL];
        float sc[UNROLL];
        uint32_t bsc[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = base + u * kWave + lane;
            int row = shift >= 0 ? (idx >> shift) : (idx / cpr);
            row = row < nrows ? row : nrows - 1;
            const int rid = __shfl(id, row, kWave);
            if (DTYPE == kFmtFP8) sc[u] = __shfl(scale, row, kWave);
            const int rskip = MODE == kModeIds ? __shfl(skip, row, kWave) : 0;
            if (idx < total && !rskip) {
                const int ch = idx - row * cpr;
                const char* src = table + (int64_t)rid * row_bytes + (int64_t)ch * IB;
                if (DTYPE == kFmtBF16) {
#if PLE_LOOKUP_NT_LOAD
                    v[u] = __builtin_nontemporal_load((const u32x4*)src);
#else
                    v[u] = *(const u32x4*)src;
#endif
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
            int rskip = 0;
            if (MODE == kModeIds) {
                int row = shift >= 0 ? (idx >> shift) : (idx / cpr);
                rskip = __shfl(skip, row < nrows ? row : nrows - 1, kWave);
            }
            if (idx < total && !rskip) {
                if (DTYPE == kFmtBF16)
                    store16(out + idx, v[u]);
                else if (DTYPE == kFmtFP8)
                    store16(out + idx, dequant8_fp8(v[u].x, v[u].y, sc[u]));
                else
                    store16(out + idx, dequant8_fp4(v[u].x, bsc[u], tscale));
            }
        }
    }
}

// IDs only: the lookup kernel's first phase.  Each wave takes 64/H
// consecutive tokens (one lane per (token, head)) and writes their IDs as one
// coalesced store.
__global__ __launch_bounds__(256) void ngram_ids_kernel(HashParams hp, const int32_t* __restrict__ tok,
                                                        const int32_t* __restrict__ qsl, int64_t T, int R,
                                                        const int32_t* __restrict__ ctx,
                                                        int32_t* __restrict__ ids) {
    const int lane = threadIdx.x & (kWave - 1);
    const int H = hp.num_heads;
    const int TW = kWave / H;
    const int64_t nwaves = (T + TW - 1) / TW;
    for (int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); wave < nwaves;
         wave += (int64_t)gridDim.x * 4) {
        const int64_t t0 = wave * TW;
        const int nt = (int)min((int64_t)TW, T - t0);
        const bool active = lane < nt * H;
        const int my_k = active ? lane / H : 0;
        const int h = active ? lane - my_k * H : 0;
        const int64_t t = t0 + my_k;
        int32_t w[PLE_MAX_CONTEXT + 1];
#pragma unroll
        for (int j = 0; j <= PLE_MAX_CONTEXT; ++j)
            w[j] = (j <= hp.context_len) ? tok[t - j >= 0 ? t - j : 0] : 0;
        int r;
        int64_t a;
        wave_find_request(qsl, R, t, t0, nt, my_k, lane, r, a);
        const int32_t id = window_id(hp, w, ctx, r, a, t, h);
        if (active) ids[t0 * H + lane] = id;
    }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_ngram_ids(const HashParams& hp, const int32_t* tok, const int32_t* qsl, int64_t T, int R,
                            const int32_t* ctx, int32_t* ids, hipStream_t s) {
    const int TW = kWave / hp.num_heads;
    const int64_t waves = (T + TW - 1) / TW;
    int64_t blocks = (waves + 3) / 4;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    hipLaunchKernelGGL(ngram_ids_kernel, dim3((unsigned)blocks), dim3(256), 0, s, hp, tok, qsl, T, R, ctx, ids);
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
    hipLaunchKernelGGL((lookup_kernel<DTYPE, MODE, UNROLL>), dim3((unsigned)blocks), dim3(PLE_LOOKUP_BLOCK), 0, s, hp,
                       g);
    return hipGetLastError();
}

hipError_t launch_lookup(const HashParams& hp, const LookupArgs& g, int dtype, int mode, hipStream_t s) {
    if (dtype == PLE_DTYPE_BF16)
        return mode == kModeHash ? launch_lookup_t<kFmtBF16, kModeHash>(hp, g, s)
                                 : launch_lookup_t<kFmtBF16, kModeIds>(hp, g, s);
    if (dtype == PLE_DTYPE_NVFP4)
        return mode == kModeHash ? launch_lookup_t<kFmtNVFP4, kModeHash>(hp, g, s)
                                 : launch_lookup_t<kFmtNVFP4, kModeIds>(hp, g, s);
    // per-row and global-scale fp8 (the scale stride tells them apart)
    return mode == kModeHash ? launch_lookup_t<kFmtFP8, kModeHash>(hp, g, s)
                             : launch_lookup_t<kFmtFP8, kModeIds>(hp, g, s);
}

}  // namespace ple
