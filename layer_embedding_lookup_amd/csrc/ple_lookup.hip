// N-gram IDs, row gather and the fused ids+gather lookup for gfx950.
//
// Method: "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels",
// 实现拆解 item 2 and 关键源码片段 (per-token n-gram IDs over ragged requests
// with EOS replacement, the carried ngram_context and int64 wraparound); the
// row lookup of "PR #54371 [Qwen4Exp] Support UVA PLE-offload and Engram
// tensor parallelism", 关键源码片段 (embedding lookup, also from pinned host
// memory); FP8 e4m3fn tables with a scale from "Support PLE-Offload for
// Qwen3.8-Flash-Next - #53899".
//
// Design for CDNA4: one lane per (token, head) pair computes the ID in
// registers (binary search over query_start_loc, window from the token
// array, Barrett reduction instead of a 64-bit divide); the IDs of a block's
// tokens stay in LDS and the block then streams its rows with 16-byte loads
// (one wave instruction moves a whole 1 KiB bf16 row), many loads in flight
// per lane, and coalesced 16-byte stores into the contiguous [tokens][H*D]
// output slab of the block.
#include "ple_launch.h"

namespace ple {

__device__ __forceinline__ int32_t pair_id(const HashParams& hp, const int32_t* __restrict__ tok,
                                           const int32_t* __restrict__ qsl, int R,
                                           const int32_t* __restrict__ ctx, int64_t t, int h) {
    const int r = find_request(qsl, R, t);
    int64_t a = qsl[r];
    a = a < 0 ? 0 : (a > t ? t : a);  // keeps every read in bounds for any qsl
    const int C = hp.context_len;
    const int32_t eos = hp.eos;
    const int order = hp.order[h];
    uint64_t acc = (uint64_t)(int64_t)tok[t] * hp.mult[h][0];
    bool crossed = false;
    for (int j = 1; j < order; ++j) {
        const int64_t p = t - j;
        int32_t raw;
        if (p >= a)
            raw = tok[p];
        else if (ctx != nullptr)
            raw = ctx[(int64_t)r * C + (C - (a - p))];
        else
            raw = eos;
        crossed |= (raw == eos);
        const int64_t s = crossed ? (int64_t)eos : (int64_t)raw;
        acc += (uint64_t)s * hp.mult[h][j];
    }
    return (int32_t)(hp.offset[h] + floor_mod_wrapped(acc, hp.vocab[h], hp.barrett[h], hp.wrap_mod[h]));
}

__global__ __launch_bounds__(256) void ngram_ids_kernel(HashParams hp, const int32_t* __restrict__ tok,
                                                        const int32_t* __restrict__ qsl, int64_t T, int R,
                                                        const int32_t* __restrict__ ctx,
                                                        int32_t* __restrict__ ids) {
    const int H = hp.num_heads;
    const int64_t total = T * H;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
         p += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = p / H;
        const int h = (int)(p - t * H);
        ids[p] = pair_id(hp, tok, qsl, R, ctx, t, h);
    }
}

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
        int64_t a = qsl[r], b = qsl[r + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        const int64_t q = (b - a) + i;  // index into ctx[r] ++ tok[a:b]
        int32_t v;
        if (q >= C)
            v = tok[a + (q - C)];
        else if (ctx != nullptr)
            v = ctx[(int64_t)r * C + q];
        else
            v = eos;
        ctx_out[p] = v;
    }
}

// fp8 e4m3fn x16 (one 16-byte chunk) -> 16 bf16 (two 16-byte chunks), each
// value float(code) * scale in fp32, then round to nearest even.
__device__ __forceinline__ void dequant16(u32x4 q, float scale, u32x4& lo, u32x4& hi) {
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
        f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
        o[2 * k] = pack_bf16x2_canon(a.x * scale, a.y * scale);
        o[2 * k + 1] = pack_bf16x2_canon(b.x * scale, b.y * scale);
    }
    lo = u32x4{o[0], o[1], o[2], o[3]};
    hi = u32x4{o[4], o[5], o[6], o[7]};
}

// One block: `tb` tokens x H heads.  Phase 1 puts the block's row IDs (and
// fp8 scales) in LDS; phase 2 streams the rows.  MODE_HASH computes the IDs,
// MODE_IDS reads (and clamps) caller IDs.
template <int DTYPE, int MODE, int UNROLL>
__global__ __launch_bounds__(256) void lookup_kernel(HashParams hp, LookupArgs g) {
    __shared__ int32_t s_id[256];
    __shared__ float s_scale[256];
    const int tid = threadIdx.x;
    const int H = g.num_heads;
    const int64_t t0 = (int64_t)blockIdx.x * g.tokens_per_block;
    const int nt = (int)min((int64_t)g.tokens_per_block, g.num_tokens - t0);
    const int nrows = nt * H;

    if (tid < nrows) {
        int32_t id;
        if (MODE == kModeHash) {
            const int i = tid / H;
            const int h = tid - i * H;
            id = pair_id(hp, g.tok, g.qsl, g.num_reqs, g.ctx, t0 + i, h);
            if (g.ids_out != nullptr) g.ids_out[t0 * H + tid] = id;
        } else {
            id = g.ids_in[t0 * H + tid];
            id = id < 0 ? 0 : (id >= g.num_rows ? (int32_t)(g.num_rows - 1) : id);
        }
        s_id[tid] = id;
        if (DTYPE == PLE_DTYPE_FP8_E4M3) s_scale[tid] = g.scales[id];
    }
    __syncthreads();

    // chunks of 16 input bytes per row: D*2/16 for bf16, D/16 for fp8
    const int cpr = DTYPE == PLE_DTYPE_BF16 ? (g.dim >> 3) : (g.dim >> 4);
    const int shift = g.cpr_log2;  // >= 0 when cpr is a power of two
    const int total = nrows * cpr;
    const char* __restrict__ table = (const char*)g.table;
    const int64_t row_bytes = DTYPE == PLE_DTYPE_BF16 ? (int64_t)g.dim * 2 : (int64_t)g.dim;
    u32x4* __restrict__ out = (u32x4*)(g.rows + t0 * H * (int64_t)g.dim);

    for (int base = tid; base < total; base += 256 * UNROLL) {
        u32x4 v[UNROLL];
        int rowi[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = base + u * 256;
            if (idx < total) {
                const int row = shift >= 0 ? (idx >> shift) : (idx / cpr);
                const int ch = idx - row * cpr;
                rowi[u] = row;
                const u32x4* src = (const u32x4*)(table + (int64_t)s_id[row] * row_bytes) + ch;
                v[u] = __builtin_nontemporal_load(src);
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = base + u * 256;
            if (idx < total) {
                if (DTYPE == PLE_DTYPE_BF16) {
                    out[idx] = v[u];
                } else {
                    u32x4 lo, hi;
                    dequant16(v[u], s_scale[rowi[u]], lo, hi);
                    out[2 * idx] = lo;
                    out[2 * idx + 1] = hi;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_ngram_ids(const HashParams& hp, const int32_t* tok, const int32_t* qsl, int64_t T, int R,
                            const int32_t* ctx, int32_t* ids, hipStream_t s) {
    const int64_t pairs = T * hp.num_heads;
    int64_t blocks = (pairs + 255) / 256;
    if (blocks > 65535 * 16) blocks = 65535 * 16;
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

int lookup_tokens_per_block(int64_t T, int H) {
    int tb = 256 / H;                      // one lane per (token, head) pair in phase 1
    int64_t target = (T + 1023) / 1024;    // aim for >= 1024 blocks (4 per CU)
    if (target < tb) tb = (int)(target < 1 ? 1 : target);
    return tb;
}

template <int DTYPE, int MODE>
static hipError_t launch_lookup_t(const HashParams& hp, const LookupArgs& g, hipStream_t s) {
    const int64_t blocks = (g.num_tokens + g.tokens_per_block - 1) / g.tokens_per_block;
    hipLaunchKernelGGL((lookup_kernel<DTYPE, MODE, 16>), dim3((unsigned)blocks), dim3(256), 0, s, hp, g);
    return hipGetLastError();
}

hipError_t launch_lookup(const HashParams& hp, const LookupArgs& g, int dtype, int mode, hipStream_t s) {
    if (dtype == PLE_DTYPE_BF16)
        return mode == kModeHash ? launch_lookup_t<PLE_DTYPE_BF16, kModeHash>(hp, g, s)
                                 : launch_lookup_t<PLE_DTYPE_BF16, kModeIds>(hp, g, s);
    return mode == kModeHash ? launch_lookup_t<PLE_DTYPE_FP8_E4M3, kModeHash>(hp, g, s)
                             : launch_lookup_t<PLE_DTYPE_FP8_E4M3, kModeIds>(hp, g, s);
}

}  // namespace ple
