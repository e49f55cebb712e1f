// Gate and dilated causal short convolution for gfx950.
//
// Method: "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels", 实现拆解
// item 2 (the gate-and-normalisation kernel and the dilated short-convolution
// kernel, with prefill and decode-with-state variants of the convolution).
//
// Gate: one wave per token; each lane keeps fp32 partial sums of h.h, k.k and
// h.k over its 16-byte chunks, the wave reduces them in double, and the same
// wave then scales the value half.  Conv: blocks of 16 tokens x 256 chunks of
// 8 channels; request starts found once per block; each lane issues all the
// tap loads of 4 tokens (16-byte chunks of rows t, t-d, ...) before using
// them; re-reads hit L2, so HBM sees each row about once; taps before a
// request's start come from the carried state.
#include "ple_launch.h"

#include <map>
#include <mutex>

#ifndef PLE_CONV_TOKENS_PER_BLOCK
#define PLE_CONV_TOKENS_PER_BLOCK 32
#endif

// Cache hints (measured on the 8k prefill step, 546 -> 520 us together):
// the gate reads hidden, key and value once, and the conv output is not read
// again by the path, so neither is allowed to push the next kernels' operands
// out of the last-level cache.  (Non-temporal conv tap loads lose the L2
// reuse of each row by four taps and are slower.)
#ifndef PLE_GATE_NT_LOAD
#define PLE_GATE_NT_LOAD 1
#endif
#ifndef PLE_CONV_NT_STORE
#define PLE_CONV_NT_STORE 1
#endif
#ifndef PLE_CONV_CPL
#define PLE_CONV_CPL 2  // conv_rows_kernel, rows wider than 256 chunks: 16-byte chunks per lane per pass (2 beat 1, 4 and 8 at 4096 channels)
#endif

namespace ple {

constexpr int kConvKMax = 8;  // kernel sizes above this use the generic kernel

__device__ __forceinline__ void acc_dot(u32x4 a, u32x4 b, float& aa, float& bb, float& ab) {
    const uint32_t x[4] = {a.x, a.y, a.z, a.w};
    const uint32_t y[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a0 = bf16_lo(x[k]), a1 = bf16_hi(x[k]);
        const float b0 = bf16_lo(y[k]), b1 = bf16_hi(y[k]);
        aa += a0 * a0 + a1 * a1;
        bb += b0 * b0 + b1 * b1;
        ab += a0 * b0 + a1 * b1;
    }
}

// The gate of one token from the wave's per-lane fp32 partial sums of h.h,
// k.k and h.k: reduced across the wave in double, then
// g = sigmoid(<h, k> / (rms(h) rms(k) sqrt(N))) with eps inside each root.
__device__ __forceinline__ float token_gate(float hh, float kk, float hk, int N, float eps) {
    double dhh = hh, dkk = kk, dhk = hk;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        dhh += __shfl_xor(dhh, off, 64);
        dkk += __shfl_xor(dkk, off, 64);
        dhk += __shfl_xor(dhk, off, 64);
    }
    const double n = (double)N;
    const double s = dhk / (sqrt(dhh / n + (double)eps) * sqrt(dkk / n + (double)eps) * sqrt(n));
    return (float)(1.0 / (1.0 + exp(-s)));
}

// 8 gated values g * v, rounded to bf16
__device__ __forceinline__ u32x4 gate_chunk(float g, u32x4 x) {
    return u32x4{pack_bf16x2(g * bf16_lo(x.x), g * bf16_hi(x.x)), pack_bf16x2(g * bf16_lo(x.y), g * bf16_hi(x.y)),
                 pack_bf16x2(g * bf16_lo(x.z), g * bf16_hi(x.z)), pack_bf16x2(g * bf16_lo(x.w), g * bf16_hi(x.w))};
}

// SCALE: also write out = bf16(g * v); otherwise only the gate (into gate and,
// when given, gate2: the fused path's own copy and the caller's).
template <int UNROLL, bool SCALE>
__global__ __launch_bounds__(256) void gate_kernel(const uint16_t* __restrict__ hidden,
                                                   const uint16_t* __restrict__ kv, int64_t T, int N, float eps,
                                                   uint16_t* __restrict__ out, float* __restrict__ gate,
                                                   float* __restrict__ gate2) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave; no block-level barrier below
    const int nch = N >> 3;
    const u32x4* __restrict__ h = (const u32x4*)(hidden + t * N);
    const u32x4* __restrict__ k = (const u32x4*)(kv + t * 2 * (int64_t)N);
    const u32x4* __restrict__ v = k + nch;
    u32x4* __restrict__ o = (u32x4*)(out + t * N);

    // a row of at most 64 x UNROLL chunks is one pass: its value half is
    // loaded with h and k, so the wave makes one round trip, not two
    const bool one_pass = SCALE && nch <= 64 * UNROLL;
    u32x4 vpre[UNROLL];
    float hh = 0.f, kk = 0.f, hk = 0.f;
    for (int base = lane; base < nch; base += 64 * UNROLL) {
        u32x4 hv[UNROLL], kv4[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = base + 64 * u;
            if (idx < nch) {
#if PLE_GATE_NT_LOAD
                hv[u] = __builtin_nontemporal_load(h + idx);
                kv4[u] = __builtin_nontemporal_load(k + idx);
                if (one_pass) vpre[u] = __builtin_nontemporal_load(v + idx);
#else
                hv[u] = h[idx];
                kv4[u] = k[idx];
                if (one_pass) vpre[u] = v[idx];
#endif
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            if (base + 64 * u < nch) acc_dot(hv[u], kv4[u], hh, kk, hk);
    }
    const float g = token_gate(hh, kk, hk, N, eps);
    if (lane == 0 && gate != nullptr) gate[t] = g;
    if (lane == 0 && gate2 != nullptr) gate2[t] = g;
    if (!SCALE) return;

    for (int base = lane; base < nch; base += 64 * UNROLL) {
        u32x4 vv[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            if (base + 64 * u < nch) vv[u] = one_pass ? vpre[u] : v[base + 64 * u];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = base + 64 * u;
            if (idx < nch) o[idx] = gate_chunk(g, vv[u]);
        }
    }
}

__device__ __forceinline__ void unpack8(u32x4 x, float f[8]) {
    f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x);
    f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
    f[4] = bf16_lo(x.z); f[5] = bf16_hi(x.z);
    f[6] = bf16_lo(x.w); f[7] = bf16_hi(x.w);
}

__device__ __forceinline__ float bf16_at(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }

// One 16-byte output chunk (8 channels) of the convolution: wq[q] holds the
// 8 x KC weights of the chunk's channels (channel-major, [8][KC] bf16) as KC
// 16-byte chunks, xv[i] the 8 inputs of tap i (token t - i*d; tap i meets
// weight KC-1-i).  fp32 accumulation from the current token back, bf16 out.
template <int KC>
__device__ __forceinline__ u32x4 conv_chunk(const u32x4 (&wq)[KC], const u32x4 (&xv)[KC]) {
    uint32_t wd[4 * KC];
#pragma unroll
    for (int q = 0; q < KC; ++q) {
        wd[4 * q] = wq[q].x; wd[4 * q + 1] = wq[q].y; wd[4 * q + 2] = wq[q].z; wd[4 * q + 3] = wq[q].w;
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        float f[8];
        unpack8(xv[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int flat = e * KC + (KC - 1 - i);  // w[c*8+e][KC-1-i]
            const float wt = (flat & 1) ? bf16_hi(wd[flat >> 1]) : bf16_lo(wd[flat >> 1]);
            acc[e] += wt * f[e];
        }
    }
    return u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                 pack_bf16x2(acc[6], acc[7])};
}

// One lane per (token, 8 channels).  KC > 0: compile-time kernel size with the
// 8 x KC weights read as KC 16-byte chunks; KC == 0: any kernel size, scalar
// weight reads.
template <int KC>
__global__ __launch_bounds__(256) void conv_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ qsl,
                                                   int64_t T, int R, const uint16_t* __restrict__ state,
                                                   const uint16_t* __restrict__ w, int N, int K_rt, int d,
                                                   uint16_t* __restrict__ y) {
    const int K = KC > 0 ? KC : K_rt;
    const int nch = N >> 3;
    const int64_t S = (int64_t)(K - 1) * d;
    const int64_t total = T * nch;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
         p += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = p / nch;
        const int ch = (int)(p - t * nch);
        const int c0 = ch * 8;
        const int r = find_request(qsl, R, t);
        int64_t a = qsl[r];
        a = a < 0 ? 0 : (a > t ? t : a);

        float wt[8][KC > 0 ? KC : 1];
        if (KC > 0) {
            const u32x4* wp = (const u32x4*)(w + (int64_t)c0 * K);
            uint32_t words[4 * (KC > 0 ? KC : 1)];
#pragma unroll
            for (int q = 0; q < (KC > 0 ? KC : 1); ++q) {
                const u32x4 v4 = wp[q];
                words[4 * q] = v4.x; words[4 * q + 1] = v4.y; words[4 * q + 2] = v4.z; words[4 * q + 3] = v4.w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int k = 0; k < (KC > 0 ? KC : 1); ++k) {
                    const int flat = e * K + k;
                    const uint32_t wd = words[flat >> 1];
                    wt[e][k] = (flat & 1) ? bf16_hi(wd) : bf16_lo(wd);
                }
        }

        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < K; ++i) {
            const int64_t pp = t - (int64_t)i * d;
            u32x4 xv = {0u, 0u, 0u, 0u};
            if (pp >= a)
                xv = *(const u32x4*)(x + pp * N + c0);
            else if (state != nullptr)
                xv = *(const u32x4*)(state + ((int64_t)r * S + (S - (a - pp))) * N + c0);
            float f[8];
            unpack8(xv, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float wv;
                if (KC > 0) {
                    // i is a loop variable here; select the tap without dynamic register indexing
                    wv = 0.f;
#pragma unroll
                    for (int k = 0; k < (KC > 0 ? KC : 1); ++k)
                        if (k == K - 1 - i) wv = wt[e][k];
                } else {
                    wv = bf16_at(w + (int64_t)(c0 + e) * K + (K - 1 - i));
                }
                acc[e] += wv * f[e];
            }
        }
        *(u32x4*)(y + t * N + c0) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                          pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    }
}

// LDS-staged convolution.  A block covers TB consecutive tokens x 64 chunks of
// 8 channels (1 KiB of each row).  It stages the rows [t0 - S, t0 + TB) of its
// channel slice in LDS once (every input element is read from HBM once, plus
// an S-row halo per tile), wave 0 finds each token's request with one
// cooperative load of query_start_loc, then lane c of each wave produces
// channel chunk c for every 4th token, reading its taps from LDS.  Taps that
// fall before the token's request start come from the carried state (a
// global read, only near request starts) or are zero.
template <int TB>
__global__ __launch_bounds__(256) void conv_lds_kernel(const uint16_t* __restrict__ x,
                                                       const int32_t* __restrict__ qsl, int64_t T, int R,
                                                       const uint16_t* __restrict__ state,
                                                       const uint16_t* __restrict__ w, int N, int K, int d,
                                                       uint16_t* __restrict__ y) {
    extern __shared__ u32x4 s_x[];  // (TB + S) rows x 64 chunks
    __shared__ uint16_t s_w[kWave * 8 * kConvKMax];  // this slice's weights, [channel][tap]
    __shared__ int32_t s_r[TB];
    __shared__ int64_t s_a[TB];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid >> 6;
    const int nch = N >> 3;
    // the channel slice varies fastest with the block id, so the slices of one
    // token tile are adjacent block ids: together they touch whole rows at once, and with
    // block ids dealt round-robin to the 8 XCDs each XCD keeps one slice (and
    // the halo rows it shares with the previous tile) in its own L2
    const int nslice = (nch + kWave - 1) / kWave;
    const int64_t t0 = (int64_t)(blockIdx.x / nslice) * TB;
    const int nt = (int)min((int64_t)TB, T - t0);
    const int S = (K - 1) * d;
    const int c = (int)(blockIdx.x % nslice) * kWave + lane;  // this lane's channel chunk
    const bool cvalid = c < nch;

    // stage rows t0 - S .. t0 + nt - 1 (row index in LDS: p - (t0 - S))
    const int nrow = nt + S;
    for (int i = wv; i < nrow; i += 4) {
        const int64_t p = t0 - S + i;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (p >= 0 && cvalid) v = *(const u32x4*)(x + p * N + (int64_t)c * 8);
        s_x[i * kWave + lane] = v;
    }
    {
        // the slice's 512 channels x K taps are contiguous in w: 64*K 16-byte chunks
        const int slice_c0 = (int)(blockIdx.x % nslice) * kWave * 8;
        const int nchunk = min(kWave, nch - (int)(blockIdx.x % nslice) * kWave) * K;
        const u32x4* wsrc = (const u32x4*)(w + (int64_t)slice_c0 * K);
        for (int i = tid; i < nchunk; i += 256) ((u32x4*)s_w)[i] = wsrc[i];
    }
    if (wv == 0) {
        const int my_k = lane < nt ? lane : 0;
        int r;
        int64_t a;
        wave_find_request(qsl, R, t0 + my_k, t0, nt, my_k, lane, r, a);
        if (lane < nt) {
            s_r[lane] = r;
            s_a[lane] = a;
        }
    }
    __syncthreads();
    if (!cvalid) return;  // no barrier below

    const int c0 = c * 8;
    // this lane's 8 channels x K taps, tap order reversed: wt[e][i] multiplies x(t - i*d)
    float wt[8][kConvKMax];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < kConvKMax; ++i)
            wt[e][i] = i < K ? __uint_as_float((uint32_t)s_w[(lane * 8 + e) * K + (K - 1 - i)] << 16) : 0.f;
    for (int k = wv; k < nt; k += 4) {
        const int64_t t = t0 + k;
        const int64_t a = s_a[k];
        const int r = s_r[k];
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kConvKMax; ++i) {
            if (i < K) {
                const int64_t p = t - (int64_t)i * d;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (p >= a)
                    v = s_x[(int)(p - (t0 - S)) * kWave + lane];
                else if (state != nullptr)
                    v = *(const u32x4*)(state + ((int64_t)r * S + (S - (a - p))) * N + c0);
                float f[8];
                unpack8(v, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += wt[e][i] * f[e];
            }
        }
        *(u32x4*)(y + t * N + c0) = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                          pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    }
}

// Persistent row-wise convolution for compile-time kernel sizes (the fast
// path).  Each block stages all N x KC weights in LDS once, then its waves
// walk tokens: a wave produces one whole output row at a time.  Tokens are
// dealt so that each XCD (block id mod 8) owns a contiguous token range and
// its waves work on neighbouring tokens together; the tap rows t-d, t-2d, ...
// a wave reads were just read by its neighbours, so they come from that XCD's
// L2 and HBM sees each input row about once.  The tap loads are issued
// speculatively together with the request lookup (one round trip); taps that
// fall before the request start are then replaced by the carried state (or
// zero).
// GATED: the conv input of token p is bf16(g[p] * v[p]) with v[p] the value
// half of kv's row p (row stride x_stride), formed here with the gate's own
// arithmetic (gate_chunk), so the gated value never goes through memory;
// carried-state rows are conv inputs already.  With gated_out, the conv
// inputs of each request's last S tokens (the rows the carried state takes)
// and of every token of a request of at most kConvInputWindow tokens (a
// speculative verify window) are written there.
template <int KC, int CPL, bool GATED>
__global__ __launch_bounds__(256) void conv_rows_kernel(ConvRowsArgs a) {
    // weights [N][KC] = nch x KC 16-byte chunks, kept in LDS tap-chunk-major
    // (s_wv[q * nch + c]) so that consecutive lanes read consecutive chunks
    extern __shared__ u32x4 s_wv[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid >> 6;
    const int N = a.N;
    const int nch = N >> 3;
    const int64_t T = a.T;
    const int64_t S = (int64_t)(KC - 1) * a.d;
    const int xcd = blockIdx.x & 7;
    const int64_t blocks_per_xcd = gridDim.x >> 3;  // the grid is a multiple of 8
    const int64_t per_xcd = (T + 7) / 8;
    const int64_t t_begin = xcd * per_xcd;
    const int64_t t_end = min(T, t_begin + per_xcd);
    const int64_t stride = blocks_per_xcd * 4;
    const int64_t t_first = t_begin + (int64_t)(blockIdx.x >> 3) * 4 + wv;

    // the first token's query_start_loc probe goes out with the weight
    // staging, so that its round trip overlaps the staging's
    QslProbe qp;
    qsl_probe_load(a.qsl, a.R, lane, qp);
    for (int i = tid; i < nch * KC; i += 256) {
        const int c = i / KC, q = i - (i / KC) * KC;
        s_wv[q * nch + c] = ((const u32x4*)a.w)[i];
    }
    __syncthreads();

    for (int64_t t = t_first; t < t_end; t += stride) {
        int r = 0;
        int64_t ra = 0;
        if (t == t_first)
            wave_find_request_probed(a.qsl, qp, a.R, t, t, 1, 0, lane, r, ra);
        else
            wave_find_request(a.qsl, a.R, t, t, 1, 0, lane, r, ra);
        // tap i of this token: the batch row t - i*d within the request, else
        // the carried state row (oldest first), else zero; resolved before any
        // load, so each pass is one round trip
        const uint16_t* src[KC];
        float gs[KC];
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int64_t p = t - (int64_t)i * a.d;
            src[i] = p >= ra ? a.x + p * a.x_stride
                             : (a.state != nullptr ? a.state + ((int64_t)r * S + (S - (ra - p))) * N : nullptr);
            gs[i] = 1.f;
            if (GATED && p >= ra) gs[i] = a.g[p];
        }
        bool keep = false;  // this token's conv input goes to gated_out
        if (GATED && a.gated_out != nullptr) {
            int64_t rb = a.qsl[r + 1];
            rb = rb < t + 1 ? t + 1 : rb;
            keep = t >= rb - S || rb - ra <= kConvInputWindow;
        }
        for (int cb = 0; cb < nch; cb += kWave * CPL) {
            u32x4 xv[CPL][KC];
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = cb + j * kWave + lane;
#pragma unroll
                for (int i = 0; i < KC; ++i) {
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (c < nch && src[i] != nullptr) v = *(const u32x4*)(src[i] + (int64_t)c * 8);
                    xv[j][i] = v;
                }
            }
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = cb + j * kWave + lane;
                if (c < nch) {
                    if (GATED) {
#pragma unroll
                        for (int i = 0; i < KC; ++i)
                            if (t - (int64_t)i * a.d >= ra) xv[j][i] = gate_chunk(gs[i], xv[j][i]);
                        if (keep) *(u32x4*)(a.gated_out + t * N + (int64_t)c * 8) = xv[j][0];
                    }
                    u32x4 wq[KC];
#pragma unroll
                    for (int q = 0; q < KC; ++q) wq[q] = s_wv[q * nch + c];
#if PLE_CONV_NT_STORE
                    __builtin_nontemporal_store(conv_chunk<KC>(wq, xv[j]), (u32x4*)(a.y + t * N + (int64_t)c * 8));
#else
                    *(u32x4*)(a.y + t * N + (int64_t)c * 8) = conv_chunk<KC>(wq, xv[j]);
#endif
                }
            }
        }
    }
}

template <int KC, int CPL, bool GATED>
static hipError_t launch_conv_rows_t(const ConvRowsArgs& a, hipStream_t s) {
    const size_t lds = (size_t)a.N * KC * 2;
    static const hipError_t attr = hipFuncSetAttribute((const void*)conv_rows_kernel<KC, CPL, GATED>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
    if (attr != hipSuccess) return attr;
    // resident blocks per device for this kernel and weight size (queried once)
    static std::mutex mu;
    static std::map<std::pair<int, size_t>, int64_t> resident;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    int64_t blocks;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = resident.find({dev, lds});
        if (it == resident.end()) {
            int cus = 256, per_cu = 1;
            (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, conv_rows_kernel<KC, CPL, GATED>, 256, lds) !=
                    hipSuccess ||
                per_cu < 1)
                per_cu = 1;
            it = resident.emplace(std::make_pair(dev, lds), (int64_t)cus * per_cu).first;
        }
        blocks = it->second;                                 // every block resident at once
    }
    const int64_t need = (a.T + 3) / 4;                      // one wave per token at most
    if (blocks > need) blocks = need;
    blocks = ((blocks + 7) / 8) * 8;                         // whole XCD rounds
    hipLaunchKernelGGL((conv_rows_kernel<KC, CPL, GATED>), dim3((unsigned)blocks), dim3(256), lds, s, a);
    return hipGetLastError();
}

// Rows of at most 256 16-byte chunks (N <= 2048) go in one pass of 4 chunks
// per lane, so a token costs one round trip; wider rows take passes of 2
// (measured best for the 4096-wide prefill).
template <int KC, bool GATED>
static hipError_t launch_conv_rows(const ConvRowsArgs& a, hipStream_t s) {
    if ((a.N >> 3) <= 4 * kWave) return launch_conv_rows_t<KC, 4, GATED>(a, s);
    return launch_conv_rows_t<KC, PLE_CONV_CPL, GATED>(a, s);
}

bool conv_rows_supported(int K, int N) { return K >= 1 && K <= 4 && (size_t)N * K * 2 <= 64 * 1024; }

// ---------------------------------------------------------------------------
// LDS-staged conv for batches of long requests (prefill).  A block of four
// waves takes TBS consecutive tokens x one 512-channel slice: it stages the
// slice of rows t0-S .. t0+nt-1 in LDS once (gated, in the fused step: each
// row multiplied by its token's gate once, not once per tap), every wave
// with eight row loads in flight, then each wave forms the outputs of every
// fourth token from the staged taps (the carried state's rows, for taps
// before a request's start, straight from global memory).  The channel slice
// varies fastest with the block id, so the slices of one token tile are
// adjacent blocks.  Same arithmetic as conv_rows_kernel (gate_chunk,
// conv_chunk), so the same bits.
// ---------------------------------------------------------------------------
#ifndef PLE_CONV_STAGED
#define PLE_CONV_STAGED 1
#endif
#ifndef PLE_CONV_STAGED_TB
#define PLE_CONV_STAGED_TB 16  // tokens per block (8, 12, 24, 32, 48 measured slower at the 8k prefill)
#endif
constexpr int kStageLoads = 8;   // staged rows in flight per wave

template <int KC, int TBS, bool GATED>
__global__ __launch_bounds__(256) void conv_staged_kernel(ConvRowsArgs a) {
    extern __shared__ u32x4 s_x[];  // (TBS + S) rows x 64 chunks
    __shared__ int32_t s_r[TBS];
    __shared__ int64_t s_a[TBS];
    __shared__ int64_t s_b[TBS];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid >> 6;
    const int N = a.N;
    const int nch = N >> 3;
    const int nslice = (nch + kWave - 1) / kWave;
    const int d = a.d;
    const int S = (KC - 1) * d;
    const int64_t t0 = (int64_t)(blockIdx.x / nslice) * TBS;
    const int nt = (int)min((int64_t)TBS, a.T - t0);
    const int c = (int)(blockIdx.x % nslice) * kWave + lane;
    const bool cv = c < nch;
    const int64_t coff = (int64_t)(cv ? c : nch - 1) * 8;  // lanes past the row stay in it
    const int nrow = nt + S;

    // Wave 0 finds the tile's tokens' requests (lane k: token t0 + k).  With
    // fewer than 64 requests (one query_start_loc entry per lane) that entry
    // goes out first and the wave's share of the staged rows right behind
    // it, so the search costs no round trip of its own; more requests are
    // searched before the staging, as their probe holds 16 registers.
    const bool few_reqs = a.R + 1 <= kWave;
    int q0 = 0;
    if (wv == 0) {
        const int my_k = lane < nt ? lane : 0;
        if (few_reqs) {
            q0 = lane <= a.R ? a.qsl[lane] : 0;
        } else {
            int r;
            int64_t ra;
            wave_find_request(a.qsl, a.R, t0 + my_k, t0, nt, my_k, lane, r, ra);
            if (lane < nt) {
                int64_t rb = a.qsl[r + 1];
                rb = rb < t0 + my_k + 1 ? t0 + my_k + 1 : rb;
                s_r[lane] = r;
                s_a[lane] = ra;
                s_b[lane] = rb;
            }
        }
    }
    // stage rows t0 - S + i (LDS row i), those before the batch as zeros
    for (int i0 = wv; i0 < nrow; i0 += 4 * kStageLoads) {
        u32x4 v[kStageLoads];
        float g[kStageLoads];
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int i = i0 + 4 * u;
            const int64_t p = t0 - S + i;
            v[u] = u32x4{0u, 0u, 0u, 0u};
            g[u] = 1.f;
            if (i < nrow && p >= 0) {
                v[u] = *(const u32x4*)(a.x + p * a.x_stride + coff);
                if (GATED) g[u] = a.g[p];
            }
        }
        if (wv == 0 && i0 == 0 && few_reqs) {
            // the request of token t0 + k: the entries qsl[1..R] at or below it
            const int my_k = lane < nt ? lane : 0;
            int r = 0;
            for (int k = 0; k < nt; ++k) {
                const uint64_t m = __ballot(lane >= 1 && lane <= a.R && (int64_t)q0 <= t0 + k);
                const int rk = (int)__popcll(m);
                if (k == my_k) r = rk < a.R - 1 ? rk : a.R - 1;
            }
            const int64_t t = t0 + my_k;
            int64_t ra = __shfl(q0, r, kWave);
            ra = ra < 0 ? 0 : (ra > t ? t : ra);
            int64_t rb = __shfl(q0, r + 1, kWave);
            rb = rb < t + 1 ? t + 1 : rb;
            if (lane < nt) {
                s_r[lane] = r;
                s_a[lane] = ra;
                s_b[lane] = rb;
            }
        }
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int i = i0 + 4 * u;
            if (i < nrow) s_x[i * kWave + lane] = GATED ? gate_chunk(g[u], v[u]) : v[u];
        }
    }
    __syncthreads();
    if (!cv) return;  // no barrier below

    u32x4 wq[KC];
#pragma unroll
    for (int q = 0; q < KC; ++q) wq[q] = ((const u32x4*)a.w)[(int64_t)c * KC + q];
    const int64_t S64 = S;
    for (int k = wv; k < nt; k += 4) {
        const int64_t t = t0 + k;
        const int r = s_r[k];
        const int64_t ra = s_a[k];
        const int64_t rb = s_b[k];
        u32x4 xv[KC];
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int64_t p = t - (int64_t)i * d;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (p >= ra)
                v = s_x[(int)(p - (t0 - S)) * kWave + lane];
            else if (a.state != nullptr)
                v = *(const u32x4*)(a.state + ((int64_t)r * S64 + (S64 - (ra - p))) * N + coff);
            xv[i] = v;
        }
#if PLE_CONV_NT_STORE
        __builtin_nontemporal_store(conv_chunk<KC>(wq, xv), (u32x4*)(a.y + t * N + coff));
#else
        *(u32x4*)(a.y + t * N + coff) = conv_chunk<KC>(wq, xv);
#endif
        if (GATED && a.gated_out != nullptr && (t >= rb - S64 || rb - ra <= kConvInputWindow))
            *(u32x4*)(a.gated_out + t * N + coff) = xv[0];
    }
}

template <int KC, bool GATED>
static hipError_t launch_conv_staged(const ConvRowsArgs& a, hipStream_t s) {
    constexpr int TBS = PLE_CONV_STAGED_TB;
    const int nslice = ((a.N >> 3) + kWave - 1) / kWave;
    const size_t lds = (size_t)(TBS + (KC - 1) * a.d) * kWave * 16;
    const int64_t blocks = (int64_t)nslice * ((a.T + TBS - 1) / TBS);
    hipLaunchKernelGGL((conv_staged_kernel<KC, TBS, GATED>), dim3((unsigned)blocks), dim3(256), lds, s, a);
    return hipGetLastError();
}

// Staging pays where a tile's tokens share their requests (prefill: requests
// of 16 tokens and more on average) and the staged rows fit 64 KiB of LDS;
// decode and verify windows keep one wave per token and row.
static bool conv_staged_pays(const ConvRowsArgs& a, int K) {
    return PLE_CONV_STAGED && a.R >= 1 && a.T >= (int64_t)16 * a.R && a.T >= 4 * PLE_CONV_STAGED_TB &&
           (PLE_CONV_STAGED_TB + (int64_t)(K - 1) * a.d) * kWave * 16 <= 64 * 1024;
}

template <int KC, bool GATED>
static hipError_t launch_conv_any(const ConvRowsArgs& a, hipStream_t s) {
    return conv_staged_pays(a, KC) ? launch_conv_staged<KC, GATED>(a, s) : launch_conv_rows<KC, GATED>(a, s);
}

hipError_t launch_conv_gated(const ConvRowsArgs& a, int K, hipStream_t s) {
    if (a.T <= 0) return hipSuccess;
    switch (K) {
        case 1: return launch_conv_any<1, true>(a, s);
        case 2: return launch_conv_any<2, true>(a, s);
        case 3: return launch_conv_any<3, true>(a, s);
        case 4: return launch_conv_any<4, true>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// state_out[r][m] = the (S-m)-th most recent conv input of state[r] ++ x[a:b].
__global__ __launch_bounds__(256) void conv_state_out_kernel(const uint16_t* __restrict__ x,
                                                             const int32_t* __restrict__ qsl, int64_t T, int R,
                                                             const uint16_t* __restrict__ state, int N, int S,
                                                             uint16_t* __restrict__ state_out) {
    // one wave per state row (r, m)
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t rows = (int64_t)R * S;
    const int wpb = blockDim.x / kWave;
    for (int64_t w = (int64_t)blockIdx.x * wpb + threadIdx.x / kWave; w < rows; w += (int64_t)gridDim.x * wpb) {
        const int r = (int)(w / S);
        const int m = (int)(w - (int64_t)r * S);
        int64_t a, b;
        carried_window(qsl, T, r, nullptr, a, b);
        carry_state_row(x, state, N, S, r, m, a, b, state_out, lane);
    }
}

// Decode tail: gate, conv and the carried state and context of a batch in
// which every request has at most kTailTokens tokens (a decode step, or a
// speculative verify window), in one launch.  One block of eight waves per
// request.  Wave j < kTailTokens takes the request's token t = a + j (if
// any): its gate from the h and k rows and the gated row g*v, which it writes
// to `gated` (the conv input), to the block's LDS and, when it is among the
// last S inputs, to its carried state row; after a block barrier, its conv
// output, whose taps inside the window come from the other token waves'
// gated rows in LDS and whose older taps come from the carried state (or are
// zero).  Waves 4-7 shift the carried state by the window length (rows n..
// of the old state), a quarter each, and write the carried context.  The
// conv's state taps, weights and the value row are loaded with the h and k
// rows, so a token costs one round trip after the request lookup.
// Arithmetic is that of gate_kernel and conv_rows_kernel (token_gate,
// gate_chunk, conv_chunk), so the results are the same bits.  Tokens past
// the kTailTokens-th of a request are left unwritten (the caller promised
// none); every access stays in bounds for any query_start_loc.
constexpr int kTailTokens = 4;

template <int KC>
__global__ __launch_bounds__(512) void decode_tail_kernel(DecodeTailArgs a) {
    constexpr int G = 4;  // 16-byte chunks per lane per pass
    extern __shared__ u32x4 s_gated[];  // [kTailTokens][nch]: the window's gated rows
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r = blockIdx.x;
    int64_t ta, tb;
    carried_window(a.qsl, a.T, r, nullptr, ta, tb);
    const int n = (int)min(tb - ta, (int64_t)(1 << 30));
    const int N = a.N, nch = N >> 3;
    const int S = (KC - 1) * a.d;
    const bool token_wave = wid < kTailTokens;  // wave-uniform

    // token wave j: slot j of the window
    const int j = token_wave ? wid : 0;
    const bool has = token_wave && j < n;
    const int64_t t = has ? ta + j : 0;
    const u32x4* __restrict__ v = (const u32x4*)(a.kv + t * 2 * (int64_t)N) + nch;
    const u32x4* __restrict__ wc = (const u32x4*)a.conv_w;  // chunk c's weights: KC chunks from c*KC
    // tap i (1..KC-1) of this token: inside the window (slot j - i*d of the
    // block's LDS) or before it (carried state row S - (i*d - j), or zero)
    auto state_tap = [&](int i) -> const u32x4* {
        const int back = i * a.d - j;  // rows before the request start
        return (back > 0 && a.state != nullptr) ? (const u32x4*)(a.state + ((int64_t)r * S + (S - back)) * N)
                                                : nullptr;
    };
    u32x4 vv[G], xv[G][KC], wq[G][KC];
    auto load_pass = [&](int c0) {
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const int c = c0 + q * kWave + lane;
            const bool in = has && c < nch;
            vv[q] = in ? v[c] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 1; i < KC; ++i) {
                const u32x4* tr = state_tap(i);
                xv[q][i] = (in && tr != nullptr) ? tr[c] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int w = 0; w < KC; ++w) wq[q][w] = in ? wc[(int64_t)c * KC + w] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    const bool one_pass = nch <= G * kWave;

    if (!token_wave) {
        // waves 4-7: carried state shift (a quarter each) and context
        const int cw = wid - kTailTokens;
        if (cw == 0 && a.ctx_out != nullptr && lane < a.C)
            a.ctx_out[(int64_t)r * a.C + lane] = carried_token(a.tok, a.ctx, a.C, a.eos, r, lane, ta, tb);
        if (a.state_out != nullptr && S > n) {
            // out rows m < S - n take old rows m + n (zeros without a state):
            // a flat copy of (S - n) * nch chunks, 16 in flight per lane
            constexpr int U = 16;
            const int all = (S - n) * nch;
            const int per = (all + 4 * kWave - 1) / (4 * kWave) * kWave;  // whole passes of 64 chunks
            const int lo = cw * per;
            const int total = min(all, lo + per);
            const u32x4* src = a.state != nullptr ? (const u32x4*)(a.state + ((int64_t)r * S + n) * N) : nullptr;
            u32x4* dst = (u32x4*)(a.state_out + (int64_t)r * S * N);
            for (int base = lo; base < total; base += U * kWave) {
                u32x4 cp[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int idx = base + u * kWave + lane;
                    cp[u] = (src != nullptr && idx < total) ? src[idx] : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int idx = base + u * kWave + lane;
                    if (idx < total) dst[idx] = cp[u];
                }
            }
        }
    } else {
        const u32x4* __restrict__ h = (const u32x4*)(a.hidden + t * N);
        const u32x4* __restrict__ k = (const u32x4*)(a.kv + t * 2 * (int64_t)N);
        if (one_pass) load_pass(0);  // independent of the gate: in flight with h and k

        // per-lane partial sums in gate_kernel's order (chunks lane, lane+64, ...)
        constexpr int UNROLL = 8;
        float hh = 0.f, kk = 0.f, hk = 0.f;
        if (has) {
            for (int base = lane; base < nch; base += 64 * UNROLL) {
                u32x4 hv[UNROLL], kv4[UNROLL];
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    const int idx = base + 64 * u;
                    if (idx < nch) {
                        hv[u] = h[idx];
                        kv4[u] = k[idx];
                    }
                }
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
                    if (base + 64 * u < nch) acc_dot(hv[u], kv4[u], hh, kk, hk);
            }
        }
        const float g = token_gate(hh, kk, hk, N, a.eps);
        if (has && lane == 0 && a.gate != nullptr) a.gate[t] = g;
        // the newest carried state rows are the window's last S gated rows
        const int srow = j + S - n;
        uint16_t* st_row = (has && a.state_out != nullptr && srow >= 0 && srow < S)
                               ? a.state_out + ((int64_t)r * S + srow) * N
                               : nullptr;

        // gated rows: to memory, LDS and the carried state
        for (int c0 = 0; c0 < nch; c0 += G * kWave) {
            if (!one_pass) load_pass(c0);
#pragma unroll
            for (int q = 0; q < G; ++q) {
                const int c = c0 + q * kWave + lane;
                if (has && c < nch) {
                    const u32x4 gv = gate_chunk(g, vv[q]);
                    s_gated[j * nch + c] = gv;
                    ((u32x4*)(a.gated + t * N))[c] = gv;
                    if (st_row != nullptr) ((u32x4*)st_row)[c] = gv;
                }
            }
        }
    }
    // the one barrier of the block: every wave reaches it, the token waves'
    // gated rows are then in LDS
    __syncthreads();
    if (!token_wave) return;

    // conv: tap 0 is this token, taps inside the window from LDS
    for (int c0 = 0; c0 < nch; c0 += G * kWave) {
        if (!one_pass) load_pass(c0);
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const int c = c0 + q * kWave + lane;
            if (has && c < nch) {
                u32x4 x[KC];
#pragma unroll
                for (int i = 0; i < KC; ++i) {
                    const int slot = j - i * a.d;
                    x[i] = slot >= 0 ? s_gated[slot * nch + c] : xv[q][i];
                }
                ((u32x4*)(a.y + t * N))[c] = conv_chunk<KC>(wq[q], x);
            }
        }
    }
}

template <int KC>
static hipError_t launch_decode_tail_t(const DecodeTailArgs& a, hipStream_t s) {
    // one request per block: waves 0-3 its tokens, waves 4-7 the state shift
    const size_t lds = (size_t)kTailTokens * (size_t)a.N * 2;
    static const hipError_t attr = hipFuncSetAttribute((const void*)decode_tail_kernel<KC>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(decode_tail_kernel<KC>, dim3((unsigned)a.R), dim3(512), lds, s, a);
    return hipGetLastError();
}

bool decode_tail_supported(int max_request_tokens, int K, int N) {
    return max_request_tokens >= 1 && max_request_tokens <= kTailTokens && K >= 1 && K <= 4 &&
           (size_t)kTailTokens * (size_t)N * 2 <= 64 * 1024;
}

hipError_t launch_decode_tail(const DecodeTailArgs& a, int K, hipStream_t s) {
    if (a.R <= 0) return hipSuccess;
    switch (K) {
        case 1: return launch_decode_tail_t<1>(a, s);
        case 2: return launch_decode_tail_t<2>(a, s);
        case 3: return launch_decode_tail_t<3>(a, s);
        case 4: return launch_decode_tail_t<4>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gate(const uint16_t* hidden, const uint16_t* kv, int64_t T, int N, float eps, uint16_t* out,
                       float* gate, hipStream_t s) {
    const int64_t blocks = (T + 3) / 4;
    hipLaunchKernelGGL((gate_kernel<8, true>), dim3((unsigned)blocks), dim3(256), 0, s, hidden, kv, T, N, eps, out,
                       gate, nullptr);
    return hipGetLastError();
}

hipError_t launch_gate_only(const uint16_t* hidden, const uint16_t* kv, int64_t T, int N, float eps, float* g,
                            float* gate, hipStream_t s) {
    // passes of 4 chunks per lane: with fewer registers every wave of the 8k
    // prefill is resident at once (the same sums in the same order as 8)
    const int64_t blocks = (T + 3) / 4;
    hipLaunchKernelGGL((gate_kernel<4, false>), dim3((unsigned)blocks), dim3(256), 0, s, hidden, kv, T, N, eps,
                       nullptr, g, gate);
    return hipGetLastError();
}

hipError_t launch_conv(const uint16_t* x, const int32_t* qsl, int64_t T, int R, const uint16_t* state,
                       const uint16_t* w, int N, int K, int d, uint16_t* y, hipStream_t s) {
    if (conv_rows_supported(K, N)) {
        ConvRowsArgs a = {};
        a.x = x;
        a.x_stride = N;
        a.qsl = qsl;
        a.T = T;
        a.R = R;
        a.state = state;
        a.w = w;
        a.N = N;
        a.d = d;
        a.y = y;
        switch (K) {
            case 1: return launch_conv_any<1, false>(a, s);
            case 2: return launch_conv_any<2, false>(a, s);
            case 3: return launch_conv_any<3, false>(a, s);
            default: return launch_conv_any<4, false>(a, s);
        }
    }
    constexpr int TB = PLE_CONV_TOKENS_PER_BLOCK;
    const int nch = N >> 3;
    const int S = (K - 1) * d;
    const size_t lds = (size_t)(TB + S) * kWave * 16;
    if (lds <= 96 * 1024 && K <= kConvKMax) {
        static const hipError_t attr = hipFuncSetAttribute((const void*)conv_lds_kernel<TB>,
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
        if (attr != hipSuccess) return attr;
        dim3 g((unsigned)(((nch + kWave - 1) / kWave) * ((T + TB - 1) / TB)));
        hipLaunchKernelGGL((conv_lds_kernel<TB>), g, dim3(256), lds, s, x, qsl, T, R, state, w, N, K, d, y);
    } else {
        const int64_t total = T * nch;
        int64_t blocks = (total + 255) / 256;
        if (blocks > (1 << 20)) blocks = 1 << 20;
        hipLaunchKernelGGL(conv_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, x, qsl, T, R, state, w, N, K, d,
                           y);
    }
    return hipGetLastError();
}

hipError_t launch_conv_state_out(const uint16_t* x, const int32_t* qsl, int64_t T, int R,
                                 const uint16_t* state, int N, int S, uint16_t* state_out, hipStream_t s) {
    int64_t blocks = ((int64_t)R * S + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(conv_state_out_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, qsl, T, R, state, N, S,
                       state_out);
    return hipGetLastError();
}

}  // namespace ple
