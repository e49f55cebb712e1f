// Gate and dilated causal short convolution for gfx950.
//
// Method: "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels", 实现拆解
// item 2 (the gate-and-normalisation kernel and the dilated short-convolution
// kernel, with prefill and decode-with-state variants of the convolution).
//
// Gate: one wave per token; each lane keeps fp32 partial sums of h.h, k.k and
// h.k over its 16-byte chunks, the wave reduces them in double, and the same
// wave then scales the value half.  Conv: one lane per (token, 8 channels),
// taps read as 16-byte chunks from the token rows t, t-d, ... (re-reads hit
// L2, so HBM sees each row about once), state rows before a request start.
#include "ple_launch.h"

namespace ple {

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

template <int UNROLL>
__global__ __launch_bounds__(256) void gate_kernel(const uint16_t* __restrict__ hidden,
                                                   const uint16_t* __restrict__ kv, int64_t T, int N, float eps,
                                                   uint16_t* __restrict__ out, float* __restrict__ gate) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave; no block-level barrier below
    const int nch = N >> 3;
    const u32x4* __restrict__ h = (const u32x4*)(hidden + t * N);
    const u32x4* __restrict__ k = (const u32x4*)(kv + t * 2 * (int64_t)N);
    const u32x4* __restrict__ v = k + nch;
    u32x4* __restrict__ o = (u32x4*)(out + t * N);

    float hh = 0.f, kk = 0.f, hk = 0.f;
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
    double dhh = hh, dkk = kk, dhk = hk;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        dhh += __shfl_xor(dhh, off, 64);
        dkk += __shfl_xor(dkk, off, 64);
        dhk += __shfl_xor(dhk, off, 64);
    }
    const double n = (double)N;
    const double s = dhk / (sqrt(dhh / n + (double)eps) * sqrt(dkk / n + (double)eps) * sqrt(n));
    const float g = (float)(1.0 / (1.0 + exp(-s)));
    if (lane == 0 && gate != nullptr) gate[t] = g;

    for (int base = lane; base < nch; base += 64 * UNROLL) {
        u32x4 vv[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            if (base + 64 * u < nch) vv[u] = v[base + 64 * u];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int idx = base + 64 * u;
            if (idx < nch) {
                const u32x4 x = vv[u];
                o[idx] = u32x4{pack_bf16x2(g * bf16_lo(x.x), g * bf16_hi(x.x)),
                               pack_bf16x2(g * bf16_lo(x.y), g * bf16_hi(x.y)),
                               pack_bf16x2(g * bf16_lo(x.z), g * bf16_hi(x.z)),
                               pack_bf16x2(g * bf16_lo(x.w), g * bf16_hi(x.w))};
            }
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

// state_out[r][m] = the (S-m)-th most recent conv input of state[r] ++ x[a:b].
__global__ __launch_bounds__(256) void conv_state_out_kernel(const uint16_t* __restrict__ x,
                                                             const int32_t* __restrict__ qsl, int64_t T, int R,
                                                             const uint16_t* __restrict__ state, int N, int S,
                                                             uint16_t* __restrict__ state_out) {
    const int nch = N >> 3;
    const int64_t total = (int64_t)R * S * nch;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
         p += (int64_t)gridDim.x * blockDim.x) {
        const int64_t rm = p / nch;
        const int ch = (int)(p - rm * nch);
        const int r = (int)(rm / S);
        const int m = (int)(rm - (int64_t)r * S);
        int64_t a = qsl[r], b = qsl[r + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        const int64_t q = (b - a) + m;  // index into state[r] ++ x[a:b]
        u32x4 v = {0u, 0u, 0u, 0u};
        if (q >= S)
            v = *(const u32x4*)(x + (a + (q - S)) * N + ch * 8);
        else if (state != nullptr)
            v = *(const u32x4*)(state + ((int64_t)r * S + q) * N + ch * 8);
        *(u32x4*)(state_out + ((int64_t)r * S + m) * N + ch * 8) = v;
    }
}

hipError_t launch_gate(const uint16_t* hidden, const uint16_t* kv, int64_t T, int N, float eps, uint16_t* out,
                       float* gate, hipStream_t s) {
    const int64_t blocks = (T + 3) / 4;
    hipLaunchKernelGGL(gate_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, s, hidden, kv, T, N, eps, out, gate);
    return hipGetLastError();
}

hipError_t launch_conv(const uint16_t* x, const int32_t* qsl, int64_t T, int R, const uint16_t* state,
                       const uint16_t* w, int N, int K, int d, uint16_t* y, hipStream_t s) {
    const int64_t total = T * (N >> 3);
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    dim3 g((unsigned)blocks), b(256);
    switch (K) {
        case 1: hipLaunchKernelGGL(conv_kernel<1>, g, b, 0, s, x, qsl, T, R, state, w, N, K, d, y); break;
        case 2: hipLaunchKernelGGL(conv_kernel<2>, g, b, 0, s, x, qsl, T, R, state, w, N, K, d, y); break;
        case 3: hipLaunchKernelGGL(conv_kernel<3>, g, b, 0, s, x, qsl, T, R, state, w, N, K, d, y); break;
        case 4: hipLaunchKernelGGL(conv_kernel<4>, g, b, 0, s, x, qsl, T, R, state, w, N, K, d, y); break;
        default: hipLaunchKernelGGL(conv_kernel<0>, g, b, 0, s, x, qsl, T, R, state, w, N, K, d, y); break;
    }
    return hipGetLastError();
}

hipError_t launch_conv_state_out(const uint16_t* x, const int32_t* qsl, int64_t T, int R,
                                 const uint16_t* state, int N, int S, uint16_t* state_out, hipStream_t s) {
    const int64_t total = (int64_t)R * S * (N >> 3);
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    hipLaunchKernelGGL(conv_state_out_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, qsl, T, R, state, N, S,
                       state_out);
    return hipGetLastError();
}

}  // namespace ple
