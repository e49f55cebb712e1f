// Device-side helpers shared by the libple kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ple.h"

namespace ple {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Per-call hash constants, passed by value as a kernel argument so that calls
// on different streams (a prefetch for the next layer beside the current one)
// never share mutable state.  One 64-byte record per head holds what every
// order up to 4 needs (kernels stage the records of 16 heads with one 16-byte
// load per lane); the multipliers of shifts 4..7 sit apart.
struct alignas(16) HeadHash {
    uint64_t mult[4];   // multiplier of shift j < 4; zero for j >= the head's order
    uint64_t barrett;   // floor((2^64 - 1) / V_h)
    uint32_t vocab;     // V_h < 2^31
    uint32_t wrap_mod;  // 2^64 mod V_h
    uint32_t offset;    // offsets[h]
    uint32_t order;     // n-gram order of head h (2..C+1)
    uint64_t pad;
};
static_assert(sizeof(HeadHash) == 64, "HeadHash is four 16-byte chunks");

struct HashParams {
    HeadHash head[PLE_MAX_HEADS];
    uint64_t mult_hi[PLE_MAX_HEADS][PLE_MAX_CONTEXT + 1 - 4];  // shifts 4..7 (context_len >= 4 only)
    int32_t num_heads;
    int32_t context_len;
    int32_t eos;
    int32_t pad;
};

// bf16 <-> fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// Same, with any NaN mapped to the canonical quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t pack_bf16x2_canon(float lo, float hi) {
    uint32_t w = pack_bf16x2(lo, hi);
    if (lo != lo) w = (w & 0xFFFF0000u) | 0x7FC0u;
    if (hi != hi) w = (w & 0x0000FFFFu) | 0x7FC00000u;
    return w;
}

// Largest r in [0, R-1] with qsl[r] <= t (the request owning token t for a
// valid qsl; an in-range index for any qsl).  R >= 1.
__device__ __forceinline__ int find_request(const int32_t* __restrict__ qsl, int R, int64_t t) {
    int lo = 0, hi = R - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if ((int64_t)qsl[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// floor((x * m) / 2^64) for 64-bit unsigned x, m.
__device__ __forceinline__ uint64_t mulhi64(uint64_t x, uint64_t m) { return __umul64hi(x, m); }

// Signed floor modulo of the wrapped 64-bit sum `acc` (read as int64) by V:
//   acc <  2^63:  acc mod V
//   acc >= 2^63:  (acc - 2^64) mod V = (acc mod V - 2^64 mod V) mod V
// acc mod V by Barrett reduction with b = floor((2^64-1)/V): the quotient
// estimate is short by at most 2, so two conditional subtractions finish it.
__device__ __forceinline__ uint32_t floor_mod_wrapped(uint64_t acc, uint32_t V, uint64_t b, uint32_t wrap) {
    uint64_t q = mulhi64(acc, b);
    uint64_t r = acc - q * (uint64_t)V;
    if (r >= V) r -= V;
    if (r >= V) r -= V;
    uint32_t rr = (uint32_t)r;
    if ((int64_t)acc < 0) rr = rr >= wrap ? rr - wrap : rr + (V - wrap);
    return rr;
}

// query_start_loc entries a wave holds for finding requests: entry
// 1 + c*64 + lane in q[c] (all of qsl[0..R] in lane order when R + 1 <= 64,
// then q[0] = qsl[lane]).  Loading is split from the search so that callers
// can put these loads in flight together with their other first loads.
struct QslProbe {
    int q[16];
};

__device__ __forceinline__ void qsl_probe_load(const int32_t* __restrict__ qsl, int R, int lane, QslProbe& p) {
    if (R + 1 <= kWave) {
        p.q[0] = lane <= R ? qsl[lane] : 0;
    } else if (R <= 16 * kWave) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int idx = 1 + c * kWave + lane;
            p.q[c] = (idx <= R) ? qsl[idx] : 0;
        }
    }
}

// Request index r and clamped start a of token t (this lane's token, the
// k-th of the wave's `ntok` consecutive tokens starting at t_first), from the
// entries qsl_probe_load fetched: the wave counts the entries <= each token
// with ballots, so finding the request costs the one round trip of the probe
// instead of a chain of dependent binary-search loads (more than 1024
// requests fall back to a binary search).  Every lane of the wave must call
// this.
__device__ __forceinline__ void wave_find_request_probed(const int32_t* __restrict__ qsl, const QslProbe& p, int R,
                                                         int64_t t, int64_t t_first, int ntok, int my_k, int lane,
                                                         int& r_out, int64_t& a_out) {
    int r;
    int64_t a;
    if (R + 1 <= kWave) {
        const int q = p.q[0];
        r = 0;
        for (int k = 0; k < ntok; ++k) {
            const int64_t tk = t_first + k;
            const uint64_t m = __ballot(lane >= 1 && lane <= R && (int64_t)q <= tk);
            const int rk = (int)__popcll(m);
            if (k == my_k) r = rk < R - 1 ? rk : R - 1;
        }
        a = __shfl(q, r, kWave);
    } else if (R <= 16 * kWave) {
        int cnt = 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int idx = 1 + c * kWave + lane;
            if (1 + c * kWave <= R) {  // wave-uniform
                for (int k = 0; k < ntok; ++k) {
                    const uint64_t m = __ballot(idx <= R && (int64_t)p.q[c] <= t_first + k);
                    if (k == my_k) cnt += (int)__popcll(m);
                }
            }
        }
        r = cnt < R - 1 ? cnt : R - 1;
        a = qsl[r];
    } else {
        r = find_request(qsl, R, t);
        a = qsl[r];
    }
    r_out = r;
    a_out = a < 0 ? 0 : (a > t ? t : a);  // keeps every read in bounds for any qsl
}

__device__ __forceinline__ void wave_find_request(const int32_t* __restrict__ qsl, int R, int64_t t,
                                                  int64_t t_first, int ntok, int my_k, int lane, int& r_out,
                                                  int64_t& a_out) {
    QslProbe p;
    qsl_probe_load(qsl, R, lane, p);
    wave_find_request_probed(qsl, p, R, t, t_first, ntok, my_k, lane, r_out, a_out);
}

// Tokens of request r that the carried state and context take in: [a, b) =
// [qsl[r], qsl[r+1]) clamped to [0, T]; with accepted (speculative decode) only
// the first accepted[r] of them.
__device__ __forceinline__ void carried_window(const int32_t* __restrict__ qsl, int64_t T, int r,
                                               const int32_t* __restrict__ accepted, int64_t& a, int64_t& b) {
    a = qsl[r];
    b = qsl[r + 1];
    a = a < 0 ? 0 : (a > T ? T : a);
    b = b < a ? a : (b > T ? T : b);
    if (accepted != nullptr) {
        const int64_t acc = accepted[r];
        b = acc <= 0 ? a : (a + acc < b ? a + acc : b);
    }
}

// One wave writes carried conv state row m of request r: row (b-a)+m of
// state[r] ++ x[a:b] (state NULL reads as zeros), N bf16 in 16-byte chunks,
// lane-contiguous, four chunks in flight per lane.
__device__ __forceinline__ void carry_state_row(const uint16_t* __restrict__ x, const uint16_t* __restrict__ state,
                                                int N, int S, int r, int m, int64_t a, int64_t b,
                                                uint16_t* __restrict__ state_out, int lane) {
    const int64_t q = (b - a) + m;
    const uint16_t* src = q >= S ? x + (a + (q - S)) * N
                                 : (state != nullptr ? state + ((int64_t)r * S + q) * N : nullptr);
    uint16_t* dst = state_out + ((int64_t)r * S + m) * N;
    const int nch = N >> 3;
    for (int c0 = 0; c0 < nch; c0 += 4 * kWave) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ch = c0 + u * kWave + lane;
            v[u] = u32x4{0u, 0u, 0u, 0u};
            if (src != nullptr && ch < nch) v[u] = *(const u32x4*)(src + ch * 8);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ch = c0 + u * kWave + lane;
            if (ch < nch) *(u32x4*)(dst + ch * 8) = v[u];
        }
    }
}

// Carried context entry i of request r: the (C-i)-th most recent raw token
// of ctx[r] ++ tok[a:b] (ctx NULL reads as EOS).
__device__ __forceinline__ int32_t carried_token(const int32_t* __restrict__ tok, const int32_t* __restrict__ ctx,
                                                 int C, int32_t eos, int r, int i, int64_t a, int64_t b) {
    const int64_t q = (b - a) + i;
    if (q >= C) return tok[a + (q - C)];
    return ctx != nullptr ? ctx[(int64_t)r * C + q] : eos;
}

}  // namespace ple
