// Speculative decode commit ("Fuse Qwen4Exp PLE kernels", 实现拆解 items 4-5:
// the short conv's speculative variant and the state the short-conv backend
// carries between steps).
//
// A verify step runs each request's candidate window [a, b) through the ids
// and conv kernels; once the drafts are checked only the first accepted[r]
// tokens stay.  This kernel writes the conv state and n-gram context the next
// step starts from, as if only those tokens had been run: the same carried
// rows as the plain state update, over the window cut to the accepted prefix.
//
// With accepted NULL the same kernel is the plain state update of a step (the
// fused path uses it so that context and conv state cost one launch).
//
// One launch does both parts: wave w < R*S copies state row (w / S, w % S)
// (one HBM read and one write per 16-byte chunk); the waves after it write
// the context, one entry per lane.  Every wave has a fixed amount of work and
// exits; the grid strides over the waves.
#include "ple_device.h"
#include "ple_launch.h"

namespace ple {

__global__ __launch_bounds__(256) void spec_commit_kernel(const int32_t* __restrict__ tok,
                                                          const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ qsl, int64_t T, int R,
                                                          const int32_t* __restrict__ accepted,
                                                          const uint16_t* __restrict__ state, int N, int S,
                                                          uint16_t* __restrict__ state_out,
                                                          const int32_t* __restrict__ ctx, int C, int32_t eos,
                                                          int32_t* __restrict__ ctx_out, int64_t state_waves,
                                                          int64_t total_waves) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    for (int64_t w = (int64_t)blockIdx.x * wpb + threadIdx.x / kWave; w < total_waves;
         w += (int64_t)gridDim.x * wpb) {
        if (w < state_waves) {
            const int r = (int)(w / S);
            const int m = (int)(w - (int64_t)r * S);
            int64_t a, b;
            carried_window(qsl, T, r, accepted, a, b);
            carry_state_row(x, state, N, S, r, m, a, b, state_out, lane);
        } else {
            const int64_t p = (w - state_waves) * kWave + lane;
            if (p < (int64_t)R * C) {
                const int r = (int)(p / C);
                const int i = (int)(p - (int64_t)r * C);
                int64_t a, b;
                carried_window(qsl, T, r, accepted, a, b);
                ctx_out[p] = carried_token(tok, ctx, C, eos, r, i, a, b);
            }
        }
    }
}

hipError_t launch_spec_commit(const int32_t* tok, const uint16_t* x, const int32_t* qsl, int64_t T, int R,
                              const int32_t* accepted, const uint16_t* state, int N, int S, uint16_t* state_out,
                              const int32_t* ctx, int C, int32_t eos, int32_t* ctx_out, hipStream_t s) {
    const int64_t state_waves = (state_out != nullptr && S > 0) ? (int64_t)R * S : 0;
    const int64_t ctx_waves = (ctx_out != nullptr && C > 0) ? ((int64_t)R * C + kWave - 1) / kWave : 0;
    const int64_t total = state_waves + ctx_waves;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(spec_commit_kernel, dim3((unsigned)blocks), dim3(256), 0, s, tok, x, qsl, T, R, accepted,
                       state, N, S, state_out, ctx, C, eos, ctx_out, state_waves, total);
    return hipGetLastError();
}

}  // namespace ple
