// Internal launch interface between the C ABI (ple_api.cpp) and the kernels.
#pragma once

#include "ple_device.h"

namespace ple {

// How the lookup kernel gets its row IDs: hashed from the tokens, read from
// caller IDs [T][H], or (list) for k below a device-side count, row
// ids_in[list[k]] (or, with rep, row rep[ids_in[list[k]]]) written to output
// row list[k] (the distinct rows of the deduplicating prefetch, then its
// repeats copied within the output)
enum { kModeHash = 0, kModeIds = 1, kModeList = 2 };

struct LookupArgs {
    const int32_t* tok;
    const int32_t* qsl;
    const int32_t* ctx;
    const int32_t* ids_in;
    const int32_t* list;        // list mode: positions into ids_in / output rows
    const int32_t* list_count;  // list mode: device count of list entries (at most num_tokens)
    const int32_t* rep;         // list mode, optional: row = rep[ids_in[...]], rep has rep_len entries
    int64_t rep_len;
    int32_t* count_out;         // list mode, optional: receives *list_count
    int32_t* ids_out;
    const void* table;
    const float* scales;          // fp8: per-row scales (scale_stride 1) or one scale (0); NVFP4: one scale
    const uint8_t* block_scales;  // NVFP4: e4m3fn code per 16 elements, [num_rows][dim/16]
    uint16_t* rows;
    int64_t num_tokens;
    int64_t num_rows;
    int32_t num_reqs;
    int32_t num_heads;
    int32_t dim;
    int32_t tokens_per_wave;
    int32_t cpr_log2;      // log2(16-byte output chunks per row), or -1
    int32_t scale_stride;  // fp8: 1 for one scale per row, 0 for one scale for the table
};

// kernel-side table formats (the fp8 per-row and global-scale tables share one kernel)
enum { kFmtBF16 = 0, kFmtFP8 = 1, kFmtNVFP4 = 3 };

// IDs [T][H]; extra blocks of the same launch set clear[0 .. clear_n) to -1
// and zero[0 .. zero_n) to 0 when those are non-NULL (zero_n at most 64).
hipError_t launch_ngram_ids(const HashParams& hp, const int32_t* tok, const int32_t* qsl, int64_t T, int R,
                            const int32_t* ctx, int32_t* ids, hipStream_t s, int32_t* clear = nullptr,
                            int64_t clear_n = 0, int32_t* zero = nullptr, int zero_n = 0);
hipError_t launch_context_out(const int32_t* tok, const int32_t* qsl, int64_t T, int R, int C, int32_t eos,
                              const int32_t* ctx, int32_t* ctx_out, hipStream_t s);
int lookup_tokens_per_wave(int H, int chunks_per_row, int dtype, int64_t num_tokens);
hipError_t launch_lookup(const HashParams& hp, const LookupArgs& g, int dtype, int mode, hipStream_t s);

// Distinct rows of ids [n] (keys and counts cleared beforehand): slot_of[i]
// = the hash-set slot of position i's ID, rep[slot] = the position whose row
// fills it, list[0 .. counts[0]) = those positions (one per distinct ID),
// repeats[0 .. counts[1]) = every other position.
hipError_t launch_dedup_insert(const int32_t* ids, int64_t n, int32_t* keys, int32_t* rep, int log2cap,
                               int32_t* slot_of, int32_t* list, int32_t* repeats, int32_t* counts, hipStream_t s);
// *num_unique = *count (0 when count is NULL), one thread.
hipError_t launch_dedup_count(const int32_t* count, int32_t* num_unique, hipStream_t s);

hipError_t launch_select_rows(const uint16_t* gathered, int E, int64_t slot, int rank, int64_t n, int width,
                              uint16_t* out, hipStream_t s);

// Device address of the current device's copy of the library's scratch array
// (PLE_NOALLOC_SCRATCH_BYTES, 256-byte aligned), looked up once per device.
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_kv_proj(const uint16_t* x, const uint16_t* w, int64_t M, int K, int O, uint16_t* kv,
                          hipStream_t s);

// Gate, conv and carried state/context for batches of at most a few tokens
// per request (decode, speculative verify windows), one launch; K = conv
// kernel size (decode_tail_supported).
struct DecodeTailArgs {
    const uint16_t* hidden;  // [T][N]
    const uint16_t* kv;      // [T][2N]
    const int32_t* qsl;      // [R+1]
    const int32_t* tok;      // [T]
    int64_t T;
    int32_t R;
    int32_t N;
    float eps;
    int32_t d;               // conv dilation
    const uint16_t* conv_w;  // [N][K]
    const uint16_t* state;   // [R][S][N] or NULL
    uint16_t* state_out;     // [R][S][N] or NULL
    const int32_t* ctx;      // [R][C] or NULL
    int32_t* ctx_out;        // [R][C] or NULL
    int32_t C;
    int32_t eos;
    uint16_t* gated;         // [T][N], the conv input
    uint16_t* y;             // [T][N]
    float* gate;             // [T] or NULL
};
bool decode_tail_supported(int max_request_tokens, int K, int N);
hipError_t launch_decode_tail(const DecodeTailArgs& a, int K, hipStream_t s);

hipError_t launch_gate(const uint16_t* hidden, const uint16_t* kv, int64_t T, int N, float eps, uint16_t* out,
                       float* gate, hipStream_t s);
// The gate alone: g[t] (and gate[t] when non-NULL), same arithmetic as launch_gate.
hipError_t launch_gate_only(const uint16_t* hidden, const uint16_t* kv, int64_t T, int N, float eps, float* g,
                            float* gate, hipStream_t s);

// Row-wise convolution (kernel sizes 1-4, N * K * 2 <= 64 KiB of weights):
// conv input of token p = x + p * x_stride (elements), or, gated,
// bf16(g[p] * x[p]) with the gate's arithmetic.
constexpr int kConvInputWindow = 16;  // requests this short keep every conv input (verify windows)
struct ConvRowsArgs {
    const uint16_t* x;
    int64_t x_stride;
    const float* g;          // [T], gated only
    const int32_t* qsl;
    int64_t T;
    int32_t R;
    const uint16_t* state;   // [R][S][N] or NULL
    const uint16_t* w;       // [N][K]
    int32_t N;
    int32_t d;
    uint16_t* y;             // [T][N]
    uint16_t* gated_out;     // gated only, [T][N] or NULL: conv inputs of each request's last S tokens and
                             // of every token of a request of at most kConvInputWindow tokens
};
bool conv_rows_supported(int K, int N);
hipError_t launch_conv_gated(const ConvRowsArgs& a, int K, hipStream_t s);
hipError_t launch_conv(const uint16_t* x, const int32_t* qsl, int64_t T, int R, const uint16_t* state,
                       const uint16_t* w, int N, int K, int d, uint16_t* y, hipStream_t s);
hipError_t launch_conv_state_out(const uint16_t* x, const int32_t* qsl, int64_t T, int R,
                                 const uint16_t* state, int N, int S, uint16_t* state_out, hipStream_t s);

// Carried conv state (state_out non-NULL, S > 0) and n-gram context (ctx_out
// non-NULL, C > 0) in one launch: over each request's whole window, or with
// accepted (speculative decode) over its first accepted[r] tokens.
hipError_t launch_spec_commit(const int32_t* tok, const uint16_t* x, const int32_t* qsl, int64_t T, int R,
                              const int32_t* accepted, const uint16_t* state, int N, int S, uint16_t* state_out,
                              const int32_t* ctx, int C, int32_t eos, int32_t* ctx_out, hipStream_t s);

}  // namespace ple
