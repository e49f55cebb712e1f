/*
 * ple.h - C ABI of libple, the MI355X (gfx950) per-layer n-gram embedding
 * (PLE / Engram) lookup path.
 *
 * The path, per decoder layer, over a ragged batch of requests:
 *   ple_ngram_ids  hash each token's preceding n-grams into per-head table rows
 *   ple_gather     fetch one row per hash head (bf16 copy, or fp8 e4m3fn with a
 *                  per-row fp32 scale dequantised to bf16)
 *   ple_lookup     the two above fused into one kernel (the hot lookup)
 *   ple_kv_proj    merged key/value projection (MFMA GEMM)
 *   ple_gate       sigmoid gate of the RMS-normalised hidden.key product, times value
 *   ple_conv       dilated causal depthwise short convolution
 *   ple_prefill_fused  all of the above in stream order
 *   ple_spec_commit    conv state and n-gram context after speculative verify
 *
 * Sources (page title, then section):
 *   [P1] "PR #54371 [Qwen4Exp] Support UVA PLE-offload and Engram tensor
 *        parallelism": 功能与动机 (tables in pinned host memory read by the GPU
 *        through unified addressing), 关键源码片段 (pinned allocation, side-stream
 *        prefetch returning early on an empty batch).
 *   [P2] "PR #56512 [DS V4.1][Engram] async prefetch for offloaded engram
 *        lookups and engram DP sharding": 功能与动机 and 实现拆解 item 4
 *        (side-stream prefetch into a persistent staging buffer; empty head
 *        shards are rejected).
 *   [P3] "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels": 实现拆解
 *        items 1-2 (ids, gate and conv kernels; merged kv_proj) and 关键源码片段
 *        (compute_ngram_ids and the ids kernel's arguments).
 *   [P4] "Support PLE-Offload for Qwen3.8-Flash-Next - #53899": FP8
 *        (float8_e4m3fn) PLE tables carrying a weight scale.
 *
 * Conventions for every call:
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - "device" pointers are HIP device addresses (hipMalloc, or the device
 *     address of mapped pinned host memory where stated); "host" pointers are
 *     read during the call only.  The caller owns all memory; the library
 *     never allocates or frees on these paths.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     only enqueue work and never synchronise (except the host-memory calls).
 *     Device buffers must stay alive until the enqueued work completes.
 *   - Return value: PLE_OK or an error code; ple_error_message() describes
 *     the last failure on the calling thread.  Argument checks run before any
 *     HIP call, so an invalid call touches no device.  Nothing is thrown
 *     across the ABI.
 *   - Preconditions not checked on the device (violations give unspecified
 *     results, never out-of-bounds table reads): query_start_loc[0] == 0,
 *     non-decreasing, query_start_loc[R] == T; token ids >= 0.
 *   - Tensors are row-major and densely packed; device pointers must be
 *     16-byte aligned.
 */
#ifndef PLE_H
#define PLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PLE_OK 0
#define PLE_ERR_INVALID_ARGUMENT 1
#define PLE_ERR_UNSUPPORTED 2
#define PLE_ERR_DEVICE 3
#define PLE_ERR_WORKSPACE 4

#define PLE_DTYPE_BF16 0
#define PLE_DTYPE_FP8_E4M3 1 /* OCP float8 e4m3fn: bias 7, max 448, NaN 0x7F/0xFF; one fp32 scale per row */
/* float8 e4m3fn codes with one fp32 scale for the whole table ([P4] review
 * thread: an FP8 PLE table with one global weight_scale) */
#define PLE_DTYPE_FP8_E4M3_GLOBAL 2
/* NVFP4 ([P4] walkthrough: NVFP4 embedding support): 4-bit e2m1 codes, two
 * per byte (element 2i in the low nibble of byte i), an e4m3fn scale per
 * 16-element block and one fp32 scale for the whole table */
#define PLE_DTYPE_NVFP4 3

#define PLE_MAX_HEADS 32
#define PLE_MAX_CONTEXT 7
#define PLE_MAX_TOKENS (1 << 24) /* tokens per call */
/* bytes of the library-owned scratch array behind ple_prefill_fused_noalloc (64 MiB per GPU) */
#define PLE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * Hash constants of one layer ([P3] 关键源码片段: layer multipliers, per-head
 * vocabulary sizes and offsets, EOS id, heads per n-gram order).
 * Orders are 2..context_len+1, order-major: global head g has order
 * 2 + g / heads_per_ngram.  This call covers the global heads
 * [first_head, first_head + num_heads) (a head shard; first_head = 0 and
 * num_heads = context_len * heads_per_ngram for the whole layer).
 */
typedef struct ple_hash_desc {
    int32_t num_heads;        /* H, 1..PLE_MAX_HEADS (0 is rejected: empty head shard) */
    int32_t heads_per_ngram;  /* >= 1 */
    int32_t context_len;      /* C = max order - 1, 1..PLE_MAX_CONTEXT */
    int32_t first_head;       /* >= 0, first_head + num_heads <= C * heads_per_ngram */
    int32_t eos_token_id;
    int32_t reserved;
    const int64_t* multipliers; /* host [H][C+1]; entry j of head h used for j < order(h) */
    const int64_t* vocab_sizes; /* host [H]; 1 <= V_h < 2^31 */
    const int64_t* offsets;     /* host [H]; >= 0; offsets[h] + V_h <= table rows and < 2^31 */
} ple_hash_desc;

/*
 * An embedding table of one layer ([P1] 关键源码片段; [P4] FP8 and NVFP4
 * tables).  Every decoded element is one fp32 value rounded once to bf16
 * (nearest, ties to even):
 *   BF16:             the stored bits
 *   FP8_E4M3:         float(e4m3fn(code)) * row_scales[row]        (one fp32 multiply)
 *   FP8_E4M3_GLOBAL:  float(e4m3fn(code)) * row_scales[0]          (one fp32 multiply)
 *   NVFP4:            (e2m1(code) * e4m3fn(block scale)) * row_scales[0]
 *                     (the first product is exact in fp32; one fp32 multiply)
 */
typedef struct ple_table_desc {
    const void* table;        /* device (or mapped host) [num_rows][row bytes]: D bf16, D fp8 codes or D/2 bytes of fp4 codes */
    int64_t num_rows;         /* 1 .. 2^31 */
    int32_t dim;              /* D <= 8192; row bytes a multiple of 16 (NVFP4: D a multiple of 32) */
    int32_t dtype;            /* PLE_DTYPE_* */
    const float* row_scales;  /* FP8_E4M3: [num_rows]; FP8_E4M3_GLOBAL and NVFP4: [1]; NULL for BF16 */
    const uint8_t* block_scales; /* NVFP4: e4m3fn codes [num_rows][D/16]; NULL otherwise */
} ple_table_desc;

/*
 * One ragged batch ([P3] 关键源码片段 compute_ngram_ids: flattened input_ids,
 * query_start_loc with R+1 entries, the carried ngram_context).
 */
typedef struct ple_batch_desc {
    const int32_t* input_ids;        /* device [T] */
    const int32_t* query_start_loc;  /* device [R+1] */
    int64_t num_tokens;              /* 0 <= T <= PLE_MAX_TOKENS */
    int32_t num_reqs;                /* R >= 0 (R == 0 requires T == 0) */
    int32_t max_request_tokens;      /* hint: 0 = unknown; 1..4 = no request has more tokens
                                        (a decode step, a speculative verify window), which lets
                                        ple_prefill_fused run gate, conv and the carried
                                        state/context as one kernel; a wrong hint gives
                                        unspecified results for the requests that break it
                                        (never out-of-bounds accesses) */
    const int32_t* ngram_context;    /* device [R][C], oldest first, or NULL (= all EOS) */
    int32_t* ngram_context_out;      /* device [R][C] or NULL: last C raw tokens of
                                        ngram_context[r] ++ request r's tokens; must not
                                        alias ngram_context */
    const uint16_t* conv_state;      /* device bf16 [R][S][N], oldest first, or NULL (= zeros);
                                        S = (conv_kernel - 1) * conv_dilation */
    uint16_t* conv_state_out;        /* device bf16 [R][S][N] or NULL; must not alias conv_state */
} ple_batch_desc;

/* Everything one layer's fused prefill needs. */
typedef struct ple_layer_desc {
    ple_hash_desc hash;
    ple_table_desc table;
    const uint16_t* kv_weight;   /* device bf16 [2N][H*D]: key rows, then value rows */
    int32_t hidden;              /* N; a multiple of 8 */
    float eps;                   /* RMS epsilon (1e-6 in the reference workloads) */
    const uint16_t* conv_weight; /* device bf16 [N][Kc]; tap Kc-1 multiplies the current token */
    int32_t conv_kernel;         /* Kc, 1..16 */
    int32_t conv_dilation;       /* d >= 1, (Kc-1)*d <= 4096 */
} ple_layer_desc;

/*
 * N-gram IDs ([P3] 实现拆解 item 2, 关键源码片段).  For token t of request r
 * (tokens [a, b) = [qsl[r], qsl[r+1])), shifts j = 0..C:
 *   raw(0) = tok[t]; raw(j) = tok[t-j] if t-j >= a, else ngram_context[r][C-(a-(t-j))],
 *   else EOS.  Once raw(j') == EOS for some 1 <= j' <= j, shift j reads EOS.
 *   ids[t][h] = offsets[h] + floormod(int64(sum_{j<order(h)} s_j * m[h][j] mod 2^64), V_h)
 * ids: device int32 [T][H].  Also writes batch->ngram_context_out when non-NULL
 * (also when T == 0 and R > 0).  batch conv fields are ignored.
 */
int ple_ngram_ids(const ple_hash_desc* hash, const ple_batch_desc* batch, int32_t* ids, void* stream);

/*
 * Row gather ([P1] 关键源码片段, the embedding lookup; [P4] FP8 and NVFP4 tables):
 *   rows[t][h*D + c] = decoded element c of table row ids[t][h], as listed at
 *   ple_table_desc (bf16: bit copy; quantised formats: one fp32 value rounded
 *   to nearest even; NaN codes or NaN scales give 0x7FC0)
 * ids: device int32 [T][H], every id in [0, num_rows) (ids outside are clamped
 * into range, so a bad id never reads outside the table).  rows: device bf16
 * [T][H*D].  table may be mapped pinned host memory (see ple_host_alloc).
 */
int ple_gather(const ple_table_desc* table, const int32_t* ids, int64_t num_tokens, int32_t num_heads,
               uint16_t* rows, void* stream);

/*
 * Fused ids + gather in one kernel: the IDs stay on chip.  rows: device bf16
 * [T][H*D] as in ple_gather; ids_out: device int32 [T][H] or NULL.  Also
 * writes batch->ngram_context_out when non-NULL.
 */
int ple_lookup(const ple_hash_desc* hash, const ple_table_desc* table, const ple_batch_desc* batch,
               int32_t* ids_out, uint16_t* rows, void* stream);

/*
 * Side-stream prefetch of one layer's rows ([P1] 关键源码片段 start_prefetch;
 * [P2] 实现拆解 item 4, persistent staging buffer): ple_lookup with the
 * layer's hash and table, into staging (device bf16 [T][H*D]).  Intended for
 * a second stream; the caller orders the streams with events.  T == 0 returns
 * at once.
 */
int ple_prefetch(const ple_layer_desc* layer, const ple_batch_desc* batch, uint16_t* staging, void* stream);

/*
 * The same staging rows with each distinct table row read once ([P1]
 * 功能与动机: rows cross the host link; [P2] 功能与动机: that read is the
 * time the prefetch hides).  Rows repeated within the batch are copied in
 * device memory from their first read instead of crossing the host link
 * again.  Same result as ple_prefetch, bit for bit.
 * workspace: device memory of ple_prefetch_dedup_workspace_bytes(T, H) bytes,
 * 256-byte aligned (IDs, a hash set, the list of distinct rows and the repeat
 * map; cleared or written before being read).  num_unique: device int32 receiving the number of distinct rows
 * (the rows read from the table), or NULL.  T*H at most 2^22
 * (PLE_ERR_UNSUPPORTED beyond; the size function then returns 0).
 */
int ple_prefetch_dedup(const ple_layer_desc* layer, const ple_batch_desc* batch, uint16_t* staging,
                       void* workspace, size_t workspace_bytes, int32_t* num_unique, void* stream);
size_t ple_prefetch_dedup_workspace_bytes(int64_t max_tokens, int32_t num_heads);

/*
 * ple_prefetch_dedup in two calls, the first then the second on one stream
 * ([P2] 功能与动机: the prefetch hides the host-link read behind the layer's
 * work).  A caller that overlaps the prefetch with other kernels can plan the
 * next layer while the current fetch runs, so that the plan's short launches
 * do not queue behind those kernels.
 * ple_prefetch_dedup_plan: the row IDs of every (token, head), the hash set of
 *   distinct IDs and the list of their first positions, into workspace (as
 *   for ple_prefetch_dedup, sized by ple_prefetch_dedup_workspace_bytes);
 *   also writes batch->ngram_context_out when given.  No staging.
 * ple_prefetch_dedup_fetch: reads the listed rows from the table into
 *   staging (device bf16 [T][H*D]) and copies each repeated row from its first
 *   read; num_unique as for ple_prefetch_dedup.  It takes the same layer
 *   table and num_heads, num_tokens = the plan's batch->num_tokens, and the
 *   workspace the plan filled, unchanged in between; the caller orders the
 *   fetch after the plan (same stream, or an event).
 * Errors as for ple_prefetch_dedup; T == 0 launches nothing except the
 * context output (plan) and the zero count (fetch with num_unique).
 */
int ple_prefetch_dedup_plan(const ple_layer_desc* layer, const ple_batch_desc* batch, void* workspace,
                            size_t workspace_bytes, void* stream);
int ple_prefetch_dedup_fetch(const ple_layer_desc* layer, int64_t num_tokens, void* workspace,
                             size_t workspace_bytes, uint16_t* staging, int32_t* num_unique, void* stream);

/*
 * Merged key/value projection ([P3] 实现拆解 item 1):
 *   kv[t][o] = bf16(sum_i x[t][i] * w[o][i]), fp32 accumulation, no bias.
 * x: device bf16 [T][K]; w: device bf16 [O][K]; kv: device bf16 [T][O].
 * K a multiple of 64 and at most 2^20, O a multiple of 16, T <= PLE_MAX_TOKENS
 * and ceil(T/128) * ceil(O/128) <= 2^24 (else PLE_ERR_UNSUPPORTED).
 */
int ple_kv_proj(const uint16_t* x, const uint16_t* w, int64_t num_tokens, int32_t k_dim, int32_t out_dim,
                uint16_t* kv, void* stream);

/*
 * Gate ([P3] 实现拆解 item 2, PLE gating and normalisation).  Per token, with
 * h = hidden[t], k = kv[t][0:N], v = kv[t][N:2N]:
 *   s = <h,k> / (sqrt(mean(h^2)+eps) * sqrt(mean(k^2)+eps) * sqrt(N)),
 *   g = 1/(1+exp(-s)),  out[t][c] = bf16(g * v[c]),  gate[t] = g (fp32).
 * hidden: device bf16 [T][N]; kv: device bf16 [T][2N]; out: device bf16 [T][N];
 * gate: device fp32 [T] or NULL.  N a multiple of 8.
 */
int ple_gate(const uint16_t* hidden, const uint16_t* kv, int64_t num_tokens, int32_t n, float eps,
             uint16_t* out, float* gate, void* stream);

/*
 * Dilated causal depthwise short convolution ([P3] 实现拆解 item 2):
 *   y[t][c] = bf16(sum_{i<Kc} w[c][Kc-1-i] * x~(t - i*d, c)),
 *   x~(p, c) = x[p][c] if p >= a (start of t's request), else
 *              conv_state[r][S-(a-p)][c] if given, else 0.
 * Uses batch->query_start_loc, num_tokens, num_reqs, conv_state and
 * conv_state_out (the last S inputs of conv_state[r] ++ x[a:b], written also
 * when T == 0 and R > 0).  x, y: device bf16 [T][N]; w: device bf16 [N][Kc].
 * y must not alias x.  N a multiple of 8.
 */
int ple_conv(const uint16_t* x, const ple_batch_desc* batch, const uint16_t* w, int32_t n, int32_t kernel,
             int32_t dilation, uint16_t* y, void* stream);

/*
 * Whole per-layer path in stream order: lookup (or the rows already staged by
 * ple_prefetch when prefetched_rows != NULL) -> kv_proj -> gate -> conv.
 * hidden: device bf16 [T][N]; out: device bf16 [T][N]; gate: device fp32 [T]
 * or NULL; workspace: device memory of at least
 * ple_prefill_workspace_bytes(layer, T) bytes, 256-byte aligned (holds rows,
 * kv and the gated value between kernels; not read before being written).
 * The conv input of token t (the gated value g * v rounded to bf16, N
 * values) is formed inside the conv; on return the conv inputs of each
 * request's last S tokens (S = (Kc-1)*d), and of every token of a request
 * of at most max(S, 16) tokens (every token when the decode tail below runs),
 * stay in the workspace as rows t of a bf16 [T][N] region at byte offset
 * round256(T*H*D*2) + round256(T*2N*2), where round256 rounds up to a
 * multiple of 256 and T = batch->num_tokens; the other rows of the region
 * are unspecified.  A speculative verify step whose windows hold at most
 * max(S, 16) tokens and that keeps one workspace per layer passes that
 * region as x to ple_spec_commit.
 * With batch->max_request_tokens in 1..4 (a decode step or speculative
 * verify windows: no request has more tokens), Kc <= 4 and N <= 8192, gate,
 * conv and the carried state and context run as one kernel ([P3] 实现拆解
 * items 2, 4 and 5: the decode and speculative conv paths with the state
 * kept by the short-conv backend); every output, the conv input in the
 * workspace included, is the same bits as without the hint.
 */
int ple_prefill_fused(const ple_layer_desc* layer, const ple_batch_desc* batch, const uint16_t* hidden,
                      const uint16_t* prefetched_rows, uint16_t* out, float* gate, void* workspace,
                      size_t workspace_bytes, void* stream);
size_t ple_prefill_workspace_bytes(const ple_layer_desc* layer, int64_t max_tokens);

/*
 * ple_prefill_fused for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same launches and the same results, bit for bit, as
 * ple_prefill_fused with the same arguments, but the intermediates (rows, kv,
 * conv input) go to a scratch array the library owns: PLE_NOALLOC_SCRATCH_BYTES
 * (64 MiB) of device memory on each GPU the library runs on, held from the
 * time the library's code is loaded on that GPU until the process ends.  This
 * call allocates and frees nothing.
 * Limit: ple_prefill_workspace_bytes(layer, T) <= PLE_NOALLOC_SCRATCH_BYTES
 * (for H*D = N = 4096, up to 2047 tokens; for H*D = N = 2048, up to 4095),
 * else PLE_ERR_WORKSPACE before any device work.
 * Every call on one GPU shares that GPU's array and leaves it holding its own
 * intermediates: calls whose work overlaps on one GPU (other streams, other
 * host threads) race and give unspecified results; order them on one stream.
 * The conv input is not handed back (use ple_prefill_fused with a workspace
 * to read it, e.g. for ple_spec_commit).
 */
int ple_prefill_fused_noalloc(const ple_layer_desc* layer, const ple_batch_desc* batch, const uint16_t* hidden,
                              const uint16_t* prefetched_rows, uint16_t* out, float* gate, void* stream);

/*
 * Pinned host memory the GPU reads directly ([P1] 功能与动机 and 关键源码片段,
 * a table allocated page-locked and read through unified addressing).
 * ple_host_alloc: page-locked, mapped, portable allocation of `bytes`;
 * *host receives the host address and *device the address kernels use (the
 * same value on this platform).  Synchronous.  ple_host_free releases it.
 */
int ple_host_alloc(size_t bytes, void** host, void** device);
int ple_host_free(void* host);

/*
 * A stream restricted to the first num_cus compute units of the current
 * device, for running the prefetch beside the main stream ([P2] 实现拆解
 * item 4 launches the lookup on a side stream with half the grid).  Default
 * priority.  Like any stream created without the non-blocking flag it
 * synchronises with the legacy null stream: run the overlapped main work on a
 * non-blocking stream.  ple_stream_destroy releases it.
 */
int ple_stream_create_cu_masked(int32_t num_cus, void** stream);
int ple_stream_destroy(void* stream);

/*
 * The one-GPU part of a table sharded across data-parallel replicas ([P1]
 * 实现拆解 item 3 and 关键源码片段 _get_dp_gather_slot: IDs of every replica
 * gathered into equal padded slots, then each replica selects its own token
 * window; [P2] 实现拆解 items 3-4: heads sharded in TP-major order so the
 * gathered shards concatenate in head order, and a kernel that takes a
 * rank's token window out of the rank-major gathered buffer).  The
 * collectives themselves are the caller's.
 *
 * ple_dp_gather_slot: slot = max(token_counts[g0 .. g0+group_size)) and
 * offset = (dp_rank - g0) * slot for the group g0 = dp_rank - dp_rank % group_size
 * that contains dp_rank (group_size 1: slot = token_counts[dp_rank], offset 0).
 * Host-only, synchronous.  token_counts: host [dp_size].
 */
int ple_dp_gather_slot(const int64_t* token_counts, int32_t dp_size, int32_t group_size, int32_t dp_rank,
                       int64_t* slot, int64_t* offset);

/*
 * ple_head_shard: heads of shard s = tp_rank * dp_size + dp_rank (TP-major)
 * out of num_heads split evenly over tp_size * dp_size shards:
 * [s * num_heads / shards, (s + 1) * num_heads / shards).  An uneven split
 * or an empty shard is rejected (PLE_ERR_UNSUPPORTED).  Host-only.
 */
int ple_head_shard(int32_t num_heads, int32_t tp_size, int32_t tp_rank, int32_t dp_size, int32_t dp_rank,
                   int32_t* first_head, int32_t* shard_heads);

/*
 * ple_select_rows: this rank's token window out of a rank-major gathered
 * buffer: gathered is device bf16 [num_shards][num_shards * slot][width]
 * (shard k's lookup of every rank's padded slot, rank r's tokens at rows
 * r*slot .. r*slot+slot-1); out is device bf16 [num_tokens][num_shards * width]
 * with out[t][k*width + c] = gathered[k][rank*slot + t][c] for
 * t < num_tokens <= slot.  width a multiple of 8; 16-byte aligned pointers.
 */
int ple_select_rows(const uint16_t* gathered, int32_t num_shards, int64_t slot, int32_t rank, int64_t num_tokens,
                    int32_t width, uint16_t* out, void* stream);

/*
 * Speculative decode commit ([P3] 实现拆解 items 4-5: the conv's speculative
 * variant and the state the short-conv backend carries between steps).  A
 * verify step runs ple_ngram_ids / ple_conv over each request's whole
 * candidate window [a, b) = [qsl[r], qsl[r+1]) (token 0 is the last accepted
 * token, the rest are drafts); afterwards only the first accepted[r] of them
 * are kept.  This call writes the state the next step starts from as if only
 * those had been run, so rejected drafts leave no trace:
 *   conv_state_out[r]    = last S rows of conv_state[r] ++ x[a : a+acc_r]
 *   ngram_context_out[r] = last C tokens of ngram_context[r] ++
 *                          input_ids[a : a+acc_r]
 * with acc_r = accepted[r] clamped to 0..b-a (conv_state / ngram_context NULL
 * read as zeros / EOS, as in ple_conv and ple_ngram_ids).  accepted: device
 * int32 [R], read on the device, so out-of-range counts are clamped rather than
 * reported.  x: the conv input of the verify step, device bf16 [T][N] (may be
 * NULL when batch->conv_state_out is NULL).  hash supplies C and EOS (may be
 * NULL when batch->ngram_context_out is NULL).  Either output may be NULL; the
 * input states are only read.  S = (conv_kernel - 1) * conv_dilation.
 */
int ple_spec_commit(const ple_hash_desc* hash, const ple_batch_desc* batch, const int32_t* accepted,
                    const uint16_t* x, int32_t n, int32_t conv_kernel, int32_t conv_dilation, void* stream);

/* Message for the last failure on the calling thread ("" if none). */
const char* ple_error_message(void);
/* Library version string. */
const char* ple_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PLE_H */
