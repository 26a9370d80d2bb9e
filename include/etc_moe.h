/*
 * etc_moe.h -- C ABI of the event-tensor MoE layer and split-K GEMM for AMD MI355X
 * (gfx950).
 *
 * Background.  An event tensor is an array of counters in global memory that encodes
 * the dependencies between tiled tasks of one persistent kernel; a task runs once its
 * counter reaches a target, and with Mixture-of-Experts routing the targets depend on
 * the router's output, so the kernel computes them on the GPU before anyone waits
 * (OpenAlex record of "Event Tensor: A Unified Abstraction for Compiling Dynamic
 * Megakernel", abstract; tutorial chapter "5 · Event Tensor et le dynamisme", §5.3 and
 * §5.5 Obstacle 1).  The batch size is a run-time argument: one compiled kernel serves
 * every token count (podcast episode page "Prompt Boundary-Aware Scheduling with Event
 * Tensors for Dynamic Kernels", summary: symbolic batch-size template; §5.3 of the
 * chapter: one compilation instead of one per batch size).
 *
 * Conventions for every entry point:
 *   - Pointers named device are HIP device pointers owned by the caller; the library
 *     never allocates, frees or keeps them after the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls are
 *     asynchronous: they enqueue one kernel and return; only etc_query_device_status
 *     synchronises the stream.
 *   - Arguments are validated on the host before any HIP call.  On any error other
 *     than ETC_ERR_HIP nothing is enqueued and no output is touched.
 *   - Tensors are dense and row-major; "[a][b]" means b is the contiguous index.
 *   - A workspace belongs to one stream at a time; calls sharing a workspace must be
 *     ordered on that stream.  It must be cleared once with etc_workspace_init after
 *     allocation; the kernel leaves it cleared again when it returns.
 */
#ifndef ETC_MOE_H
#define ETC_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ETC_OK = 0,
  ETC_ERR_INVALID_ARG = 1, /* a pointer, size or enum is out of range */
  ETC_ERR_UNSUPPORTED = 2, /* valid shape the library does not handle (see each call) */
  ETC_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
  ETC_ERR_HIP = 4,         /* a HIP runtime call failed (device state unknown) */
  ETC_ERR_TIMEOUT = 5,     /* device status: a wait saw no progress for 5 s (its limit
                              restarts whenever what it watches changes), the kernel
                              stopped early and its outputs are not valid */
  ETC_ERR_NO_DEVICE = 6    /* no usable gfx950 device is current */
} etc_status;

typedef enum { ETC_DTYPE_F32 = 0, ETC_DTYPE_BF16 = 1 } etc_dtype;

/* Static: every workgroup draws the next ticket of one fixed topological task order
 * and waits on that task's counters.  Dynamic: a ready queue in global memory; the
 * producer whose signal completes a counter enqueues the dependents, and workgroups
 * only ever take ready tasks.  (Episode summary of the podcast page: static suits
 * regular work, dynamic pays off under irregularity such as MoE routing; chapter §5.5
 * Obstacle 3: online balancing through atomics.)  Dedicated (etc_moe_layer only):
 * workgroup 0 is a scheduler that watches the event counters of a window of the
 * static order and hands ready tasks to two-slot mailboxes of the other workgroups,
 * preferring the XCD static mode would use; workers never wait on a counter (chapter,
 * Q&A on the Cluster Launch Control: MPK's scheduler units feeding worker queues).
 * Needs at least two workgroups; uses at most 257 (the scheduler tracks 256 workers). */
typedef enum { ETC_SCHED_STATIC = 0, ETC_SCHED_DYNAMIC = 1, ETC_SCHED_DEDICATED = 2 } etc_sched_mode;

/* Atomic: the down-projection tiles add gate * y straight into a float32 accumulator
 * (order of additions varies run to run).  Ordered: they store y and the finalize
 * task sums the k slots of each token in slot order (bit-reproducible). */
typedef enum { ETC_COMBINE_ATOMIC = 0, ETC_COMBINE_ORDERED = 1 } etc_combine;

/* debug flags */
#define ETC_FLAG_KEEP_COUNTERS 0x1u /* do not clear the event counters on exit, so the
                                       caller can read them (etc_moe_workspace_layout);
                                       call etc_workspace_init before the next call */
#define ETC_FLAG_TRACE 0x2u /* etc_moe_layer: every task appends one 32-byte record to the
                               trace region of the workspace (etc_moe_workspace_layout
                               words 13-14): uint64 task word (kind in bits 0-3: 1 routing,
                               2 scan, 3 gate/up, 4 down, 5 finalize; layer bits 4-7;
                               then 14-bit fields a, b, c, d from bit 8 on), uint64 start
                               of the claim (100 MHz device clock), uint32 workgroup,
                               uint32 ticks spent claiming and waiting, uint32 ticks
                               running, uint32 zero.  The number of records is int32 word
                               10 of the workspace after the call. */
#define ETC_FLAG_ALLOW_DYNAMIC 0x4u /* etc_moe_layer: accept mode ETC_SCHED_DYNAMIC.  Without
                                       this bit the mode returns ETC_ERR_UNSUPPORTED: an early
                                       run of the dynamic MoE scheduler on MI355X did not
                                       terminate and the cause has not been identified, so
                                       the mode runs only where the caller asks for it (the
                                       CPU execution harness).  Split-K ignores the bit. */

/* Weights of one MoE layer (all device pointers).  dtype is the call's dtype except
 * gamma and router_bias, which are always float32.  Layouts follow nn.Linear
 * ([out][in]): w_router [E][H], w_gate [E][F][H], w_up [E][F][H], w_down [E][H][F]. */
typedef struct {
  const float* gamma;       /* [H] RMSNorm scale */
  const void* w_router;     /* [E][H] */
  const float* router_bias; /* [E] or NULL (added to the logits) */
  const void* w_gate;       /* [E][F][H] */
  const void* w_up;         /* [E][F][H] */
  const void* w_down;       /* [E][H][F] */
} etc_moe_weights;

/* Optional routing outputs (device pointers, any may be NULL).  When given, the kernel
 * uses them as its working storage for that array, so they hold the layer's routing
 * after the call. */
typedef struct {
  int32_t* topk_idx;      /* [L][T][k] experts in slot order (largest logit first) */
  float* topk_w;          /* [L][T][k] gate weights (softmax over the k selected) */
  int32_t* expert_counts; /* [L][E] tokens routed to each expert */
  int32_t* sorted_assign; /* [L][T*k] t*k+j grouped by expert, tokens ascending */
} etc_moe_routing;

/*
 * etc_moe_layer -- num_layers chained MoE layers in one persistent kernel.
 *
 * Per layer and token t: xn = RMSNorm(x_t) (float32 math, gamma, eps); logits =
 * xn W_r^T (+ bias) in float32; the top_k experts by logit (ties to the lower index);
 * gates = softmax over the selected logits; per-expert counts, their exclusive scan and
 * the permutation grouping (token, slot) pairs by expert with tokens ascending; for
 * each expert the rows X = dtype(xn) of its tokens go through h = dtype(silu(X W_g^T) *
 * (X W_u^T)) and y = h W_d^T with float32 accumulation; out_t = dtype(sum_j gate_tj *
 * y_tj).  The output of layer l is the input of layer l+1.  (The pages name the MoE
 * routing with data-dependent event counters computed from router outputs -- episode
 * summary of "Prompt Boundary-Aware Scheduling with Event Tensors for Dynamic Kernels"
 * -- but no formula; the readings taken for each stage are those stated here.)
 *
 *   tokens       T, 0 <= T <= max_tokens (T == 0 is a no-op returning ETC_OK)
 *   hidden       H, a multiple of 128
 *   experts      E, 1..256
 *   top_k        k, 1..min(E, 16)
 *   ffn          F, a multiple of 64
 *   num_layers   L, 1..4
 *   dtype        storage type of x, out, layer_out and all weights but gamma/bias
 *   eps          RMSNorm epsilon (> 0 or 0)
 *   weights      host array of L etc_moe_weights
 *   x            device [T][H] layer-0 input
 *   out          device [T][H] output of the last layer
 *   layer_out    device [L-1][T][H] outputs of layers 0..L-2, or NULL (then they live
 *                in the workspace)
 *   routing      optional outputs, or NULL
 *   workspace    device, 256-byte aligned, >= etc_moe_workspace_size(max_tokens, ...)
 *   max_tokens   capacity the workspace was sized for
 *   mode, combine  see the enums
 *   flags        ETC_FLAG_* bits (0 for normal use)
 *   workers      persistent workgroups to launch; 0 = one per resident slot of the
 *                device (CUs x occupancy), larger values are clamped to that
 *   stream       hipStream_t
 * Errors: ETC_ERR_INVALID_ARG (null pointer, size or enum out of range, unaligned
 * pointer -- every tensor pointer must be 16-byte aligned), ETC_ERR_UNSUPPORTED
 * (H % 128, F % 64, E > 256, k > 16, L > 4; and mode ETC_SCHED_DYNAMIC unless flags
 * has ETC_FLAG_ALLOW_DYNAMIC), ETC_ERR_WORKSPACE, ETC_ERR_HIP, ETC_ERR_NO_DEVICE.  Device-side timeouts are
 * reported by etc_query_device_status.
 */
etc_status etc_moe_layer(int32_t tokens, int32_t hidden, int32_t experts, int32_t top_k,
                         int32_t ffn, int32_t num_layers, etc_dtype dtype, float eps,
                         const etc_moe_weights* weights, const void* x, void* out,
                         void* layer_out, const etc_moe_routing* routing, void* workspace,
                         size_t workspace_bytes, int32_t max_tokens, etc_sched_mode mode,
                         etc_combine combine, uint32_t flags, int32_t workers, void* stream);

/* Bytes of workspace etc_moe_layer needs for up to max_tokens tokens (0 on invalid
 * arguments).  The ordered combine needs an extra float32 [max_tokens*k][H] buffer. */
size_t etc_moe_workspace_size(int32_t max_tokens, int32_t hidden, int32_t experts,
                              int32_t top_k, int32_t ffn, int32_t num_layers,
                              etc_dtype dtype, etc_combine combine);

/* Where the event counters of layer `layer` live inside a workspace, as byte offsets
 * from its start, for inspection after a call with ETC_FLAG_KEEP_COUNTERS.  Writes
 * ETC_LAYOUT_WORDS int64 values to out_offsets (host memory):
 *   [0] ev_route (1 int32)   [1] ev_scan (1 int32)   [2] ev_gu ([max_rt][n1] int32)
 *   [3] ev_comb ([n_rt] int32)   [4] ev_done ([n_rt] int32)   [5] plan words (int32)
 *   [6] max_rt   [7] n1   [8] n_rt(max_tokens)   [9] rows per routing tile
 *   [10] rows per expert tile   [11] ffn columns per gate/up tile
 *   [12] hidden columns per down tile   [13] trace region   [14] trace records it holds
 *   [15] ev_perm (1 int32: routing tiles whose pairs are placed in the permutation)
 *   [16] ev_rq ([n_rt] int32: router slices of each routing tile that have reported).
 * The plan words are: [0] row tiles RT, [1] gate/up tasks, [2] down tasks,
 * [3] finalize tasks, [4] ffn chunks of the down projection nS, [5] gate/up tiles per
 * chunk, [6] first static ticket of the next layer, [7] router slices per routing tile
 * Q (the call cuts each tile's router along H into Q tasks when the routing tiles
 * would leave at least half of the workgroups idle; Q = 1 otherwise). */
#define ETC_LAYOUT_WORDS 17
etc_status etc_moe_workspace_layout(int32_t max_tokens, int32_t hidden, int32_t experts,
                                    int32_t top_k, int32_t ffn, int32_t num_layers,
                                    etc_dtype dtype, etc_combine combine, int32_t layer,
                                    int64_t* out_offsets);

/*
 * etc_splitk_gemm -- C = A B with the K range cut into split_k slices.
 *
 * Each (output tile, slice) partial task writes a float32 partial tile and signals the
 * tile's event counter; the tile's reduction runs once that counter reaches split_k
 * and adds the partials in slice order 0..split_k-1 (episode summary of "Prompt
 * Boundary-Aware Scheduling with Event Tensors for Dynamic Kernels": the split-K
 * summation example of fine-grained dependencies).  Static mode puts the reductions
 * after all partials in ticket order; dynamic mode lets the partial task whose signal
 * completes the counter run the reduction.
 *
 *   M, N, K    sizes; M >= 1, N a multiple of 128, K a multiple of 64 * split_k
 *   split_k    1..64
 *   A          device bfloat16 [M][K]
 *   B          device bfloat16 [K][N]
 *   C          device float32 [M][N]
 *   workspace  device, 256-byte aligned, >= etc_splitk_workspace_size(M, N, split_k)
 *   workers    as for etc_moe_layer
 * Errors: ETC_ERR_INVALID_ARG, ETC_ERR_UNSUPPORTED (shape constraints above),
 * ETC_ERR_WORKSPACE, ETC_ERR_HIP, ETC_ERR_NO_DEVICE.
 */
etc_status etc_splitk_gemm(int32_t M, int32_t N, int32_t K, int32_t split_k, const void* A,
                           const void* B, float* C, void* workspace, size_t workspace_bytes,
                           etc_sched_mode mode, uint32_t flags, int32_t workers,
                           void* stream);

size_t etc_splitk_workspace_size(int32_t M, int32_t N, int32_t split_k);

/*
 * etc_decode_attention -- decode attention (one query token per request) over key/value
 * caches of per-request length, in one persistent kernel.
 *
 * For request b with context length L_b, KV head g and query head h = g*group + i:
 * s_t = scale * q[b,h] . K[g][kv_start[b] + t] for t < L_b, out[b,h] = softmax(s) V.  The
 * cache of each request is cut into chunks of 256 tokens; every (request, KV head,
 * chunk) task writes a partial (largest score, sum of exp(s - max), exp-weighted value
 * sum) and adds 1 to the (request, KV head) counter; the head's output is merged once
 * the counter reaches ceil(L_b / 256), a target the kernel computes from the device array
 * of lengths before anyone waits (tutorial chapter "5 · Event Tensor et le dynamisme",
 * §5.1: context length as a source of shape dynamism; §5.5 Obstacle 1: targets computed
 * at run time on the GPU; podcast episode page "Prompt Boundary-Aware Scheduling with
 * Event Tensors for Dynamic Kernels", summary: the split-K summation example).  One
 * compiled kernel serves any mix of lengths.
 *
 *   batch        requests B, 1 <= B <= max_batch
 *   kv_heads     H_kv >= 1
 *   group        query heads per KV head, 1..8 (1: multi-head attention)
 *   head_dim     must be 128
 *   context_lens device int32 [B]: L_b >= 1
 *   kv_start     device int32 [B]: cache row of request b's first token; rows
 *                kv_start[b] .. kv_start[b] + L_b - 1 must lie in [0, kv_rows)
 *   kv_rows      rows of each cache
 *   scale        score scale (typically 1/sqrt(head_dim))
 *   q            device bfloat16 [B][H_kv*group][128]
 *   k_cache, v_cache  device bfloat16 [H_kv][kv_rows][128] (head-major: the rows of one
 *                KV head are contiguous, so a chunk of one request is one contiguous run)
 *   out          device float32 [B][H_kv*group][128]
 *   workspace    device, 256-byte aligned, >= etc_decode_attention_workspace_size(
 *                max_batch, kv_heads, group, head_dim, max_total_tokens)
 *   max_batch, max_total_tokens  the capacity the workspace was sized for: at most
 *                max_batch requests whose lengths sum to at most max_total_tokens
 *   mode         static: partial tickets, then one merge ticket per (request, KV head)
 *                that waits on its counter; dynamic: the partial whose signal completes
 *                the counter merges (last arriver)
 *   flags, workers, stream  as for etc_moe_layer (ETC_FLAG_KEEP_COUNTERS applies)
 * Errors: ETC_ERR_INVALID_ARG (null or misaligned pointer -- q, the caches and out must
 * be 16-byte aligned, the int32 arrays 4-byte aligned --, batch out of range, kv_rows < 1,
 * NaN scale, bad enum), ETC_ERR_UNSUPPORTED (head_dim != 128, group > 8, max_batch >
 * 2048), ETC_ERR_WORKSPACE, ETC_ERR_HIP, ETC_ERR_NO_DEVICE.  The lengths and start rows
 * are device data: a length below 1 or rows outside the cache make the kernel skip all
 * work and leave ETC_ERR_INVALID_ARG in the device status, and lengths summing to more
 * than max_total_tokens leave ETC_ERR_WORKSPACE (etc_query_device_status); out is then
 * not written.
 */
etc_status etc_decode_attention(int32_t batch, int32_t kv_heads, int32_t group, int32_t head_dim,
                                const int32_t* context_lens, const int32_t* kv_start,
                                int32_t kv_rows, float scale, const void* q, const void* k_cache,
                                const void* v_cache, float* out, void* workspace,
                                size_t workspace_bytes, int32_t max_batch, int64_t max_total_tokens,
                                etc_sched_mode mode, uint32_t flags, int32_t workers, void* stream);

/* Bytes of workspace etc_decode_attention needs (0 on invalid arguments). */
size_t etc_decode_attention_workspace_size(int32_t max_batch, int32_t kv_heads, int32_t group,
                                           int32_t head_dim, int64_t max_total_tokens);

/*
 * etc_splitk_gemm_noalloc -- etc_splitk_gemm without a caller workspace and without any
 * allocation, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The partials and counters live in a 16 MiB array in the library's device memory, one
 * per GPU, held until the process ends; calls whose workspace would exceed it
 * (etc_splitk_workspace_size(M, N, split_k) > 16 MiB) return ETC_ERR_WORKSPACE before
 * any HIP call.  Each call first clears the array's control words and counters with a
 * small fill kernel on `stream` (no memset), then runs the same kernel as
 * etc_splitk_gemm, so results are identical.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (different streams without ordering) race and
 * must not be made.  The first call on a device looks up the array's device address
 * (hipGetSymbolAddress); no call allocates.
 *
 *   M, N, K, split_k, A, B, C, mode, flags, workers, stream  as for etc_splitk_gemm
 *   status   device int32 [1] or NULL: the kernel writes its device status there (0, or
 *            ETC_ERR_TIMEOUT); with NULL a device timeout goes unreported
 * Errors: as etc_splitk_gemm, with ETC_ERR_WORKSPACE for shapes beyond the array.
 */
etc_status etc_splitk_gemm_noalloc(int32_t M, int32_t N, int32_t K, int32_t split_k, const void* A,
                                   const void* B, float* C, int32_t* status, etc_sched_mode mode,
                                   uint32_t flags, int32_t workers, void* stream);

/* Clear a freshly allocated workspace (enqueues a memset of all workspace_bytes on
 * `stream`).  Needed once after allocation, and after a call that failed with a
 * device timeout or used ETC_FLAG_KEEP_COUNTERS. */
etc_status etc_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Synchronises `stream`, then returns the device status left in the workspace by the
 * last call: ETC_OK, ETC_ERR_TIMEOUT, or (etc_decode_attention) ETC_ERR_INVALID_ARG or
 * ETC_ERR_WORKSPACE for device-side lengths out of range.  ETC_ERR_HIP if the copy
 * fails.  The status word persists until etc_workspace_init. */
etc_status etc_query_device_status(const void* workspace, void* stream);

/* Human-readable name of a status code (static storage). */
const char* etc_status_string(etc_status status);

/* Persistent workgroups a call would launch on the current device with workers = 0,
 * for the MoE kernel (kind 0, given dtype) or the split-K kernel (kind 1); 0 if no
 * device.  Lets callers size tests; does not launch anything. */
int32_t etc_default_workers(int32_t kind, etc_dtype dtype);

/* ABI version of this header: (major << 16) | minor. */
#define ETC_ABI_VERSION 0x00010002
int32_t etc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ETC_MOE_H */
