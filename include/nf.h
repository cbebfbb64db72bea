/*
 * nf.h -- C ABI of the nano-batched decoder-layer step for MI355X (gfx950).
 *
 * What the library computes.  One step of a Llama-family pre-norm decoder
 * layer over a batch that mixes decode tokens with a chunk of prefill tokens:
 *   h = RMSNorm(x) * g_attn; [q|k|v] = h W_qkv^T; rotary embedding on q, k;
 *   k, v appended to a paged KV cache; causal GQA attention over the cache;
 *   x1 = x + attn W_o^T; h2 = RMSNorm(x1) * g_ffn;
 *   out = x1 + SwiGLU-FFN(h2)        (dense), or
 *   out = x1 + sum_{e in top-k} w_e SwiGLU-FFN_e(h2)   (mixture of experts).
 * The batch may be split into nano-batches, each operation duplicated per
 * nano-batch, so that the compute-bound GEMMs of one nano-batch run while the
 * memory-bound attention of another runs on a separate partition of the
 * device's compute units (nano-batching and the device-level pipeline with
 * execution-unit scheduling: "How it works" on the bytedragons Nanoflow page;
 * README "Introduction" and "Abstract" on the ossradar Nanoflow page).  The
 * plan -- nano-batch count, sizes, operation order and resource split -- is
 * the four-dimensional search point of the "Search Space 4D" card on the
 * do-not-panic "NanoFlow and the Future of LLM Serving" page.  Splitting
 * never changes the result: rows are independent.
 *
 * The host forms the batch and owns the page tables (asynchronous CPU
 * control flow, README "Introduction"); the device runs the step.
 *
 * Conventions.
 *  - Every call returns nf_status; on failure nf_last_error() (thread-local)
 *    holds a message.  No exception crosses the ABI.
 *  - "device" pointers are HIP device allocations on the layer's device;
 *    "host" pointers are ordinary CPU memory read before the call returns.
 *  - Streams are hipStream_t passed as void* (NULL = the null stream).
 *  - Weights, the KV pool and activations are caller-owned; the library owns
 *    only its streams, events, workspace, metadata buffers and cos/sin table.
 *  - All argument validation happens before anything is launched.
 */
#ifndef NF_H
#define NF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nf_status {
  NF_OK = 0,
  NF_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent batch */
  NF_ERR_OUT_OF_RANGE = 2,  /* index or size beyond a declared capacity   */
  NF_ERR_UNSUPPORTED = 3,   /* valid but not implemented (page size etc.) */
  NF_ERR_NO_PLAN = 4,       /* plan does not fit the batch                */
  NF_ERR_HIP = 5            /* a HIP runtime call failed                  */
} nf_status;

typedef enum nf_dtype { NF_F32 = 0, NF_BF16 = 1 } nf_dtype;

/* Layer shape.  Requirements: n_q_heads % n_kv_heads == 0 with at most 16
 * query heads per KV head; head_dim a multiple of 32, <= 256 (bf16 layers:
 * head_dim == 128); hidden and ffn multiples of 8; top_k <= n_experts <= 64,
 * top_k <= 8; max_tokens >= 1; max_pos >= 1.  bf16 layers: every GEMM
 * operand (max_tokens * top_k rows of the widest activation, and each weight
 * matrix) stays under 4 GiB, since the GEMMs address operands with 32-bit byte
 * offsets (NF_ERR_OUT_OF_RANGE otherwise). */
typedef struct nf_shape {
  int32_t hidden;       /* H */
  int32_t n_q_heads;    /* nq */
  int32_t n_kv_heads;   /* nkv; query head h uses KV head h / (nq / nkv) */
  int32_t head_dim;     /* d */
  int32_t ffn;          /* F, per expert */
  int32_t n_experts;    /* 1 = dense FFN */
  int32_t top_k;        /* experts per token (1 for dense) */
  int32_t dtype;        /* nf_dtype of weights, activations and KV pool */
  float rms_eps;        /* RMSNorm epsilon */
  double rope_theta;    /* rotary base; frequency j = theta^(-2j/d) */
  int32_t max_tokens;   /* capacity: tokens per step */
  int32_t max_pos;      /* capacity: positions 0..max_pos-1 */
} nf_shape;

/* Layer weights: device pointers in the layer dtype, caller-owned, read-only,
 * valid for the layer's lifetime.  Every matrix is row-major with output
 * features first (K-contiguous rows):
 *   attn_norm [H], ffn_norm [H]
 *   w_qkv  [(nq + 2 nkv) * d][H]  rows: Q heads, then K heads, then V heads,
 *                                 each head's d rows contiguous
 *   w_o    [H][nq * d]
 *   w_gate [E][F][H], w_up [E][F][H], w_down [E][H][F]                  */
typedef struct nf_weights {
  const void* attn_norm;
  const void* w_qkv;
  const void* w_o;
  const void* ffn_norm;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
} nf_weights;

/* One step's batch.  Tokens are ordered by request; request r owns tokens
 * req_q_start[r] .. req_q_start[r] + req_q_len[r] - 1 (contiguous, in order,
 * starts increasing), at positions req_pos0[r] + i (req_pos0 = tokens already
 * cached).  Its logical page i is pool page page_indices[page_indptr[r] + i];
 * it needs at least ceil((req_pos0 + req_q_len) / page_size) pages and no
 * page may belong to two requests.  A decode request has req_q_len == 1; a
 * prefill chunk has req_q_len > 1.  The step writes K/V for the new positions
 * and reads keys 0..p for a token at position p. */
typedef struct nf_batch {
  int32_t n_tokens;            /* T, 0 <= T <= max_tokens                  */
  int32_t n_requests;          /* R                                        */
  const void* x;               /* device [T][H] layer dtype                */
  void* out;                   /* device [T][H] layer dtype (not aliasing x) */
  const int32_t* req_q_start;  /* host [R] */
  const int32_t* req_q_len;    /* host [R] */
  const int32_t* req_pos0;     /* host [R] */
  const int32_t* pos;          /* host [T]; must equal req_pos0 + offset    */
  const int32_t* page_indptr;  /* host [R + 1], page_indptr[0] == 0         */
  const int32_t* page_indices; /* host [page_indptr[R]]                     */
  const float* router_logits;  /* device [T][E] fp32 (MoE layers only)      */
} nf_batch;

#define NF_MAX_NANO 4

typedef enum nf_order {
  /* per GEMM stream: norm+QKV+RoPE/append of nano-batch j+1 are issued before
   * the O-proj/FFN of nano-batch j, so j's attention overlaps j+1's QKV */
  NF_ORDER_PIPELINED = 0,
  /* nano-batch j finishes every operation before j+1 starts */
  NF_ORDER_SEQUENTIAL = 1
} nf_order;

/* Nano-batch plan: count, sizes, operation order and resource split. */
typedef struct nf_plan {
  int32_t count;                  /* 1..NF_MAX_NANO                          */
  int32_t sizes[NF_MAX_NANO];     /* tokens per nano-batch; sum must be T   */
  int32_t order;                  /* nf_order                                */
  int32_t n_streams;              /* 1: all work on the caller's stream;
                                     2: GEMM stream + attention stream       */
  int32_t gemm_cus_per_xcd;       /* n_streams == 2 only: the GEMM stream may use
                                     the first gemm_cus_per_xcd CUs of every
                                     XCD; 0 = every CU                       */
  int32_t attn_cus_per_xcd;       /* n_streams == 2 only: the attention stream
                                     may use the last attn_cus_per_xcd CUs of
                                     every XCD; 0 = the CUs the GEMM stream
                                     does not have (every CU if it has all).
                                     The two ranges may overlap: waves of both
                                     streams then share those CUs (matrix
                                     cores vs memory pipes).                 */
  int32_t attn_waves_per_cu;      /* 0: one attention workgroup per work item;
                                     1..16: a persistent attention grid of
                                     that many single-wave workgroups per CU
                                     of its budget, each looping over work
                                     items, so attention leaves room on every
                                     CU for the GEMM's workgroups            */
} nf_plan;

typedef struct nf_search_opts {
  int32_t max_count;      /* largest nano-batch count tried (<= NF_MAX_NANO) */
  int32_t warmup;         /* untimed steps per measured candidate            */
  int32_t reps;           /* timed steps per measured candidate              */
  int32_t top_k;          /* candidates timed again after the first pass      */
} nf_search_opts;

typedef struct nf_layer nf_layer;
typedef struct nf_kv_pool nf_kv_pool;
typedef struct nf_graph nf_graph;

/* ---- layer ---------------------------------------------------------------
 * nf_layer_create: validates the shape, binds the caller's weights (pointers
 * kept), allocates the workspace on the current HIP device and builds the
 * fp32 cos/sin table (angles in fp64).  For bf16 mixture-of-experts layers
 * it also copies the expert weights once into the MFMA operand order of the
 * weight-streaming expert GEMMs (E * 3 * F * H * 2 bytes, owned by the
 * layer), so weights must not change while the layer exists.  The default plan is
 * one nano-batch on the caller's stream.  Errors: NF_ERR_INVALID_ARG (null
 * pointers, inconsistent shape), NF_ERR_UNSUPPORTED (head_dim or dtype
 * outside the list above), NF_ERR_HIP (allocation failure).
 * Diagnostics read from the environment (for measurements; not needed for
 * normal use): NF_ATTN_VARIANT=0|1 fixes the bf16 attention kernel of layers
 * created afterwards to one-wave work items (0, split page ranges plus a
 * merge) or four-wave workgroups (1); by default four-wave workgroups run
 * unless the plan bounds the attention waves per CU.  NF_SEARCH_VERBOSE
 * prints each plan the search re-times; NF_PROBE_VERBOSE prints the MFMA
 * probe's rate per shape (both to stderr). */
nf_status nf_layer_create(const nf_shape* shape, const nf_weights* w, nf_layer** out);
void nf_layer_destroy(nf_layer* layer);   /* waits for the layer's streams */

/* ---- KV pool --------------------------------------------------------------
 * Paged KV cache (the PagedAttention block pool: "How it differs from vLLM
 * and TensorRT-LLM" on the hysenlabs Nanoflow page).  K and V each hold
 * [n_pages][n_kv_heads] blocks of page_size * head_dim elements in the layer
 * dtype.  page_size must be 16 (NF_ERR_UNSUPPORTED otherwise) and head_dim a
 * multiple of 32.  Inside a block, key slot s (0..15) and dimension d sit at
 *   K: (d / 32) * 512 + (16 * ((d % 32) / 8) + s) * 8 + d % 8
 *   V: (d / 32) * 512 + ((d % 16) + 16 * (s / 4)) * 8 + 4 * ((d / 16) % 2) + s % 4
 * i.e. in the operand order of the attention kernel's matrix-core
 * instructions: every 512-element run is what the 64 lanes of a wavefront
 * load with one contiguous 16-byte-per-lane read (8 elements each), which on
 * gfx950 roughly doubles the bandwidth one CU can draw compared with
 * row-major pages. */
nf_status nf_kv_pool_bytes(const nf_shape* shape, int32_t n_pages, int32_t page_size,
                           size_t* k_bytes, size_t* v_bytes);
nf_status nf_kv_pool_create(const nf_layer* layer, int32_t n_pages, int32_t page_size,
                            void* k_dev, void* v_dev, nf_kv_pool** out);
/* Frees the pool object and its offload staging (waiting for the device when
 * there is any); may run before or after nf_layer_destroy of its layer. */
void nf_kv_pool_destroy(nf_kv_pool* pool);

/* Offloads whole pool pages to host memory, the KV offload of retired
 * requests that the hysenlabs Nanoflow page (section "KV-cache offload to
 * SSD, and the bandwidth arithmetic behind it") and the ossradar page
 * ("Introduction") describe as running beside the inference operations (the
 * SSD leg is not part of this library).  For i < n, page pages[i]'s K block
 * (n_kv_heads x page_size x head_dim elements, in the pool's layout) is
 * written to host_k + i * block and its V block to host_v + i * block, block
 * = n_kv_heads * page_size * head_dim * element size.  The pages are gathered
 * on `stream` into a staging buffer the pool owns, then copied to the host
 * with two DMA transfers (the copy engines, not the compute units), so an
 * offload on its own stream can run beside a step.  host_k / host_v:
 * caller-owned host memory of n * block bytes each; pinned memory
 * (hipHostMalloc, torch pin_memory) keeps the call asynchronous.  `pages`
 * may be reused on return; a page may appear more than once.  Offloads on
 * one pool must not overlap each other; the pages must not be written while
 * the offload reads them (the pool's layer need not exist any more).  Errors:
 * NF_ERR_INVALID_ARG (null pool, negative n, null arrays with n > 0),
 * NF_ERR_OUT_OF_RANGE (a page outside the pool), NF_ERR_HIP. */
nf_status nf_kv_offload(nf_kv_pool* pool, const int32_t* pages, int32_t n, void* host_k, void* host_v,
                        void* stream);

/* ---- plan -----------------------------------------------------------------
 * nf_plan_set validates count, order, streams and CU split against the device
 * (sizes are checked against each batch at step time) and (re)creates the
 * CU-masked streams.  Errors: NF_ERR_INVALID_ARG, NF_ERR_OUT_OF_RANGE,
 * NF_ERR_HIP. */
nf_status nf_plan_set(nf_layer* layer, const nf_plan* plan);
nf_status nf_plan_get(const nf_layer* layer, nf_plan* plan);

/* nf_batch_validate: host-only check of a batch (and optionally a plan)
 * against a shape and a pool geometry; makes no HIP call.  It runs the same
 * checks nf_layer_step runs before launching. */
nf_status nf_batch_validate(const nf_shape* shape, int32_t n_pages, int32_t page_size,
                            const nf_batch* batch, const nf_plan* plan);

/* ---- step -----------------------------------------------------------------
 * Enqueue one layer step after prior work on `stream`; `stream` is ordered
 * after the step completes.  Asynchronous to the host; host arrays of the
 * batch may be reused once the call returns.  Writes batch->out, the pool
 * slots of the batch's new positions and the layer's workspace.  Calls on
 * one layer must not overlap on different host threads. */
nf_status nf_layer_step(nf_layer* layer, nf_kv_pool* pool, const nf_batch* batch, void* stream);

/* ---- multi-layer step -------------------------------------------------------
 * Runs layers[0..n_layers-1] in order on one batch, each with its own KV pool
 * (pools[l] created for layers[l]): batch->x is layer 0's input, each layer
 * reads the previous one's output (a buffer of the producing layer, grown to
 * [T][H] on first use), and the last layer writes batch->out.  The layers
 * must be distinct objects with the same hidden size, dtype, max_tokens,
 * expert count and device; mixture-of-experts layers all route with
 * batch->router_logits.  Every layer runs layer 0's plan.
 * With two streams, two or more nano-batches and the pipelined order, the
 * nano-batches are pipelined across layers.  The hysenlabs Nanoflow page
 * (section "Nano-batching and the device-level pipeline") has nano-batching
 * break the dependency between sequential operations so a device-level
 * pipeline can co-schedule them; a nano-batch's rows depend only on its own
 * rows of the previous layer, so here the pipeline continues across layer
 * boundaries: nano-batch j's norm, QKV and RoPE/append of layer l + 1 are
 * issued right after its O-projection and FFN of layer l, before nano-batch
 * j + 1's of layer l, so j's attention in layer l + 1 runs beside j + 1's
 * GEMMs and no layer boundary drains the pipeline.  Otherwise each layer
 * runs as nf_layer_step would run it.  The
 * result equals that of nf_layer_step applied layer by layer (bit for bit:
 * the same kernels on the same rows).  Asynchronous like nf_layer_step; calls
 * on the same layers must not overlap.  Errors: NF_ERR_INVALID_ARG (null
 * argument, n_layers < 1, a pool of another layer, a repeated layer, layers
 * that differ), then any error of nf_layer_step. */
nf_status nf_stack_step(nf_layer* const* layers, nf_kv_pool* const* pools, int32_t n_layers, const nf_batch* batch,
                        void* stream);

/* Records nf_stack_step(layers, pools, n_layers, batch) as a HIP graph, whose
 * replays (nf_graph_launch) redo exactly that step, launch for launch, with no
 * host work per kernel.  It first runs the step once on `stream` (writing
 * batch->out and the batch's pool slots), synchronises, copies each layer's
 * step metadata (positions, page tables, attention work items) into device
 * buffers the graph owns, then captures the launches on a stream of its own
 * (`stream` may be the null stream, which cannot be captured).  The graph
 * reads batch->x, writes batch->out, the batch's pool slots and the layers'
 * buffers at every replay, so those must stay allocated, and replays must
 * not overlap each other or steps on the same layers; a layer's buffers are
 * never freed before nf_layer_destroy, so a later larger step does not
 * invalidate the graph.  The host arrays of `batch` may be reused on return.
 * Errors: as nf_stack_step; NF_ERR_INVALID_ARG for an empty batch;
 * NF_ERR_UNSUPPORTED for a plan with a CU split (a graph keeps no stream's CU
 * mask) or with per-kernel timing on; NF_ERR_HIP if the capture fails. */
nf_status nf_stack_graph_create(nf_layer* const* layers, nf_kv_pool* const* pools, int32_t n_layers,
                                const nf_batch* batch, void* stream, nf_graph** out);
/* Enqueues one replay on `stream`.  Errors: NF_ERR_INVALID_ARG, NF_ERR_HIP. */
nf_status nf_graph_launch(nf_graph* graph, void* stream);
/* Waits for the device, then frees the graph and its metadata buffers. */
void nf_graph_destroy(nf_graph* graph);

/* ---- plan search -----------------------------------------------------------
 * Profile-driven choice of the plan for this batch.  It stands in for the
 * automatic search of nano-batch number, size, order and resource split in
 * the abstract on the codewithpapers NanoFlow page, whose four dimensions the
 * "Search Space" card of the do-not-panic NanoFlow page lists, and for the
 * Gurobi-based solver of the ossradar Nanoflow page.  The candidates are the unsplit plan and, for every
 * count 2..opts->max_count, equal and attention-balanced sizes, each on one
 * stream and on two streams with several (GEMM, attention) CU budgets and
 * attention residency limits.  After three untimed steps of the unsplit
 * plan, every candidate is timed on this batch for two steps; the `top_k`
 * fastest, and the unsplit plan, are timed again with `warmup` + `reps` steps
 * and the fastest of those is kept.  Runs steps on this batch (so it writes
 * batch->out and the batch's pool slots with the values a step writes),
 * synchronises `stream`, sets the chosen plan on the layer and returns it in
 * *out.  `times_ms`, if not NULL, receives {measured ms per step of the
 * chosen plan, number of candidates}.  An empty batch returns the unsplit
 * plan without running anything.  Errors: NF_ERR_INVALID_ARG for a null
 * argument, any error of nf_layer_step. */
nf_status nf_plan_search(nf_layer* layer, nf_kv_pool* pool, const nf_batch* batch,
                         const nf_search_opts* opts, nf_plan* out, double* times_ms,
                         void* stream);

/* ---- intermediates ----------------------------------------------------------
 * Device pointer and row stride (elements) of an intermediate of the last
 * step, in the layer dtype: 0 q_rot [T][nq*d], 1 attn [T][nq*d],
 * 2 x1 [T][H], 3 act [T][F] (dense layers), 4 qkv [T][(nq+2nkv)*d].
 * For MoE layers, 5 route_idx int32 [T][top_k], 6 route_w fp32 [T][top_k],
 * 7 route_perm int32 [T*top_k], 8 expert_offsets int32 [E+1] (per
 * nano-batch, at the nano-batch's token offset / top_k-scaled offset). */
nf_status nf_layer_intermediate(const nf_layer* layer, int32_t which, const void** dev_ptr,
                                int64_t* row_stride);

/* ---- per-kernel timing ------------------------------------------------------
 * When on, every kernel launch of a step (or only those of kind `only_kind`,
 * if not NULL) records the kernel's own start and end timestamps into a pair
 * of HIP events (hipExtLaunchKernel), on the stream it is launched on, so the
 * duration holds no marker packet or queue gap.  nf_profile_read
 * synchronises those events and returns, per
 * kernel kind, the number of launches and the summed duration (ms) since
 * profiling was switched on; kinds with no launches are omitted.  Names are
 * static strings.  Enabling resets the totals. */
nf_status nf_profile_enable(nf_layer* layer, int32_t on, const char* only_kind);
nf_status nf_profile_read(nf_layer* layer, int32_t max_kinds, const char** names,
                          int64_t* launches, double* total_ms, int32_t* n_kinds);

/* ---- device probes ----------------------------------------------------------
 * Measured peaks of the current device: dense bf16 MFMA TFLOP/s (register-only
 * MFMA chains on every CU) and HBM read GB/s (streaming `bytes` bytes, at
 * least 1 GiB recommended).  nf_probe_cu_map fills xcc[i] with the XCD that
 * CU-mask bit i dispatches to (n = CU count), or -1 for every bit when the
 * expected striping (bit i -> XCD i % 8) could not be confirmed.  A CU mask
 * must leave every XCD at least one CU; the plan's split does. */
nf_status nf_probe_mfma_bf16_tflops(double* tflops);
nf_status nf_probe_hbm_read_gbps(size_t bytes, double* gbps);
/* Average time (ms) of the layer's bf16 GEMM kernel on an M x N x K problem
 * (C = A B^T, mode 0 plain, 1 residual, 2 SwiGLU with N act columns), on
 * library-allocated buffers filled with pseudo-random values (A uniform in
 * [-1, 1), B with standard deviation 0.02).  tile_cfg < 0 and k_splits <= 0
 * let the library choose for a stream that may use `cus` CUs; out_cfg and
 * out_splits (may be NULL) return what ran.  A given tile_cfg must be one that
 * nf_gemm_bf16 accepts for this shape and mode, else NF_ERR_INVALID_ARG, as
 * for N or K not multiples of 8 or reps <= 0.  max(M, N) * K * 2 bytes must
 * stay under 4 GiB (NF_ERR_OUT_OF_RANGE).  Buffers and events are freed on
 * every return path. */
nf_status nf_probe_gemm_bf16_ms(int32_t M, int32_t N, int32_t K, int32_t mode, int32_t tile_cfg,
                                int32_t k_splits, int32_t cus, int32_t reps, double* ms,
                                int32_t* out_cfg, int32_t* out_splits);
nf_status nf_probe_cu_map(int32_t* xcc, int32_t n);

/* ---- one GEMM ------------------------------------------------------------------
 * One bf16 GEMM exactly as the layer runs its projections, on caller device
 * buffers, for verification and tuning (not the layer's hot path):
 *   mode 0: C = A B^T;  mode 1: C = A B^T + R;  mode 2: C = silu(A B^T) * (A B2^T)
 * with A [M][K] (row stride lda), B and B2 [N][K] (ldb), R and C [M][N] (ldr,
 * ldc), strides in elements, fp32 accumulation, one bf16 rounding of C.
 * tile_cfg < 0 and k_splits <= 0 let the library choose for a stream that
 * may use `cus` CUs (cus <= 0: all); a given tile_cfg must be one of the
 * layer's LDS-tiled configurations (0..6, or 10..30 with K % 64 == 0) or of
 * its weight-streaming ones (40..51: N % 32 == 0, K a multiple of the
 * configuration's chunk, two n-blocks per wave exactly for mode 2), for which
 * B is first copied into operand order.  That copy and the split-K workspace
 * are allocated and freed inside, and the call returns after the GEMM
 * finished on `stream` (NULL: the null stream).  out_cfg and
 * out_splits (may be NULL) return what ran.  Operands must stay under 4 GiB
 * (NF_ERR_OUT_OF_RANGE); NF_ERR_INVALID_ARG for other bad arguments. */
nf_status nf_gemm_bf16(int32_t M, int32_t N, int32_t K, int32_t mode, const void* A, int64_t lda,
                       const void* B, const void* B2, int64_t ldb, const void* R, int64_t ldr, void* C,
                       int64_t ldc, int32_t tile_cfg, int32_t k_splits, int32_t cus, void* stream,
                       int32_t* out_cfg, int32_t* out_splits);

/* ---- errors ---------------------------------------------------------------- */
const char* nf_last_error(void);
const char* nf_status_string(nf_status s);

#ifdef __cplusplus
}
#endif
#endif /* NF_H */
