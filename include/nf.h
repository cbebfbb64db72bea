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
  NF_ORDER_SEQUENTIAL = 1,
  /* per GEMM stream, round t issues the front half of nano-batch t, the
   * O-projection of t-1 and the FFN of t-2: attention(t) runs beside the
   * O-projection of t-1 and the FFN of t-2, and a collective after an
   * O-projection (nf_layer_set_allreduce_emulation) beside the next
   * nano-batch's O-projection */
  NF_ORDER_DEEP = 2,
  /* n_streams == 2 only: two lanes.  Nano-batch j runs every operation of
   * its own (front, attention, O-projection, FFN) on stream j mod 2, so one
   * lane's attention shares the chip with the other lane's GEMMs as each
   * kernel frees CUs.  Lane 1 starts once nano-batch 0's front is done (one
   * wait); the attention of a nano-batch j >= 2 whose first request began
   * in an earlier nano-batch (a prefill chunk cut by the plan) also waits
   * for the front of nano-batch j - 1, which appended keys it reads; the
   * caller's stream joins both lanes at the end (one wait).  Each lane's GEMMs take
   * their tiles for the lane's share of the chip: its CU budget under a CU
   * split (gemm_cus_per_xcd for lane 0, the attention budget for lane 1),
   * else half the CUs, so that a lane's GEMM of half the tokens keeps full-K
   * 256 x 256 tiles instead of split-K ones sized for the whole chip. */
  NF_ORDER_LANES = 3
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
                                     1..16: a persistent attention grid that
                                     holds that many waves per CU of its
                                     budget, each workgroup looping over work
                                     items: four-wave workgroups (33 KB of LDS
                                     each) for multiples of 4, single-wave
                                     ones otherwise, so attention leaves
                                     registers and LDS on every CU for the
                                     GEMM's workgroups, which then use tiles
                                     that fit beside it (128 x 128)          */
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
 * nf_layer_create: one decoder layer of the Llama / Mixtral families the
 * ossradar Nanoflow README lists ("News"; Mixtral 8x7B also in the abstract
 * on the codewithpapers page), whose operations the device-level pipeline
 * runs ("How it works" on the bytedragons Nanoflow page: the GEMMs
 * compute-bound, attention and the KV cache memory-bound).  It validates the
 * shape, binds the caller's weights (pointers
 * kept), allocates the workspace on the current HIP device and builds the
 * fp32 cos/sin table (angles in fp64).  For bf16 mixture-of-experts layers
 * it also copies the expert weights once into the MFMA operand order of the
 * weight-streaming expert GEMMs (E * 3 * F * H * 2 bytes, owned by the
 * layer).  Every bf16 layer (hidden % 8 == 0) also folds the attention
 * RMSNorm into the QKV projection: it keeps W_qkv with the norm gain applied
 * to its columns ((nq + 2 nkv) * d * H * 2 bytes, made once, rounded to bf16),
 * the projection reads the layer input itself, and each row's 1 / RMS scales
 * q, k and v in RoPE/append.  Weights must therefore not change while the
 * layer exists.  The default plan is
 * one nano-batch on the caller's stream.  Errors: NF_ERR_INVALID_ARG (null
 * pointers, inconsistent shape), NF_ERR_UNSUPPORTED (head_dim or dtype
 * outside the list above), NF_ERR_HIP (allocation failure).
 * Diagnostics read from the environment (for measurements; not needed for
 * normal use): NF_ATTN_VARIANT=0|1 fixes the bf16 attention kernel of layers
 * created afterwards to one-wave work items (0, split page ranges plus a
 * merge) or four-wave workgroups (1); by default four-wave workgroups run
 * unless the plan bounds the attention waves per CU.  NF_SEARCH_VERBOSE
 * prints each plan the search re-times; NF_PROBE_VERBOSE prints the MFMA
 * probe's rate per shape (both to stderr).  NF_GEMM_OVERRIDE=
 * "M,N,K,mode=cfg:splits;..." (read once per process) forces LDS-pipelined
 * configuration cfg (10..30) and the K split on every dense bf16 GEMM of that
 * shape and mode (0 plain, 1 residual, 2 SwiGLU), for timing configurations
 * inside the step; results then differ from the default choice by rounding
 * only.  NF_NORM_FOLD=0 keeps the attention RMSNorm as a kernel of its own
 * (normalised rows, then the QKV GEMM) in layers created afterwards. */
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

/* Conversion between the pool's layout and the plain paged-cache layout
 * [n][n_kv_heads][page_size][head_dim] (page, KV head, key slot, dimension;
 * row-major, the layer dtype), so a caller holding a conventional PagedAttention
 * block pool ("How it differs from vLLM and TensorRT-LLM" on the hysenlabs
 * Nanoflow page) can hand its cache to the step and read it back.
 * nf_kv_pool_import writes, for i < n, the K and V blocks of pool page
 * pages[i] from entry i of k_src / v_src; nf_kv_pool_export reads them into
 * k_dst / v_dst.  pages: host int32 [n], pool pages in range (a page listed
 * twice on import: the later entry wins); NULL means pages 0..n-1 (n <=
 * n_pages).  k_src / v_src / k_dst / v_dst: caller-owned device buffers of
 * n * n_kv_heads * page_size * head_dim elements, not overlapping the pool.
 * Enqueued on `stream` (NULL: the null stream); the page list may be reused on
 * return.  Calls on one pool must not overlap each other, nor a step or an
 * offload that touches the same pages.  Moves bits only (no rounding).
 * Errors, before anything is launched: NF_ERR_INVALID_ARG (null pool,
 * negative n, null buffers with n > 0), NF_ERR_OUT_OF_RANGE (a page outside
 * the pool, n beyond the pool without a list); NF_ERR_HIP. */
nf_status nf_kv_pool_import(nf_kv_pool* pool, const int32_t* pages, int32_t n, const void* k_src,
                            const void* v_src, void* stream);
nf_status nf_kv_pool_export(nf_kv_pool* pool, const int32_t* pages, int32_t n, void* k_dst, void* v_dst,
                            void* stream);

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
 * nf_plan_set fixes the four choices the abstract on the codewithpapers
 * NanoFlow page has the system make per batch -- number, size and ordering of
 * the nano-batches and their share of the GPU's resources -- here the
 * partition of every XCD's compute units between the GEMM and attention
 * streams (partitioning a device's functional units: "How it works" on the
 * bytedragons Nanoflow page).  It validates count, order, streams and CU
 * split against the device (sizes are checked against each batch at step
 * time) and creates the plan's CU-masked stream pair if it does not exist.
 * Masked pairs belong to the device, not the layer: every layer on a device
 * shares them, at most two stay alive, and the least recently used one is
 * drained and destroyed when a third budget is needed (each masked stream
 * holds a hardware queue; dozens of them slowed masked steps severalfold).
 * They live until the process ends.  Errors: NF_ERR_INVALID_ARG,
 * NF_ERR_OUT_OF_RANGE, NF_ERR_HIP. */
nf_status nf_plan_set(nf_layer* layer, const nf_plan* plan);
nf_status nf_plan_get(const nf_layer* layer, nf_plan* plan);

/* Emulation of the network-bound operation of a tensor-parallel layer, the
 * third resource nano-batching overlaps with compute- and memory-bound work
 * (README "Introduction" on the ossradar Nanoflow page; "The problem
 * Nanoflow attacks" on the hysenlabs page).  A layer that is one GPU's shard
 * (row-parallel O and down projections) needs an all-reduce of each of those
 * outputs across the GPUs; on one GPU it is the identity, and this switch
 * stands in for it: after the O-projection and after the down projection of
 * every nano-batch, its [T_j][H] rows make a send leg (to a staging buffer)
 * and a receive leg (into the buffer the next operation reads) on a third
 * stream, 2 * T_j * H elements moved per collective -- the per-GPU volume of
 * a two-phase all-reduce, rounded up from 2 * (7/8) * T_j * H for 8 GPUs.
 * mode 0: off; 1: both legs on the copy engines (DMA, no compute units); 2:
 * both legs by a copy kernel of `copy_workgroups` workgroups (a collective
 * library's CU channels).  The FFN half of a nano-batch waits for its
 * O-projection's collective, and the step's stream for the last collective;
 * results are bit-identical to mode 0.  Allocates three [max_tokens][H]
 * buffers on first use.  Not for stack graphs.  Errors: NF_ERR_INVALID_ARG,
 * NF_ERR_UNSUPPORTED (hidden not a whole number of 16-byte units), NF_ERR_HIP. */
nf_status nf_layer_set_allreduce_emulation(nf_layer* layer, int32_t mode, int32_t copy_workgroups);

/* nf_batch_validate: host-only check of a batch (and optionally a plan)
 * against a shape and a pool geometry; makes no HIP call.  It runs the same
 * checks nf_layer_step runs before launching. */
nf_status nf_batch_validate(const nf_shape* shape, int32_t n_pages, int32_t page_size,
                            const nf_batch* batch, const nf_plan* plan);

/* ---- step -----------------------------------------------------------------
 * One iteration of the layer over a batch the host formed (decode tokens and
 * a prefill chunk together), run as the plan's nano-batches: every operation
 * is duplicated per nano-batch so the compute-, memory-bound operations of
 * different nano-batches overlap (abstract on the codewithpapers NanoFlow
 * page; "Nano-batching and the device-level pipeline" on the hysenlabs
 * Nanoflow page); the result equals the unsplit layer's up to rounding.
 * Enqueue the step after prior work on `stream`; `stream` is ordered
 * after the step completes.  Asynchronous to the host; host arrays of the
 * batch may be reused once the call returns.  Writes batch->out, the pool
 * slots of the batch's new positions and the layer's workspace.  Calls on
 * one layer must not overlap on different host threads.  Errors: those of
 * nf_batch_validate (nothing launched), NF_ERR_HIP; after a HIP failure
 * partway through the launches the call waits for what it had enqueued
 * before returning, and the next step runs as if none had failed.  For tests
 * of these paths, NF_FAULT=after:<n> in the environment makes the n-th
 * checked HIP call of the next nf_layer_step / nf_stack_step report failure
 * without being made. */
nf_status nf_layer_step(nf_layer* layer, nf_kv_pool* pool, const nf_batch* batch, void* stream);

/* ---- serving loop ----------------------------------------------------------
 * The asynchronous CPU control flow around nf_layer_step: batch formation,
 * KV page management and retirement of finished requests, which the ossradar
 * Nanoflow README ("Introduction") measures at over a tenth of inference time
 * when done in step with the device, and which the hysenlabs page ("The
 * failure modes the design accepts") has the host run one iteration ahead.
 * A loop owns a layer's pool pages (all of them, through a free list) and
 * serves requests added with nf_loop_add_request: rows_in holds the input row
 * of each position 0 .. max_len-1 (the prompt, then the rows fed back for
 * generated positions), rows_out receives the layer's output row for every
 * position processed (both device [max_len][H] in the layer dtype,
 * 16-byte aligned, caller-owned, valid until the loop is destroyed).  Each
 * iteration schedules one token per request past its prompt and then chunks
 * of prompts (at most max_prefill_tokens prompt tokens, max_tokens in all),
 * runs the layer with its plan (its nano-batch count spread evenly over the
 * batch), copies the outputs and writes, per token, whether out[t][0] >
 * eos_threshold into pinned host memory.  A position at or past
 * prompt_len - 1 whose flag is set ends its request, as does its last
 * position.  Requests are admitted in order once the free pages hold their
 * whole max_len.  async = 1: iteration i + 1 is formed (pages allocated) and
 * launched before iteration i's flags are read, and requests that ended at i
 * retire when i + 2 is formed (one more token each, counted as wasted);
 * async = 0: the flags are read after every iteration.  nf_loop_run returns
 * when every request has ended; nf_loop_request_length gives the number of
 * positions up to and including a request's end (-1 while it runs).  The
 * layer must be dense; calls on one loop must not overlap, nor steps on its
 * layer and pool.  Errors: NF_ERR_INVALID_ARG, NF_ERR_OUT_OF_RANGE (a request
 * longer than the pool), NF_ERR_HIP, any error of nf_layer_step. */
typedef struct nf_loop nf_loop;
typedef struct nf_loop_opts {
  int32_t max_tokens;           /* tokens per iteration, 1 .. layer max_tokens */
  int32_t max_prefill_tokens;   /* prompt tokens per iteration                  */
  int32_t async;                /* 1: read flags one iteration late           */
  float eos_threshold;          /* a position ends its request when out[t][0] > this */
} nf_loop_opts;
typedef struct nf_loop_stats {
  int32_t iterations, finished;
  int64_t tokens;               /* token positions processed                 */
  int64_t wasted_tokens;        /* of those, after their request had ended    */
  double host_us;               /* host time forming, launching, retiring     */
  double wall_us;               /* wall time of nf_loop_run                   */
} nf_loop_stats;
nf_status nf_loop_create(nf_layer* layer, nf_kv_pool* pool, const nf_loop_opts* opts, nf_loop** out);
nf_status nf_loop_add_request(nf_loop* loop, int32_t prompt_len, int32_t max_len, const void* rows_in,
                              void* rows_out, int32_t* id);
nf_status nf_loop_run(nf_loop* loop, void* stream, nf_loop_stats* stats);
nf_status nf_loop_request_length(const nf_loop* loop, int32_t id, int32_t* length);
void nf_loop_destroy(nf_loop* loop);   /* waits for the device */

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

/* ---- plan model ------------------------------------------------------------
 * The event-graph step-time model the plan search ranks candidates with.  A
 * step is four operations per nano-batch j -- F (RMSNorm, QKV, RoPE/append),
 * A (attention), O (O-projection with the FFN norm), N (gate/up and down) --
 * in the plan's issue order on one stream, or with A on a second stream.
 * Each nano-batch runs F -> A -> O -> N; a dependency across streams costs
 * wait_us.  Solo durations: front_us / oproj_us / ffn_us per launch at the
 * nano-batch sizes tokens[0 .. n_points-1] (ascending), interpolated
 * piecewise linearly (proportionally for one point); attention
 * attn_base_us + attn_us_per_page * (work items x KV pages of the
 * nano-batch); gap_us added per operation.  While both streams run, the GEMM
 * side progresses at 1 / slow_gemm and attention at 1 / slow_attn of its
 * solo rate (interference of concurrent operations, the consideration the
 * codewithpapers abstract names for the search).  scale_gemm / scale_attn
 * (values <= 0 read as 1) multiply every duration of that side whether or
 * not the other runs: the cost of a CU budget, which confines a side also
 * when it runs alone.  The plan search measures
 * these inputs on the device; nf_plan_predict evaluates the model alone on
 * the host (no HIP call) for a plan and batch: *us = predicted step time.
 * Errors: NF_ERR_INVALID_ARG (null argument, n_points outside
 * 1..NF_PROFILE_POINTS), any nf_batch_validate error of the plan on the
 * batch's token count. */
#define NF_PROFILE_POINTS 8
typedef struct nf_plan_profile {
  int32_t n_points;
  double tokens[NF_PROFILE_POINTS];
  double front_us[NF_PROFILE_POINTS];
  double oproj_us[NF_PROFILE_POINTS];
  double ffn_us[NF_PROFILE_POINTS];
  double attn_base_us, attn_us_per_page;
  double gap_us;
  double slow_gemm, slow_attn, wait_us;
  double scale_gemm, scale_attn;
  double lane_rate;       /* lanes order: the rate (of its solo rate) at which each of two
                             operations of one class runs while both lanes run them
                             (0: one half) */
} nf_plan_profile;
nf_status nf_plan_predict(const nf_plan_profile* prof, const nf_shape* shape, const nf_plan* plan,
                          const nf_batch* batch, double* us);

/* ---- plan search -----------------------------------------------------------
 * Profile-driven choice of the plan for this batch.  It stands in for the
 * automatic search of nano-batch number, size, order and resource split in
 * the abstract on the codewithpapers NanoFlow page (which has the search
 * weigh the interference of concurrent operations), whose four dimensions
 * the "Search Space" card of the do-not-panic NanoFlow page lists, and for
 * the Gurobi-based solver of the ossradar Nanoflow page:
 *  1. solo profiles: after ten settling steps, the batch run as
 *     1..opts->max_count equal nano-batches, and a prefix of its requests of
 *     about T/8 tokens, on one stream with every kernel timed, giving the
 *     nf_plan_profile inputs (front, O-projection and FFN durations per
 *     nano-batch size, attention per KV page unit, the per-operation gap),
 *     scaled to the same steps timed without per-kernel events;
 *  2. interference: for each two-stream resource split -- all CUs to both
 *     sides; attention held to 8 or 4 waves per CU; GEMM + attention CUs per
 *     XCD of 28 + 4, 24 + 8, 20 + 12, 16 + 16, 12 + 20 and 8 + 24 -- two equal
 *     nano-batches run overlapped once, giving that split's co-run slowdowns
 *     (unmasked) or per-side scale factors (CU budgets), and the cross-stream
 *     wait fitted so that the model meets the run; then the same two
 *     nano-batches as two lanes (NF_ORDER_LANES), which fits the profile's
 *     lane_rate (and, if that cannot slow the model enough, its wait);
 *  3. every candidate is predicted with the model of nf_plan_predict:
 *     counts 1..max_count; sizes equal, attention-balanced, in 64-token
 *     steps (two nano-batches), quarter / half / quarter (three), and the
 *     decode requests apart from a trailing prefill chunk; the pipelined and
 *     deep orders on two streams for each split, two lanes, and one stream;
 *  4. the `top_k` best predictions and the unsplit plan are timed with
 *     `warmup` + `reps` steps, and the fastest is kept.
 * Runs steps on this batch (so it writes batch->out); the pool pages holding
 * the batch's new positions are copied aside before the first step and
 * copied back before returning, so the pool ends bit-identical to how it was
 * (it is not read-only while the search runs: nothing else may use it
 * meanwhile).  Synchronises `stream`, sets the chosen plan on the layer and
 * returns it in *out.  `times_ms`, if not NULL, receives {measured ms per
 * step of the chosen plan, number of candidates predicted}.
 * nf_plan_search_report returns the plans the last search on this layer ran
 * (the calibration runs, then the timed candidates) with their predicted and
 * measured ms per step, and calibration[i] = 1 for a calibration run (whose
 * cross-stream wait or lane rate was fitted to make the model meet it) else 0: *n = their
 * number, the first min(n, max) copied to the arrays (each may be NULL).  An empty batch returns the unsplit plan
 * without running anything.  Errors: NF_ERR_INVALID_ARG for a null argument,
 * NF_ERR_UNSUPPORTED with per-kernel timing on, any error of nf_layer_step. */
nf_status nf_plan_search(nf_layer* layer, nf_kv_pool* pool, const nf_batch* batch,
                         const nf_search_opts* opts, nf_plan* out, double* times_ms,
                         void* stream);
nf_status nf_plan_search_report(const nf_layer* layer, int32_t max, nf_plan* plans, double* predicted_ms,
                                double* measured_ms, int32_t* calibration, int32_t* n);

/* ---- intermediates ----------------------------------------------------------
 * Device pointer and row stride (elements) of an intermediate of the last
 * step, in the layer dtype: 0 q_rot [T][nq*d], 1 attn [T][nq*d],
 * 2 x1 [T][H], 3 act [T][F] (dense layers), 4 qkv [T][(nq+2nkv)*d] (in bf16
 * layers that fold the attention RMSNorm: with each row's 1 / RMS applied
 * where the QKV GEMM was split over K, since RoPE/append writes its reduced
 * sums there, and without it where the GEMM stored them itself).
 * For MoE layers, 5 route_idx int32 [T][top_k], 6 route_w fp32 [T][top_k],
 * 7 route_perm int32 [T*top_k], 8 expert_offsets int32 [E+1] (per
 * nano-batch, at the nano-batch's token offset / top_k-scaled offset). */
nf_status nf_layer_intermediate(const nf_layer* layer, int32_t which, const void** dev_ptr,
                                int64_t* row_stride);

/* nf_layer_debug_capture: per-stage parity access.  q_rot, attn, x1 and act
 * are the step's own working buffers, so keeping them costs the step nothing
 * and capture is on from nf_layer_create.  With on == 0 the library makes no
 * promise about them: nf_layer_intermediate refuses every index with
 * NF_ERR_UNSUPPORTED until capture is switched on again (the next step then
 * refills them).  No device work; NF_ERR_INVALID_ARG for a null layer. */
nf_status nf_layer_debug_capture(nf_layer* layer, int32_t on);

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
 * least 1 GiB recommended).
 * nf_probe_cu_map measures which XCD and which CU every CU-mask bit selects
 * (the partition of the device's units that the plan's CU split relies on,
 * "How it works" on the bytedragons Nanoflow page): for each aligned group of
 * 8 mask bits (one CU of every XCD under the runtime's bit i -> XCD i % 8
 * rule; a mask must leave every XCD a CU) it runs single-wave workgroups on a
 * stream masked to that group and reads their XCC_ID and the CU field of
 * HW_ID (bits 15..8: shader engine, array, CU).  xcc[i] receives bit i's XCD
 * and cu[i] (may be NULL) that CU field; both are -1 for every bit when a
 * group did not show 8 distinct XCDs with one CU each or an XCD's groups did
 * not select distinct CUs (the plans then fall back to the striping rule).
 * Measured once per device and cached.  nf_probe_budget_cus runs the same
 * probe on a stream masked the way a plan's budget is (CUs first ..
 * first + count - 1 of every XCD, by the measured map) and returns the
 * distinct (XCD << 16 | CU field) pairs its workgroups ran on, sorted, in
 * xcc_cu[0 .. min(*n_out, max) - 1].  Errors: NF_ERR_INVALID_ARG,
 * NF_ERR_OUT_OF_RANGE (a budget beyond the XCD's CUs), NF_ERR_HIP. */
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
nf_status nf_probe_cu_map(int32_t* xcc, int32_t* cu, int32_t n);
nf_status nf_probe_budget_cus(int32_t first, int32_t count, int32_t* xcc_cu, int32_t max, int32_t* n_out);

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

/* Size of the device array that holds nf_gemm_bf16_noalloc's scratch memory. */
#define NF_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* nf_gemm_bf16 for callers that cannot allocate device memory: code under HIP
 * stream capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, arithmetic, tile choice and result bits as nf_gemm_bf16, with
 * three differences:
 *  - its only scratch memory, the fp32 split-K partial slices (M x N x
 *    splits x 4 bytes, N doubled for mode 2), lives in a file-scope device
 *    array of NF_NOALLOC_SCRATCH_BYTES that each GPU the library runs on
 *    holds from its first call until the process ends; larger needs return
 *    NF_ERR_OUT_OF_RANGE (choose fewer k_splits or split the problem);
 *  - it calls no hipMalloc, hipFree or other allocating routine, and does
 *    not synchronise: it returns once the GEMM is enqueued on `stream`;
 *  - the weight-streaming configurations (tile_cfg >= 40, which read an
 *    operand-order copy of B) are NF_ERR_UNSUPPORTED.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams or threads, not ordered by the caller) race on the
 * partials and give wrong results.  The partial slices are written in full
 * before they are read, so nothing needs clearing between calls.  The device
 * address of the array is looked up once per device, on the first call made
 * with that device current. */
nf_status nf_gemm_bf16_noalloc(int32_t M, int32_t N, int32_t K, int32_t mode, const void* A, int64_t lda,
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
