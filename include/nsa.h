/*
 * nsa.h -- C ABI of libnsa.so: the VideoNSA attention layer forward pass on
 * AMD Instinct MI355X (gfx950), as hand-written HIP kernels.
 *
 * What the layer computes (VideoNSA paper summary page, "Method"; model card,
 * "Model Architecture"; paper summary "Key claims", §2.2):
 *   tokens are split by position into vision and text tokens. Vision tokens
 *   run the three NSA branches -- compression (each 64-token frame block is
 *   averaged and mapped through a learned linear map into one block key and
 *   value, then attended), selection (the top-k blocks ranked by an
 *   importance score are attended token by token) and a causal sliding window
 *   -- and per-head sigmoid gates mix the three outputs. Text tokens use dense
 *   causal GQA over every earlier position. Outputs land at the tokens'
 *   original positions.
 * Readings where the pages leave a step open (all shared with the oracle):
 *   a compressed block is visible once complete; the learned map is y = W x
 *   on the block mean (no bias), one W for keys and one for values, shared by
 *   the KV heads; query head h reads KV head h / (Hq/Hkv); a block's
 *   importance for KV group g is the sum over the group's query heads of the
 *   normalised compression-attention probability; ties go to the lower block
 *   index; the query's own block is always selected and counts toward k; the
 *   window holds exactly `window` keys including the query; a query with no
 *   complete block gets a zero compression output; vision queries see vision
 *   keys only; the softmax scale defaults to 1/sqrt(head_dim).
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device memory; "host" marks host memory.
 *   - All tensors are dense, row-major, with the last dimension contiguous,
 *     and 16-byte aligned, except gate logits, selected block indices and
 *     log-sum-exp outputs (float32 / int32 arrays accessed element by
 *     element), which need only their 4-byte element alignment.
 *   - The caller owns every buffer, including the workspace; the library
 *     allocates nothing and keeps no state between calls (the opt-in
 *     benchmark timing below is the one exception: while enabled it creates
 *     HIP events and keeps per-kernel totals).
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     asynchronously; the call does not synchronise.
 *   - Every argument is validated before anything is enqueued. On any
 *     non-OK status nothing has been written or launched.
 *   - Kernel faults surface at the caller's next synchronisation;
 *     NSA_ERR_HIP reports errors returned by launches themselves. The
 *     prefill kernels' waits on each other inside a workgroup are bounded:
 *     one that gives up (about 0.1 s without progress, which a correct run
 *     never reaches) ends its kernel normally with NaN outputs and sets the
 *     status word of the call's workspace, which nsa_workspace_status reads.
 *   - Value range: queries, values and the compressed keys/values are used
 *     in fp16 by the kernels (bf16 -> fp16 is exact inside fp16's range), so
 *     their magnitudes must stay below 65504; larger bf16 inputs overflow to
 *     infinity and give non-finite outputs for the rows that touch them.
 */
#ifndef NSA_H_
#define NSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NSA_OK = 0,
  NSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer    */
  NSA_ERR_UNSUPPORTED = 2, /* valid arguments outside what the kernels take */
  NSA_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than needed */
  NSA_ERR_HIP = 4,         /* a HIP launch reported an error                */
  NSA_ERR_KERNEL = 5       /* a kernel gave up a bounded wait (see
                              nsa_workspace_status)                         */
} nsa_status;

typedef enum {
  NSA_DTYPE_BF16 = 0, /* q, k, v, w_cmp_* in bfloat16                          */
  NSA_DTYPE_FP32 = 1  /* q, k, v, w_cmp_* in float32 (block scores computed from
                         split-bf16 operands to near-fp32 accuracy)             */
} nsa_dtype;

/* ------------------------------------------------------------------ prefill
 * One sequence of n_tokens tokens (VideoNSA paper summary page, "Method":
 * the tokens split into a vision set and a text set by position; the three
 * NSA branches run on the vision set, text tokens get dense causal GQA).
 * The vision tokens may lie anywhere: one run, or several runs with text
 * between them (several clips or images in one prompt). The branches see the
 * vision tokens in position order, so blocks of 64 are counted over that
 * order (a block may straddle two runs) and the window counts vision tokens;
 * a text token attends to every earlier token of either kind and itself.
 * Several runs cost 4 bytes of workspace per token (row maps) and one small
 * launch per 16,384 tokens to build them.
 * Supported: head_dim in {64, 128}, block_size == 64, n_q_heads % n_kv_heads
 * == 0 with at most 8 query heads per KV head, top_k >= 1, window >= 1,
 * N_v / 64 <= 8192. */
typedef struct {
  int64_t n_tokens;   /* N = vision + text tokens                                 */
  int32_t n_q_heads;  /* Hq                                                       */
  int32_t n_kv_heads; /* Hkv                                                      */
  int32_t head_dim;   /* d                                                        */
  int32_t block_size; /* B: compression block == selection block (64)            */
  int32_t top_k;      /* k: selected blocks per (query, KV group), own block incl. */
  int32_t window;     /* w: sliding-window keys, the query included              */
  float scale;        /* softmax scale; <= 0 selects 1/sqrt(d)                    */
  int32_t dtype;      /* nsa_dtype of q, k, v, w_cmp_k, w_cmp_v                   */
} nsa_prefill_desc;

/* Bytes of device workspace nsa_prefill needs for this descriptor and mask.
 * is_vision: host, [N] uint8 (1 = vision token). Returns 0 and leaves
 * *bytes untouched if the arguments are invalid or unsupported (the status
 * says which). */
nsa_status nsa_prefill_workspace_size(const nsa_prefill_desc *desc,
                                      const uint8_t *is_vision,
                                      size_t *bytes);

/* Forward pass of the layer for one sequence.
 *   q            device [N, Hq, d]   (dtype)   queries after positional encoding
 *   k, v         device [N, Hkv, d]  (dtype)   keys / values
 *   is_vision    host   [N] uint8              1 = vision token, 0 = text token
 *   w_cmp_k      device [d, d]       (dtype)   compression map for keys, y = W x
 *   w_cmp_v      device [d, d]       (dtype)   compression map for values
 *   gate_logits  device [N, Hq, 3]   float32   (cmp, sel, swa) logits; a
 *                sigmoid turns them into gates; text rows are not read
 *   out          device [N, Hq, d]   float32   written for every token
 * Optional outputs (NULL to skip):
 *   k_cmp_out, v_cmp_out device [N_v/B, Hkv, d] float32  compressed keys/values
 *                as computed in fp32, before the kernels round them to fp16
 *                (bf16 hi/lo parts for fp32 keys) for their own use
 *   sel_idx_out  device [N_v, Hkv, top_k] int32  selected block indices per
 *                vision query (vision-local numbering), ascending, -1 padded
 *   lse_out      device [N_v, Hq] float32  log-sum-exp of the compression
 *                attention logits (-inf where no block is complete yet)
 *   workspace    device, >= nsa_prefill_workspace_size bytes, 256-B aligned
 */
nsa_status nsa_prefill(const nsa_prefill_desc *desc, const void *q, const void *k,
                       const void *v, const uint8_t *is_vision, const void *w_cmp_k,
                       const void *w_cmp_v, const float *gate_logits, float *out,
                       float *k_cmp_out, float *v_cmp_out, int32_t *sel_idx_out,
                       float *lse_out, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Several independent sequences in one call (varlen batch): tokens of
 * sequence i are rows cu_seqlens[i] .. cu_seqlens[i+1]-1 of q, k, v,
 * is_vision, gate_logits and out (cu_seqlens: host [n_seqs + 1], starting at 0,
 * strictly increasing, ending at desc->n_tokens). Each sequence is its own
 * layer call: its vision tokens, blocks, selection and window never reach
 * another sequence, and its text tokens see only its own earlier tokens. The
 * optional outputs are concatenated over the sequences in order: k_cmp_out /
 * v_cmp_out [sum of N_v,i / B, Hkv, d], sel_idx_out [sum of N_v,i, Hkv, top_k]
 * (numbering local to each sequence), lse_out [sum of N_v,i, Hq]. The
 * sequences run one after another on the stream and share the workspace,
 * sized for the largest (nsa_prefill_varlen_workspace_size). Every
 * sequence is validated before anything is enqueued. Each sequence's slices
 * meet nsa_prefill's alignment whenever the whole arrays do (a slice starts a
 * whole number of d-element rows, or 4-byte elements, into its array). */
nsa_status nsa_prefill_varlen_workspace_size(const nsa_prefill_desc *desc, int32_t n_seqs,
                                             const int64_t *cu_seqlens,
                                             const uint8_t *is_vision, size_t *bytes);
nsa_status nsa_prefill_varlen(const nsa_prefill_desc *desc, int32_t n_seqs,
                              const int64_t *cu_seqlens, const void *q, const void *k,
                              const void *v, const uint8_t *is_vision, const void *w_cmp_k,
                              const void *w_cmp_v, const float *gate_logits, float *out,
                              float *k_cmp_out, float *v_cmp_out, int32_t *sel_idx_out,
                              float *lse_out, void *workspace, size_t workspace_bytes,
                              void *stream);

/* -------------------------------------------------------------- dense mode
 * Dense-NSA inference (VideoNSA paper summary page, "Key claims" and
 * "Results": the sparse-trained weights run under full attention): every
 * token, vision or text, attends to every earlier token and itself with
 * dense causal GQA (query head h reads KV head h / (Hq / Hkv)); no branches,
 * gates or compression. Uses n_tokens, n_q_heads, n_kv_heads, head_dim,
 * scale and dtype of the descriptor; block_size, top_k and window are not
 * read. Supported: head_dim in {64, 128}, at most 8 query heads per KV head
 * (7 at d = 128). fp32 inputs are used as fp16 (products in fp16, fp32
 * accumulation).
 *   q            device [N, Hq, d]   (dtype)
 *   k, v         device [N, Hkv, d]  (dtype)
 *   out          device [N, Hq, d]   float32
 *   lse_out      device [N, Hq] float32 natural-log log-sum-exp of the scaled
 *                logits, or NULL
 *   workspace    device, >= nsa_prefill_dense_workspace_size bytes, 256-B
 *                aligned (the packed key/value tiles: 4 * N * Hkv * d bytes
 *                rounded up to whole 64-token blocks, plus fp16 copies of q, k,
 *                v for fp32 inputs)
 * Errors as for nsa_prefill: nothing is launched unless the status is NSA_OK. */
nsa_status nsa_prefill_dense_workspace_size(const nsa_prefill_desc *desc, size_t *bytes);
nsa_status nsa_prefill_dense(const nsa_prefill_desc *desc, const void *q, const void *k,
                             const void *v, float *out, float *lse_out, void *workspace,
                             size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------- backward
 * Gradients of the layer for training (model card, "Training Details"; paper
 * summary, "Method": the model is trained end to end). The selection of
 * blocks is discrete and has no gradient: the caller passes the forward's
 * sel_idx (nsa_prefill's sel_idx_out). Given dout = dL/d(out), writes
 *   dq [N, Hq, d], dk, dv [N, Hkv, d], dw_cmp_k, dw_cmp_v [d, d],
 *   dgate [N, Hq, 3] (dL/d gate logit; zero on text rows), all float32,
 * through the three branches of the vision rows, the text rows' dense
 * attention and both compression maps. Same descriptor and inputs as
 * nsa_prefill; supported: bf16, one vision run (text before and/or after),
 * the head sizes and limits of nsa_prefill; else NSA_ERR_UNSUPPORTED.
 * Arithmetic: fp16 operands on the matrix cores (q, k, v exactly; dout, the
 * probabilities, the score gradients and the compressed keys / values
 * rounded to fp16) with fp32 accumulation, so q, k, v, dout and the
 * compressed keys / values must lie within the fp16 range (a value outside
 * it sets bit 1 of the workspace's status word, nsa_workspace_status). The
 * query side walks each workgroup's selected tiles through an LDS ring with
 * bounded waits; a wait that gives up sets bit 0 of the status word and
 * leaves NaN in that workgroup's dq rows (never a hang).
 * Every gradient element is written by one thread in a fixed order, so
 * results are bitwise repeatable.
 *   sel_idx   device [N_v, Hkv, top_k] int32 (may be NULL when N_v = 0): the
 *             forward's list (ascending, -1 padded, the own block last); any
 *             other contents give meaningless gradients, never an access
 *             outside the inputs
 *   dout      device [N, Hq, d] float32
 *   workspace device, >= nsa_prefill_backward_workspace_size bytes, 256-B aligned */
nsa_status nsa_prefill_backward_workspace_size(const nsa_prefill_desc *desc, const uint8_t *is_vision,
                                               size_t *bytes);
nsa_status nsa_prefill_backward(const nsa_prefill_desc *desc, const void *q, const void *k, const void *v,
                                const uint8_t *is_vision, const void *w_cmp_k, const void *w_cmp_v,
                                const float *gate_logits, const int32_t *sel_idx, const float *dout,
                                float *dq, float *dk, float *dv, float *dw_cmp_k, float *dw_cmp_v,
                                float *dgate, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------- gate prologue
 * Gate logits from hidden states (VideoNSA paper summary page, "Method";
 * model card, "Model Architecture": a two-layer MLP and a sigmoid give each
 * head its three branch gates). Reading: logits = W2 . act(W1 . x + b1) + b2
 * per token, W1 [d_hidden, d_model], W2 [3 Hq, d_hidden] with row 3 h + c
 * giving head h's logit for branch c (compression, selection, window), so the
 * output is exactly the gate_logits argument of nsa_prefill; the pages give
 * neither the width nor the activation, so both are the caller's. The
 * sigmoid is applied by the layer. Enqueue it before nsa_prefill on the same
 * stream to feed the layer from hidden states.
 * Supported: bf16 x / W1 / W2 (fp32 biases, optional), d_model a multiple of
 * 64, d_hidden a multiple of 128, 3 Hq <= 96, N <= 2^30 and N d_hidden <= 2^37;
 * anything else returns NSA_ERR_UNSUPPORTED. Arithmetic: bf16 products with
 * fp32 sums for the hidden layer, which is kept in fp16; fp16 products with
 * fp32 sums for the logits.
 *   x            device [N, d_model]       bf16
 *   w1, b1       device [d_hidden, d_model] bf16, [d_hidden] float32 or NULL
 *   w2, b2       device [3 Hq, d_hidden]   bf16, [3 Hq] float32 or NULL
 *   gate_logits  device [N, Hq, 3]         float32 (written)
 *   workspace    device, >= nsa_gate_workspace_size bytes (2 N d_hidden), 256-B aligned */
typedef enum { NSA_ACT_SILU = 0, NSA_ACT_GELU_TANH = 1, NSA_ACT_RELU = 2 } nsa_activation;
typedef struct {
  int64_t n_tokens;
  int32_t d_model;
  int32_t d_hidden;
  int32_t n_q_heads;
  int32_t activation; /* nsa_activation */
  int32_t dtype;      /* NSA_DTYPE_BF16 */
} nsa_gate_desc;
nsa_status nsa_gate_workspace_size(const nsa_gate_desc *desc, size_t *bytes);
nsa_status nsa_gate_logits(const nsa_gate_desc *desc, const void *x, const void *w1,
                           const float *b1, const void *w2, const float *b2,
                           float *gate_logits, void *workspace, size_t workspace_bytes,
                           void *stream);

/* ------------------------------------------------------------------- decode
 * One new query per sequence, at the last slot (L-1) of its vision cache
 * (VideoNSA paper summary page, "Method"; evaluated exactly as prefill's row
 * L-1): its own key and value are already in slot L-1; the floor(L/B)
 * complete blocks have compressed keys and values and are all visible; block
 * (L-1)/B is the query's own -- the last complete block when B divides L,
 * else the partial block after them. So a generating caller appends each new
 * token's key and value, and pools a block (nsa_cmp_pool over its 64 rows,
 * written at row b of the compressed cache) once the block is complete.
 * Supported: bf16, head_dim in {64, 128}, block_size == 64, at most 8 query
 * heads per KV head, top_k <= 64, window <= cache_len, cache_len <= 8192 * 64.
 * cache_capacity: rows allocated per sequence in k_cache / v_cache (their
 * sequence stride; 0 means cache_len; must be >= cache_len); the compressed
 * caches then hold floor(cache_capacity / B) rows per sequence. */
typedef struct {
  int32_t batch;      /* Bt sequences                        */
  int32_t cache_len;  /* L tokens per sequence               */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t top_k;
  int32_t window;
  float scale;        /* <= 0 selects 1/sqrt(d)              */
  int32_t dtype;      /* NSA_DTYPE_BF16 only                 */
  int32_t cache_capacity; /* rows per sequence; 0 = cache_len */
} nsa_decode_desc;

nsa_status nsa_decode_workspace_size(const nsa_decode_desc *desc, size_t *bytes);

/*   q            device [Bt, Hq, d]        bf16
 *   k_cache      device [Bt, C, Hkv, d]    bf16  (C = cache capacity; rows
 *   v_cache      device [Bt, C, Hkv, d]    bf16   0..L-1 are read)
 *   k_cmp, v_cmp device [Bt, C/B, Hkv, d]  bf16  compressed cache, rows
 *                0..floor(L/B)-1 read (for example from nsa_cmp_pool)
 *   gate_logits  device [Bt, Hq, 3]        float32
 *   out          device [Bt, Hq, d]        float32
 *   sel_idx_out  device [Bt, Hkv, top_k]   int32 or NULL (ascending, -1 padded)
 *   lse_out      device [Bt, Hq]           float32 or NULL
 */
nsa_status nsa_decode(const nsa_decode_desc *desc, const void *q, const void *k_cache,
                      const void *v_cache, const void *k_cmp, const void *v_cmp,
                      const float *gate_logits, float *out, int32_t *sel_idx_out,
                      float *lse_out, void *workspace, size_t workspace_bytes,
                      void *stream);

/* nsa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same step with the same results, its scratch taken from a fixed array of
 * NSA_DECODE_NOALLOC_SCRATCH_BYTES in device memory that the library holds on
 * every GPU it runs on until the process ends. No allocation happens in the
 * call. Needs plan <= that size (nsa_decode_workspace_size reports the need;
 * 16 sequences of 131,072 tokens with 28 query heads and d 128 use about
 * 17 MB); a larger step returns NSA_ERR_WORKSPACE before anything is
 * launched. All calls on one GPU share its array, and the contents of one
 * call are not kept for the next: calls that overlap in time on the same
 * GPU (several streams or host threads) race and must be serialised by the
 * caller. Arguments and errors otherwise as nsa_decode. */
#define NSA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
nsa_status nsa_decode_noalloc(const nsa_decode_desc *desc, const void *q, const void *k_cache,
                              const void *v_cache, const void *k_cmp, const void *v_cmp,
                              const float *gate_logits, float *out, int32_t *sel_idx_out,
                              float *lse_out, void *stream);

/* Appends one token per sequence to the decode caches and keeps the
 * compressed caches current, so that nsa_decode can run at length cache_len
 * next (the streaming use described above, in one call): k_new / v_new
 * device [Bt, Hkv, d] bf16 are written to row cache_len - 1 of k_cache /
 * v_cache [Bt, C, Hkv, d]; when 64 divides cache_len, the block that token
 * completes (rows cache_len - 64 .. cache_len - 1 of every sequence) is
 * pooled -- block mean, then y = W x with w_cmp_k / w_cmp_v [d, d] bf16, fp32
 * arithmetic, bf16 rounding -- into row cache_len / 64 - 1 of k_cmp / v_cmp
 * [Bt, C/64, Hkv, d]. Reads batch, cache_len, n_kv_heads, head_dim,
 * block_size, dtype and cache_capacity of the descriptor (C =
 * cache_capacity, or cache_len when 0). All pointers are required and
 * 16-byte aligned. Supported: bf16, block_size 64, head_dim 64 or 128. */
nsa_status nsa_cache_append(const nsa_decode_desc *desc, const void *k_new, const void *v_new,
                            void *k_cache, void *v_cache, const void *w_cmp_k,
                            const void *w_cmp_v, void *k_cmp, void *v_cmp, void *stream);

/* ------------------------------------------------------------- compression
 * The compression branch's pooling step on its own (VideoNSA model card,
 * "Model Architecture": frame KV blocks are averaged; paper summary,
 * "Method": a learned map turns each block into one key/value): for each of
 * the n_rows/B complete blocks b and head g,
 *   out[b, g, :] = W * mean(x[b*B .. b*B+B-1, g, :]).
 *   x     device [n_rows, n_heads, d] (dtype)
 *   w     device [d, d]               (dtype), y = W x
 *   out_bf16 device [n_rows/B, n_heads, d] bf16 or NULL
 *   out_f32  device [n_rows/B, n_heads, d] float32 or NULL
 * Used to build the compressed cache that nsa_decode reads. */
nsa_status nsa_cmp_pool(int64_t n_rows, int32_t n_heads, int32_t head_dim,
                        int32_t block_size, int32_t dtype, const void *x, const void *w,
                        void *out_bf16, float *out_f32, void *stream);

/* ------------------------------------------------------------- benchmark
 * Opt-in per-kernel timing (for benchmarks; off by default). While enabled,
 * each kernel launched by the library is bracketed by two HIP events on its
 * launch stream. nsa_timing_read() waits for the recorded events, folds them
 * into per-kernel totals and returns the number of distinct kernels; names
 * point into library storage valid until the next read or reset. Entries are
 * copied for the first max_entries kernels (arrays may be NULL). The
 * registry is process-wide (calls from several threads are serialised by a
 * lock). */
nsa_status nsa_timing_enable(int enable);
nsa_status nsa_timing_reset(void);
int nsa_timing_read(int max_entries, const char **names, double *total_ms, int *counts);

/* Matrix-core peak probe (measurement aid; computes nothing of the layer).
 * Launches n_wg workgroups of four waves; each wave runs `iters` rounds of
 * 128 v_mfma_f32_16x16x32_bf16 products (bf16 operands, fp32 accumulators,
 * eight independent chains) and writes one float per lane to
 * out[n_wg * 256] (device, caller-owned) so the work cannot be dropped.
 * Work per call: n_wg * 4 * iters * 128 * 16384 flops; time it with events
 * on `stream`.
 * NSA_ERR_INVALID_ARG for n_wg < 1, iters < 1 or out == NULL. */
nsa_status nsa_probe_mfma_bf16(int32_t n_wg, int32_t iters, float *out, void *stream);

/* Block-stream probe (measurement aid; computes nothing of the layer): the
 * fabric rate of the selection kernel's access pattern. Launches n_wg
 * workgroups of eight waves; each reads `iters` pseudo-random whole 32 KB
 * blocks of buf (n_blocks blocks, device, 16-byte aligned, caller-owned;
 * every block index is taken modulo n_blocks) with 16-byte loads, two
 * blocks in flight, and writes one checksum word per thread to
 * out[n_wg * 512] (device, caller-owned). Bytes read per call:
 * n_wg * iters * 32768; time it with events on `stream`. With buf much
 * larger than the L2 the rate is what L2 misses of such blocks reach.
 * NSA_ERR_INVALID_ARG for a NULL or misaligned pointer, n_blocks < 1,
 * n_wg < 1, or iters not a positive even number. */
nsa_status nsa_probe_block_stream(const void *buf, int64_t n_blocks, int32_t n_wg, int32_t iters,
                                  uint32_t *out, void *stream);

/* Status word of a prefill or backward workspace (the first 4 bytes of the
 * workspace passed to nsa_prefill, nsa_prefill_varlen or
 * nsa_prefill_backward, cleared at the start of every such call): waits on
 * `stream` for the work enqueued so far, copies the word to *flags and
 * returns NSA_ERR_KERNEL if it is nonzero, NSA_OK otherwise. Bit 0: a bounded
 * wait gave up and that call's outputs are invalid (prefill). Bit 1: a value
 * converted to fp16 for the matrix cores left the fp16 range (q, a value or
 * a compressed key / value in prefill; q, k, v, dout or a compressed key /
 * value in the backward), so the results hold infinities or NaN.
 * workspace: device, 256-B aligned; NSA_ERR_INVALID_ARG for NULL arguments. */
nsa_status nsa_workspace_status(const void *workspace, void *stream, int32_t *flags);

/* Test aid: the number of s_sleep rounds a bounded wait of the prefill
 * kernels (and of the backward's query-side selection walk) spins before
 * giving up, for calls enqueued afterwards in this
 * process (rounds <= 0 restores the default, about 0.1 s). A tiny limit
 * makes the waits give up, so that the failure path -- every kernel ending
 * normally, NaN outputs, the status word set -- can be exercised. */
nsa_status nsa_debug_set_spin_limit(int32_t rounds);

/* Static description of a status code. */
const char *nsa_status_string(nsa_status status);

/* Library version, "major.minor.patch". */
const char *nsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H_ */
