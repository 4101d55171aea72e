/*
 * bpt.h — C ABI of the MI355X (gfx950) Blockwise Parallel Transformer layer
 * forward.
 *
 * What one call computes (BPT paper review, "Blockwise Parallel Transformer
 * for Large Context Models", §三 "核心公式" and Algorithm 1; conventions of
 * "PyTorch 2.3 实现多头自注意力…" §2–§4 and "Transformer QKV 矩阵计算…" §1–§2):
 *
 *   QKV = x·Wqkvᵀ + bqkv           projected for the whole sequence first
 *   A_i = softmax(Q_i K^T / sqrt(d)) V   per head, per query block i, computed
 *                                  by an inner loop over key/value blocks
 *                                  with running max / sum statistics (the
 *                                  review's Eq. 3 "Scaling"), causal: key<=query
 *   y_i = x_i + A_i·Woᵀ + bo       output projection and residual
 *   out_i = y_i + max(0, y_i·W1ᵀ + b1)·W2ᵀ + b2   position-wise FFN, residual
 *
 * No s×s score matrix and no s×f FFN intermediate is ever stored: the FFN
 * runs over one bounded group of query blocks at a time.
 *
 * Conventions shared by every entry point:
 *  - All tensors are dense row-major. Pointers named x, W*, b*, out, A_out,
 *    y_out and workspace are DEVICE pointers on the current HIP device; the
 *    bpt_shape pointer and the size_t / int64_t out-parameters are HOST
 *    pointers.
 *  - One dtype per call (shape->dtype) for x, every weight, every bias and
 *    out. Products accumulate in fp32. BPT_BF16: inputs and outputs bf16,
 *    intermediates (Q, K, V, A, H) stored as bf16 with round-to-nearest-even.
 *    BPT_F32: everything fp32 (no reduced precision anywhere).
 *  - Weights are in the [out, in] layout, the weight of PyTorch's nn.Linear
 *    (each output feature's row is contiguous; the product is x·Wᵀ). The
 *    pages' formulas write x·W with W = [in, out]; a caller holding that
 *    form passes its transpose. Wqkv [3h, h] with row blocks [Q | K | V] and
 *    head n of each block at rows n·d … n·d+d−1, d = h / heads (the layout of
 *    nn.MultiheadAttention's in_proj_weight); Wo [h, h]; W1 [f, h];
 *    W2 [h, f]. Biases: bqkv [3h], bo [h], b1 [f], b2 [h]. x and out are
 *    [batch, seq, h].
 *  - B_q and B_kv are the method's query- and key/value-block SIZES in
 *    tokens. Each must be a multiple of 16 in [16, seq] and divide seq. In
 *    the bf16 attention a workgroup owns R query rows, R the largest of 256,
 *    128, 64, 32, 16 that divides B_q (a query block is B_q / R workgroups;
 *    R = 16 fills half of the 32-wide MFMA tile), and walks the keys in LDS
 *    stages of S, the largest of 64, 32, 16 that divides B_kv, folding the
 *    running max / sum once per stage (a key/value block is B_kv / S
 *    stages; stages never straddle a block). bpt_layer_attention_tile
 *    reports (R, S). B_q also sets the FFN group (G query blocks, see
 *    bpt_layer_epilogue_rows). The fp32 path and the backward keep their
 *    own fixed tiles. The result does not depend on B_q or B_kv beyond
 *    floating-point summation order.
 *  - Ownership: the caller owns every buffer, including the workspace; the
 *    library allocates no device memory and keeps no pointer after the call
 *    returns (the one exception is bpt_layer_fwd_noalloc's fixed scratch,
 *    described there).
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream). Work is
 *    enqueued asynchronously; argument errors are detected and returned
 *    before anything is enqueued; a failed launch returns BPT_ERR_HIP.
 *  - Calls are reentrant across streams when their workspaces differ.
 *  - All pointers must be 16-byte aligned. `out` may be exactly `x` (in
 *    place); any other overlap of `out` with an input, a weight or the
 *    workspace is BPT_ERR_ALIAS.
 */
#ifndef BPT_H_
#define BPT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BPT_F32 = 0, BPT_BF16 = 1 } bpt_dtype;

typedef struct {
  int64_t batch;  /* b  >= 1 */
  int64_t seq;    /* s  >= 16, a multiple of 16 */
  int64_t hidden; /* h  a multiple of 64 */
  int64_t heads;  /* nh with h % nh == 0 and d = h/nh in {32, 64, 128} */
  int64_t ffn;    /* f  a multiple of 64 */
  int32_t dtype;  /* a bpt_dtype */
} bpt_shape;

typedef enum {
  BPT_OK = 0,
  BPT_ERR_NULL = 1,      /* a required pointer is NULL */
  BPT_ERR_SHAPE = 2,     /* h % nh != 0, d not in {32,64,128}, h or f not a multiple of 64,
                            seq not a positive multiple of 16, batch < 1 */
  BPT_ERR_BLOCK = 3,     /* B_q or B_kv not a multiple of 16, outside [16, seq], or not dividing seq */
  BPT_ERR_DTYPE = 4,     /* dtype is neither BPT_F32 nor BPT_BF16 */
  BPT_ERR_ALIGN = 5,     /* a device pointer is not 16-byte aligned */
  BPT_ERR_ALIAS = 6,     /* out overlaps an input, a weight or the workspace (out == x is allowed) */
  BPT_ERR_WORKSPACE = 7, /* workspace_bytes is smaller than bpt_layer_workspace_bytes() */
  BPT_ERR_DEVICE = 8,    /* the current device is not gfx950, or cannot be queried */
  BPT_ERR_HIP = 9,       /* a kernel launch or copy failed */
  BPT_ERR_SIZE = 10,     /* a size computation overflows */
  BPT_ERR_DROPOUT = 11,  /* dropout rate not in [0, 1), or a mask shape not a multiple of 16 */
  BPT_ERR_SCRATCH = 12   /* bpt_layer_fwd_noalloc: the call needs more than its fixed scratch */
} bpt_status;

typedef void *bpt_stream_t; /* a hipStream_t */

/* Bytes of device workspace bpt_layer_fwd needs for this shape and blocking.
 * Host-only; touches no device. Status BPT_OK and *bytes set, or an
 * argument error. */
int bpt_layer_workspace_bytes(const bpt_shape *shape, int64_t B_q, int64_t B_kv, int causal,
                              size_t *bytes);

/* Rows of one epilogue group: the FFN runs over G consecutive query blocks
 * (G·B_q rows of the flattened [batch·seq] token axis) at a time, so the
 * hidden activation held at once is G·B_q × f. Host-only. */
int bpt_layer_epilogue_rows(const bpt_shape *shape, int64_t B_q, int64_t *rows);

/* One BPT layer forward (see the top of this file). Asynchronous on
 * `stream`. Returns BPT_OK or a bpt_status error code; on an argument error
 * nothing is enqueued and `out` is untouched. */
int bpt_layer_fwd(const bpt_shape *shape, const void *x, const void *Wqkv, const void *bqkv,
                  const void *Wo, const void *bo, const void *W1, const void *b1, const void *W2,
                  const void *b2, int64_t B_q, int64_t B_kv, int causal, void *out,
                  void *workspace, size_t workspace_bytes, bpt_stream_t stream);

/* bpt_layer_workspace_bytes / bpt_layer_fwd with the FFN group size chosen
 * by the caller: ffn_rows tokens of the flattened [batch·seq] axis per group,
 * a multiple of B_q in [B_q, batch·seq], or 0 for the default of
 * bpt_layer_epilogue_rows. ffn_rows = batch·seq runs the FFN over the whole
 * sequence at once, i.e. without the blockwise FFN of the BPT review (§三,
 * 内存分析), whose activation memory it measures against. A value that is
 * not a multiple of B_q or out of range is BPT_ERR_BLOCK. */
int bpt_layer_workspace_bytes_ex(const bpt_shape *shape, int64_t B_q, int64_t B_kv, int causal,
                                 int64_t ffn_rows, size_t *bytes);
int bpt_layer_fwd_ex(const bpt_shape *shape, const void *x, const void *Wqkv, const void *bqkv,
                     const void *Wo, const void *bo, const void *W1, const void *b1,
                     const void *W2, const void *b2, int64_t B_q, int64_t B_kv, int causal,
                     int64_t ffn_rows, void *out, void *workspace, size_t workspace_bytes,
                     bpt_stream_t stream);

/* Training-mode forward: bpt_layer_fwd_ex with dropout of rate dropout_p on
 * both residual branches,
 *     y   = x + D0 ∘ (A·Woᵀ + bo) / (1 - p),
 *     out = y + D1 ∘ (max(0, y·W1ᵀ + b1)·W2ᵀ + b2) / (1 - p).
 * The BPT review's memory analysis (§三, 内存分析) counts a b·c·h dropout mask
 * in the blockwise FFN and its JAX listing gives each FFN chunk its own
 * dropout stream; the PyTorch 2.3 MHSA page (§5) drops the projected
 * attention output before the residual. Attention probabilities are not
 * dropped. Masks: element (token t = batch·seq + position, channel j) of site
 * z (0: attention branch, 1: FFN branch) is dropped iff the 16-bit uniform
 * number j % 16 of Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC 2011) with
 * key (seed, z) and counter (t, j / 16, 0, 0) is below T = round(p·65536);
 * uniform i is bits 16·(i % 4) .. 16·(i % 4) + 15 of output word i / 4. Kept
 * values are scaled by 65536 / (65536 - T), so the drop probability is
 * exactly T / 65536. The masks depend only on (seed, site, token, channel),
 * not on B_q, B_kv or ffn_rows. dropout_p = 0 is bpt_layer_fwd_ex exactly.
 * dropout_p outside [0, 1) (or NaN) is BPT_ERR_DROPOUT. Other arguments,
 * layouts, ownership and errors as bpt_layer_fwd_ex. */
int bpt_layer_fwd_train(const bpt_shape *shape, const void *x, const void *Wqkv,
                        const void *bqkv, const void *Wo, const void *bo, const void *W1,
                        const void *b1, const void *W2, const void *b2, int64_t B_q,
                        int64_t B_kv, int causal, int64_t ffn_rows, double dropout_p,
                        uint64_t seed, void *out, void *workspace, size_t workspace_bytes,
                        bpt_stream_t stream);

/* Backward pass of the inference forward (dropout off), bf16 only: for an
 * upstream gradient dout = dL/d out [batch, seq, h] (bf16), writes dx
 * [batch, seq, h] (bf16) and the fp32 gradients of every weight and bias, each
 * in its parameter's layout ([out, in] weights): dWqkv [3h, h], dbqkv [3h],
 * dWo [h, h], dbo [h], dW1 [f, h], db1 [f], dW2 [h, f], db2 [h]. Each is
 * overwritten, not accumulated. The forward is recomputed inside the call,
 * block by block (the BPT review, §三: the method composes with
 * rematerialisation): the attention keeps only each row's log-sum-exp and the
 * FFN's hidden activations exist for one group of rows at a time (the
 * forward's group size); no seq × seq or seq × f array exists. The chain rule,
 * with Z = Q·Kᵀ/√d and P = softmax(Z): dV = Pᵀ·dO, dZ = P ∘ (dO·Vᵀ − rowsum(dO ∘
 * O)), dQ = dZ·K/√d, dK = dZᵀ·Q/√d; the derivative of max(0, v) at 0 is 0.
 * Inputs and weights as bpt_layer_fwd; ffn_rows as bpt_layer_fwd_ex (0: the
 * default group size). workspace: device scratch of at least
 * bpt_layer_bwd_workspace_bytes bytes, owned by the caller. Errors as
 * bpt_layer_fwd_ex, plus BPT_ERR_DTYPE for fp32 shapes; the outputs may not
 * overlap each other, an input or the workspace (BPT_ERR_ALIAS).
 * Asynchronous on `stream`. */
int bpt_layer_bwd_workspace_bytes(const bpt_shape *shape, int64_t B_q, int64_t B_kv, int causal,
                                  int64_t ffn_rows, size_t *bytes);
int bpt_layer_bwd(const bpt_shape *shape, const void *x, const void *Wqkv, const void *bqkv,
                  const void *Wo, const void *bo, const void *W1, const void *b1, const void *W2,
                  const void *b2, int64_t B_q, int64_t B_kv, int causal, int64_t ffn_rows,
                  const void *dout, void *dx, float *dWqkv, float *dbqkv, float *dWo, float *dbo,
                  float *dW1, float *db1, float *dW2, float *db2, void *workspace,
                  size_t workspace_bytes, bpt_stream_t stream);

/* Backward pass of the training-mode forward (bpt_layer_fwd_train with the
 * same dropout_p and seed), bf16 only. The masks depend only on (seed, site,
 * token, channel), so they are regenerated, not stored. Each dropped branch
 * is its mask times 65536 / (65536 - T) times the undropped branch, and the
 * chain rule passes the branch's upstream gradient through the same factor:
 *     dW2, db2 and dH take dout ∘ M1 (the FFN branch),
 *     dWo, dbo and the attention's dO take dy ∘ M0 (the attention branch),
 * while the residual paths keep the unmasked dout and dy (dy = dout + dH·W1,
 * dx = dy + dQKV·Wqkv). The BPT review's memory analysis (§三, 内存分析)
 * counts the training FFN's dropout mask; the PyTorch 2.3 MHSA page (§5)
 * places the attention branch's. dropout_p = 0 is bpt_layer_bwd exactly;
 * dropout_p outside [0, 1) (or NaN) is BPT_ERR_DROPOUT. Arguments, workspace
 * (bpt_layer_bwd_workspace_bytes), outputs, ownership and errors otherwise as
 * bpt_layer_bwd. */
int bpt_layer_bwd_train(const bpt_shape *shape, const void *x, const void *Wqkv,
                        const void *bqkv, const void *Wo, const void *bo, const void *W1,
                        const void *b1, const void *W2, const void *b2, int64_t B_q,
                        int64_t B_kv, int causal, int64_t ffn_rows, double dropout_p,
                        uint64_t seed, const void *dout, void *dx, float *dWqkv, float *dbqkv,
                        float *dWo, float *dbo, float *dW1, float *db1, float *dW2, float *db2,
                        void *workspace, size_t workspace_bytes, bpt_stream_t stream);

/* A training step without the recomputation: a forward that leaves its
 * activations where the backward reads them, and the backward from them.
 *
 * bpt_layer_fwd_for_bwd computes out as bpt_layer_fwd_train does (dropout_p
 * = 0: as bpt_layer_fwd_ex). It writes into `workspace` what the backward
 * would otherwise recompute: Q (scaled) and K head-major, V transposed, the
 * attention output A with each row's log-sum-exp, and y = x + A·Woᵀ + bo
 * (its branch through the dropout mask in training mode). The attention runs
 * at the 256-row, 64-key tile whatever B_q and B_kv, the tile that writes
 * the log-sum-exp and that the recomputing backward uses too. B_q still sets
 * the FFN group size (with ffn_rows, as bpt_layer_fwd_ex). workspace: at
 * least bpt_layer_bwd_workspace_bytes bytes. out may not overlap x (the
 * backward reads x again), a weight or the workspace (BPT_ERR_ALIAS).
 *
 * bpt_layer_bwd_from_fwd is bpt_layer_bwd_train without the recomputed
 * forward: it starts from the workspace that bpt_layer_fwd_for_bwd filled.
 * Between the two calls the caller keeps that workspace unchanged and passes
 * the same shape, x, weights, B_q, B_kv, causal, ffn_rows, dropout_p and
 * seed (the library keeps no state, so it cannot check this). The backward
 * consumes what the forward kept (it may overwrite it), so every
 * bpt_layer_bwd_from_fwd needs its own bpt_layer_fwd_for_bwd before it. The
 * gradients are bitwise those of bpt_layer_bwd_train with the same
 * arguments, because the forward part runs the same kernels on the same
 * inputs.
 *
 * The pair holds 5·b·s·h bf16 activations and b·heads·s floats between the
 * calls, all inside the backward's workspace: memory still linear in s, no
 * seq × seq or seq × f array, as the BPT review's memory analysis (§三)
 * requires. Arguments otherwise, outputs, ownership and errors as
 * bpt_layer_bwd_train; both calls are asynchronous on `stream`. */
int bpt_layer_fwd_for_bwd(const bpt_shape *shape, const void *x, const void *Wqkv,
                          const void *bqkv, const void *Wo, const void *bo, const void *W1,
                          const void *b1, const void *W2, const void *b2, int64_t B_q,
                          int64_t B_kv, int causal, int64_t ffn_rows, double dropout_p,
                          uint64_t seed, void *out, void *workspace, size_t workspace_bytes,
                          bpt_stream_t stream);
int bpt_layer_bwd_from_fwd(const bpt_shape *shape, const void *x, const void *Wqkv,
                           const void *bqkv, const void *Wo, const void *bo, const void *W1,
                           const void *b1, const void *W2, const void *b2, int64_t B_q,
                           int64_t B_kv, int causal, int64_t ffn_rows, double dropout_p,
                           uint64_t seed, const void *dout, void *dx, float *dWqkv,
                           float *dbqkv, float *dWo, float *dbo, float *dW1, float *db1,
                           float *dW2, float *db2, void *workspace, size_t workspace_bytes,
                           bpt_stream_t stream);

/* Test hook: the keep mask that bpt_layer_fwd_train applies at dropout site
 * `site` (0 or 1) for tokens token0 .. token0 + tokens - 1 and channels
 * 0 .. channels - 1, written to the device buffer `keep` as one byte per
 * element (1 = kept, 0 = dropped), row-major [tokens, channels]. Same
 * generator code as the layer's epilogue. channels must be a multiple of 16
 * and dropout_p in [0, 1) (else BPT_ERR_DROPOUT); tokens, channels >= 0 and
 * token0 >= 0 (else BPT_ERR_SHAPE); keep must be non-NULL and 16-byte
 * aligned when the mask is non-empty. Asynchronous on `stream`. */
int bpt_debug_dropout_keep(int64_t tokens, int64_t channels, int64_t token0, double dropout_p,
                           uint64_t seed, int site, void *keep, bpt_stream_t stream);

/* Test hook, same kernels as bpt_layer_fwd_ex (ffn_rows as there, 0: the
 * default FFN group): runs the layer and also copies the merged-head
 * attention output A [batch, seq, h] into A_out, the first-residual
 * activation y [batch, seq, h] into y_out, and the hidden activations
 * H = max(0, y·W1ᵀ + b1) of the LAST FFN group into H_out: rows
 * T - n .. T - 1 of the flattened token axis (T = batch·seq, G the group
 * size, n = T - G·floor((T - 1) / G)), as [n, ffn], i.e. the bounded
 * scratch as the last group's W2 product read it. Any of A_out, y_out,
 * H_out may be NULL to skip it; all have the call's dtype; they may not
 * overlap each other, an input or the workspace (BPT_ERR_ALIAS). */
int bpt_debug_intermediates(const bpt_shape *shape, const void *x, const void *Wqkv,
                            const void *bqkv, const void *Wo, const void *bo, const void *W1,
                            const void *b1, const void *W2, const void *b2, int64_t B_q,
                            int64_t B_kv, int causal, int64_t ffn_rows, void *out, void *A_out,
                            void *y_out, void *H_out, void *workspace, size_t workspace_bytes,
                            bpt_stream_t stream);

/* Test and timing hook: only the QKV projection and the blockwise attention
 * of bpt_layer_fwd (the same kernels), writing A [batch, seq, h] to A_out.
 * With run_qkv == 0 the projection is skipped and the Q/K/V already in the
 * workspace (from an earlier call with the same shape and workspace) are
 * reused, so the attention kernel can be timed alone. */
int bpt_debug_attention(const bpt_shape *shape, const void *x, const void *Wqkv,
                        const void *bqkv, int64_t B_q, int64_t B_kv, int causal, int run_qkv,
                        void *A_out, void *workspace, size_t workspace_bytes,
                        bpt_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer
 * of bpt_layer_fwd_ex (same kernels, same schedule, bitwise the same out)
 * with its workspace taken from a fixed scratch array that the library holds
 * in device memory, BPT_NOALLOC_SCRATCH_BYTES per GPU it runs on, from the
 * first call on that GPU until the process ends. The caller passes inputs,
 * weights and out only. Nothing is allocated on the call path (no hipMalloc,
 * no hipFree, no allocating library routine).
 * Errors: as bpt_layer_fwd_ex; BPT_ERR_SCRATCH (before anything is
 * enqueued) when bpt_layer_workspace_bytes_ex(shape, B_q, B_kv, causal,
 * ffn_rows) exceeds BPT_NOALLOC_SCRATCH_BYTES (a smaller ffn_rows shrinks
 * the FFN's share); BPT_ERR_HIP if the scratch's device address cannot be
 * obtained. Every call on one GPU uses the same scratch: calls that overlap
 * in time on one GPU (on different streams, or from different threads
 * without ordering) race and give undefined results; calls ordered on one
 * stream are safe. The scratch keeps the last call's contents; the layer
 * reads nothing from it that the same call did not write first. */
#define BPT_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int bpt_layer_fwd_noalloc(const bpt_shape *shape, const void *x, const void *Wqkv,
                          const void *bqkv, const void *Wo, const void *bo, const void *W1,
                          const void *b1, const void *W2, const void *b2, int64_t B_q,
                          int64_t B_kv, int causal, int64_t ffn_rows, void *out,
                          bpt_stream_t stream);

/* Algorithmic FLOPs of one layer forward: 6bsh² (QKV) + 2bsh² (Wo) + 4bshf
 * (FFN) + attention, where attention counts 4·d FLOPs per (query, key) pair
 * per head that the softmax keeps: 4bs²h non-causal, 2bhs(s+1) causal.
 * Bias, residual, ReLU and softmax element work are not counted. Returns a
 * negative value for an invalid shape. */
double bpt_layer_algorithmic_flops(const bpt_shape *shape, int causal);

/* The attention tile a call with these block sizes runs: *rows = query
 * rows per workgroup, *keys = keys per LDS stage. bf16: the tile B_q and
 * B_kv select (see the conventions above); fp32: a fixed 64 × 32 tile.
 * Errors as bpt_layer_workspace_bytes; rows / keys are host pointers. */
int bpt_layer_attention_tile(const bpt_shape *shape, int64_t B_q, int64_t B_kv, int64_t *rows,
                             int64_t *keys);

/* Static text for a status code. */
const char *bpt_status_string(int status);

/* Library version string. */
const char *bpt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BPT_H_ */
