/*
 * libtpshard — one tensor-parallel rank's shard of a Megatron-style
 * Transformer layer, as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   "Megatron-LM：张量并行与大规模训练", §2.1 MLP 层的张量并行 — the MLP
 *     Z = GeLU(X A) B with A split by columns into A_i [h, 4h/N] and B by rows
 *     into B_i [4h/N, h]; each rank forms the partial Z_i = GeLU(X A_i) B_i with no
 *     communication and one all-reduce adds the Z_i.
 *   same page, §2.2 Self-Attention 的张量并行 — heads split across ranks, the
 *     output projection split by rows, one all-reduce after it.
 *   m.youleyou.com/wenzhang/3143730, 一、切分权重 §1.1/§1.2 and 二、MLP层 §2.1 — the
 *     row/column splits with their backward (g's backward copies dZ to every rank,
 *     f's backward adds the ranks' input gradients); 三、Self-Attention层 §3.1 —
 *     column split of the Q, K, V weights by whole heads, head count divisible
 *     by the rank count; 三、§3.2 — the layer's backward and its two all-reduces;
 *     四、Embedding层 §4.1 — vocabulary-parallel input embedding that zeroes ids a
 *     rank does not hold; §4.2 — the output layer through the same row-split table;
 *     五、Cross-Entropy层 — the loss from per-rank sums of exp, without gathering
 *     the logits; 二、§2.2 — an all-reduce is a reduce-scatter plus an all-gather.
 *   www.discosf.com/news/5875844, 2.3 序列并行与激活重计算 — LayerNorm and Dropout
 *     on each rank's slice of the sequence; activation recompute in the backward.
 *   "Megatron-LM 介绍" (apxml.com), 核心贡献 item 1 — ColumnParallelLinear.
 *
 * Common conventions for every call:
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major and
 *     contiguous, 16-byte aligned. Nothing is allocated or freed by the library,
 *     no call synchronises or clears memory, and every call may be recorded in a
 *     HIP graph. Scratch memory comes from caller workspaces sized by the
 *     matching *_workspace() function. A workspace whose call runs a bf16
 *     product whose tiles of 256 x 192 output elements leave the last round of
 *     the 256-workgroup grid at most half full also holds that product's
 *     stream-K area (100.7 MB of float32 partial tiles, after the call's other
 *     scratch): its k-range is split over all 256 workgroups and the split tiles
 *     are summed in a fixed order, so results are reproducible. Calls that share
 *     one workspace must not overlap in time.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream of
 *     the current device. Work is enqueued asynchronously on it; the call returns
 *     after the launches, not after the kernels finish.
 *   - Every argument is checked on the host before any launch. On a bad argument
 *     nothing is launched and TP_ERR_INVALID_ARG / TP_ERR_UNSUPPORTED /
 *     TP_ERR_WORKSPACE is returned; a failed launch returns TP_ERR_HIP. A
 *     non-OK return sets a per-thread message readable with tp_last_error().
 *     Nothing aborts or throws across this interface.
 *   - bf16 means bfloat16 (1 sign, 8 exponent, 7 mantissa bits); every
 *     float32 -> bf16 store rounds to nearest, ties to even. Products are
 *     accumulated in float32.
 *   - Matrix dimensions named h, f, K, N below must be multiples of 8 (16-byte
 *     vectors); token counts M may be any value >= 0 (M = 0 launches nothing).
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tp_status {
  TP_OK = 0,
  TP_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size, lo > hi, ... */
  TP_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels handle (alignment, dims % 8) */
  TP_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace() size */
  TP_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} tp_status;

typedef enum tp_dtype { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

typedef enum tp_activation { TP_ACT_NONE = 0, TP_ACT_GELU = 1 } tp_activation;

/* Optional stream-K workspace of the linear layers and the MLP forward: `ws` may be
 * NULL (every product then runs one output tile per workgroup); a non-NULL `ws`
 * must hold at least the size the matching *_workspace() query returns, else
 * TP_ERR_WORKSPACE. A bf16 product whose 256 x 192 tiles leave the last round of
 * the 256-workgroup grid at most half full then splits its k-range over all
 * workgroups (the query returns 0 when no product of the call does). */

/* Workspace of tp_column_linear / tp_row_linear for an [M, K] x [K, N] product
 * (0 for TP_F32, which never uses one). */
size_t tp_linear_workspace(tp_dtype dt, int64_t M, int64_t K, int64_t N);

/* Column-parallel linear layer of one rank: Y = act(X W).
 * [Megatron-LM 介绍, 核心贡献 item 1 (ColumnParallelLinear); Megatron-LM：张量并行与
 *  大规模训练, §2.1, 列并行 — the rank holds a column block W = A_i of A.]
 *   dt     TP_BF16: X, W, U_out, Y_out are bf16. TP_F32: all float32.
 *   X      [M, K]   the replicated layer input.
 *   W      [K, N]   the rank's column block, stored [in, out].
 *   U_out  [M, N]   nullable; receives X W (before the activation) when act is
 *                   TP_ACT_GELU. Must be NULL when act is TP_ACT_NONE.
 *   Y_out  [M, N]   act(X W). GeLU is the exact form u * Phi(u).
 *   ws     nullable stream-K workspace of tp_linear_workspace(dt, M, K, N) bytes.
 * K and N must be multiples of 8; a bf16 operand must stay below 2 GiB
 * (TP_ERR_UNSUPPORTED otherwise). */
tp_status tp_column_linear(tp_dtype dt, int64_t M, int64_t K, int64_t N,
                           const void* X, const void* W, void* U_out, void* Y_out,
                           int act, void* ws, size_t ws_bytes, void* stream);

/* Row-parallel linear layer of one rank: the float32 partial Z = Y W that the
 * all-reduce adds over ranks.
 * [Megatron-LM：张量并行与大规模训练, §2.1, 行并行 — Z_i = Y_i B_i.]
 *   Y [M, K] (dt), W [K, N] (dt) the rank's row block, Z_out [M, N] float32.
 *   ws nullable stream-K workspace of tp_linear_workspace(dt, M, K, N) bytes.
 * K and N must be multiples of 8; bf16 operands below 2 GiB. */
tp_status tp_row_linear(tp_dtype dt, int64_t M, int64_t K, int64_t N,
                        const void* Y, const void* W, float* Z_out,
                        void* ws, size_t ws_bytes, void* stream);

/* MLP forward of one rank: U_i = X A_i, Y_i = GeLU(U_i), Z_i = Y_i B_i.
 * [Megatron-LM：张量并行与大规模训练, §2.1 MLP 层的张量并行 and its pseudo-code;
 *  m.youleyou.com/wenzhang/3143730, 二、MLP层 §2.1.]
 *   X [M, h], A_i [h, f], B_i [f, h] (dt); f is the rank's share 4h/N.
 *   U_i [M, f] (dt) nullable — saved pre-activation for the backward.
 *   Y_i [M, f] (dt) required — the activation, also needed by the backward.
 *   Z_i [M, h] float32 — this rank's partial of Z (sum over ranks with
 *   tp_shard_sum in place of the all-reduce).
 *   ws nullable stream-K workspace of tp_mlp_fwd_workspace(dt, M, h, f) bytes
 *   (shared by the two products, which run one after the other).
 * h and f must be multiples of 8; bf16 operands below 2 GiB. Two kernels:
 * column GEMM + GeLU epilogue, then row GEMM. */
tp_status tp_mlp_fwd(tp_dtype dt, int64_t M, int64_t h, int64_t f,
                     const void* X, const void* A_i, const void* B_i,
                     void* U_i, void* Y_i, float* Z_i, void* ws, size_t ws_bytes, void* stream);
size_t tp_mlp_fwd_workspace(tp_dtype dt, int64_t M, int64_t h, int64_t f);

/* MLP backward of one rank, bf16 inputs, float32 outputs. With the replicated
 * upstream gradient dZ (g's backward is the identity):
 *   dU_i = (dZ B_i^T) * GeLU'(U_i)   -> bf16 [M, f] in the workspace
 *   dB_i = Y_i^T dZ                  -> float32 [f, h]
 *   dA_i = X^T dU_i                  -> float32 [h, f]
 *   dX_i = dU_i A_i^T                -> float32 [M, h], the partial that f's
 *                                       backward adds over ranks.
 * [m.youleyou.com/wenzhang/3143730, 一、切分权重 §1.1/§1.2 (backward of the row and
 *  column splits) and 二、MLP层 §2.1 (g's and f's backward).]
 *   X [M,h], A_i [h,f], B_i [f,h], U_i [M,f], Y_i [M,f], dZ [M,h]: bf16.
 *   Any of dX_i, dA_i, dB_i may be NULL to skip that product.
 *   U_i and Y_i may be NULL: activation recompute. U_i and Y_i are then formed
 *   again from X and A_i by the forward's own column GEMM + GeLU (same bits),
 *   at the cost of one more M x f x h product. [discosf.com/news/5875844, §2.3
 *   序列并行与激活重计算 (activation recomputation).]
 *   ws: device workspace of at least tp_mlp_bwd_workspace(M, h, f) bytes, or
 *   tp_mlp_bwd_recompute_workspace(M, h, f) bytes when U_i or Y_i is NULL.
 * The backward is bf16 only (the float32 path serves the tiny forward
 * configuration), so it takes no dtype. Operands must stay below 2 GiB.
 * Kernels run in the order [U/Y recompute], dU, dB, dA, dX on `stream`. */
tp_status tp_mlp_bwd(int64_t M, int64_t h, int64_t f,
                     const void* X, const void* A_i, const void* B_i,
                     const void* U_i, const void* Y_i, const void* dZ,
                     float* dX_i, float* dA_i, float* dB_i,
                     void* ws, size_t ws_bytes, void* stream);
size_t tp_mlp_bwd_workspace(int64_t M, int64_t h, int64_t f);
/* Workspace of tp_mlp_bwd when U_i or Y_i is NULL: dU_i, U_i and Y_i, bf16 [M, f] each. */
size_t tp_mlp_bwd_recompute_workspace(int64_t M, int64_t h, int64_t f);

/* Allocation-free MLP backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, products and results as tp_mlp_bwd with U_i and
 * Y_i given, but no workspace: dU_i lives in a scratch array of the library,
 * tp_mlp_bwd_noalloc_max_bytes() bytes (80 MiB) per device, held from the
 * library's first use on a device until the process ends. Nothing in it needs
 * clearing between calls; every call on one device shares it, so calls that
 * overlap in time on one device race. The products run one tile per workgroup
 * (no stream-K split), so results can differ from tp_mlp_bwd's by float32
 * summation order.
 *   M * f * 2 bytes above the scratch size -> TP_ERR_UNSUPPORTED; U_i or Y_i
 *   NULL (activation recompute would need more scratch) -> TP_ERR_INVALID_ARG;
 *   other arguments as tp_mlp_bwd. No hipMalloc, hipFree or allocating library
 *   call is made; the first call on a device looks up the scratch's address. */
tp_status tp_mlp_bwd_noalloc(int64_t M, int64_t h, int64_t f,
                             const void* X, const void* A_i, const void* B_i,
                             const void* U_i, const void* Y_i, const void* dZ,
                             float* dX_i, float* dA_i, float* dB_i, void* stream);
size_t tp_mlp_bwd_noalloc_max_bytes(void);

/* Causal (or full) softmax attention over one rank's local heads, bf16.
 * [Megatron-LM：张量并行与大规模训练, §2.2; m.youleyou.com/wenzhang/3143730,
 *  三、Self-Attention层 §3.1.]
 *   QKV [b*s, 3*Hl*d] bf16: per token [Q heads | K heads | V heads], local head j
 *       at columns j*d .. (j+1)*d of each block.
 *   O   [b*s, Hl*d] bf16: O_j = softmax(Q_j K_j^T / sqrt(d)) V_j per sequence;
 *       with causal != 0 query t sees keys u <= t.
 * d must be 64, 128 or 384 (GPT-3's 12288 / 96 heads and PaLM's 18432 / 48 heads;
 * "Megatron-LM：张量并行与大规模训练", §5.6 and §5.7), and
 * (s + 128) * 3 * n_heads_local * d * 2 < 2^31 (one sequence's rows are addressed
 * with 32-bit byte offsets); otherwise TP_ERR_UNSUPPORTED. Softmax in float32, P
 * rounded to bf16 for the P V product. */
tp_status tp_attn_core(int64_t b, int64_t s, int64_t n_heads_local, int64_t d_head,
                       int causal, const void* QKV, void* O, void* stream);

/* One rank's attention block: QKV = X Wqkv_i (bf16), O = tp_attn_core(QKV),
 * out_partial = O Wo_i (float32 partial added by the all-reduce).
 * [Megatron-LM：张量并行与大规模训练, §2.2 (QKV projection split by heads,
 *  row-parallel output projection); m.youleyou.com/wenzhang/3143730, 三、
 *  Self-Attention层 §3.1 (column split of Q, K, V by heads; B split by rows).]
 *   X [b*s, h] bf16; Wqkv_i [h, 3*Hl*d] bf16; Wo_i [Hl*d, h] bf16;
 *   out_partial [b*s, h] float32.
 *   ws: at least tp_attn_fwd_workspace(b, s, h, Hl, d) bytes; on return it holds
 *   QKV bf16 [b*s, 3*Hl*d] followed (at a 256-byte aligned offset) by O bf16
 *   [b*s, Hl*d], then the stream-K area when one of the two products uses it.
 *   GEMM operands must stay below 2 GiB. */
tp_status tp_attn_fwd(int64_t b, int64_t s, int64_t h, int64_t n_heads_local,
                      int64_t d_head, int causal, const void* X, const void* Wqkv_i,
                      const void* Wo_i, float* out_partial, void* ws, size_t ws_bytes,
                      void* stream);
size_t tp_attn_fwd_workspace(int64_t b, int64_t s, int64_t h, int64_t n_heads_local,
                             int64_t d_head);

/* Vocabulary-parallel input embedding of one rank (bit copy, no arithmetic):
 *   out[t, :] = E_i[ids[t] - lo, :] if lo <= ids[t] < hi, else zeros.
 * [m.youleyou.com/wenzhang/3143730, 四、Embedding层 §4.1.] Ids outside [lo, hi) —
 * including ids outside the whole vocabulary — give zero rows; that is not an error.
 *   ids [n_tokens] int32; E_i [hi-lo, h] bf16; out [n_tokens, h] bf16.
 *   Requires 0 <= lo < hi and h a multiple of 8. */
tp_status tp_vocab_embed(const int32_t* ids, int64_t n_tokens, const void* E_i,
                         int64_t lo, int64_t hi, int64_t h, void* out, void* stream);

/* tp_attn_core that also writes the per-query log-sum-exp the backward needs:
 *   lse float32 [b, Hl, s] = log sum_u exp(q.k_u / sqrt(d)) over the visible keys.
 * P enters the P V product as two bf16 operands, bf16(P) and bf16(P - bf16(P)),
 * so the stored O (which the backward's gradients are formed from) carries
 * about 16 bits of P instead of 8. */
tp_status tp_attn_core_train(int64_t b, int64_t s, int64_t n_heads_local, int64_t d_head, int causal,
                             const void* QKV, void* O, float* lse, void* stream);

/* Training forward of the attention shard: as tp_attn_fwd, but Q|K|V, the head
 * outputs O and the per-query log-sum-exp go to caller buffers, kept for the backward.
 *   QKV bf16 [b*s, 3*Hl*d], O bf16 [b*s, Hl*d], lse float32 [b, Hl, s]:
 *   lse = log sum_u exp(q.k_u / sqrt(d)) over the visible keys (natural log). */
tp_status tp_attn_fwd_train(int64_t b, int64_t s, int64_t h, int64_t n_heads_local, int64_t d_head,
                            int causal, const void* X, const void* Wqkv_i, const void* Wo_i,
                            float* out_partial, void* QKV, void* O, float* lse, void* stream);

/* Attention core backward over the local heads [m.youleyou.com/wenzhang/3143730,
 * 三、Self-Attention层 §3.2 (the layer's backward, per head, then the input
 * gradient's all-reduce); the head formula as in tp_attn_core]:
 *   P = exp(q.k / sqrt(d) - lse), dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO*O)),
 *   dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d); written as bf16 dQKV [b*s, 3*Hl*d] in the
 *   [Q | K | V] layout of QKV. dO bf16 [b*s, Hl*d]; lse from tp_attn_fwd_train.
 *   Deterministic (no atomics). ws: tp_attn_core_bwd_workspace(b, s, Hl, d) bytes
 *   (rowsum(dO*O) and the float32 partials of walks cut into chunks). */
tp_status tp_attn_core_bwd(int64_t b, int64_t s, int64_t n_heads_local, int64_t d_head, int causal,
                           const void* QKV, const void* O, const void* dO, const float* lse,
                           void* dQKV, void* ws, size_t ws_bytes, void* stream);
size_t tp_attn_core_bwd_workspace(int64_t b, int64_t s, int64_t n_heads_local, int64_t d_head);

/* Backward of one rank's attention shard [same page, 三、§3.2; "Megatron-LM：张量并行与
 * 大规模训练" §2.2]: with dOut bf16 [b*s, h] (replicated, the output all-reduce's
 * backward is the identity):
 *   dWo_i = O^T dOut (float32 [Hl*d, h]), dO = dOut Wo_i^T (bf16, workspace),
 *   dQKV = core backward (bf16, workspace), dWqkv_i = X^T dQKV (float32 [h, 3*Hl*d]),
 *   dX_i = dQKV Wqkv_i^T (float32 [b*s, h], the partial the input all-reduce adds).
 *   QKV, O, lse: saved by tp_attn_fwd_train. ws: tp_attn_bwd_workspace(...) bytes. */
tp_status tp_attn_bwd(int64_t b, int64_t s, int64_t h, int64_t n_heads_local, int64_t d_head,
                      int causal, const void* X, const void* Wqkv_i, const void* Wo_i,
                      const void* QKV, const void* O, const float* lse, const void* dOut,
                      float* dX_i, float* dWqkv_i, float* dWo_i, void* ws, size_t ws_bytes,
                      void* stream);
size_t tp_attn_bwd_workspace(int64_t b, int64_t s, int64_t h, int64_t n_heads_local,
                             int64_t d_head);

/* Vocabulary-parallel output layer + cross-entropy, one rank's part
 * [m.youleyou.com/wenzhang/3143730, 四、Embedding层 §4.2 (the output layer maps
 *  back to the vocabulary with the row-split word embedding) and 五、Cross-Entropy层
 *  (per-rank row sums of e = exp(logit), all-reduced into the softmax
 *  denominator, then each row's cross-entropy and the scalar sum)]:
 *   logits_i = H E_i^T                       (float32, never stored)
 *   rowmax_i[m] = max_n logits_i[m, n]        -> float32 [M]
 *   sumexp_i[m] = sum_n exp(logits_i[m, n] - rowmax_i[m]) -> float32 [M]
 *   tlogit_i[m] = logits_i[m, t[m] - lo] if lo <= t[m] < hi, else 0 -> float32 [M]
 *   H [M,h] and E_i [hi-lo, h]: bf16; targets [M] int32 (device).
 *   The page's sum of e over the rank's columns is exp(rowmax_i) * sumexp_i: it is
 *   carried relative to the row maximum so that no logit overflows float32.
 *   The GEMM's epilogue reduces each row over each 48-column slot to (max, sum of
 *   exp) and stores the target logits; the slots are then merged in column order,
 *   so the results are reproducible bit for bit.
 *   Requires 0 <= lo < hi, h and hi-lo multiples of 8, operands below 2 GiB.
 *   ws: at least tp_vocab_ce_workspace(M, h, lo, hi) bytes (the slot statistics,
 *   8 bytes per row and slot, four slots per 192 columns, and the GEMM's stream-K
 *   area); its contents on return are unspecified. */
tp_status tp_vocab_ce_partials(int64_t M, int64_t h, int64_t lo, int64_t hi, const void* H,
                               const void* E_i, const int32_t* targets, float* rowmax_i,
                               float* sumexp_i, float* tlogit_i, void* ws, size_t ws_bytes,
                               void* stream);
size_t tp_vocab_ce_workspace(int64_t M, int64_t h, int64_t lo, int64_t hi);

/* The all-reduce stand-ins of the vocabulary-parallel loss on one GPU, and the
 * loss itself [same page, 五、Cross-Entropy层]:
 *   mx[m] = max_i rowmax_parts[i][m] (a max all-reduce),
 *   S[m] = sum_i sumexp_parts[i][m] * exp(rowmax_parts[i][m] - mx[m]) (rank order),
 *   T[m] = sum_i tlogit_parts[i][m], loss_rows[m] = mx[m] + log S[m] - T[m],
 *   *loss_sum = sum_m loss_rows[m] (fixed order).
 *   rowmax_parts, sumexp_parts, tlogit_parts: HOST arrays of n_parts device
 *   pointers, 1 <= n_parts <= 16. loss_rows [M] and loss_sum [1]: float32 (device). */
tp_status tp_vocab_ce_loss(int64_t M, const float* const* rowmax_parts,
                           const float* const* sumexp_parts, const float* const* tlogit_parts,
                           int n_parts, float* loss_rows, float* loss_sum, void* stream);

/* Sequence parallelism around the tensor-parallel MLP [www.discosf.com/news/5875844,
 * 2.3 序列并行与激活重计算 (LayerNorm and Dropout run on each rank's slice of the
 * sequence instead of on the whole sequence everywhere); m.youleyou.com/wenzhang/3143730,
 * 二、§2.2 (the all-reduce is a reduce-scatter followed by an all-gather)].
 * Rank i owns rows [i*s/N, (i+1)*s/N) of the sequence.
 *
 * LayerNorm of one rank's rows (the page does not write LayerNorm out; this is the
 * standard one): per row, mean and biased variance over h in float32,
 *   Y = bf16((X - mean) / sqrt(var + eps) * gamma + beta)   (round to nearest even)
 *   X [rows, h] float32, gamma/beta [h] float32, Y [rows, h] bf16; h % 8 == 0,
 *   h <= 32768. Y may point into the rows of a gathered [s, h] buffer. */
tp_status tp_layernorm(int64_t rows, int64_t h, const float* X, const float* gamma,
                       const float* beta, float eps, void* Y, void* stream);

/* All-gather stand-in on one GPU: out = [slices[0]; ...; slices[n-1]], each slice
 * bf16 [rows, h], out bf16 [n*rows, h]. slices: HOST array of n device pointers,
 * 1 <= n <= 16; h % 8 == 0. */
tp_status tp_sp_all_gather(int n_parts, const void* const* slices, int64_t rows, int64_t h,
                           void* out, void* stream);

/* Reduce-scatter stand-in for rank `rank`, fused with Dropout and the residual add:
 *   O = ((P_0 + P_1) + ...) + P_{n-1} over rows [rank*s/n, (rank+1)*s/n) (float32, rank order)
 *   out = residual + (keep ? O / keep_prob : 0)  (keep NULL: out = residual + O)
 * partials: HOST array of n device pointers to float32 [s, h]; residual and out float32
 * [s/n, h] (out may equal residual; residual NULL: no residual add, as in the backward,
 * where this is the all-gather's backward); keep: uint8 [s/n, h] (nonzero = kept, the
 * drawn mask is an input), 4-byte aligned, keep_prob in (0, 1]. s % n == 0, h % 8 == 0. */
tp_status tp_sp_reduce_scatter(int n_parts, const float* const* partials, int64_t s, int64_t h,
                               int rank, const float* residual, const uint8_t* keep,
                               float keep_prob, float* out, void* stream);

/* Backward of the sequence-parallel block on one rank's rows (the chain rule through
 * the operators above; the page gives the forward split only):
 *
 * LayerNorm backward: with xh = (X - mean) * rstd and g = dY * gamma per row,
 *   dX = rstd * (g - mean(g) - xh * mean(g * xh)) (+ dRes, the residual path's gradient,
 *   if not NULL), dgamma = sum_rows dY * xh, dbeta = sum_rows dY (this rank's partials,
 *   overwritten; the ranks' partials are then all-reduced). X, dY, dRes, dX float32
 *   [rows, h]; gamma, dgamma, dbeta float32 [h]; h % 8 == 0, h <= 24576.
 *   ws: tp_layernorm_bwd_workspace(rows, h) bytes. Deterministic. */
tp_status tp_layernorm_bwd(int64_t rows, int64_t h, const float* X, const float* gamma,
                           const float* dY, const float* dRes, float eps, float* dX,
                           float* dgamma, float* dbeta, void* ws, size_t ws_bytes, void* stream);
size_t tp_layernorm_bwd_workspace(int64_t rows, int64_t h);

/* Dropout backward into the MLP backward's bf16 input: out = bf16(keep ? dY / keep_prob : 0)
 * (keep NULL: out = bf16(dY)). dY float32 [rows, h], out bf16 [rows, h] (may point into the
 * rows of a gathered [s, h] buffer); keep 4-byte aligned. */
tp_status tp_sp_dropout_bwd(int64_t rows, int64_t h, const float* dY, const uint8_t* keep,
                            float keep_prob, void* out, void* stream);

/* Shard-sum standing in for the all-reduce of N partials on one GPU:
 *   out = ((P_0 + P_1) + P_2) + ... + P_{N-1}, elementwise, in float32, in this
 *   fixed order (so the result is reproducible bit for bit).
 * [Megatron-LM：张量并行与大规模训练, §2.1, 行并行 (Z = Z_1 + ... + Z_N);
 *  m.youleyou.com/wenzhang/3143730, 二、MLP层 §2.1 (g's forward adds the partials).]
 *   partials: HOST array of n_partials device pointers, 1 <= n_partials <= 16.
 *   dt TP_F32: float32 partials and out. TP_BF16: bf16 partials widened to
 *   float32, summed in order, the sum rounded once to bf16.
 *   out may alias partials[0]. numel >= 0. */
tp_status tp_shard_sum(tp_dtype dt, const void* const* partials, int n_partials,
                       int64_t numel, void* out, void* stream);

/* Human-readable name of a status code (static string). */
const char* tp_status_string(tp_status s);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* tp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TPSHARD_H */
