/*
 * sas.h -- C ABI of the MI355X (gfx950) gated block-sparse attention library.
 *
 * The library computes the training-time attention of SAS ("SAS: Simple
 * Attention Sparsification via End-to-End Optimization of Context Ranking",
 * arXiv 2609.13141): per query block, the always-kept current block (unit
 * gate, causal) plus the Top-K historical blocks chosen from selector scores,
 * each historical block carrying its softmax-normalised log gate inside the
 * attention softmax (Sec. 4.3, Eq. 9), and the matching backward pass
 * including the block log-gate gradient (App. E) and the selector-score
 * gradient (App. D.3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers owned by the caller.  The
 *    library never allocates, frees or retains device memory; scratch space
 *    is passed in explicitly (sas_gated_attn_bwd).
 *  - Every call validates its arguments on the host and, when they are
 *    valid, enqueues its kernels on `stream` (a hipStream_t; NULL = the
 *    default stream) and returns without synchronising.  Argument errors are
 *    reported BEFORE anything is enqueued; nothing is written then.
 *  - Return value: SAS_OK (0) or a negative sas_status.  sas_last_error()
 *    returns a thread-local message describing the last non-OK return.
 *  - No exceptions cross the ABI.  There is no global mutable state other
 *    than that thread-local message.
 *  - Outputs are overwritten, never accumulated: every element of every
 *    output buffer is written.
 *
 * Shapes and layouts (all contiguous, row-major, element strides implied):
 *    B  = batch, Hq = query heads, Hkv = kv heads (Hq % Hkv == 0, G = Hq/Hkv),
 *    N  = seq_len, D = head_dim, b = block_size (N % b == 0), C = N / b.
 *    q, d_o, dq           [B, Hq,  N, D]   (dtype: bf16 or fp32)
 *    o                    [B, Hq,  N, D]   (o_dtype: bf16 or fp32)
 *    k, v, dk, dv         [B, Hkv, N, D]   (dtype: bf16 or fp32)
 *    lse                  [B, Hq,  N]      fp32, natural-log LSE of each query row
 *    scores, log_gate,
 *    dlog_gate, dscores   [B, Hs, C, C]    fp32, row = query block i,
 *                                          column = context block m
 *    tau, sel_cnt         [B, Hs, C]       fp32 / int32
 *    sel_idx              [B, Hs, C, sel_cap] int32
 *  Query head h reads kv head h / G.  Hs = n_score_heads (Hkv by default):
 *  gates, threshold and selection are shared by the Hq / Hs query heads of a
 *  score head (by default the G heads of a kv group: the per-query-group block
 *  selection of the paper's grouped-query setting) and by the b queries of a
 *  query block; the gradient of a shared gate is the sum over its uses.
 *
 * Supported problem sizes: D in {64, 128}; b in {16, 32, 64}; C <= 8192;
 * K >= 0.  bf16 with D = 128 and b = 64 runs on the matrix-core (MFMA) path;
 * every other supported combination runs on a plain vector-ALU HIP path with
 * identical semantics.
 */
#ifndef SAS_H_
#define SAS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAS_ABI_VERSION 7

typedef enum sas_dtype {
  SAS_BF16 = 0, /* q/k/v/o/d_o/dq/dk/dv are bfloat16 (fp32 accumulation) */
  SAS_FP32 = 1  /* all tensors float32 */
} sas_dtype;

/* Gate activation (Sec. 4.1 "Components of learnable ranking", Tab. 1):
 * log g of a historical block from its selector score s.  The current block
 * keeps g0 = 1 in every variant (Eq. 4). */
typedef enum sas_gate_act {
  SAS_GATE_SOFTMAX = 0, /* log g_m = s_m - LSE_{historical}(s)  (Eq. 6, default) */
  SAS_GATE_SIGMOID = 1, /* log g_m = log sigmoid(s_m)          (Tab. 1 row 5)    */
  SAS_GATE_RAW = 2      /* log g_m = s_m, raw logit injection   (Tab. 1 row 6)    */
} sas_gate_act;

/* Gate position (Sec. 4.1, Tab. 1 rows 2 and 3). */
typedef enum sas_gate_pos {
  SAS_GATE_INNER = 0, /* o = softmax(q K^T + log g) V            (Eq. 9, default) */
  SAS_GATE_OUTER = 1  /* o = softmax(q K^T) (g . V): each block's value rows are
                         scaled by its gate after the softmax                   */
} sas_gate_pos;

/* Ranking preservation (Sec. 4.1, Eq. 7, Tab. 1 rows 7 and 8). */
typedef enum sas_gate_rank {
  SAS_GATE_SOFT = 0,    /* continuous gates log g (the method)                   */
  SAS_GATE_HARD_STE = 1 /* hard Top-K gates, straight-through estimator: the
                           forward gives the selected blocks unit gates (zero
                           bias); the backward gives every historical block a
                           gate gradient dg (selected: its dS sum; dropped: the
                           attention mass its tokens would get under the
                           selected set's normaliser, Eq. 7), written to
                           dlog_gate, and dscores = g (dg - sum_l g_l dg_l).
                           Softmax activation and inner position only.  The
                           dropped blocks' gradients are full-scope work: on
                           the matrix-core path one more kernel pass over
                           every historical block of each gate row.        */
} sas_gate_rank;

typedef enum sas_status {
  SAS_OK = 0,
  SAS_E_INVALID = -1,     /* malformed argument (null pointer, bad shape ...) */
  SAS_E_UNSUPPORTED = -2, /* well-formed but outside the supported sizes      */
  SAS_E_WORKSPACE = -3,   /* workspace missing or smaller than required       */
  SAS_E_CAPACITY = -4,    /* device-side: a row selected more than sel_cap    */
  SAS_E_HIP = -5          /* a HIP runtime call or kernel launch failed       */
} sas_status;

typedef struct sas_problem {
  int32_t batch;      /* B   >= 1                                            */
  int32_t n_q_heads;  /* Hq  >= 1                                            */
  int32_t n_kv_heads; /* Hkv >= 1, divides Hq                                */
  int32_t seq_len;    /* N   >= b, multiple of block_size                    */
  int32_t head_dim;   /* D   in {64, 128}                                    */
  int32_t block_size; /* b   in {16, 32, 64}                                 */
  int32_t budget_k;   /* K   >= 0: historical blocks kept per query block    */
  int32_t dtype;      /* a sas_dtype                                          */
  int32_t o_dtype;    /* sas_dtype of the forward output o (and of the o read
                         by the backward).  SAS_BF16 is the usual half-size
                         output; SAS_FP32 keeps o unrounded (the bf16 forward
                         then also splits P into two bf16 terms for the PV
                         product).  Must be SAS_FP32 when dtype is SAS_FP32.  */
  float sm_scale;     /* scale of q.k; <= 0 selects 1/sqrt(D).  It never
                         multiplies the log gate (App. E, Alg. 3/4).          */
  int32_t gate_act;   /* a sas_gate_act (SAS_GATE_SOFTMAX for the method)      */
  int32_t gate_pos;   /* a sas_gate_pos (SAS_GATE_INNER for the method).  Both
                         positions run on the matrix-core path for bf16 with
                         D = 128 and b = 64.                                   */
  int32_t gate_rank;  /* a sas_gate_rank (SAS_GATE_SOFT for the method)        */
  int32_t n_score_heads; /* Hs: rows of the gate tables per batch element.
                         0 or Hkv: one gate / selection per query group (the
                         per-group selection of the paper's GQA setting);
                         Hq: one per query head (the training kernel's
                         per-head log gates, App. E); score head s covers
                         query heads s*(Hq/Hs) .. +Hq/Hs-1.                  */
  const int32_t* seq_lens; /* optional DEVICE int32 [B]: valid tokens n_b of each
                         sequence (variable-length batch in the padded
                         [.., N, ..] layout; NULL = every sequence has N).
                         Sequence b has ceil(n_b / b) blocks, the last one
                         possibly ragged; query rows t >= n_b are padding
                         (o, lse, dq written as 0; they attend nothing and
                         contribute no gradient); gate rows i >= ceil(n_b / b)
                         select nothing (sel_cnt 0, tau +inf; log_gate still
                         written; dlog_gate and dscores 0).  Values outside
                         [0, N] are clamped into it.  Padding rows must hold
                         finite values (their content never reaches a valid
                         row).  bf16 / D = 128 / b = 64 problems run on
                         the matrix-core path.                                */
  const int32_t* cu_seqlens; /* optional DEVICE int32 [B + 1]: packed batch
                         (the cu_seqlens convention of varlen attention):
                         sequence b holds tokens cu_seqlens[b] ..
                         cu_seqlens[b+1]-1 of tensors laid out
                         q, o, dO, dq [T, Hq, D]; k, v, dk, dv [T, Hkv, D];
                         lse [Hq, T] (T = total_tokens); seq_len is then
                         the longest sequence's padded extent N (a multiple
                         of block_size; gate tables stay [B, Hs, C, C] with
                         C = N / block_size).  Blocks, ragged last blocks
                         and empty gate rows as for seq_lens; rows of
                         other sequences are never read as keys nor
                         written.  Offsets are clamped into [0, T] and
                         lengths into [0, N].  Exclusive with seq_lens.
                         bf16 / D = 128 / b = 64 problems run on the
                         matrix-core path.                                    */
  int64_t total_tokens; /* T: rows per head of the packed tensors, in
                         [1, B * N] (ignored without cu_seqlens)              */
} sas_problem;

/* ABI version of the loaded library (SAS_ABI_VERSION). */
int32_t sas_abi_version(void);

/* Thread-local description of the last non-OK status returned on this thread
 * ("" if none).  The pointer stays valid until the next library call on the
 * same thread. */
const char* sas_last_error(void);

/*
 * sas_gate_threshold -- gate activation and Top-K as a threshold.
 *
 * Defined by Sec. 4.1 Eq. 4 (current block has unit gate), Sec. 4.2.2 Eq. 6
 * (softmax gate: log g_m = s_m - LSE(s) over the historical blocks),
 * Sec. 4.3 Alg. 1 (I = Top-K) and App. E (Top-K encoded as a per-query
 * threshold: a block is active when it reaches the threshold).
 *
 * For every row (b, h_kv, i) (softmax activation; with SAS_GATE_SIGMOID the
 * m < i entries are log sigmoid(s[i, m]), with SAS_GATE_RAW s[i, m] itself):
 *   log_gate[.., i, m] = s[i, m] - LSE_{m' < i} s[i, m']   for m < i,
 *                        0                                 for m = i,
 *                        -inf                              for m > i;
 *   tau[.., i]  = the K-th largest of {s[i, m] : m < i} if 1 <= K < i,
 *                 -inf if K >= i (every historical block kept),
 *                 +inf if K == 0 and i >= 1 (none kept);
 *   I_i = {m < i : s[i, m] >= tau_i}, compared in fp32 (ties at tau are
 *   all kept, so |I_i| can exceed K only through exact ties);
 *   sel_idx[.., i, 0 .. cnt-1] = I_i in ascending order, remaining slots -1;
 *   sel_cnt[.., i] = |I_i| (the true count, even if it exceeds sel_cap).
 * The threshold is found by a most-significant-bit-first radix select on
 * order-preserving integer keys of the fp32 scores (no sort).
 *
 * Inputs : scores  fp32 [B,Hkv,C,C]; entries m >= i are never read; the
 *          entries m < i must be finite.
 * Outputs: log_gate fp32 [B,Hkv,C,C], tau fp32 [B,Hkv,C],
 *          sel_idx int32 [B,Hkv,C,sel_cap], sel_cnt int32 [B,Hkv,C].
 * sel_cap: >= min(K, C-1); sel_cap = C-1 can never overflow.
 * d_status: optional device int32; when non-NULL it is set to
 *          SAS_E_CAPACITY by any row whose |I_i| exceeds sel_cap (it is
 *          never cleared by the library; the caller zeroes it).
 */
int32_t sas_gate_threshold(const sas_problem* p, const float* scores, float* log_gate, float* tau,
                           int32_t* sel_idx, int32_t* sel_cnt, int32_t sel_cap, int32_t* d_status,
                           void* stream);

/*
 * sas_gated_attn_fwd -- gated block-sparse attention forward.
 *
 * Defined by Sec. 4.3 Eq. 9 and the App. E forward (Alg. 3): for query token t
 * of block i and query head h, the attended keys are the tokens u <= t of
 * block i (bias 0) and every token of each selected block m in I_i
 * (bias log_gate[i, m]):
 *   z_u = sm_scale * q_t . k_u + bias_u,  o_t = sum_u softmax(z)_u v_u,
 *   lse_t = log sum_u exp(z_u).
 * Unselected blocks are skipped entirely, never materialised.  With
 * gate_pos = SAS_GATE_OUTER the logits carry no bias and the value rows of a
 * selected block m are multiplied by g = exp(log_gate[i, m]) instead:
 *   o_t = sum_u softmax(sm_scale q_t . k_u)_u g_{blk(u)} v_u  (lse ungated).
 *
 * Inputs : q, k, v (dtype), log_gate fp32 (only entries m in I_i are read),
 *          sel_idx / sel_cnt as written by sas_gate_threshold (the first
 *          min(sel_cnt, sel_cap) entries of each row are used; they must be
 *          ascending block indices < i).
 * Outputs: o (o_dtype) [B,Hq,N,D], lse fp32 [B,Hq,N].
 */
int32_t sas_gated_attn_fwd(const sas_problem* p, const void* q, const void* k, const void* v,
                           const float* log_gate, const int32_t* sel_idx, const int32_t* sel_cnt,
                           int32_t sel_cap, void* o, float* lse, void* stream);

/* Bytes of device workspace sas_gated_attn_bwd needs for problem p and the
 * given sel_cap (0 if p or sel_cap is invalid; then sas_last_error says why).
 *
 * The sum of these parts, each rounded up to 256 bytes, with
 * Hs = score heads (n_kv_heads, or n_q_heads with per-head gates),
 * C = blocks per sequence, nrow = B Hs C gate rows, ncol = B Hkv C key
 * columns, E = B Hs sum_{i<C} min(i, sel_cap) selected entries:
 *   vector-ALU path (fp32, or head_dim != 128, or block_size != 64):
 *     4 B Hq N (Delta);
 *   matrix-core path, in addition:
 *     4 B Hq N (-LSE in log2 units), 4 ncol ceil(C Hs / (32 Hkv)) (column
 *     bit masks), 16 ncol + 12 (column lengths and offsets, chunk offsets
 *     and counts),
 *     4 (E + nrow) (column lists), and per column chunk 65536 bytes (fp32
 *     dK and dV partials of a column split over several chunks) + 20 bytes
 *     (schedule), for at most (E + nrow + ncol (cc - 1)) / cc chunks of up
 *     to cc entries, cc = 16 with group gates and min(64, 16 G) with
 *     per-head gates.
 * The partials dominate: about 0.5 GiB for batch 1, 32 / 8 heads, 32k
 * tokens, sel_cap 16, and 3.0 GiB at 128k tokens with sel_cap 32. */
size_t sas_gated_attn_bwd_workspace_size(const sas_problem* p, int32_t sel_cap);

/*
 * sas_gated_attn_bwd -- gated block-sparse attention backward.
 *
 * Defined by the App. E backward (Alg. 4): P is recomputed from lse;
 * dS = P * (dO V^T - Delta);
 *   dq = sm_scale dS K,  dk = sm_scale dS^T Q,  dv = P^T dO
 * (dk, dv summed over the G query heads of each kv head).  Delta is the row
 * correction of App. E, rowsum(O * dO), which equals sum_u P_u dP_u for the
 * probabilities P of the row.  The first (query-major) pass forms dS for dq
 * with Delta = rowsum(o * dO) and accumulates sum_u P_u dP_u of its
 * recomputed P; the second (key-major) pass uses that sum for dS, so dk and
 * dlog_gate carry no rounding of o;
 *   dlog_gate[i, m] = sum of dS over the query tokens of block i (all G heads)
 *                     and the key tokens of block m, for m in I_i; 0 elsewhere
 *                     (unselected, diagonal and upper-triangle entries);
 * and, if dscores != NULL, the selector-score gradient of App. D.3 with the
 * sparse-scope rule of Eq. 8:
 *   dscores[i, m] = dlog_gate[i, m] - exp(log_gate[i, m]) * sum_{l<i} dlog_gate[i, l]
 *   for m < i; 0 for m >= i (softmax activation; SAS_GATE_SIGMOID:
 *   dlog_gate[i, m] * (1 - exp(log_gate[i, m])); SAS_GATE_RAW: dlog_gate[i, m]).
 * With gate_pos = SAS_GATE_OUTER the value rows carry their gates: dP = dO
 * (g . V)^T, dv = g . (P^T dO), and dlog_gate[i, m] = g_m dg_m = the sum of
 * P * dP over the block (Eq. 5, outer form).
 *
 * Inputs : q, k, v, d_o (dtype), o (o_dtype), lse from the forward, log_gate (all
 *          entries m < i are read when dscores != NULL), sel_idx, sel_cnt.
 * Outputs: dq, dk, dv (dtype), dlog_gate fp32 [B,Hkv,C,C], dscores fp32
 *          [B,Hkv,C,C] or NULL.
 * workspace: device memory of at least
 *          sas_gated_attn_bwd_workspace_size(p, sel_cap) bytes, 256-byte
 *          aligned, owned by the caller, not preserved across calls; calls
 *          that share a workspace must not overlap in time.
 * The dq, dlog_gate and dscores results are bitwise deterministic; so are dk
 * and dv (split partial sums are reduced in a fixed order).
 */
int32_t sas_gated_attn_bwd(const sas_problem* p, const void* q, const void* k, const void* v,
                           const void* o, const void* d_o, const float* lse, const float* log_gate,
                           const int32_t* sel_idx, const int32_t* sel_cnt, int32_t sel_cap,
                           void* dq, void* dk, void* dv, float* dlog_gate, float* dscores,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two stages of sas_gated_attn_bwd, for callers that schedule (or time)
 * them separately.  Calling sas_gated_attn_bwd_dq and then
 * sas_gated_attn_bwd_dkdv on the same stream with the same workspace is
 * exactly sas_gated_attn_bwd.
 *
 * sas_gated_attn_bwd_dq -- the query-major stage (App. E backward, first pass
 * of Alg. 4): dq (with Delta = rowsum(o * dO)), and the row sums
 * sum_u P_u dP_u kept in the workspace.  It also records, in the workspace,
 * which query blocks attend each key block (the transpose of the selection)
 * for the key-major stage.
 */
int32_t sas_gated_attn_bwd_dq(const sas_problem* p, const void* q, const void* k, const void* v,
                              const void* o, const void* d_o, const float* lse,
                              const float* log_gate, const int32_t* sel_idx,
                              const int32_t* sel_cnt, int32_t sel_cap, void* dq, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * sas_gated_attn_bwd_dkdv -- the key-major stage (second pass of Alg. 4):
 * dk = sm_scale dS^T Q and dv = P^T dO for every key block, summed over the
 * diagonal query block and every query block that selected it, and over the
 * G heads of the kv group; dlog_gate (every entry written, as described for
 * sas_gated_attn_bwd) and, if dscores != NULL, the selector-score gradient
 * (App. D.3).  It reads Delta and the selection transpose that
 * sas_gated_attn_bwd_dq left in `workspace`; it must follow that call, on the
 * same stream, with the same workspace, problem, inputs and selection.
 */
int32_t sas_gated_attn_bwd_dkdv(const sas_problem* p, const void* q, const void* k,
                                const void* v, const void* d_o, const float* lse,
                                const float* log_gate, const int32_t* sel_idx,
                                const int32_t* sel_cnt, int32_t sel_cap, void* dk, void* dv,
                                float* dlog_gate, float* dscores, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Sparse decode (one new query token per sequence)
 *
 * The inference step of the paper (Sec. 4.3, Alg. 2; Sec. 5.1 "Inference
 * implementation"): per query group (kv head) the Top-K historical blocks
 * are chosen from selector scores, and the new token attends its current
 * block plus the selected blocks, gathered from a paged KV cache, with a plain
 * softmax (no gates at inference):  o = softmax(sm_scale q K_S^T) V_S.
 *
 * Sequence s holds n_s = seq_lens[s] tokens, the newest one being the query
 * (its K / V already in the cache).  Its current block is c_s = (n_s - 1) / b
 * (tokens c_s * b .. n_s - 1 are attended); its historical blocks are
 * 0 .. c_s - 1.  K counts historical blocks; K >= c_s keeps them all; K = 0
 * keeps none.
 *
 * Layouts (contiguous):
 *    q, o                 [B, Hq, D]          (dtype)
 *    k_pool, v_pool       [P, Hkv, b, D]      (dtype): page p holds one block
 *                                              of b tokens for every kv head
 *    block_table          [B, max_blocks]     int32: page of logical block m
 *    seq_lens             [B]                 int32, 1 <= n_s <= max_blocks * b
 *    scores               [B, Hkv, max_blocks] fp32 selector scores; entries
 *                                              m >= c_s are never read
 *    tau                  [B, Hkv]            fp32
 *    sel_idx              [B, Hkv, sel_cap]   int32, ascending, padded with -1
 *    sel_cnt              [B, Hkv]            int32
 *    lse                  [B, Hq]             fp32, natural log
 * Query head h reads kv head h / G.  seq_lens, block_table and the selection
 * live in device memory and are checked by the kernels: an out-of-range
 * length is clamped into [1, max_blocks * b], an out-of-range page or a
 * selected index outside [0, c_s) contributes nothing, and each of these sets
 * *d_status = SAS_E_INVALID when d_status is non-NULL (never cleared by the
 * library).  Every other convention of this header applies (caller-owned
 * device memory, host validation before any launch, thread-local messages).
 * Supported: D in {64, 128}, b in {16, 32, 64}, max_blocks <= 16384,
 * G = Hq / Hkv <= 64, dtype bf16 or fp32.
 * ------------------------------------------------------------------------ */
typedef struct sas_decode_problem {
  int32_t batch;       /* B sequences, one query token each                    */
  int32_t n_q_heads;   /* Hq                                                   */
  int32_t n_kv_heads;  /* Hkv, divides Hq                                      */
  int32_t head_dim;    /* D in {64, 128}                                       */
  int32_t block_size;  /* b in {16, 32, 64}: tokens per block = per page       */
  int32_t max_blocks;  /* row length of scores / block_table                   */
  int32_t pool_blocks; /* P: pages in k_pool / v_pool                          */
  int32_t budget_k;    /* K >= 0 historical blocks per query group             */
  int32_t dtype;       /* sas_dtype of q, k_pool, v_pool, o                    */
  float sm_scale;      /* <= 0 selects 1/sqrt(D)                               */
} sas_decode_problem;

/*
 * sas_decode_select -- per-group Top-K of the selector scores (Alg. 2 step
 * "I = Top-K(s, K)"; Sec. 5.1: Top-K blocks per query group).  As in the
 * training path the set is a threshold: tau = the K-th largest fp32 score of
 * the historical blocks and I = {m < c_s : s_m >= tau} (ties at tau all kept,
 * so |I| can exceed K only through exact ties), found by a most-significant-
 * digit-first radix select over order-preserving integer keys (no sort), one
 * workgroup per (sequence, kv head).
 * Outputs: tau (nullable; -inf when K >= c_s, +inf when K = 0 < c_s),
 * sel_idx (ascending, remaining slots -1), sel_cnt (the true count); a count
 * above sel_cap sets *d_status = SAS_E_CAPACITY.
 * sel_cap: >= max(1, min(K, max_blocks - 1)) and <= 65534.
 */
int32_t sas_decode_select(const sas_decode_problem* p, const float* scores,
                          const int32_t* seq_lens, float* tau, int32_t* sel_idx, int32_t* sel_cnt,
                          int32_t sel_cap, int32_t* d_status, void* stream);

/* Bytes of device workspace sas_decode_attn needs (0 if p or sel_cap is
 * invalid; sas_last_error says why). */
size_t sas_decode_workspace_size(const sas_decode_problem* p, int32_t sel_cap);

/*
 * sas_decode_attn -- attention of each new token over its current block and
 * its selected blocks (Alg. 2: S = B0 u U_{m in I} B_m,
 * o = softmax(q K_S^T) V_S; Sec. 5.1: only the selected KV blocks are
 * gathered from the paged cache; the G query heads of a group share them).
 * Reads the first min(sel_cnt, sel_cap) entries of each sel_idx row (as
 * written by sas_decode_select, or any ascending list of blocks < c_s).
 * Outputs: o (dtype) [B, Hq, D], lse fp32 [B, Hq].
 * workspace: >= sas_decode_workspace_size(p, sel_cap) bytes, 256-byte
 * aligned, caller-owned, not preserved; calls sharing it must not overlap.
 * Results are bitwise deterministic (tile partials merged in a fixed order).
 */
int32_t sas_decode_attn(const sas_decode_problem* p, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* sel_idx, const int32_t* sel_cnt, int32_t sel_cap, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, int32_t* d_status,
                        void* stream);

/*
 * sas_decode_attn_noalloc -- sas_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, with the
 * tile partials in a fixed scratch array that the library holds on each
 * device (SAS_DECODE_SCRATCH_BYTES = 32 MiB, allocated when the library's
 * code object is loaded on the device and kept until the process ends)
 * instead of a workspace argument.  No device memory is allocated or freed.
 * Arguments, layouts and outputs as for sas_decode_attn; the scratch is the
 * one of the current device, so `stream` must belong to the current device.
 * Errors: as sas_decode_attn, and SAS_E_WORKSPACE (before any launch) when
 * the problem needs more than SAS_DECODE_SCRATCH_BYTES, i.e.
 * 4 * batch * n_kv_heads * (sel_cap + 1) * (n_q_heads / n_kv_heads) *
 * (head_dim + 2) bytes rounded up to 256.
 * Every call on one device shares that device's scratch: calls that overlap
 * in time on one device (other streams, other host threads) race and must be
 * serialised by the caller.  The scratch keeps the last call's partials;
 * nothing in it needs clearing between calls.
 */
#define SAS_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int32_t sas_decode_attn_noalloc(const sas_decode_problem* p, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* sel_idx,
                                const int32_t* sel_cnt, int32_t sel_cap, void* o, float* lse,
                                int32_t* d_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAS_H_ */
