/*
 * moe.h - C ABI of the MI355X (gfx950) Mixture-of-Experts layer forward pass.
 *
 * The layer follows the six steps of LLM Internals section 14.2.1 ("one MoE
 * forward pass: six steps and shapes") and the four router steps of the AI
 * Knowledge Map page "Mixture of Experts (MoE)":
 *   score     l = X W_g (+ optional per-expert offset)          -> moe_route
 *   select    top-k, gates renormalised inside the chosen set   -> moe_route
 *             or every expert takes its top-C tokens  -> moe_route_expert_choice
 *   dispatch  stable sort of token slots by expert, capacity    -> moe_dispatch
 *   experts   grouped SwiGLU GEMM, m_i rows per expert          -> moe_grouped_ffn
 *   combine   gate-weighted sum through the inverse permutation -> moe_combine
 *   all       one fused call                                    -> moe_forward
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major.
 *     The library never allocates, frees or synchronises; scratch memory is a
 *     caller-provided workspace of at least the size the matching
 *     *_workspace_size function returns (256-byte aligned).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call is asynchronous on that stream; data-dependent sizes (rows
 *     per expert, kept rows) stay on the device.
 *   - Weight storage: every matrix is stored with its reduction dimension
 *     contiguous.  Router Wg[E][d] (logical W_g[d,E] transposed); gate/up
 *     W1,W3[G][F][d] (logical [G,d,F] transposed); down W2[G][d][F] (logical
 *     [G,F,d] transposed).  Activations X[T][d], H[rows][F], Y[T][d].
 *     A caller that holds the weights in the logical layout of LLM Internals
 *     14.2.1 step 5 (x[m_i, d] times W_i[d, F], i.e. W1/W3 as [G][d][F], W2
 *     as [G][F][d], W_g as [d][E]) must transpose each matrix once, when
 *     the weights are loaded: W1[g].T, W3[g].T, W2[g].T and W_g.T, made
 *     contiguous.  The reason is the matrix-core operand format: both MFMA
 *     operands take 8 consecutive K-elements per lane, so with K contiguous
 *     in memory one 16-byte load per lane feeds a fragment straight from
 *     global memory through LDS, for the token rows and the weight rows
 *     alike; the library performs no transposition per call.
 *   - dtype: MOE_BF16 (bf16 storage, fp32 accumulation, fp32 router scores)
 *     or MOE_F32.  Integers are int32.
 *   - Supported shapes: d and F multiples of 128, 1 <= E <= 256, 1 <= k <= E,
 *     k <= 16 (top-k routing), T >= 0.  Otherwise MOE_EUNSUPPORTED.
 *   - Errors: arguments are validated on the host before anything is
 *     launched; a negative return means nothing was enqueued (except
 *     MOE_EHIP, which reports a failed launch).  moe_last_error() returns a
 *     thread-local message describing the last failure.
 *   - Results are bitwise reproducible run to run: no floating-point atomics.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };
/* Expert-weight storage: the layer dtype, or FP8 E4M3 codes with one fp32
 * scale per output channel (W = value(code) * scale; bf16 layers only). */
enum moe_wtype { MOE_W_DTYPE = 0, MOE_W_FP8 = 1 };
enum moe_score { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 };
/* Who chooses: every token its top-k experts, or every expert its top-C
 * tokens (moe_route_expert_choice). */
enum moe_routing { MOE_TOKEN_CHOICE = 0, MOE_EXPERT_CHOICE = 1 };
enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* invalid argument (null pointer, k > E, ...)     */
  MOE_EUNSUPPORTED = -2,  /* valid but unsupported shape or dtype            */
  MOE_EWORKSPACE = -3,    /* workspace smaller than *_workspace_size()       */
  MOE_EHIP = -4           /* HIP runtime error while launching               */
};

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Capacity C = ceil(cf * N * k / E) (AI Knowledge Map "MoE", capacity
 * formula; GShard form in LLM Internals 14.2.3).  cf is taken as the exact
 * decimal its shortest round-trip representation spells, so the result is
 * exact (1.25 * 8192 * 2 / 64 = 320).  Returns C >= 0, or a negative
 * moe_status for cf <= 0, non-finite cf, N < 0, k < 1 or E < 1. */
int64_t moe_capacity(double cf, int64_t N, int k, int E);

/* ---------------------------------------------------------------- route --
 * Router scoring and top-k (LLM Internals 14.2.1 steps 2-3; AI Knowledge Map
 * "MoE" router steps 1-4; eq. 16 of the DeepSeek-V3 report as restated in
 * LLM Internals 14.2.3 for the selection-only bias).
 *   X[T][d] (dtype), Wg[E][d] (dtype)
 *   bias[E]          fp32 selection-only bias (sigmoid router) or NULL
 *   logit_offset[E]  fp32 added to every token's logits, or NULL
 *   score            MOE_SOFTMAX: p = softmax(l) in fp32 over all E; the
 *                    top-k key is the logit itself.
 *                    MOE_SIGMOID: s = sigmoid(l) per cell; the key is s + b,
 *                    evaluated in fp64; the gate uses the raw s.
 *   renorm           1: gates g_e / sum_{chosen} g; 0: the raw p or s.
 *   n_group, topk_group  group-limited routing (LLM Internals 14.2.3,
 *                    node-limited routing with groups of experts standing in
 *                    for nodes): n_group <= 1 disables it.  Otherwise E is
 *                    split into n_group groups of E / n_group consecutive
 *                    experts; a group's score is the sum of its
 *                    max(1, k / topk_group) highest affinities (p, or s
 *                    without the bias); only the topk_group best groups
 *                    (lower id on ties) are eligible for the top-k.  Needs
 *                    E % n_group == 0, n_group <= 64, 1 <= topk_group <=
 *                    n_group and k <= topk_group * E / n_group.
 * Outputs (device):
 *   logits[T][E]     fp32 logits (with the offset) or NULL
 *   topk_ids[T][k]   int32, key descending, ties to the lower expert id
 *   topk_w[T][k]     fp32 gates in the same order
 *   prob_sum[E]      fp32 sum over tokens of the full-row p (or s), or NULL
 *   backup_ids[T][n_backup]  the next n_backup choices after the top-k in
 *                    the same key order (-1 for an expert outside the
 *                    chosen groups), for moe_dispatch's overflow re-route;
 *                    0 <= n_backup <= min(k, E - k); NULL when n_backup = 0
 */
size_t moe_route_workspace_size(int64_t T, int d, int E);
int moe_route(const void* X, int dtype, int64_t T, int d, const void* Wg,
              int E, const float* bias, const float* logit_offset, int score,
              int k, int renorm, int n_group, int topk_group, float* logits,
              int32_t* topk_ids, float* topk_w, float* prob_sum, int n_backup,
              int32_t* backup_ids, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------- expert-choice route --
 * Expert-choice routing (LLM Internals 14.2.3, the expert-choice paradigm:
 * every expert takes a fixed number of tokens from the batch; oscine.io
 * "MoE 03: efficiency frontiers", expert-choice routing: each expert picks
 * the C tokens it scores highest).  Scores as in moe_route: the full-row
 * softmax over the E experts (MOE_SOFTMAX) or the sigmoid affinity
 * (MOE_SIGMOID); no bias, no groups.  Expert e takes the Ce = min(C, T)
 * tokens with the highest score in column e, ties to the lower token index;
 * the decision is taken on fp64 keys (log p, or the logit for sigmoid).  A
 * token may be taken by several experts or by none.  Slot s = t*E + e.
 *   X[T][d], Wg[E][d] (dtype); logit_offset[E] fp32 or NULL; C >= 0.
 * Outputs (device):
 *   logits[T][E]      fp32 logits (with the offset) or NULL
 *   offsets[E+1]      int32, offsets[e] = e * Ce
 *   sorted_slot[E*Ce] int32 slots t*E + e of the taken tokens, grouped by
 *                     expert, ascending token index inside; or NULL
 *   slot_row[T*E]     int32 row of slot t*E + e in that order, -1 if the
 *                     expert did not take the token
 *   gates[T*E]        fp32 score of the taken slots (no renormalisation:
 *                     the number of experts per token varies), 0 elsewhere
 * Feed offsets / sorted_slot (row r's token = sorted_slot[r] / E) to
 * moe_grouped_ffn and slot_row / gates with k = E to moe_combine.
 */
size_t moe_route_expert_choice_workspace_size(int64_t T, int d, int E);
int moe_route_expert_choice(const void* X, int dtype, int64_t T, int d,
                            const void* Wg, int E, const float* logit_offset,
                            int score, int64_t C, float* logits,
                            int32_t* offsets, int32_t* sorted_slot,
                            int32_t* slot_row, float* gates, void* ws,
                            size_t ws_bytes, void* stream);

/* ------------------------------------------------------------- dispatch --
 * Dispatch permutation with an optional capacity drop (LLM Internals 14.2.1
 * step 4; AI Knowledge Map "MoE" capacity and overflow-by-drop).  Slot
 * s = t*k + j.  rank(s) = number of earlier slots with the same expert; a
 * slot is kept iff capacity <= 0 or rank(s) < capacity.
 *   topk_ids[T][k]     int32 expert ids (0 <= id < E)
 * Outputs (device, int32):
 *   counts[E]          requests per expert before the drop
 *   offsets[E+1]       exclusive scan of min(counts, capacity)
 *   sorted_slot[T*k]   first n_kept entries: kept slots grouped by expert,
 *                      increasing slot order inside an expert
 *   slot_row[T*k]      row of slot s in the sorted order, -1 if dropped
 *   n_kept[1]          number of kept slots R
 * Optional overflow re-route (AI Knowledge Map "MoE", the second/backup
 * way of handling a capacity overflow): with capacity > 0 and n_backup > 0,
 * backup_ids[T][n_backup] (moe_route's) give one backup round after the
 * drop.  The m-th dropped slot of token t (j ascending) proposes
 * backup_ids[t][m-1] (-1: none); experts accept proposals in slot order while
 * they have room (capacity minus their first-pass rows); the rest stay
 * dropped.  An expert's rows are then its first-pass slots followed by its
 * accepted proposals, each in slot order; offsets / n_kept count both.
 * Optional gather (step 4's data movement): if X and X_sorted are non-NULL,
 *   X_sorted[r][:] = X[sorted_slot[r] / k][:] for r < n_kept (dtype, [.,d]).
 */
size_t moe_dispatch_workspace_size(int64_t T, int k, int E);
int moe_dispatch(const int32_t* topk_ids, int64_t T, int k, int E,
                 int64_t capacity, const int32_t* backup_ids, int n_backup,
                 int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                 int32_t* slot_row, int32_t* n_kept, const void* X, int dtype,
                 int d, void* X_sorted, void* ws, size_t ws_bytes,
                 void* stream);

/* --------------------------------------------------------- grouped FFN --
 * Grouped SwiGLU expert FFN (LLM Internals 14.2.1 step 5; one expert is the
 * three matrices of 14.2.2): for every group g and row r in
 * [offsets[g], offsets[g+1]):
 *   h = silu(a_r W1_g) * (a_r W3_g)       (rounded to bf16 for MOE_BF16)
 *   Yrows[r][:] = h W2_g                   (fp32)
 * where a_r = A[row_token[r]] if row_token != NULL (A is then X[T][d]) and
 * a_r = A[r] otherwise (A is X_sorted).
 *   offsets[G+1]   device int32, non-decreasing, offsets[G] <= max_rows
 *   W1, W3[G][F][d], W2[G][d][F] (dtype)
 *   max_rows       host upper bound of offsets[G] (sizes the launch)
 *   Yrows[max_rows][d] fp32 output; rows past offsets[G] are untouched.
 */
size_t moe_grouped_ffn_workspace_size(int64_t max_rows, int G, int d, int F,
                                      int dtype);
int moe_grouped_ffn(const void* A, const int32_t* row_token,
                    const int32_t* offsets, int G, const void* W1,
                    const void* W3, const void* W2, int dtype, int d, int F,
                    int64_t max_rows, float* Yrows, void* ws, size_t ws_bytes,
                    void* stream);

/* Same computation with FP8 expert weights (the DeepSeek-V3 weight format
 * of LLM Internals 14.2.5's intensity model): A is bf16, W1/W3/W2 hold OCP
 * FP8 E4M3 codes in the layout above, and every output channel has one fp32
 * scale: W1_scale, W3_scale [G][F], W2_scale [G][d].  The weights used are
 * value(code) * scale; codes are widened to bf16 exactly inside the kernel
 * and the scales multiply the fp32 accumulators.  The workspace size is
 * moe_grouped_ffn_workspace_size(max_rows, G, d, F, MOE_BF16). */
int moe_grouped_ffn_fp8(const void* A, const int32_t* row_token,
                        const int32_t* offsets, int G, const uint8_t* W1,
                        const uint8_t* W3, const uint8_t* W2,
                        const float* W1_scale, const float* W3_scale,
                        const float* W2_scale, int d, int F, int64_t max_rows,
                        float* Yrows, void* ws, size_t ws_bytes, void* stream);

/* -------------------------------------------------------------- combine --
 * Combine (LLM Internals 14.2.1 step 6; AI Knowledge Map "MoE"
 * y = sum_{e in S} g_e E_e(x)):
 *   Y[t][:] = sum_{j: slot_row[t*k+j] >= 0} topk_w[t][j] * Yrows[slot_row[t*k+j]][:]
 *             + shared[t][:]          (if shared != NULL)
 * accumulated in fp32 and rounded once to dtype.  Dropped slots add nothing.
 *   Yrows[.][d] fp32, slot_row[T*k], topk_w[T][k] fp32, shared[T][d] fp32.
 * 1 <= k <= 256 (expert-choice routing passes k = E).
 */
int moe_combine(const float* Yrows, const int32_t* slot_row,
                const float* topk_w, int64_t T, int k, int d,
                const float* shared, void* Y, int dtype, void* stream);

/* Selection-bias update (LLM Internals 14.2.3: DeepSeek-V3 keeps a per-expert
 * bias that is not learned by back-propagation; after each step overloaded
 * experts lose gamma and underloaded ones gain gamma; the report used
 * gamma = 0.001, then 0).  In place on device memory:
 *   bias[e] -= gamma  if counts[e] > T*k/E,
 *   bias[e] += gamma  if counts[e] < T*k/E,  unchanged if equal
 * (compared exactly as counts[e]*E vs T*k).  counts[E]: the step's pre-drop
 * loads (moe_dispatch's or moe_aux's counts); gamma finite and >= 0. */
int moe_bias_update(const int32_t* counts, int64_t T, int k, int E,
                    float gamma, float* bias, void* stream);

/* Balance statistic E * sum_e f_e P_e (LLM Internals 14.2.3 balance loss
 * without alpha): f_e = counts[e] / (T*k), P_e = prob_sum[e] / T.
 * Writes one fp64 value to device memory `out`. */
int moe_balance(const int32_t* counts, const float* prob_sum, int64_t T,
                int k, int E, double* out, void* stream);

/* -------------------------------------------------------------- forward --
 * The whole layer in one call: route -> dispatch (+capacity) -> grouped
 * SwiGLU (routed experts and the optional shared expert of LLM Internals
 * 14.2.4, width F, weight 1) -> combine.  Y has X's shape (no residual). */
typedef struct moe_layer {
  int dtype;               /* MOE_BF16 or MOE_F32                           */
  int score;               /* MOE_SOFTMAX or MOE_SIGMOID                    */
  int renorm;              /* renormalise gates inside the chosen set        */
  int d, E, k, F;
  int n_shared;            /* 0 or 1                                         */
  double capacity_factor;  /* <= 0: no capacity limit                        */
  const void* Wg;          /* [E][d]                                         */
  const float* bias;       /* [E] or NULL                                    */
  const float* logit_offset; /* [E] or NULL                                  */
  const void* W1;          /* [E][F][d]                                      */
  const void* W3;          /* [E][F][d]                                      */
  const void* W2;          /* [E][d][F]                                      */
  const void* Ws1;         /* shared expert [F][d], or NULL                  */
  const void* Ws3;         /* [F][d]                                         */
  const void* Ws2;         /* [d][F]                                         */
  int wtype;               /* MOE_W_DTYPE, or MOE_W_FP8 (dtype MOE_BF16):
                              W1..Ws2 then hold E4M3 codes with the scales: */
  const float* W1_scale;   /* [E][F]                                         */
  const float* W3_scale;   /* [E][F]                                         */
  const float* W2_scale;   /* [E][d]                                         */
  const float* Ws1_scale;  /* [F]  (shared expert)                           */
  const float* Ws3_scale;  /* [F]                                            */
  const float* Ws2_scale;  /* [d]                                            */
  int n_group;             /* group-limited routing as in moe_route; <= 1 off */
  int topk_group;
  int routing;             /* MOE_TOKEN_CHOICE, or MOE_EXPERT_CHOICE: every
                              expert takes C = min(T, moe_capacity(cf, T, k,
                              E)) tokens (cf = 1 when capacity_factor <= 0;
                              k is then the mean experts per token), as in
                              moe_route_expert_choice.  Needs renorm = 0, no
                              bias and n_group <= 1.  moe_aux then holds
                              slot_row and topk_w as [T][E] (slot t*E + e),
                              sorted_slot as [E*C], counts[e] = C, n_kept =
                              E*C; topk_ids, prob_sum, balance and health must
                              be NULL.                                        */
  int reroute;             /* 1: overflow re-route of moe_dispatch with
                              min(k, E - k) backups per token (top-k routing
                              with a capacity factor); 0: overflow dropped   */
} moe_layer;

/* Optional device outputs of moe_forward; any member may be NULL. */
typedef struct moe_aux {
  float* logits;           /* [T][E]  */
  int32_t* topk_ids;       /* [T][k]  */
  float* topk_w;           /* [T][k]  */
  float* prob_sum;         /* [E]     */
  int32_t* counts;         /* [E]     */
  int32_t* offsets;        /* [E+1]   */
  int32_t* sorted_slot;    /* [T*k]   */
  int32_t* slot_row;       /* [T*k]   */
  int32_t* n_kept;         /* [1]     */
  float* Yrows;            /* [R_max + n_shared*T][d] expert output rows,
                              R_max = T*k (E*C with expert choice)          */
  double* balance;         /* [1]     */
  double* health;          /* [4] router health (LLM Internals 14.2.3's three
                              signals, AI Knowledge Map's load CV): mean
                              per-token routing entropy of the full-row
                              distribution (sigmoid scores normalised to sum
                              1), entropy of the pre-drop load fractions
                              counts/(T*k), std/mean of the per-expert
                              counts, drop rate 1 - R/(T*k)               */
} moe_aux;

size_t moe_forward_workspace_size(const moe_layer* L, int64_t T);
int moe_forward(const moe_layer* L, const void* X, int64_t T, void* Y,
                const moe_aux* aux, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------ forward, no allocation --
 * For callers that cannot allocate device memory or call hipMalloc (code
 * under HIP graph capture, tight serving loops, harnesses that forbid it):
 * moe_forward with its workspace taken from a fixed array of
 * moe_forward_noalloc_max_bytes() = 64 MiB that the library holds in device
 * memory, one per GPU, until the process ends.  The caller still passes X,
 * Y and the optional moe_aux outputs.  A layer and batch whose
 * moe_forward_workspace_size() exceeds that size is rejected with
 * MOE_EWORKSPACE before anything is launched (decode-sized batches fit;
 * large prefill batches use moe_forward with a workspace).  Nothing is
 * allocated or freed; the array's device address is looked up once per
 * device.  All calls on one GPU share the array and it keeps the last
 * call's contents (every buffer the forward reads is written by the same
 * call first), so calls that overlap on one GPU, on different streams or
 * threads, race: serialise them.  Results are bit-identical to
 * moe_forward's. */
size_t moe_forward_noalloc_max_bytes(void);
int moe_forward_noalloc(const moe_layer* L, const void* X, int64_t T, void* Y,
                        const moe_aux* aux, void* stream);

/* ------------------------------------------------------------- timing --
 * Optional event timing of moe_forward's phases, for benchmarks.
 * moe_timing_enable(n): n > 0 creates a pool of n HIP events (runtime
 *   objects, no device buffers) and makes later moe_forward calls record one
 *   event on their stream at each phase boundary: begin, route, dispatch,
 *   tile_map, ffn_up (gate/up GEMM + SwiGLU), ffn_down, combine, aux.  Marks
 *   beyond the pool are dropped.  n = 0 stops timing and frees the pool.
 * moe_timing_read(names, name_len, ms, max): waits for the recorded events,
 *   writes up to `max` marks (name into names + i*name_len, NUL-terminated;
 *   ms[i] = milliseconds since the previous mark of the same call, -1 for a
 *   call's first mark), clears them and returns how many were written, or a
 *   negative moe_status. */
int moe_timing_enable(int n);
int moe_timing_read(char* names, int name_len, float* ms, int max);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
