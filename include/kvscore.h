/*
 * kvscore.h — C ABI of libkvscore: output-perturbation KV-cache eviction scoring on
 * AMD Instinct MI355X (gfx950).
 *
 * The pipeline, run once after prefill for every (sequence, layer, KV head) "unit":
 *
 *   kvscore_attn_fwd   window-query attention forward: a_i, logsumexp_i, the argmax
 *                      key j*_i of each row and that pair's term (isolated exactly).
 *   kvscore_score      per-token score partials per query tile:
 *                      sum_i p_ij/(1-p_ij) * ||a_i - v_j||_2 over rows i (pairs i, j*_i
 *                      excluded), recomputing p_ij from the logsumexp and expanding
 *                      ||a - v||^2 = ||a||^2 - 2 a.v + ||v||^2.
 *   kvscore_merge      sums the query-tile partials in a fixed order and adds the
 *                      isolated argmax terms: score[l][g][j].
 *   kvscore_budget     (host) per-layer budgets from a sensitivity profile.
 *   kvscore_topk       per unit: the highest-scoring candidates (optionally by a
 *                      max-pooled key, optionally pinning sinks) plus the W most
 *                      recent tokens, as ascending positions in a packed array.
 *   kvscore_compact    gathers the kept K and V rows into a packed ragged cache.
 *   kvscore_topk_heads / kvscore_compact_heads  the same with head budgets chosen jointly
 *                      over the KV heads of a layer.
 *   kvscore_decode_attn  decode attention of new query tokens over that cache.
 *
 * Sources (the web pages this library implements):
 *   DropKV: Decoupling Residual-Output Perturbation for Near-Optimal KV-Cache Eviction
 *     (ai.info summary page) -- "Key Contributions" 1 and 3 and "Methodology in Plain
 *     English": the per-token score p_j/(1-p_j)*||a - v_j||_2 computed from the full
 *     cache, accumulated over the last w queries, the recent w tokens always kept,
 *     keep the largest scores; the fused design (attention forward reusing the
 *     logsumexp, scoring kernel that recomputes logits tile by tile and expands the
 *     squared distance, split-K merge).
 *   RippleKV: Cross-Layer KV Cache Allocation via Perturbation Propagation --
 *     "Problem Formulation" Eq. 3-5 (per-layer retained positions, sum of budgets
 *     = B) and "Sensitivity Guided Layer Budget Allocation" Eq. 9-12.
 *   PyramidKV blog page, "Observation Window and Aggregated Attention Eviction":
 *     scores summed over the heads that share the cache.
 *
 * Conventions (all entry points):
 *   - Every buffer is owned by the caller. The library never allocates or frees
 *     memory. Device pointers must be device memory on the current HIP device.
 *   - `stream` is a hipStream_t (NULL = default stream). Device entry points only
 *     enqueue work on it; nothing synchronises. Results are valid once the stream
 *     has reached that point.
 *   - Return 0 on success or a KVSCORE_E* code; kvscore_last_error() then gives a
 *     message (thread-local). Arguments are validated before any launch: on a
 *     validation error nothing is enqueued.
 *   - Scores are deterministic: no floating-point atomics; every sum has a fixed order.
 *   - Non-finite inputs are outside the contract (results undefined, no fault). The
 *     attention forward multiplies P by V, and the score pass a by V, in fp16: |v|
 *     must stay below 65504 (larger magnitudes saturate); entries below 2^-14 lose
 *     precision as fp16 subnormals (absolute error <= 2^-25).
 *   - Accuracy of the scores (mode L2) against an fp64 evaluation: within 1e-3 relative
 *     for value rows of zero mean (measured up to 7e-5 on the test workloads). The score
 *     pass expands ||a - v||^2 = ||a||^2 - 2 a.v + ||v||^2 with a rounded to fp16, so
 *     value rows that share a common offset mu (v = mu + noise of standard deviation
 *     sigma per element) lose accuracy in proportion to r = ||mu|| / (sigma sqrt(d)):
 *     measured 5e-5 at r = 3, 1.7e-4 at r = 10, 6.5e-4 at r = 30. The 1e-3 bound holds
 *     for r up to about 30; subtract such an offset from V (scores do not change) when
 *     it is larger.
 *
 * Data layout. A unit is u = (l*S + s)*Hkv + g (layer-major); G = Hq/Hkv; a unit has
 * R = G*W query rows r = hl*W + i (hl = head within the group, i = window row), which
 * are query heads h = g*G + hl at token position t_i = n_s - W + i. Row r sees keys
 * 0..t_i (causal). Token indices j are positions within the sequence (0..n_s-1).
 *   q_win : bf16 [L][S][Hq][W][d] contiguous  (rows of unit u: [u*R, (u+1)*R))
 *   k, v  : bf16, row (l, g, token t) at base + l*stride[0] + g*stride[1] + t*stride[2]
 *           elements, t = cu_seqlens[s] + j; head_dim elements contiguous; every row
 *           16-byte aligned.
 *   per-row outputs (a: fp32 [rows][d]; lse, dom: fp32 [rows]; jstar: int32 [rows]),
 *           rows = L*S*Hq*W in the q_win row order.
 *   partial: fp32 [L][Hkv][Tq][N], Tq = kvscore_num_query_tiles(), N = cu_seqlens[S].
 *   score : fp32 [L][Hkv][N].
 *   segment offsets: int64 [U+1], U = L*S*Hkv, segment u = unit u; its length is the
 *           budget b[s][l]. kept_pos: int32 [offsets[U]]; k_out, v_out: bf16
 *           [offsets[U]][d].
 */
#ifndef KVSCORE_H
#define KVSCORE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVSCORE_OK 0
#define KVSCORE_EINVAL 1     /* bad shape, stride, alignment, pointer or option */
#define KVSCORE_EWORKSPACE 2 /* workspace missing or smaller than kvscore_workspace_size() */
#define KVSCORE_EBUDGET 3    /* infeasible budget request */
#define KVSCORE_EDEVICE 4    /* a HIP call or launch failed (message has the HIP error) */

#define KVSCORE_MODE_L2 0 /* sum_i c_ij * ||a_i - v_j||          (default) */
#define KVSCORE_MODE_SQ 1 /* sum_i (c_ij * ||a_i - v_j||)^2      ("squared" variant) */
#define KVSCORE_MODE_ATTN 2 /* sum_i p_ij: the aggregated window attention score
                               (PyramidKV page, "Observation Window and Aggregated
                               Attention Eviction"; SnapKV's ranking) */

#define KVSCORE_MAX_SEQS 64   /* sequences per call */
#define KVSCORE_MAX_ROWS 1024 /* G*W query rows per unit */
#define KVSCORE_MAX_UNITS 65535 /* L*S*Hkv units per call (a launch grid dimension) */

#define KVSCORE_WS_ATTN_FWD 0
#define KVSCORE_WS_SCORE 1
#define KVSCORE_WS_TOPK 2
#define KVSCORE_WS_TOPK_HEADS 3

typedef struct kvscore_problem {
  int32_t num_seqs;          /* S, 1..KVSCORE_MAX_SEQS */
  int32_t num_layers;        /* L >= 1 */
  int32_t num_q_heads;       /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;      /* Hkv >= 1; num_layers * num_seqs * num_kv_heads <= KVSCORE_MAX_UNITS */
  int32_t head_dim;          /* d: 64 or 128 */
  int32_t window;            /* W >= 1; every sequence must be longer than W */
  const int64_t* cu_seqlens; /* HOST array [S+1]: 0 = cu[0] < cu[1] < ... ; n_s = cu[s+1]-cu[s] */
  int64_t k_strides[3];      /* layer, KV-head, token strides of k in elements (token stride < 2^22) */
  int64_t v_strides[3];      /* same for v */
  int32_t mode;              /* KVSCORE_MODE_L2, KVSCORE_MODE_SQ or KVSCORE_MODE_ATTN */
  float softmax_scale;       /* multiplies q.k; <= 0 selects 1/sqrt(d); inf/NaN: EINVAL */
} kvscore_problem;

/* Version as major*10000 + minor*100 + patch. */
int32_t kvscore_version(void);

/* Message for the last error returned on this thread ("" if none). */
const char* kvscore_last_error(void);

/* Number of query tiles Tq the score pass splits a unit's G*W rows into. */
int32_t kvscore_num_query_tiles(const kvscore_problem* p);

/* Bytes of device workspace the entry point `which` (KVSCORE_WS_*) needs for p
 * (0 when it needs none). Returns 0 and sets the error on an invalid problem. */
size_t kvscore_workspace_size(const kvscore_problem* p, int32_t which);

/*
 * Window-query attention forward (DropKV page, Key Contribution 3: the
 * FlashAttention-2-style forward whose logsumexp the scorer reuses).
 * For every row: s_ij = scale * q_i.k_j (j <= t_i), lse_i = ln sum_j exp(s_ij),
 * a_i = sum_j p_ij v_j, jstar_i = argmax_j s_ij (lowest j on ties), and
 * dom_i = c* ||a_i - v_j*|| with c* = p* / (1 - p*), evaluated exactly as
 * p* ||a_i^(-j*) - v_j*|| (a^(-j) = output without key j), squared in mode SQ; in
 * mode ATTN, dom_i = p* (that pair's attention weight).
 * Inputs q_win, k, v (device, bf16). Outputs a, lse, jstar, dom (device).
 * workspace: device, >= kvscore_workspace_size(p, KVSCORE_WS_ATTN_FWD) bytes,
 * 256-byte aligned; contents are scratch. That size is 0 (workspace may be NULL) when
 * every sequence fits in one key chunk of the pass; otherwise it holds one record per
 * (unit, query tile, chunk).
 */
int kvscore_attn_fwd(const kvscore_problem* p, const void* q_win, const void* k, const void* v, float* a,
                     float* lse, int32_t* jstar, float* dom, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Score pass (DropKV page, "Methodology in Plain English", engineering paragraph):
 * for each unit, query tile qt and token j,
 *   partial[l][g][qt][cu_s + j] = sum over rows i of the tile with j <= t_i, j != jstar_i
 *       of c_ij * ||a_i - v_j||  (mode SQ: (c_ij * ||a_i - v_j||)^2; mode ATTN: p_ij,
 *       which reads no V, a or its norms),
 *   c_ij = p_ij / (1 - p_ij), p_ij = exp(s_ij - lse_i) recomputed from q and k,
 *   ||a_i - v_j||^2 = ||a_i||^2 - 2 a_i.v_j + ||v_j||^2 with a_i rounded to fp16.
 * Inputs: q_win, k, v (bf16), a, lse, jstar from kvscore_attn_fwd (device).
 * Output: partial (device). workspace: >= kvscore_workspace_size(p, KVSCORE_WS_SCORE).
 */
int kvscore_score(const kvscore_problem* p, const void* q_win, const void* k, const void* v, const float* a,
                  const float* lse, const int32_t* jstar, float* partial, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Split-K merge (DropKV page, Key Contribution 3): score[l][g][j] = the Tq partials
 * summed in ascending tile order, plus the isolated argmax terms dom_r of the unit's
 * rows with jstar_r = j, summed in row order. All device pointers.
 * With one query tile (Tq = 1) partial has score's layout, and the two may be the
 * same buffer: the terms are then added in place and the tile sum (a copy) is skipped.
 * Otherwise they must not overlap (KVSCORE_EINVAL when they are equal).
 */
int kvscore_merge(const kvscore_problem* p, const float* partial, const int32_t* jstar, const float* dom,
                  float* score, void* stream);

/*
 * Host-only layer budgets (RippleKV page, Eq. 9-12 under Eq. 5) for one sequence:
 *   s_hat = (s - min)/(max - min) (all 0 for a constant profile)   Eq. 9
 *   w~ = exp(ln(ratio) * s_hat)                                      Eq. 10
 *   w  = clip(w~, 1/gamma, gamma) rescaled to mean one               Eq. 11
 *   x_l = total/L * w_l                                              Eq. 12
 * then, if some x_l leaves [lo, hi], the x_l = clip(lambda*w_l, lo, hi) that still
 * sum to total, and largest-remainder rounding (ties to the lower layer) so that
 * sum b_l = total exactly. gamma = INFINITY (or <= 0) disables the clip.
 * sens: host [L] doubles (finite). budgets_out: host [L]. ratio >= 1.
 * Errors: KVSCORE_EINVAL (bad argument), KVSCORE_EBUDGET (total < L*lo or > L*hi).
 */
int kvscore_budget(const double* sens, int32_t num_layers, double ratio, double gamma, int64_t total,
                   int32_t lo, int32_t hi, int32_t* budgets_out);

/*
 * Host-only PyramidKV layer schedule (PyramidKV page, "Layer-Adaptive Dynamic Budget
 * Allocation"): b_l ~ lo + (C_max - lo) * (1 - l/(L-1))^gamma for 0-based l, with C_max
 * chosen so that the layers share `total` (the uniform total, reallocated). A layer with
 * factor 0 (the top one, gamma > 0) stays at lo; if some x_l = lo + lam*f_l would exceed
 * hi, the x_l = clip(lo + lam*f_l, lo, hi) that still sum to total are used; then
 * largest-remainder rounding (ties to the lower layer) gives sum b_l = total exactly.
 * budgets_out: host [L]. gamma >= 0 (1 = linear decay).
 * Errors: KVSCORE_EINVAL (bad argument), KVSCORE_EBUDGET (total < L*lo, or above
 * what the schedule can reach: each layer with a positive factor at hi, the others at lo).
 */
int kvscore_budget_pyramid(int32_t num_layers, double gamma, int64_t total, int32_t lo, int32_t hi,
                           int32_t* budgets_out);

/*
 * Host-only: packed segment offsets from per-(sequence, layer) budgets.
 * budgets: host int32 [S][L], each in [W, n_s]; offsets_out: host int64 [U+1] with
 * offsets[u+1] - offsets[u] = budgets[s][l] for u = (l*S + s)*Hkv + g.
 */
int kvscore_segment_offsets(const kvscore_problem* p, const int32_t* budgets, int64_t* offsets_out);

/*
 * Per-unit selection (DropKV page, "Methodology in Plain English": keep the largest
 * individual scores, pin the recent w tokens, max-pool over neighbouring scores after
 * SnapKV; "Preserve Attention Sinks": keep the first tokens; RippleKV Eq. 4: retained
 * positions per layer). For unit u with budget b = budgets[s][l] and ns = min(n_sink,
 * n_s - W): keep every j < ns, every j >= n_s - W, and the k = b - W - ns competitors
 * ns <= j < n_s - W with the largest ranking key (ties to the lower j); write them
 * ascending to kept_pos[seg_offsets[u] ..]. The ranking key is score[j], or with
 * pool > 1 the maximum of score over [j - pool/2, j + pool/2] within [0, n_s - W).
 * score: device fp32 [L][Hkv][N] (values >= 0). budgets: HOST int32 [S][L], each in
 * [W + ns, n_s] (validated here). seg_offsets: DEVICE copy of
 * kvscore_segment_offsets(p, budgets). kept_pos: device int32 [offsets[U]].
 * pool: odd, 1 <= pool <= 255 (1 = no pooling). n_sink >= 0 (0 = no sinks).
 * workspace: device, kvscore_workspace_size(p, KVSCORE_WS_TOPK) bytes (the pooled
 * keys), needed only when pool > 1 (may be NULL otherwise).
 * Errors: KVSCORE_EINVAL (bad pool / n_sink / pointer), KVSCORE_EBUDGET (a budget
 * outside [W + ns, n_s]), KVSCORE_EWORKSPACE.
 */
int kvscore_topk(const kvscore_problem* p, const float* score, const int32_t* budgets,
                 const int64_t* seg_offsets, int32_t* kept_pos, int32_t pool, int32_t n_sink, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * Selection with head budgets chosen jointly over the KV heads of each (sequence, layer)
 * (AdaDropKV: AdaKV's head budget allocation on the DropKV score, DropKV page, results on
 * adaptive head budgets; the rule itself is not on the pages, this is its plainest
 * reading). The layer keeps Hkv * b rows in all (b = budgets[s][l]); every head keeps its
 * first ns = min(n_sink, n_s - W) positions and its W most recent ones; the remaining
 * Hkv * (b - W - ns) slots go to the competitors (g, j), ns <= j < n_s - W, of all the
 * layer's heads with the largest ranking key (score or max-pooled score, as in
 * kvscore_topk), ties to the lower head, then the lower position.
 * workspace: device, kvscore_workspace_size(p, KVSCORE_WS_TOPK_HEADS) bytes, 256-byte
 * aligned: the select's scratch (per-layer state, per-chunk histograms, counts and
 * bitmasks, each layer's list of sampled-band keys), then the pooled keys; with pool = 1
 * only the scratch part (that size minus kvscore_workspace_size(p, KVSCORE_WS_TOPK)) is
 * needed. Calls on one stream reuse it. budgets (host) also choose which kernels are
 * launched (a sampled band for every layer, or histogram passes for those without one);
 * the result does not depend on that choice.
 * The other arguments as kvscore_topk; seg_offsets is still the DEVICE copy of
 * kvscore_segment_offsets(p, budgets) (it gives each layer's block). The heads' own
 * segments are data-dependent: their offsets go to head_offsets (device int64 [U+1],
 * inside the same blocks, head_offsets[U] = seg_offsets[U]) and their positions,
 * ascending, to kept_pos[head_offsets[u] ..]. Consume them with kvscore_compact_heads.
 */
int kvscore_topk_heads(const kvscore_problem* p, const float* score, const int32_t* budgets,
                       const int64_t* seg_offsets, int64_t* head_offsets, int32_t* kept_pos, int32_t pool,
                       int32_t n_sink, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Compaction into the packed ragged cache (RippleKV Eq. 4): for every segment u and
 * slot r in it, k_out[off[u] + r] = k row (l, g, cu_s + kept_pos[off[u] + r]), same
 * for v; a bit-exact copy. budgets: HOST [S][L] (sizes the launch); seg_offsets,
 * kept_pos: device; k_out, v_out: device bf16 [offsets[U]][d], 16-byte aligned.
 */
int kvscore_compact(const kvscore_problem* p, const void* k, const void* v, const int32_t* budgets,
                    const int64_t* seg_offsets, const int32_t* kept_pos, void* k_out, void* v_out,
                    void* stream);

/*
 * The same compaction for the segments of kvscore_topk_heads: head_offsets is its device
 * output; budgets (HOST [S][L]) size the launch for segments up to min(n_s, Hkv * b).
 */
int kvscore_compact_heads(const kvscore_problem* p, const void* k, const void* v, const int32_t* budgets,
                          const int64_t* head_offsets, const int32_t* kept_pos, void* k_out, void* v_out,
                          void* stream);

/*
 * Decode attention over the packed ragged cache (RippleKV page, "Problem Formulation":
 * during decoding every new query attends to the cached states, the retained pairs of
 * Eq. 4 after compression; GraceKV page, physical cache packing: one cache of its own
 * length per (layer, KV head)). For layer l, sequence s and query head h = g*G + hl, with
 * segment u = (l*S + s)*Hkv + g = rows off[u] .. off[u+1]-1 of the cache:
 *   out[l][s][h] = sum_r softmax_r(scale * k_r . q[l][s][h]) v_r,
 *   lse[l][s][h] = log sum_r exp(scale * k_r . q[l][s][h]).
 * Every row of a segment takes part (they all precede the new token; to attend to
 * appended tokens, lay them out inside the segments). Only num_seqs, num_layers,
 * num_q_heads, num_kv_heads (G = Hq/Hkv <= 8), head_dim (64 or 128) and softmax_scale of
 * p are used.
 *   q: device bf16 [L][S][Hq][d] contiguous, 16-byte aligned.
 *   k_cache, v_cache: device bf16 [off[U]][d], 16-byte aligned (kvscore_compact's
 *     k_out / v_out, or any cache laid out the same way).
 *   seg_offsets_host: HOST int64 [U+1], off[0] = 0, every segment non-empty (validated;
 *     sizes the launch). seg_offsets: its DEVICE copy.
 *   out: device fp32 [L][S][Hq][d]; lse: device fp32 [L][S][Hq] (natural log).
 *   workspace: device, kvscore_decode_workspace_size(p, seg_offsets_host) bytes.
 * Deterministic: the key splits and every partial sum are merged in a fixed order.
 * Errors: KVSCORE_EINVAL (shape, offsets, pointer or alignment), KVSCORE_EWORKSPACE.
 */
size_t kvscore_decode_workspace_size(const kvscore_problem* p, const int64_t* seg_offsets_host);
int kvscore_decode_attn(const kvscore_problem* p, const void* q, const void* k_cache, const void* v_cache,
                        const int64_t* seg_offsets_host, const int64_t* seg_offsets, float* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same decode attention with no workspace argument, for callers that cannot
 * allocate device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation). The split records go to a fixed device array of
 * KVSCORE_DECODE_SCRATCH_BYTES inside the library; each GPU holds its own copy from the
 * first call on it until the process ends. Nothing here allocates: no hipMalloc, no
 * hipFree, no allocating library call. Arguments, outputs and errors as
 * kvscore_decode_attn, plus KVSCORE_EWORKSPACE when the segments need more scratch than
 * the array holds (kvscore_decode_workspace_size() > KVSCORE_DECODE_SCRATCH_BYTES; then
 * use kvscore_decode_attn). Every call on one GPU uses that GPU's one array: calls that
 * may overlap on one GPU (several streams, or several threads) race and must be ordered
 * by the caller. The array keeps the last call's records; no call relies on its contents.
 */
#define KVSCORE_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int kvscore_decode_attn_noalloc(const kvscore_problem* p, const void* q, const void* k_cache, const void* v_cache,
                                const int64_t* seg_offsets_host, const int64_t* seg_offsets, float* out, float* lse,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVSCORE_H */
