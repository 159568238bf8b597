/*
 * ssw.h -- C ABI of libssw.so: Stochastic Attention (SA), sliding-window attention (SWA) and the
 * gated SA+SWA layer on AMD Instinct MI355X (gfx950): forward, and forward + backward for
 * training.
 *
 * The operation (from the pages):
 *   [SA-ja] "技術的概要：確率的アテンション" (gist.science/ja/paper/2604.00754), 手法 › 中核メカニズム:
 *     1. Permute: draw sigma ~ Uniform(S_n) for each layer, reorder the Q, K, V token rows by it;
 *     2. window attention: run standard sliding-window attention of window w in the permuted
 *        space (理論的性質 › 因果的制約: in the autoregressive setting the causal mask keeps only
 *        tokens that precede the query in the original order);
 *     3. Undo permute: apply sigma^-1 to the output.
 *   ゲート付き SA と SWA の組み合わせ: Y = g_sa (.) Y_sa + g_swa (.) Y_swa.
 *   [HYB] notes on "Rethinking the Role of Efficient Attention in Hybrid Architectures",
 *     ハイブリッドアーキテクチャの定義: SWA restricts position t to the w tokens before it.
 *
 * Exact semantics implemented (the readings of what the pages leave open):
 *   sigma[p] is the ORIGINAL index of the token at permuted slot p (gather convention).
 *   Query at slot p sees the keys at slots q with |p - q| <= w - 1, truncated at 0 and n - 1;
 *   when causal, only those with sigma[q] <= sigma[p].  With sigma = identity this is causal SWA
 *   over [t - w + 1, t].  Scores are scaled by 1/sqrt(d).  Query head h reads KV head
 *   h / (Hq / Hkv).  The output row of slot p is written at original position sigma[p].
 *
 * Layouts (all row-major, contiguous, token-major "BSHD"):
 *   q, out  [B, n, Hq,  d]     k, v  [B, n, Hkv, d]     element type given by `dtype`
 *   sigma   int32 [n]          one permutation per call, shared by every batch row and head
 *   gate    float32 [B, n, Hq] (single-path calls, optional)
 *   gates   float32 [2, B, n, Hq] (gated call; g_sa first, then g_swa), indexed by ORIGINAL
 *           token position, broadcast over d.
 *
 * Ownership and execution: every tensor pointer of the forward calls is a DEVICE pointer owned
 * by the caller; the library never allocates, frees or keeps them.  Work is enqueued on
 * `stream` (a hipStream_t; NULL = the default stream) and the call returns without waiting.
 * q, k, v and out must not overlap.  Inputs are not modified.
 *
 * Errors: every entry point returns SSW_OK (0) or a negative ssw_status and never aborts or
 * throws.  Arguments are checked before anything is enqueued; on an error nothing is launched
 * and ssw_last_error() (per calling thread) describes it.  B == 0 or n == 0 is a valid empty
 * call that does nothing.
 */
#ifndef SSW_H
#define SSW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSW_F32 = 0, SSW_BF16 = 1 } ssw_dtype;

typedef enum {
  SSW_OK = 0,
  SSW_EINVAL = -1,   /* window < 1, negative size, NULL required pointer, causal not 0/1 */
  SSW_ESHAPE = -2,   /* Hq not a multiple of Hkv, or sizes whose index range overflows:
                        n * Hq * d * element size must be <= 2^31 - 4096 bytes, n <= 2^24 - 64,
                        n * Hq / Hkv <= 2^31 - 4096 and B * Hkv < 65536 */
  SSW_EDTYPE = -3,   /* d not 64 or 128, or dtype not SSW_F32 / SSW_BF16 */
  SSW_EALIGN = -4,   /* q, k, v, out not 16-byte aligned; sigma, gates not 4-byte aligned */
  SSW_ENOTPERM = -5, /* sigma is not a permutation of [0, n) (only detected when checked) */
  SSW_EHIP = -6      /* a HIP runtime call or kernel launch failed */
} ssw_status;

/* Stochastic Attention forward ([SA-ja] 中核メカニズム steps 1-3, 因果的制約).
 *   q, k, v   device, layouts above, element type `dtype`.
 *   sigma     device int32[n], a permutation of [0, n).  It is trusted; set the environment
 *             variable SSW_VALIDATE=1 to have every call copy it back and check it (slow,
 *             synchronous; returns SSW_ENOTPERM on failure).
 *   window    w >= 1 (values >= n behave as n: full attention, causal or not).
 *   causal    0 or 1.
 *   gate      device float32 [B, n, Hq] or NULL: out = gate (.) Y_sa when given, else Y_sa.
 *   out       device, [B, n, Hq, d], type `dtype`; fully overwritten.
 *   d         64 or 128.  dtype SSW_F32 or SSW_BF16 (fp32 accumulation either way; bf16
 *             results are rounded to nearest even once, at the store). */
int ssw_sa_forward(const void* q, const void* k, const void* v, const int32_t* sigma,
                   int window, int causal, const float* gate, void* out,
                   int B, int n, int Hq, int Hkv, int d, int dtype, void* stream);

/* Sliding-window attention forward ([HYB] ハイブリッドアーキテクチャの定義): the same operator
 * with sigma = identity.  `sigma` must be NULL (anything else is SSW_EINVAL).  Other arguments
 * as in ssw_sa_forward. */
int ssw_swa_forward(const void* q, const void* k, const void* v, const int32_t* sigma,
                    int window, int causal, const float* gate, void* out,
                    int B, int n, int Hq, int Hkv, int d, int dtype, void* stream);

/* Gated dual path ([SA-ja] ゲート付き SA と SWA の組み合わせ):
 *   out = g_sa (.) SA(q, k, v; sigma, w, causal) + g_swa (.) SWA(q, k, v; w, causal).
 *   gates     device float32 [2, B, n, Hq], required.  Both paths use the same w and causal.
 * Two kernels run back to back on `stream`: the SA pass leaves g_sa (.) Y_sa in `out` as an
 * intermediate, at the scattered rows sigma[p], then the SWA pass reads it at its own rows, adds
 * g_swa (.) Y_swa and stores the sum.  For fp32 the intermediate is fp32.  For bf16 it is held,
 * in the same two bytes per element, as fp16 bits of g_sa (.) Y_sa * 2^-4, so the result is in
 * effect rounded to bf16 once: for |g_sa (.) Y_sa| >= 2^-10 that keeps 3 more significand bits
 * than bf16; below it the step is a fixed 2^-20 (absolute error <= 2^-21 = 4.8e-7), as fine as
 * bf16's own step down to |g_sa (.) Y_sa| = 2^-13.  It needs |g_sa (.) Y_sa| < 1.05e6 (true
 * whenever |V| < 1.05e6: Y is a convex combination of V rows); larger values become infinite.
 * Between the two passes `out` holds that intermediate, not a result.  Other arguments as in
 * ssw_sa_forward. */
int ssw_gated_sa_swa_forward(const void* q, const void* k, const void* v, const int32_t* sigma,
                             int window, int causal, const float* gates, void* out,
                             int B, int n, int Hq, int Hkv, int d, int dtype, void* stream);

/* Same as ssw_gated_sa_swa_forward, and additionally times each of its two kernels (the SA
 * pass runs first): the given HIP events (hipEvent_t created by the caller; each may be NULL) are attached to the kernels'
 * dispatches, so ev_swa_start / ev_swa_end are recorded when the SWA pass starts and ends and
 * ev_sa_start / ev_sa_end likewise for the SA pass.  No separate event packets are queued, so the
 * calls run back to back as in the untimed form and hipEventElapsedTime gives each kernel's own
 * duration. */
int ssw_gated_sa_swa_forward_timed(const void* q, const void* k, const void* v,
                                   const int32_t* sigma, int window, int causal,
                                   const float* gates, void* out, int B, int n, int Hq, int Hkv,
                                   int d, int dtype, void* stream, void* ev_swa_start,
                                   void* ev_swa_end, void* ev_sa_start, void* ev_sa_end);

/* ---- Variant: one sigma per batch row and/or per KV head ----
 *
 * [SA-ja] 中核メカニズム draws one permutation per layer; sharing it across the batch and the
 * heads is this library's default reading.  These calls let every (batch row b, KV head g) use
 * its own permutation, found at sigma + b * sigma_batch_stride + g * sigma_head_stride
 * (elements; each a permutation of [0, n); strides >= 0, and 0 shares it along that axis).  The
 * query heads of one KV head share its sigma, since they attend to the same gathered K/V rows.
 * Other arguments as in ssw_sa_forward / ssw_gated_sa_swa_forward (the SWA path of the gated
 * call needs no sigma).  SSW_VALIDATE=1 checks every permutation used. */
int ssw_sa_forward_ex(const void* q, const void* k, const void* v, const int32_t* sigma,
                      int64_t sigma_batch_stride, int64_t sigma_head_stride, int window,
                      int causal, const float* gate, void* out, int B, int n, int Hq, int Hkv,
                      int d, int dtype, void* stream);

int ssw_gated_sa_swa_forward_ex(const void* q, const void* k, const void* v, const int32_t* sigma,
                                int64_t sigma_batch_stride, int64_t sigma_head_stride, int window,
                                int causal, const float* gates, void* out, int B, int n, int Hq,
                                int Hkv, int d, int dtype, void* stream);

/* ---- Gate projections of the gated layer ----
 *
 * [SA-ja] ゲート付き SA と SWA の組み合わせ computes g_sa and g_swa by independent sigmoid
 * projections of the layer input.  This call computes both in one pass over x:
 *     gates[p][r][h] = sigmoid(sum_k x[r][k] * w_t[p * Hq + h][k] + bias[p * Hq + h])
 * for path p (0: SA, 1: SWA), token row r (= b * n + i) and query head h, directly in the
 * [2, B, n, Hq] layout ssw_gated_sa_swa_forward takes.
 *   x      device bf16 [rows, Hm], 16-byte aligned; Hm a multiple of 16.
 *   w_t    device bf16 [2 * Hq, Hm] (a linear layer's weight layout: one row per output),
 *          16-byte aligned; 1 <= Hq <= 64.
 *   bias   device float32 [2 * Hq] or NULL.
 *   gates  device float32 [2, rows, Hq], overwritten.
 * fp32 accumulation; bf16 only (SSW_EDTYPE otherwise). */
int ssw_gate_projection(const void* x, const void* w_t, const float* bias, float* gates, int rows,
                        int Hm, int Hq, int dtype, void* stream);

/* ---- Training: forward with the rows' log-sum-exp, backward, gated forward and backward ----
 *
 * The pages pretrain a model from scratch with the gated layer ([SA-ja] 主要な貢献 item 3 and
 * 結果, 事前学習), so the layer has a backward pass.  It is the exact gradient of the forward
 * above (chain rule through its definition; no page prescribes more).  With A the attention
 * output of a row (SA or SWA), y = g (.) A its gated form (g = 1 when no gate is given),
 * P the row's softmax weights, s = 1/sqrt(d) and dy = dL/dy:
 *   dV_j += P_j g dy,   dS_j = P_j (<g dy, V_j> - <g dy, A>),
 *   dQ = s sum_j dS_j K_j,   dK_j += s dS_j Q,   dg = <dy, A>.
 * The training calls take bf16 tensors only (SSW_EDTYPE otherwise); accumulation is fp32 and
 * every bf16 result is rounded to nearest even at its store. */

/* SA forward without a gate that also stores, for every row, lse = log sum_j exp(s <Q, K_j>)
 * over the row's neighbours (natural log; the backward rebuilds P from it).
 *   out       device [B, n, Hq, d]: A (no gate), fully overwritten.
 *   lse       device float32 [B, n, Hq], indexed by original token; fully overwritten.
 * Other arguments as in ssw_sa_forward (fp32 and bf16 both allowed here). */
int ssw_sa_forward_lse(const void* q, const void* k, const void* v, const int32_t* sigma,
                       int window, int causal, void* out, float* lse,
                       int B, int n, int Hq, int Hkv, int d, int dtype, void* stream);

/* The same for SWA (sigma must be NULL). */
int ssw_swa_forward_lse(const void* q, const void* k, const void* v, const int32_t* sigma,
                        int window, int causal, void* out, float* lse,
                        int B, int n, int Hq, int Hkv, int d, int dtype, void* stream);

/* SA backward of y = gate (.) A, A = SA(q, k, v; sigma, w, causal).
 *   q, k, v, sigma, window, causal   as given to the forward.
 *   gate      device float32 [B, n, Hq] or NULL (gate 1).
 *   out, lse  A and lse as stored by ssw_sa_forward_lse.
 *   dout      device [B, n, Hq, d]: dL/dy.
 *   dq        device [B, n, Hq, d];  dk, dv  device [B, n, Hkv, d].  Written whole, or, when
 *             accumulate = 1, the gradients are added to what they hold (each element read,
 *             added in fp32, rounded once).
 *   dgate     device float32 [B, n, Hq] or NULL: dL/dgate = <dy, A> per row (overwritten).
 *   delta     device float32 [B, n, Hq]: scratch the call overwrites (g <dy, A> per row).
 *   accumulate  0 or 1.
 * Two kernels run back to back on `stream` (dQ, which also writes delta and dgate, then dK/dV).
 * dq, dk, dv, dgate and delta must not overlap each other or the inputs.  bf16 only. */
int ssw_sa_backward(const void* q, const void* k, const void* v, const int32_t* sigma,
                    int window, int causal, const float* gate, const void* out, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* dgate, float* delta,
                    int accumulate, int B, int n, int Hq, int Hkv, int d, int dtype, void* stream);

/* The same for SWA (sigma must be NULL; out and lse from ssw_swa_forward_lse). */
int ssw_swa_backward(const void* q, const void* k, const void* v, const int32_t* sigma,
                     int window, int causal, const float* gate, const void* out,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     float* dgate, float* delta, int accumulate, int B, int n, int Hq, int Hkv,
                     int d, int dtype, void* stream);

/* Training forward of the gated layer: y_swa, lse_swa = SWA with lse; y_sa, lse_sa = SA with
 * lse; then out = g_sa (.) y_sa + g_swa (.) y_swa from the stored bf16 values (one rounding).
 * Three kernels on `stream`.  y_sa, y_swa device [B, n, Hq, d]; lse_sa, lse_swa device float32
 * [B, n, Hq]; all overwritten.  Keep y_sa, lse_sa, y_swa, lse_swa for the backward.  bf16 only;
 * other arguments as in ssw_gated_sa_swa_forward. */
int ssw_gated_sa_swa_forward_train(const void* q, const void* k, const void* v,
                                   const int32_t* sigma, int window, int causal,
                                   const float* gates, void* out, void* y_sa, float* lse_sa,
                                   void* y_swa, float* lse_swa, int B, int n, int Hq, int Hkv,
                                   int d, int dtype, void* stream);

/* Backward of the gated layer: dq, dk, dv (overwritten) = the SA path's gradients with gate g_sa
 * plus the SWA path's with gate g_swa; dgates device float32 [2, B, n, Hq] or NULL receives
 * (<dy, y_sa>, <dy, y_swa>).  delta is scratch as in ssw_sa_backward.  Four kernels on
 * `stream`; the SWA path adds to the SA path's bf16 results, so dq, dk, dv are rounded twice. */
int ssw_gated_sa_swa_backward(const void* q, const void* k, const void* v, const int32_t* sigma,
                              int window, int causal, const float* gates, const void* y_sa,
                              const float* lse_sa, const void* y_swa, const float* lse_swa,
                              const void* dout, void* dq, void* dk, void* dv, float* dgates,
                              float* delta, int B, int n, int Hq, int Hkv, int d, int dtype,
                              void* stream);

/* The same backward for callers that cannot allocate memory (code under HIP graph capture, tight
 * training loops, harnesses that forbid hipMalloc): no delta argument; Delta lives in a device
 * array of the library itself (16 MiB per GPU, held until the process ends), so the call
 * allocates nothing.  Limit: B * n * Hq <= 4194304 (2^22), else SSW_ESHAPE.  Every call on one
 * GPU shares that array, so calls that overlap on one GPU (other streams, other threads) race and
 * must be ordered by the caller.  The first call on a device looks the array's address up
 * (SSW_EHIP if that fails).  Other arguments, results and errors as in
 * ssw_gated_sa_swa_backward. */
int ssw_gated_sa_swa_backward_noalloc(const void* q, const void* k, const void* v,
                                      const int32_t* sigma, int window, int causal,
                                      const float* gates, const void* y_sa, const float* lse_sa,
                                      const void* y_swa, const float* lse_swa, const void* dout,
                                      void* dq, void* dk, void* dv, float* dgates, int B, int n,
                                      int Hq, int Hkv, int d, int dtype, void* stream);

/* ---- Decode: one new token per batch row over a KV cache ----
 *
 * The pages apply SA to pretrained models without training ([SA-ja] 主要な貢献 item 3, 結果),
 * i.e. generating from a cache, but do not say how sigma evolves as the cache grows.  Reading:
 * sigma is drawn once per layer over the full context length n_max, and decoding the token at
 * position t computes exactly row t of causal SA over that length (中核メカニズム, 因果的制約):
 * the query attends to the cached tokens sigma[q] for slots |q - sigma^-1(t)| <= w - 1 with
 * sigma[q] <= t, all of which precede t.  The SWA step attends to positions [t - w + 1, t].
 *   q         device [B, Hq, d]: the new token's query of each batch row.
 *   k_cache, v_cache  device [B, n_max, Hkv, d]: positions 0..pos[b] of row b filled (the new
 *             token's own K/V included).  Only positions <= pos[b] are read.
 *   sigma, inv_sigma  device int32 [n_max]: the layer's permutation and its inverse.
 *   pos       device int32 [B]: t of each batch row, in [0, n_max) (rows may differ).  A position
 *             outside that range makes that row's output NaN.
 *   window    w >= 1 (values >= n_max behave as n_max).
 *   gate      device float32 [B, Hq] or NULL (single path); gates [2, B, Hq] (gated call).
 *   out       device [B, Hq, d], overwritten.
 * Hq / Hkv must be <= 8 (SSW_ESHAPE otherwise).  fp32 or bf16; one kernel launch. */
int ssw_sa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* sigma,
                  const int32_t* inv_sigma, const int32_t* pos, int window, const float* gate,
                  void* out, int B, int n_max, int Hq, int Hkv, int d, int dtype, void* stream);

/* SWA decode step: sigma and inv_sigma must be NULL. */
int ssw_swa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* sigma,
                   const int32_t* inv_sigma, const int32_t* pos, int window, const float* gate,
                   void* out, int B, int n_max, int Hq, int Hkv, int d, int dtype, void* stream);

/* Gated decode step: out = g_sa (.) SA step + g_swa (.) SWA step in one kernel (gates required). */
int ssw_gated_sa_swa_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* sigma, const int32_t* inv_sigma, const int32_t* pos,
                            int window, const float* gates, void* out, int B, int n_max, int Hq,
                            int Hkv, int d, int dtype, void* stream);

/* Host helpers (HOST pointers, no GPU needed). */

/* sigma ~ Uniform(S_n) for one layer ([SA-ja] 中核メカニズム step 1) from a seeded Fisher-Yates
 * shuffle (Durstenfeld form, i from n-1 down to 1, j = floor(r * (i + 1) / 2^64)) driven by
 * splitmix64 (Steele, Lea & Flood 2014; state starts at `seed`).  Writes sigma_out[n] and, when
 * inv_out is not NULL, inv_out[n] with inv_out[sigma_out[p]] = p.  n >= 0. */
int ssw_make_permutation(uint64_t seed, int n, int32_t* sigma_out, int32_t* inv_out);

/* inv_out[sigma[p]] = p (the un-permute map of [SA-ja] step 3); SSW_ENOTPERM if sigma is not a
 * permutation of [0, n). */
int ssw_inverse_permutation(const int32_t* sigma, int n, int32_t* inv_out);

/* SSW_OK if sigma (host int32[n]) is a permutation of [0, n), else SSW_ENOTPERM.  [SA-ja]
 * 中核メカニズム step 1 draws sigma uniformly from the permutations of the n positions, so the
 * forward calls take sigma to be one (they trust it unless SSW_VALIDATE=1 makes them run this
 * check first).  No GPU; sigma is not modified; n >= 0. */
int ssw_check_permutation(const int32_t* sigma, int n);

/* Debug: the random neighbourhood of every token ([SA-ja] 中核メカニズム: the neighbours of
 * token i are the tokens whose permuted slots lie within w - 1 of i's slot, and in causal mode
 * only those not after i; with sigma NULL the SWA window of [HYB] ハイブリッドアーキテクチャの
 * 定義), as a bitmask computed on the device with the membership test the attention kernels use.
 * bits (device uint32 [n][ceil(n/32)], owned by the caller, fully overwritten): bit j of row i is
 * set iff original token i attends to original token j.  sigma: device int32[n] or NULL.
 * Enqueued on `stream`.  Errors: SSW_EINVAL (n < 0, window < 1, causal not 0 or 1, bits NULL),
 * SSW_ESHAPE (n > 65536: the mask takes n^2 / 8 bytes; meant for small n), SSW_EALIGN (sigma or
 * bits not 4-byte aligned), SSW_EHIP (a launch failed). */
int ssw_neighbor_mask(const int32_t* sigma, int n, int window, int causal, uint32_t* bits,
                      void* stream);

/* Receptive-field growth over depth, for the theory check of [SA-ja] 理論的性質 (受容野の
 * 成長): SWA's field grows linearly with depth, SA's exponentially, and full coverage takes
 * O(log_w n) SA layers.  Host computation, no GPU.
 *   With the neighbour sets of the attention kernels (mode 0: SA, 1: SWA, 2: the gated layer's
 *   union of both; causal 0 or 1) and layer l's sigma = ssw_make_permutation(seeds[l], n):
 *     R_0(i) = {i},   R_l(i) = union of R_{l-1}(j) over the neighbours j of i at layer l.
 *   coverage_out[l - 1] = sum_i |R_l(i)| / (number of pairs): the share of pairs (j <= i when
 *   causal, all n^2 otherwise) whose information has reached i after l layers.
 *   n in [1, 32768] (memory ~ n^2 / 4 bytes); seeds (host, `layers` entries; NULL allowed for
 *   mode 1); coverage_out (host, `layers` doubles). */
int ssw_receptive_field_coverage(int n, int window, int layers, const uint64_t* seeds, int mode,
                                 int causal, double* coverage_out);

/* Message describing the most recent failed call on the calling thread ("" if none).  The string
 * belongs to the library (thread-local storage) and stays valid until that thread's next failed
 * call; it is not a passage of the method but the error channel of every entry point above. */
const char* ssw_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SSW_H */
