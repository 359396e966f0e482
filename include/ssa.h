/*
 * ssa.h -- skip-softmax (BLASST) sparse attention for MI355X (gfx950), C ABI.
 *
 * The library computes the non-causal self-attention forward of video
 * diffusion transformers with KV-tile skipping, and the companion
 * calibration pass that measures skip ratios at many thresholds at once.
 *
 * Method sources (web pages, cited by title and section):
 *  [README]  ModelOpt diffusers sparsity README, "Skip-Softmax Sparse
 *            Attention for Diffusion Models": introduction, "Threshold
 *            Modes", "Known Issues".
 *  [TRITON]  ModelOpt pull request "skip-softmax ... via dedicated Triton
 *            kernels": "Changes / Triton kernels", "Kernel backends",
 *            "Method", "Calibration", "Threshold modes".
 *  [PR1166]  ModelOpt pull request #1166 "Add the Skip softmax for
 *            diffusion": "Usage" (br = bc = 128, non-causal, threshold trials).
 *  [TRTLLM]  TensorRT-LLM pull request "Add SkipSoftmax sparse attention
 *            support for visual generation": "Use Cases", "Priority Order".
 *  [DOCS]    TensorRT-LLM docs "VisualGen Sparse Attention (Beta)":
 *            "Skip Softmax Attention", "User Configuration".
 *
 * Conventions shared by every entry point
 *  - Every function returns an int status: 0 = SSA_OK, > 0 = a warning (the
 *    outputs are valid), < 0 = an error (outputs untouched unless stated).
 *    Nothing falls back silently to dense attention.
 *  - Tensors are bf16 (q, k, v may instead be fp8 e4m3, see SSA_DTYPE_*),
 *    packed "varlen": token-major [T, H, D] with T the sum
 *    of the B sequence lengths (the [B, S, H, D] -> varlen conversion of
 *    [TRITON] "Kernel backends"). Element (token t, head h, dim d) sits at
 *    t * stride_token + h * stride_head + d; D is contiguous. Base pointers
 *    must be 16-byte aligned and both strides multiples of 8 elements.
 *    Each head's rows, up to the end of its last tile, must lie within
 *    2^32 - 1 bytes of its first row (the kernels' buffer offsets are 32-bit:
 *    SSA_ERR_UNSUPPORTED otherwise); with H > 1, stride_head is at most 2^47
 *    (SSA_ERR_INVALID_ARG otherwise).
 *  - Device pointers are caller-owned device memory (e.g. torch CUDA/HIP
 *    tensors). The library allocates no device memory and keeps no state
 *    between calls; it is reentrant. GPU work is enqueued on `stream`
 *    (a hipStream_t, NULL = the legacy default stream) and is asynchronous:
 *    outputs are ready once the stream is synchronized. Kernel-launch
 *    failures are reported as SSA_ERR_HIP.
 *  - Calls that overlap on the same output buffers race; the caller orders them.
 */
#ifndef SSA_H_
#define SSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define SSA_OK                   0
#define SSA_WARN_EXTRAPOLATED    1  /* target sparsity outside the calibrated range */
#define SSA_ERR_INVALID_ARG     -1  /* null pointer, bad shape/stride/alignment, NaN */
#define SSA_ERR_UNSUPPORTED     -2  /* head_dim or block not built, too many heads */
#define SSA_ERR_THRESHOLD_RANGE -3  /* resolved lambda outside [0, 1] */
#define SSA_ERR_NO_FORMULA      -4  /* target sparsity requested without a formula */
#define SSA_ERR_FIT_DEGENERATE  -5  /* fewer than two distinct usable sparsities */
#define SSA_ERR_HIP             -6  /* HIP runtime / kernel launch failure */

typedef void* ssa_stream_t; /* hipStream_t */

/* ---- problem description ----------------------------------------------- */
/* Self-attention over B packed sequences: q, k and v share cu_seqlens
 * (S_q = S_k per sequence). Diffusion self-attention is non-causal
 * ([PR1166] "Usage": is_causal False); causal = 1 selects the prefill form
 * (query i attends keys 0..i of its sequence; [PR1166] "Usage" and [TRTLLM]
 * "Use Cases" carry the LLM prefill threshold key). The tile size
 * block = Br = Bc is part of the method's definition, because skip decisions
 * are taken per Br x Bc tile ([PR1166] "Usage": br = bc = 128). */
typedef struct ssa_problem {
  int32_t batch;             /* B >= 1 sequences                                  */
  int32_t num_heads;         /* H in [1, 512]                                     */
  int32_t head_dim;          /* D in {64, 128}                                    */
  int32_t block;             /* Br = Bc in {64, 128}                              */
  const int32_t* cu_seqlens; /* HOST array [B + 1]: cu[0] = 0, non-decreasing;
                                sequence b is tokens [cu[b], cu[b+1]); empty
                                sequences are allowed. The library sees only the
                                tensors' pointers, so cu[B] <= T (the rows the
                                tensors hold) is the caller's duty; the Python
                                binding checks it before any launch            */
  int64_t stride_token;      /* elements between tokens, same for q, k, v, o       */
  int64_t stride_head;       /* elements between heads, same for q, k, v, o        */
  double sm_scale;           /* softmax scale; 0 selects 1 / sqrt(D)               */
  int32_t causal;            /* 0 = non-causal, 1 = causal (keys 0..i for query i) */
  int32_t dtype;             /* SSA_DTYPE_*: element type of q, k and v (o is bf16) */
  double scale_q, scale_k, scale_v; /* SSA_DTYPE_FP8_E4M3: dequantization scales,
                                value = code * scale, each finite and > 0; ignored
                                otherwise                                          */
  const uint8_t* block_scale_q;      /* SSA_DTYPE_MXFP8_QK: DEVICE E8M0 scales of q,
                                        [T, H, D / 32] bytes; ignored otherwise   */
  const uint8_t* block_scale_k;      /* the same for k                             */
  int64_t block_scale_stride_token;  /* bytes between tokens of both scale arrays  */
  int64_t block_scale_stride_head;   /* bytes between heads of both scale arrays   */
} ssa_problem;

/* Element types of q, k, v. SSA_DTYPE_FP8_E4M3 is the OCP e4m3 ("e4m3fn")
 * byte format with one scale per tensor: Q K^T and P V run on the fp8
 * matrix cores, P is rounded to e4m3 (round to nearest even) for P V, the
 * skip test uses the fp32 scores of the dequantized values, and o is bf16
 * with the same element strides. Row starts must be 16-byte aligned (strides
 * multiples of 16 elements). ([TRTLLM] "Use Cases" and [DOCS] list FP8
 * attention beside BF16.) */
#define SSA_DTYPE_BF16     0
#define SSA_DTYPE_FP8_E4M3 1
/* SSA_DTYPE_MXFP8_QK: block-scaled ("MXFP8") q and k with bf16 v ([DOCS]
 * "Skip Softmax Attention": skip-softmax combined with block-scaled Q/K).
 * q and k are OCP e4m3 bytes; each run of 32 consecutive elements along D
 * of one (token, head) row shares one E8M0 scale byte (value 2^(e - 127);
 * e = 255 is not allowed), so value = code * scale. Q K^T runs on the fp8
 * matrix cores with these block scales (exact products, fp32 sums), the
 * skip test uses those fp32 scores, and v, P, P.V and o are as in bf16 mode.
 * Element strides are shared by q, k, v, o and must be multiples of 16; the
 * scale arrays' base pointers must be aligned to D / 32 bytes and their two
 * strides multiples of D / 32 bytes. */
#define SSA_DTYPE_MXFP8_QK 2

/* ---- thresholds for the forward ---------------------------------------- */
/* How the per-(sequence, head) threshold reaches the kernel ([README]
 * "Threshold Modes"; [TRITON] "Threshold modes"):
 *   SSA_THRESH_LAMBDA       value = lambda in [0, 1]; kernel compares against
 *                           log2(lambda). lambda = 0 is dense (nothing skipped).
 *   SSA_THRESH_LOG2         value = log2(lambda) passed through unchanged
 *                           ("raw" threshold); -inf is dense; must be <= 0.
 *   SSA_THRESH_SCALE_FACTOR value = scale factor sf; lambda = sf / S_b with S_b
 *                           the key length of sequence b ([README] "Threshold
 *                           Modes", calibrated row). sf = 0 is dense.
 * A resolved lambda outside [0, 1] (or NaN) is SSA_ERR_THRESHOLD_RANGE. */
#define SSA_THRESH_LAMBDA       0
#define SSA_THRESH_LOG2         1
#define SSA_THRESH_SCALE_FACTOR 2

typedef struct ssa_thresholds {
  int32_t kind;          /* SSA_THRESH_*                                         */
  int32_t count;         /* 1 (same for all heads) or H (one value per head)     */
  const double* values;  /* HOST array of `count` values                          */
} ssa_thresholds;

/* ---- the forward ------------------------------------------------------- */
/* Skip-softmax FlashAttention forward ([TRITON] "Triton kernels", the forward
 * kernel; [README] introduction). For each sequence b, head h and Q-block i
 * (rows i*block .. i*block+block-1), KV tiles j = 0, 1, ... are visited in
 * ascending order. With s = (q . k) * sm_scale * log2(e), rowmax_r the tile's
 * maximum score in row r and m_r the running maximum before the tile,
 * d = max over the block's valid rows of (rowmax_r - m_r); the tile is
 * skipped when d < log2(lambda): its V is not loaded, no exponential and no
 * P.V is computed, and the running statistics are left unchanged. Kept tiles
 * update the online softmax as in FlashAttention. The first tile is never
 * skipped. With causal = 1, Q-block i visits tiles 0..i only; keys after a
 * query are excluded from its scores, row maxima and softmax. Scores are
 * accumulated in fp32 from bf16 inputs, P is rounded to bf16 for the P.V
 * product, O is rounded to bf16.
 *
 *  q, k, v    device, bf16 [T, H, D] (see conventions)
 *  o          device, bf16 [T, H, D], written for every valid token
 *  th         host, thresholds (see above)
 *  skipped_bh device uint64 [B * H] or NULL: skipped KV tiles per (b, h)
 *  total_bh   device uint64 [B * H] or NULL: visited KV tiles per (b, h)
 *             (nQ^2 non-causal, nQ (nQ + 1) / 2 causal)
 *             (both are overwritten, not accumulated: the library zeroes them)
 *  tile_mask  device uint8 [B, H, nq_max, nk_max] or NULL (debug): 0 = tile
 *             kept, 1 = skipped, 2 = no such tile; dims from ssa_tile_mask_dims.
 * Errors: SSA_ERR_INVALID_ARG, SSA_ERR_UNSUPPORTED, SSA_ERR_THRESHOLD_RANGE,
 * SSA_ERR_HIP. */
int ssa_attn_fwd(const ssa_problem* p, const void* q, const void* k, const void* v, void* o,
                 const ssa_thresholds* th, uint64_t* skipped_bh, uint64_t* total_bh,
                 uint8_t* tile_mask, ssa_stream_t stream);

/* nq_max = nk_max = ceil(max_b S_b / block): the tile_mask's last two dims. */
int ssa_tile_mask_dims(const ssa_problem* p, int64_t* nq_max, int64_t* nk_max);

/* ---- calibration ------------------------------------------------------- */
/* Calibration pass ([TRITON] "Triton kernels", the calibration kernel):
 * computes full (dense) attention into `o` while counting, for n thresholds
 * at once, the KV tiles that the forward would skip at each lambda_k: one
 * per-work-group row of counts, no atomics. Decisions use exactly the
 * forward's arithmetic, so counts[w][k] equals the number of tiles the
 * forward skips in work-group w at lambda_k.
 *
 *  lambdas  host double [n], ascending, each in (0, 1]; n in [1, 64]
 *           (e.g. 16 values log-spaced over [1e-6, 0.7], or the threshold
 *           trial list of [PR1166] "Usage")
 *  counts   device int32 [num_wg, n]: counts[w * n + k]
 *  tiles    device int32 [num_wg]: KV tiles visited by work-group w
 * Work-group w enumerates (b, h, i) sequence-major, then head, then Q-block:
 * w = sum_{b' < b} H * nQ_b' + h * nQ_b + i with nQ_b = ceil(S_b / block).
 * num_wg comes from ssa_calib_num_workgroups.
 * Errors: SSA_ERR_INVALID_ARG, SSA_ERR_UNSUPPORTED, SSA_ERR_THRESHOLD_RANGE,
 * SSA_ERR_HIP. */
int ssa_attn_calibrate(const ssa_problem* p, const void* q, const void* k, const void* v,
                       void* o, const double* lambdas, int32_t n, int32_t* counts,
                       int32_t* tiles, ssa_stream_t stream);

int ssa_calib_num_workgroups(const ssa_problem* p, int64_t* num_wg);

/* Host-side reduction of a calibration pass into per-sequence tile sparsity
 * ("tile skip ratios", [README] "Quick Start"): sparsity[b * n + k] =
 * sum of counts over sequence b's work-groups / sum of their tiles.
 * counts/tiles are HOST copies of the calibrate outputs. Sequences with no
 * tiles get NaN. */
int ssa_calibration_sparsity(const ssa_problem* p, const int32_t* counts, const int32_t* tiles,
                             int32_t n, double* sparsity);

/* Log-space fit of scale_factor = a * exp(b * sparsity) ([README]
 * introduction; [TRITON] "Calibration": log-space fitting minimises relative
 * error and records the observed sparsity range). Point i is (lambda[i],
 * sparsity[i], seq_k[i]) with scale_factor_i = lambda[i] * seq_k[i]; ordinary
 * least squares of ln(scale_factor) on sparsity over the points with
 * 0 < sparsity < 1 and lambda > 0 (0 and 1 are plateaus with no slope
 * information). s_min / s_max are the smallest / largest fitted sparsity.
 * All pointers are host. Errors: SSA_ERR_INVALID_ARG (also a NaN or infinite
 * value in any point), SSA_ERR_FIT_DEGENERATE. */
typedef struct ssa_calib_result {
  double a, log_a, b;  /* scale_factor = a * exp(b * s) = exp(log_a + b * s) */
  double s_min, s_max; /* observed sparsity range of the fitted points       */
  int32_t n_used;      /* points used                                        */
} ssa_calib_result;

int ssa_calibration_fit(const double* lambda, const double* sparsity, const double* seq_k,
                        int32_t n, ssa_calib_result* out);

/* Linear-space variant of the fit: minimises sum_i (a e^{b s_i} - y_i)^2 with
 * y_i = lambda_i * seq_k_i over the same usable points ([TRITON]
 * "Calibration" / "Config & conversion": fit_logspace = False is the
 * calibrator's default, the log-space fit the recommended one for
 * diffusion). For fixed b the best a is closed-form, so b maximises
 * H(b) = (sum y e^{bs})^2 / sum e^{2bs}. The search scans b over the
 * log-space slope +- 100 in steps of 0.1, then bisects dH/db = 0 around the
 * best grid point. Errors: SSA_ERR_INVALID_ARG, SSA_ERR_FIT_DEGENERATE (also
 * when the optimum lies at the edge of the scan). */
int ssa_calibration_fit_linear(const double* lambda, const double* sparsity, const double* seq_k,
                               int32_t n, ssa_calib_result* out);

/* Calibration counts pooled over passes, one group per key length
 * (multi-sample accumulation: samples of one shape share a group;
 * multi-shape calibration: each resolution keeps its own group, see [README]
 * "Known Issues", resolution-dependent fit). The caller owns the arrays and
 * sets n_groups = 0 (and n_lambda = 0 or the pass's n) before the first add.
 * Every pass added must use the same threshold list. */
typedef struct ssa_calib_pool {
  int32_t n_lambda;    /* thresholds per pass; 0 = take the first pass's n          */
  int32_t max_groups;  /* capacity of the arrays below                               */
  int32_t n_groups;    /* groups in use, in order of first appearance                */
  int64_t* seq_k;      /* [max_groups] key length of each group                      */
  int64_t* skipped;    /* [max_groups * n_lambda] skipped tiles per threshold        */
  int64_t* visited;    /* [max_groups] visited tiles                                 */
} ssa_calib_pool;

/* Add one calibration pass (HOST copies of its counts [num_wg, n] and tiles
 * [num_wg]) to the pool: sequence b's work-groups go to the group of key
 * length S_b; empty sequences are ignored. Errors: SSA_ERR_INVALID_ARG (also
 * n != pool->n_lambda, or more key lengths than max_groups; the pool is then
 * unchanged). */
int ssa_calibration_pool_add(const ssa_problem* p, const int32_t* counts, const int32_t* tiles,
                             int32_t n, ssa_calib_pool* pool);

/* Fit points of the pool, group-major: point g * n_lambda + k is
 * (lambdas[k], skipped[g][k] / visited[g], seq_k[g]); writes
 * n_groups * n_lambda points to each output array. */
int ssa_calibration_pool_points(const ssa_calib_pool* pool, const double* lambdas, double* lambda_out,
                                double* sparsity_out, double* seq_k_out, int32_t* n_points);

/* ---- threshold resolution ---------------------------------------------- */
/* Resolve the user/checkpoint threshold sources into lambda and log2(lambda)
 * for a sequence of seq_k keys. Fields are read only when their flag is set
 * in `set`; the first available source wins, in this order:
 *   1. raw log2 threshold                 ([TRITON] "Method": raw first)
 *   2. fixed lambda                       ([README] "Threshold Modes")
 *   3. scale factor: lambda = sf / seq_k  ([TRTLLM] "Priority Order" 1)
 *   4. target sparsity with a formula: sf = a * exp(b * target) (a given as a
 *      or log_a), lambda = sf / seq_k    ([README] "Threshold Modes";
 *      [TRTLLM] "Priority Order" 2-3)
 *   5. static default lambda = 0.1       ([README] "Threshold Modes")
 * A target without (a or log_a) and b is SSA_ERR_NO_FORMULA ([TRTLLM] "Use
 * Cases" 1b; [DOCS] "User Configuration"). With SSA_SPEC_RANGE set, a target
 * outside [s_min, s_max] still resolves but returns SSA_WARN_EXTRAPOLATED
 * ([README] "Known Issues"). lambda outside [0, 1] or NaN is
 * SSA_ERR_THRESHOLD_RANGE; seq_k < 1 with sources 3-4 is SSA_ERR_INVALID_ARG.
 * lambda = 0 gives log2_lambda = -inf (dense). All pointers are host. */
#define SSA_SPEC_RAW_LOG2     (1u << 0)
#define SSA_SPEC_LAMBDA       (1u << 1)
#define SSA_SPEC_SCALE_FACTOR (1u << 2)
#define SSA_SPEC_TARGET       (1u << 3)
#define SSA_SPEC_A            (1u << 4)
#define SSA_SPEC_LOG_A        (1u << 5)
#define SSA_SPEC_B            (1u << 6)
#define SSA_SPEC_RANGE        (1u << 7)

typedef struct ssa_threshold_spec {
  uint32_t set; /* OR of SSA_SPEC_* flags */
  double raw_log2, lambda, scale_factor, target_sparsity;
  double a, log_a, b, s_min, s_max;
} ssa_threshold_spec;

int ssa_resolve_threshold(const ssa_threshold_spec* spec, int64_t seq_k, double* lambda,
                          double* log2_lambda);

/* ---- timestep and layer gating (host) ---------------------------------- */
/* Which attention forwards of a denoising run use skip-softmax, and with what
 * scale factor ([DOCS] "Checkpoint Config", "User Configuration", "Mapping
 * disabled_until_timestep to Actual Denoising Steps"; [TRTLLM] "Use Cases"
 * 1d). All pointers are host; no GPU work. Patterns are fnmatch(3) patterns
 * (case-sensitive, no backslash escapes: *, ?, [...], [!...]) matched against
 * the full module name and against its component-relative name (the name
 * without its first dotted component), so "blocks.0.attn1" matches
 * "transformer.blocks.0.attn1" and "transformer_2.blocks.0.attn1". */
#define SSA_GATE_BASE     0  /* base scale factor applies                      */
#define SSA_GATE_TIMESTEP 1  /* dense: forward timestep >= the cutoff           */
#define SSA_GATE_IGNORED  2  /* dense: layer matches an ignore pattern          */
#define SSA_GATE_OVERRIDE 3  /* first matching per-layer override (0 = dense)   */

typedef struct ssa_layer_override {
  const char* pattern;  /* fnmatch pattern                                 */
  double scale_factor;  /* threshold_scale_factor for matching layers; 0 = dense */
} ssa_layer_override;

typedef struct ssa_gate_spec {
  double disabled_until_timestep;      /* NaN = no cutoff; else in [0, 1]           */
  const char* const* ignore;           /* n_ignore patterns (NULL when n_ignore 0)  */
  int32_t n_ignore;
  const ssa_layer_override* overrides; /* n_overrides entries, first match wins     */
  int32_t n_overrides;
} ssa_gate_spec;

/* Effective threshold_scale_factor of layer `layer` for one forward whose
 * normalized timesteps are timesteps[0..n_timesteps) (per-token timesteps
 * reduce to their largest value). Rules in order: dense while that timestep
 * >= disabled_until_timestep (equality is dense); dense when an ignore pattern
 * matches; the first matching override; else base_scale_factor. Writes
 * *scale_factor (0 = dense) and *rule (SSA_GATE_*). The result feeds
 * ssa_attn_fwd with SSA_THRESH_SCALE_FACTOR (lambda = sf / S_b).
 * Errors: SSA_ERR_INVALID_ARG (NULL, n_timesteps < 1, NaN timestep, cutoff
 * outside [0, 1], negative or NaN scale factors). */
int ssa_gate_layer(const ssa_gate_spec* g, const char* layer, const double* timesteps,
                   int32_t n_timesteps, double base_scale_factor, double* scale_factor, int32_t* rule);

/* Normalized runtime timesteps of an n_steps flow-matching schedule with
 * num_train_timesteps T and flow shift f:
 * s[i] = 1 - i (1 - 1/T) / n_steps, shifted = f s / (1 + (f - 1) s),
 * t[i] = (1 - 1/T) shifted ([DOCS] "Mapping disabled_until_timestep to
 * Actual Denoising Steps", 40-step example with T = 1000, f = 3; the final
 * (1 - 1/T) factor is this library's reading of the unprinted conversion to
 * runtime timesteps, chosen because it reproduces the printed table).
 * Errors: SSA_ERR_INVALID_ARG (NULL, n_steps < 1, T < 1, f <= 0 or NaN). */
int ssa_flow_timesteps(int32_t n_steps, int32_t num_train_timesteps, double flow_shift, double* t);

/* dense_steps = count(t[i] >= cutoff) over t[0..n); cutoff NaN gives 0.
 * Errors: SSA_ERR_INVALID_ARG (NULL, n < 0, cutoff outside [0, 1]). */
int ssa_gate_dense_steps(const double* t, int32_t n, double cutoff, int32_t* dense_steps);

/* Human-readable text for a status code (static storage, never NULL). */
const char* ssa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H_ */
