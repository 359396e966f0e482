// Host side of the skip-softmax attention library: argument validation,
// threshold conversion, launch planning, calibration reduction, the
// log-space exponential fit and threshold resolution. All entry points are
// the C ABI declared in include/ssa.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "ssa.h"
#include "ssa_internal.h"

namespace {

constexpr int kMaxHeads = ssa::kMaxBHPerLaunch;  // one sequence's heads must fit one launch

constexpr int64_t kMaxHeadStride = (int64_t)1 << 47;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Checks shared by every entry point that takes a problem.
int validate_problem(const ssa_problem* p) {
  if (p == nullptr || p->cu_seqlens == nullptr) return SSA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->num_heads < 1 || p->head_dim < 1 || p->block < 1) return SSA_ERR_INVALID_ARG;
  if (p->num_heads > kMaxHeads) return SSA_ERR_UNSUPPORTED;
  if (!ssa::supported(p->head_dim, p->block)) return SSA_ERR_UNSUPPORTED;
  if (p->cu_seqlens[0] != 0) return SSA_ERR_INVALID_ARG;
  // A token step beyond 32 bits cannot be addressed by the kernels' buffer
  // offsets; a head step beyond 2^47 elements spans more than any device
  // address range. Bounding both first keeps the products below in range.
  if (p->stride_token > (int64_t)UINT32_MAX) return SSA_ERR_UNSUPPORTED;
  if (p->num_heads > 1 && (p->stride_head > kMaxHeadStride || p->stride_head < 0)) return SSA_ERR_INVALID_ARG;
  for (int b = 0; b < p->batch; ++b) {
    const int64_t s = (int64_t)p->cu_seqlens[b + 1] - p->cu_seqlens[b];
    if (s < 0) return SSA_ERR_INVALID_ARG;
    // work-groups of one sequence and tile-mask rows are indexed in int32
    if (ceil_div(s, p->block) * p->num_heads > INT32_MAX / 2) return SSA_ERR_UNSUPPORTED;
    // K/V tiles are fetched through 32-bit buffer offsets from the head's first row
    // (bf16 V in the block-scaled mode bounds both)
    const int64_t esize = p->dtype == SSA_DTYPE_FP8_E4M3 ? 1 : 2;
    if (s > 0 && ((s - 1) * p->stride_token + p->block * p->stride_token + p->head_dim) * esize > (int64_t)UINT32_MAX)
      return SSA_ERR_UNSUPPORTED;
  }
  // 16-byte aligned rows; distinct tokens (and heads, when H > 1) start at
  // least one row apart. Full non-overlap of the layout is the caller's duty.
  if (p->stride_token % 8 != 0 || p->stride_head % 8 != 0) return SSA_ERR_INVALID_ARG;
  if (p->stride_token < p->head_dim) return SSA_ERR_INVALID_ARG;
  if (p->num_heads > 1 && p->stride_head < p->head_dim) return SSA_ERR_INVALID_ARG;
  if (!(p->sm_scale >= 0.0) || !isfinite(p->sm_scale)) return SSA_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return SSA_ERR_INVALID_ARG;
  if (p->dtype != SSA_DTYPE_BF16 && p->dtype != SSA_DTYPE_FP8_E4M3 && p->dtype != SSA_DTYPE_MXFP8_QK)
    return SSA_ERR_INVALID_ARG;
  // 16-byte aligned e4m3 rows
  if (p->dtype != SSA_DTYPE_BF16 && (p->stride_token % 16 != 0 || p->stride_head % 16 != 0))
    return SSA_ERR_INVALID_ARG;
  if (p->dtype == SSA_DTYPE_FP8_E4M3) {
    // positive finite dequantization scales
    for (double sc : {p->scale_q, p->scale_k, p->scale_v})
      if (!(sc > 0.0) || !isfinite(sc)) return SSA_ERR_INVALID_ARG;
  }
  return SSA_OK;
}

// Block-scale arrays of the MXFP8 q/k mode (forward and calibration only):
// present, aligned to one row of scales (D / 32 bytes, read as one load),
// strides in whole rows, and every head's rows within a 32-bit buffer range.
int validate_block_scales(const ssa_problem* p) {
  if (p->dtype != SSA_DTYPE_MXFP8_QK) return SSA_OK;
  const int64_t row = p->head_dim / 32;
  if (p->block_scale_q == nullptr || p->block_scale_k == nullptr) return SSA_ERR_INVALID_ARG;
  if ((uintptr_t)p->block_scale_q % row != 0 || (uintptr_t)p->block_scale_k % row != 0) return SSA_ERR_INVALID_ARG;
  const int64_t st = p->block_scale_stride_token, sh = p->block_scale_stride_head;
  if (st < row || st % row != 0 || sh < 0 || sh % row != 0) return SSA_ERR_INVALID_ARG;
  if (sh > kMaxHeadStride) return SSA_ERR_INVALID_ARG;
  if (st > (int64_t)UINT32_MAX) return SSA_ERR_UNSUPPORTED;
  if (p->num_heads > 1 && sh < row) return SSA_ERR_INVALID_ARG;
  for (int b = 0; b < p->batch; ++b) {
    const int64_t s = (int64_t)p->cu_seqlens[b + 1] - p->cu_seqlens[b];
    // rows up to the end of the last tile are addressed (and read as zero past S)
    if (s > 0 && (s + p->block) * st > (int64_t)UINT32_MAX) return SSA_ERR_UNSUPPORTED;
  }
  return SSA_OK;
}

inline int seq_len(const ssa_problem* p, int b) { return p->cu_seqlens[b + 1] - p->cu_seqlens[b]; }

int validate_tensors(const void* q, const void* k, const void* v, const void* o) {
  if (!q || !k || !v || !o) return SSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SSA_ERR_INVALID_ARG;
  return SSA_OK;
}

double effective_scale(const ssa_problem* p) {
  return p->sm_scale > 0.0 ? p->sm_scale : 1.0 / sqrt((double)p->head_dim);
}

// lambda in [0, 1] -> log2(lambda) rounded to fp32; 0 -> -inf.
float lambda_to_t(double lam) { return lam == 0.0 ? -INFINITY : (float)log2(lam); }

// The kernel-facing log2 threshold of head h of a sequence with S keys.
int threshold_for(const ssa_thresholds* th, int h, int S, float* t) {
  const double v = th->values[th->count == 1 ? 0 : h];
  switch (th->kind) {
    case SSA_THRESH_LAMBDA:
      if (!(v >= 0.0 && v <= 1.0)) return SSA_ERR_THRESHOLD_RANGE;
      *t = lambda_to_t(v);
      return SSA_OK;
    case SSA_THRESH_LOG2:
      if (isnan(v) || v > 0.0) return SSA_ERR_THRESHOLD_RANGE;
      *t = (float)v;
      return SSA_OK;
    case SSA_THRESH_SCALE_FACTOR: {
      if (!(v >= 0.0) || isinf(v)) return SSA_ERR_THRESHOLD_RANGE;
      if (S == 0) { *t = -INFINITY; return SSA_OK; }  // no tiles at all
      const double lam = v / (double)S;
      if (lam > 1.0) return SSA_ERR_THRESHOLD_RANGE;
      *t = lambda_to_t(lam);
      return SSA_OK;
    }
    default:
      return SSA_ERR_INVALID_ARG;
  }
}

struct Plan {
  std::vector<ssa::LaunchParams> launches;
};

// Split the batch into launches: at most kMaxSeqPerLaunch sequences and
// kMaxBHPerLaunch (sequence, head) thresholds each, and an int32 grid.
// `ts` is [B * H] log2 thresholds (forward) or empty (calibration).
void plan_launches(const ssa_problem* p, const ssa::LaunchParams& tmpl, const std::vector<float>& ts,
                   Plan* plan) {
  const int B = p->batch, H = p->num_heads;
  int64_t wg_abs = 0;
  int b0 = 0;
  while (b0 < B) {
    ssa::LaunchParams lp = tmpl;
    int n = 0;
    int64_t wg = 0;
    lp.tok_start[0] = p->cu_seqlens[b0];
    lp.wg_start[0] = 0;
    while (b0 + n < B && n < ssa::kMaxSeqPerLaunch && (n + 1) * H <= ssa::kMaxBHPerLaunch) {
      const int64_t w = ceil_div(seq_len(p, b0 + n), p->block) * H;
      if (n > 0 && wg + w > INT32_MAX / 2) break;
      for (int h = 0; h < H && !ts.empty(); ++h) lp.t_bh[n * H + h] = ts[(size_t)(b0 + n) * H + h];
      wg += w;
      ++n;
      lp.tok_start[n] = p->cu_seqlens[b0 + n];
      lp.wg_start[n] = (int32_t)wg;
    }
    lp.nseq = n;
    lp.total_wg = (int32_t)wg;
    // XCD order (map_workgroup): chunked when eight heads' K/V exceed half the
    // Infinity Cache or when there are too few heads to balance over 8 XCDs
    int64_t max_s = 0;
    for (int i = 0; i < n; ++i) max_s = std::max<int64_t>(max_s, seq_len(p, b0 + i));
    const int64_t kv_head = max_s * p->head_dim * ((tmpl.fp8 || tmpl.mxqk ? 1 : 2) + (tmpl.fp8 ? 1 : 2));
    lp.xcd_chunked = (n * H < ssa::kXcdChunkMinHeads || 8 * kv_head > ssa::kXcdChunkKvBytes) ? 1 : 0;
    lp.seq_abs0 = b0;
    lp.wg_abs0 = wg_abs;
    plan->launches.push_back(lp);
    wg_abs += wg;
    b0 += n;
  }
}

ssa::LaunchParams base_params(const ssa_problem* p, const void* q, const void* k, const void* v, void* o) {
  ssa::LaunchParams lp;
  memset(&lp, 0, sizeof(lp));
  lp.q = (const uint16_t*)q;
  lp.k = (const uint16_t*)k;
  lp.v = (const uint16_t*)v;
  lp.o = (uint16_t*)o;
  lp.stride_tok = p->stride_token;
  lp.stride_head = p->stride_head;
  const bool fp8 = p->dtype == SSA_DTYPE_FP8_E4M3;
  // * log2(e); e4m3 scores also carry the q and k dequantization scales
  lp.scale_log2 = (float)(effective_scale(p) * 1.4426950408889634 * (fp8 ? p->scale_q * p->scale_k : 1.0));
  lp.num_heads = p->num_heads;
  lp.causal = p->causal;
  lp.fp8 = fp8 ? 1 : 0;
  lp.v_scale = fp8 ? (float)p->scale_v : 1.0f;
  if (p->dtype == SSA_DTYPE_MXFP8_QK) {  // the block scales are applied inside the MFMA
    lp.mxqk = 1;
    lp.q_bscale = p->block_scale_q;
    lp.k_bscale = p->block_scale_k;
    lp.bs_tok = p->block_scale_stride_token;
    lp.bs_head = p->block_scale_stride_head;
  }
  return lp;
}

int hip_status(int e) { return e == 0 ? SSA_OK : SSA_ERR_HIP; }

}  // namespace

extern "C" {

const char* ssa_status_string(int status) {
  switch (status) {
    case SSA_OK: return "ok";
    case SSA_WARN_EXTRAPOLATED: return "warning: target sparsity outside the calibrated range (extrapolated)";
    case SSA_ERR_INVALID_ARG: return "invalid argument";
    case SSA_ERR_UNSUPPORTED: return "unsupported configuration (head_dim/block not built or too many heads)";
    case SSA_ERR_THRESHOLD_RANGE: return "threshold out of range: lambda must lie in [0, 1]";
    case SSA_ERR_NO_FORMULA: return "target sparsity given without a calibration formula";
    case SSA_ERR_FIT_DEGENERATE: return "degenerate fit: fewer than two distinct usable sparsities";
    case SSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int ssa_tile_mask_dims(const ssa_problem* p, int64_t* nq_max, int64_t* nk_max) {
  const int st = validate_problem(p);
  if (st != SSA_OK) return st;
  if (nq_max == nullptr || nk_max == nullptr) return SSA_ERR_INVALID_ARG;
  int64_t n = 0;
  for (int b = 0; b < p->batch; ++b) {
    const int64_t t = ceil_div(seq_len(p, b), p->block);
    if (t > n) n = t;
  }
  *nq_max = n;
  *nk_max = n;
  return SSA_OK;
}

int ssa_calib_num_workgroups(const ssa_problem* p, int64_t* num_wg) {
  const int st = validate_problem(p);
  if (st != SSA_OK) return st;
  if (num_wg == nullptr) return SSA_ERR_INVALID_ARG;
  int64_t n = 0;
  for (int b = 0; b < p->batch; ++b) n += ceil_div(seq_len(p, b), p->block) * p->num_heads;
  *num_wg = n;
  return SSA_OK;
}

int ssa_attn_fwd(const ssa_problem* p, const void* q, const void* k, const void* v, void* o,
                 const ssa_thresholds* th, uint64_t* skipped_bh, uint64_t* total_bh, uint8_t* tile_mask,
                 ssa_stream_t stream) {
  int st = validate_problem(p);
  if (st != SSA_OK) return st;
  st = validate_tensors(q, k, v, o);
  if (st != SSA_OK) return st;
  st = validate_block_scales(p);
  if (st != SSA_OK) return st;
  if (th == nullptr || th->values == nullptr) return SSA_ERR_INVALID_ARG;
  if (th->count != 1 && th->count != p->num_heads) return SSA_ERR_INVALID_ARG;
  const int B = p->batch, H = p->num_heads;
  std::vector<float> ts((size_t)B * H);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      st = threshold_for(th, h, seq_len(p, b), &ts[(size_t)b * H + h]);
      if (st != SSA_OK) return st;
    }
  int64_t nq = 0, nk = 0;
  ssa_tile_mask_dims(p, &nq, &nk);
  int64_t mask_bytes = 0;
  if (tile_mask && (__builtin_mul_overflow((int64_t)B * H, nq, &mask_bytes) ||
                    __builtin_mul_overflow(mask_bytes, nk, &mask_bytes)))
    return SSA_ERR_UNSUPPORTED;

  ssa::LaunchParams tmpl = base_params(p, q, k, v, o);
  tmpl.skipped_bh = skipped_bh;
  tmpl.total_bh = total_bh;
  tmpl.tile_mask = tile_mask;
  tmpl.mask_nq = nq;
  tmpl.mask_nk = nk;
  Plan plan;
  plan_launches(p, tmpl, ts, &plan);

  if (skipped_bh) { st = hip_status(ssa::launch_fill_u64(skipped_bh, (int64_t)B * H, stream)); if (st) return st; }
  if (total_bh) { st = hip_status(ssa::launch_fill_u64(total_bh, (int64_t)B * H, stream)); if (st) return st; }
  if (tile_mask) {
    st = hip_status(ssa::launch_fill_u8(tile_mask, mask_bytes, 2, stream));
    if (st) return st;
  }
  for (const auto& lp : plan.launches) {
    st = hip_status(ssa::launch_forward(p->head_dim, p->block, false, lp, stream));
    if (st) return st;
  }
  return SSA_OK;
}

int ssa_attn_calibrate(const ssa_problem* p, const void* q, const void* k, const void* v, void* o,
                       const double* lambdas, int32_t n, int32_t* counts, int32_t* tiles,
                       ssa_stream_t stream) {
  int st = validate_problem(p);
  if (st != SSA_OK) return st;
  st = validate_tensors(q, k, v, o);
  if (st != SSA_OK) return st;
  st = validate_block_scales(p);
  if (st != SSA_OK) return st;
  if (lambdas == nullptr || counts == nullptr || tiles == nullptr) return SSA_ERR_INVALID_ARG;
  if (n < 1 || n > ssa::kMaxCalib) return SSA_ERR_INVALID_ARG;
  ssa::LaunchParams tmpl = base_params(p, q, k, v, o);
  for (int i = 0; i < n; ++i) {
    if (!(lambdas[i] > 0.0 && lambdas[i] <= 1.0)) return SSA_ERR_THRESHOLD_RANGE;
    if (i > 0 && lambdas[i] < lambdas[i - 1]) return SSA_ERR_INVALID_ARG;
    tmpl.cal_t[i] = lambda_to_t(lambdas[i]);
  }
  tmpl.ncal = n;
  tmpl.counts = counts;
  tmpl.tiles = tiles;
  Plan plan;
  plan_launches(p, tmpl, std::vector<float>(), &plan);
  for (const auto& lp : plan.launches) {
    st = hip_status(ssa::launch_forward(p->head_dim, p->block, true, lp, stream));
    if (st) return st;
  }
  return SSA_OK;
}

int ssa_calibration_sparsity(const ssa_problem* p, const int32_t* counts, const int32_t* tiles, int32_t n,
                             double* sparsity) {
  const int st = validate_problem(p);
  if (st != SSA_OK) return st;
  if (counts == nullptr || tiles == nullptr || sparsity == nullptr || n < 1 || n > ssa::kMaxCalib)
    return SSA_ERR_INVALID_ARG;
  int64_t w = 0;
  for (int b = 0; b < p->batch; ++b) {
    const int64_t nwg = ceil_div(seq_len(p, b), p->block) * p->num_heads;
    int64_t tot = 0;
    std::vector<int64_t> sum(n, 0);
    for (int64_t i = 0; i < nwg; ++i, ++w) {
      tot += tiles[w];
      for (int k = 0; k < n; ++k) sum[k] += counts[w * n + k];
    }
    for (int k = 0; k < n; ++k) sparsity[(int64_t)b * n + k] = tot > 0 ? (double)sum[k] / (double)tot : NAN;
  }
  return SSA_OK;
}

int ssa_calibration_fit(const double* lambda, const double* sparsity, const double* seq_k, int32_t n,
                        ssa_calib_result* out) {
  if (lambda == nullptr || sparsity == nullptr || seq_k == nullptr || out == nullptr || n < 0)
    return SSA_ERR_INVALID_ARG;
  // usable points: 0 < s < 1 (plateaus carry no slope), lambda > 0, seq_k > 0
  std::vector<double> xs, ys;
  for (int i = 0; i < n; ++i) {
    const double s = sparsity[i], lam = lambda[i], sk = seq_k[i];
    if (!isfinite(s) || !isfinite(lam) || !isfinite(sk)) return SSA_ERR_INVALID_ARG;
    if (!(s > 0.0 && s < 1.0) || !(lam > 0.0) || !(sk > 0.0)) continue;
    xs.push_back(s);
    ys.push_back(log(lam * sk));  // ln(scale_factor)
  }
  const size_t m = xs.size();
  if (m < 2) return SSA_ERR_FIT_DEGENERATE;
  double xm = 0.0, ym = 0.0, lo = xs[0], hi = xs[0];
  for (size_t i = 0; i < m; ++i) {
    xm += xs[i];
    ym += ys[i];
    lo = xs[i] < lo ? xs[i] : lo;
    hi = xs[i] > hi ? xs[i] : hi;
  }
  if (!(hi > lo)) return SSA_ERR_FIT_DEGENERATE;
  xm /= (double)m;
  ym /= (double)m;
  double sxx = 0.0, sxy = 0.0;
  for (size_t i = 0; i < m; ++i) {
    sxx += (xs[i] - xm) * (xs[i] - xm);
    sxy += (xs[i] - xm) * (ys[i] - ym);
  }
  const double b = sxy / sxx;
  const double log_a = ym - b * xm;
  out->a = exp(log_a);
  out->log_a = log_a;
  out->b = b;
  out->s_min = lo;
  out->s_max = hi;
  out->n_used = (int32_t)m;
  return SSA_OK;
}

int ssa_resolve_threshold(const ssa_threshold_spec* spec, int64_t seq_k, double* lambda, double* log2_lambda) {
  if (spec == nullptr || lambda == nullptr || log2_lambda == nullptr) return SSA_ERR_INVALID_ARG;
  const uint32_t set = spec->set;
  double lam;
  int status = SSA_OK;
  if (set & SSA_SPEC_RAW_LOG2) {
    const double r = spec->raw_log2;
    if (isnan(r) || r > 0.0) return SSA_ERR_THRESHOLD_RANGE;
    *lambda = exp2(r);
    *log2_lambda = r;
    return SSA_OK;
  } else if (set & SSA_SPEC_LAMBDA) {
    lam = spec->lambda;
  } else if (set & SSA_SPEC_SCALE_FACTOR) {
    if (seq_k < 1) return SSA_ERR_INVALID_ARG;
    lam = spec->scale_factor / (double)seq_k;
  } else if (set & SSA_SPEC_TARGET) {
    const double tgt = spec->target_sparsity;
    if (isnan(tgt) || seq_k < 1) return SSA_ERR_INVALID_ARG;
    if (!(set & SSA_SPEC_B) || !(set & (SSA_SPEC_A | SSA_SPEC_LOG_A))) return SSA_ERR_NO_FORMULA;
    double log_a;
    if (set & SSA_SPEC_LOG_A) {
      log_a = spec->log_a;
    } else {
      if (!(spec->a > 0.0)) return SSA_ERR_INVALID_ARG;
      log_a = log(spec->a);
    }
    lam = exp(log_a + spec->b * tgt) / (double)seq_k;
    if ((set & SSA_SPEC_RANGE) && !(tgt >= spec->s_min && tgt <= spec->s_max)) status = SSA_WARN_EXTRAPOLATED;
  } else {
    lam = 0.1;  // static default
  }
  if (isnan(lam) || lam < 0.0 || lam > 1.0) return SSA_ERR_THRESHOLD_RANGE;
  *lambda = lam;
  *log2_lambda = lam == 0.0 ? -INFINITY : log2(lam);
  return status;
}

}  // extern "C"
