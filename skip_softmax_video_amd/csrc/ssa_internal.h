// Internal interface between the host library (ssa_host.cpp) and the HIP
// kernels (ssa_kernel.hip). Not part of the public C ABI.
#pragma once

#include <stdint.h>

namespace ssa {

// Limits of one kernel launch; the host splits larger batches into several
// launches on the same stream.
constexpr int kMaxSeqPerLaunch = 32;   // sequences per launch
constexpr int kMaxBHPerLaunch = 512;   // (sequence, head) thresholds per launch
constexpr int kMaxCalib = 64;          // thresholds of one calibration pass

// Everything a launch needs, passed by value as the kernel argument
// (about 2.8 KB, below the 4 KB kernel-argument limit).
struct LaunchParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t stride_tok;  // elements
  int64_t stride_head; // elements
  float scale_log2;    // sm_scale * log2(e)
  int32_t num_heads;
  int32_t causal;                            // 1: Q-block i visits KV tiles 0..i, keys after the query masked
  int32_t fp8;                               // 1: q, k, v are e4m3 bytes (o stays bf16)
  float v_scale;                             // fp8: dequantization scale of v (1 for bf16)
  int32_t mxqk;                              // 1: q, k are e4m3 bytes with E8M0 block scales (v bf16)
  const uint8_t* q_bscale;                   // mxqk: [T, H, D / 32] scales of q and k
  const uint8_t* k_bscale;
  int64_t bs_tok, bs_head;                   // mxqk: byte strides of the scale arrays
  int32_t nseq;                              // sequences in this launch
  int32_t total_wg;                          // work-groups in this launch
  int32_t seq_abs0;                          // batch index of the first sequence
  int32_t tok_start[kMaxSeqPerLaunch + 1];   // token offset of each sequence (+ end)
  int32_t wg_start[kMaxSeqPerLaunch + 1];    // first work-group of each sequence (+ end)
  // forward outputs (optional)
  uint64_t* skipped_bh;  // [B*H] indexed by absolute batch index
  uint64_t* total_bh;
  uint8_t* tile_mask;    // [B, H, mask_nq, mask_nk]
  int64_t mask_nq, mask_nk;
  // calibration outputs
  int32_t* counts;       // [num_wg_total, ncal]
  int32_t* tiles;        // [num_wg_total]
  int64_t wg_abs0;       // absolute work-group index of this launch's first work-group
  int32_t ncal;
  float cal_t[kMaxCalib];          // log2 thresholds of the calibration pass
  float t_bh[kMaxBHPerLaunch];     // log2 threshold per (local sequence, head)
};
static_assert(sizeof(LaunchParams) <= 4096, "the launch parameters travel as one kernel argument (4 KB limit)");

// Kernel launchers (ssa_kernel.hip). Return a hipError_t as int.
int launch_forward(int head_dim, int block, bool calibrate, const LaunchParams& p, void* stream);
int launch_fill_u8(uint8_t* dst, int64_t n, uint8_t value, void* stream);
int launch_fill_u64(uint64_t* dst, int64_t n, void* stream);
bool supported(int head_dim, int block);

}  // namespace ssa
