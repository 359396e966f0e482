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
  int32_t xcd_chunked;                       // work-group order across XCDs (map_workgroup)
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

#ifdef __HIPCC__
#define SSA_HOST_DEVICE __host__ __device__
#else
#define SSA_HOST_DEVICE
#endif

// What one work-group computes: Q-block `qb` of head `h` of local sequence
// `b`, whose S tokens start at token `tok0`, visiting `nk` KV tiles; `row`
// is its row in the per-launch work-group numbering of the count tables.
struct WorkItem {
  int b, h, qb, nk, tok0, S, row;
};

// Work-group `bid` of a launch -> its work item. The hardware deals
// work-group i to XCD i % 8, and the work-groups resident on one XCD should
// be consecutive Q-blocks of one head, which stream the same K/V tiles
// through that XCD's L2. Two orders do that:
//  * contiguous: XCD x takes the logical ids [x * (G / 8) + min(x, G % 8),
//    ...), so each XCD walks its own heads and the eight XCDs have eight
//    heads' K/V in flight;
//  * chunked (xcd_chunked): logical ids are cut into chunks of kXcdChunk and
//    the chunks dealt round-robin, XCD x taking chunks x, x + 8, ...; the
//    eight XCDs then work on neighbouring chunks of the same head, whose K/V
//    the Infinity Cache serves to all of them, and every XCD gets a share of
//    every head. Work-groups past the last whole round of 8 chunks keep their
//    own id.
// The host picks chunked when eight heads' K/V would not fit in half the
// Infinity Cache, or when the launch has too few (sequence, head) pairs to
// balance whole heads over the XCDs; the contiguous order keeps the better
// L2 hit rate otherwise. Logical ids run sequence-major, then head, then
// Q-block; in the causal form the longest Q-blocks (most KV tiles) of each
// head come first.
constexpr int kXcdChunk = 32;
constexpr int64_t kXcdChunkKvBytes = 128ll << 20;  // chunked above this much K/V for 8 heads
constexpr int kXcdChunkMinHeads = 16;              // chunked below this many (sequence, head) pairs
SSA_HOST_DEVICE inline WorkItem map_workgroup(const LaunchParams& p, int bid, int block) {
  const int G = p.total_wg;
  const int k = bid >> 3, xcd = bid & 7;  // the XCD and this work-group's position in its stream
  int L;
  if (p.xcd_chunked) {
    const int whole = G / (8 * kXcdChunk) * (8 * kXcdChunk);
    L = bid < whole ? ((k / kXcdChunk) * 8 + xcd) * kXcdChunk + k % kXcdChunk : bid;
  } else {
    L = xcd * (G >> 3) + (xcd < (G & 7) ? xcd : (G & 7)) + k;
  }
  WorkItem w;
  w.b = 0;
  while (w.b + 1 < p.nseq && p.wg_start[w.b + 1] <= L) ++w.b;
  w.tok0 = p.tok_start[w.b];
  w.S = p.tok_start[w.b + 1] - w.tok0;
  const int nQ = (w.S + block - 1) / block;
  const int rem = L - p.wg_start[w.b];
  w.h = rem / nQ;
  w.qb = p.causal ? nQ - 1 - (rem - w.h * nQ) : rem - w.h * nQ;
  w.nk = p.causal ? w.qb + 1 : nQ;
  w.row = p.wg_start[w.b] + w.h * nQ + w.qb;
  return w;
}

// Kernel launchers (ssa_kernel.hip). Return a hipError_t as int.
int launch_forward(int head_dim, int block, bool calibrate, const LaunchParams& p, void* stream);
int launch_fill_u8(uint8_t* dst, int64_t n, uint8_t value, void* stream);
int launch_fill_u64(uint64_t* dst, int64_t n, void* stream);

// The (head_dim, block) pairs the kernels are built for.
inline bool supported(int head_dim, int block) {
  return (head_dim == 64 || head_dim == 128) && (block == 64 || block == 128);
}

}  // namespace ssa
