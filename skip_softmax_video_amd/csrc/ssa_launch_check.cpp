// Host-only stand-in for the kernel launchers of ssa_kernel.hip, linked into
// the sanitizer build of the host library (g++ -fsanitize=address,undefined;
// it is never part of libssa.so). Instead of launching, each launcher walks
// every work-group of the planned launch through the kernels' own mapping
// (map_workgroup in ssa_internal.h) and records the largest element index the
// kernels would touch in each caller buffer, so that a CPU test can compare
// the host's launch plan with the buffer sizes the caller was asked for:
//   [0] launches, [1] work-groups, [2] largest skipped_bh/total_bh index,
//   [3] largest tile_mask index, [4] largest counts index, [5] largest tiles
//   index, [6] one past the last token row read or written, [7] largest
//   u64 fill, [8] largest u8 fill, [9] work-groups mapped twice or not at all.
// Indices are -1 when nothing was touched.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "ssa_internal.h"

namespace {

constexpr int kStats = 10;
int64_t g_stats[kStats];
bool g_init = false;

void reset() {
  for (int i = 0; i < kStats; ++i) g_stats[i] = -1;
  g_stats[0] = 0;
  g_stats[1] = 0;
  g_stats[9] = 0;
  g_init = true;
}

void upd(int i, int64_t v) {
  if (!g_init) reset();
  if (v > g_stats[i]) g_stats[i] = v;
}

}  // namespace

namespace ssa {

int launch_forward(int head_dim, int block, bool calibrate, const LaunchParams& p, void* stream) {
  (void)head_dim;
  (void)stream;
  if (!g_init) reset();
  if (p.total_wg <= 0) return 0;
  g_stats[0] += 1;
  g_stats[1] += p.total_wg;
  std::vector<int> seen((size_t)p.total_wg, 0);
  const int H = p.num_heads;
  for (int bid = 0; bid < p.total_wg; ++bid) {
    const WorkItem w = map_workgroup(p, bid, block);
    if (w.row < 0 || w.row >= p.total_wg) {
      g_stats[9] += 1;
      continue;
    }
    seen[(size_t)w.row] += 1;
    upd(6, (int64_t)w.tok0 + w.S);  // q/o rows of the block and K/V rows of the head stay below this
    if (calibrate) {
      upd(4, (p.wg_abs0 + w.row) * (int64_t)p.ncal + p.ncal - 1);
      upd(5, p.wg_abs0 + w.row);
    } else {
      const int64_t bh = (int64_t)(p.seq_abs0 + w.b) * H + w.h;
      if (p.skipped_bh != nullptr || p.total_bh != nullptr) upd(2, bh);
      if (p.tile_mask != nullptr) upd(3, (bh * p.mask_nq + w.qb) * p.mask_nk + w.nk - 1);
    }
  }
  for (int r = 0; r < p.total_wg; ++r)
    if (seen[(size_t)r] != 1) g_stats[9] += 1;
  return 0;
}

int launch_fill_u8(uint8_t* dst, int64_t n, uint8_t value, void* stream) {
  (void)dst;
  (void)value;
  (void)stream;
  upd(8, n);
  return 0;
}

int launch_fill_u64(uint64_t* dst, int64_t n, void* stream) {
  (void)dst;
  (void)stream;
  upd(7, n);
  return 0;
}

}  // namespace ssa

extern "C" int ssa_check_extents(int64_t* out, int n) {
  if (!g_init) reset();
  if (out == nullptr || n < kStats) return -1;
  memcpy(out, g_stats, sizeof(g_stats));
  reset();
  return kStats;
}
