// Skip-softmax (BLASST) FlashAttention forward and calibration kernels for
// MI355X (gfx950, CDNA4).
//
// Method: ModelOpt pull request "skip-softmax ... via dedicated Triton
// kernels", section "Changes / Triton kernels" -- inside the FlashAttention
// loop, when a KV tile's largest score sits well under the running softmax
// maximum the loop moves on without fetching V, exponentiating or adding to
// the output; a calibration variant runs the full attention and counts, for
// N thresholds in the same pass, the tiles each would have left out. ModelOpt README "Skip-Softmax Sparse
// Attention for Diffusion Models", section "Threshold Modes": the comparison
// is in log2 units against log2(lambda).
//
// Work decomposition (one work-group = one Br-row Q-block of one head):
//   * Br = Bc = BLK query rows / keys per tile; BLK/32 waves, each owning 32
//     query rows. D = head dim. Two work-groups share a CU (<= 256 VGPRs +
//     AGPRs per wave, 64 KB of LDS per work-group), so each SIMD runs two
//     waves that hide each other's LDS, barrier and memory latency.
//   * Scores are computed transposed, S^T = K_j Q^T, so that each lane holds
//     whole query rows' worth of keys and the per-row max and sum are
//     in-register reductions plus cross-lane swaps. bf16 uses
//     v_mfma_f32_16x16x32_bf16 (lane l holds queries l % 16 and 16 + l % 16,
//     4 keys of every 16-key block; partners in lanes l ^ 16, ^ 32, ^ 48),
//     which does the work of the 32x32x16 shape for less energy per FLOP.
//     The e4m3 and block-scaled modes use the 32x32x64 scaled MFMA (lane l
//     holds query l % 32, 16 keys per 32-key block; partner lane l ^ 32).
//   * The same registers, rounded to the P.V operand type, are the B
//     operand of O^T += V_j^T P^T; V_j^T is read from the row-major V tile
//     in LDS with transposing reads (ds_read_b64_tr_b16 / _b8). The per-lane
//     key order inside a P.V step is permuted identically on both operands.
//   * O^T accumulates in registers with each lane owning the same query rows
//     as in the scores, so the rescale factors and row sums are per-lane
//     values. The accumulator is rescaled lazily: the exponent base only
//     moves when some row's maximum rose by more than 2^8, which keeps
//     P <= 256 and the result unchanged up to rounding.
//   * K and V tiles go global -> LDS with buffer_load_dwordx4 ... lds (no
//     register staging). Each wave instruction fills 1 KB of LDS; the
//     16-byte granules of a row are XOR-swizzled so that the MFMA operand
//     reads (ds_read_b128 for K, ds_read_b64_tr_b16 for V) avoid bank
//     conflicts. Rows past the end of a sequence fall outside the buffer
//     descriptor's range and read as zero: their scores are masked to -inf
//     and their P is 0.
//   * Skip vote: every lane forms x = rowmax * sm_scale * log2(e) - m for its
//     queries (m = running max before the tile; -inf on the first tile, so
//     x = +inf and the first tile is always kept). A wave keeps the tile if
//     any valid row has x >= t (one ballot); the work-group ORs the waves'
//     flags through LDS, so d = max_r x_r < t exactly when nobody keeps.
//     The calibration instantiation never skips: each wave reduces x to its
//     maximum (DPP), the work-group takes d = the maximum over waves, and
//     lane k (holding threshold k) counts d < t_k; one row of counts per
//     work-group is written at the end (no atomics).
//   * V_j is fetched only when the vote kept the tile, issued right after
//     the vote so that it lands while the softmax runs; K_{j+1} is fetched
//     into a second K buffer during S^T = K_j Q^T where LDS allows, else as
//     soon as every wave is done reading K_j (see the tile loop).
//   * Work-groups are remapped so that the ones resident on an XCD (8 per
//     MI355X, 4 MB L2 each) are consecutive Q-blocks of one head and stream
//     the same K/V tiles through that XCD's L2 (map_workgroup: each XCD its
//     own range of heads, or, when eight heads' K/V would overflow the
//     Infinity Cache, runs of 32 Q-blocks dealt round-robin so that the
//     eight XCDs share one head's K/V there).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) void lds_void;

// Exponent-base slack of the lazy rescale (log2 units): P <= 2^8.
constexpr float kRescaleSlack = 8.0f;
// Buffer descriptor word 3 for raw (untyped) dword access on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;

template <int D, int BLK>
struct Shape {
  static constexpr int NW = BLK / 32;     // waves per work-group (32 query rows each)
  static constexpr int NT = NW * 64;      // threads per work-group
  static constexpr int KB = BLK / 32;     // 32-key blocks per KV tile
  static constexpr int DS = D / 16;       // 16-wide d steps of S^T = K Q^T
  static constexpr int MB = D / 32;       // 32-wide d blocks of O^T
  static constexpr int KS = BLK / 16;     // 16-key steps of O^T += V^T P^T
  static constexpr int CH = D / 8;        // 16-byte granules per row
  static constexpr int GRAN = BLK * CH;   // granules per tile
  static constexpr int DMA = GRAN / NT;   // direct loads per thread per tile
  static_assert(GRAN % NT == 0, "tile must split evenly over the threads");
  static_assert(CH == 8 || CH == 16, "head_dim 64 or 128");
};

// XOR swizzle of the 16-byte granules of a K row: the 32 rows read by one
// ds_read_b128 (same granule column) land on distinct bank groups.
template <int CH>
__device__ __forceinline__ int swz_k(int row) { return row & (CH - 1); }

// XOR swizzle of a V row: one ds_read_b64_tr_b16 reads 4 consecutive rows x
// 2 granules per 16 lanes (4 granules per 32 lanes); these land on distinct
// bank groups for 32- and 64-bank LDS alike.
template <int CH>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (CH == 16) {
    return (0xCA60 >> (4 * (row & 3))) & 15;  // rows 0..3 -> 0, 6, 10, 12
  } else {
    return 2 * (row & 3);
  }
}

// XOR swizzle of a V row read by the 16x16 layout's transposing reads: 8
// consecutive rows x 2 granules per 32 lanes (4 rows per 16 lanes) land on
// distinct bank groups for 32- and 64-bank LDS (head_dim 128; head_dim 64
// rows are 128 bytes, where 4 consecutive rows are kept apart).
template <int CH>
__device__ __forceinline__ int swz_v16(int row) {
  if constexpr (CH == 16) {
    return 2 * (row & 7);
  } else {
    return 2 * (row & 3);
  }
}

// Which swizzle a tile copy applies.
enum class Swz { K, V, V16 };

// global -> LDS copy of one BLK x D tile with buffer_load_dwordx4 ... lds.
// The buffer descriptor covers exactly the head's valid rows (base = the
// head's first row, `bytes` = extent of rows [0, S)), so rows past the end of
// the sequence read as zero (hardware range check, no branch).
// Wave w's instruction i fills granules [g0, g0 + 64) of the LDS tile, g0 =
// (i * NW + w) * 64; lane l fills granule g0 + l, i.e. row (g0 + l) / CH at
// swizzled position (g0 + l) % CH, and so loads logical granule
// position ^ swz(row) of that row. An instruction covers RPI = 64 / CH rows;
// the row offset goes in the scalar soffset, the lane's position within the
// instruction in a per-lane voffset that does not change between tiles.
template <int D>
__device__ __forceinline__ uint32_t head_extent(int rows, int64_t stride_tok) {
  return rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * stride_tok + D) * 2) : 0u;
}

// With di > 1 only instructions i0, i0 + di, ... are issued, so a tile fetch
// can be spread over the steps of a product.
template <int D, int BLK, Swz SW>
__device__ __forceinline__ void dma_load(const uint16_t* head, uint32_t bytes, uint16_t* lds, int row0,
                                         int64_t stride_tok, int wave, int lane, int i0 = 0, int di = 1) {
  using SH = Shape<D, BLK>;
  constexpr int RPI = 64 / SH::CH;
  // rows repeat their swizzle with this period
  constexpr int PERIOD = SW == Swz::K ? SH::CH : SW == Swz::V ? 4 : (SH::CH == 16 ? 8 : 4);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)head, 0, bytes, kBufferFlags);
  const int lrow = lane / SH::CH;
  auto lane_off = [&](int row) {
    const int sw = SW == Swz::K ? swz_k<SH::CH>(row) : SW == Swz::V ? swz_v<SH::CH>(row) : swz_v16<SH::CH>(row);
    const int chunk = (lane % SH::CH) ^ sw;
    return (uint32_t)(((int64_t)lrow * stride_tok + chunk * 8) * 2);
  };
  // When consecutive instructions advance by whole swizzle periods (the usual
  // case) every instruction has the same per-lane offset: compute it once.
  const uint32_t voff0 = lane_off(RPI * wave + lrow);
#pragma unroll
  for (int i = i0; i < SH::DMA; i += di) {
    const int rin = RPI * (i * SH::NW + wave);  // first row of this instruction within the tile
    const uint32_t voff = (RPI * SH::NW) % PERIOD == 0 ? voff0 : lane_off(rin + lrow);
    const uint32_t soff = (uint32_t)((int64_t)(row0 + rin) * stride_tok * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + (i * SH::NW + wave) * 512), 16, voff, soff, 0,
                                             0);
  }
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value and its partner in lane l ^ 32
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// the same with the partner in lane l ^ 16
__device__ __forceinline__ float xrow_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xrow_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A operand of the 16x16x32 S^T = K Q^T for 16-key block kb, 32-wide d
// step s: K[16 kb + l16][32 s + 8 lq .. + 7] (l16 = l % 16, lq = l / 16).
// The K swizzle of row 16 kb + l16 is l16 (it repeats every 16 rows), so
// k16_off(s) serves every key block: block kb adds 16 rows (an immediate).
template <class SH>
__device__ __forceinline__ uint32_t k16_off(int s, int lane) {
  const int l16 = lane & 15, lq = lane >> 4;
  return (uint32_t)((l16 * SH::CH + ((4 * s + lq) ^ swz_k<SH::CH>(l16))) * 16);
}
template <class SH>
__device__ __forceinline__ bf16x8 read_k16(const uint8_t* k_lds, int kb, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(k_lds + off + kb * 16 * SH::CH * 16);
}

// A operand of the 16x16x32 O^T += V^T P^T for 32-key step ks, 16-wide d
// block mb: lane l gets column d = 16 mb + l16 at keys 32 ks + 4 lq + (0..3)
// (slots 0-3) and 32 ks + 16 + 4 lq + (0..3) (slots 4-7), the key order of
// P's slots. Each transposing read covers 4 rows x 16 columns per 16 lanes:
// source lane i names row i / 4 and columns 4 (i % 4) .. + 3, and lane j
// receives column j. vt16_off gives this lane's byte offset for d block mb
// at ks = 0; the row swizzle repeats every 8 rows, so the second read and
// later steps are that offset plus constants (which the LDS instructions
// take as immediates).
template <class SH>
__device__ __forceinline__ uint32_t vt16_off(int mb, int lane) {
  const int row = 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int col = 16 * mb + 4 * (lane & 3);  // element column, a multiple of 4
  return (uint32_t)(((row * SH::CH + ((col >> 3) ^ swz_v16<SH::CH>(row))) * 8 + (col & 7)) * 2);
}
template <class SH>
__device__ __forceinline__ bf16x8 read_vt16(const uint8_t* v_lds, int ks, uint32_t off) {
  constexpr uint32_t kRow = SH::CH * 16;  // bytes per V row
  const uint8_t* lo = v_lds + off + 32 * ks * kRow;
  const shortx4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)lo);
  const shortx4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(lo + 16 * kRow));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand of O^T += V^T P^T for 16-key step s, d block mb: two transposing
// LDS reads give lane l the 8 keys (in the permuted slot order shared with
// P) of column d = 32 mb + l % 32.
template <class SH>
__device__ __forceinline__ bf16x8 read_vt(const uint16_t* v_lds, int s, int mb, int tr_row, int tr_chunk,
                                          int tr_elem) {
  const int r_lo = 16 * s + tr_row;
  const int r_hi = r_lo + 8;
  const int c = 4 * mb + tr_chunk;
  const uint16_t* lo = v_lds + (r_lo * SH::CH + (c ^ swz_v<SH::CH>(r_lo))) * 8 + tr_elem;
  const uint16_t* hi = v_lds + (r_hi * SH::CH + (c ^ swz_v<SH::CH>(r_hi))) * 8 + tr_elem;
  const shortx4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)lo);
  const shortx4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }

// Tile row maximum in log2 units (rounded product) and its margin over the
// running maximum (rounded difference). Never contracted into one FMA, so
// every instantiation (forward, calibration, bf16, fp8) takes bit-identical
// skip decisions from the same scores.
__device__ __forceinline__ void tile_margin(float tile_max, float c2, float m, float& rowmax, float& x) {
#pragma clang fp contract(off)
  rowmax = tile_max * c2;
  x = rowmax - m;
}

// Maximum of x over the wave's 64 lanes (DPP steps within quads, half rows
// and rows of 16 lanes, then row broadcasts), read back from lane 63 so that
// it is wave-uniform.
__device__ __forceinline__ float wave_max(float x) {
#define SSA_DPP_MAX(CTRL, ROWS)                                                                 \
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), \
                                                          CTRL, ROWS, 0xF, false)))
  SSA_DPP_MAX(0xB1, 0xF);   // quad_perm [1, 0, 3, 2]
  SSA_DPP_MAX(0x4E, 0xF);   // quad_perm [2, 3, 0, 1]
  SSA_DPP_MAX(0x141, 0xF);  // row_half_mirror
  SSA_DPP_MAX(0x140, 0xF);  // row_mirror: every lane holds its row's maximum
  SSA_DPP_MAX(0x142, 0xA);  // row_bcast:15 into rows 1 and 3
  SSA_DPP_MAX(0x143, 0xC);  // row_bcast:31 into rows 2 and 3: lane 63 holds the maximum
#undef SSA_DPP_MAX
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// ===========================================================================
// FP8 (OCP e4m3) variant: the same tile loop with Q K^T and P V on the
// fp8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales).
// Q, K, V are e4m3 with per-tensor dequantization scales; scores are
// (q8 . k8) * scale_q * scale_k * sm_scale * log2(e) in fp32, so the skip
// test is the bf16 kernel's test on the dequantized values. P is rounded to
// e4m3 for the P.V product (P <= 2^8 by the lazy rescale, inside e4m3's
// range); O = scale_v * acc / l is written as bf16.
// ===========================================================================
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) intx2 lds_intx2;

constexpr int kE8M0One = 127;  // block scale 2^0 for the scaled MFMA

template <int D, int BLK>
struct Shape8 {
  static constexpr int NW = BLK / 32;     // waves (32 query rows each)
  static constexpr int NT = NW * 64;
  static constexpr int KB = BLK / 32;     // 32-key blocks of S^T
  static constexpr int DS = D / 64;       // 64-wide d steps of S^T = K Q^T
  static constexpr int MB = D / 32;       // 32-wide d blocks of O^T
  static constexpr int KS = BLK / 64;     // 64-key steps of O^T += V^T P^T
  static constexpr int CH = D / 16;       // 16-byte granules per row (1 byte per element)
  static constexpr int GRAN = BLK * CH;
  static constexpr int DMA = GRAN / NT;
  static_assert(GRAN % NT == 0, "tile must split evenly over the threads");
  static_assert(CH == 4 || CH == 8, "head_dim 64 or 128");
};

// K rows: the 16 rows one ds_read_b128 pass serves read the same granule
// column; XOR with (row / (16 / CH)) spreads them over all banks.
template <int CH>
__device__ __forceinline__ int swz_k8(int row) { return (row / (16 / CH)) & (CH - 1); }

// V rows: a ds_read_b64_tr_b8 pass reads 32 contiguous bytes (two granules)
// from each of 8 rows {0..3, 8..11} (+4 for the other half-wave); an even
// XOR keeps each granule pair together and puts the 8 rows on distinct banks.
template <int CH>
__device__ __forceinline__ int swz_v8(int row) {
  if constexpr (CH == 8) {
    return 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1));
  } else {
    return 2 * ((row >> 3) & 1);
  }
}

// global -> LDS copy of one BLK x D e4m3 tile (same scheme as dma_load).
template <int D, int BLK, bool IS_V>
__device__ __forceinline__ void dma_load8(const uint8_t* head, uint32_t bytes, uint8_t* lds, int row0,
                                          int64_t stride_tok, int wave, int lane, int i0 = 0, int di = 1) {
  using SH = Shape8<D, BLK>;
  constexpr int RPI = 64 / SH::CH;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)head, 0, bytes, kBufferFlags);
  const int lrow = lane / SH::CH;
#pragma unroll
  for (int i = i0; i < SH::DMA; i += di) {
    const int rin = RPI * (i * SH::NW + wave);
    const int row = rin + lrow;
    const int chunk = (lane % SH::CH) ^ (IS_V ? swz_v8<SH::CH>(row) : swz_k8<SH::CH>(row));
    const uint32_t voff = (uint32_t)((int64_t)lrow * stride_tok + chunk * 16);
    const uint32_t soff = (uint32_t)((int64_t)(row0 + rin) * stride_tok);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + (i * SH::NW + wave) * 1024), 16, voff, soff, 0,
                                             0);
  }
}

template <int D>
__device__ __forceinline__ uint32_t head_extent8(int rows, int64_t stride_tok) {
  return rows > 0 ? (uint32_t)((int64_t)(rows - 1) * stride_tok + D) : 0u;
}

// A operand of S^T = K Q^T (32x32x64): key 32 kb + l32, d bytes [64 s + 32 hl, +32)
template <class SH>
__device__ __forceinline__ intx8 read_k8(const uint8_t* k_lds, int kb, int s, int l32, int hl) {
  const int row = 32 * kb + l32;
  const int g0 = 4 * s + 2 * hl;
  const int sw = swz_k8<SH::CH>(row);
  const uint4 a = *reinterpret_cast<const uint4*>(k_lds + (row * SH::CH + (g0 ^ sw)) * 16);
  const uint4 b = *reinterpret_cast<const uint4*>(k_lds + (row * SH::CH + ((g0 + 1) ^ sw)) * 16);
  return intx8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// A operand of O^T += V^T P^T for 64-key step s, d block mb: four transposing
// byte reads give lane l the 32 keys (in P's slot order) of column
// d = 32 mb + l % 32. Read t covers slots 8t..8t+7: this lane supplies row
// tr_off[t] / row bytes of the step, granule 2 mb + g (stored at position
// (2 mb + g) ^ tr_sw[t]; the XOR is even, so g stays the low bit) and byte
// 8 c of it; tr_off[t] holds the row, g and c parts.
template <class SH>
__device__ __forceinline__ intx8 read_vt8(const uint8_t* v_lds, int s, int mb, const int* tr_off,
                                          const int* tr_sw) {
  intx8 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint8_t* ptr = v_lds + s * 64 * (SH::CH * 16) + tr_off[t] + ((2 * mb) ^ tr_sw[t]) * 16;
    const intx2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2*)ptr);
    r[2 * t] = x[0];
    r[2 * t + 1] = x[1];
  }
  return r;
}

// ===========================================================================
// Block-scaled q/k (MXFP8) variant: S^T = K Q^T on the fp8 matrix cores with
// one E8M0 scale per 32 consecutive d of every q and k row; v is bf16, and
// the skip vote, softmax, P and O^T += V^T P^T are those of the bf16 kernel.
// In v_mfma_scale_f32_32x32x64_f8f6f4 lane l holds row l % 32 of each
// operand; its bytes 0-15 are reduction indices 16 (l / 32) .. +15 and its
// bytes 16-31 are 32 + 16 (l / 32) .. +15, and the scale of reduction block
// 0 (indices 0-31) is supplied by lane l % 32, that of block 1 by lane
// l % 32 + 32 (measured on gfx950). So for the 64-wide d step s a lane
// gathers d [64 s + 16 h, +16) and [64 s + 32 + 16 h, +16) (h = l / 32) and
// supplies the scale of MX block 2 s + h. A scale row (D / 32 bytes of one
// token and head) is fetched with one buffer load; rows past the sequence end
// read as zero.
// ===========================================================================
// A operand of the block-scaled S^T = K Q^T: key 32 kb + l32, d granules
// 4 s + hl and 4 s + 2 + hl (16 bytes each), in the order the scales need.
template <class SH>
__device__ __forceinline__ intx8 read_k8_mx(const uint8_t* k_lds, int kb, int s, int l32, int hl) {
  const int row = 32 * kb + l32;
  const int sw = swz_k8<SH::CH>(row);
  const uint4 a = *reinterpret_cast<const uint4*>(k_lds + (row * SH::CH + ((4 * s + hl) ^ sw)) * 16);
  const uint4 b = *reinterpret_cast<const uint4*>(k_lds + (row * SH::CH + ((4 * s + 2 + hl) ^ sw)) * 16);
  return intx8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}
// Scale row at byte voff (per lane) + soff (uniform); the range check covers
// both, so rows at or past the sequence end read as zero.
template <int D>
__device__ __forceinline__ uint32_t load_scale_row(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  if constexpr (D == 128) {
    return __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)voff, (int)soff, 0);
  } else {
    return __builtin_amdgcn_raw_buffer_load_b16(rsrc, (int)voff, (int)soff, 0);
  }
}

// ===========================================================================
// Score layouts. After S^T = K_j Q^T each lane holds some of the wave's 32
// query rows and, for each, some of the tile's keys; the tile loop reaches
// the scores only through these descriptions.
//   L32 (32x32 MFMA results): lane l holds query l % 32; register r of
//       32-key block kb is key 32 kb + 8 (r / 4) + 4 (l / 32) + r % 4. The
//       rest of the row is in lane l ^ 32.
//   L16 (16x16 MFMA results): lane l holds queries l % 16 and 16 + l % 16
//       (rows i = 0, 1); register r of 16-key block kb is key
//       16 kb + 4 (l / 16) + r. Each row is spread over lanes l, l ^ 16,
//       l ^ 32 and l ^ 48.
// ===========================================================================
template <int BLK>
struct L32 {
  static constexpr int NR = 1;  // query rows per lane
  using Scores = floatx16[BLK / 32];
  __device__ static int row(int, int lane) { return lane & 31; }
  __device__ static void mask(Scores& sc, int lane, const int (&kmax)[NR]) {
#pragma unroll
    for (int kb = 0; kb < BLK / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (key >= kmax[0]) sc[kb][r] = -INFINITY;
      }
  }
  // the tile's maximum of each row, in every lane holding it
  __device__ static void row_max(const Scores& sc, float (&mx)[NR]) {
    float m = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BLK / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, sc[kb][r]);
    mx[0] = xhalf_max(m);
  }
  // total of a per-lane partial over the row's lanes
  __device__ static float row_sum(float x) { return xhalf_sum(x); }
};

template <int BLK>
struct L16 {
  static constexpr int NR = 2;
  static constexpr int KB = BLK / 16;  // 16-key blocks
  using Scores = floatx4[NR][KB];
  __device__ static int row(int i, int lane) { return 16 * i + (lane & 15); }
  __device__ static void mask(Scores& sc, int lane, const int (&kmax)[NR]) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * kb + 4 * (lane >> 4) + r;
          if (key >= kmax[i]) sc[i][kb][r] = -INFINITY;
        }
  }
  __device__ static void row_max(const Scores& sc, float (&mx)[NR]) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, sc[i][kb][r]);
      mx[i] = xhalf_max(xrow_max(m));
    }
  }
  __device__ static float row_sum(float x) { return xhalf_sum(xrow_sum(x)); }
};

// ===========================================================================
// Operand policies. The tile loop below is written once; what differs between
// the bf16, e4m3 and block-scaled q/k modes is how Q, K and V are held and
// multiplied, and that lives in these classes (each names its score layout;
// a QK and a PV policy that work together share it):
//   Qk*: the Q fragment (loaded once), the K tile fetch (with its per-lane
//        block scales in the MX mode) and S^T = K_j Q^T into 4 accumulator
//        blocks of 32 keys. scores() takes a hook that it calls once per d
//        step, before that step's MFMAs; fetch_part(.., s, on) is the share
//        of a tile fetch that goes with step s, so the next K tile can stream
//        in during this one (with on = false its loads have an empty range:
//        they touch no memory and leave zeros, which keeps the loop free of
//        branches around them);
//   Pv*: the V tile fetch, the softmax numerator P (exponentials, the row
//        sum and the rounding to the P.V operand type) and O^T += V_j^T P^T.
// ===========================================================================

// bf16 Q and K: v_mfma_f32_16x16x32_bf16 (layout L16). A K fragment is read
// one d step ahead of its MFMAs and feeds both of the lane's query rows.
// (The 16x16 shape does the same work as 32x32x16 for less energy per FLOP;
// at the part's power limit that is what the bf16 kernel runs at.)
template <int D, int BLK>
struct QkBf16 {
  using SH = Shape<D, BLK>;
  using Layout = L16<BLK>;
  static constexpr int NR = Layout::NR;
  static constexpr int KB = Layout::KB;
  static constexpr int DS = D / 32;  // 32-wide d steps
  static constexpr int LDS_BYTES = BLK * D * 2;
  const uint16_t* kbase;
  uint32_t bytes;
  int64_t stride;
  bf16x8 qf[NR][DS];  // B operand: query row i, d [32 s + 8 (l / 16), + 8)

  __device__ QkBf16(const LaunchParams& p, const WorkItem& w, int64_t head_off, const int (&qrow)[NR],
                    const bool (&qvalid)[NR], int lane)
      : kbase(p.k + head_off), bytes(head_extent<D>(w.S, p.stride_tok)), stride(p.stride_tok) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const uint16_t* qp = p.q + head_off + (int64_t)(qvalid[i] ? qrow[i] : 0) * p.stride_tok + 8 * (lane >> 4);
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (qvalid[i]) raw = *reinterpret_cast<const uint4*>(qp + 32 * s);
        qf[i][s] = __builtin_bit_cast(bf16x8, raw);
      }
    }
  }
  __device__ void fetch(uint8_t* lds, int j, int wave, int lane) {
    dma_load<D, BLK, Swz::K>(kbase, bytes, reinterpret_cast<uint16_t*>(lds), j * BLK, stride, wave, lane);
  }
  __device__ void fetch_part(uint8_t* lds, int j, int wave, int lane, int s, bool on) {
    dma_load<D, BLK, Swz::K>(kbase, on ? bytes : 0u, reinterpret_cast<uint16_t*>(lds), j * BLK, stride, wave, lane,
                             s, DS);
  }
  __device__ void advance() {}
  template <class Hook>
  __device__ void scores(typename Layout::Scores& sc, const uint8_t* lds, int lane, Hook&& hook) const {
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sc[i][kb] = floatx4{};
    uint32_t koff[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) koff[s] = k16_off<SH>(s, lane);
    bf16x8 ka[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) ka[kb] = read_k16<SH>(lds, kb, koff[0]);
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      hook(s);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = ka[kb];
        if (s + 1 < DS) ka[kb] = read_k16<SH>(lds, kb, koff[s + 1]);
#pragma unroll
        for (int i = 0; i < NR; ++i) sc[i][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[i][s], sc[i][kb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// e4m3 Q and K with per-tensor scales: the scaled MFMA with unit block scales
// (the per-tensor factors are folded into the score scale on the host).
template <int D, int BLK>
struct QkFp8 {
  using SH = Shape8<D, BLK>;
  using Layout = L32<BLK>;
  static constexpr int NR = Layout::NR;
  static constexpr int LDS_BYTES = BLK * D;
  const uint8_t* kbase;
  uint32_t bytes;
  int64_t stride;
  intx8 qf[SH::DS];

  __device__ QkFp8(const LaunchParams& p, const WorkItem& w, int64_t head_off, const int (&qrows)[NR],
                   const bool (&qvalids)[NR], int lane)
      : kbase(reinterpret_cast<const uint8_t*>(p.k) + head_off), bytes(head_extent8<D>(w.S, p.stride_tok)),
        stride(p.stride_tok) {
    const int qrow = qrows[0], hl = lane >> 5;
    const bool qvalid = qvalids[0];
    // B operand: query qrow, d bytes [64 s + 32 hl, +32)
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + head_off + (int64_t)(qvalid ? qrow : 0) * p.stride_tok +
                        32 * hl;
#pragma unroll
    for (int s = 0; s < SH::DS; ++s) {
      uint4 a = make_uint4(0u, 0u, 0u, 0u), c = make_uint4(0u, 0u, 0u, 0u);
      if (qvalid) {
        a = *reinterpret_cast<const uint4*>(qp + 64 * s);
        c = *reinterpret_cast<const uint4*>(qp + 64 * s + 16);
      }
      qf[s] = intx8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
    }
  }
  __device__ void fetch(uint8_t* lds, int j, int wave, int lane) {
    dma_load8<D, BLK, false>(kbase, bytes, lds, j * BLK, stride, wave, lane);
  }
  __device__ void fetch_part(uint8_t* lds, int j, int wave, int lane, int s, bool on) {
    dma_load8<D, BLK, false>(kbase, on ? bytes : 0u, lds, j * BLK, stride, wave, lane, s, SH::DS);
  }
  __device__ void advance() {}
  template <class Hook>
  __device__ void scores(typename Layout::Scores& sc, const uint8_t* k_lds, int lane, Hook&& hook) const {
    const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb) sc[kb] = floatx16{};
#pragma unroll
    for (int s = 0; s < SH::DS; ++s) {
      hook(s);
      intx8 ka[SH::KB];
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb) ka[kb] = read_k8<SH>(k_lds, kb, s, l32, hl);
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb)
        sc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[kb], qf[s], sc[kb], 0, 0, 0, kE8M0One, 0,
                                                                 kE8M0One);
    }
  }
};

// Block-scaled (MX) e4m3 Q and K: the scaled MFMA with one E8M0 scale per 32
// d of every row; each lane fetches its key rows' scales with the K tile.
template <int D, int BLK>
struct QkMx {
  using SH = Shape8<D, BLK>;
  using Layout = L32<BLK>;
  static constexpr int NR = Layout::NR;
  static constexpr int LDS_BYTES = BLK * D;
  const uint8_t* kbase;
  uint32_t bytes;
  int64_t stride;
  __amdgpu_buffer_rsrc_t ks_rsrc, ks_rsrc_off;  // K scale rows; the same with an empty range
  uint32_t sc_lane, sc_blk, sc_tile;
  intx8 qf[SH::DS];
  uint32_t qsc[SH::DS];
  uint32_t ks[SH::KB];     // scale rows of this lane's keys in the K tile in use
  uint32_t ks_nx[SH::KB];  // the same for the next tile when it is fetched during this one

  __device__ QkMx(const LaunchParams& p, const WorkItem& w, int64_t head_off, const int (&qrows)[NR],
                  const bool (&qvalids)[NR], int lane)
      : kbase(reinterpret_cast<const uint8_t*>(p.k) + head_off), bytes(head_extent8<D>(w.S, p.stride_tok)),
        stride(p.stride_tok) {
    const int qrow = qrows[0], hl = lane >> 5;
    const bool qvalid = qvalids[0];
    constexpr int SROW = D / 32;  // scale bytes per row
    const int64_t sc_off = (int64_t)w.tok0 * p.bs_tok + (int64_t)w.h * p.bs_head;
    const uint32_t sc_bytes = w.S > 0 ? (uint32_t)((int64_t)(w.S - 1) * p.bs_tok + SROW) : 0u;
    ks_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k_bscale + sc_off), 0, sc_bytes, kBufferFlags);
    ks_rsrc_off = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k_bscale + sc_off), 0, 0u, kBufferFlags);
    const __amdgpu_buffer_rsrc_t qs_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.q_bscale + sc_off), 0, sc_bytes, kBufferFlags);
    // lane: key 32 kb + l32 (the host keeps (S + BLK) * bs_tok within 32 bits)
    const int l32 = qrow & 31;
    sc_lane = (uint32_t)(l32 * p.bs_tok);
    sc_blk = (uint32_t)(32 * p.bs_tok);
    sc_tile = (uint32_t)(BLK * p.bs_tok);
    // Q fragment (B operand): query qrow, d bytes [64 s + 16 hl, +16) and
    // [64 s + 32 + 16 hl, +16), and the scale of its MX block 2 s + hl
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + head_off + (int64_t)(qvalid ? qrow : 0) * p.stride_tok +
                        16 * hl;
#pragma unroll
    for (int s = 0; s < SH::DS; ++s) {
      uint4 a = make_uint4(0u, 0u, 0u, 0u), c = make_uint4(0u, 0u, 0u, 0u);
      if (qvalid) {
        a = *reinterpret_cast<const uint4*>(qp + 64 * s);
        c = *reinterpret_cast<const uint4*>(qp + 64 * s + 32);
      }
      qf[s] = intx8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
    }
    const uint32_t qs = load_scale_row<D>(qs_rsrc, sc_lane, (uint32_t)((qrow - l32) * p.bs_tok));
#pragma unroll
    for (int s = 0; s < SH::DS; ++s) qsc[s] = qs >> (8 * (2 * s + hl));  // byte 0: this lane's block
  }
  __device__ void fetch(uint8_t* lds, int j, int wave, int lane) {
    dma_load8<D, BLK, false>(kbase, bytes, lds, j * BLK, stride, wave, lane);
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb) ks[kb] = load_scale_row<D>(ks_rsrc, sc_lane, j * sc_tile + kb * sc_blk);
  }
  // the scale rows go with step 0; advance() makes them current once S^T of this tile is done
  __device__ void fetch_part(uint8_t* lds, int j, int wave, int lane, int s, bool on) {
    dma_load8<D, BLK, false>(kbase, on ? bytes : 0u, lds, j * BLK, stride, wave, lane, s, SH::DS);
    if (s == 0) {
      const __amdgpu_buffer_rsrc_t r = on ? ks_rsrc : ks_rsrc_off;
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb) ks_nx[kb] = load_scale_row<D>(r, sc_lane, j * sc_tile + kb * sc_blk);
    }
  }
  __device__ void advance() {
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb) ks[kb] = ks_nx[kb];
  }
  template <class Hook>
  __device__ void scores(typename Layout::Scores& sc, const uint8_t* k_lds, int lane, Hook&& hook) const {
    const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb) sc[kb] = floatx16{};
#pragma unroll
    for (int s = 0; s < SH::DS; ++s) {
      hook(s);
      intx8 ka[SH::KB];
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb) ka[kb] = read_k8_mx<SH>(k_lds, kb, s, l32, hl);
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb)
        sc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[kb], qf[s], sc[kb], 0, 0, 0,
                                                                 (int)(ks[kb] >> (8 * (2 * s + hl))), 0, (int)qsc[s]);
    }
  }
};

// O^T accumulators and the epilogue of each layout: zeroing, the lazy
// rescale by a per-row factor, and the store of O = acc * inv as bf16.
// L32: lane l holds query l % 32, d = 32 mb + 8 g + 4 (l / 32) + e in
// register 4 g + e of block mb.
template <int D>
struct AccL32 {
  static constexpr int NR = 1;
  static constexpr int MB = D / 32;
  using Acc = floatx16[MB];
  __device__ static void zero(Acc& acc) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx16{};
  }
  __device__ static void rescale(Acc& acc, const float (&alpha)[NR]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha[0];
  }
  __device__ static void store(const Acc& acc, const float (&inv)[NR], uint16_t* obase, const int (&qrow)[NR],
                               const bool (&qvalid)[NR], int64_t stride, int lane) {
    if (!qvalid[0]) return;
    uint16_t* op = obase + (int64_t)qrow[0] * stride + 4 * (lane >> 5);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 f = {acc[mb][4 * g] * inv[0], acc[mb][4 * g + 1] * inv[0], acc[mb][4 * g + 2] * inv[0],
                           acc[mb][4 * g + 3] * inv[0]};
        *reinterpret_cast<bf16x4*>(op + 32 * mb + 8 * g) = __builtin_convertvector(f, bf16x4);
      }
  }
};

// L16: lane l holds queries 16 i + l % 16 (i = 0, 1), d = 16 mb + 4 (l / 16) + r
// in register r of block [i][mb].
template <int D>
struct AccL16 {
  static constexpr int NR = 2;
  static constexpr int MB = D / 16;
  using Acc = floatx4[NR][MB];
  __device__ static void zero(Acc& acc) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[i][mb] = floatx4{};
  }
  __device__ static void rescale(Acc& acc, const float (&alpha)[NR]) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[i][mb] *= alpha[i];
  }
  __device__ static void store(const Acc& acc, const float (&inv)[NR], uint16_t* obase, const int (&qrow)[NR],
                               const bool (&qvalid)[NR], int64_t stride, int lane) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (!qvalid[i]) continue;
      uint16_t* op = obase + (int64_t)qrow[i] * stride + 4 * (lane >> 4);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const floatx4 f = acc[i][mb] * inv[i];
        *reinterpret_cast<bf16x4*>(op + 16 * mb) = __builtin_convertvector(f, bf16x4);
      }
    }
  }
};

// bf16 V and P in layout L32 (the block-scaled q/k mode's P.V): P rounded to
// bf16 feeds O^T += V^T P^T (v_mfma_f32_32x32x16_bf16) directly from the
// score registers; V^T comes from the row-major V tile through transposing
// LDS reads, two 16-key steps ahead of their MFMAs.
template <int D, int BLK>
struct PvBf16 : AccL32<D> {
  using SH = Shape<D, BLK>;
  using Layout = L32<BLK>;
  using typename AccL32<D>::Acc;
  static constexpr int NR = Layout::NR;
  static constexpr int LDS_BYTES = BLK * D * 2;
  using PFrag = bf16x8[SH::KS];
  const uint16_t* vbase;
  uint32_t bytes;
  int64_t stride;
  int tr_row, tr_chunk, tr_elem;  // V^T read position: row in a 16-key step, granule, element

  __device__ PvBf16(const LaunchParams& p, const WorkItem& w, int64_t head_off, int lane)
      : vbase(p.v + head_off), bytes(head_extent<D>(w.S, p.stride_tok)), stride(p.stride_tok) {
    const int hl = lane >> 5;
    tr_row = 4 * hl + ((lane & 15) >> 2);
    tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr_elem = 4 * (lane & 1);
  }
  __device__ static float out_scale(const LaunchParams&) { return 1.0f; }
  __device__ void fetch(uint8_t* lds, int j, int wave, int lane) {
    dma_load<D, BLK, Swz::V>(vbase, bytes, reinterpret_cast<uint16_t*>(lds), j * BLK, stride, wave, lane);
  }
  // P = 2^(s * c2 - m) in the slot order of the P.V B operand; l += row sum
  __device__ static void make_p(const typename Layout::Scores& sc, float c2, const float (&nm)[NR], float (&l)[NR],
                                PFrag& pb) {
#pragma unroll
    for (int s = 0; s < SH::KS; ++s) {
      floatx8 e;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        e[r] = fast_exp2(fmaf(sc[s >> 1][8 * (s & 1) + r], c2, nm[0]));
        l[0] += e[r];
      }
      pb[s] = __builtin_convertvector(e, bf16x8);
    }
  }
  __device__ void accumulate(Acc& acc, const uint8_t* lds, const PFrag& pb) const {
    const uint16_t* v_lds = reinterpret_cast<const uint16_t*>(lds);
    bf16x8 va[3][SH::MB];
#pragma unroll
    for (int s = 0; s < 2 && s < SH::KS; ++s)
#pragma unroll
      for (int mb = 0; mb < SH::MB; ++mb) va[s][mb] = read_vt<SH>(v_lds, s, mb, tr_row, tr_chunk, tr_elem);
#pragma unroll
    for (int s = 0; s < SH::KS; ++s) {
      if (s + 2 < SH::KS) {
#pragma unroll
        for (int mb = 0; mb < SH::MB; ++mb)
          va[(s + 2) % 3][mb] = read_vt<SH>(v_lds, s + 2, mb, tr_row, tr_chunk, tr_elem);
      }
#pragma unroll
      for (int mb = 0; mb < SH::MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s % 3][mb], pb[s], acc[mb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// e4m3 V with a per-tensor scale: P rounded to e4m3 (two values per
// v_cvt_pk_fp8_f32), V^T gathered by transposing byte reads, P.V on the
// scaled MFMA with unit block scales; O carries scale_v.
template <int D, int BLK>
struct PvFp8 : AccL32<D> {
  using SH = Shape8<D, BLK>;
  using Layout = L32<BLK>;
  using typename AccL32<D>::Acc;
  static constexpr int NR = Layout::NR;
  static constexpr int LDS_BYTES = BLK * D;
  using PFrag = intx8[SH::KS];
  const uint8_t* vbase;
  uint32_t bytes;
  int64_t stride;
  int tr_off[4], tr_sw[4];

  __device__ PvFp8(const LaunchParams& p, const WorkItem& w, int64_t head_off, int lane)
      : vbase(reinterpret_cast<const uint8_t*>(p.v) + head_off), bytes(head_extent8<D>(w.S, p.stride_tok)),
        stride(p.stride_tok) {
    // source lane (2e + c) of each 16-lane group supplies key slot e of a
    // transposing read, columns 16 g + 8 c of the 32-wide d block
    const int hl = lane >> 5;
    const int e = (lane & 15) >> 1, c = lane & 1, g = (lane & 31) >> 4;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int key = 32 * (tt >> 1) + 16 * (tt & 1) + 8 * (e >> 2) + 4 * hl + (e & 3);
      tr_off[tt] = key * (SH::CH * 16) + g * 16 + 8 * c;
      tr_sw[tt] = swz_v8<SH::CH>(key);
    }
  }
  __device__ static float out_scale(const LaunchParams& p) { return p.v_scale; }
  __device__ void fetch(uint8_t* lds, int j, int wave, int lane) {
    dma_load8<D, BLK, true>(vbase, bytes, lds, j * BLK, stride, wave, lane);
  }
  // P^T for 64-key step s: byte 16 u + r is score register r of key block 2 s + u
  __device__ static void make_p(const typename Layout::Scores& sc, float c2, const float (&nm)[NR], float (&l)[NR],
                                PFrag& pb) {
#pragma unroll
    for (int s = 0; s < SH::KS; ++s)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = 2 * s + (w >> 2);
        const int r0 = 4 * (w & 3);
        float e0 = fast_exp2(fmaf(sc[kb][r0], c2, nm[0]));
        float e1 = fast_exp2(fmaf(sc[kb][r0 + 1], c2, nm[0]));
        float e2 = fast_exp2(fmaf(sc[kb][r0 + 2], c2, nm[0]));
        float e3 = fast_exp2(fmaf(sc[kb][r0 + 3], c2, nm[0]));
        l[0] += (e0 + e1) + (e2 + e3);
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, word, true);
        pb[s][w] = word;
      }
  }
  __device__ void accumulate(Acc& acc, const uint8_t* v_lds, const PFrag& pb) const {
#pragma unroll
    for (int s = 0; s < SH::KS; ++s) {
      intx8 va[SH::MB];
#pragma unroll
      for (int mb = 0; mb < SH::MB; ++mb) va[mb] = read_vt8<SH>(v_lds, s, mb, tr_off, tr_sw);
#pragma unroll
      for (int mb = 0; mb < SH::MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[mb], pb[s], acc[mb], 0, 0, 0, kE8M0One, 0,
                                                                  kE8M0One);
    }
  }
};

// bf16 V and P on v_mfma_f32_16x16x32_bf16 (layout L16): P rounded to bf16
// feeds O^T += V^T P^T from the score registers, slots 0-3 from 16-key block
// 2 ks and slots 4-7 from block 2 ks + 1 of each 32-key step; V^T comes from
// the row-major V tile through transposing LDS reads one step ahead.
template <int D, int BLK>
struct PvBf16x16 : AccL16<D> {
  using SH = Shape<D, BLK>;
  using Layout = L16<BLK>;
  using typename AccL16<D>::Acc;
  static constexpr int NR = Layout::NR;
  static constexpr int MB = D / 16;   // 16-wide d blocks
  static constexpr int KS = BLK / 32;  // 32-key steps
  static constexpr int LDS_BYTES = BLK * D * 2;
  using PFrag = bf16x8[NR][KS];
  const uint16_t* vbase;
  uint32_t bytes;
  int64_t stride;
  uint32_t voff[MB];  // V^T read offsets (bytes, ks = 0) of this lane per d block

  __device__ PvBf16x16(const LaunchParams& p, const WorkItem& w, int64_t head_off, int lane)
      : vbase(p.v + head_off), bytes(head_extent<D>(w.S, p.stride_tok)), stride(p.stride_tok) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) voff[mb] = vt16_off<SH>(mb, lane);
  }
  __device__ static float out_scale(const LaunchParams&) { return 1.0f; }
  __device__ void fetch(uint8_t* lds, int j, int wave, int lane) {
    dma_load<D, BLK, Swz::V16>(vbase, bytes, reinterpret_cast<uint16_t*>(lds), j * BLK, stride, wave, lane);
  }
  // P = 2^(s * c2 - m) in the slot order of the P.V B operand; l += row sum
  __device__ static void make_p(const typename Layout::Scores& sc, float c2, const float (&nm)[NR], float (&l)[NR],
                                PFrag& pb) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        floatx8 e;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          e[r] = fast_exp2(fmaf(sc[i][2 * ks + (r >> 2)][r & 3], c2, nm[i]));
          l[i] += e[r];
        }
        pb[i][ks] = __builtin_convertvector(e, bf16x8);
      }
  }
  __device__ void accumulate(Acc& acc, const uint8_t* lds, const PFrag& pb) const {
    // V^T fragments two steps ahead: the first two steps' reads all issue before any MFMA
    bf16x8 va[2][MB];
#pragma unroll
    for (int s0 = 0; s0 < 2 && s0 < KS; ++s0)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) va[s0][mb] = read_vt16<SH>(lds, s0, voff[mb]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 a = va[ks & 1][mb];
        if (ks + 2 < KS) va[ks & 1][mb] = read_vt16<SH>(lds, ks + 2, voff[mb]);
#pragma unroll
        for (int i = 0; i < NR; ++i)
          acc[i][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[i][ks], acc[i][mb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// ===========================================================================
// The tile loop (forward and calibration), one work-group per Q-block.
//
// Two buffering schemes for K, chosen by LDS size (two work-groups share a
// CU's 160 KB):
//   * double K, when two K tiles and one V tile fit in 64 KB (every e4m3 and
//     block-scaled shape, bf16 with head_dim 64 or 64-row tiles) and the
//     kernel skips tiles (not the calibration pass): K_{j+1} is issued into
//     the other K buffer at the start of S^T = K_j Q^T. A skipped tile then
//     costs its product, the vote and one barrier (every wave voted to skip
//     and waited for its share of K_{j+1} before it); a kept tile adds the V
//     fetch and a second barrier before P.V, after which both tiles are in.
//   * single K otherwise (bf16 with head_dim 128 and 128-row tiles, where K
//     and V take 32 KB each, and every calibration pass): K_{j+1} is fetched
//     after the vote, once every wave is done reading K_j, and every tile
//     ends with a wait and a barrier.
// With one barrier per skipped tile a fast wave can reach the next tile's
// vote before a slow one has read this tile's, so the vote slots alternate
// by tile parity (the slot of tile j is rewritten at tile j + 2, after a
// barrier every wave passes only once it has read tile j's votes).
// ===========================================================================
template <class QK, class PV, bool CALIB>
struct Buffering {
  static constexpr bool kDoubleK = !CALIB && 2 * QK::LDS_BYTES + PV::LDS_BYTES <= 64 * 1024;
  static constexpr int K1_BYTES = kDoubleK ? QK::LDS_BYTES : 16;  // unused in the other schemes
  static constexpr int K1_ALIGN = kDoubleK ? 1024 : 16;
};

template <int D, int BLK, class QK, class PV, bool CALIB>
__global__ __launch_bounds__(2 * BLK, 2) void fwd_kernel(const LaunchParams p) {  // 2*BLK = 64 * BLK / 32 threads
  using LY = typename QK::Layout;
  static_assert(__is_same(LY, typename PV::Layout), "the QK and PV policies must share the score layout");
  constexpr int NR = LY::NR;    // query rows per lane
  constexpr int NW = BLK / 32;  // waves, 32 query rows each
  constexpr bool kDoubleK = Buffering<QK, PV, CALIB>::kDoubleK;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[QK::LDS_BYTES];
  __shared__ alignas(Buffering<QK, PV, CALIB>::K1_ALIGN) uint8_t k_lds1[Buffering<QK, PV, CALIB>::K1_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[PV::LDS_BYTES];
  __shared__ uint64_t vote[2][NW];  // by tile parity
  __shared__ float dvote[2][NW];    // calibration: each wave's maximum of x

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps tile addressing scalar
  const int lane = tid & 63;

  const WorkItem w = map_workgroup(p, blockIdx.x, BLK);
  const int b = w.b, h = w.h, qb = w.qb, nK = w.nk, S = w.S;
  const int H = p.num_heads;
  const int64_t head_off = (int64_t)w.tok0 * p.stride_tok + (int64_t)h * p.stride_head;  // elements

  int qloc[NR], qrow[NR];  // this lane's rows: within the wave's 32, and within the sequence
  bool qvalid[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    qloc[i] = LY::row(i, lane);
    qrow[i] = qb * BLK + wave * 32 + qloc[i];
    qvalid[i] = qrow[i] < S;
  }
  QK qk(p, w, head_off, qrow, qvalid, lane);
  qk.fetch(k_lds, 0, wave, lane);
  PV pv(p, w, head_off, lane);

  const float c2 = p.scale_log2;
  const float t = CALIB ? 0.0f : p.t_bh[b * H + h];
  const int ncal = CALIB ? p.ncal : 0;
  const float my_t = (CALIB && lane < ncal) ? p.cal_t[lane] : INFINITY;  // lane k holds threshold k
  int ncount = 0;

  float m_true[NR], m_use[NR], l[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    m_true[i] = -INFINITY;  // running max of the method (log2 units), updated on kept tiles
    m_use[i] = -INFINITY;   // exponent base, m_use <= m_true < m_use + slack
    l[i] = 0.0f;            // partial row sum over this lane's keys
  }
  typename PV::Acc acc;
  PV::zero(acc);
  int skipped = 0;

  wait_dma();
  __syncthreads();

  // One tile. kcur holds K_j; in the double-K scheme K_{j+1} goes to knext.
  // Both are always the named LDS arrays (the loop below is unrolled by two
  // in that scheme), so the compiler sees that the reads of kcur do not
  // depend on the copy into knext and adds no wait for it.
  auto tile = [&](uint8_t* kcur, uint8_t* knext, const int j) __attribute__((always_inline)) {
    const int nvalid = min(BLK, S - j * BLK);
    const bool more = j + 1 < nK;
    constexpr bool pf = kDoubleK;  // K_{j+1} streams into knext during this tile's S^T

    // ---- S^T = K_j Q^T (always paid) -------------------------------------
    typename LY::Scores sc;
    if constexpr (kDoubleK) {
      qk.scores(sc, kcur, lane, [&](int s) __attribute__((always_inline)) {
        qk.fetch_part(knext, j + 1, wave, lane, s, more);  // empty range at the last tile
      });
      qk.advance();
    } else {
      qk.scores(sc, kcur, lane, [](int) {});
    }
    // keys past the sequence end; causal: keys after each row's query (diagonal tile)
    if (p.causal ? j == qb : nvalid < BLK) {
      int kmax[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) kmax[i] = (p.causal && j == qb) ? min(nvalid, wave * 32 + qloc[i] + 1) : nvalid;
      LY::mask(sc, lane, kmax);
    }

    // ---- tile row max and the skip vote ----------------------------------
    float tmax[NR], rowmax[NR], x[NR];
    LY::row_max(sc, tmax);
    float xw = -INFINITY;  // this lane's largest margin over its valid rows
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      tile_margin(tmax[i], c2, m_true[i], rowmax[i], x[i]);  // m_true = -inf gives x = +inf
      if (!qvalid[i]) x[i] = -INFINITY;
      xw = fmaxf(xw, x[i]);
    }
    bool wait_k = false;
    if constexpr (CALIB) {
      // d = max over valid rows; "some row has x >= t_k" is exactly d >= t_k
      const float dw = wave_max(xw);
      if (lane == 0) dvote[j & 1][wave] = dw;
    } else {
      const bool kw = wave_any(xw >= t);
      if (lane == 0) vote[j & 1][wave] = kw ? 1ull : 0ull;
      // A wave that keeps the tile knows it is kept and waits for its share of
      // K_{j+1} with V_j, before the second barrier. The others wait now, so
      // that when every wave skips, K_{j+1} is complete at this barrier.
      wait_k = pf && !kw;
    }
    if (wait_k) wait_dma();
    __syncthreads();  // votes (and K_{j+1}) visible; every wave is done reading K_j and V_{j-1}

    bool keep;
    if constexpr (CALIB) {
      float d = dvote[j & 1][0];
#pragma unroll
      for (int v = 1; v < NW; ++v) d = fmaxf(d, dvote[j & 1][v]);
      ncount += d < my_t ? 1 : 0;  // lanes >= ncal hold +inf and are never written out
      keep = true;
    } else {
      uint64_t all = vote[j & 1][0];
#pragma unroll
      for (int v = 1; v < NW; ++v) all |= vote[j & 1][v];
      keep = __builtin_amdgcn_readfirstlane(all != 0 ? 1 : 0) != 0;  // work-group uniform
      skipped += keep ? 0 : 1;
      if (p.tile_mask != nullptr && tid == 0)
        p.tile_mask[((int64_t)((p.seq_abs0 + b) * H + h) * p.mask_nq + qb) * p.mask_nk + j] = keep ? 0 : 1;
    }

    if (!pf && more) qk.fetch(kcur, j + 1, wave, lane);
    typename PV::PFrag pb;
    if (keep) {
      pv.fetch(v_lds, j, wave, lane);

      // ---- online softmax (log2 domain), overlapping the V fetch ---------
      bool up = false;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        m_true[i] = fmaxf(m_true[i], rowmax[i]);
        up = up || rowmax[i] > m_use[i] + kRescaleSlack;
      }
      if (wave_any(up)) {
        float alpha[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const float m_new = fmaxf(m_use[i], rowmax[i]);
          alpha[i] = fast_exp2(m_use[i] - m_new);  // 0 when m_use was -inf
          l[i] *= alpha[i];
          m_use[i] = m_new;
        }
        PV::rescale(acc, alpha);
      }
      float nm[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) nm[i] = -m_use[i];
      PV::make_p(sc, c2, nm, l, pb);
    }
    if (!pf || keep) {
      wait_dma();
      __syncthreads();  // V_j and K_{j+1} (with its scales) visible
    }

    // ---- O^T += V_j^T P^T ------------------------------------------------
    if (keep) pv.accumulate(acc, v_lds, pb);
  };

  if constexpr (kDoubleK) {
    for (int j = 0; j < nK; j += 2) {
      tile(k_lds, k_lds1, j);
      if (j + 1 < nK) tile(k_lds1, k_lds, j + 1);
    }
  } else {
    for (int j = 0; j < nK; ++j) tile(k_lds, k_lds, j);
  }

  // ---- epilogue ---------------------------------------------------------
  float inv[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) inv[i] = PV::out_scale(p) / LY::row_sum(l[i]);
  PV::store(acc, inv, p.o + head_off, qrow, qvalid, p.stride_tok, lane);
  if constexpr (CALIB) {
    if (wave == 0 && lane < ncal) p.counts[(p.wg_abs0 + w.row) * ncal + lane] = ncount;
    if (tid == 0) p.tiles[p.wg_abs0 + w.row] = nK;
  } else {
    if (tid == 0) {
      const int64_t bh = (int64_t)(p.seq_abs0 + b) * H + h;
      if (p.skipped_bh != nullptr) atomicAdd((unsigned long long*)&p.skipped_bh[bh], (unsigned long long)skipped);
      if (p.total_bh != nullptr) atomicAdd((unsigned long long*)&p.total_bh[bh], (unsigned long long)nK);
    }
  }
}

__global__ void fill_u8_kernel(uint8_t* dst, int64_t n, uint8_t value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = value;
}

__global__ void fill_u64_kernel(uint64_t* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = 0;
}

template <int D, int BLK, bool CALIB>
int launch(const LaunchParams& p, hipStream_t stream) {
  const dim3 grid(p.total_wg), threads(2 * BLK);  // BLK / 32 waves
  if (p.fp8) {
    hipLaunchKernelGGL((fwd_kernel<D, BLK, QkFp8<D, BLK>, PvFp8<D, BLK>, CALIB>), grid, threads, 0, stream, p);
  } else if (p.mxqk) {
    hipLaunchKernelGGL((fwd_kernel<D, BLK, QkMx<D, BLK>, PvBf16<D, BLK>, CALIB>), grid, threads, 0, stream, p);
  } else {
    hipLaunchKernelGGL((fwd_kernel<D, BLK, QkBf16<D, BLK>, PvBf16x16<D, BLK>, CALIB>), grid, threads, 0, stream, p);
  }
  return (int)hipGetLastError();
}

int grid_for(int64_t n) {
  int64_t blocks = (n + 255) / 256;
  return (int)(blocks < 4096 ? (blocks < 1 ? 1 : blocks) : 4096);
}

}  // namespace

int launch_forward(int head_dim, int block, bool calibrate, const LaunchParams& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (p.total_wg <= 0) return 0;
#define SSA_DISPATCH(DD, BB)                                                  \
  if (head_dim == DD && block == BB)                                          \
    return calibrate ? launch<DD, BB, true>(p, s) : launch<DD, BB, false>(p, s);
  SSA_DISPATCH(64, 64)
  SSA_DISPATCH(64, 128)
  SSA_DISPATCH(128, 64)
  SSA_DISPATCH(128, 128)
#undef SSA_DISPATCH
  return (int)hipErrorInvalidValue;
}

int launch_fill_u8(uint8_t* dst, int64_t n, uint8_t value, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_u8_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, n, value);
  return (int)hipGetLastError();
}

int launch_fill_u64(uint64_t* dst, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_u64_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, n);
  return (int)hipGetLastError();
}

}  // namespace ssa
