// Skip-softmax (BLASST) FlashAttention forward and calibration kernels for
// MI355X (gfx950, CDNA4).
//
// Method: ModelOpt pull request "skip-softmax ... via dedicated Triton
// kernels", section "Changes / Triton kernels" -- inside the FlashAttention
// loop, a KV tile whose maximum score lies far below the running softmax
// maximum is skipped (no V load, no softmax, no accumulation); a calibration
// variant computes full attention while counting, for N thresholds at once,
// the tiles that would be skipped. ModelOpt README "Skip-Softmax Sparse
// Attention for Diffusion Models", section "Threshold Modes": the comparison
// is in log2 units against log2(lambda).
//
// Work decomposition (one work-group = one Br-row Q-block of one head):
//   * Br = Bc = BLK query rows / keys per tile; BLK/32 waves, each owning 32
//     query rows. D = head dim. Two work-groups share a CU (<= 256 VGPRs +
//     AGPRs per wave, 64 KB of LDS per work-group), so each SIMD runs two
//     waves that hide each other's LDS, barrier and memory latency.
//   * Scores are computed transposed, S^T = K_j Q^T, with
//     v_mfma_f32_32x32x16_bf16: lane l then holds query (l % 32) and 16 keys
//     per 32-key block, so the per-row max and sum are in-register
//     reductions plus one v_permlane32_swap with lane l ^ 32.
//   * The same registers, rounded to bf16, are the B operand of
//     O^T += V_j^T P^T; V_j^T is read from the row-major V tile in LDS with
//     ds_read_b64_tr_b16 (4x16 transposing read). The per-lane key order
//     inside a 16-key MFMA step is permuted identically on both operands.
//   * O^T accumulates in registers; lane l owns query (l % 32), so the
//     rescale factor and row sum are per-lane scalars. The accumulator is
//     rescaled lazily: the exponent base only moves when some row's maximum
//     rose by more than 2^8, which keeps P <= 256 and the result unchanged
//     up to rounding.
//   * K and V tiles go global -> LDS with buffer_load_dwordx4 ... lds (no
//     register staging). Each wave instruction fills 1 KB of LDS; the
//     16-byte granules of a row are XOR-swizzled so that the MFMA operand
//     reads (ds_read_b128 for K, ds_read_b64_tr_b16 for V) avoid bank
//     conflicts. Rows past the end of a sequence fall outside the buffer
//     descriptor's range and read as zero: their scores are masked to -inf
//     and their P is 0.
//   * Skip vote: every lane forms x = rowmax * sm_scale * log2(e) - m for its
//     query (m = running max before the tile; -inf on the first tile, so x =
//     +inf and the first tile is always kept). A wave keeps the tile if any
//     valid lane has x >= t (one ballot); the work-group ORs the waves'
//     flags through LDS, so d = max_r x_r < t exactly when nobody keeps.
//     The calibration instantiation never skips: each wave reduces x to its
//     maximum (DPP), the work-group takes d = the maximum over waves, and
//     lane k (holding threshold k) counts d < t_k; one row of counts per
//     work-group is written at the end (no atomics).
//   * V_j is fetched only when the vote kept the tile, issued right after
//     the vote so that it lands while the softmax runs; K_{j+1} is fetched
//     as soon as every wave is done reading K_j.
//   * Work-groups are remapped so that each XCD (8 per MI355X, 4 MB L2 each)
//     receives a contiguous range of Q-blocks of the same head: co-resident
//     work-groups stream the same K/V tiles through their XCD's L2.
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

template <int D, int BLK, bool IS_V>
__device__ __forceinline__ void dma_load(const uint16_t* head, uint32_t bytes, uint16_t* lds, int row0,
                                         int64_t stride_tok, int wave, int lane) {
  using SH = Shape<D, BLK>;
  constexpr int RPI = 64 / SH::CH;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)head, 0, bytes, kBufferFlags);
  const int lrow = lane / SH::CH;
#pragma unroll
  for (int i = 0; i < SH::DMA; ++i) {
    const int rin = RPI * (i * SH::NW + wave);  // first row of this instruction within the tile
    const int row = rin + lrow;
    const int chunk = (lane % SH::CH) ^ (IS_V ? swz_v<SH::CH>(row) : swz_k<SH::CH>(row));
    const uint32_t voff = (uint32_t)(((int64_t)lrow * stride_tok + chunk * 8) * 2);
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

// A operand of S^T = K Q^T for key block kb, d step s: K[32 kb + l32][16 s + 8 hl .. + 7]
template <class SH>
__device__ __forceinline__ bf16x8 read_k(const uint16_t* k_lds, int kb, int s, int l32, int hl) {
  const int row = 32 * kb + l32;
  const int gran = row * SH::CH + ((2 * s + hl) ^ swz_k<SH::CH>(row));
  return *reinterpret_cast<const bf16x8*>(k_lds + gran * 8);
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

template <int D, int BLK, bool CALIB>
__global__ __launch_bounds__(2 * BLK, 2) void fwd_kernel(const LaunchParams p) {  // 2*BLK = Shape::NT
  using SH = Shape<D, BLK>;
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[BLK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[BLK * D];
  __shared__ uint64_t vote[SH::NW];
  __shared__ float dvote[SH::NW];  // calibration: each wave's maximum of x

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps tile addressing scalar
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- XCD-aware work-group -> (sequence, head, Q-block) ------------------
  // Hardware dispatches work-group i to XCD i % 8; XCD x takes logical ids
  // [x*q + min(x, r), ...) so each XCD walks consecutive Q-blocks of a head.
  const int G = p.total_wg;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int L = xcd * (G >> 3) + min(xcd, G & 7) + (bid >> 3);
  int b = 0;
  while (b + 1 < p.nseq && p.wg_start[b + 1] <= L) ++b;
  const int tok0 = p.tok_start[b];
  const int S = p.tok_start[b + 1] - tok0;
  const int nQ = (S + BLK - 1) / BLK;
  const int rem = L - p.wg_start[b];
  const int h = rem / nQ;
  // causal: the longest Q-blocks (most KV tiles) are dispatched first
  const int qb = p.causal ? nQ - 1 - (rem - h * nQ) : rem - h * nQ;
  const int nK = p.causal ? qb + 1 : nQ;
  const int row = p.wg_start[b] + h * nQ + qb;  // (sequence, head, Q-block) index of count-table rows
  const int H = p.num_heads;
  const int64_t head_off = (int64_t)tok0 * p.stride_tok + (int64_t)h * p.stride_head;
  const uint16_t* kbase = p.k + head_off;
  const uint16_t* vbase = p.v + head_off;

  const uint32_t head_bytes = head_extent<D>(S, p.stride_tok);
  dma_load<D, BLK, false>(kbase, head_bytes, k_lds, 0, p.stride_tok, wave, lane);

  // ---- Q fragment: B operand of S^T = K Q^T, held for the whole loop ------
  const int qrow = qb * BLK + wave * 32 + l32;
  const bool qvalid = qrow < S;
  bf16x8 qf[SH::DS];
  {
    const uint16_t* qp = p.q + head_off + (int64_t)(qvalid ? qrow : 0) * p.stride_tok + 8 * hl;
#pragma unroll
    for (int s = 0; s < SH::DS; ++s) {
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (qvalid) raw = *reinterpret_cast<const uint4*>(qp + 16 * s);
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  const float c2 = p.scale_log2;
  const float t = CALIB ? 0.0f : p.t_bh[b * H + h];
  const int ncal = CALIB ? p.ncal : 0;
  const float my_t = (CALIB && lane < ncal) ? p.cal_t[lane] : INFINITY;  // lane k holds threshold k
  int ncount = 0;

  float m_true = -INFINITY;  // running max of the method (log2 units), updated on kept tiles
  float m_use = -INFINITY;   // exponent base, m_use <= m_true < m_use + slack
  float l = 0.0f;            // partial row sum over this lane's keys
  floatx16 acc[SH::MB];
#pragma unroll
  for (int mb = 0; mb < SH::MB; ++mb) acc[mb] = floatx16{};
  int skipped = 0;

  // V^T operand read positions (ds_read_b64_tr_b16): row within a 16-key
  // step and byte offset within the row, before the swizzle.
  const int tr_row = 4 * hl + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_elem = 4 * (lane & 1);  // element offset inside the granule

  wait_dma();
  __syncthreads();

  for (int j = 0; j < nK; ++j) {
    const int nvalid = min(BLK, S - j * BLK);

    // ---- S^T = K_j Q^T (always paid) -------------------------------------
    // operands of step s + 1 are read from LDS while step s multiplies
    floatx16 sc[SH::KB];
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb) sc[kb] = floatx16{};
    bf16x8 ka[2][SH::KB];
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb) ka[0][kb] = read_k<SH>(k_lds, kb, 0, l32, hl);
#pragma unroll
    for (int s = 0; s < SH::DS; ++s) {
      if (s + 1 < SH::DS) {
#pragma unroll
        for (int kb = 0; kb < SH::KB; ++kb) ka[(s + 1) & 1][kb] = read_k<SH>(k_lds, kb, s + 1, l32, hl);
      }
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb)
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s & 1][kb], qf[s], sc[kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // keys past the sequence end; causal: keys after this lane's query (diagonal tile)
    const int kmax = (p.causal && j == qb) ? min(nvalid, wave * 32 + l32 + 1) : nvalid;
    if (p.causal ? j == qb : nvalid < BLK) {
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= kmax) sc[kb][r] = -INFINITY;
        }
    }

    // ---- tile row max and the skip vote ----------------------------------
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    float rowmax, x;
    tile_margin(xhalf_max(mx), c2, m_true, rowmax, x);  // m_true = -inf gives x = +inf
    if (!qvalid) x = -INFINITY;
    if constexpr (CALIB) {
      // d = max over valid rows; "some row has x >= t_k" is exactly d >= t_k
      const float dw = wave_max(x);
      if (lane == 0) dvote[wave] = dw;
    } else {
      const bool kw = wave_any(x >= t);
      if (lane == 0) vote[wave] = kw ? 1ull : 0ull;
    }
    __syncthreads();  // votes visible; every wave is done reading K_j and V_{j-1}

    bool keep;
    if constexpr (CALIB) {
      float d = dvote[0];
#pragma unroll
      for (int w = 1; w < SH::NW; ++w) d = fmaxf(d, dvote[w]);
      ncount += d < my_t ? 1 : 0;  // lanes >= ncal hold +inf and are never written out
      keep = true;
    } else {
      uint64_t all = vote[0];
#pragma unroll
      for (int w = 1; w < SH::NW; ++w) all |= vote[w];
      keep = __builtin_amdgcn_readfirstlane(all != 0 ? 1 : 0) != 0;  // work-group uniform
      skipped += keep ? 0 : 1;
      if (p.tile_mask != nullptr && tid == 0)
        p.tile_mask[((int64_t)((p.seq_abs0 + b) * H + h) * p.mask_nq + qb) * p.mask_nk + j] = keep ? 0 : 1;
    }

    if (j + 1 < nK) dma_load<D, BLK, false>(kbase, head_bytes, k_lds, (j + 1) * BLK, p.stride_tok, wave, lane);
    bf16x8 pb[SH::KS];
    if (keep) {
      dma_load<D, BLK, true>(vbase, head_bytes, v_lds, j * BLK, p.stride_tok, wave, lane);

      // ---- online softmax (log2 domain), overlapping the V fetch ---------
      m_true = fmaxf(m_true, rowmax);
      if (wave_any(rowmax > m_use + kRescaleSlack)) {
        const float m_new = fmaxf(m_use, rowmax);
        const float alpha = fast_exp2(m_use - m_new);  // 0 when m_use was -inf
        l *= alpha;
#pragma unroll
        for (int mb = 0; mb < SH::MB; ++mb) acc[mb] *= alpha;
        m_use = m_new;
      }
      const float nm = -m_use;
#pragma unroll
      for (int s = 0; s < SH::KS; ++s) {
        floatx8 e;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          e[r] = fast_exp2(fmaf(sc[s >> 1][8 * (s & 1) + r], c2, nm));
          l += e[r];
        }
        pb[s] = __builtin_convertvector(e, bf16x8);
      }
    }
    wait_dma();
    __syncthreads();  // K_{j+1} and V_j visible

    if (keep) {
      // ---- O^T += V_j^T P^T ----------------------------------------------
      // V^T operands are read two 16-key steps ahead of their MFMAs (3-deep
      // register ring, fully unrolled); sched_barrier keeps the schedule.
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
  }

  // ---- epilogue ---------------------------------------------------------
  const float inv = 1.0f / xhalf_sum(l);
  if (qvalid) {
    uint16_t* op = p.o + head_off + (int64_t)qrow * p.stride_tok;
#pragma unroll
    for (int mb = 0; mb < SH::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 f = {acc[mb][4 * g] * inv, acc[mb][4 * g + 1] * inv, acc[mb][4 * g + 2] * inv,
                           acc[mb][4 * g + 3] * inv};
        const bf16x4 o4 = __builtin_convertvector(f, bf16x4);
        *reinterpret_cast<bf16x4*>(op + 32 * mb + 8 * g + 4 * hl) = o4;
      }
  }
  if constexpr (CALIB) {
    if (wave == 0 && lane < ncal) p.counts[(p.wg_abs0 + row) * ncal + lane] = ncount;
    if (tid == 0) p.tiles[p.wg_abs0 + row] = nK;
  } else {
    if (tid == 0) {
      const int64_t bh = (int64_t)(p.seq_abs0 + b) * H + h;
      if (p.skipped_bh != nullptr) atomicAdd((unsigned long long*)&p.skipped_bh[bh], (unsigned long long)skipped);
      if (p.total_bh != nullptr) atomicAdd((unsigned long long*)&p.total_bh[bh], (unsigned long long)nK);
    }
  }
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
                                          int64_t stride_tok, int wave, int lane) {
  using SH = Shape8<D, BLK>;
  constexpr int RPI = 64 / SH::CH;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)head, 0, bytes, kBufferFlags);
  const int lrow = lane / SH::CH;
#pragma unroll
  for (int i = 0; i < SH::DMA; ++i) {
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

template <int D, int BLK, bool CALIB>
__global__ __launch_bounds__(2 * BLK, 2) void fwd_kernel_fp8(const LaunchParams p) {
  using SH = Shape8<D, BLK>;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[BLK * D];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds[BLK * D];
  __shared__ uint64_t vote[SH::NW];
  __shared__ float dvote[SH::NW];  // calibration: each wave's maximum of x

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  const int G = p.total_wg;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int L = xcd * (G >> 3) + min(xcd, G & 7) + (bid >> 3);
  int b = 0;
  while (b + 1 < p.nseq && p.wg_start[b + 1] <= L) ++b;
  const int tok0 = p.tok_start[b];
  const int S = p.tok_start[b + 1] - tok0;
  const int nQ = (S + BLK - 1) / BLK;
  const int rem = L - p.wg_start[b];
  const int h = rem / nQ;
  const int qb = p.causal ? nQ - 1 - (rem - h * nQ) : rem - h * nQ;
  const int nK = p.causal ? qb + 1 : nQ;
  const int row = p.wg_start[b] + h * nQ + qb;
  const int H = p.num_heads;
  const int64_t head_off = (int64_t)tok0 * p.stride_tok + (int64_t)h * p.stride_head;  // elements = bytes
  const uint8_t* q8 = reinterpret_cast<const uint8_t*>(p.q);
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + head_off;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + head_off;
  const uint32_t head_bytes = head_extent8<D>(S, p.stride_tok);

  dma_load8<D, BLK, false>(kbase, head_bytes, k_lds, 0, p.stride_tok, wave, lane);

  // Q fragment: B operand of S^T = K Q^T: query qrow, d bytes [64 s + 32 hl, +32)
  const int qrow = qb * BLK + wave * 32 + l32;
  const bool qvalid = qrow < S;
  intx8 qf[SH::DS];
  {
    const uint8_t* qp = q8 + head_off + (int64_t)(qvalid ? qrow : 0) * p.stride_tok + 32 * hl;
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

  const float c2 = p.scale_log2;  // includes scale_q * scale_k
  const float t = CALIB ? 0.0f : p.t_bh[b * H + h];
  const int ncal = CALIB ? p.ncal : 0;
  const float my_t = (CALIB && lane < ncal) ? p.cal_t[lane] : INFINITY;  // lane k holds threshold k
  int ncount = 0;
  float m_true = -INFINITY, m_use = -INFINITY, l = 0.0f;
  floatx16 acc[SH::MB];
#pragma unroll
  for (int mb = 0; mb < SH::MB; ++mb) acc[mb] = floatx16{};
  int skipped = 0;

  // V^T transposing-read sources: source lane (2e + c) of each 16-lane group
  // supplies key slot e of the read, columns 16 g + 8 c of the 32-wide block.
  int tr_off[4], tr_sw[4];
  {
    const int e = (lane & 15) >> 1, c = lane & 1, g = (lane & 31) >> 4;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int key = 32 * (tt >> 1) + 16 * (tt & 1) + 8 * (e >> 2) + 4 * hl + (e & 3);
      tr_off[tt] = key * (SH::CH * 16) + g * 16 + 8 * c;
      tr_sw[tt] = swz_v8<SH::CH>(key);
    }
  }

  wait_dma();
  __syncthreads();

  for (int j = 0; j < nK; ++j) {
    const int nvalid = min(BLK, S - j * BLK);
    floatx16 sc[SH::KB];
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb) sc[kb] = floatx16{};
#pragma unroll
    for (int s = 0; s < SH::DS; ++s) {
      intx8 ka[SH::KB];
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb) ka[kb] = read_k8<SH>(k_lds, kb, s, l32, hl);
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb)
        sc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[kb], qf[s], sc[kb], 0, 0, 0, kE8M0One, 0,
                                                                 kE8M0One);
    }
    const int kmax = (p.causal && j == qb) ? min(nvalid, wave * 32 + l32 + 1) : nvalid;
    if (p.causal ? j == qb : nvalid < BLK) {
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= kmax) sc[kb][r] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    float rowmax, x;
    tile_margin(xhalf_max(mx), c2, m_true, rowmax, x);
    if (!qvalid) x = -INFINITY;
    if constexpr (CALIB) {
      const float dw = wave_max(x);
      if (lane == 0) dvote[wave] = dw;
    } else {
      const bool kw = wave_any(x >= t);
      if (lane == 0) vote[wave] = kw ? 1ull : 0ull;
    }
    __syncthreads();

    bool keep;
    if constexpr (CALIB) {
      float d = dvote[0];
#pragma unroll
      for (int w = 1; w < SH::NW; ++w) d = fmaxf(d, dvote[w]);
      ncount += d < my_t ? 1 : 0;
      keep = true;
    } else {
      uint64_t all = vote[0];
#pragma unroll
      for (int w = 1; w < SH::NW; ++w) all |= vote[w];
      keep = __builtin_amdgcn_readfirstlane(all != 0 ? 1 : 0) != 0;
      skipped += keep ? 0 : 1;
      if (p.tile_mask != nullptr && tid == 0)
        p.tile_mask[((int64_t)((p.seq_abs0 + b) * H + h) * p.mask_nq + qb) * p.mask_nk + j] = keep ? 0 : 1;
    }

    if (j + 1 < nK) dma_load8<D, BLK, false>(kbase, head_bytes, k_lds, (j + 1) * BLK, p.stride_tok, wave, lane);
    intx8 pb[SH::KS];
    if (keep) {
      dma_load8<D, BLK, true>(vbase, head_bytes, v_lds, j * BLK, p.stride_tok, wave, lane);
      m_true = fmaxf(m_true, rowmax);
      if (wave_any(rowmax > m_use + kRescaleSlack)) {
        const float m_new = fmaxf(m_use, rowmax);
        const float alpha = fast_exp2(m_use - m_new);
        l *= alpha;
#pragma unroll
        for (int mb = 0; mb < SH::MB; ++mb) acc[mb] *= alpha;
        m_use = m_new;
      }
      const float nm = -m_use;
      // P^T for 64-key step s: byte 16 u + r is score register r of key block 2 s + u
#pragma unroll
      for (int s = 0; s < SH::KS; ++s)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int kb = 2 * s + (w >> 2);
          const int r0 = 4 * (w & 3);
          float e0 = fast_exp2(fmaf(sc[kb][r0], c2, nm));
          float e1 = fast_exp2(fmaf(sc[kb][r0 + 1], c2, nm));
          float e2 = fast_exp2(fmaf(sc[kb][r0 + 2], c2, nm));
          float e3 = fast_exp2(fmaf(sc[kb][r0 + 3], c2, nm));
          l += (e0 + e1) + (e2 + e3);
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, word, true);
          pb[s][w] = word;
        }
    }
    wait_dma();
    __syncthreads();

    if (keep) {
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
  }

  const float inv = p.v_scale / xhalf_sum(l);
  if (qvalid) {
    uint16_t* op = p.o + head_off + (int64_t)qrow * p.stride_tok;
#pragma unroll
    for (int mb = 0; mb < SH::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 f = {acc[mb][4 * g] * inv, acc[mb][4 * g + 1] * inv, acc[mb][4 * g + 2] * inv,
                           acc[mb][4 * g + 3] * inv};
        const bf16x4 o4 = __builtin_convertvector(f, bf16x4);
        *reinterpret_cast<bf16x4*>(op + 32 * mb + 8 * g + 4 * hl) = o4;
      }
  }
  if constexpr (CALIB) {
    if (wave == 0 && lane < ncal) p.counts[(p.wg_abs0 + row) * ncal + lane] = ncount;
    if (tid == 0) p.tiles[p.wg_abs0 + row] = nK;
  } else {
    if (tid == 0) {
      const int64_t bh = (int64_t)(p.seq_abs0 + b) * H + h;
      if (p.skipped_bh != nullptr) atomicAdd((unsigned long long*)&p.skipped_bh[bh], (unsigned long long)skipped);
      if (p.total_bh != nullptr) atomicAdd((unsigned long long*)&p.total_bh[bh], (unsigned long long)nK);
    }
  }
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

template <int D, int BLK, bool CALIB>
__global__ __launch_bounds__(2 * BLK, 2) void fwd_kernel_mxqk(const LaunchParams p) {
  using SH = Shape<D, BLK>;   // bf16 V tile, softmax, P.V
  using S8 = Shape8<D, BLK>;  // e4m3 K tile, S^T
  constexpr int SROW = D / 32;  // scale bytes per row
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[BLK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[BLK * D];
  __shared__ uint64_t vote[SH::NW];
  __shared__ float dvote[SH::NW];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  const int G = p.total_wg;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int L = xcd * (G >> 3) + min(xcd, G & 7) + (bid >> 3);
  int b = 0;
  while (b + 1 < p.nseq && p.wg_start[b + 1] <= L) ++b;
  const int tok0 = p.tok_start[b];
  const int S = p.tok_start[b + 1] - tok0;
  const int nQ = (S + BLK - 1) / BLK;
  const int rem = L - p.wg_start[b];
  const int h = rem / nQ;
  const int qb = p.causal ? nQ - 1 - (rem - h * nQ) : rem - h * nQ;
  const int nK = p.causal ? qb + 1 : nQ;
  const int row = p.wg_start[b] + h * nQ + qb;
  const int H = p.num_heads;
  const int64_t head_off = (int64_t)tok0 * p.stride_tok + (int64_t)h * p.stride_head;  // elements
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + head_off;
  const uint16_t* vbase = p.v + head_off;
  const uint32_t k_bytes = head_extent8<D>(S, p.stride_tok);
  const uint32_t v_bytes = head_extent<D>(S, p.stride_tok);
  const int64_t sc_off = (int64_t)tok0 * p.bs_tok + (int64_t)h * p.bs_head;
  const uint32_t sc_bytes = S > 0 ? (uint32_t)((int64_t)(S - 1) * p.bs_tok + SROW) : 0u;
  const __amdgpu_buffer_rsrc_t ks_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k_bscale + sc_off), 0, sc_bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t qs_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.q_bscale + sc_off), 0, sc_bytes, kBufferFlags);

  // K tile 0 and the scale rows of its keys (lane: key 32 kb + l32; the
  // host keeps (S + BLK) * bs_tok within 32 bits)
  const uint32_t sc_lane = (uint32_t)(l32 * p.bs_tok);
  const uint32_t sc_blk = (uint32_t)(32 * p.bs_tok);  // one 32-key block
  dma_load8<D, BLK, false>(kbase, k_bytes, k_lds, 0, p.stride_tok, wave, lane);
  uint32_t ks[S8::KB];
#pragma unroll
  for (int kb = 0; kb < S8::KB; ++kb) ks[kb] = load_scale_row<D>(ks_rsrc, sc_lane, kb * sc_blk);

  // Q fragment (B operand): query qrow, d bytes [64 s + 16 hl, +16) and
  // [64 s + 32 + 16 hl, +16), and the scale of its MX block 2 s + hl
  const int qrow = qb * BLK + wave * 32 + l32;
  const bool qvalid = qrow < S;
  intx8 qf[S8::DS];
  uint32_t qsc[S8::DS];
  {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + head_off + (int64_t)(qvalid ? qrow : 0) * p.stride_tok +
                        16 * hl;
#pragma unroll
    for (int s = 0; s < S8::DS; ++s) {
      uint4 a = make_uint4(0u, 0u, 0u, 0u), c = make_uint4(0u, 0u, 0u, 0u);
      if (qvalid) {
        a = *reinterpret_cast<const uint4*>(qp + 64 * s);
        c = *reinterpret_cast<const uint4*>(qp + 64 * s + 32);
      }
      qf[s] = intx8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
    }
    const uint32_t qs = load_scale_row<D>(qs_rsrc, sc_lane, (uint32_t)((qb * BLK + wave * 32) * p.bs_tok));
#pragma unroll
    for (int s = 0; s < S8::DS; ++s) qsc[s] = qs >> (8 * (2 * s + hl));  // byte 0: this lane's block
  }

  const float c2 = p.scale_log2;
  const float t = CALIB ? 0.0f : p.t_bh[b * H + h];
  const int ncal = CALIB ? p.ncal : 0;
  const float my_t = (CALIB && lane < ncal) ? p.cal_t[lane] : INFINITY;
  int ncount = 0;
  float m_true = -INFINITY, m_use = -INFINITY, l = 0.0f;
  floatx16 acc[SH::MB];
#pragma unroll
  for (int mb = 0; mb < SH::MB; ++mb) acc[mb] = floatx16{};
  int skipped = 0;
  const int tr_row = 4 * hl + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_elem = 4 * (lane & 1);

  wait_dma();
  __syncthreads();

  for (int j = 0; j < nK; ++j) {
    const int nvalid = min(BLK, S - j * BLK);

    // ---- S^T = K_j Q^T with the block scales (always paid) ---------------
    floatx16 sc[SH::KB];
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb) sc[kb] = floatx16{};
#pragma unroll
    for (int s = 0; s < S8::DS; ++s) {
      intx8 ka[S8::KB];
#pragma unroll
      for (int kb = 0; kb < S8::KB; ++kb) ka[kb] = read_k8_mx<S8>(k_lds, kb, s, l32, hl);
#pragma unroll
      for (int kb = 0; kb < S8::KB; ++kb)
        sc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[kb], qf[s], sc[kb], 0, 0, 0,
                                                                 (int)(ks[kb] >> (8 * (2 * s + hl))), 0, (int)qsc[s]);
    }
    const int kmax = (p.causal && j == qb) ? min(nvalid, wave * 32 + l32 + 1) : nvalid;
    if (p.causal ? j == qb : nvalid < BLK) {
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= kmax) sc[kb][r] = -INFINITY;
        }
    }

    // ---- tile row max and the skip vote ----------------------------------
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    float rowmax, x;
    tile_margin(xhalf_max(mx), c2, m_true, rowmax, x);
    if (!qvalid) x = -INFINITY;
    if constexpr (CALIB) {
      const float dw = wave_max(x);
      if (lane == 0) dvote[wave] = dw;
    } else {
      const bool kw = wave_any(x >= t);
      if (lane == 0) vote[wave] = kw ? 1ull : 0ull;
    }
    __syncthreads();  // votes visible; every wave is done reading K_j and V_{j-1}

    bool keep;
    if constexpr (CALIB) {
      float d = dvote[0];
#pragma unroll
      for (int w = 1; w < SH::NW; ++w) d = fmaxf(d, dvote[w]);
      ncount += d < my_t ? 1 : 0;
      keep = true;
    } else {
      uint64_t all = vote[0];
#pragma unroll
      for (int w = 1; w < SH::NW; ++w) all |= vote[w];
      keep = __builtin_amdgcn_readfirstlane(all != 0 ? 1 : 0) != 0;
      skipped += keep ? 0 : 1;
      if (p.tile_mask != nullptr && tid == 0)
        p.tile_mask[((int64_t)((p.seq_abs0 + b) * H + h) * p.mask_nq + qb) * p.mask_nk + j] = keep ? 0 : 1;
    }

    if (j + 1 < nK) {
      dma_load8<D, BLK, false>(kbase, k_bytes, k_lds, (j + 1) * BLK, p.stride_tok, wave, lane);
#pragma unroll
      for (int kb = 0; kb < S8::KB; ++kb)
        ks[kb] = load_scale_row<D>(ks_rsrc, sc_lane, (uint32_t)((j + 1) * BLK * p.bs_tok) + kb * sc_blk);
    }
    bf16x8 pb[SH::KS];
    if (keep) {
      dma_load<D, BLK, true>(vbase, v_bytes, v_lds, j * BLK, p.stride_tok, wave, lane);
      m_true = fmaxf(m_true, rowmax);
      if (wave_any(rowmax > m_use + kRescaleSlack)) {
        const float m_new = fmaxf(m_use, rowmax);
        const float alpha = fast_exp2(m_use - m_new);
        l *= alpha;
#pragma unroll
        for (int mb = 0; mb < SH::MB; ++mb) acc[mb] *= alpha;
        m_use = m_new;
      }
      const float nm = -m_use;
#pragma unroll
      for (int s = 0; s < SH::KS; ++s) {
        floatx8 e;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          e[r] = fast_exp2(fmaf(sc[s >> 1][8 * (s & 1) + r], c2, nm));
          l += e[r];
        }
        pb[s] = __builtin_convertvector(e, bf16x8);
      }
    }
    wait_dma();
    __syncthreads();  // K_{j+1}, its scales and V_j visible

    if (keep) {
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
  }

  const float inv = 1.0f / xhalf_sum(l);
  if (qvalid) {
    uint16_t* op = p.o + head_off + (int64_t)qrow * p.stride_tok;
#pragma unroll
    for (int mb = 0; mb < SH::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 f = {acc[mb][4 * g] * inv, acc[mb][4 * g + 1] * inv, acc[mb][4 * g + 2] * inv,
                           acc[mb][4 * g + 3] * inv};
        const bf16x4 o4 = __builtin_convertvector(f, bf16x4);
        *reinterpret_cast<bf16x4*>(op + 32 * mb + 8 * g + 4 * hl) = o4;
      }
  }
  if constexpr (CALIB) {
    if (wave == 0 && lane < ncal) p.counts[(p.wg_abs0 + row) * ncal + lane] = ncount;
    if (tid == 0) p.tiles[p.wg_abs0 + row] = nK;
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
  if (p.fp8) {
    using SH = Shape8<D, BLK>;
    hipLaunchKernelGGL((fwd_kernel_fp8<D, BLK, CALIB>), dim3(p.total_wg), dim3(SH::NT), 0, stream, p);
  } else if (p.mxqk) {
    using SH = Shape<D, BLK>;
    hipLaunchKernelGGL((fwd_kernel_mxqk<D, BLK, CALIB>), dim3(p.total_wg), dim3(SH::NT), 0, stream, p);
  } else {
    using SH = Shape<D, BLK>;
    hipLaunchKernelGGL((fwd_kernel<D, BLK, CALIB>), dim3(p.total_wg), dim3(SH::NT), 0, stream, p);
  }
  return (int)hipGetLastError();
}

int grid_for(int64_t n) {
  int64_t blocks = (n + 255) / 256;
  return (int)(blocks < 4096 ? (blocks < 1 ? 1 : blocks) : 4096);
}

}  // namespace

bool supported(int head_dim, int block) {
  return (head_dim == 64 || head_dim == 128) && (block == 64 || block == 128);
}

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
