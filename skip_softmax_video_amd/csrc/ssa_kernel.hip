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
//     query rows. D = head dim.
//   * Scores are computed transposed, S^T = K_j Q^T, with
//     v_mfma_f32_32x32x16_bf16: lane l then holds query (l % 32) and 16 keys
//     per 32-key block, so the per-row max and sum are in-register
//     reductions plus one exchange with lane l ^ 32.
//   * The same registers, rounded to bf16, are the B operand of
//     O^T += V_j^T P^T; V_j^T comes straight from the row-major V tile in LDS
//     through ds_read_b64_tr_b16 (4x16 transposing LDS read), so V needs no
//     register transpose. The per-lane key order inside a 16-key MFMA step is
//     permuted identically on both operands (the contraction does not care).
//   * O^T accumulates in registers; lane l owns query (l % 32), so the
//     online-softmax rescale factor and row sum are per-lane scalars.
//   * Skip vote: every lane forms x = rowmax * sm_scale * log2(e) - m for its
//     query (m = running max before the tile, -inf on the first tile, so x =
//     +inf and the first tile is always kept); the wave max goes to LDS and
//     the work-group max d decides for the whole tile: skip iff d < t.
//     The calibration instantiation evaluates d < t_k for up to 64
//     thresholds, one per lane of wave 0, never skips, and writes one row of
//     counts per work-group (no atomics).
//   * K_{j+1} is prefetched into registers before the vote; V_j is read
//     from global memory only after the vote kept the tile.
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

template <int D, int BLK>
struct Shape {
  static constexpr int NW = BLK / 32;     // waves per work-group (32 query rows each)
  static constexpr int NT = NW * 64;      // threads per work-group
  static constexpr int KB = BLK / 32;     // 32-key blocks per KV tile
  static constexpr int DS = D / 16;       // 16-wide d steps of S^T = K Q^T
  static constexpr int MB = D / 32;       // 32-wide d blocks of O^T
  static constexpr int KS = BLK / 16;     // 16-key steps of O^T += V^T P^T
  static constexpr int K_LD = D + 8;      // K row stride in LDS (elements): +16 B
  static constexpr int V_LD = D + 16;     // V row stride in LDS (elements): +32 B
  static constexpr int CH = D / 8;        // 16-byte chunks per row
  static constexpr int LOADS = BLK * CH / NT;  // 16-byte loads per thread per tile
  static_assert(BLK * CH % NT == 0, "tile must split evenly over the threads");
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Load one BLK x D bf16 tile (rows row0.. of the head, row-major, 16 B per
// thread per step, 16 consecutive threads per 256-byte row) into registers;
// rows at or beyond `nvalid` read as zero.
template <int D, int BLK>
__device__ __forceinline__ void load_tile(uint4* r, const uint16_t* base,
                                          int64_t stride_tok, int nvalid, int tid) {
  using SH = Shape<D, BLK>;
#pragma unroll
  for (int i = 0; i < SH::LOADS; ++i) {
    const int c = i * SH::NT + tid;
    const int row = c / SH::CH;
    const int col = (c % SH::CH) * 8;
    r[i] = make_uint4(0u, 0u, 0u, 0u);
    if (row < nvalid) r[i] = *reinterpret_cast<const uint4*>(base + (int64_t)row * stride_tok + col);
  }
}

template <int D, int BLK, int LD>
__device__ __forceinline__ void store_tile(uint16_t* lds, const uint4* r, int tid) {
  using SH = Shape<D, BLK>;
#pragma unroll
  for (int i = 0; i < SH::LOADS; ++i) {
    const int c = i * SH::NT + tid;
    const int row = c / SH::CH;
    const int col = (c % SH::CH) * 8;
    *reinterpret_cast<uint4*>(lds + row * LD + col) = r[i];
  }
}

template <int D, int BLK, bool CALIB>
__global__ __launch_bounds__(2 * BLK) void fwd_kernel(const LaunchParams p) {  // 2*BLK = Shape::NT
  using SH = Shape<D, BLK>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BLK * SH::K_LD];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[BLK * SH::V_LD];
  __shared__ float red[SH::NW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
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
  const int qb = rem - h * nQ;
  const int nK = nQ;
  const int H = p.num_heads;
  const int64_t head_off = (int64_t)tok0 * p.stride_tok + (int64_t)h * p.stride_head;

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
  float tcal = -INFINITY;
  int ncount = 0;
  if (CALIB && lane < p.ncal) tcal = p.cal_t[lane];

  float m = -INFINITY;   // running max, log2 units
  float l = 0.0f;        // partial row sum over this lane's keys
  floatx16 acc[SH::MB];
#pragma unroll
  for (int mb = 0; mb < SH::MB; ++mb) acc[mb] = floatx16{};
  int skipped = 0;

  const uint16_t* kbase = p.k + head_off;
  const uint16_t* vbase = p.v + head_off;
  uint4 regs[SH::LOADS];
  load_tile<D, BLK>(regs, kbase, p.stride_tok, min(BLK, S), tid);
  store_tile<D, BLK, SH::K_LD>(k_lds, regs, tid);
  __syncthreads();

  for (int j = 0; j < nK; ++j) {
    const int nvalid = min(BLK, S - j * BLK);

    // ---- S^T = K_j Q^T (always paid) -------------------------------------
    floatx16 sc[SH::KB];
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb) sc[kb] = floatx16{};
#pragma unroll
    for (int s = 0; s < SH::DS; ++s) {
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(k_lds + (32 * kb + l32) * SH::K_LD + 16 * s + 8 * hl);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc[kb], 0, 0, 0);
      }
    }
    if (nvalid < BLK) {
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= nvalid) sc[kb][r] = -INFINITY;
        }
    }

    // ---- tile row max and the skip vote ----------------------------------
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float rowmax = mx * c2;
    const float x = qvalid ? rowmax - m : -INFINITY;  // m = -inf gives +inf
    const float wx = wave_max(x);
    if (lane == 0) red[wave] = wx;

    // prefetch K_{j+1} while the vote settles
    const bool more = j + 1 < nK;
    if (more) load_tile<D, BLK>(regs, kbase + (int64_t)(j + 1) * BLK * p.stride_tok, p.stride_tok,
                                min(BLK, S - (j + 1) * BLK), tid);
    __syncthreads();  // votes visible; every wave is done reading K_j and V_{j-1}

    float d = red[0];
#pragma unroll
    for (int w = 1; w < SH::NW; ++w) d = fmaxf(d, red[w]);
    bool keep;
    if constexpr (CALIB) {
      ncount += (d < tcal) ? 1 : 0;
      keep = true;
    } else {
      keep = !(d < t);
      skipped += keep ? 0 : 1;
      if (p.tile_mask != nullptr && tid == 0)
        p.tile_mask[((int64_t)((p.seq_abs0 + b) * H + h) * p.mask_nq + qb) * p.mask_nk + j] = keep ? 0 : 1;
    }

    if (more) store_tile<D, BLK, SH::K_LD>(k_lds, regs, tid);
    if (keep) {
      uint4 vr[SH::LOADS];
      load_tile<D, BLK>(vr, vbase + (int64_t)j * BLK * p.stride_tok, p.stride_tok, nvalid, tid);
      store_tile<D, BLK, SH::V_LD>(v_lds, vr, tid);
    }
    __syncthreads();  // K_{j+1} and V_j visible

    if (keep) {
      // ---- online softmax (log2 domain) ----------------------------------
      const float m_new = fmaxf(m, rowmax);
      const float alpha = fast_exp2(m - m_new);  // 0 when m was -inf
      const float nm = -m_new;
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < SH::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(sc[kb][r], c2, nm));
          sc[kb][r] = e;
          ps += e;
        }
      l = l * alpha + ps;
      m = m_new;
#pragma unroll
      for (int mb = 0; mb < SH::MB; ++mb) acc[mb] *= alpha;

      // ---- O^T += V_j^T P^T ----------------------------------------------
      const int tr_row = 4 * hl + ((lane & 15) >> 2);
      const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int s = 0; s < SH::KS; ++s) {
        const floatx8 pf = (s & 1) ? __builtin_shufflevector(sc[s >> 1], sc[s >> 1], 8, 9, 10, 11, 12, 13, 14, 15)
                                   : __builtin_shufflevector(sc[s >> 1], sc[s >> 1], 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 pb = __builtin_convertvector(pf, bf16x8);
#pragma unroll
        for (int mb = 0; mb < SH::MB; ++mb) {
          const uint16_t* vp = v_lds + (16 * s + tr_row) * SH::V_LD + 32 * mb + tr_col;
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vp));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vp + 8 * SH::V_LD));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[mb], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue ---------------------------------------------------------
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt;
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
    if (wave == 0 && lane < p.ncal) p.counts[(p.wg_abs0 + L) * p.ncal + lane] = ncount;
    if (tid == 0) p.tiles[p.wg_abs0 + L] = nK;
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
  using SH = Shape<D, BLK>;
  hipLaunchKernelGGL((fwd_kernel<D, BLK, CALIB>), dim3(p.total_wg), dim3(SH::NT), 0, stream, p);
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
