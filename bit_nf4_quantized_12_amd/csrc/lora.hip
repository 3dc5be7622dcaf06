// The rank-r side of the LoRA linear layer.
//
// "QLoRA: Efficient Fine-Tuning of Quantized Language Models"
// (mbrenndoerfer.com), section "Low-Rank Adaptation (LoRA)": the adapter
// update is B A with A r x d and B d x r; "QLoRA: Efficient Finetuning of
// Quantized LLMs" (inquiringlines.com), abstract: gradients are
// backpropagated through the frozen 4-bit weight into the adapters.
//
// Kernels:
//   proj     P = L R^T over a slice of the reduction (T = X A^T, U = dY B),
//            float32 partial sums, no LDS traffic beyond a final reduction.
//   finalize sums the slices: float32 P [M, r] and bf16(scale * P) padded to
//            rp columns (the operand of the GEMM epilogue).
//   grad     G = P^T Q over a slice of the M rows (dA = s U^T X,
//            dB^T = s T^T dY): Q rows are transposed in registers with
//            v_perm (no LDS), P is split into bf16 hi + lo so the float32
//            intermediate keeps ~16 bits of precision in the MFMA.
//   grad_reduce  sums the M slices in a fixed order (deterministic), scales
//            and writes bf16 (optionally transposed).
//   relayout small copies: transpose / zero-pad of A and B.
#include "launch.hpp"

namespace qlora {
namespace {

__device__ __forceinline__ uint4 load8_masked(const uint16_t* __restrict__ base, int64_t ld,
                                              int64_t row, int64_t nrows, int64_t col,
                                              int64_t ncols, bool vec) {
  if (row >= nrows || col >= ncols) return make_uint4(0, 0, 0, 0);
  const uint16_t* p = base + row * ld + col;
  if (vec && col + 8 <= ncols) return *reinterpret_cast<const uint4*>(p);
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (col + i < ncols) ? p[i] : 0u;
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// P[split][M][rp] = L[M, Kr] R[r, Kr]^T over reduction slice `split`.
// KW = waves sharing one 16-row tile (each takes a quarter of the slice);
// with KW = 1 every wave owns its own 16 rows.
template <int KW>
__global__ __launch_bounds__(256) void proj_kernel(const uint16_t* __restrict__ L,
                                                    const uint16_t* __restrict__ R, int M, int Kr,
                                                    int r, int rp, int kslice,
                                                    float* __restrict__ part) {
  __shared__ float red[(KW > 1) ? 4 * 16 * 256 : 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int rows_per_wg = 16 * (4 / KW);
  const int m0 = blockIdx.x * rows_per_wg + 16 * (w / KW);
  const int ks = blockIdx.y;
  const int kbeg = ks * kslice;
  const int kend = min(Kr, kbeg + kslice);
  const int nt = rp >> 4;
  const bool vec = (Kr & 7) == 0;

  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k = kbeg + 32 * (w % KW); k < kend; k += 32 * KW) {
    const int col = k + 8 * (l >> 4);
    const bf16x8 a = __builtin_bit_cast(bf16x8, load8_masked(L, Kr, m0 + (l & 15), M, col, kend, vec));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < nt) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, load8_masked(R, Kr, 16 * j + (l & 15), r, col, kend, vec));
        acc[j] = mfma16(a, b, acc[j]);
      }
    }
  }

  // D[i][j]: lane holds rows 4 (l >> 4) + v, column l & 15 of each 16 x 16 tile
  if (KW == 1) {
    float* dst = part + (int64_t)ks * M * rp;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= nt) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + 4 * (l >> 4) + v;
        if (row < M) dst[(int64_t)row * rp + 16 * j + (l & 15)] = acc[j][v];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= nt) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(w * 16 + 4 * (l >> 4) + v) * 256 + 16 * j + (l & 15)] = acc[j][v];
    }
    __syncthreads();
    float* dst = part + (int64_t)ks * M * rp;
    for (int idx = tid; idx < 16 * rp; idx += 256) {
      const int i = idx / rp, j = idx % rp;
      const float s = red[(0 * 16 + i) * 256 + j] + red[(1 * 16 + i) * 256 + j] +
                      red[(2 * 16 + i) * 256 + j] + red[(3 * 16 + i) * 256 + j];
      const int row = m0 + i;
      if (row < M) dst[(int64_t)row * rp + j] = s;
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// Same product for Kr % 64 == 0, streamed: a workgroup owns 64 rows of L, a
// reduction slice and one 64-column block z of the result (rows 64 z .. of
// R); each 64-deep step brings an L tile (64 x 64) and an R tile (64 x 64)
// into LDS by LDS-DMA, four stages deep, so that ~48 KB per workgroup are in
// flight. Wave w computes rows 16 w .. 16 w + 15 against the block's 64
// columns (4 MFMA tiles). The rp_total columns come in segments of zper
// blocks (r_seg valid rows of R each): block z belongs to segment
// g = z / zper, reads L + g segL and rows 64 (z % zper) .. of R + g segR
// (row pitches ldL, ldR). One segment (zper >= blocks) is the plain
// product; several are grouped linears sharing L or slicing L and R by
// columns. Rows of R past r_seg and rows of L past M are clamped (their
// products land in columns / rows nobody reads).
constexpr int PJ_STAGES = 4;
__device__ __forceinline__ int pj_swz(int R) { return lds_swz(R); }

// Workgroup -> (x, y, z) of a gx x gy x gz grid launched as 8 ceil(gx gy gz
// / 8) workgroups in one dimension. When the z blocks read the same input
// tile (zshare: the rank blocks of one row tile), workgroup g, which runs on
// XCD g % 8, takes item g / 8 of XCD i's contiguous range [i per,
// (i + 1) per) of the order with z fastest, then x, then y: the blocks that
// share a tile run at the same time on one XCD and fetch it from HBM once,
// through that XCD's L2 (as a 3-D grid they ran in separate rounds, each
// reading it again). Otherwise the order is the 3-D grid's own (x fastest,
// then y, then z, dealt round robin over the XCDs), which streams
// neighbouring column tiles together and measured faster there.
struct Wg3 {
  int x, y, z;
  bool ok;
};
__device__ __forceinline__ Wg3 xcd_wg3(int gx, int gy, int gz, bool zshare) {
  const int total = gx * gy * gz;
  Wg3 r;
  if (zshare && gz > 1) {
    const int per = (total + 7) / 8;
    const int u = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    r.ok = u < total;
    r.z = u % gz;
    const int rest = u / gz;
    r.x = rest % gx;
    r.y = rest / gx;
  } else {
    const int u = (int)blockIdx.x;
    r.ok = u < total;
    r.x = u % gx;
    const int rest = u / gx;
    r.y = rest % gy;
    r.z = rest / gy;
  }
  return r;
}
inline unsigned xcd_grid(int gx, int gy, int gz) { return 8u * (unsigned)((gx * gy * gz + 7) / 8); }

__global__ __launch_bounds__(256) void proj_stream_kernel(const uint16_t* __restrict__ L, int64_t ldL,
                                                           int64_t segL, const uint16_t* __restrict__ R,
                                                           int64_t ldR, int64_t segR, int zper, int M,
                                                           int Kr, int r_seg, int rp_total, int kslice,
                                                           int nsplit, float* __restrict__ part) {
  __shared__ __align__(16) uint16_t sm[PJ_STAGES][2][64 * 64];
  const Wg3 wg = xcd_wg3((M + 63) / 64, nsplit, rp_total / 64, segL == 0);
  if (!wg.ok) return;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = wg.x * 64;
  const int ks = wg.y;
  const int z = wg.z;
  const int kbeg = ks * kslice;
  const int nsteps = max(0, min(Kr - kbeg, kslice)) / 64;
  const int zs = z / zper, zb = z - zs * zper;
  const int rvalid = min(64, r_seg - 64 * zb);
  L += zs * segL;
  R += zs * segR + (int64_t)64 * zb * ldR;

  // DMA lanes: wave w fills rows 16 w .. 16 w + 15 of both tiles, two 1 KB
  // instructions each; lane i -> row 16 w + 8 j + (i >> 3), physical chunk
  // i & 7 = logical chunk (i & 7) ^ swz(row)
  uint32_t loff[2], roff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * w + 8 * j + (l >> 3);
    const int c = (l & 7) ^ pj_swz(row);
    loff[j] = (uint32_t)(min(m0 + row, M - 1) * ldL + 8 * c) * 2u;
    roff[j] = (uint32_t)(min(row, rvalid - 1) * ldR + 8 * c) * 2u;
  }
  auto issue = [&](int step) {
    const int slot = step % PJ_STAGES;
    const int k = kbeg + 64 * min(step, nsteps - 1);
    const char* lb = reinterpret_cast<const char*>(L) + (size_t)k * 2;
    const char* rb = reinterpret_cast<const char*>(R) + (size_t)k * 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(lb + loff[j]), (lds_void_t*)(&sm[slot][0][(16 * w + 8 * j) * 64]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(rb + roff[j]), (lds_void_t*)(&sm[slot][1][(16 * w + 8 * j) * 64]), 16, 0, 0);
    }
  };

  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ck0 = 8 * ((0 + (l >> 4)) ^ pj_swz(l & 15));
  const int ck1 = 8 * ((4 + (l >> 4)) ^ pj_swz(l & 15));

  if (nsteps > 0) {
#pragma unroll
    for (int st = 0; st < PJ_STAGES - 1; ++st) issue(st);
    for (int step = 0; step < nsteps; ++step) {
      // 4 DMA instructions per thread per stage and no other vector memory
      // op in the loop: the oldest stage has landed once at most
      // (stages - 2) * 4 remain outstanding. LDS reads of the previous step
      // are complete (lgkmcnt 0) before any wave passes the barrier and
      // refills their slot. A plain s_barrier: __syncthreads would also wait
      // for the in-flight prefetches.
      __builtin_amdgcn_s_waitcnt((4 * (PJ_STAGES - 2)) | (7 << 4) | (0 << 8));
      __builtin_amdgcn_s_barrier();
      issue(step + PJ_STAGES - 1);  // refills the slot read one step ago
      const uint16_t* lt = sm[step % PJ_STAGES][0];
      const uint16_t* rt = sm[step % PJ_STAGES][1];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ck = kk ? ck1 : ck0;
        const bf16x8 a = lds_load8(reinterpret_cast<const __bf16*>(lt + (16 * w + (l & 15)) * 64 + ck));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 b = lds_load8(reinterpret_cast<const __bf16*>(rt + (16 * j + (l & 15)) * 64 + ck));
          acc[j] = mfma16(a, b, acc[j]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // drain the overrun prefetches before exit
  }
  float* dst = part + (int64_t)ks * M * rp_total + 64 * z;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + 16 * w + 4 * (l >> 4) + v;
      if (row < M) dst[(int64_t)row * rp_total + 16 * j + (l & 15)] = acc[j][v];
    }
}

// Sum the reduction slices: P32 [M, r] float32 (may be null) and
// Ps [M, rp] = bf16(scale * P), zero in columns r .. rp-1. A thread takes 4
// adjacent columns (rp % 4 == 0); slices are added in order, from 0.
__device__ __forceinline__ float4 sum_slices(const float* __restrict__ part, int nsplit, int64_t slice, int64_t i4) {
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float4* p4 = reinterpret_cast<const float4*>(part + i4);
  const int64_t st = slice / 4;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float4 x = p4[s * st];
    v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
  }
  return v;
}

__device__ __forceinline__ void store_hi_lo(uint16_t* __restrict__ Ph, uint16_t* __restrict__ Pl, int64_t i4,
                                            const float (&sv)[4]) {
  uint16_t h[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 b = (__bf16)sv[e];
    h[e] = __builtin_bit_cast(uint16_t, b);
    lo[e] = __builtin_bit_cast(uint16_t, (__bf16)(sv[e] - (float)b));
  }
  *reinterpret_cast<uint2*>(Ph + i4) = make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
  if (Pl) *reinterpret_cast<uint2*>(Pl + i4) = make_uint2(lo[0] | (uint32_t)lo[1] << 16, lo[2] | (uint32_t)lo[3] << 16);
}

__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ part, int nsplit,
                                                        int M, int Mp, int r, int rp, float scale,
                                                        float* __restrict__ P32,
                                                        uint16_t* __restrict__ Ph,
                                                        uint16_t* __restrict__ Pl) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= (int64_t)Mp * rp) return;
  const int64_t m = i4 / rp;
  const int j0 = (int)(i4 % rp);
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (m < M) v = sum_slices(part, nsplit, (int64_t)M * rp, i4);
  const float vv[4] = {v.x, v.y, v.z, v.w};
  float sv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool ok = m < M && j0 + e < r;
    if (ok && P32) P32[m * r + j0 + e] = vv[e];
    sv[e] = ok ? scale * vv[e] : 0.0f;
  }
  store_hi_lo(Ph, Pl, i4, sv);
}

// part[s][j][c] = sum over rows m of slice s of P[m][j] * Q[m][c],
// j in [64 jc, 64 jc + 64), c in [128 cg, 128 cg + 128).
__global__ __launch_bounds__(256) void grad_kernel(const float* __restrict__ P,
                                                    const uint16_t* __restrict__ Q, int M, int C,
                                                    int r, int rp, int mchunk,
                                                    float* __restrict__ part) {
  __shared__ float red[2 * 64 * 129];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int cg = blockIdx.x, s = blockIdx.y, jc = blockIdx.z;
  const int mbeg = s * mchunk;
  const int mend = min(M, mbeg + mchunk);
  const int c0 = cg * 128 + 8 * (l & 15);
  const int g = l >> 4;
  const bool vec = (C & 7) == 0;

  f32x4 acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int m = mbeg + 32 * w; m < mend; m += 128) {
    uint4 rq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) rq[i] = load8_masked(Q, C, m + 8 * g + i, mend, c0, C, vec);
    // B operand for column c0 + cc: Q[m + 8g + i][c0 + cc], i = 0..7
    bf16x8 bq[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x0 = (&rq[2 * i].x)[e], x1 = (&rq[2 * i + 1].x)[e];
        lo[i] = __builtin_amdgcn_perm(x1, x0, 0x05040100u);  // element 2e of rows 2i, 2i+1
        hi[i] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);  // element 2e+1
      }
      bq[2 * e] = __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3]));
      bq[2 * e + 1] = __builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j = jc * 64 + 16 * jt + (l & 15);
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = m + 8 * g + i;
        pv[i] = (j < r && row < mend) ? P[(int64_t)row * r + j] : 0.0f;
      }
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 h0 = (__bf16)pv[2 * i], h1 = (__bf16)pv[2 * i + 1];
        const float r0 = pv[2 * i] - (float)h0, r1 = pv[2 * i + 1] - (float)h1;
        hw[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        lw[i] = pack_bf16(r0, r1);
      }
      const bf16x8 ah = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      const bf16x8 al = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        acc[jt][cc] = mfma16(ah, bq[cc], acc[jt][cc]);
        acc[jt][cc] = mfma16(al, bq[cc], acc[jt][cc]);
      }
    }
  }

  // reduce the four waves: 3,2 -> LDS, 0,1 add; 1 -> LDS, 0 adds
  auto put = [&](int slot) {
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[slot * 64 * 129 + l * 129 + jt * 32 + cc * 4 + v] = acc[jt][cc][v];
  };
  auto add = [&](int slot) {
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[jt][cc][v] += red[slot * 64 * 129 + l * 129 + jt * 32 + cc * 4 + v];
  };
  if (w >= 2) put(w - 2);
  __syncthreads();
  if (w < 2) add(w);
  __syncthreads();
  if (w == 1) put(0);
  __syncthreads();
  if (w == 0) {
    add(0);
    float* dst = part + (int64_t)s * rp * C;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = jc * 64 + 16 * jt + 4 * (l >> 4) + v;
        if (j >= rp) continue;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const int c = c0 + cc;
          if (c < C) dst[(int64_t)j * C + c] = acc[jt][cc][v];
        }
      }
  }
}

// P [M, r] float32 -> Pt_hi, Pt_lo [rp, Mp] bf16 with Pt_hi + Pt_lo ~ P^T
// to ~16 bits (hi = bf16(p), lo = bf16(p - hi)); zero for j >= r or m >= M.
// part[s][j][c] (TRANS: part[s][c][j]) = sum over the rows m of slice s of
// P[m][j] Q[m][c], with P = hi + lo, two bf16 planes [Mp, rp] (rows past M
// zero) and Q [M, C] bf16, C % 8 == 0. A workgroup (8 waves) owns 64 j
// (block jc) x 128 c; each 64-row step brings the Q tile (64 x 128, 256 B
// rows) and the two P tiles (64 x 64, 128 B rows) into LDS by LDS-DMA, four
// stages deep. Both operands are row-major in m, the reduction index, so
// MFMA fragments are read with the LDS transpose load ds_read_b64_tr_b16:
// within each group of 16 lanes, lane s addresses 4 consecutive elements of
// row 8 g + (s >> 2) (+ 4 for the second half), columns c0 + 4 (s & 3), and
// lane o receives column c0 + o of those rows. No transposed copy of either
// input is made. Wave w owns j rows 16 (w & 3) .. + 15 and columns
// 64 (w >> 2) .. + 63 (4 MFMA tiles, two waves per SIMD); the hi and lo
// products go into the same fp32 accumulators. Q rows past M are clamped (P
// is zero there), columns past C too (unstored).
constexpr int GT_STAGES = 4;
constexpr int GT_STAGE = 8192 + 4096 + 4096;  // elements: Q | P hi | P lo
// 16-byte chunk swizzles that keep the transposed fragment reads free of
// LDS bank conflicts (measured): 128 B rows (P) and 256 B rows (Q).
__device__ __forceinline__ int gt_swz_p(int R) { return (((R >> 1) & 1) << 1) ^ (((R >> 3) & 1) << 2); }
__device__ __forceinline__ int gt_swz_q(int R) { return ((R & 3) << 1) ^ (((R >> 3) & 1) << 3); }

// s_waitcnt immediate: vmcnt <= vm (6 bits: [3:0] and [15:14]), lgkmcnt 0,
// expcnt not waited on
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (0 << 8); }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s_t;
__device__ __forceinline__ uint2 tr_load(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)p));
}
__device__ __forceinline__ bf16x8 frag(uint2 a, uint2 b) {
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// One 64-row step on an LDS stage: all fragments are read first, then the
// 16 MFMAs. The stage pointer is a restrict parameter: once inlined, its
// loads carry alias-scope information telling the wait-count pass that they
// do not read the stages being filled by the LDS-DMA in flight (otherwise it
// forces vmcnt(0) before them; the kernel's own wait covers the stage read).
__device__ __forceinline__ void gt_step(const uint16_t* __restrict__ st, const int (&aoff)[2][2],
                                        const int (&boff)[2][2][4], f32x4 (&acc)[4]) {
  uint2 ah[2][2], al[2][2], bq[2][4][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ah[kk][h] = tr_load(st + aoff[kk][h]);
      al[kk][h] = tr_load(st + 4096 + aoff[kk][h]);
#pragma unroll
      for (int b = 0; b < 4; ++b) bq[kk][b][h] = tr_load(st + boff[kk][h][b]);
    }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const bf16x8 fh = frag(ah[kk][0], ah[kk][1]), fl = frag(al[kk][0], al[kk][1]);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bf16x8 fb = frag(bq[kk][b][0], bq[kk][b][1]);
      acc[b] = mfma16(fh, fb, acc[b]);
      acc[b] = mfma16(fl, fb, acc[b]);
    }
  }
}

template <bool TRANS>
__global__ __launch_bounds__(512) void grad_tr_kernel(const uint16_t* __restrict__ Ph,
                                                       const uint16_t* __restrict__ Pl,
                                                       const uint16_t* __restrict__ Q, int M,
                                                       int Mp, int C, int rp, int mchunk, int segC,
                                                       int rseg, int nsplit, float* __restrict__ part) {
  extern __shared__ __align__(16) uint16_t gsm[];
  const Wg3 wg = xcd_wg3((C + 127) / 128, nsplit, rseg / 64, true);
  if (!wg.ok) return;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jb = w & 3, ch = w >> 2;
  const int cbase = wg.x * 128;
  const int s = wg.y;
  const int jc = wg.z;
  const int mbeg = s * mchunk;
  const int nsteps = max(0, min(Mp - mbeg, mchunk)) / 64;

  // DMA lanes. Q: instruction q of wave w fills rows 8 w + 4 q .. + 3, lane i
  // the physical chunk i & 15 of row 8 w + 4 q + (i >> 4). P: wave w fills
  // rows 8 w .. + 7, lane i chunk i & 7 of row 8 w + (i >> 3).
  int qrow[2];
  uint32_t qcol[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    qrow[q] = 8 * w + 4 * q + (l >> 4);
    qcol[q] = (uint32_t)min(cbase + 8 * ((l & 15) ^ gt_swz_q(qrow[q])), C - 8) * 2u;
  }
  // segmented (grouped linears): the columns of segment cbase / segC pair
  // with plane columns (cbase / segC) rseg .. + rseg only; otherwise segC = 0
  // and the plane block is jc alone. The result has rseg rows j.
  const int pcol0 = (segC ? (cbase / segC) * rseg : 0) + jc * 64;
  const int prow = 8 * w + (l >> 3);
  const uint32_t poff = (uint32_t)((mbeg + prow) * rp + pcol0 + 8 * ((l & 7) ^ gt_swz_p(prow))) * 2u;
  auto issue = [&](int step) {
    uint16_t* st = gsm + (step % GT_STAGES) * GT_STAGE;
    const int ms = min(step, nsteps - 1) * 64;
    const char* qb = reinterpret_cast<const char*>(Q);
    const char* hb = reinterpret_cast<const char*>(Ph) + (size_t)ms * rp * 2;
    const char* lb = reinterpret_cast<const char*>(Pl) + (size_t)ms * rp * 2;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = min(mbeg + ms + qrow[q], M - 1);  // rows past M: P is zero there
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(qb + ((size_t)row * C * 2 + qcol[q])),
                                       (lds_void_t*)(st + (8 * w + 4 * q) * 128), 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(hb + poff), (lds_void_t*)(st + 8192 + 8 * w * 64), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(lb + poff), (lds_void_t*)(st + 12288 + 8 * w * 64), 16, 0, 0);
  };

  // transposed-read addresses (elements, within a stage) for the two row
  // halves h of a 32-row substep kk: lane (g = l >> 4, si = l & 15)
  const int g = l >> 4, si = l & 15;
  int aoff[2][2], boff[2][2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int R = 32 * kk + 8 * g + 4 * h + (si >> 2);
      const int ca = 16 * jb + 4 * (si & 3);
      aoff[kk][h] = 8192 + R * 64 + 8 * ((ca >> 3) ^ gt_swz_p(R)) + (ca & 7);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int cb = 64 * ch + 16 * b + 4 * (si & 3);
        boff[kk][h][b] = R * 128 + 8 * ((cb >> 3) ^ gt_swz_q(R)) + (cb & 7);
      }
    }

  f32x4 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nsteps > 0) {
#pragma unroll
    for (int st = 0; st < GT_STAGES - 1; ++st) issue(st);
    for (int step = 0; step < nsteps; ++step) {
      // 4 DMA instructions per thread per stage, nothing else in flight: the
      // oldest stage has landed once at most (stages - 2) * 4 remain. LDS
      // reads of the previous step are complete before any wave passes the
      // barrier and refills their slot (a plain s_barrier: __syncthreads
      // would also wait for the prefetches in flight).
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * (GT_STAGES - 2)));
      __builtin_amdgcn_s_barrier();
      issue(step + GT_STAGES - 1);
      gt_step(gsm + (step % GT_STAGES) * GT_STAGE, aoff, boff, acc);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  // D layout: lane holds j = 16 jb + 4 g + v, c = cbase + 64 ch + 16 b + si
  const int j0 = jc * 64 + 16 * jb + 4 * g;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int c = cbase + 64 * ch + 16 * b + si;
    if (c >= C) continue;
    if (!TRANS) {
#pragma unroll
      for (int v = 0; v < 4; ++v) part[((int64_t)s * rseg + j0 + v) * C + c] = acc[b][v];
    } else {
      *reinterpret_cast<float4*>(part + ((int64_t)s * C + c) * rseg + j0) =
          make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    }
  }
}

// out = bf16(scale * sum_s part[s][j][c]); j < r, c < C. Transposed: out[c][j].
__global__ __launch_bounds__(256) void grad_reduce_kernel(const float* __restrict__ part,
                                                           int nsplit, int r, int rp, int C,
                                                           float scale, bool transpose, bool part_trans,
                                                           uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)r * C) return;
  int64_t j, c;
  if (transpose) { c = idx / r; j = idx % r; } else { j = idx / C; c = idx % C; }
  // partials are [s][j][c], or [s][c][j] when produced for a transposed output
  const int64_t off = part_trans ? c * rp + j : j * C + c;
  float v = 0.0f;
  for (int s = 0; s < nsplit; ++s) v += part[(int64_t)s * rp * C + off];
  const __bf16 h = (__bf16)(scale * v);
  out[idx] = __builtin_bit_cast(uint16_t, h);
}

// out[i][j] (pitch ldo, i < rows_out, j < cols_out) = in[j][i] if transpose
// else in[i][j], zero outside the input [rows_in, cols_in] (pitch ldi).
__global__ __launch_bounds__(256) void relayout_kernel(const uint16_t* __restrict__ in,
                                                        int64_t rows_in, int64_t cols_in,
                                                        int64_t ldi, bool transpose,
                                                        uint16_t* __restrict__ out,
                                                        int64_t rows_out, int64_t cols_out,
                                                        int64_t ldo) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows_out * cols_out) return;
  const int64_t i = idx / cols_out, j = idx % cols_out;
  const int64_t si = transpose ? j : i, sj = transpose ? i : j;
  out[i * ldo + j] = (si < rows_in && sj < cols_in) ? in[si * ldi + sj] : (uint16_t)0;
}

// The backward's two small transposes in one launch: Bt [r, N] = B^T and
// At [K, rp] = A^T with zero columns r .. rp-1 (when At is not null).
__global__ __launch_bounds__(256) void transpose2_kernel(const uint16_t* __restrict__ B,
                                                          const uint16_t* __restrict__ A, int N,
                                                          int K, int r, int rA, int rp,
                                                          uint16_t* __restrict__ Bt,
                                                          uint16_t* __restrict__ At) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nb = (int64_t)r * N;
  if (idx < nb) {
    const int64_t j = idx / N, n = idx - j * N;
    Bt[idx] = B[n * r + j];
    return;
  }
  const int64_t ia = idx - nb;
  if (!At || ia >= (int64_t)K * rp) return;
  const int64_t k = ia / rp, j = ia - k * rp;
  At[ia] = j < rA ? A[j * K + k] : (uint16_t)0;
}

// finalize_kernel for the U partials, and in the same launch the hi / lo
// planes of scale * T (T float32 [M, r]) into Th / Tl, both [Mp, rp].
__global__ __launch_bounds__(256) void finalize2_kernel(const float* __restrict__ part, int nsplit,
                                                         int M, int Mp, int r, int rp, float scale,
                                                         float* __restrict__ P32,
                                                         uint16_t* __restrict__ Ph,
                                                         uint16_t* __restrict__ Pl,
                                                         const float* __restrict__ T,
                                                         uint16_t* __restrict__ Th,
                                                         uint16_t* __restrict__ Tl) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= (int64_t)Mp * rp) return;
  const int64_t m = i4 / rp;
  const int j0 = (int)(i4 % rp);
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (m < M) v = sum_slices(part, nsplit, (int64_t)M * rp, i4);
  const float vv[4] = {v.x, v.y, v.z, v.w};
  float sv[4], tv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool ok = m < M && j0 + e < r;
    if (ok && P32) P32[m * r + j0 + e] = vv[e];
    sv[e] = ok ? scale * vv[e] : 0.0f;
    tv[e] = ok ? scale * T[m * r + j0 + e] : 0.0f;
  }
  store_hi_lo(Ph, Pl, i4, sv);
  store_hi_lo(Th, Tl, i4, tv);
}

// Both adapter-gradient reductions in one launch: dA [r, C1] from partials
// [s][rp][C1] (first r * C1 / 4 threads) and dB [C2, r] from partials
// [s][C2][rp], each bf16(scale * sum over the slices), the slices added in
// order from 0. A thread takes 4 adjacent partials (16-byte loads, all
// slices' loads issued before the adds); C1 and rp are multiples of 4.
__device__ __forceinline__ float4 sum4(const float* __restrict__ p, int64_t stride, int ns) {
  float4 v = *reinterpret_cast<const float4*>(p);
  int sp = 1;
  for (; sp + 4 <= ns; sp += 4) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const float4*>(p + (sp + u) * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v.x += x[u].x; v.y += x[u].y; v.z += x[u].z; v.w += x[u].w;
    }
  }
  for (; sp < ns; ++sp) {
    const float4 x = *reinterpret_cast<const float4*>(p + sp * stride);
    v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
  }
  return v;
}
__global__ __launch_bounds__(256) void grad_reduce2_kernel(const float* __restrict__ partA, int nsA,
                                                            int C1, uint16_t* __restrict__ dA,
                                                            const float* __restrict__ partB, int nsB,
                                                            int C2, uint16_t* __restrict__ dB, int rA,
                                                            int rpA, int rB, int rpB, float scale) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t na = (int64_t)rA * C1 / 4;
  if (idx < na) {
    const int64_t j = idx / (C1 / 4), c = (idx % (C1 / 4)) * 4;
    const float4 v = sum4(partA + j * C1 + c, (int64_t)rpA * C1, nsA);
    *reinterpret_cast<uint2*>(dA + j * C1 + c) =
        make_uint2(pack_bf16(scale * v.x, scale * v.y), pack_bf16(scale * v.z, scale * v.w));
    return;
  }
  const int64_t ib = idx - na;
  if (ib >= (int64_t)C2 * (rpB / 4)) return;
  const int64_t c = ib / (rpB / 4), j = (ib % (rpB / 4)) * 4;
  if (j >= rB) return;
  const float4 v = sum4(partB + c * rpB + j, (int64_t)C2 * rpB, nsB);
  const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (j + e < rB) dB[c * rB + j + e] = __builtin_bit_cast(uint16_t, (__bf16)(scale * vv[e]));
}

}  // namespace

hipError_t launch_proj_seg(const uint16_t* L, int64_t ldL, int64_t segL, const uint16_t* R, int64_t ldR,
                           int64_t segR, int zper, int M, int Kr, int r_seg, int rp_total, int nsplit, float* part,
                           hipStream_t s) {
  const int kslice = ((Kr + nsplit - 1) / nsplit + 63) / 64 * 64;
  const dim3 grid(xcd_grid((M + 63) / 64, nsplit, rp_total / 64));
  hipLaunchKernelGGL(proj_stream_kernel, grid, dim3(256), 0, s, L, ldL, segL, R, ldR, segR, zper, M, Kr, r_seg,
                     rp_total, kslice, nsplit, part);
  return hipGetLastError();
}

hipError_t launch_proj(const uint16_t* L, const uint16_t* R, int M, int Kr, int r, int rp,
                       int nsplit, float* part, hipStream_t s) {
  if (Kr % 64 == 0) return launch_proj_seg(L, Kr, 0, R, Kr, 0, rp / 64, M, Kr, r, rp, nsplit, part, s);
  const int kslice = ((Kr + nsplit - 1) / nsplit + 31) / 32 * 32;
  if (M <= 16) {
    dim3 grid(1, nsplit);
    hipLaunchKernelGGL(proj_kernel<4>, grid, dim3(256), 0, s, L, R, M, Kr, r, rp, kslice, part);
  } else {
    dim3 grid((M + 63) / 64, nsplit);
    hipLaunchKernelGGL(proj_kernel<1>, grid, dim3(256), 0, s, L, R, M, Kr, r, rp, kslice, part);
  }
  return hipGetLastError();
}

hipError_t launch_finalize(const float* part, int nsplit, int M, int Mp, int r, int rp, float scale,
                           float* P32, uint16_t* Ph, uint16_t* Pl, hipStream_t s) {
  const int64_t total = (int64_t)Mp * rp / 4;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part,
                     nsplit, M, Mp, r, rp, scale, P32, Ph, Pl);
  return hipGetLastError();
}

hipError_t launch_grad(const float* P, const uint16_t* Q, int M, int C, int r, int rp, int nsplit,
                       float* part, hipStream_t s) {
  const int mchunk = ((M + nsplit - 1) / nsplit + 31) / 32 * 32;
  dim3 grid((C + 127) / 128, nsplit, (rp + 63) / 64);
  hipLaunchKernelGGL(grad_kernel, grid, dim3(256), 0, s, P, Q, M, C, r, rp, mchunk, part);
  return hipGetLastError();
}

hipError_t launch_grad_reduce(const float* part, int nsplit, int r, int rp, int C, float scale,
                              bool transpose, bool part_trans, uint16_t* out, hipStream_t s) {
  const int64_t total = (int64_t)r * C;
  hipLaunchKernelGGL(grad_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     part, nsplit, r, rp, C, scale, transpose, part_trans, out);
  return hipGetLastError();
}

hipError_t launch_grad_tr(const uint16_t* Ph, const uint16_t* Pl, const uint16_t* Q, int M, int Mp, int C,
                          int rp, int nsplit, bool trans, float* part, hipStream_t s, int segC, int rseg) {
  if (!segC) rseg = rp;
  const size_t smem = (size_t)GT_STAGES * GT_STAGE * sizeof(uint16_t);
  static std::atomic<uint32_t> lds_ok[2];
  hipError_t e = ensure_lds(reinterpret_cast<const void*>(&grad_tr_kernel<false>), (int)smem, lds_ok[0]);
  if (e == hipSuccess) e = ensure_lds(reinterpret_cast<const void*>(&grad_tr_kernel<true>), (int)smem, lds_ok[1]);
  if (e != hipSuccess) return e;
  const int mchunk = ((Mp + nsplit - 1) / nsplit + 63) / 64 * 64;
  const dim3 grid(xcd_grid((C + 127) / 128, nsplit, rseg / 64));
  if (trans)
    hipLaunchKernelGGL(grad_tr_kernel<true>, grid, dim3(512), smem, s, Ph, Pl, Q, M, Mp, C, rp, mchunk, segC, rseg,
                       nsplit, part);
  else
    hipLaunchKernelGGL(grad_tr_kernel<false>, grid, dim3(512), smem, s, Ph, Pl, Q, M, Mp, C, rp, mchunk, segC, rseg,
                       nsplit, part);
  return hipGetLastError();
}

hipError_t launch_relayout(const uint16_t* in, int64_t rows_in, int64_t cols_in, int64_t ldi,
                           bool transpose, uint16_t* out, int64_t rows_out, int64_t cols_out,
                           int64_t ldo, hipStream_t s) {
  const int64_t total = rows_out * cols_out;
  hipLaunchKernelGGL(relayout_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, in,
                     rows_in, cols_in, ldi, transpose, out, rows_out, cols_out, ldo);
  return hipGetLastError();
}

hipError_t launch_transpose2(const uint16_t* B, const uint16_t* A, int N, int K, int r, int rA, int rp,
                             uint16_t* Bt, uint16_t* At, hipStream_t s) {
  const int64_t total = (int64_t)r * N + (At ? (int64_t)K * rp : 0);
  hipLaunchKernelGGL(transpose2_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, B, A, N, K, r,
                     rA, rp, Bt, At);
  return hipGetLastError();
}

hipError_t launch_finalize2(const float* part, int nsplit, int M, int Mp, int r, int rp, float scale,
                            float* P32, uint16_t* Ph, uint16_t* Pl, const float* T, uint16_t* Th,
                            uint16_t* Tl, hipStream_t s) {
  const int64_t total = (int64_t)Mp * rp / 4;
  hipLaunchKernelGGL(finalize2_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, nsplit, M,
                     Mp, r, rp, scale, P32, Ph, Pl, T, Th, Tl);
  return hipGetLastError();
}

hipError_t launch_grad_reduce2(const float* partA, int nsA, int C1, uint16_t* dA, const float* partB, int nsB,
                               int C2, uint16_t* dB, int rA, int rpA, int rB, int rpB, float scale, hipStream_t s) {
  const int64_t total = (int64_t)rA * C1 / 4 + (int64_t)C2 * (rpB / 4);
  hipLaunchKernelGGL(grad_reduce2_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, partA, nsA,
                     C1, dA, partB, nsB, C2, dB, rA, rpA, rB, rpB, scale);
  return hipGetLastError();
}

}  // namespace qlora
