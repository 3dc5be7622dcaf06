// Merged weight for deployment: Wm = bf16(W^ + scale B A).
//
// "QLoRA: Efficient Fine-Tuning of Quantized Language Models"
// (mbrenndoerfer.com), section "Low-Rank Adaptation (LoRA)": the adapted
// layer computes x_out = (W_q + B A) x_in, so after finetuning the adapters
// can be folded into one dense weight and the layer served without the
// rank-r path. W^ is the exact float32 dequantised weight (any stored
// format); the rank-r sum is float32, j ascending; one rounding to bf16.
//
// A workgroup (256 threads) owns 32 rows x 256 columns: lane k of the tile
// accumulates column k for the 32 rows over 64-deep chunks of the rank. A's
// column k comes straight from global memory (64 loads per chunk, coalesced
// across the wave; A stays in L2 for all row blocks); B's chunk is staged in
// LDS transposed (64 x 32 float32, 8 KB) and read as broadcast 16-byte reads.
// HBM traffic is 0.5 B of codes read and 2 B written per weight. This
// general form serves any K; merge_mfma_kernel below serves K % 64 == 0.
#include "launch.hpp"

// W^ and scale * (B A) are each rounded to float32 before their sum:
// contraction into FMAs is off for the operators written in this file; the
// rank-r sums use explicit FMAs or MFMA.
#pragma clang fp contract(off)

namespace qlora {
namespace {

constexpr int MG_ROWS = 32, MG_COLS = 256, MG_R = 64;  // MG_COLS = threads

template <bool ABS>
__global__ __launch_bounds__(256) void merge_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ c2,
                                                     const float* __restrict__ c1, const float* __restrict__ absmax,
                                                     const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                     int N, int K, int r, float scale, uint16_t* __restrict__ out,
                                                     Levels lv) {
  __shared__ __align__(16) float sB[MG_R][MG_ROWS];  // transposed: [j][row]
  __shared__ float sq[16];
  const int t = threadIdx.x;
  if (t < 16) sq[t] = lv.q[t];
  const int k0 = blockIdx.x * MG_COLS, n0 = blockIdx.y * MG_ROWS;
  const int k = k0 + t;
  const int kc = min(k, K - 1);  // columns past K: clamped read, not stored
  float acc[MG_ROWS];
#pragma unroll
  for (int i = 0; i < MG_ROWS; ++i) acc[i] = 0.0f;

  for (int j0 = 0; j0 < r; j0 += MG_R) {
    const int jn = min(MG_R, r - j0);
    float a[MG_R];
#pragma unroll
    for (int j = 0; j < MG_R; ++j)
      a[j] = j < jn ? __uint_as_float((uint32_t)A[(int64_t)(j0 + j) * K + kc] << 16) : 0.0f;
    __syncthreads();  // the previous chunk's LDS reads are done
    for (int idx = t; idx < MG_ROWS * MG_R; idx += 256) {
      const int i = idx / MG_R, j = idx % MG_R;
      const bool ok = n0 + i < N && j < jn;
      sB[j][i] = ok ? __uint_as_float((uint32_t)B[(int64_t)(n0 + i) * r + j0 + j] << 16) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MG_R; ++j) {
      const float4* bj = reinterpret_cast<const float4*>(sB[j]);
#pragma unroll
      for (int i4 = 0; i4 < MG_ROWS / 4; ++i4) {
        const float4 bv = bj[i4];
        acc[4 * i4 + 0] = __builtin_fmaf(bv.x, a[j], acc[4 * i4 + 0]);
        acc[4 * i4 + 1] = __builtin_fmaf(bv.y, a[j], acc[4 * i4 + 1]);
        acc[4 * i4 + 2] = __builtin_fmaf(bv.z, a[j], acc[4 * i4 + 2]);
        acc[4 * i4 + 3] = __builtin_fmaf(bv.w, a[j], acc[4 * i4 + 3]);
      }
    }
  }
  if (k >= K) return;
#pragma unroll
  for (int i = 0; i < MG_ROWS; ++i) {
    const int n = n0 + i;
    if (n >= N) break;
    const int64_t e = (int64_t)n * K + k;
    const uint32_t code = (codes[e >> 1] >> (4 * (e & 1))) & 15u;
    const float w = sq[code] * block_const<ABS>(c2, c1, absmax, e >> 6);
    const __bf16 h = (__bf16)(w + scale * acc[i]);
    out[e] = __builtin_bit_cast(uint16_t, h);
  }
}

// MFMA form for K % 64 == 0 (every row starts a block): the rank-r product
// B A of a 64-row x 256-column tile on v_mfma_f32_16x16x32_bf16 (bf16
// products are exact in float32; the float32 sums in the hardware's order),
// then the same epilogue rounding as merge_kernel. Per 64-deep rank chunk
// the workgroup (8 wave64) stages B's 64 x 64 tile (waves 4-7) and the
// transposed A chunk (256 k x 64 j, transposed in registers by 8 x 8
// blocks, a column pair at a time straight into LDS; waves 0-3) in LDS; wave w owns rows 16 (w & 3) .. + 15 and
// columns 128 (w >> 2) .. + 127 (8 MFMA tiles). The scaled products then
// pass through LDS as float32 so that each lane finishes 8 adjacent outputs
// of one row with one 16 B store; the lane's codes and block constants are
// fetched before the products. HBM traffic: 0.5 B of codes read and 2 B
// written per weight (A and B stay in L2).
constexpr int MM_ROWS = 64, MM_COLS = 256, MM_J = 64, MM_NT = 512;
constexpr int MM_ITEMS = MM_ROWS * MM_COLS / 8 / MM_NT;  // 8-column output chunks per lane
constexpr int MM_BS = MM_J + 8;     // sB / sAt row stride (bf16): 144 B rows
constexpr int MM_OS = MM_COLS + 4;  // sOut row stride (float32)
constexpr int MM_LDS = MM_ROWS * MM_OS * 4;  // >= (64 + 256) * MM_BS * 2
static_assert((MM_ROWS + MM_COLS) * MM_BS * 2 <= MM_LDS, "staging fits in the output buffer");

// Column c of an 8 x 8 bf16 block whose row e is in[e] (8 columns): the
// 8 rows' elements c, row pairs packed low / high.
__device__ __forceinline__ uint4 column8(const uint4 (&in)[8], int c) {
  uint32_t wd[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t lo = (&in[2 * h].x)[c >> 1], hi = (&in[2 * h + 1].x)[c >> 1];
    wd[h] = __builtin_amdgcn_perm(hi, lo, (c & 1) ? 0x07060302u : 0x05040100u);
  }
  return make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

template <bool ABS>
__global__ __launch_bounds__(MM_NT) __attribute__((amdgpu_waves_per_eu(4))) void merge_mfma_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ c2,
                                                            const float* __restrict__ c1,
                                                            const float* __restrict__ absmax,
                                                            const uint16_t* __restrict__ A,
                                                            const uint16_t* __restrict__ B, int N, int K, int r,
                                                            float scale, uint16_t* __restrict__ out, Levels lv) {
  extern __shared__ __align__(16) unsigned char mm_smem[];
  uint16_t* sB = reinterpret_cast<uint16_t*>(mm_smem);  // [64][MM_BS]
  uint16_t* sAt = sB + MM_ROWS * MM_BS;                 // [256][MM_BS]
  float* sOut = reinterpret_cast<float*>(mm_smem);      // [64][MM_OS], after the products
  __shared__ float sq[16];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k0 = blockIdx.x * MM_COLS, n0 = blockIdx.y * MM_ROWS;
  if (tid < 16) sq[tid] = lv.q[tid];

  // the lane's output chunks: item tid + MM_NT i is row item >> 5, columns
  // 8 (item & 31) .. + 7; codes (one word = 8 weights) and raw constants first
  uint32_t cw[MM_ITEMS], c2b[MM_ITEMS];
  float craw[MM_ITEMS], g1[MM_ITEMS];
#pragma unroll
  for (int i = 0; i < MM_ITEMS; ++i) {
    const int item = tid + MM_NT * i;
    const int n = min(n0 + (item >> 5), N - 1), kk = min(k0 + 8 * (item & 31), K - 8);
    const int64_t e = (int64_t)n * K + kk;  // multiple of 8
    cw[i] = *reinterpret_cast<const uint32_t*>(codes + (e >> 1));
    if (ABS) {
      craw[i] = absmax[e >> 6];
    } else {
      c2b[i] = c2[e >> 6];
      g1[i] = c1[e >> 14];
    }
  }

  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int wr = 16 * (w & 3), wc = 128 * (w >> 2);  // the wave's rows and columns
  const bool astage = w < 4;                          // wave-uniform role
  const int u = tid & 255;
  const int jb = u & 7, kb = u >> 3;                  // A: the 8 x 8 block (j 8 jb.., k 8 kb..)
  const int brow = u >> 2, bj = (u & 3) * 16;         // B: row brow, 16 rank columns from bj
  const int bn = min(n0 + brow, N - 1);
  const int acol = min(k0 + 8 * kb, K - 8);  // columns past K: clamped, not stored
  for (int j0 = 0; j0 < r; j0 += MM_J) {
    __syncthreads();  // the previous chunk's fragment reads are done
    if (astage) {
      uint4 av[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + 8 * jb + e;
        const uint4 v = *reinterpret_cast<const uint4*>(A + (int64_t)min(j, r - 1) * K + acol);
        av[e] = j < r ? v : make_uint4(0, 0, 0, 0);
      }
      // transposed: column c of the block is row 8 kb + c of sAt
#pragma unroll
      for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(sAt + (8 * kb + c) * MM_BS + 8 * jb) = column8(av, c);
    } else {
      uint32_t bw[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + bj + 2 * q;
        const uint32_t x0 = B[(int64_t)bn * r + min(j, r - 1)], x1 = B[(int64_t)bn * r + min(j + 1, r - 1)];
        bw[q] = (j < r ? x0 : 0u) | ((j + 1 < r ? x1 : 0u) << 16);
      }
      *reinterpret_cast<uint4*>(sB + brow * MM_BS + bj) = make_uint4(bw[0], bw[1], bw[2], bw[3]);
      *reinterpret_cast<uint4*>(sB + brow * MM_BS + bj + 8) = make_uint4(bw[4], bw[5], bw[6], bw[7]);
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < MM_J; jj += 32) {
      // row operand: B rows wr + (l & 15), rank slots jj + 8 (l >> 4) ..
      const bf16x8 fa = *reinterpret_cast<const bf16x8*>(sB + (wr + (l & 15)) * MM_BS + jj + 8 * (l >> 4));
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        // column operand: A^T rows (columns k) wc + 16 t + (l & 15), the same rank slots
        const bf16x8 fb =
            *reinterpret_cast<const bf16x8*>(sAt + (wc + 16 * t + (l & 15)) * MM_BS + jj + 8 * (l >> 4));
        acc[t] = mfma16(fa, fb, acc[t]);
      }
    }
  }
  __syncthreads();  // all fragment reads done: sOut overlays the staging
  // D layout: lane holds rows 4 (l >> 4) + v of the wave's 16, column l & 15
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      sOut[(wr + 4 * (l >> 4) + v) * MM_OS + wc + 16 * t + (l & 15)] = scale * acc[t][v];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MM_ITEMS; ++i) {
    const int item = tid + MM_NT * i;
    const int row = item >> 5, kk = k0 + 8 * (item & 31);
    const int n = n0 + row;
    if (n >= N || kk >= K) continue;
    const float4 p0 = *reinterpret_cast<const float4*>(sOut + row * MM_OS + 8 * (item & 31));
    const float4 p1 = *reinterpret_cast<const float4*>(sOut + row * MM_OS + 8 * (item & 31) + 4);
    const float lo[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const float cb = ABS ? craw[i] : e4m3_value(c2b[i]) * g1[i];
    uint32_t hw[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float w0 = sq[(cw[i] >> (8 * h)) & 15u] * cb;
      const float w1 = sq[(cw[i] >> (8 * h + 4)) & 15u] * cb;
      hw[h] = pack_bf16(w0 + lo[2 * h], w1 + lo[2 * h + 1]);
    }
    *reinterpret_cast<uint4*>(out + (int64_t)n * K + kk) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  }
}

}  // namespace

template <bool ABS>
static hipError_t launch_merge_mfma(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* absmax,
                                    int codebook, const uint16_t* A, const uint16_t* B, int N, int K, int r,
                                    float scale, uint16_t* out, hipStream_t s) {
  static std::atomic<uint32_t> lds_ok{0};  // more than 64 KB of LDS needs an opt-in
  const hipError_t e = ensure_lds(reinterpret_cast<const void*>(&merge_mfma_kernel<ABS>), MM_LDS, lds_ok);
  if (e != hipSuccess) return e;
  const dim3 grid((K + MM_COLS - 1) / MM_COLS, (N + MM_ROWS - 1) / MM_ROWS);
  hipLaunchKernelGGL(merge_mfma_kernel<ABS>, grid, dim3(MM_NT), MM_LDS, s, codes, c2, c1, absmax, A, B, N, K, r, scale,
                     out, host_levels(codebook));
  return hipGetLastError();
}

hipError_t launch_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* absmax, int codebook,
                        const uint16_t* A, const uint16_t* B, int N, int K, int r, float scale, uint16_t* out,
                        hipStream_t s) {
  if (K % 64 == 0)
    return absmax ? launch_merge_mfma<true>(codes, c2, c1, absmax, codebook, A, B, N, K, r, scale, out, s)
                  : launch_merge_mfma<false>(codes, c2, c1, absmax, codebook, A, B, N, K, r, scale, out, s);
  const dim3 grid((K + MG_COLS - 1) / MG_COLS, (N + MG_ROWS - 1) / MG_ROWS);
  if (absmax)
    hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(256), 0, s, codes, c2, c1, absmax, A, B, N, K, r, scale, out,
                       host_levels(codebook));
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(256), 0, s, codes, c2, c1, absmax, A, B, N, K, r, scale, out,
                       host_levels(codebook));
  return hipGetLastError();
}

}  // namespace qlora
