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
// HBM traffic is 0.5 B of codes read and 2 B written per weight.
#include "launch.hpp"

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
    const float w = __fmul_rn(sq[code], block_const<ABS>(c2, c1, absmax, e >> 6));
    const __bf16 h = (__bf16)__fadd_rn(w, __fmul_rn(scale, acc[i]));
    out[e] = __builtin_bit_cast(uint16_t, h);
  }
}

}  // namespace

hipError_t launch_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* absmax, int codebook,
                        const uint16_t* A, const uint16_t* B, int N, int K, int r, float scale, uint16_t* out,
                        hipStream_t s) {
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
