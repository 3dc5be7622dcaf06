// Few-token forward (M <= 16): Y = X W~^T + s T B^T, bound by reading the
// 4-bit weight from HBM.
//
// "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com),
// "Method": dequantise to BFloat16, multiply in 16-bit. With at most 16
// tokens each weight is used at most 16 times, so the kernel streams the
// codes once: every lane unpacks its 8 codes straight into the B operand of
// a v_mfma_f32_16x16x32_bf16 (no LDS staging), the X rows (padded to 16 with
// zeros) are the A operand. A workgroup owns 64 weight rows and a slice of
// K; its 4 waves split the slice and meet in LDS. Slices are summed, and the
// LoRA term added, by gemv_finalize.
#include "launch.hpp"

namespace qlora {
namespace {

__global__ __launch_bounds__(256) void gemv_kernel(const uint16_t* __restrict__ X,
                                                    const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ c2,
                                                    const float* __restrict__ c1, int N, int K,
                                                    int M, int kslice, float* __restrict__ part,
                                                    Levels lv) {
  __shared__ float sq[16];
  __shared__ float red[4][4][16][17];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  if (tid < 16) sq[tid] = lv.q[tid];
  __syncthreads();
  const int n0 = blockIdx.x * 64;
  const int ks = blockIdx.y;
  const int kbeg = ks * kslice;
  const int kend = min(K, kbeg + kslice);

  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int xr = l & 15;
  for (int k = kbeg + 32 * w; k < kend; k += 128) {
    const int col = k + 8 * (l >> 4);
    uint4 xv = make_uint4(0, 0, 0, 0);
    if (xr < M) xv = *reinterpret_cast<const uint4*>(X + (int64_t)xr * K + col);
    const bf16x8 a = __builtin_bit_cast(bf16x8, xv);
    uint32_t cw[4];
    float chat[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = n0 + 16 * t + (l & 15);
      if (n < N) {
        const int64_t e = (int64_t)n * K + col;
        cw[t] = *reinterpret_cast<const uint32_t*>(codes + (e >> 1));
        chat[t] = block_scale(c2, c1, e >> 6);
      } else {
        cw[t] = 0x77777777u;
        chat[t] = 0.0f;
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = __fmul_rn(sq[(cw[t] >> (8 * i)) & 15u], chat[t]);
        const float x1 = __fmul_rn(sq[(cw[t] >> (8 * i + 4)) & 15u], chat[t]);
        o[i] = pack_bf16(x0, x1);
      }
      const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
      acc[t] = mfma16(a, b, acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[w][t][4 * (l >> 4) + v][l & 15] = acc[t][v];
  __syncthreads();
  // 4 tiles x 16 rows x 16 columns = 1024 sums
  float* dst = part + (int64_t)ks * M * N;
  for (int idx = tid; idx < 1024; idx += 256) {
    const int t = idx >> 8, m = (idx >> 4) & 15, c = idx & 15;
    const int n = n0 + 16 * t + c;
    if (m < M && n < N)
      dst[(int64_t)m * N + n] = red[0][t][m][c] + red[1][t][m][c] + red[2][t][m][c] + red[3][t][m][c];
  }
}

// Y[m][n] = bf16( sum_s part[s][m][n] + scale * sum_j T[m][j] B[n][j] )
__global__ __launch_bounds__(256) void gemv_finalize_kernel(const float* __restrict__ part,
                                                             int nsplit, int M, int N,
                                                             const float* __restrict__ T,
                                                             const uint16_t* __restrict__ B, int r,
                                                             float scale, uint16_t* __restrict__ Y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * N) return;
  const int64_t m = idx / N, n = idx % N;
  float v = 0.0f;
  for (int s = 0; s < nsplit; ++s) v += part[(int64_t)s * M * N + idx];
  float lo = 0.0f;
  for (int j = 0; j < r; ++j) lo = __builtin_fmaf(T[m * r + j], bf16lo(B[n * r + j]), lo);
  const __bf16 h = (__bf16)(v + scale * lo);
  Y[idx] = __builtin_bit_cast(uint16_t, h);
}

}  // namespace

hipError_t launch_gemv(const uint16_t* X, const uint8_t* codes, const uint8_t* c2, const float* c1,
                       int N, int K, int M, int nsplit, float* part, hipStream_t s) {
  const int kslice = ((K + nsplit - 1) / nsplit + 63) / 64 * 64;
  dim3 grid((N + 63) / 64, nsplit);
  hipLaunchKernelGGL(gemv_kernel, grid, dim3(256), 0, s, X, codes, c2, c1, N, K, M, kslice, part,
                     host_levels());
  return hipGetLastError();
}

hipError_t launch_gemv_finalize(const float* part, int nsplit, int M, int N, const float* T,
                                const uint16_t* B, int r, float scale, uint16_t* Y, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  hipLaunchKernelGGL(gemv_finalize_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     part, nsplit, M, N, T, B, r, scale, Y);
  return hipGetLastError();
}

}  // namespace qlora
