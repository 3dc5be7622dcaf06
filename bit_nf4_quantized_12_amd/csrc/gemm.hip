// Dequant-in-LDS bf16 MFMA GEMM on the frozen NF4 weight, with the rank-r
// LoRA product fused into the epilogue.
//
// "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com),
// "Method": the stored weight is dequantised to BFloat16 and multiplied in
// 16-bit. Forward (Y = X W~^T + (sT) B^T) and the input gradient
// (dX = dY W~ + (sU) A, the weight used "transposed") share this kernel; the
// LoRA side follows "QLoRA: Efficient Fine-Tuning of Quantized Language
// Models" (mbrenndoerfer.com), section "Low-Rank Adaptation (LoRA)".
//
// Tile 128 x 128 outputs, 64-deep reduction steps, 4 wave64 in 2 x 2, each
// wave 64 x 64 outputs = 4 x 4 v_mfma_f32_16x16x32_bf16 tiles. Per step the
// activation tile (bf16) is copied to LDS and the weight tile is unpacked
// from 4-bit codes in registers, scaled by its block constant c^ and written
// to LDS as bf16; LDS is double buffered (one barrier per step). Rows are
// padded to 72 elements so the 16-lane column reads of the MFMA operands hit
// 64 distinct banks.
#include "launch.hpp"

namespace qlora {



namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDP = 72;

// 8 bf16 of row `row`, columns [col, col+8) of a [rows, ld] matrix; zeros
// outside [0, nrows) x [0, ncols). `vec` means ld % 8 == 0 (16-byte rows).
__device__ __forceinline__ uint4 load_row8(const uint16_t* __restrict__ base, int64_t ld, int row,
                                           int nrows, int col, int ncols, bool vec) {
  if (row >= nrows) return make_uint4(0, 0, 0, 0);
  const uint16_t* p = base + (int64_t)row * ld + col;
  if (vec && col + 8 <= ncols) return *reinterpret_cast<const uint4*>(p);
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (col + i < ncols) ? p[i] : 0u;
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// 8 codes (one word) -> 8 bf16 of W~ = bf16(q[code] * chat), as 4 packed pairs.
__device__ __forceinline__ void dequant8(uint32_t word, float chat, const float* __restrict__ sq,
                                         uint32_t o[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = __fmul_rn(sq[(word >> (8 * i)) & 15u], chat);
    const float b = __fmul_rn(sq[(word >> (8 * i + 4)) & 15u], chat);
    o[i] = pack_bf16(a, b);
  }
}

template <bool TW, bool LORA>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmParams p) {
  __shared__ __align__(16) uint16_t sA[2][BM * LDP];
  __shared__ __align__(16) uint16_t sB[2][BN * LDP];
  __shared__ float sq[16];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  const int n0 = blockIdx.x * BN;  // output column tile
  const int m0 = blockIdx.y * BM;  // output row tile
  if (tid < 16) sq[tid] = p.lv.q[tid];

  const bool vec = (p.Kred & 7) == 0;
  const int nk = (p.Kred + BK - 1) / BK;

  uint4 ra[4];   // activation prefetch
  uint4 rw;      // 32 codes
  float chat;    // their block constant

  auto prefetch = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = tid + 256 * c;
      const int row = id >> 3, col8 = id & 7;
      ra[c] = load_row8(p.act, p.Kred, m0 + row, p.M, k0 + 8 * col8, p.Kred, vec);
    }
    int64_t n, col;
    if (!TW) {  // W rows are output columns; one block per row per step
      n = n0 + (tid >> 1);
      col = k0 + 32 * (tid & 1);
    } else {    // W rows are the reduction; 2 blocks per row per step
      n = k0 + l;
      col = n0 + 32 * w;
    }
    if (n < p.wN && col < p.wK) {
      const int64_t e = n * p.wK + col;
      rw = *reinterpret_cast<const uint4*>(p.codes + (e >> 1));
      chat = block_scale(p.c2, p.c1, e >> 6);
    } else {
      rw = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
      chat = 0.0f;
    }
  };

  auto store_lds = [&](int st) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = tid + 256 * c;
      const int row = id >> 3, col8 = id & 7;
      *reinterpret_cast<uint4*>(&sA[st][row * LDP + 8 * col8]) = ra[c];
    }
    uint32_t o[16];
    dequant8(rw.x, chat, sq, o + 0);
    dequant8(rw.y, chat, sq, o + 4);
    dequant8(rw.z, chat, sq, o + 8);
    dequant8(rw.w, chat, sq, o + 12);
    if (!TW) {
      uint16_t* dst = &sB[st][(tid >> 1) * LDP + 32 * (tid & 1)];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint4*>(dst + 8 * c) = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    } else {
      // transpose into [output column][reduction]: element i of this lane's
      // 32 is W~[k0 + l][n0 + 32 w + i]
      uint16_t* dst = &sB[st][(32 * w) * LDP + l];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dst[(2 * i) * LDP] = (uint16_t)(o[i] & 0xFFFFu);
        dst[(2 * i + 1) * LDP] = (uint16_t)(o[i] >> 16);
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  __syncthreads();  // sq ready
  prefetch(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) prefetch(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = lds_load8(reinterpret_cast<const __bf16*>(&sA[st][(wm * 64 + 16 * i + (l & 15)) * LDP + 32 * kk + 8 * (l >> 4)]));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = lds_load8(reinterpret_cast<const __bf16*>(&sB[st][(wn * 64 + 16 * j + (l & 15)) * LDP + 32 * kk + 8 * (l >> 4)]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_lds(st ^ 1);
    __syncthreads();
  }

  // LoRA epilogue: acc += lora_l[rows, :] . lora_r[cols, :]^T
  if (LORA) {
    for (int kr = 0; kr < p.rp; kr += 32) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = load_row8(p.lora_l, p.rp, m0 + wm * 64 + 16 * i + (l & 15), p.M, kr + 8 * (l >> 4), p.rp, true);
        a[i] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v = load_row8(p.lora_r, p.rp, n0 + wn * 64 + 16 * j + (l & 15), p.Nout, kr + 8 * (l >> 4), p.rp, true);
        b[j] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + 16 * j + (l & 15);
      if (col >= p.Nout) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm * 64 + 16 * i + 4 * (l >> 4) + v;
        if (row < p.M) {
          const __bf16 h = (__bf16)acc[i][j][v];
          p.out[(int64_t)row * p.Nout + col] = __builtin_bit_cast(uint16_t, h);
        }
      }
    }
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, bool transposed_w, hipStream_t s) {
  dim3 grid((p.Nout + BN - 1) / BN, (p.M + BM - 1) / BM);
  const bool lora = p.lora_l != nullptr;
  if (transposed_w) {
    if (lora) hipLaunchKernelGGL((gemm_kernel<true, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_kernel<true, false>), grid, dim3(256), 0, s, p);
  } else {
    if (lora) hipLaunchKernelGGL((gemm_kernel<false, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_kernel<false, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace qlora
