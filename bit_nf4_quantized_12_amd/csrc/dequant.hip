// Dequantisation of the stored blockwise 4-bit formats (NF4, Int4 or FP4
// levels; double-quantised constants or fp32 block absmax).
//
// "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com),
// "Method": whenever a stored weight is used it is dequantised to BFloat16.
// Per weight: W^ = fp32(q[code] * c^_b) with c^_b = fp32(e4m3(c2_b) * c1_g)
// (c^_b = the stored fp32 absmax without double quantisation);
// the bf16 output is W~ = bf16(W^), round to nearest even.
//
// Each lane turns one 4-byte word of codes (8 weights, inside one block)
// into 32 B (fp32) or 16 B (bf16) of output. The 16 levels sit in LDS, where
// a lookup is conflict free (16 distinct dwords in 16 banks: equal codes
// broadcast). Bandwidth kernel: 0.5 + 1/64 B read and 4 or 2 B written per
// weight. Workgroup b owns one contiguous run of 1024 words (8192 weights):
// step u of its 4 writes words 1024 b + 256 u + thread, so every store
// instruction covers 1 KB (bf16) of consecutive output and a workgroup's
// writes stay within 16 KB. (A grid-stride loop with a lane's words a grid
// apart ran 25 % slower with the same instructions.) The output is written
// with nontemporal stores (streamed once).
#include "launch.hpp"

namespace qlora {
namespace {

template <bool BF16>
__device__ __forceinline__ void emit8(void* __restrict__ out, int64_t e, uint32_t word, float chat,
                                      const float* __restrict__ sq) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = __fmul_rn(sq[(word >> (4 * i)) & 15u], chat);
  if (BF16) {
    uint4 o = make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                         pack_bf16(f[6], f[7]));
    const u32x4 ov = {o.x, o.y, o.z, o.w};
    __builtin_nontemporal_store(ov, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + e));
  } else {
    typedef float f4v __attribute__((ext_vector_type(4)));
    f4v* p = reinterpret_cast<f4v*>(reinterpret_cast<float*>(out) + e);
    const f4v a = {f[0], f[1], f[2], f[3]}, b = {f[4], f[5], f[6], f[7]};
    __builtin_nontemporal_store(a, p);
    __builtin_nontemporal_store(b, p + 1);
  }
}

constexpr int kDqUnroll = 4;                  // words per thread
constexpr int kDqWords = 256 * kDqUnroll;     // words per workgroup

template <bool BF16, bool ABS>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ c2,
                                                       const float* __restrict__ c1,
                                                       const float* __restrict__ absmax, int64_t n,
                                                       void* __restrict__ out, Levels lv) {
  __shared__ float sq[16];
  if (threadIdx.x < 16) sq[threadIdx.x] = lv.q[threadIdx.x];
  __syncthreads();

  const int64_t nwords = n >> 3;  // full 8-weight words
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
  const int64_t w0 = (int64_t)blockIdx.x * kDqWords + threadIdx.x;
  if (w0 + 256 * (kDqUnroll - 1) < nwords) {
    uint32_t wd[kDqUnroll];
    float cs[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) wd[u] = cw[w0 + 256 * u];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) cs[u] = block_const<ABS>(c2, c1, absmax, (w0 + 256 * u) >> 3);
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) emit8<BF16>(out, (w0 + 256 * u) * 8, wd[u], cs[u], sq);
  } else {
    // the last workgroup's partial run
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t wi = w0 + 256 * u;
      if (wi < nwords) emit8<BF16>(out, wi * 8, cw[wi], block_const<ABS>(c2, c1, absmax, wi >> 3), sq);
    }
  }

  // short tail (n % 8 weights), one thread
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t e = nwords * 8; e < n; ++e) {
      const uint32_t code = (codes[e >> 1] >> (4 * (e & 1))) & 15u;
      const float v = __fmul_rn(sq[code], block_const<ABS>(c2, c1, absmax, e >> 6));
      if (BF16) {
        const __bf16 h = (__bf16)v;
        reinterpret_cast<uint16_t*>(out)[e] = __builtin_bit_cast(uint16_t, h);
      } else {
        reinterpret_cast<float*>(out)[e] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* absmax,
                          int64_t n, int codebook, bool bf16_out, void* out, hipStream_t s) {
  int64_t blocks = ((n >> 3) + kDqWords - 1) / kDqWords;  // < 2^31: n <= 2^43 (checked by the caller)
  if (blocks < 1) blocks = 1;
  const Levels& lv = host_levels(codebook);
  const dim3 g((unsigned)blocks), t(256);
  if (bf16_out && absmax)
    hipLaunchKernelGGL((dequant_kernel<true, true>), g, t, 0, s, codes, c2, c1, absmax, n, out, lv);
  else if (bf16_out)
    hipLaunchKernelGGL((dequant_kernel<true, false>), g, t, 0, s, codes, c2, c1, absmax, n, out, lv);
  else if (absmax)
    hipLaunchKernelGGL((dequant_kernel<false, true>), g, t, 0, s, codes, c2, c1, absmax, n, out, lv);
  else
    hipLaunchKernelGGL((dequant_kernel<false, false>), g, t, 0, s, codes, c2, c1, absmax, n, out, lv);
  return hipGetLastError();
}

}  // namespace qlora
