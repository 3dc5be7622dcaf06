// Optimizer step of the LoRA adapters with optimizer state in HBM or paged
// out to pinned host memory.
//
// "QLoRA: Efficient Fine-Tuning of Quantized Language Models"
// (mbrenndoerfer.com), section "Paged Optimizers", and "QLoRA: Efficient
// Finetuning of Quantized LLMs", Introduction, contribution (3): optimizer
// state may live in CPU memory while GPU memory is short. The pages name no
// update rule; this is AdamW (bias-corrected moments, decoupled weight
// decay), float32 master weights and moments, bf16 gradients.
//
// The kernel reads and writes the moments through whatever address it is
// given: device memory, or pinned host memory mapped into the GPU's address
// space (then every access crosses the host link; nothing is staged). A
// streaming kernel: per parameter 2 B gradient + 3 x 4 B state read, 3 x 4 B
// written (+ 2 B for the bf16 copy of the updated weight).
#include "launch.hpp"

namespace qlora {
namespace {

typedef float f32v4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void adamw1(float& p, float& m, float& v, float g, const AdamW& a) {
  m = __fadd_rn(__fmul_rn(a.beta1, m), __fmul_rn(a.one_minus_beta1, g));
  v = __fadd_rn(__fmul_rn(a.beta2, v), __fmul_rn(a.one_minus_beta2, __fmul_rn(g, g)));
  const float mh = __fmul_rn(m, a.bc1);
  const float vh = __fmul_rn(v, a.bc2);
  const float upd = __fdiv_rn(mh, __fadd_rn(__fsqrt_rn(vh), a.eps));
  p = __fsub_rn(p, __fmul_rn(a.lr, __fadd_rn(__fmul_rn(a.weight_decay, p), upd)));
}

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, uint16_t* __restrict__ p16,
                                                     const uint16_t* __restrict__ g, float* __restrict__ m,
                                                     float* __restrict__ v, int64_t n, AdamW a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n8 = n >> 3;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 gw = reinterpret_cast<const uint4*>(g)[i];
    f32v4* p4 = reinterpret_cast<f32v4*>(p) + 2 * i;
    f32v4* m4 = reinterpret_cast<f32v4*>(m) + 2 * i;
    f32v4* v4 = reinterpret_cast<f32v4*>(v) + 2 * i;
    f32v4 pp[2] = {p4[0], p4[1]}, mm[2] = {m4[0], m4[1]}, vv[2] = {v4[0], v4[1]};
    const uint32_t gh[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gf = (e & 1) ? bf16hi(gh[e >> 1]) : bf16lo(gh[e >> 1]);
      float pe = pp[e >> 2][e & 3], me = mm[e >> 2][e & 3], ve = vv[e >> 2][e & 3];
      adamw1(pe, me, ve, gf, a);
      pp[e >> 2][e & 3] = pe;
      mm[e >> 2][e & 3] = me;
      vv[e >> 2][e & 3] = ve;
    }
    p4[0] = pp[0]; p4[1] = pp[1];
    m4[0] = mm[0]; m4[1] = mm[1];
    v4[0] = vv[0]; v4[1] = vv[1];
    if (p16) {
      reinterpret_cast<uint4*>(p16)[i] =
          make_uint4(pack_bf16(pp[0][0], pp[0][1]), pack_bf16(pp[0][2], pp[0][3]),
                     pack_bf16(pp[1][0], pp[1][1]), pack_bf16(pp[1][2], pp[1][3]));
    }
  }
  // the last n % 8 parameters, one thread each
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e = n8 * 8 + t;
  if (t < (n & 7)) {
    float pe = p[e], me = m[e], ve = v[e];
    const float gf = __uint_as_float((uint32_t)g[e] << 16);
    adamw1(pe, me, ve, gf, a);
    p[e] = pe;
    m[e] = me;
    v[e] = ve;
    if (p16) {
      const __bf16 h = (__bf16)pe;
      p16[e] = __builtin_bit_cast(uint16_t, h);
    }
  }
}

}  // namespace

hipError_t launch_adamw(float* p, uint16_t* p16, const uint16_t* g, float* m, float* v, int64_t n,
                        const AdamW& a, hipStream_t s) {
  const int64_t n8 = n >> 3;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, p16, g, m, v, n, a);
  return hipGetLastError();
}

}  // namespace qlora
