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
// written (+ 2 B for the bf16 copy of the updated weight). Thread t of
// workgroup b updates parameters 1024 b + 4 t .. + 3, so each fp32 access
// instruction covers 1 KB of consecutive memory (512 B for the bf16 ones);
// lanes 32 B apart in a grid-stride loop ran 12 % slower.
#include "launch.hpp"

// Every operation of the update is rounded on its own: contraction into
// FMAs is off for the operators written in this file (it would make the
// rounding depend on code shape). Square root and division are the
// correctly rounded ones (HIP's default for float32 sqrt and divide).
#pragma clang fp contract(off)

namespace qlora {
namespace {

typedef float f32v4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void adamw1(float& p, float& m, float& v, float g, const AdamW& a) {
  m = a.beta1 * m + a.one_minus_beta1 * g;
  v = a.beta2 * v + a.one_minus_beta2 * (g * g);
  const float mh = m * a.bc1;
  const float vh = v * a.bc2;
  const float upd = mh / (__builtin_sqrtf(vh) + a.eps);
  p = p - a.lr * (a.weight_decay * p + upd);
}

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, uint16_t* __restrict__ p16,
                                                     const uint16_t* __restrict__ g, float* __restrict__ m,
                                                     float* __restrict__ v, int64_t n, AdamW a) {
  const int64_t e = (int64_t)blockIdx.x * 1024 + 4 * threadIdx.x;
  if (e + 4 <= n) {
    const uint2 gw = *reinterpret_cast<const uint2*>(g + e);
    f32v4* p4 = reinterpret_cast<f32v4*>(p + e);
    f32v4* m4 = reinterpret_cast<f32v4*>(m + e);
    f32v4* v4 = reinterpret_cast<f32v4*>(v + e);
    f32v4 pp = *p4, mm = *m4, vv = *v4;
    const float gf[4] = {bf16lo(gw.x), bf16hi(gw.x), bf16lo(gw.y), bf16hi(gw.y)};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float pe = pp[k], me = mm[k], ve = vv[k];
      adamw1(pe, me, ve, gf[k], a);
      pp[k] = pe;
      mm[k] = me;
      vv[k] = ve;
    }
    *p4 = pp;
    *m4 = mm;
    *v4 = vv;
    if (p16) *reinterpret_cast<uint2*>(p16 + e) = make_uint2(pack_bf16(pp[0], pp[1]), pack_bf16(pp[2], pp[3]));
    return;
  }
  // the last n % 4 parameters (e < n < e + 4)
  for (int64_t k = e; k < n; ++k) {
    float pe = p[k], me = m[k], ve = v[k];
    adamw1(pe, me, ve, __uint_as_float((uint32_t)g[k] << 16), a);
    p[k] = pe;
    m[k] = me;
    v[k] = ve;
    if (p16) {
      const __bf16 h = (__bf16)pe;
      p16[k] = __builtin_bit_cast(uint16_t, h);
    }
  }
}

}  // namespace

hipError_t launch_adamw(float* p, uint16_t* p16, const uint16_t* g, float* m, float* v, int64_t n,
                        const AdamW& a, hipStream_t s) {
  const int64_t blocks = (n + 1023) / 1024;  // < 2^31: n <= 2^40 (checked by the caller)
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, p16, g, m, v, n, a);
  return hipGetLastError();
}

}  // namespace qlora
