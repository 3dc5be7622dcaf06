// Blockwise 4-bit quantiser (NF4, or the Int4 / FP4 comparison types) with
// or without double quantisation of the block constants.
//
// "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com),
// "Method": step (3) of "4-bit NormalFloat Quantization" (normalise each
// block of 64 into [-1, 1] by its absolute maximum, then take the nearest
// level) and "Double Quantization" (quantise the block constants again).
//
// One workgroup (4 wave64) per group of 256 blocks = 16384 weights = 32 KB
// of bf16. Loads are 16 B per lane and fully coalesced; the block absmax is
// a max over the 8 lanes that hold a block (DPP, no LDS); the group max is a
// wave reduction plus 4 LDS slots. The weights are read and the codes
// written with nontemporal accesses (streamed once; measured +4-5 % on a
// cold 3.4 GB pass). HBM traffic is the algorithmic minimum:
// 2 B read and 0.5 + 1/64 + 4/16384 B written per weight (0.5 + 4/64 B
// without double quantisation, when the fp32 block absmax is stored as is).
// The data type only changes the search table passed in.
#include "launch.hpp"

namespace qlora {
namespace {

__device__ __forceinline__ float dpp_max8(float v) {
  // lanes of one block: 8 consecutive lanes. xor 1, xor 2 inside a quad,
  // then the mirror inside 8 lanes pairs the two quads. v is an absolute
  // value (finite weights), so the float order is the unsigned order of the
  // bits and an integer max does it (one instruction per step with the DPP
  // operand folded in, no NaN canonicalisation).
  uint32_t u = __float_as_uint(v);
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, true));
  return __uint_as_float(u);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// x = RN32(w / c) for one block. r = RN32(1 / c). With r correctly rounded,
// q0 = RN(w r), e = w - c q0 (exact through the fused multiply-add) and
// RN(q0 + e r) is the correctly rounded quotient (Markstein's theorem) as
// long as nothing under- or overflows, which `fast` guarantees; otherwise
// the IEEE division is used.
__device__ __forceinline__ float div_block(float w, float c, float r, bool fast) {
  if (fast) {
    const float q0 = w * r;
    const float e = __builtin_fmaf(-c, q0, w);
    return __builtin_fmaf(e, r, q0);
  }
  return w / c;
}

// r = RN32(1 / c) for a block max c in [2^-100, 2^100] (a bf16 value: at most
// 8 significant bits): the hardware reciprocal (within 1 ulp) refined by one
// Newton step through fused multiply-adds, e = 1 - c y0 being exact. Checked
// exhaustively over the 128 bf16 significands (the step commutes with
// power-of-two scaling inside that range), it is correctly rounded even from
// a start 2 ulps away; it replaces an IEEE division (about 10 instructions)
// per block and lane.
__device__ __forceinline__ float rcp_bf16(float c) {
  const float y0 = __builtin_amdgcn_rcpf(c);
  const float e = __builtin_fmaf(-c, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}

// |x| <= 1, so the cell is in [0, 2 scale] (a NaN converts to cell 0)
__device__ __forceinline__ uint32_t nearest_code(float x, const float2* __restrict__ tab, float scale) {
  const int cell = (int)__builtin_fmaf(x, scale, scale);
  const float2 t = tab[cell];
  return (uint32_t)__float_as_int(t.y) + (x > t.x ? 1u : 0u);
}

// E4M3 (OCP, bias 7) code of rho in [0, 1], round to nearest even.
__device__ __forceinline__ uint32_t e4m3_code(float rho) {
  if (rho >= 0x1p-6f) {
    const uint32_t b = __float_as_uint(rho);
    uint32_t kept = b >> 20;
    const uint32_t rem = b & 0xFFFFFu;
    kept += (rem > 0x80000u || (rem == 0x80000u && (kept & 1u))) ? 1u : 0u;
    return kept - ((127u - 7u) << 3);
  }
  return (uint32_t)__builtin_rintf(rho * 512.0f);  // subnormal: m * 2^-9, m in 0..8
}

// Codes of this lane's 8 chunks of 8 weights (chunk j: elements
// gbase + 4096 wave + 512 j + 8 lane ..), their block maxima (bmax[j], the
// same on the 8 lanes of a block) and the running group max. FULL: the whole
// group lies inside the tensor.
template <bool FULL>
__device__ __forceinline__ void quant_rows(const uint16_t* __restrict__ w, uint8_t* __restrict__ codes, int64_t n,
                                           int64_t gbase, int wave, int lane, const float2* __restrict__ tab,
                                           float scale, float (&bmax)[8], float& gmax) {
  const int64_t e0 = gbase + wave * 4096 + lane * 8;
  uint4 v[8];
  if constexpr (FULL) {
    // all 32 KB of the group in flight at once
    const u32x4* wp = reinterpret_cast<const u32x4*>(w + e0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 t = __builtin_nontemporal_load(wp + 64 * j);
      v[j] = make_uint4(t[0], t[1], t[2], t[3]);
    }
  }
  uint32_t* cp = reinterpret_cast<uint32_t*>(codes + (e0 >> 1));

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (!FULL) {
      // a tensor's last group: element loads, one chunk at a time (this path
      // runs once per tensor; loading it all up front would set the
      // kernel's register budget, and so its occupancy, for every group)
      const int64_t e = e0 + j * 512;
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = (e + i < n) ? w[e + i] : 0u;
      v[j] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
    float f[8];
    f[0] = bf16lo(v[j].x); f[1] = bf16hi(v[j].x);
    f[2] = bf16lo(v[j].y); f[3] = bf16hi(v[j].y);
    f[4] = bf16lo(v[j].z); f[5] = bf16hi(v[j].z);
    f[6] = bf16lo(v[j].w); f[7] = bf16hi(v[j].w);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    m = dpp_max8(m);
    bmax[j] = m;
    gmax = fmaxf(gmax, m);

    // an all-zero block is divided by 1: its weights are +-0 and map to the
    // exact zero like any x = 0
    const float md = m > 0.0f ? m : 1.0f;
    const bool fast = md >= 0x1p-100f && md <= 0x1p100f;
    const float r = rcp_bf16(md);  // used by the lanes with `fast` only
    uint32_t word = 0;
    if (__all(fast)) {
      // every block of the wave in range (wave-uniform branch): the
      // straight-line correctly rounded quotient
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= nearest_code(div_block(f[i], md, r, true), tab, scale) << (4 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= nearest_code(div_block(f[i], md, r, fast), tab, scale) << (4 * i);
    }
    if constexpr (FULL) {
      __builtin_nontemporal_store(word, cp + 64 * j);
    } else {
      const int64_t e = e0 + j * 512;
      if (e + 8 <= n) {
        __builtin_nontemporal_store(word, cp + 64 * j);
      } else if (e < n) {
        // short tail: elements past n get code 0, bytes past ceil(n/2) are not written
        const int valid = (int)(n - e);
        const uint32_t keep = (1u << (4 * valid)) - 1u;
        word &= keep;
        const int bytes = (valid + 1) >> 1;
        for (int b = 0; b < bytes; ++b) codes[(e >> 1) + b] = (uint8_t)(word >> (8 * b));
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the chunks apart (registers)
    }
  }
}

__global__ __launch_bounds__(256) void quantize_kernel(QuantBatch bt, QuantTable qt) {
  __shared__ float2 s_tab[kQuantCells + 1];
  __shared__ float s_wmax[4];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  if (tid <= kQuantCells) s_tab[tid] = make_float2(qt.thr[tid], __int_as_float(qt.base[tid]));

  // this workgroup's tensor (uniform scan over at most kQuantBatch entries)
  // and its group within that tensor
  int ti = 0;
  while (ti + 1 < bt.count && (int64_t)blockIdx.x >= bt.gstart[ti + 1]) ++ti;
  const uint16_t* __restrict__ w = bt.w[ti];
  const int64_t n = bt.n[ti];
  uint8_t* __restrict__ codes = bt.codes[ti];
  uint8_t* __restrict__ c2 = bt.c2[ti];
  float* __restrict__ c1 = bt.c1[ti];
  float* __restrict__ absmax_out = bt.absmax[ti];
  const int64_t grp = (int64_t)blockIdx.x - bt.gstart[ti];
  __syncthreads();

  const int64_t gbase = grp * kGroup;
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const bool full = gbase + kGroup <= n;

  float bmax[8];
  float gmax = 0.0f;
  // A full group (all but a tensor's last) takes the straight path: no
  // bounds checks, and every load and store at a constant offset from one
  // per-lane base (the checks and 64-bit index arithmetic of the general
  // path cost about as many instructions as the search itself).
  if (full) {
    quant_rows<true>(w, codes, n, gbase, wave, lane, s_tab, qt.scale, bmax, gmax);
  } else {
    quant_rows<false>(w, codes, n, gbase, wave, lane, s_tab, qt.scale, bmax, gmax);
  }

  if (absmax_out) {
    // no double quantisation: the exact block absmax is the stored constant
    if ((lane & 7) == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t b = (gbase >> 6) + wave * 64 + j * 8 + (lane >> 3);
        if (b < nb) absmax_out[b] = bmax[j];
      }
    }
    return;
  }
  gmax = wave_max(gmax);
  if (lane == 0) s_wmax[wave] = gmax;
  __syncthreads();
  const float g = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
  if (tid == 0) c1[grp] = g;
  if ((lane & 7) == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t b = (gbase >> 6) + wave * 64 + j * 8 + (lane >> 3);
      if (b < nb) {
        uint32_t code = 0;
        if (g > 0.0f) code = e4m3_code(bmax[j] / g);
        c2[b] = (uint8_t)code;
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize_batch(const QuantBatch& b, int codebook, hipStream_t s) {
  const int64_t groups = b.gstart[b.count];
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)groups), dim3(256), 0, s, b, host_quant_table(codebook));
  return hipGetLastError();
}

hipError_t launch_quantize(const void* w, int64_t n, int codebook, uint8_t* codes, uint8_t* c2, float* c1,
                           float* absmax, hipStream_t s) {
  QuantBatch b{};
  b.count = 1;
  b.gstart[0] = 0;
  b.gstart[1] = (n + kGroup - 1) / kGroup;
  b.w[0] = reinterpret_cast<const uint16_t*>(w);
  b.n[0] = n;
  b.codes[0] = codes;
  b.c2[0] = c2;
  b.c1[0] = c1;
  b.absmax[0] = absmax;
  return launch_quantize_batch(b, codebook, s);
}

}  // namespace qlora
