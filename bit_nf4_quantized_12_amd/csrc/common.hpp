// Shared definitions of the gfx950 NF4 + double-quantisation + LoRA library.
//
// Storage format (NF4 with double quantisation) follows "QLoRA: Efficient
// Finetuning of Quantized LLMs" (inquiringlines.com), section "Method",
// paragraphs "4-bit NormalFloat Quantization" and "Double Quantization":
// blocks of 64 weights with one absmax constant each, and those constants
// quantised again (8-bit float) relative to the max of a group of 256 blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;                     // weights per absmax constant
constexpr int kGroupBlocks = 256;              // absmax constants per c1
constexpr int kGroup = kBlock * kGroupBlocks;  // weights per c1 (16384)

// The 16 NF4 levels, ascending (code 0 = -1, code 7 = 0, code 15 = +1).
struct Levels {
  float q[16];
};

// 4-bit data types. NF4 is the pages' type; Int4 (k / 7, k = -7..7) and FP4
// (the E2M1 values over 6) are the types the pages compare it with, in the
// plainest common form (the pages do not define them). All three hold the
// exact zero at code 7; Int4 and FP4 have 15 values and repeat +1 at code 15.
enum Codebook { kNF4 = 0, kInt4 = 1, kFP4 = 2, kNumCodebooks = 3 };

// Nearest-level search table for the quantiser. [-1, 1] is cut into
// 2 * scale equal cells (at most 32); each cell holds at most one decision
// threshold (the fp32 value T with: code > j  <=>  x > T_j), so
//   code(x) = base[cell(x)] + (x > thr[cell(x)]),
//   cell(x) = trunc(fma(x, scale, scale)),
// which is 2 * scale exactly for x = 1: that entry is the code of x = 1
// (no clamp needed for |x| <= 1). Cells without a threshold carry thr = +2
// (never exceeded).
constexpr int kQuantCells = 32;
struct QuantTable {
  float thr[kQuantCells + 1];
  int32_t base[kQuantCells + 1];
  float scale;
};

// Host side (tables.hip). Built once, immutable afterwards.
const Levels& host_levels(int codebook = kNF4);
const QuantTable& host_quant_table(int codebook = kNF4);
// Nonzero if the tables could not be built consistently.
int tables_status();

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// OCP FP8 E4M3 byte (sign ignored: constants are never negative) -> float.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 7u;
  const float sub = (float)m * 0x1p-9f;
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e ? nrm : sub;
}

// Dequantised block constant c^ = fp32(e4m3(c2[b]) * c1[b / 256]).
__device__ __forceinline__ float block_scale(const uint8_t* __restrict__ c2,
                                             const float* __restrict__ c1, int64_t b) {
  const float d = e4m3_value(c2[b]);
  const float g = c1[b >> 8];
  return __fmul_rn(d, g);
}

// Block constant: the fp32 absmax stored as is (ABS: no double
// quantisation), else the double-quantised one. A template parameter rather
// than a run-time test, so that hot loops stay one basic block.
template <bool ABS>
__device__ __forceinline__ float block_const(const uint8_t* __restrict__ c2, const float* __restrict__ c1,
                                             const float* __restrict__ absmax, int64_t b) {
  if (ABS) return absmax[b];
  return block_scale(c2, c1, b);
}

// LDS tiles of 64 bf16 per row (128 B) store the 16-byte chunk c of row R
// at chunk c ^ lds_swz(R). An MFMA operand fragment read (lane l: row l & 15,
// chunk l >> 4, ds_read_b128) then needs no more LDS cycles than a linear
// read on gfx950; an XOR with (R & 7) alone measured 2-way bank conflicts.
__device__ __forceinline__ int lds_swz(int R) { return (R & 7) ^ (((R >> 1) & 1) << 2); }

// Inline-tuned LDS load/store of 16 bytes.
__device__ __forceinline__ bf16x8 lds_load8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace qlora
