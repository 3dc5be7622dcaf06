// Host-side launchers of the library's kernels (one per .hip file).
#pragma once

#include <atomic>

#include "common.hpp"

namespace qlora {

// Opt kernel fn in to `bytes` of dynamic LDS (above the default 64 KB) on
// the current device. The attribute is per device, so `done` keeps one bit
// per device (devices past 31 set it on every call).
inline hipError_t ensure_lds(const void* fn, int bytes, std::atomic<uint32_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint32_t bit = dev < 32 ? (1u << dev) : 0u;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

struct GemmParams {
  const uint16_t* act;     // [M, Kred] bf16, row pitch Kred
  const uint8_t* codes;    // NF4 codes of W [wN, wK]
  const uint8_t* c2;
  const float* c1;
  const float* absmax;     // fp32 block constants (no double quantisation), or null
  int64_t wN, wK;
  const uint16_t* lora_l;  // [M, lora_ld] bf16 (scale folded in), or null
  const uint16_t* lora_r;  // [Nout, rp] bf16, or null
  int rp;                  // multiple of 64, columns past r are zero
  int lora_ld;             // row pitch of lora_l (rp, or more for grouped linears)
  int lora_seg;            // > 0: output columns n use lora_l columns (n / lora_seg) rp .. + rp
  uint16_t* out;           // [M, Nout] bf16
  int M, Nout, Kred;
  Levels lv;
  // split reduction: ksplit > 1 splits of kchunk 64-deep steps write float32
  // partial tiles to part [ksplit][M][Nout], summed into out afterwards
  int ksplit = 1, kchunk = 0;
  float* part = nullptr;
};

// Output tile of the GEMM: 512 x 128 from 1024 rows on (half the unpacking
// per MFMA), else 256 x 256; when that leaves fewer than 192 tiles (most of
// the 256 CUs idle), 128 x 128.
enum GemmTile { kTile512x128 = 0, kTile256x256 = 1, kTile128x128 = 2 };
inline int64_t gemm_tiles(int64_t M, int64_t Nout, int64_t bm, int64_t bn) {
  return ((M + bm - 1) / bm) * ((Nout + bn - 1) / bn);
}
inline GemmTile gemm_tile(int64_t M, int64_t Nout) {
  const bool big = M >= 1024;
  if (gemm_tiles(M, Nout, big ? 512 : 256, big ? 128 : 256) >= 192) return big ? kTile512x128 : kTile256x256;
  return kTile128x128;
}

// Splits of the reduction: with 128 x 128 tiles, enough splits for ~256
// workgroups, at most 4, each at least 4 steps of 64; none otherwise.
// Returns the split count (every split non-empty) and the steps per split.
inline int gemm_ksplit(int64_t M, int64_t Nout, int64_t Kred, int* kchunk) {
  const int64_t nk = (Kred + 63) / 64;
  int64_t ks = 1;
  if (gemm_tile(M, Nout) == kTile128x128) {
    const int64_t tiles = gemm_tiles(M, Nout, 128, 128);
    ks = (256 + tiles - 1) / tiles;
    if (ks > 4) ks = 4;
    if (ks > nk / 4) ks = nk / 4;
    if (ks < 1) ks = 1;
  }
  const int64_t ch = (nk + ks - 1) / ks;
  *kchunk = (int)ch;
  return (int)((nk + ch - 1) / ch);
}

// Several tensors quantised by one launch: workgroups gstart[t] ..
// gstart[t+1]-1 take the 16384-weight groups of tensor t.
constexpr int kQuantBatch = 16;
struct QuantBatch {
  int count;
  int64_t gstart[kQuantBatch + 1];
  const uint16_t* w[kQuantBatch];
  int64_t n[kQuantBatch];
  uint8_t* codes[kQuantBatch];
  uint8_t* c2[kQuantBatch];
  float* c1[kQuantBatch];
  float* absmax[kQuantBatch];
};
hipError_t launch_quantize_batch(const QuantBatch& b, int codebook, hipStream_t s);

// Double-quantised constants (c2, c1) when absmax is null; otherwise the
// fp32 block absmax, and c2 / c1 are unused.
hipError_t launch_quantize(const void* w, int64_t n, int codebook, uint8_t* codes, uint8_t* c2, float* c1,
                           float* absmax, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* absmax,
                          int64_t n, int codebook, bool bf16_out, void* out, hipStream_t s);
hipError_t launch_gemm(const GemmParams& p, bool transposed_w, hipStream_t s);
hipError_t launch_proj(const uint16_t* L, const uint16_t* R, int M, int Kr, int r, int rp,
                       int nsplit, float* part, hipStream_t s);
// Streamed projection (Kr % 64 == 0, rp_total % 64 == 0), part
// [nsplit][M][rp_total]. The result's 64-column blocks come in segments of
// zper blocks; segment g multiplies L + g segL by rows of R + g segR (r_seg
// valid rows), row pitches ldL / ldR.
hipError_t launch_proj_seg(const uint16_t* L, int64_t ldL, int64_t segL, const uint16_t* R, int64_t ldR,
                           int64_t segR, int zper, int M, int Kr, int r_seg, int rp_total, int nsplit, float* part,
                           hipStream_t s);
hipError_t launch_finalize(const float* part, int nsplit, int M, int Mp, int r, int rp, float scale,
                           float* P32, uint16_t* Ph, uint16_t* Pl, hipStream_t s);
hipError_t launch_grad(const float* P, const uint16_t* Q, int M, int C, int r, int rp, int nsplit,
                       float* part, hipStream_t s);
hipError_t launch_grad_reduce(const float* part, int nsplit, int r, int rp, int C, float scale,
                              bool transpose, bool part_trans, uint16_t* out, hipStream_t s);
// segC > 0: the columns of segment c / segC pair only with plane columns
// (c / segC) rseg .. + rseg (grouped linears); the result then has rseg rows.
hipError_t launch_grad_tr(const uint16_t* Ph, const uint16_t* Pl, const uint16_t* Q, int M, int Mp, int C,
                          int rp, int nsplit, bool trans, float* part, hipStream_t s, int segC = 0,
                          int rseg = 0);
hipError_t launch_relayout(const uint16_t* in, int64_t rows_in, int64_t cols_in, int64_t ldi,
                           bool transpose, uint16_t* out, int64_t rows_out, int64_t cols_out,
                           int64_t ldo, hipStream_t s);
// Bt [r, N] = B^T for B [N, r]; At [K, rp] = A^T zero-padded for A [rA, K] (if At).
hipError_t launch_transpose2(const uint16_t* B, const uint16_t* A, int N, int K, int r, int rA, int rp,
                             uint16_t* Bt, uint16_t* At, hipStream_t s);
hipError_t launch_finalize2(const float* part, int nsplit, int M, int Mp, int r, int rp, float scale,
                            float* P32, uint16_t* Ph, uint16_t* Pl, const float* T, uint16_t* Th,
                            uint16_t* Tl, hipStream_t s);
hipError_t launch_grad_reduce2(const float* partA, int nsA, int C1, uint16_t* dA, const float* partB, int nsB,
                               int C2, uint16_t* dB, int rA, int rpA, int rB, int rpB, float scale, hipStream_t s);
// Few tokens (M <= 16): T [M, R] = X A^T (float32, A the R rows of the
// segments' adapters stacked), then Y [M, N] = X W~^T + scale T_z B^T (rows
// of segment z = n / segN use T columns z rseg .. + rseg; segN = 0: one
// segment, rseg = R), two launches. Y null: T only.
hipError_t launch_fewtok(const uint16_t* X, const uint8_t* codes, const uint8_t* c2, const float* c1,
                         const float* absmax, int codebook, int N, int K, int M, const uint16_t* A, int R,
                         const uint16_t* B, int rseg, int segN, float scale, uint16_t* Y, float* T,
                         hipStream_t s);

// Merged weight out [N, K] = bf16(W^ + scale B A) (merge.hip); absmax null:
// double-quantised constants.
hipError_t launch_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, const float* absmax, int codebook,
                        const uint16_t* A, const uint16_t* B, int N, int K, int r, float scale, uint16_t* out,
                        hipStream_t s);

// AdamW step (optim.hip): bc1 = 1 / (1 - beta1^t), bc2 = 1 / (1 - beta2^t).
struct AdamW {
  float lr, beta1, beta2, one_minus_beta1, one_minus_beta2, eps, weight_decay, bc1, bc2;
};
hipError_t launch_adamw(float* p, uint16_t* p16, const uint16_t* g, float* m, float* v, int64_t n,
                        const AdamW& a, hipStream_t s);

}  // namespace qlora
