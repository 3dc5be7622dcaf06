// Few-token forward (M <= 16): Y = X W~^T + s T B^T, bound by reading the
// 4-bit weight from HBM.
//
// "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com),
// "Method": dequantise to BFloat16, multiply in 16-bit. With at most 16
// tokens each weight is used at most 16 times, so the kernel streams the
// codes exactly once, straight from HBM into registers:
//
//  * a workgroup (16 wave64) owns 16 weight rows over the whole of K; the
//    waves take 128-column chunks round robin, two at a time with both
//    chunks' loads in flight before any unpacking, and meet in LDS at the
//    end, so there are no split-K partial sums in memory;
//  * per chunk a lane loads 16 B of codes = 32 weights of its row (one
//    global_load_dwordx4), unpacks them through its block's 16-entry bf16
//    table with v_perm byte selects, and feeds four
//    v_mfma_f32_16x16x32_bf16 with X rows (padded to 16 with zeros) as the
//    A operand. The reduction order inside a chunk is permuted (MFMA k-slot
//    8 g + e of product i is column 32 g + 8 i + e of the chunk), identically
//    for both operands;
//  * the epilogue sums the split-K partials of T = X A^T (LoRA projection,
//    a separate small kernel) and adds s T B^T before the bf16 store.
#include "launch.hpp"

namespace qlora {
namespace {

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 16-entry bf16(q[c] * c^) table as byte planes (see the GEMM kernel).
__device__ __forceinline__ void gv_table(float chat, const Levels& lv, uint32_t L[4], uint32_t H[4]) {
  uint32_t P[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) P[i] = pack_bf16(__fmul_rn(lv.q[2 * i], chat), __fmul_rn(lv.q[2 * i + 1], chat));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    L[j] = perm(P[2 * j + 1], P[2 * j], 0x06040200u);
    H[j] = perm(P[2 * j + 1], P[2 * j], 0x07050301u);
  }
}

// 8 codes -> 8 bf16 of W~ in natural order (4 packed pairs).
__device__ __forceinline__ uint4 gv_lookup8(uint32_t d, const uint32_t L[4], const uint32_t H[4]) {
  const uint32_t se = d & 0x07070707u;
  const uint32_t so = (d >> 4) & 0x07070707u;
  const uint32_t ce = ((d >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t co = ((d >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t Le = perm(perm(L[3], L[2], se), perm(L[1], L[0], se), ce);
  const uint32_t He = perm(perm(H[3], H[2], se), perm(H[1], H[0], se), ce);
  const uint32_t Lo = perm(perm(L[3], L[2], so), perm(L[1], L[0], so), co);
  const uint32_t Ho = perm(perm(H[3], H[2], so), perm(H[1], H[0], so), co);
  const uint32_t E0 = perm(He, Le, 0x05010400u), E1 = perm(He, Le, 0x07030602u);
  const uint32_t O0 = perm(Ho, Lo, 0x05010400u), O1 = perm(Ho, Lo, 0x07030602u);
  return make_uint4(perm(O0, E0, 0x05040100u), perm(O0, E0, 0x07060302u), perm(O1, E1, 0x05040100u),
                    perm(O1, E1, 0x07060302u));
}

constexpr int GV_WAVES = 16;

template <bool ABS>
__global__ __launch_bounds__(64 * GV_WAVES) void gemv_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ c2,
    const float* __restrict__ c1, const float* __restrict__ absmax, int N, int K, int M,
    const float* __restrict__ tpart, int tsplit, int rp,
    const uint16_t* __restrict__ B, int r, float scale, uint16_t* __restrict__ Y, float* __restrict__ T_out,
    int segN, int tld, Levels lv) {
  __shared__ float red[GV_WAVES][16][17];
  __shared__ float sT[16][257];
  __shared__ uint16_t sB[16 * 256];  // the workgroup's 16 rows of B
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16;
  // grouped linears: rows of segment z = n0 / segN use T columns z r .. + r
  // (T_out [M, tld] gets them from the segment's first workgroup)
  const int zc = segN ? (n0 / segN) * r : 0;
  const bool t_writer = segN ? (n0 % segN) == 0 : blockIdx.x == 0;
  const int c = l & 15, g = l >> 4;
  const int n = min(n0 + c, N - 1);  // rows past N: clamped read, result not stored
  const bool xok = c < M;            // A-operand row = X row c (zero past M)
  const uint16_t* xrow = X + (int64_t)min(c, M - 1) * K;
  const int64_t rowe = (int64_t)n * K;
  const int nchunks = (K + 127) / 128;

  // this lane's 32 columns of chunk ch; K % 64 == 0, so only the upper half
  // of the last chunk can be missing (clamped read, c^ = 0)
  auto chunk_load = [&](int ch, uint4& cw, float& chat, int& kcc) {
    const int kc = 128 * ch + 32 * g;
    const bool kok = kc < K && ch < nchunks;
    kcc = kok ? kc : K - 32;
    const int64_t e = rowe + kcc;
    cw = *reinterpret_cast<const uint4*>(codes + (e >> 1));
    const float s2 = block_const<ABS>(c2, c1, absmax, e >> 6);
    chat = kok ? s2 : 0.0f;
  };
  auto chunk_mma = [&](const uint4& cw, float chat, int kcc, f32x4& acc) {
    uint32_t L[4], H[4];
    gv_table(chat, lv, L, H);
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 xv = *reinterpret_cast<const uint4*>(xrow + kcc + 8 * i);
      xv = xok ? xv : make_uint4(0, 0, 0, 0);
      const uint4 wv = gv_lookup8(words[i], L, H);
      acc = mfma16(__builtin_bit_cast(bf16x8, xv), __builtin_bit_cast(bf16x8, wv), acc);
    }
  };

  // With r <= 64 the epilogue operands are fetched before the weight stream
  // so their latency overlaps it: thread t holds B element t (rows n0 ..
  // n0 + 15, r columns) and the first 16 split-K partials of T element t
  // (t < M r); a longer split is summed after the main loop. Larger ranks
  // fetch them after the main loop.
  const bool pre = r <= 64;
  const int nb = 16 * r, nt = M * r;
  const bool hasb = pre && tid < nb, hast = pre && tid < nt;
  const int br = hasb ? tid / r : 0, bj = hasb ? tid % r : 0;
  const uint16_t bval = hasb ? B[(int64_t)min(n0 + br, N - 1) * r + bj] : (uint16_t)0;
  const int tm = hast ? tid / r : 0, tj = hast ? tid % r : 0;
  float tp[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) tp[k] = (hast && k < tsplit) ? tpart[((int64_t)k * M + tm) * rp + zc + tj] : 0.0f;

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int ch = w; ch < nchunks; ch += 2 * GV_WAVES) {
    uint4 cw0, cw1;
    float s0, s1;
    int k0, k1;
    chunk_load(ch, cw0, s0, k0);
    chunk_load(ch + GV_WAVES, cw1, s1, k1);  // past the end: zero contribution
    chunk_mma(cw0, s0, k0, acc);
    chunk_mma(cw1, s1, k1, acc);
  }
  // D[m][n]: lane holds X rows 4 g + v, weight row c
#pragma unroll
  for (int v = 0; v < 4; ++v) red[w][4 * g + v][c] = acc[v];

  // B rows n0 .. n0 + 15 (r columns each) and T = sum of the split-K
  // partials of X A^T (rows < M, columns < r) into LDS
  if (pre) {
    // 16 r <= 1024 and M r <= 1024 threads (M <= 16)
    if (hasb) sB[br * r + bj] = bval;
    if (hast) {
      float s = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) s += tp[k];
      for (int k = 16; k < tsplit; ++k) s += tpart[((int64_t)k * M + tm) * rp + zc + tj];
      sT[tm][tj] = s;
      if (t_writer && T_out) T_out[(int64_t)tm * tld + zc + tj] = s;
    }
  } else {
    for (int idx = tid; idx < 16 * r; idx += 64 * GV_WAVES) {
      const int rr = idx / r, j = idx % r;
      sB[rr * r + j] = B[(int64_t)min(n0 + rr, N - 1) * r + j];
    }
    for (int idx = tid; idx < M * r; idx += 64 * GV_WAVES) {
      const int m = idx / r, j = idx % r;
      float s = 0.0f;
      for (int k = 0; k < tsplit; ++k) s += tpart[((int64_t)k * M + m) * rp + zc + j];
      sT[m][j] = s;
      if (t_writer && T_out) T_out[(int64_t)m * tld + zc + j] = s;
    }
  }
  __syncthreads();
  // thread -> (m, row): m = tid >> 4, row = tid & 15 (first 256 threads)
  const int m = tid >> 4, rr = tid & 15;
  if (tid < 256 && m < M && n0 + rr < N) {
    float y = 0.0f;
#pragma unroll
    for (int q = 0; q < GV_WAVES; ++q) y += red[q][m][rr];
    float lo = 0.0f;
    for (int j = 0; j < r; ++j) lo = __builtin_fmaf(sT[m][j], bf16lo(sB[rr * r + j]), lo);
    const __bf16 h = (__bf16)(y + scale * lo);
    Y[(int64_t)m * N + n0 + rr] = __builtin_bit_cast(uint16_t, h);
  }
}

}  // namespace

hipError_t launch_gemv(const uint16_t* X, const uint8_t* codes, const uint8_t* c2, const float* c1,
                       const float* absmax, int codebook, int N, int K, int M, const float* tpart, int tsplit,
                       int rp, const uint16_t* B, int r, float scale, uint16_t* Y, float* T_out, hipStream_t s,
                       int segN, int tld) {
  if (!tld) tld = r;
  if (absmax)
    hipLaunchKernelGGL(gemv_kernel<true>, dim3((N + 15) / 16), dim3(64 * GV_WAVES), 0, s, X, codes, c2, c1, absmax,
                       N, K, M, tpart, tsplit, rp, B, r, scale, Y, T_out, segN, tld, host_levels(codebook));
  else
    hipLaunchKernelGGL(gemv_kernel<false>, dim3((N + 15) / 16), dim3(64 * GV_WAVES), 0, s, X, codes, c2, c1, absmax,
                       N, K, M, tpart, tsplit, rp, B, r, scale, Y, T_out, segN, tld, host_levels(codebook));
  return hipGetLastError();
}

}  // namespace qlora
