// Few-token forward (M <= 16): Y = X W~^T + s T B^T, bound by reading the
// 4-bit weight from HBM.
//
// "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com),
// "Method": dequantise to BFloat16, multiply in 16-bit. With at most 16
// tokens each weight is used at most 16 times, so the kernel streams the
// codes exactly once, straight from HBM into registers:
//
//  * a workgroup (8 wave64) owns 16 weight rows over the whole of K; the
//    waves take 128-column chunks round robin, 4 at a time with all four
//    chunks' loads in flight before any unpacking, and meet in LDS at the
//    end, so there are no split-K partial sums in memory. Workgroups are
//    small enough for two per CU, so a 7B projection's codes are almost all
//    in flight at once;
//  * per chunk a lane loads 16 B of codes = 32 weights of its row (one
//    global_load_dwordx4), unpacks them through its block's 16-entry bf16
//    table with v_perm byte selects, and feeds four
//    v_mfma_f32_16x16x32_bf16 with X rows as the A operand. X rows past M
//    are read as zero by a buffer load whose offset lies past the buffer
//    (no memory traffic); their output rows are never stored. The reduction
//    order inside a chunk is permuted (MFMA k-slot 8 g + e of product i is
//    column 32 g + 8 i + e of the chunk), identically for both operands;
//  * the epilogue sums the split-K partials of T = X A^T (proj_small_kernel
//    below, a separate launch) and adds s T B^T before the bf16 store.
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

constexpr int GV_WAVES = 8;            // waves per workgroup
constexpr int GV_D = 4;                // 128-column chunks in flight per wave
constexpr int GV_NT = 64 * GV_WAVES;
constexpr int GV_PRE = 4;              // T partials per element fetched before the weight stream

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16 B of a bf16 matrix through a buffer resource: zero when off is past the
// resource's size (then nothing is read).
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// X [M, K] bf16 as a buffer; lane row c >= M reads past the end (zeros).
struct XRows {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t row_off, end;  // byte offset of this lane's row, or end when c >= M
  __device__ XRows(const uint16_t* X, int M, int K, int c) {
    end = (uint32_t)M * (uint32_t)K * 2u;  // < 2^32: M max(N, K) < 2^31
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, (int)end, 0x00020000);
    row_off = c < M ? (uint32_t)c * (uint32_t)K * 2u : end;
  }
  // 4 x 8 bf16 at columns k, k + 8, k + 16, k + 24 of this lane's row
  __device__ __forceinline__ void load4(int k, uint4 (&v)[4]) const {
    const uint32_t o = row_off == end ? end : row_off + 2u * (uint32_t)k;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = buf_load16(rs, o == end ? end : o + 16u * i);
  }
};

template <bool ABS>
__global__ __launch_bounds__(GV_NT) __attribute__((amdgpu_waves_per_eu(4))) void gemv_kernel(
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
  const XRows xr(X, M, K, c);
  const int64_t rowe = (int64_t)n * K;
  const int nchunks = (K + 127) / 128;

  // Epilogue operands first, so that their latency overlaps the weight
  // stream: thread t owns T elements t and t + GV_NT (< M r) with their first
  // GV_PRE split partials, and B elements t and t + GV_NT (< 16 r).
  const int nb = 16 * r, nt = M * r;
  // Addresses are clamped so that every load is unconditional (one batch,
  // no waits between them); unused values are masked afterwards.
  float tp[2][GV_PRE];
  uint16_t bval[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int idx = tid + e * GV_NT;
    const bool hb = idx < nb, ht = idx < nt;
    const int br = hb ? idx / r : 0, bj = hb ? idx % r : 0;
    bval[e] = B[(int64_t)min(n0 + br, N - 1) * r + bj];  // stored only when hb
    const int tm = ht ? idx / r : 0, tj = ht ? idx % r : 0;
#pragma unroll
    for (int k = 0; k < GV_PRE; ++k) tp[e][k] = tpart[((int64_t)min(k, tsplit - 1) * M + tm) * rp + zc + tj];
  }

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int cb = w; cb < nchunks; cb += GV_D * GV_WAVES) {
    // this lane's 32 columns of each chunk; K % 64 == 0, so only the upper
    // half of the last chunk can be missing (clamped read, c^ = 0)
    uint4 cw[GV_D];
    float craw[GV_D], g1[GV_D];
    uint32_t c2b[GV_D];
    int kc[GV_D];
#pragma unroll
    for (int i = 0; i < GV_D; ++i) {
      const int ch = min(cb + i * GV_WAVES, nchunks - 1);  // past the end: a repeat, masked below
      kc[i] = min(128 * ch + 32 * g, K - 32);
      const int64_t e = rowe + kc[i];
      cw[i] = *reinterpret_cast<const uint4*>(codes + (e >> 1));
      if (ABS) {
        craw[i] = absmax[e >> 6];
      } else {
        c2b[i] = c2[e >> 6];
        g1[i] = c1[e >> 14];
      }
    }
    uint4 xv[GV_D][4];
#pragma unroll
    for (int i = 0; i < GV_D; ++i) xr.load4(kc[i], xv[i]);
    // Every chunk slot is multiplied (no branch, so the compiler keeps all
    // loads ahead of the first product); a slot past the end, or the missing
    // upper half of a last chunk, has c^ = 0 and X = 0 and adds exact zeros.
#pragma unroll
    for (int i = 0; i < GV_D; ++i) {
      const bool ok = 128 * (cb + i * GV_WAVES) + 32 * g < K;
      const float cf = ABS ? craw[i] : __fmul_rn(e4m3_value(c2b[i]), g1[i]);
      uint32_t L[4], H[4];
      gv_table(ok ? cf : 0.0f, lv, L, H);
      const uint32_t words[4] = {cw[i].x, cw[i].y, cw[i].z, cw[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 wv = gv_lookup8(words[q], L, H);
        const uint4 x = ok ? xv[i][q] : make_uint4(0, 0, 0, 0);
        acc = mfma16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, wv), acc);
      }
    }
  }
  // D[m][n]: lane holds X rows 4 g + v, weight row c
#pragma unroll
  for (int v = 0; v < 4; ++v) red[w][4 * g + v][c] = acc[v];

  // B rows n0 .. n0 + 15 (r columns each) and T = sum of the split-K
  // partials of X A^T (rows < M, columns < r) into LDS; partials are added
  // in split order from 0
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    // keeps the compiler from consuming (and waiting for) the early loads
    // before the weight stream
#pragma unroll
    for (int k = 0; k < GV_PRE; ++k) asm volatile("" : "+v"(tp[e][k]));
    const int idx = tid + e * GV_NT;
    if (idx < nb) sB[idx] = bval[e];
    if (idx < nt) {
      const int tm = idx / r, tj = idx % r;
      float s = 0.0f;
#pragma unroll
      for (int k = 0; k < GV_PRE; ++k) s += k < tsplit ? tp[e][k] : 0.0f;
      for (int k = GV_PRE; k < tsplit; ++k) s += tpart[((int64_t)k * M + tm) * rp + zc + tj];
      sT[tm][tj] = s;
      if (t_writer && T_out) T_out[(int64_t)tm * tld + zc + tj] = s;
    }
  }
  // r > 64: the rest of B and T
  for (int idx = tid + 2 * GV_NT; idx < nb; idx += GV_NT) {
    const int rr = idx / r, j = idx % r;
    sB[idx] = B[(int64_t)min(n0 + rr, N - 1) * r + j];
  }
  for (int idx = tid + 2 * GV_NT; idx < nt; idx += GV_NT) {
    const int m = idx / r, j = idx % r;
    float s = 0.0f;
    for (int k = 0; k < tsplit; ++k) s += tpart[((int64_t)k * M + m) * rp + zc + j];
    sT[m][j] = s;
    if (t_writer && T_out) T_out[(int64_t)m * tld + zc + j] = s;
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

// T partials for few tokens (M <= 16): part[ks][m][j] = sum over reduction
// slice ks (kslice columns, a multiple of 128) of X[m][k] R[j][k], for
// j < rows. R is the rank-side factor (A, or [A_1; ..; A_g]); a workgroup
// (4 wave64) owns 16 of its rows, and its waves take 128-column chunks round
// robin, two at a time with all loads in flight, like gemv_kernel with
// plain bf16 in place of the 4-bit codes.
constexpr int PS_WAVES = 4;
__global__ __launch_bounds__(64 * PS_WAVES) void proj_small_kernel(const uint16_t* __restrict__ X,
                                                                    const uint16_t* __restrict__ R, int M, int K,
                                                                    int rows, int rp, int kslice,
                                                                    float* __restrict__ part) {
  __shared__ float red[PS_WAVES][16][17];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j0 = blockIdx.x * 16, ks = blockIdx.y;
  const int c = l & 15, g = l >> 4;
  const XRows xr(X, M, K, c);
  const uint16_t* rrow = R + (int64_t)min(j0 + c, rows - 1) * K;  // rows past the end: clamped, not stored
  const int kb = ks * kslice, ke = min(K, kb + kslice);
  const int nch = (ke - kb + 127) / 128;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int cb = w; cb < nch; cb += 2 * PS_WAVES) {
    uint4 av[2][4], xv[2][4];
    bool ok[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = cb + i * PS_WAVES;  // wave-uniform
      const int k = kb + 128 * ch + 32 * g;
      ok[i] = ch < nch && k < ke;      // only the upper half of the last chunk can be missing
      const int kk = ok[i] ? k : kb;   // else a repeat of valid columns, masked below
#pragma unroll
      for (int q = 0; q < 4; ++q) av[i][q] = *reinterpret_cast<const uint4*>(rrow + kk + 8 * q);
      xr.load4(kk, xv[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // a masked slot adds exact zeros
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 a = ok[i] ? av[i][q] : make_uint4(0, 0, 0, 0);
        acc = mfma16(__builtin_bit_cast(bf16x8, xv[i][q]), __builtin_bit_cast(bf16x8, a), acc);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) red[w][4 * g + v][c] = acc[v];
  __syncthreads();
  const int m = tid >> 4, jj = tid & 15;
  if (m < M && j0 + jj < rows) {
    float t = 0.0f;
#pragma unroll
    for (int q = 0; q < PS_WAVES; ++q) t += red[q][m][jj];
    part[((int64_t)ks * M + m) * rp + j0 + jj] = t;
  }
}

}  // namespace

hipError_t launch_gemv(const uint16_t* X, const uint8_t* codes, const uint8_t* c2, const float* c1,
                       const float* absmax, int codebook, int N, int K, int M, const float* tpart, int tsplit,
                       int rp, const uint16_t* B, int r, float scale, uint16_t* Y, float* T_out, hipStream_t s,
                       int segN, int tld) {
  if (!tld) tld = r;
  if (absmax)
    hipLaunchKernelGGL(gemv_kernel<true>, dim3((N + 15) / 16), dim3(GV_NT), 0, s, X, codes, c2, c1, absmax, N, K,
                       M, tpart, tsplit, rp, B, r, scale, Y, T_out, segN, tld, host_levels(codebook));
  else
    hipLaunchKernelGGL(gemv_kernel<false>, dim3((N + 15) / 16), dim3(GV_NT), 0, s, X, codes, c2, c1, absmax, N, K,
                       M, tpart, tsplit, rp, B, r, scale, Y, T_out, segN, tld, host_levels(codebook));
  return hipGetLastError();
}

int proj_small_splits(int K, int* kslice) {
  int ts = (K + 1023) / 1024;
  if (ts > GV_PRE) ts = GV_PRE;
  const int ks = ((K + ts - 1) / ts + 127) / 128 * 128;
  *kslice = ks;
  return (K + ks - 1) / ks;
}

hipError_t launch_proj_small(const uint16_t* X, const uint16_t* R, int M, int K, int rows, int rp, float* part,
                             hipStream_t s) {
  int kslice = 0;
  const int ts = proj_small_splits(K, &kslice);
  hipLaunchKernelGGL(proj_small_kernel, dim3((rows + 15) / 16, ts), dim3(64 * PS_WAVES), 0, s, X, R, M, K, rows, rp,
                     kslice, part);
  return hipGetLastError();
}

}  // namespace qlora
