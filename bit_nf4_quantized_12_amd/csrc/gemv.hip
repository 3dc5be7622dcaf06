// Few-token forward (M <= 16): Y = X W~^T + s T B^T with T = X A^T, bound by
// reading the 4-bit weight from HBM.
//
// "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com),
// "Method": dequantise to BFloat16, multiply in 16-bit. The LoRA term follows
// "QLoRA: Efficient Fine-Tuning of Quantized Language Models"
// (mbrenndoerfer.com), section "Low-Rank Adaptation (LoRA)". With at most 16
// tokens each weight is used at most 16 times, so the kernel streams the codes
// exactly once, straight from HBM into registers.
//
// Two launches on the stream: the first computes T (each workgroup a few
// columns of T = X A^T over the whole reduction, float32, written once; the
// backward's recompute of T runs the same launch, so a saved and a recomputed
// T are bit-identical), the second streams the weight and adds s T B^T at its
// epilogue. With more than 8 tokens, extra workgroups of the first launch
// read the weight ahead of the second (into the Infinity Cache). (A single
// launch whose first workgroups published T to the others through a counter
// measured 2-3x slower: while the weight stream saturates HBM, the release,
// the atomic and the polls each wait behind that traffic, and the handoff
// took 5-10 us.)
//
//  * stream layout: 8 wave64; lane l has weight row c = l & 15 of the
//    workgroup and slot s = 4 w + (l >> 4) of 32; slot s takes the 64-weight
//    blocks s, s + 32, s + 64, .. of its row, one block (32 B of codes, one
//    constant) per step, the loads of two steps issued together. A block's 16-entry
//    table of bf16(q[c] c^) turns its 8 code words into 8
//    v_mfma_f32_16x16x32_bf16 B operands (v_perm byte selects, exact W~); the
//    A operand is X (token m = l & 15, the same 64 columns; tokens past M read
//    as zero by out-of-range buffer loads, no memory traffic).
//  * the 8 waves' partial 16 x 16 tiles meet in LDS; the epilogue adds
//    s T B^T in float32 (four accumulators per output) before the one bf16
//    rounding.
#include "launch.hpp"

namespace qlora {
namespace {

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 16-entry bf16(q[c] * c^) table as byte planes: L[j] holds the low bytes of
// entries 4j .. 4j+3, H[j] the high bytes.
__device__ __forceinline__ void ft_table(float chat, const Levels& lv, uint32_t L[4], uint32_t H[4]) {
  uint32_t P[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) P[i] = pack_bf16(__fmul_rn(lv.q[2 * i], chat), __fmul_rn(lv.q[2 * i + 1], chat));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    L[j] = perm(P[2 * j + 1], P[2 * j], 0x06040200u);
    H[j] = perm(P[2 * j + 1], P[2 * j], 0x07050301u);
  }
}

// 8 codes (element i in nibble i) -> 8 bf16 of W~ in natural order. Selector
// bytes: the low 3 bits pick an entry inside a half table, bit 3 the half.
__device__ __forceinline__ uint4 ft_lookup8(uint32_t d, const uint32_t L[4], const uint32_t H[4]) {
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

constexpr int FT_WAVES = 8;
constexpr int FT_NT = 64 * FT_WAVES;
constexpr int FT_SLOTS = 4 * FT_WAVES;  // 64-column blocks per workgroup step
constexpr int FT_D = 2;                 // steps whose loads are issued together
constexpr int FT_RMAX = 256;            // rank columns of one segment

// 16 B of a bf16 matrix through a buffer resource: zero when off is past the
// resource's size (then nothing is read).
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Row `row` of a bf16 matrix [rows, K] as a buffer; rows past `rows` read as
// zero (this lane's offset is then the buffer's end).
struct RowBuf {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t base, end;
  __device__ RowBuf(const uint16_t* p, int rows, int K, int row) {
    end = (uint32_t)rows * (uint32_t)K * 2u;  // < 2^32 (checked on the host)
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, (int)end, 0x00020000);
    base = row < rows ? (uint32_t)row * (uint32_t)K * 2u : end;
  }
  // the 64 bf16 of block b (columns 64 b ..) of this lane's row
  __device__ __forceinline__ void load_block(int b, uint4 (&v)[8]) const {
    const uint32_t o = base == end ? end : base + 128u * (uint32_t)b;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = buf_load16(rs, o == end ? end : o + 16u * i);
  }
};

}  // namespace

struct FewTokParams {
  const uint16_t* X;     // [M, K]
  const uint8_t* codes;  // weight [N, K]
  const uint8_t* c2;
  const float* c1;
  const float* absmax;   // fp32 block constants (no double quantisation), or null
  const uint16_t* A;     // [R, K] (the segments' A stacked)
  const uint16_t* B;     // [N, rseg]
  uint16_t* Y;           // [M, N]
  float* T;              // [M, R] float32: written by the producers
  int M, N, K, R, rseg, segN;  // segN: rows per segment (grouped), 0 = one segment
  int P, J;              // T workgroups, T columns each (T launch)
  float scale;
  Levels lv;
};

namespace {

// Sum over the 64 lanes of a wave in a fixed butterfly order: xor 1 and 2
// inside quads, the half-row and row mirrors (lane i with 7 - i, then with
// 15 - i), then xor 16 and 32. Every step adds two values whose order does
// not matter (a + b == b + a), so all lanes end with the same bits, the
// same on every run.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Producer: T[m][j] = sum_k X[m][k] A[j][k] for j in [j0, j0 + J) (J <= 16),
// m < M. Per column j and group of up to 16 tokens, thread t takes the
// 8-column chunks t, t + FT_NT, .. (the A chunk and the tokens' X chunks in
// flight together) and multiplies in float32 (bf16 products are exact); the
// FT_NT partial sums of each (m, j) are added in a fixed order: within each
// wave in registers (wave_sum), then the 8 wave sums in wave order. The
// T-only launch of the backward runs this same code.
constexpr int FT_PM = 16;  // tokens per pass (M <= 16: one pass)
constexpr int FT_W = FT_NT / 64;
__device__ void ft_produce(const FewTokParams& p, int j0, float* red) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int nch = p.K >> 3;
  const int nj = min(p.J, p.R - j0);
  for (int jj = 0; jj < nj; ++jj) {
    const uint16_t* arow = p.A + (int64_t)(j0 + jj) * p.K;
    for (int m0 = 0; m0 < p.M; m0 += FT_PM) {
      const int mc = min(FT_PM, p.M - m0);  // tokens in this pass (uniform)
      float acc[FT_PM];
#pragma unroll
      for (int i = 0; i < FT_PM; ++i) acc[i] = 0.0f;
      for (int ch = tid; ch < nch; ch += FT_NT) {
        const uint4 av = *reinterpret_cast<const uint4*>(arow + 8 * ch);
        uint4 xv[FT_PM];
        const uint16_t* xp = p.X + (int64_t)m0 * p.K + 8 * ch;
#pragma unroll
        for (int i = 0; i < FT_PM; ++i, xp += p.K)
          if (i < mc) xv[i] = *reinterpret_cast<const uint4*>(xp);
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int i = 0; i < FT_PM; ++i) {
          if (i >= mc) continue;
          const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
          float a = acc[i];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            a = __builtin_fmaf(bf16lo(xw[q]), bf16lo(aw[q]), a);
            a = __builtin_fmaf(bf16hi(xw[q]), bf16hi(aw[q]), a);
          }
          acc[i] = a;
        }
      }
#pragma unroll
      for (int i = 0; i < FT_PM; ++i)
        if (i < mc) acc[i] = wave_sum(acc[i]);
      if (l == 0) {
#pragma unroll
        for (int i = 0; i < FT_PM; ++i)
          if (i < mc) red[i * FT_W + w] = acc[i];
      }
      __syncthreads();
      if (tid < mc) {
        float t = red[tid * FT_W];
#pragma unroll
        for (int v = 1; v < FT_W; ++v) t += red[tid * FT_W + v];
        p.T[(int64_t)(m0 + tid) * p.R + j0 + jj] = t;
      }
      __syncthreads();  // red is reused by the next pass
    }
  }
}

// Workgroups P .. of the T launch read the stored weight that the next
// launch streams (codes, then the block constants), 16 bytes per lane, 8
// loads in flight, and drop the data: the lines land in the Infinity Cache
// while T's reduction chain, which leaves HBM idle, runs, and the weight
// stream then reads them from there instead of from HBM.
constexpr int FT_PF_LOADS = 8;
__device__ void ft_touch(const uint8_t* base, size_t bytes, int wg, int nwg) {
  const size_t chunk = (size_t)FT_NT * 16 * FT_PF_LOADS;  // bytes per workgroup round
  const size_t n16 = bytes / 16;  // whole 16-byte pieces (a shorter tail is left out)
  if (n16 == 0) return;
  uint32_t sink = 0;
  for (size_t c = (size_t)wg * chunk; c < bytes; c += (size_t)nwg * chunk) {
    uint4 v[FT_PF_LOADS];
#pragma unroll
    for (int i = 0; i < FT_PF_LOADS; ++i) {
      const size_t e = min(c / 16 + (size_t)i * FT_NT + threadIdx.x, n16 - 1);
      v[i] = reinterpret_cast<const uint4*>(base)[e];
    }
#pragma unroll
    for (int i = 0; i < FT_PF_LOADS; ++i) sink ^= v[i].x;
  }
  asm volatile("" ::"v"(sink));
}

// T = X A^T: workgroup w < P computes columns w J .. w J + J - 1; the
// others (forward only) read the weight ahead of its stream.
__global__ __launch_bounds__(FT_NT) void fewtok_t_kernel(FewTokParams p) {
  __shared__ float pred[FT_PM * FT_W];
  if ((int)blockIdx.x >= p.P) {
    const int wg = blockIdx.x - p.P, nwg = gridDim.x - p.P;
    const size_t n = (size_t)p.N * p.K;
    ft_touch(p.codes, n / 2, wg, nwg);
    if (p.absmax)
      ft_touch(reinterpret_cast<const uint8_t*>(p.absmax), (n / 64) * 4, wg, nwg);
    else
      ft_touch(p.c2, n / 64, wg, nwg);
    return;
  }
  ft_produce(p, blockIdx.x * p.J, pred);
}

// Y = X W~^T + scale T_z B^T: workgroup w owns weight rows 16 w .. 16 w + 15.
template <bool ABS>
__global__ __launch_bounds__(FT_NT) __attribute__((amdgpu_waves_per_eu(4))) void fewtok_kernel(FewTokParams p) {
  __shared__ float red[FT_WAVES][16][17];
  __shared__ float sT[16][FT_RMAX + 4];
  __shared__ uint16_t sB[16][FT_RMAX + 8];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = l & 15, g = l >> 4;
  const int slot = 4 * w + g;
  const int n0 = blockIdx.x * 16;
  const int n = min(n0 + c, p.N - 1);  // rows past N: clamped read, result not stored
  const int nbk = p.K >> 6;
  const int64_t rowb = (int64_t)n * nbk;  // first block of this lane's row
  const RowBuf xr(p.X, p.M, p.K, c);
  const int steps = (nbk + FT_SLOTS - 1) / FT_SLOTS;
  // grouped linears: rows of segment z use T columns z rseg .. + rseg
  const int zc = p.segN ? (n0 / p.segN) * p.rseg : 0;

  // T[m][zc .. zc + rseg) (float32, written by the previous launch on this
  // stream), zero-padded to a multiple of 4 columns: elements idx = tid and
  // tid + FT_NT of the [M, rs4] block fetched before the weight stream (all
  // of it for M rs4 <= 1024), the rest at the epilogue
  const int rs4 = (p.rseg + 3) & ~3;
  auto t_elem = [&](int idx) -> float {
    const int m = idx / rs4, j = idx - m * rs4;
    return idx < p.M * rs4 && j < p.rseg ? p.T[(int64_t)m * p.R + zc + j] : 0.0f;
  };
  const float tv0 = t_elem(tid), tv1 = t_elem(tid + FT_NT);

  // B rows n0 .. n0 + 15 (rseg bf16 each), fetched before the weight stream:
  // 16-byte pieces when rseg % 8 == 0, else single elements (<= 8 a thread)
  const bool bvec = (p.rseg & 7) == 0;
  const int nbv = bvec ? 2 * p.rseg : 16 * p.rseg;
  uint4 bv = make_uint4(0, 0, 0, 0);
  uint16_t bs[8];
  if (bvec) {
    if (tid < nbv) {
      const int br = tid / (p.rseg / 8), bc = tid % (p.rseg / 8);
      bv = *reinterpret_cast<const uint4*>(p.B + (int64_t)min(n0 + br, p.N - 1) * p.rseg + 8 * bc);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = tid + FT_NT * k;
      const int br = idx / p.rseg, bc = idx - br * p.rseg;
      bs[k] = idx < nbv ? p.B[(int64_t)min(n0 + br, p.N - 1) * p.rseg + bc] : (uint16_t)0;
    }
  }

  // Loads of step i: the lane's 32 B of codes, its block constant, and the
  // 64 X values of token c at the block's columns. Addresses are clamped so
  // that every load is unconditional; a step past the row's end is masked.
  struct Step {
    uint4 cw0, cw1;
    uint4 xv[8];
    float craw;
    uint32_t c2b;
    float g1;
  };
  auto issue = [&](int i, Step& st) {
    const int b = min(slot + FT_SLOTS * i, nbk - 1);
    const int64_t e = rowb + b;  // block index
    const uint4* cp = reinterpret_cast<const uint4*>(p.codes + 32 * e);
    st.cw0 = cp[0];
    st.cw1 = cp[1];
    if (ABS) {
      st.craw = p.absmax[e];
    } else {
      st.c2b = p.c2[e];
      st.g1 = p.c1[e >> 8];
    }
    xr.load_block(b, st.xv);
  };

  // Batches of FT_D steps: a batch's loads are all issued, then consumed in
  // order (no load is outstanding across the loop edge, so every wait is a
  // counted one). A step past the row's end reloads a valid block and is
  // masked: c^ = 0 and X = 0 add exact zeros.
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < steps; i += FT_D) {
    Step st[FT_D];
    // scheduling barriers keep the issue order (step 0's loads before step
    // 1's) and the compute order, so step d waits only for its own loads
#pragma unroll
    for (int d = 0; d < FT_D; ++d) {
      issue(i + d, st[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int d = 0; d < FT_D; ++d) {
      if (d) __builtin_amdgcn_sched_barrier(0);
      const bool ok = slot + FT_SLOTS * (i + d) < nbk;
      const float cf = ABS ? st[d].craw : __fmul_rn(e4m3_value(st[d].c2b), st[d].g1);
      uint32_t L[4], H[4];
      ft_table(ok ? cf : 0.0f, p.lv, L, H);
      const uint32_t words[8] = {st[d].cw0.x, st[d].cw0.y, st[d].cw0.z, st[d].cw0.w,
                                 st[d].cw1.x, st[d].cw1.y, st[d].cw1.z, st[d].cw1.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint4 wv = ft_lookup8(words[t], L, H);
        const uint4 x = ok ? st[d].xv[t] : make_uint4(0, 0, 0, 0);
        acc = mfma16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, wv), acc);
      }
    }
  }
  // D[m][row]: lane holds tokens 4 g + v, weight row c
#pragma unroll
  for (int v = 0; v < 4; ++v) red[w][4 * g + v][c] = acc[v];
  if (bvec) {
    if (tid < nbv) {
      const int br = tid / (p.rseg / 8), bc = tid % (p.rseg / 8);
      *reinterpret_cast<uint4*>(&sB[br][8 * bc]) = bv;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = tid + FT_NT * k;
      const int br = idx / p.rseg, bc = idx - br * p.rseg;
      if (idx < nbv) sB[br][bc] = bs[k];
    }
  }

  for (int idx = tid; idx < p.M * rs4; idx += FT_NT) {
    const float v = idx == tid ? tv0 : idx == tid + FT_NT ? tv1 : t_elem(idx);
    sT[idx / rs4][idx % rs4] = v;
  }
  if (tid < 16 * 4) sB[tid >> 2][p.rseg + (tid & 3)] = 0;
  __syncthreads();
  // outputs (m, row): y = sum of the waves' tiles + s sum_j T[m][j] B[row][j]
  if (tid < 16 * p.M) {
    const int m = tid >> 4, rr = tid & 15;
    float y = 0.0f;
#pragma unroll
    for (int q = 0; q < FT_WAVES; ++q) y += red[q][m][rr];
    // columns rseg .. rseg+3 of sT / sB are zero
    float lo[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < p.rseg; j += 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) lo[e] = __builtin_fmaf(sT[m][j + e], bf16lo(sB[rr][j + e]), lo[e]);
    }
    const float lsum = (lo[0] + lo[1]) + (lo[2] + lo[3]);
    const float out = y + p.scale * lsum;
    if (n0 + rr < p.N) p.Y[(int64_t)m * p.N + n0 + rr] = __builtin_bit_cast(uint16_t, (__bf16)out);
  }
}

}  // namespace

// T launch: J = ceil(R / 256) T columns per workgroup (at most 16, so R <=
// 4096), P = ceil(R / J) workgroups.
static void ft_producers(int R, int* P, int* J) {
  int j = (R + 255) / 256;
  if (j < 1) j = 1;
  *J = j;
  *P = (R + j - 1) / j;
}

hipError_t launch_fewtok(const uint16_t* X, const uint8_t* codes, const uint8_t* c2, const float* c1,
                         const float* absmax, int codebook, int N, int K, int M, const uint16_t* A, int R,
                         const uint16_t* B, int rseg, int segN, float scale, uint16_t* Y, float* T,
                         hipStream_t s) {
  FewTokParams p;
  p.X = X;
  p.codes = codes;
  p.c2 = c2;
  p.c1 = c1;
  p.absmax = absmax;
  p.A = A;
  p.B = B;
  p.Y = Y;
  p.T = T;
  p.M = M;
  p.N = N;
  p.K = K;
  p.R = R;
  p.rseg = rseg;
  p.segN = segN;
  ft_producers(R, &p.P, &p.J);
  p.scale = scale;
  p.lv = host_levels(codebook);
  // forward with more than 8 tokens: one reading workgroup per 64 KB of the
  // stored weight, at most 256 beside the T workgroups. (With 8 tokens or
  // fewer the reading outlasts T's own chain and the stream gains less than
  // that: measured slower at M = 1, 4-7 % faster at M = 16.)
  const size_t wbytes = (size_t)N * K / 2;
  const int npf = Y && M > 8 ? (int)std::min<size_t>(256, (wbytes + 65535) / 65536) : 0;
  hipLaunchKernelGGL(fewtok_t_kernel, dim3(p.P + npf), dim3(FT_NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !Y) return e;
  const dim3 grid((N + 15) / 16);
  if (absmax)
    hipLaunchKernelGGL(fewtok_kernel<true>, grid, dim3(FT_NT), 0, s, p);
  else
    hipLaunchKernelGGL(fewtok_kernel<false>, grid, dim3(FT_NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
