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
// Tile BM x BN outputs (256 x 256, or 512 x 128 for large M), 64-deep
// reduction steps (one NF4 block), 8 wave64 in (BM / 128) x (BN / 64), each
// wave 128 x 64 outputs = 8 x 4 v_mfma_f32_16x16x32_bf16 tiles (128 float32
// accumulators per lane), two waves per SIMD: while one wave keeps the matrix
// core busy the other issues its unpacking VALU work. The unpack work per
// step grows with BN and the MFMA work with BM x BN, so the 512 x 128 tile
// halves the unpacking per MFMA at the same LDS read volume per step. LDS
// holds two stages of the activation tile and of the weight tile (bf16,
// 128 or 160 KB in all, 16-byte chunks XOR-swizzled per row so MFMA operand
// reads are conflict free). The activation tile is streamed global -> LDS
// by LDS-DMA (global_load_lds_dwordx4); no registers involved.
//
// Weight tiles are unpacked in registers: each thread owns BN / 8 codes of
// one block per step (half or a quarter of it), builds the block's 16-entry
// table of bf16(q[c] * c^) (16 multiplies, 8 conversions, 8 byte shuffles)
// and maps every code through it with v_perm byte selects -- no LDS lookups,
// exact W~. Codes are fetched two steps ahead, activations one step ahead.
//
// Workgroups are ordered so that each XCD (workgroup id mod 8) owns a
// contiguous band of output tiles: the activation rows and weight columns
// it streams stay in that XCD's L2.
#include "launch.hpp"

namespace qlora {
namespace {

constexpr int BK = 64, NT = 512;

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 16-entry table of one block, as byte planes: L[j] holds the low bytes of
// entries 4j..4j+3, H[j] the high bytes.
struct BlockTable {
  uint32_t L[4], H[4];
};

__device__ __forceinline__ BlockTable make_table(float chat, const Levels& lv) {
  uint32_t P[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) P[i] = pack_bf16(__fmul_rn(lv.q[2 * i], chat), __fmul_rn(lv.q[2 * i + 1], chat));
  BlockTable t;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t.L[j] = perm(P[2 * j + 1], P[2 * j], 0x06040200u);
    t.H[j] = perm(P[2 * j + 1], P[2 * j], 0x07050301u);
  }
  return t;
}

// Look up the 8 codes of one word (element i in nibble i). Returns the bf16
// of even elements in E (e0|e2<<16, e4|e6<<16) and odd ones in O (e1|e3<<16,
// e5|e7<<16). Selector bytes: low 3 bits pick an entry inside a half table,
// bit 3 picks the half.
__device__ __forceinline__ void lookup8_split(uint32_t d, const BlockTable& t, uint32_t E[2],
                                              uint32_t O[2]) {
  const uint32_t se = d & 0x07070707u;
  const uint32_t so = (d >> 4) & 0x07070707u;
  const uint32_t ce = ((d >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t co = ((d >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t Le = perm(perm(t.L[3], t.L[2], se), perm(t.L[1], t.L[0], se), ce);
  const uint32_t He = perm(perm(t.H[3], t.H[2], se), perm(t.H[1], t.H[0], se), ce);
  const uint32_t Lo = perm(perm(t.L[3], t.L[2], so), perm(t.L[1], t.L[0], so), co);
  const uint32_t Ho = perm(perm(t.H[3], t.H[2], so), perm(t.H[1], t.H[0], so), co);
  E[0] = perm(He, Le, 0x05010400u);
  E[1] = perm(He, Le, 0x07030602u);
  O[0] = perm(Ho, Lo, 0x05010400u);
  O[1] = perm(Ho, Lo, 0x07030602u);
}

// The same 8 weights as 4 packed pairs in natural order (e0|e1<<16, ...).
__device__ __forceinline__ void lookup8(uint32_t d, const BlockTable& t, uint32_t out[4]) {
  uint32_t E[2], O[2];
  lookup8_split(d, t, E, O);
  out[0] = perm(O[0], E[0], 0x05040100u);
  out[1] = perm(O[0], E[0], 0x07060302u);
  out[2] = perm(O[1], E[1], 0x05040100u);
  out[3] = perm(O[1], E[1], 0x07060302u);
}

// 8 bf16 of row `row`, columns [col, col+8) of a [rows, ld] matrix; zeros
// outside [0, nrows) x [0, ncols). `vec` means ld % 8 == 0 (16-byte rows).
__device__ __forceinline__ uint4 load_row8(const uint16_t* __restrict__ base, int64_t ld, int row,
                                           int nrows, int col, int ncols, bool vec) {
  if (row >= nrows || col >= ncols) return make_uint4(0, 0, 0, 0);
  const uint16_t* p = base + (int64_t)row * ld + col;
  if (vec && col + 8 <= ncols) return *reinterpret_cast<const uint4*>(p);
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (col + i < ncols) ? p[i] : 0u;
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// LDS tiles are 256 rows x 64 bf16 (128 B rows, no padding), 16-byte chunks
// XOR-swizzled per row (lds_swz).
__device__ __forceinline__ int swz(int R) { return lds_swz(R); }
__device__ __forceinline__ int tile_off(int R, int c) { return R * 64 + 8 * (c ^ swz(R)); }

// The QW code words (8 QW codes of one block) a thread unpacks in a step,
// and their block constant.
template <int QW>
struct WPart {
  uint32_t c[QW];
  float chat;
};

// Thread -> weight codes of a step (QW words = 8 QW codes; TPR = 8 / QW
// threads share a block). Forward: thread t owns tile row t / TPR (weight
// row n0 + t / TPR), part t % TPR of the step's block. Input gradient: lane
// l owns weight row k0 + l, wave w the weight columns n0 + 8 QW w ..
template <bool TW, int QW>
__device__ __forceinline__ void wlane(int tid, int n0, int64_t& row, int64_t& col) {
  constexpr int TPR = 8 / QW;
  const int w = tid >> 6, l = tid & 63;
  if (!TW) {
    row = n0 + tid / TPR;
    col = 8 * QW * (tid % TPR);
  } else {
    row = l;
    col = n0 + 8 * QW * w;
  }
}

// Unpack word q (weights 8q .. 8q+7 of this thread's codes) into the
// weight tile of an LDS stage.
template <bool TW, int QW>
__device__ __forceinline__ void store_wword(uint32_t word, int q, const BlockTable& t,
                                            uint16_t* __restrict__ dst, int tid) {
  constexpr int TPR = 8 / QW;
  if (!TW) {
    // tile row tid / TPR, reduction chunk QW (tid % TPR) + q
    uint32_t o[4];
    lookup8(word, t, o);
    *reinterpret_cast<uint4*>(dst + tile_off(tid / TPR, QW * (tid % TPR) + q)) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    // element e of the word is W~[k0 + l][n0 + 8 QW w + 8 q + e]: tile row
    // 8 QW w + 8 q + e, reduction position l
    const int w = tid >> 6, l = tid & 63;
    uint32_t E[2], O[2];
    lookup8_split(word, t, E, O);
    const int r0 = 8 * QW * w + 8 * q;
    const uint16_t v[8] = {(uint16_t)E[0], (uint16_t)O[0], (uint16_t)(E[0] >> 16), (uint16_t)(O[0] >> 16),
                           (uint16_t)E[1], (uint16_t)O[1], (uint16_t)(E[1] >> 16), (uint16_t)(O[1] >> 16)};
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[tile_off(r0 + e, l >> 3) + (l & 7)] = v[e];
  }
}

template <bool TW, int QW>
__device__ __forceinline__ void store_wpart(const WPart<QW>& h, const Levels& lv, uint16_t* __restrict__ dst, int tid) {
  const BlockTable t = make_table(h.chat, lv);
#pragma unroll
  for (int q = 0; q < QW; ++q) store_wword<TW, QW>(h.c[q], q, t, dst, tid);
}

// QW code words at codes + (e >> 1) (e a multiple of 8 QW).
template <int QW>
__device__ __forceinline__ void load_words(const uint8_t* __restrict__ codes, int64_t e, uint32_t (&c)[QW]) {
  if (QW == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(codes + (e >> 1));
    c[0] = v.x; c[1] = v.y; c[2] = v.z; c[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(codes + (e >> 1));
    c[0] = v.x; c[1] = v.y;
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

template <int BM, int BN, bool TW, bool LORA, bool VEC, bool ABS>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(GemmParams p) {
  constexpr int WN = BN / 64;        // waves along the output columns
  constexpr int QW = BN / 64;        // code words unpacked per thread per step
  constexpr int XJ = BM / 64;        // activation LDS-DMA instructions per wave per step
  static_assert((BM / 128) * WN == NT / 64, "8 waves of 128 x 64");
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sA = smem;                // [2][BM * 64] activation tiles
  uint16_t* sB = smem + 2 * BM * 64;  // [2][BN * 64] weight tiles

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int wm = wu / WN, wn = wu % WN;

  // XCD-aware tile order: workgroup g runs on XCD g % 8; XCD x owns the
  // contiguous tile range [x * per, (x + 1) * per) in row-major tile order.
  // Split reduction (few tiles): work item u = tile t, split ks of the
  // reduction steps [ks kchunk, ks kchunk + kchunk); splits write float32
  // partial tiles that a second kernel sums.
  const int gn = (p.Nout + BN - 1) / BN;
  const int gm = (p.M + BM - 1) / BM;
  const int tiles = gn * gm;
  const int total = tiles * p.ksplit;
  const int per = (total + 7) / 8;
  const int u = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (u >= total) return;
  const int t = u / p.ksplit, ksp = u - t * p.ksplit;
  const int m0 = (t / gn) * BM;
  const int n0 = (t % gn) * BN;
  const int nk = (p.Kred + BK - 1) / BK;
  const int kchunk = p.ksplit > 1 ? p.kchunk : nk;
  const int kbeg = ksp * kchunk;
  const int kend = min(nk, kbeg + kchunk);

  // ---- activation tile of step kt -> stage st --------------------------------------
  // VEC (Kred % 64 == 0): LDS-DMA, 16 B per lane; instruction j of wave w
  // fills rows (BM / 8) w + 8 j .. +7 (1 KB), lane i the physical chunk i & 7
  // of row (BM / 8) w + 8 j + (i >> 3), i.e. the logical chunk
  // (i & 7) ^ swz(row). Rows past the end are clamped (they only feed
  // unstored outputs); steps past the end reload the last step (prefetch
  // overrun, never used). Lane byte offsets are fixed; the step moves a
  // uniform base.
  uint32_t xoff[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int R = (BM / 8) * wu + 8 * j + (l >> 3);
    const int row = min(m0 + R, p.M - 1);
    xoff[j] = (uint32_t)(row * p.Kred + 8 * ((l & 7) ^ swz(R))) * 2u;
  }
  auto load_x = [&](int kt, int st) {
    if (VEC) {
      const int ke = min(kt, nk - 1);
      const char* base = reinterpret_cast<const char*>(p.act) + (size_t)ke * (BK * 2);
#pragma unroll
      for (int j = 0; j < XJ; ++j)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(base + xoff[j]),
                                         (lds_void_t*)(sA + st * BM * 64 + ((BM / 8) * wu + 8 * j) * 64), 16, 0, 0);
    } else {
      const int k0 = kt * BK;
#pragma unroll
      for (int c = 0; c < BM / 64; ++c) {
        const int id = tid + NT * c;
        const uint4 v = load_row8(p.act, p.Kred, m0 + (id >> 3), p.M, k0 + 8 * (id & 7), p.Kred, false);
        *reinterpret_cast<uint4*>(&sA[st * BM * 64 + tile_off(id >> 3, id & 7)]) = v;
      }
    }
  };

  // ---- weight codes of step kt ------------------------------------------------------
  int64_t wrow, wcol;
  wlane<TW, QW>(tid, n0, wrow, wcol);
  const int64_t wstep = TW ? (int64_t)BK * p.wK : (int64_t)BK;  // elements per step
  // VEC: every step is a full 64 reduction rows (forward: columns), so only
  // the output side can run past the end: clamp it (unstored outputs).
  const int64_t wbase = TW ? wrow * p.wK + min(wcol, p.wK - 8 * QW)
                           : min(wrow, p.wN - 1) * p.wK + wcol;
  auto load_w = [&](int kt) -> WPart<QW> {
    WPart<QW> h;
    if (VEC) {
      const int ke = min(kt, nk - 1);
      const int64_t e = (int64_t)ke * wstep + wbase;
      load_words<QW>(p.codes, e, h.c);
      h.chat = block_const<ABS>(p.c2, p.c1, p.absmax, e >> 6);
    } else {
      // general reduction length: codes past the reduction end get c^ = 0
      // (their unpacked weights are exact zeros, which zero the reduction
      // tail); other out-of-range reads are clamped.
      int64_t n = TW ? (int64_t)kt * BK + wrow : wrow;
      int64_t col = TW ? wcol : (int64_t)kt * BK + wcol;
      const bool ok = n < p.wN && col < p.wK;
      n = min(n, p.wN - 1);
      col = min(col, p.wK - 8 * QW);
      const int64_t e = n * p.wK + col;
      load_words<QW>(p.codes, e, h.c);
      const float chat = block_const<ABS>(p.c2, p.c1, p.absmax, e >> 6);
      h.chat = ok ? chat : 0.0f;
    }
    return h;
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: stage 0 complete, codes of the next step in flight
  load_x(kbeg, 0);
  WPart<QW> wnext = load_w(kbeg);
  store_wpart<TW, QW>(wnext, p.lv, sB, tid);
  wnext = load_w(kbeg + 1);
  __builtin_amdgcn_s_waitcnt(0);  // stage 0 LDS-DMA landed (vmcnt = lgkmcnt = 0)
  __syncthreads();

  const int arow = wm * 128 + (l & 15);
  const int brow = wn * 64 + (l & 15);
  // logical chunk of a fragment: 4 kk + (l >> 4); all fragment rows of a
  // lane share swz(row) = swz(l & 15)
  const int ck0 = 8 * ((0 + (l >> 4)) ^ swz(l & 15));
  const int ck1 = 8 * ((4 + (l >> 4)) ^ swz(l & 15));

  for (int kt = kbeg; kt < kend; ++kt) {
    const int st = (kt - kbeg) & 1;
    load_x(kt + 1, st ^ 1);
    const WPart<QW> wcur = wnext;
    wnext = load_w(kt + 2);

    const uint16_t* a_s = sA + st * BM * 64;
    const uint16_t* b_s = sB + st * BN * 64;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ck = kk ? ck1 : ck0;
      bf16x8 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = lds_load8(reinterpret_cast<const __bf16*>(b_s + (brow + 16 * j) * 64 + ck));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 a = lds_load8(reinterpret_cast<const __bf16*>(a_s + (arow + 16 * i) * 64 + ck));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a, b[j], acc[i][j]);
      }
    }
    // unpack the next weight tile into the other stage (free since the last
    // barrier); steps past the end unpack a clamped block into an unused stage
    store_wpart<TW, QW>(wcur, p.lv, sB + (st ^ 1) * BN * 64, tid);
    __builtin_amdgcn_s_waitcnt(0);  // this step's LDS-DMA and LDS writes are complete
    __syncthreads();
  }

  if (LORA && ksp == 0) {
    // acc += lora_l[rows, :] lora_r[cols, :]^T, 64 rank columns per step
    // (rp is a multiple of 64, zero padded), staged through LDS stage 0 by
    // LDS-DMA like the main loop; the loop ended on a barrier.
    // grouped linears: this tile's segment of output columns uses its own
    // rp columns of lora_l (tiles never straddle segments)
    const int lcol0 = p.lora_seg ? (n0 / p.lora_seg) * p.rp : 0;
    for (int kr = 0; kr < p.rp; kr += BK) {
#pragma unroll
      for (int j = 0; j < BM / 64; ++j) {
        const int R = (BM / 8) * wu + 8 * j + (l >> 3);
        const int c = (l & 7) ^ swz(R);
        const int ra = min(m0 + R, p.M - 1);
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(p.lora_l + (int64_t)ra * p.lora_ld + lcol0 + kr + 8 * c),
                                         (lds_void_t*)(sA + ((BM / 8) * wu + 8 * j) * 64), 16, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < BN / 64; ++j) {
        const int R = (BN / 8) * wu + 8 * j + (l >> 3);
        const int c = (l & 7) ^ swz(R);
        const int rb = min(n0 + R, p.Nout - 1);
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(p.lora_r + (int64_t)rb * p.rp + kr + 8 * c),
                                         (lds_void_t*)(sB + ((BN / 8) * wu + 8 * j) * 64), 16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ck = kk ? ck1 : ck0;
        bf16x8 b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = lds_load8(reinterpret_cast<const __bf16*>(sB + (brow + 16 * j) * 64 + ck));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bf16x8 a = lds_load8(reinterpret_cast<const __bf16*>(sA + (arow + 16 * i) * 64 + ck));
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a, b[j], acc[i][j]);
        }
      }
      __syncthreads();
    }
  }

  // D layout of a 16 x 16 tile: lane holds rows 4 (l >> 4) + v, column l & 15
  float* __restrict__ part = p.ksplit > 1 ? p.part + (int64_t)ksp * p.M * p.Nout : nullptr;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + 16 * j + (l & 15);
      if (col >= p.Nout) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm * 128 + 16 * i + 4 * (l >> 4) + v;
        if (row < p.M) {
          if (part) {
            part[(int64_t)row * p.Nout + col] = acc[i][j][v];
          } else {
            const __bf16 h = (__bf16)acc[i][j][v];
            p.out[(int64_t)row * p.Nout + col] = __builtin_bit_cast(uint16_t, h);
          }
        }
      }
    }
}

// out = bf16(sum over the splits of the float32 partial tiles), fixed order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int ksplit, int64_t mn,
                                                             uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  // 16-byte partial loads need mn % 4 == 0; the 8-byte store an aligned out
  if (i + 4 <= mn && (mn & 3) == 0 && ((uintptr_t)out & 7) == 0) {
    float4 acc = *reinterpret_cast<const float4*>(part + i);
    for (int s = 1; s < ksplit; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)s * mn + i);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<uint2*>(out + i) = make_uint2(pack_bf16(acc.x, acc.y), pack_bf16(acc.z, acc.w));
    return;
  }
  for (int64_t e = i; e < min(mn, i + 4); ++e) {
    float a = part[e];
    for (int s = 1; s < ksplit; ++s) a += part[(int64_t)s * mn + e];
    out[e] = __builtin_bit_cast(uint16_t, (__bf16)a);
  }
}

template <int BM, int BN, bool TW, bool LORA, bool VEC, bool ABS>
hipError_t launch_variant(const GemmParams& p, hipStream_t s) {
  constexpr size_t smem_bytes = 2 * (BM + BN) * 64 * sizeof(uint16_t);
  static std::atomic<uint32_t> lds_ok{0};
  const hipError_t le =
      ensure_lds(reinterpret_cast<const void*>(&gemm_kernel<BM, BN, TW, LORA, VEC, ABS>), (int)smem_bytes, lds_ok);
  if (le != hipSuccess) return le;
  const int tiles = ((p.Nout + BN - 1) / BN) * ((p.M + BM - 1) / BM);
  const int grid = 8 * ((tiles * p.ksplit + 7) / 8);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, TW, LORA, VEC, ABS>), dim3(grid), dim3(NT), smem_bytes, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.ksplit <= 1) return e;
  const int64_t mn = (int64_t)p.M * p.Nout;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((mn / 4 + 255) / 256 + 1)), dim3(256), 0, s, p.part,
                     p.ksplit, mn, p.out);
  return hipGetLastError();
}

template <bool TW, bool LORA, bool ABS>
hipError_t launch_rows(const GemmParams& p, hipStream_t s) {
  // reductions in whole 64-element steps take the DMA / uniform-address
  // path; from 1024 rows on the 512 x 128 tile (half the unpacking per MFMA)
  const bool vec = p.Kred % BK == 0;
  if (p.M >= 1024)
    return vec ? launch_variant<512, 128, TW, LORA, true, ABS>(p, s)
               : launch_variant<512, 128, TW, LORA, false, ABS>(p, s);
  return vec ? launch_variant<256, 256, TW, LORA, true, ABS>(p, s)
             : launch_variant<256, 256, TW, LORA, false, ABS>(p, s);
}

template <bool TW, bool LORA>
hipError_t launch_fmt(const GemmParams& p, hipStream_t s) {
  return p.absmax ? launch_rows<TW, LORA, true>(p, s) : launch_rows<TW, LORA, false>(p, s);
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, bool transposed_w, hipStream_t s) {
  const bool lora = p.lora_l != nullptr;
  if (transposed_w) return lora ? launch_fmt<true, true>(p, s) : launch_fmt<true, false>(p, s);
  return lora ? launch_fmt<false, true>(p, s) : launch_fmt<false, false>(p, s);
}

}  // namespace qlora
