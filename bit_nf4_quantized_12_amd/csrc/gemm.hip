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
// Tile BM x BN outputs (256 x 256, or 512 x 128 for large M, or 128 x 128
// when even 256 x 256 leaves most CUs idle), 64-deep reduction steps (one NF4
// block), 8 wave64 in (BM / WM) x (BN / 64), each wave WM x 64 outputs
// (WM = 128: 8 x 4 v_mfma_f32_16x16x32_bf16 tiles, 128 float32 accumulators
// per lane; WM = 32 for the 128 x 128 tile), two waves per SIMD: while one wave keeps the matrix
// core busy the other issues its unpacking VALU work. The unpack work per
// step grows with BN and the MFMA work with BM x BN, so the 512 x 128 tile
// halves the unpacking per MFMA at the same LDS read volume per step. LDS
// holds two stages of the activation tile and of the weight tile (bf16,
// 64, 128 or 160 KB in all, 16-byte chunks XOR-swizzled per row so MFMA operand
// reads are conflict free). The activation tile is streamed global -> LDS
// by LDS-DMA, no registers involved: 512-row tiles issue it as buffer loads
// spread over the first half-step's MFMAs, the others as global loads at
// the top of the step. 512-row tiles also touch the activation band in L2
// three steps ahead of that DMA.
//
// Weight tiles are unpacked in registers: each thread owns BN / 8 codes of
// one block per step (a quarter or half of it), the block's 16-entry table
// of bf16(q[c] * c^) is built by the lanes that share the block (with a
// quarter each, every lane of a quad computes 4 entries and DPP broadcasts
// them; with a half, each lane computes all 16), and every code is mapped
// through it with v_perm byte selects -- no LDS lookups, exact W~. Codes are
// fetched two steps ahead, activations one step ahead.
//
// Workgroups are ordered so that each XCD (workgroup id mod 8) owns a
// contiguous band of output tiles: the activation rows and weight columns
// it streams stay in that XCD's L2. Outputs are stored as bf16 pairs of
// adjacent columns (or float32 partials when the reduction is split).
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

// The table of a block shared by the 4 lanes of a quad (forward orientation
// with 2 code words per thread: lanes 4r .. 4r + 3 hold the 4 parts of tile
// row r, one block): lane p computes entries 4p .. 4p + 3 from its own levels
// lq = q[4p .. 4p + 3] and the quad exchanges the byte planes by DPP. The
// table is bit-identical to make_table's (the same products, packed and
// permuted the same way, only computed by one lane each).
__device__ __forceinline__ BlockTable make_table_quad(float chat, const float (&lq)[4]) {
  const uint32_t pa = pack_bf16(__fmul_rn(lq[0], chat), __fmul_rn(lq[1], chat));
  const uint32_t pb = pack_bf16(__fmul_rn(lq[2], chat), __fmul_rn(lq[3], chat));
  const int lo = (int)perm(pb, pa, 0x06040200u), hi = (int)perm(pb, pa, 0x07050301u);
  BlockTable t;
  // quad_perm [j, j, j, j]: every lane of the quad reads lane j
  t.L[0] = (uint32_t)__builtin_amdgcn_mov_dpp(lo, 0x00, 0xF, 0xF, false);
  t.L[1] = (uint32_t)__builtin_amdgcn_mov_dpp(lo, 0x55, 0xF, 0xF, false);
  t.L[2] = (uint32_t)__builtin_amdgcn_mov_dpp(lo, 0xAA, 0xF, 0xF, false);
  t.L[3] = (uint32_t)__builtin_amdgcn_mov_dpp(lo, 0xFF, 0xF, 0xF, false);
  t.H[0] = (uint32_t)__builtin_amdgcn_mov_dpp(hi, 0x00, 0xF, 0xF, false);
  t.H[1] = (uint32_t)__builtin_amdgcn_mov_dpp(hi, 0x55, 0xF, 0xF, false);
  t.H[2] = (uint32_t)__builtin_amdgcn_mov_dpp(hi, 0xAA, 0xF, 0xF, false);
  t.H[3] = (uint32_t)__builtin_amdgcn_mov_dpp(hi, 0xFF, 0xF, 0xF, false);
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
// The input gradient's weight tiles take the same swizzle with the chunk
// also XORed by 2 ((R >> 4) & 3): a fragment read covers 16 consecutive rows
// (one group, a constant extra XOR: still conflict free), while its unpack
// has the 4 lanes of a quad write one reduction position of 4 rows 16 apart,
// which the extra XOR sends to different banks.
template <bool TW>
__device__ __forceinline__ int bswz(int R) { return TW ? lds_swz(R) ^ (((R >> 4) & 3) << 1) : lds_swz(R); }
template <bool TW>
__device__ __forceinline__ int btile_off(int R, int c) { return R * 64 + 8 * (c ^ bswz<TW>(R)); }

// The QW code words (8 QW codes of one block) a thread unpacks in a step,
// and their block constant.
template <int QW>
struct WPart {
  uint32_t c[QW];
  float g;       // c1 of the block's group, or the block's fp32 absmax (no DQ)
  uint32_t c2b;  // E4M3 byte of the block constant (double quantisation)
  bool ok;       // false: codes past the reduction end (their c^ is 0)
};

// The block constant c^ of a WPart, decoded when the codes are unpacked (not
// when they are loaded, so that the loads can stay in flight).
template <bool ABS, int QW>
__device__ __forceinline__ float wpart_chat(const WPart<QW>& h) {
  const float c = ABS ? h.g : __fmul_rn(e4m3_value(h.c2b), h.g);
  return h.ok ? c : 0.0f;
}

// Thread -> weight codes of a step (QW words = 8 QW codes; TPR = 8 / QW
// threads share a block). Forward: thread t owns tile row t / TPR (weight
// row n0 + t / TPR), part t % TPR of the step's block. Input gradient with 2
// words a thread: the 4 lanes of a quad share one block, weight row
// k0 + 2 ((l >> 2) & 7) + (l >> 5) + 16 (w & 3), columns
// n0 + 64 (w >> 2) + 16 (l & 3) .. (a quad reads 32 contiguous bytes and
// builds one table; lanes l and l + 32 hold adjacent rows of the same
// columns); with 4 words: lane l owns weight row k0 + l, wave w the weight
// columns n0 + 8 QW w ..
template <bool TW, int QW>
__device__ __forceinline__ void wlane(int tid, int n0, int64_t& row, int64_t& col) {
  constexpr int TPR = 8 / QW;
  const int w = tid >> 6, l = tid & 63;
  if (!TW) {
    row = n0 + tid / TPR;
    col = 8 * QW * (tid % TPR);
  } else if (QW == 2) {
    row = 2 * ((l >> 2) & 7) + (l >> 5) + 16 * (w & 3);
    col = n0 + 64 * (w >> 2) + 16 * (l & 3);
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
    *reinterpret_cast<uint4*>(dst + btile_off<TW>(tid / TPR, QW * (tid % TPR) + q)) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    // element e of the word is W~[k0 + k][n0 + r0 + e] (wlane's row k and
    // column r0 + e of the tile): tile row r0 + e, reduction position k
    const int w = tid >> 6, l = tid & 63;
    uint32_t E[2], O[2];
    lookup8_split(word, t, E, O);
    const int r0 = 8 * QW * w + 8 * q;
    const int k = l;
    const uint16_t v[8] = {(uint16_t)E[0], (uint16_t)O[0], (uint16_t)(E[0] >> 16), (uint16_t)(O[0] >> 16),
                           (uint16_t)E[1], (uint16_t)O[1], (uint16_t)(E[1] >> 16), (uint16_t)(O[1] >> 16)};
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[btile_off<TW>(r0 + e, k >> 3) + (k & 7)] = v[e];
  }
}

// Input gradient, 2 words a thread: lanes l and l + 32 hold reduction
// positions k and k + 1 (k even) of the same 16 columns. One lane swap per
// packed pair leaves each lane both positions of 8 columns (lanes below 32:
// the first 8, the others: the last 8), stored as bf16 pairs k | k + 1.
__device__ __forceinline__ void store_tw2(const uint32_t (&c)[2], const BlockTable& t, uint16_t* __restrict__ dst,
                                          int tid) {
  const int w = tid >> 6, l = tid & 63;
  uint32_t E0[2], O0[2], E1[2], O1[2];
  lookup8_split(c[0], t, E0, O0);
  lookup8_split(c[1], t, E1, O1);
  const uint32_t a[4] = {E0[0], O0[0], E0[1], O0[1]};
  const uint32_t b[4] = {E1[0], O1[0], E1[1], O1[1]};
  uint32_t X[4], Y[4];  // split pairs of positions k (X) and k + 1 (Y)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(a[i], b[i], false, false);
    X[i] = r[0];
    Y[i] = r[1];
  }
  const int k = 2 * ((l >> 2) & 7) + 16 * (w & 3);
  const int r0 = 64 * (w >> 2) + 16 * (l & 3) + 8 * (l >> 5);
  const uint32_t v[8] = {perm(Y[0], X[0], 0x05040100u), perm(Y[1], X[1], 0x05040100u),
                         perm(Y[0], X[0], 0x07060302u), perm(Y[1], X[1], 0x07060302u),
                         perm(Y[2], X[2], 0x05040100u), perm(Y[3], X[3], 0x05040100u),
                         perm(Y[2], X[2], 0x07060302u), perm(Y[3], X[3], 0x07060302u)};
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<uint32_t*>(dst + btile_off<true>(r0 + e, k >> 3) + (k & 7)) = v[e];
}

template <bool TW, int QW>
__device__ __forceinline__ void store_wpart(const WPart<QW>& h, float chat, const Levels& lv, const float (&lq)[4],
                                            uint16_t* __restrict__ dst, int tid) {
  const BlockTable t = QW == 2 ? make_table_quad(chat, lq) : make_table(chat, lv);
  if constexpr (TW && QW == 2) {
    store_tw2(h.c, t, dst, tid);
  } else {
#pragma unroll
    for (int q = 0; q < QW; ++q) store_wword<TW, QW>(h.c[q], q, t, dst, tid);
  }
}

// QW code words at codes + (e >> 1) (e a multiple of 8 QW).
template <int QW>
__device__ __forceinline__ void load_words(const uint8_t* __restrict__ codes, int64_t e, uint32_t (&c)[QW]) {
  if constexpr (QW == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(codes + (e >> 1));
    c[0] = v.x; c[1] = v.y; c[2] = v.z; c[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(codes + (e >> 1));
    c[0] = v.x; c[1] = v.y;
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// Buffer resource over `bytes` bytes at p (raw: no stride, no swizzle), and
// a 16-byte-per-lane LDS-DMA through it (buffer_load_dwordx4 ... lds) to the
// LDS row block at `lds`, lane i filling lds + 16 i. The builtins sit in
// device functions: written directly in a kernel body, the buffer DMA
// builtin drops the kernel's host-side launch stub.
struct BufRsrc {
  __amdgpu_buffer_rsrc_t rs;
  __device__ BufRsrc(const void* p, uint32_t bytes) {
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
  }
};
__device__ __forceinline__ void dma16(const BufRsrc& r, uint16_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.rs, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}
// One dword through the same resource: brings its cache line into L2 (the
// value itself is not needed).
__device__ __forceinline__ uint32_t touch4(const BufRsrc& r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r.rs, (int)voff, (int)soff, 0);
}

template <int BM, int BN, bool TW, bool LORA, bool VEC, bool ABS>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(GemmParams p) {
  constexpr int WN = BN / 64;        // waves along the output columns
  constexpr int WM = BM * WN / 8;    // output rows per wave (8 waves)
  constexpr int MI = WM / 16;        // 16-row MFMA tiles per wave
  constexpr int QW = BN / 64;        // code words unpacked per thread per step
  constexpr int XJ = BM / 64;        // activation LDS-DMA instructions per wave per step
  static_assert((BM / WM) * WN == NT / 64 && WM % 16 == 0, "8 waves of WM x 64");
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
  // uniform offset. 512-row tiles load through a buffer resource based at
  // the tile's first row (measured 0.5-2 % faster there than the same DMA as
  // a global load; the smaller tiles keep the global form, which needs fewer
  // registers). The whole activation is below 2^32 bytes (its M Kred
  // elements are below 2^31), so every offset fits 32 bits and every read is
  // inside the tensor. Instructions jb .. je - 1 of the step are issued.
  constexpr bool XBUF = BM == 512;
  const int xrow0 = XBUF ? m0 : 0;
  uint32_t xoff[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int R = (BM / 8) * wu + 8 * j + (l >> 3);
    const int row = min(m0 + R, p.M - 1);
    xoff[j] = (uint32_t)((row - xrow0) * p.Kred + 8 * ((l & 7) ^ swz(R))) * 2u;
  }
  const BufRsrc xrs(reinterpret_cast<const uint16_t*>(p.act) + (size_t)xrow0 * p.Kred,
                    (uint32_t)((size_t)(p.M - xrow0) * p.Kred * 2u));
  auto load_x = [&](int kt, int st, int jb, int je) {
    if (VEC) {
      const int ke = min(kt, nk - 1);
#pragma unroll
      for (int j = jb; j < je; ++j) {
        uint16_t* dst = sA + st * BM * 64 + ((BM / 8) * wu + 8 * j) * 64;
        if (XBUF) {
          dma16(xrs, dst, xoff[j], (uint32_t)ke * (BK * 2));
        } else {
          const char* src = reinterpret_cast<const char*>(p.act) + (size_t)ke * (BK * 2) + xoff[j];
          __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
        }
      }
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

  // L2 prefetch of the activation tile PFD steps ahead (512-row tiles). The
  // workgroups an XCD runs at once stream the same activation band (the tile
  // order gives them consecutive output-column tiles), so each touches 1/32
  // of the band's lines -- 16 rows, two 64-byte halves of each row's
  // 128-byte step segment, 2 rows per wave (lane l takes address l & 3, so
  // the instruction needs no branch) -- and the band's next tiles are in
  // that XCD's L2 before the DMA asks for them. Without it the DMA of a band
  // larger than the Infinity Cache waits on HBM at the end of the step. The
  // loaded dwords are discarded.
  constexpr bool PF = VEC && BM == 512;
  constexpr int PFD = 3;
  uint32_t pfoff = 0, pf = 0;
  if (PF) {
    const int R = 16 * ((t % gn) & 31) + 2 * wu + ((l >> 1) & 1);
    const int row = min(m0 + R, p.M - 1);
    pfoff = (uint32_t)((row - xrow0) * p.Kred) * 2u + (uint32_t)(l & 1) * 64u;
  }
  auto prefetch_x = [&](int kt) {
    if (PF) pf = touch4(xrs, pfoff, (uint32_t)min(kt, nk - 1) * (BK * 2));
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
      if (ABS) {
        h.g = p.absmax[e >> 6];
      } else {
        h.c2b = p.c2[e >> 6];
        h.g = p.c1[e >> 14];
      }
      h.ok = true;
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
      if (ABS) {
        h.g = p.absmax[e >> 6];
      } else {
        h.c2b = p.c2[e >> 6];
        h.g = p.c1[e >> 14];
      }
      h.ok = ok;
    }
    return h;
  };

  // this lane's 4 levels for the quad-shared table (2 words per thread)
  float lq[4];
  {
    const int qp = tid & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lq[i] = qp == 0 ? p.lv.q[i] : qp == 1 ? p.lv.q[4 + i] : qp == 2 ? p.lv.q[8 + i] : p.lv.q[12 + i];
  }

  f32x4 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: stage 0 complete, codes of the next step in flight
  load_x(kbeg, 0, 0, XJ);
  WPart<QW> w0 = load_w(kbeg), w1;
  store_wpart<TW, QW>(w0, wpart_chat<ABS>(w0), p.lv, lq, sB, tid);
  w1 = load_w(kbeg + 1);
  __builtin_amdgcn_s_waitcnt(0);  // stage 0 LDS-DMA landed (vmcnt = lgkmcnt = 0)
  __syncthreads();

  const int arow = wm * WM + (l & 15);
  const int brow = wn * 64 + (l & 15);
  // logical chunk of a fragment: 4 kk + (l >> 4); all fragment rows of a
  // lane share swz(row) = swz(l & 15)
  const int ck0 = 8 * ((0 + (l >> 4)) ^ swz(l & 15));
  const int ck1 = 8 * ((4 + (l >> 4)) ^ swz(l & 15));

  // Step kt (stage st): the activation LDS-DMA of step kt + 1, the code loads
  // of step kt + 2 into `next`, the MFMAs of step kt, and the unpack of `cur`
  // (the codes of step kt + 1, loaded a step earlier) into the other stage.
  // With the small tile (few output tiles: a few hundred tokens, short steps)
  // the code loads stay in flight across the step's barrier: a scheduling
  // barrier keeps them after the DMA, so the end-of-step vmcnt(NCODE) waits
  // for the DMA only, and the loop is unrolled by two so that the two code
  // buffers alternate in fixed registers (a copy would wait for the loads).
  // The large tiles have no registers to spare for that (it spills) and wait
  // for everything at the end of each step.
  constexpr bool KEEP = WM == 32 && VEC;
  // 512-row tiles issue the next step's activation DMA in pieces between the
  // first half-step's MFMA groups (one instruction behind the MFMAs of each
  // fragment row): measured 3-5 % faster than one burst of 8 ahead of all
  // the MFMAs, which stalls the wave before its first MFMA while the vector
  // memory path is still busy. The pieces stay where they are written
  // because the compiler keeps them in order with the fragment reads of the
  // same LDS array; handing the stages over as unaliased pointers lets it
  // gather them into a burst again (measured 15 % slower).
  constexpr bool SPREAD = VEC && !KEEP && BM == 512;
  static_assert(!SPREAD || XJ == MI, "one DMA instruction per fragment row");
  constexpr int NCODE = ABS ? 2 : 3;  // code words + block constant(s)
  constexpr int kStepWait = KEEP ? (NCODE | (7 << 4)) : 0;  // vmcnt(NCODE), expcnt any, lgkmcnt(0)
  auto step = [&](int kt, int st, WPart<QW>& next, const WPart<QW>& cur) {
    prefetch_x(kt + PFD);
    if (!SPREAD) load_x(kt + 1, st ^ 1, 0, XJ);
    if (KEEP) __builtin_amdgcn_sched_barrier(0);
    next = load_w(kt + 2);
    if (KEEP) {
      // `cur` was loaded a step ago and may still be in flight (the previous
      // step's end waited for its DMA only). Its loads are older than this
      // step's XJ DMA instructions and NCODE code loads, so vmcnt(XJ + NCODE)
      // retires them. The compiler does not insert this wait itself: it
      // counts the mix of LDS-DMA and register loads as out of order, and at
      // the loop's first step it emitted no wait before reading `cur`.
      __builtin_amdgcn_s_waitcnt((XJ + NCODE) | (7 << 4) | (15 << 8));
      __builtin_amdgcn_sched_barrier(0);
    }

    const uint16_t* a_s = sA + st * BM * 64;
    const uint16_t* b_s = sB + st * BN * 64;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ck = kk ? ck1 : ck0;
      bf16x8 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = lds_load8(reinterpret_cast<const __bf16*>(b_s + (brow + 16 * j) * 64 + (TW ? ck ^ (16 * j) : ck)));
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const bf16x8 a = lds_load8(reinterpret_cast<const __bf16*>(a_s + (arow + 16 * i) * 64 + ck));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a, b[j], acc[i][j]);
        if (SPREAD && kk == 0) load_x(kt + 1, st ^ 1, i, i + 1);
      }
    }
    // unpack the next weight tile into the other stage (free since the last
    // barrier); steps past the end unpack a clamped block into an unused stage
    store_wpart<TW, QW>(cur, wpart_chat<ABS>(cur), p.lv, lq, sB + (st ^ 1) * BN * 64, tid);
    __builtin_amdgcn_s_waitcnt(kStepWait);  // this step's LDS-DMA and LDS writes are complete
    __builtin_amdgcn_s_barrier();
    // the prefetch register stays allocated until its load has completed
    // (reusing it earlier would make the compiler wait for that load)
    if (PF) asm volatile("" ::"v"(pf));
  };
  if (KEEP) {
    int kt = kbeg;
    for (; kt + 1 < kend; kt += 2) {
      step(kt, 0, w0, w1);
      step(kt + 1, 1, w1, w0);
    }
    if (kt < kend) step(kt, 0, w0, w1);
  } else {
    for (int kt = kbeg; kt < kend; ++kt) {
      step(kt, (kt - kbeg) & 1, w0, w1);
      w1 = w0;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

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
        const int c = (l & 7) ^ bswz<TW>(R);
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
        for (int j = 0; j < 4; ++j) b[j] = lds_load8(reinterpret_cast<const __bf16*>(sB + (brow + 16 * j) * 64 + (TW ? ck ^ (16 * j) : ck)));
#pragma unroll
        for (int i = 0; i < MI; ++i) {
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
  if (!part && (p.Nout & 1) == 0) {
    // bf16 pairs of adjacent columns, one 4-byte store each: lanes l and l ^ 1
    // (columns c, c ^ 1) swap halves of their 4 rows, so the even lane holds
    // rows 0-1 and the odd lane rows 2-3 of both columns (same rounding)
    const bool odd = l & 1;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 a = acc[i][j];
        const float s0 = odd ? a[0] : a[2], s1 = odd ? a[1] : a[3];
        const float r0 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s0), 0xB1, 0xF, 0xF, false));
        const float r1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s1), 0xB1, 0xF, 0xF, false));
        const int col = n0 + wn * 64 + 16 * j + (l & 14);
        const int row = m0 + wm * WM + 16 * i + 4 * (l >> 4) + (odd ? 2 : 0);
        const uint32_t w0 = odd ? pack_bf16(r0, a[2]) : pack_bf16(a[0], r0);
        const uint32_t w1 = odd ? pack_bf16(r1, a[3]) : pack_bf16(a[1], r1);
        if (col < p.Nout) {
          uint16_t* o = p.out + (int64_t)row * p.Nout + col;
          if (row < p.M) *reinterpret_cast<uint32_t*>(o) = w0;
          if (row + 1 < p.M) *reinterpret_cast<uint32_t*>(o + p.Nout) = w1;
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + 16 * j + (l & 15);
      if (col >= p.Nout) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm * WM + 16 * i + 4 * (l >> 4) + v;
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
  // reductions in whole 64-element steps take the DMA / uniform-address path
  const bool vec = p.Kred % BK == 0;
  switch (gemm_tile(p.M, p.Nout)) {
    case kTile512x128:
      return vec ? launch_variant<512, 128, TW, LORA, true, ABS>(p, s)
                 : launch_variant<512, 128, TW, LORA, false, ABS>(p, s);
    case kTile256x256:
      return vec ? launch_variant<256, 256, TW, LORA, true, ABS>(p, s)
                 : launch_variant<256, 256, TW, LORA, false, ABS>(p, s);
    default:
      return vec ? launch_variant<128, 128, TW, LORA, true, ABS>(p, s)
                 : launch_variant<128, 128, TW, LORA, false, ABS>(p, s);
  }
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
