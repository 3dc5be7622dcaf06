// C ABI of the library: argument validation (before any HIP call),
// workspace layout and the launch sequence of each entry point.
// The operations themselves are defined in include/qlora.h.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>

#include "qlora.h"
#include "launch.hpp"


using namespace qlora;

namespace {

constexpr int kGemvMaxM = 16;

// Scratch of qlora_linear_fwd_noalloc, for callers that cannot allocate: one
// copy per GPU for the life of the process. In host code `scratch` only names
// the symbol; its device address (per device) comes from hipGetSymbolAddress
// and is what kernels get. No forward kernel reads a scratch byte it has not
// written in the same call, so nothing needs clearing; calls that overlap on
// one GPU share it and race.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch on the device of `stream` (which must be the
// current device), looked up once per device.
int scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QLORA_ERR_DEVICE;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return QLORA_ERR_DEVICE;
    if (sdev != dev) return QLORA_ERR_DEVICE;
  }
  if (dev < 0 || dev >= kMaxDevices) return QLORA_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return QLORA_ERR_DEVICE;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
inline int clampi(int64_t v, int64_t lo, int64_t hi) { return (int)(v < lo ? lo : (v > hi ? hi : v)); }
// Every [rows, cols] operand of the linear layer is indexed in 32 bits:
// max(64 ceil(M / 64), rp) rows times max(N, K, rp) elements, with
// rp = 64 ceil(r / 64), must stay below 2^31 (so byte offsets stay below
// 2^32). The rank side counts as rows too: B^T [r, N], A^T [K, rp] and the
// gradient partials [rp, N] / [rp, K] are indexed like the token-side planes.
inline bool index_fits(int64_t M, int64_t N, int64_t K, int64_t r) {
  const int64_t Mp = cdiv(M, 64) * 64, rp = cdiv(r, 64) * 64;
  return std::max(Mp, rp) * std::max(std::max(N, K), rp) < (int64_t(1) << 31);
}

// Reduction splits. Each aims at a few hundred workgroups on 256 CUs.
inline int proj_splits(int64_t M, int64_t Kr) {
  // ~512 workgroups of 64 rows; every slice keeps at least 4 steps of 64
  const int64_t max_split = std::max<int64_t>(1, Kr / 256);
  return clampi(cdiv(512, cdiv(M, 64)), 1, std::min<int64_t>(64, max_split));
}
inline int grad_splits(int64_t M, int64_t C, int64_t rp) {
  // The gradient kernel holds one workgroup per CU (128 KB of LDS), so a
  // launch of w s workgroups takes ceil(w s / 256) rounds of 1/s of the rows
  // each: pick s (<= 8, each slice at least 8 steps of 64 rows) minimising
  // ceil(w s / 256) / s; ties go to fewer splits (less partial traffic).
  const int64_t w = cdiv(C, 128) * cdiv(rp, 64);
  const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(8, cdiv(M, 512)));
  int64_t best = 1;
  for (int64_t sp = 2; sp <= smax; ++sp)
    if (cdiv(w * sp, 256) * best < cdiv(w * best, 256) * sp) best = sp;
  return (int)best;
}

struct Layout {
  // byte offsets into the workspace; kNone when unused
  size_t partT = 0, T32 = 0, Ts = 0, Bpad = 0;                       // forward
  size_t Bt = 0, At = 0, partU = 0, U32 = 0, PtH = 0, PtL = 0, TtH = 0, TtL = 0;  // backward
  size_t gpartA = 0, gpartB = 0;
  size_t partY = 0, partX = 0;  // split-reduction partials of the Y / dX GEMMs
  size_t fwd_total = 0, bwd_total = 0;
  int tsplit = 1, usplit = 1, sA = 1, sB = 1;
  int ksY = 1, kcY = 0, ksX = 1, kcX = 0;
};

// r is the total rank (g r_seg for g grouped segments); the dB gradient of
// grouped linears runs one segment's r_seg columns per workgroup.
Layout plan(int64_t M, int64_t N, int64_t K, int64_t r, int64_t groups = 1) {
  Layout L;
  const int64_t rp = cdiv(r, 64) * 64;
  // forward (few tokens: T32 holds T [M, r] as the few-token kernel writes it)
  L.tsplit = M <= kGemvMaxM ? 1 : proj_splits(M, K);
  size_t o = 0;
  L.partT = o; o = al256(o + (M <= kGemvMaxM ? 0 : (size_t)L.tsplit * M * rp * 4));
  L.T32 = o;   o = al256(o + (size_t)M * r * 4);
  L.Ts = o;    o = al256(o + (size_t)M * rp * 2);
  L.Bpad = o;  o = al256(o + (rp != r ? (size_t)N * rp * 2 : 0));
  if (M > kGemvMaxM) L.ksY = gemm_ksplit(M, N, K, &L.kcY);
  L.partY = o; o = al256(o + (L.ksY > 1 ? (size_t)L.ksY * M * N * 4 : 0));
  L.fwd_total = o;
  // backward (T recompute reuses the forward region [partT, Ts))
  L.usplit = proj_splits(M, N);
  o = L.Bpad;  // T partials, T32 and Ts precede
  L.Bt = o;    o = al256(o + (size_t)r * N * 2);
  L.At = o;    o = al256(o + (size_t)K * rp * 2);
  L.partU = o; o = al256(o + (size_t)L.usplit * M * rp * 4);
  L.U32 = o;   o = al256(o + (size_t)M * r * 4);
  const int64_t rpB = groups > 1 ? r / groups : rp;  // grouped: r_seg, a multiple of 64
  L.sA = grad_splits(M, K, rp);
  L.sB = grad_splits(M, N, rpB);
  const int64_t Mp = cdiv(M, 64) * 64;
  L.PtH = o;   o = al256(o + (size_t)rp * Mp * 2);
  L.PtL = o;   o = al256(o + (size_t)rp * Mp * 2);
  L.TtH = o;   o = al256(o + (size_t)rp * Mp * 2);
  L.TtL = o;   o = al256(o + (size_t)rp * Mp * 2);
  L.gpartA = o; o = al256(o + (size_t)L.sA * rp * K * 4);
  L.gpartB = o; o = al256(o + (size_t)L.sB * rp * N * 4);
  L.ksX = gemm_ksplit(M, K, N, &L.kcX);
  L.partX = o; o = al256(o + (L.ksX > 1 ? (size_t)L.ksX * M * K * 4 : 0));
  L.bwd_total = o;
  return L;
}

// A stored weight in any supported format: double-quantised constants
// (c2, c1) or fp32 block absmax, and a level table.
struct WView {
  const uint8_t* codes = nullptr;
  const uint8_t* c2 = nullptr;
  const float* c1 = nullptr;
  const float* absmax = nullptr;
  int64_t N = 0, K = 0;
  int cb = kNF4;
};

int view_nf4(const qlora_nf4_weight* W, WView& v) {
  if (!W) return QLORA_ERR_NULL;
  if (!W->codes || !W->c2_fp8 || !W->c1) return QLORA_ERR_NULL;
  if (!aligned(W->codes, 16) || !aligned(W->c2_fp8, 16) || !aligned(W->c1, 4)) return QLORA_ERR_ALIGN;
  v.codes = W->codes;
  v.c2 = W->c2_fp8;
  v.c1 = W->c1;
  v.absmax = nullptr;
  v.N = W->rows;
  v.K = W->cols;
  v.cb = kNF4;
  return QLORA_OK;
}

int check_format(int codebook, int double_quant) {
  if (codebook < 0 || codebook >= kNumCodebooks) return QLORA_ERR_UNSUPPORTED;
  if (double_quant != 0 && double_quant != 1) return QLORA_ERR_UNSUPPORTED;
  return QLORA_OK;
}

int view_4bit(const qlora_4bit_weight* W, WView& v) {
  if (!W) return QLORA_ERR_NULL;
  const int f = check_format(W->codebook, W->double_quant);
  if (f != QLORA_OK) return f;
  if (!W->codes || !W->consts || (W->double_quant && !W->c1)) return QLORA_ERR_NULL;
  if (!aligned(W->codes, 16) || !aligned(W->consts, 16) || (W->double_quant && !aligned(W->c1, 4)))
    return QLORA_ERR_ALIGN;
  v.codes = W->codes;
  v.c2 = W->double_quant ? static_cast<const uint8_t*>(W->consts) : nullptr;
  v.c1 = W->double_quant ? W->c1 : nullptr;
  v.absmax = W->double_quant ? nullptr : static_cast<const float*>(W->consts);
  v.N = W->rows;
  v.K = W->cols;
  v.cb = W->codebook;
  return QLORA_OK;
}

// The linear layer's operand checks (no workspace).
int check_linear_args(const WView& W, const void* X, const void* A, const void* B, int64_t M, int64_t r,
                      float scale) {
  if (!X || !A || !B) return QLORA_ERR_NULL;
  const int64_t N = W.N, K = W.K;
  if (M < 1 || N < 1 || K < 64 || (K % 64) != 0) return QLORA_ERR_SHAPE;
  if (r < 1 || r > 256) return QLORA_ERR_SHAPE;
  if (!index_fits(M, N, K, r) || N * K >= (int64_t(1) << 40)) return QLORA_ERR_SHAPE;
  if (!std::isfinite(scale)) return QLORA_ERR_UNSUPPORTED;
  if (!aligned(X, 16) || !aligned(A, 16) || !aligned(B, 16)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

int check_linear(const WView& W, const void* X, const void* A, const void* B,
                 int64_t M, int64_t r, float scale, const void* ws, size_t ws_bytes) {
  const int st = check_linear_args(W, X, A, B, M, r, scale);
  if (st != QLORA_OK) return st;
  if (!ws) return QLORA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return QLORA_ERR_ALIGN;
  (void)ws_bytes;
  return QLORA_OK;
}

// Device-usable address of an array: device memory as is, pinned host
// memory through its device mapping. Returns false for pageable or managed
// memory (and clears the error an unknown pointer leaves behind).
bool device_address(const void* p, void** out) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (at.type == hipMemoryTypeDevice) {
    *out = const_cast<void*>(p);
    return true;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer) {
    const char* base = static_cast<const char*>(at.hostPointer ? at.hostPointer : p);
    *out = static_cast<char*>(at.devicePointer) + (static_cast<const char*>(p) - base);
    return true;
  }
  return false;
}

#define QLORA_TRY(expr)                                \
  do {                                                 \
    if ((expr) != hipSuccess) return QLORA_ERR_DEVICE; \
  } while (0)

// T (float32 [M, r]) recomputed for the backward: few tokens run the few-token
// kernel's T producers alone (so a saved and a recomputed T are bit-identical),
// more tokens the streamed projection and its reduction. A [r, K] (the stacked
// A of grouped linears: r = g r_seg).
hipError_t recompute_T(const WView& W, const Layout& L, char* base, const uint16_t* X, const uint16_t* A,
                       int64_t M, int64_t K, int64_t r, hipStream_t s, float** T) {
  float* T32 = reinterpret_cast<float*>(base + L.T32);
  *T = T32;
  if (M <= kGemvMaxM)
    return launch_fewtok(X, W.codes, W.c2, W.c1, W.absmax, W.cb, (int)W.N, (int)K, (int)M, A, (int)r, nullptr,
                         (int)r, 0, 0.0f, nullptr, T32, s);
  const int rp = (int)(cdiv(r, 64) * 64);
  float* partT = reinterpret_cast<float*>(base + L.partT);
  uint16_t* Ts = reinterpret_cast<uint16_t*>(base + L.Ts);
  hipError_t e = launch_proj(X, A, (int)M, (int)K, (int)r, rp, L.tsplit, partT, s);
  if (e != hipSuccess) return e;
  return launch_finalize(partT, L.tsplit, (int)M, (int)M, (int)r, rp, 1.0f, T32, Ts, nullptr, s);
}

// out = act op(W~) (+ L R^T when L is given: L [M, rp], R [Nout, rp]).
int matmul_impl(const WView& W, const void* act, int64_t M, int transposed, void* out, void* stream,
                const void* lora_l = nullptr, const void* lora_r = nullptr, int64_t rp = 0) {
  if (!act || !out) return QLORA_ERR_NULL;
  const int64_t N = W.N, K = W.K;
  if (M < 1 || N < 1 || K < 64 || (K % 64) != 0) return QLORA_ERR_SHAPE;
  if (transposed != 0 && transposed != 1) return QLORA_ERR_UNSUPPORTED;
  if (M * std::max(N, K) >= (int64_t(1) << 31) || N * K >= (int64_t(1) << 40)) return QLORA_ERR_SHAPE;
  if (lora_l) {
    const int64_t nout = transposed ? K : N;
    if (rp < 64 || rp > 4096 || rp % 64 != 0 || std::max(M, nout) * rp >= (int64_t(1) << 31))
      return QLORA_ERR_SHAPE;
    if (!aligned(lora_l, 16) || !aligned(lora_r, 16)) return QLORA_ERR_ALIGN;
  }
  if (!aligned(act, 16) || !aligned(out, 16)) return QLORA_ERR_ALIGN;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    GemmParams p;
    p.act = static_cast<const uint16_t*>(act);
    p.codes = W.codes;
    p.c2 = W.c2;
    p.c1 = W.c1;
    p.absmax = W.absmax;
    p.wN = N;
    p.wK = K;
    p.lora_l = static_cast<const uint16_t*>(lora_l);
    p.lora_r = static_cast<const uint16_t*>(lora_r);
    p.rp = lora_l ? (int)rp : 0;
    p.lora_ld = lora_l ? (int)rp : 0;
    p.lora_seg = 0;
    p.out = static_cast<uint16_t*>(out);
    p.M = (int)M;
    p.Nout = (int)(transposed ? K : N);
    p.Kred = (int)(transposed ? N : K);
    p.lv = host_levels(W.cb);
    QLORA_TRY(launch_gemm(p, transposed == 1, (hipStream_t)stream));
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

int fwd_impl(const WView& W, const void* X, const void* A, const void* B, int64_t M, int64_t r, float scale,
             void* Y, float* T_save, void* ws, size_t ws_bytes, void* stream) {
  int st = check_linear(W, X, A, B, M, r, scale, ws, ws_bytes);
  if (st != QLORA_OK) return st;
  if (!Y) return QLORA_ERR_NULL;
  if (!aligned(Y, 16) || (T_save && !aligned(T_save, 4))) return QLORA_ERR_ALIGN;
  const int64_t N = W.N, K = W.K;
  const Layout L = plan(M, N, K, r);
  if (ws_bytes < L.fwd_total) return QLORA_ERR_WORKSPACE;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char* base = static_cast<char*>(ws);
    const int rp = (int)(cdiv(r, 64) * 64);
    float* partT = reinterpret_cast<float*>(base + L.partT);
    float* T32 = T_save ? T_save : reinterpret_cast<float*>(base + L.T32);
    uint16_t* Ts = reinterpret_cast<uint16_t*>(base + L.Ts);
    const uint16_t* Xh = static_cast<const uint16_t*>(X);
    const uint16_t* Ah = static_cast<const uint16_t*>(A);
    const uint16_t* Bh = static_cast<const uint16_t*>(B);

    if (M <= kGemvMaxM) {
      // few tokens: T (into T_save, else the workspace), then one launch
      // streams the weight and adds the LoRA term
      QLORA_TRY(launch_fewtok(Xh, W.codes, W.c2, W.c1, W.absmax, W.cb, (int)N, (int)K, (int)M, Ah, (int)r, Bh,
                              (int)r, 0, scale, static_cast<uint16_t*>(Y), T32, s));
      return QLORA_OK;
    }
    // T = X A^T: split-K partials [tsplit][M][rp]
    QLORA_TRY(launch_proj(Xh, Ah, (int)M, (int)K, (int)r, rp, L.tsplit, partT, s));
    // Ts = bf16(scale * T) [M, rp], T float32 [M, r]
    QLORA_TRY(launch_finalize(partT, L.tsplit, (int)M, (int)M, (int)r, rp, scale, T32, Ts, nullptr, s));
    const uint16_t* Br = Bh;
    if (rp != r) {
      uint16_t* Bpad = reinterpret_cast<uint16_t*>(base + L.Bpad);
      QLORA_TRY(launch_relayout(Bh, N, r, r, false, Bpad, N, rp, rp, s));
      Br = Bpad;
    }
    GemmParams p;
    p.act = Xh;
    p.codes = W.codes;
    p.c2 = W.c2;
    p.c1 = W.c1;
    p.absmax = W.absmax;
    p.wN = N;
    p.wK = K;
    p.lora_l = Ts;
    p.lora_r = Br;
    p.rp = rp;
    p.lora_ld = rp;
    p.lora_seg = 0;
    p.out = static_cast<uint16_t*>(Y);
    p.M = (int)M;
    p.Nout = (int)N;
    p.Kred = (int)K;
    p.lv = host_levels(W.cb);
    p.ksplit = L.ksY;
    p.kchunk = L.kcY;
    p.part = reinterpret_cast<float*>(base + L.partY);
    QLORA_TRY(launch_gemm(p, false, s));
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

int bwd_impl(const WView& W, const void* X, const void* A, const void* B, const void* dY, const float* T_saved,
             int64_t M, int64_t r, float scale, void* dX, void* dA, void* dB, void* ws, size_t ws_bytes,
             void* stream) {
  int st = check_linear(W, X, A, B, M, r, scale, ws, ws_bytes);
  if (st != QLORA_OK) return st;
  if (!dY || !dA || !dB) return QLORA_ERR_NULL;
  if (!aligned(dY, 16) || !aligned(dA, 16) || !aligned(dB, 16) || (dX && !aligned(dX, 16)) ||
      (T_saved && !aligned(T_saved, 4)))
    return QLORA_ERR_ALIGN;
  const int64_t N = W.N, K = W.K;
  const Layout L = plan(M, N, K, r);
  if (ws_bytes < L.bwd_total) return QLORA_ERR_WORKSPACE;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char* base = static_cast<char*>(ws);
    const int rp = (int)(cdiv(r, 64) * 64);
    const uint16_t* Xh = static_cast<const uint16_t*>(X);
    const uint16_t* Ah = static_cast<const uint16_t*>(A);
    const uint16_t* Bh = static_cast<const uint16_t*>(B);
    const uint16_t* dYh = static_cast<const uint16_t*>(dY);
    uint16_t* Bt = reinterpret_cast<uint16_t*>(base + L.Bt);
    uint16_t* At = reinterpret_cast<uint16_t*>(base + L.At);
    float* partU = reinterpret_cast<float*>(base + L.partU);
    float* U32 = reinterpret_cast<float*>(base + L.U32);
    // hi / lo bf16 planes [Mp, rp] of s U and of s T (rows past M zero);
    // the hi plane of s U is also the row operand of the dX epilogue
    const int Mp = (int)(cdiv(M, 64) * 64);
    uint16_t* PtH = reinterpret_cast<uint16_t*>(base + L.PtH);
    uint16_t* PtL = reinterpret_cast<uint16_t*>(base + L.PtL);
    uint16_t* TtH = reinterpret_cast<uint16_t*>(base + L.TtH);
    uint16_t* TtL = reinterpret_cast<uint16_t*>(base + L.TtL);
    float* gpartA = reinterpret_cast<float*>(base + L.gpartA);
    float* gpartB = reinterpret_cast<float*>(base + L.gpartB);
    const bool streamed_dB = N % 8 == 0;  // dB through the transpose-read kernel

    // T (float32 [M, r]): saved by the forward, or recomputed
    const float* T = T_saved;
    if (!T) {
      float* T32 = nullptr;
      QLORA_TRY(recompute_T(W, L, base, Xh, Ah, M, K, r, s, &T32));
      T = T32;
    }
    // U = dY B: B^T [r, N] is the row operand of the projection; A^T [K, rp]
    // is the column operand of the dX epilogue (one launch for both)
    QLORA_TRY(launch_transpose2(Bh, Ah, (int)N, (int)K, (int)r, (int)r, rp, Bt, dX ? At : nullptr, s));
    QLORA_TRY(launch_proj(dYh, Bt, (int)M, (int)N, (int)r, rp, L.usplit, partU, s));
    if (streamed_dB)
      QLORA_TRY(launch_finalize2(partU, L.usplit, (int)M, Mp, (int)r, rp, scale, U32, PtH, PtL, T, TtH, TtL, s));
    else
      QLORA_TRY(launch_finalize(partU, L.usplit, (int)M, Mp, (int)r, rp, scale, U32, PtH, PtL, s));

    if (dX) {
      // dX = dY W~ + (s U) A
      GemmParams p;
      p.act = dYh;
      p.codes = W.codes;
      p.c2 = W.c2;
      p.c1 = W.c1;
      p.absmax = W.absmax;
      p.wN = N;
      p.wK = K;
      p.lora_l = PtH;
      p.lora_r = At;
      p.rp = rp;
      p.lora_ld = rp;
      p.lora_seg = 0;
      p.out = static_cast<uint16_t*>(dX);
      p.M = (int)M;
      p.Nout = (int)K;
      p.Kred = (int)N;
      p.lv = host_levels(W.cb);
      p.ksplit = L.ksX;
      p.kchunk = L.kcX;
      p.part = reinterpret_cast<float*>(base + L.partX);
      QLORA_TRY(launch_gemm(p, true, s));
    }
    // dA = (s U)^T X  [r, K] (K % 64 == 0); dB = s dY^T T  [N, r], computed as
    // ((s T)^T dY)^T. The rank-r factor enters as its hi + lo bf16 planes.
    QLORA_TRY(launch_grad_tr(PtH, PtL, Xh, (int)M, Mp, (int)K, rp, L.sA, false, gpartA, s));
    if (streamed_dB) {
      QLORA_TRY(launch_grad_tr(TtH, TtL, dYh, (int)M, Mp, (int)N, rp, L.sB, true, gpartB, s));
      QLORA_TRY(launch_grad_reduce2(gpartA, L.sA, (int)K, static_cast<uint16_t*>(dA), gpartB, L.sB, (int)N,
                                    static_cast<uint16_t*>(dB), (int)r, rp, (int)r, rp, 1.0f, s));
    } else {
      QLORA_TRY(launch_grad_reduce(gpartA, L.sA, (int)r, rp, (int)K, 1.0f, false, false, static_cast<uint16_t*>(dA), s));
      QLORA_TRY(launch_grad(T, dYh, (int)M, (int)N, (int)r, rp, L.sB, gpartB, s));
      QLORA_TRY(launch_grad_reduce(gpartB, L.sB, (int)r, rp, (int)N, scale, true, false, static_cast<uint16_t*>(dB), s));
    }
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}


// ---- grouped linears: g segments of output columns sharing one input ---------------------
// W is [g Ns, K] (the segments' weights stacked), A [g r, K], B [g Ns, r];
// segment i computes Y_i = X W_i~^T + s (X A_i^T) B_i^T, and the backward
// sums dX over the segments. Needs Ns % 256 == 0 (no GEMM tile straddles two
// segments) and r % 64 == 0 (each segment's rank is whole 64-column blocks).
int check_grouped(const WView& W, int64_t g, int64_t r) {
  if (g < 1 || g > 16) return QLORA_ERR_SHAPE;
  if (g == 1) return QLORA_OK;
  if (W.N % g != 0 || (W.N / g) % 256 != 0 || r % 64 != 0) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

int fwd_grouped_impl(const WView& W, int64_t g, const void* X, const void* A, const void* B, int64_t M, int64_t r,
                     float scale, void* Y, float* T_save, void* ws, size_t ws_bytes, void* stream) {
  int st = check_grouped(W, g, r);
  if (st != QLORA_OK) return st;
  if (g == 1) return fwd_impl(W, X, A, B, M, r, scale, Y, T_save, ws, ws_bytes, stream);
  const int64_t R = g * r;
  st = check_linear(W, X, A, B, M, r, scale, ws, ws_bytes);
  if (st != QLORA_OK) return st;
  if (!Y) return QLORA_ERR_NULL;
  if (!aligned(Y, 16) || (T_save && !aligned(T_save, 4))) return QLORA_ERR_ALIGN;
  const int64_t N = W.N, K = W.K, Ns = N / g;
  const Layout L = plan(M, N, K, R, g);
  if (ws_bytes < L.fwd_total) return QLORA_ERR_WORKSPACE;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char* base = static_cast<char*>(ws);
    float* partT = reinterpret_cast<float*>(base + L.partT);
    float* T32 = T_save ? T_save : reinterpret_cast<float*>(base + L.T32);
    uint16_t* Ts = reinterpret_cast<uint16_t*>(base + L.Ts);
    const uint16_t* Xh = static_cast<const uint16_t*>(X);
    const uint16_t* Ah = static_cast<const uint16_t*>(A);
    const uint16_t* Bh = static_cast<const uint16_t*>(B);
    if (M <= kGemvMaxM) {
      QLORA_TRY(launch_fewtok(Xh, W.codes, W.c2, W.c1, W.absmax, W.cb, (int)N, (int)K, (int)M, Ah, (int)R, Bh,
                              (int)r, (int)Ns, scale, static_cast<uint16_t*>(Y), T32, s));
      return QLORA_OK;
    }
    // T = X [A_1; ..; A_g]^T: one pass over X for all segments
    QLORA_TRY(launch_proj(Xh, Ah, (int)M, (int)K, (int)R, (int)R, L.tsplit, partT, s));
    QLORA_TRY(launch_finalize(partT, L.tsplit, (int)M, (int)M, (int)R, (int)R, scale, T32, Ts, nullptr, s));
    GemmParams p;
    p.act = Xh;
    p.codes = W.codes;
    p.c2 = W.c2;
    p.c1 = W.c1;
    p.absmax = W.absmax;
    p.wN = N;
    p.wK = K;
    p.lora_l = Ts;
    p.lora_r = Bh;
    p.rp = (int)r;
    p.lora_ld = (int)R;
    p.lora_seg = (int)Ns;
    p.out = static_cast<uint16_t*>(Y);
    p.M = (int)M;
    p.Nout = (int)N;
    p.Kred = (int)K;
    p.lv = host_levels(W.cb);
    p.ksplit = L.ksY;
    p.kchunk = L.kcY;
    p.part = reinterpret_cast<float*>(base + L.partY);
    QLORA_TRY(launch_gemm(p, false, s));
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

int bwd_grouped_impl(const WView& W, int64_t g, const void* X, const void* A, const void* B, const void* dY,
                     const float* T_saved, int64_t M, int64_t r, float scale, void* dX, void* dA, void* dB,
                     void* ws, size_t ws_bytes, void* stream) {
  int st = check_grouped(W, g, r);
  if (st != QLORA_OK) return st;
  if (g == 1) return bwd_impl(W, X, A, B, dY, T_saved, M, r, scale, dX, dA, dB, ws, ws_bytes, stream);
  const int64_t R = g * r;
  st = check_linear(W, X, A, B, M, r, scale, ws, ws_bytes);
  if (st != QLORA_OK) return st;
  if (!dY || !dA || !dB) return QLORA_ERR_NULL;
  if (!aligned(dY, 16) || !aligned(dA, 16) || !aligned(dB, 16) || (dX && !aligned(dX, 16)) ||
      (T_saved && !aligned(T_saved, 4)))
    return QLORA_ERR_ALIGN;
  const int64_t N = W.N, K = W.K, Ns = N / g;
  const Layout L = plan(M, N, K, R, g);
  if (ws_bytes < L.bwd_total) return QLORA_ERR_WORKSPACE;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char* base = static_cast<char*>(ws);
    const uint16_t* Xh = static_cast<const uint16_t*>(X);
    const uint16_t* Ah = static_cast<const uint16_t*>(A);
    const uint16_t* Bh = static_cast<const uint16_t*>(B);
    const uint16_t* dYh = static_cast<const uint16_t*>(dY);
    uint16_t* Bt = reinterpret_cast<uint16_t*>(base + L.Bt);
    uint16_t* At = reinterpret_cast<uint16_t*>(base + L.At);
    float* partU = reinterpret_cast<float*>(base + L.partU);
    float* U32 = reinterpret_cast<float*>(base + L.U32);
    const int Mp = (int)(cdiv(M, 64) * 64);
    uint16_t* PtH = reinterpret_cast<uint16_t*>(base + L.PtH);
    uint16_t* PtL = reinterpret_cast<uint16_t*>(base + L.PtL);
    uint16_t* TtH = reinterpret_cast<uint16_t*>(base + L.TtH);
    uint16_t* TtL = reinterpret_cast<uint16_t*>(base + L.TtL);
    float* gpartA = reinterpret_cast<float*>(base + L.gpartA);
    float* gpartB = reinterpret_cast<float*>(base + L.gpartB);
    const float* T = T_saved;
    if (!T) {
      float* T32 = nullptr;
      QLORA_TRY(recompute_T(W, L, base, Xh, Ah, M, K, R, s, &T32));
      T = T32;
    }
    // B^T [r, N] (segment i in columns i Ns ..) and [A_1; ..; A_g]^T [K, R]
    QLORA_TRY(launch_transpose2(Bh, Ah, (int)N, (int)K, (int)r, (int)R, (int)R, Bt, dX ? At : nullptr, s));
    // U_i = dY_i B_i: segment i reads dY and B^T at column offset i Ns
    const int usplit = proj_splits(M, Ns);
    QLORA_TRY(launch_proj_seg(dYh, N, Ns, Bt, N, Ns, (int)(r / 64), (int)M, (int)Ns, (int)r, (int)R, usplit, partU,
                              s));
    QLORA_TRY(launch_finalize2(partU, usplit, (int)M, Mp, (int)R, (int)R, scale, U32, PtH, PtL, T, TtH, TtL, s));
    if (dX) {
      // dX = sum_i (dY_i W_i~ + (s U_i) A_i) = dY W~ + (s U) [A_1; ..; A_g]
      GemmParams p;
      p.act = dYh;
      p.codes = W.codes;
      p.c2 = W.c2;
      p.c1 = W.c1;
      p.absmax = W.absmax;
      p.wN = N;
      p.wK = K;
      p.lora_l = PtH;
      p.lora_r = At;
      p.rp = (int)R;
      p.lora_ld = (int)R;
      p.lora_seg = 0;
      p.out = static_cast<uint16_t*>(dX);
      p.M = (int)M;
      p.Nout = (int)K;
      p.Kred = (int)N;
      p.lv = host_levels(W.cb);
      p.ksplit = L.ksX;
      p.kchunk = L.kcX;
      p.part = reinterpret_cast<float*>(base + L.partX);
      QLORA_TRY(launch_gemm(p, true, s));
    }
    // dA_i = (s U_i)^T X for all segments in one pass over X; dB_i from dY_i
    // and segment i's columns of s T only
    QLORA_TRY(launch_grad_tr(PtH, PtL, Xh, (int)M, Mp, (int)K, (int)R, L.sA, false, gpartA, s));
    QLORA_TRY(launch_grad_tr(TtH, TtL, dYh, (int)M, Mp, (int)N, (int)R, L.sB, true, gpartB, s, (int)Ns, (int)r));
    QLORA_TRY(launch_grad_reduce2(gpartA, L.sA, (int)K, static_cast<uint16_t*>(dA), gpartB, L.sB, (int)N,
                                  static_cast<uint16_t*>(dB), (int)R, (int)R, (int)r, (int)r, 1.0f, s));
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

}  // namespace

extern "C" {

int qlora_levels(int codebook, float out[16]) {
  if (!out) return QLORA_ERR_NULL;
  if (codebook < 0 || codebook >= kNumCodebooks) return QLORA_ERR_UNSUPPORTED;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    const Levels& lv = host_levels(codebook);
    for (int i = 0; i < 16; ++i) out[i] = lv.q[i];
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

int qlora_nf4_levels(float out[16]) { return qlora_levels(kNF4, out); }

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "null pointer argument";
    case QLORA_ERR_SHAPE: return "size out of range or inconsistent";
    case QLORA_ERR_ALIGN: return "pointer not aligned (16 bytes; 4 for c1/T; 256 for workspace)";
    case QLORA_ERR_UNSUPPORTED: return "unsupported mode or value";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_DEVICE: return "HIP call failed";
    case QLORA_ERR_SCRATCH: return "sizes need more than the library's fixed scratch (qlora_linear_fwd_noalloc)";
    default: return "unknown status";
  }
}

int qlora_quantize_4bit(const void* w_bf16, int64_t n, int codebook, int double_quant, uint8_t* codes,
                        void* consts, float* c1, void* stream) {
  const int f = check_format(codebook, double_quant);
  if (f != QLORA_OK) return f;
  if (!w_bf16 || !codes || !consts || (double_quant && !c1)) return QLORA_ERR_NULL;
  // one workgroup per 16384-weight group, fewer than 2^31 of them
  if (n < 1 || cdiv(n, kGroup) >= (int64_t(1) << 31)) return QLORA_ERR_SHAPE;
  if (!aligned(w_bf16, 16) || !aligned(codes, 16) || !aligned(consts, 16) || (double_quant && !aligned(c1, 4)))
    return QLORA_ERR_ALIGN;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    uint8_t* c2 = double_quant ? static_cast<uint8_t*>(consts) : nullptr;
    float* absmax = double_quant ? nullptr : static_cast<float*>(consts);
    QLORA_TRY(launch_quantize(w_bf16, n, codebook, codes, c2, double_quant ? c1 : nullptr, absmax,
                              (hipStream_t)stream));
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

int qlora_quantize_4bit_batch(int count, const void* const* w_bf16, const int64_t* n, int codebook,
                              int double_quant, uint8_t* const* codes, void* const* consts, float* const* c1,
                              void* stream) {
  const int f = check_format(codebook, double_quant);
  if (f != QLORA_OK) return f;
  if (count < 1 || count > kQuantBatch) return QLORA_ERR_SHAPE;
  if (!w_bf16 || !n || !codes || !consts || (double_quant && !c1)) return QLORA_ERR_NULL;
  QuantBatch b{};
  b.count = count;
  b.gstart[0] = 0;
  for (int t = 0; t < count; ++t) {
    if (!w_bf16[t] || !codes[t] || !consts[t] || (double_quant && !c1[t])) return QLORA_ERR_NULL;
    if (n[t] < 1) return QLORA_ERR_SHAPE;
    if (!aligned(w_bf16[t], 16) || !aligned(codes[t], 16) || !aligned(consts[t], 16) ||
        (double_quant && !aligned(c1[t], 4)))
      return QLORA_ERR_ALIGN;
    b.gstart[t + 1] = b.gstart[t] + cdiv(n[t], kGroup);
    b.w[t] = static_cast<const uint16_t*>(w_bf16[t]);
    b.n[t] = n[t];
    b.codes[t] = codes[t];
    b.c2[t] = double_quant ? static_cast<uint8_t*>(consts[t]) : nullptr;
    b.c1[t] = double_quant ? c1[t] : nullptr;
    b.absmax[t] = double_quant ? nullptr : static_cast<float*>(consts[t]);
  }
  if (b.gstart[count] >= (int64_t(1) << 31)) return QLORA_ERR_SHAPE;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    QLORA_TRY(launch_quantize_batch(b, codebook, (hipStream_t)stream));
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

int qlora_quantize_nf4_dq(const void* w_bf16, int64_t n, uint8_t* codes, uint8_t* c2_fp8,
                          float* c1, void* stream) {
  if (!w_bf16 || !codes || !c2_fp8 || !c1) return QLORA_ERR_NULL;
  return qlora_quantize_4bit(w_bf16, n, kNF4, 1, codes, c2_fp8, c1, stream);
}

// one dequantisation workgroup per 8192 weights, at most 2^31 - 1 of them
constexpr int64_t kMaxDequant = (int64_t)1 << 43;

int qlora_dequant_4bit(const uint8_t* codes, const void* consts, const float* c1, int64_t n, int codebook,
                       int double_quant, int out_dtype, void* out, void* stream) {
  const int f = check_format(codebook, double_quant);
  if (f != QLORA_OK) return f;
  if (!codes || !consts || (double_quant && !c1) || !out) return QLORA_ERR_NULL;
  if (n < 1 || n > kMaxDequant) return QLORA_ERR_SHAPE;
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16) return QLORA_ERR_UNSUPPORTED;
  if (!aligned(codes, 16) || !aligned(consts, 16) || (double_quant && !aligned(c1, 4)) || !aligned(out, 16))
    return QLORA_ERR_ALIGN;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    const uint8_t* c2 = double_quant ? static_cast<const uint8_t*>(consts) : nullptr;
    const float* absmax = double_quant ? nullptr : static_cast<const float*>(consts);
    QLORA_TRY(launch_dequant(codes, c2, double_quant ? c1 : nullptr, absmax, n, codebook, out_dtype == QLORA_BF16,
                             out, (hipStream_t)stream));
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

int qlora_dequant(const uint8_t* codes, const uint8_t* c2_fp8, const float* c1, int64_t n,
                  int out_dtype, void* out, void* stream) {
  if (!codes || !c2_fp8 || !c1 || !out) return QLORA_ERR_NULL;
  return qlora_dequant_4bit(codes, c2_fp8, c1, n, kNF4, 1, out_dtype, out, stream);
}

int qlora_nf4_matmul(const qlora_nf4_weight* W, const void* act, int64_t M, int transposed,
                     void* out, void* stream) {
  WView v;
  const int st = view_nf4(W, v);
  return st != QLORA_OK ? st : matmul_impl(v, act, M, transposed, out, stream);
}

int qlora_4bit_matmul(const qlora_4bit_weight* W, const void* act, int64_t M, int transposed,
                      void* out, void* stream) {
  WView v;
  const int st = view_4bit(W, v);
  return st != QLORA_OK ? st : matmul_impl(v, act, M, transposed, out, stream);
}

int qlora_4bit_matmul_lora(const qlora_4bit_weight* W, const void* act, int64_t M, int transposed,
                           const void* L, const void* R, int64_t rp, void* out, void* stream) {
  WView v;
  const int st = view_4bit(W, v);
  if (st != QLORA_OK) return st;
  if (!L || !R) return QLORA_ERR_NULL;
  return matmul_impl(v, act, M, transposed, out, stream, L, R, rp);
}

int qlora_adamw_step(float* param_f32, void* param_bf16, const void* grad_bf16, float* m, float* v,
                     int64_t n, const qlora_adamw_params* h, void* stream) {
  if (!param_f32 || !grad_bf16 || !m || !v || !h) return QLORA_ERR_NULL;
  if (n < 1 || n > ((int64_t)1 << 40)) return QLORA_ERR_SHAPE;  // one workgroup per 1024 parameters
  if (!aligned(param_f32, 16) || !aligned(grad_bf16, 16) || !aligned(m, 16) || !aligned(v, 16) ||
      (param_bf16 && !aligned(param_bf16, 16)))
    return QLORA_ERR_ALIGN;
  const bool ok = std::isfinite(h->lr) && h->lr >= 0.0f && h->beta1 >= 0.0f && h->beta1 < 1.0f &&
                  h->beta2 >= 0.0f && h->beta2 < 1.0f && std::isfinite(h->eps) && h->eps > 0.0f &&
                  std::isfinite(h->weight_decay) && h->weight_decay >= 0.0f && h->step >= 1;
  if (!ok) return QLORA_ERR_UNSUPPORTED;
  try {
    void *dp = nullptr, *dp16 = nullptr, *dg = nullptr, *dm = nullptr, *dv = nullptr;
    if (!device_address(param_f32, &dp) || !device_address(grad_bf16, &dg) || !device_address(m, &dm) ||
        !device_address(v, &dv) || (param_bf16 && !device_address(param_bf16, &dp16)))
      return QLORA_ERR_UNSUPPORTED;
    AdamW a;
    a.lr = h->lr;
    a.beta1 = h->beta1;
    a.beta2 = h->beta2;
    a.one_minus_beta1 = (float)(1.0 - (double)h->beta1);
    a.one_minus_beta2 = (float)(1.0 - (double)h->beta2);
    a.eps = h->eps;
    a.weight_decay = h->weight_decay;
    a.bc1 = (float)(1.0 / (1.0 - std::pow((double)h->beta1, (double)h->step)));
    a.bc2 = (float)(1.0 / (1.0 - std::pow((double)h->beta2, (double)h->step)));
    QLORA_TRY(launch_adamw(static_cast<float*>(dp), static_cast<uint16_t*>(dp16), static_cast<const uint16_t*>(dg),
                           static_cast<float*>(dm), static_cast<float*>(dv), n, a, (hipStream_t)stream));
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

int qlora_merge_lora(const qlora_4bit_weight* W, const void* A, const void* B, int64_t r, float scale, void* out,
                     void* stream) {
  WView v;
  const int st = view_4bit(W, v);
  if (st != QLORA_OK) return st;
  if (!A || !B || !out) return QLORA_ERR_NULL;
  if (v.N < 1 || v.K < 1 || r < 1 || r > 256 || v.N * v.K >= (int64_t(1) << 40) || v.N >= (int64_t(1) << 31) ||
      v.K >= (int64_t(1) << 31))
    return QLORA_ERR_SHAPE;
  if (!std::isfinite(scale)) return QLORA_ERR_UNSUPPORTED;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(out, 16)) return QLORA_ERR_ALIGN;
  try {
    if (tables_status() != 0) return QLORA_ERR_UNSUPPORTED;
    QLORA_TRY(launch_merge(v.codes, v.c2, v.c1, v.absmax, v.cb, static_cast<const uint16_t*>(A),
                           static_cast<const uint16_t*>(B), (int)v.N, (int)v.K, (int)r, scale,
                           static_cast<uint16_t*>(out), (hipStream_t)stream));
    return QLORA_OK;
  } catch (...) {
    return QLORA_ERR_DEVICE;
  }
}

size_t qlora_linear_grouped_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r, int64_t groups) {
  if (groups < 1 || groups > 16 || M < 1 || N < 1 || K < 64 || (K % 64) != 0 || r < 1 || r > 256) return 0;
  if (groups > 1 && (N % groups != 0 || (N / groups) % 256 != 0 || r % 64 != 0)) return 0;
  if (!index_fits(M, N, K, groups * r)) return 0;
  const Layout L = plan(M, N, K, groups * r, groups);
  return std::max(L.fwd_total, L.bwd_total);
}

int qlora_linear_fwd_grouped(const qlora_4bit_weight* W, int64_t groups, const void* X, const void* A,
                             const void* B, int64_t M, int64_t r, float scale, void* Y, float* T_save, void* ws,
                             size_t ws_bytes, void* stream) {
  WView v;
  const int st = view_4bit(W, v);
  return st != QLORA_OK ? st : fwd_grouped_impl(v, groups, X, A, B, M, r, scale, Y, T_save, ws, ws_bytes, stream);
}

int qlora_linear_bwd_grouped(const qlora_4bit_weight* W, int64_t groups, const void* X, const void* A,
                             const void* B, const void* dY, const float* T_saved, int64_t M, int64_t r,
                             float scale, void* dX, void* dA, void* dB, void* ws, size_t ws_bytes, void* stream) {
  WView v;
  const int st = view_4bit(W, v);
  return st != QLORA_OK ? st
                        : bwd_grouped_impl(v, groups, X, A, B, dY, T_saved, M, r, scale, dX, dA, dB, ws, ws_bytes,
                                           stream);
}

size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (M < 1 || N < 1 || K < 64 || (K % 64) != 0 || r < 1 || r > 256) return 0;
  if (!index_fits(M, N, K, r)) return 0;
  const Layout L = plan(M, N, K, r);
  return std::max(L.fwd_total, L.bwd_total);
}

int qlora_linear_fwd(const qlora_nf4_weight* W, const void* X, const void* A, const void* B,
                     int64_t M, int64_t r, float scale, void* Y, float* T_save, void* ws,
                     size_t ws_bytes, void* stream) {
  WView v;
  const int st = view_nf4(W, v);
  return st != QLORA_OK ? st : fwd_impl(v, X, A, B, M, r, scale, Y, T_save, ws, ws_bytes, stream);
}

int qlora_linear_fwd_noalloc(const qlora_nf4_weight* W, const void* X, const void* A, const void* B,
                             int64_t M, int64_t r, float scale, void* Y, float* T_save, void* stream) {
  WView v;
  int st = view_nf4(W, v);
  if (st != QLORA_OK) return st;
  // every argument check of the workspace form, and the size limit, before
  // any HIP call
  st = check_linear_args(v, X, A, B, M, r, scale);
  if (st != QLORA_OK) return st;
  if (!Y) return QLORA_ERR_NULL;
  if (!aligned(Y, 16) || (T_save && !aligned(T_save, 4))) return QLORA_ERR_ALIGN;
  if (plan(M, v.N, v.K, r).fwd_total > kScratchBytes) return QLORA_ERR_SCRATCH;
  void* ptr = nullptr;
  st = scratch_address(static_cast<hipStream_t>(stream), &ptr);
  if (st != QLORA_OK) return st;
  return fwd_impl(v, X, A, B, M, r, scale, Y, T_save, ptr, kScratchBytes, stream);
}

int qlora_linear_fwd_4bit(const qlora_4bit_weight* W, const void* X, const void* A, const void* B,
                          int64_t M, int64_t r, float scale, void* Y, float* T_save, void* ws,
                          size_t ws_bytes, void* stream) {
  WView v;
  const int st = view_4bit(W, v);
  return st != QLORA_OK ? st : fwd_impl(v, X, A, B, M, r, scale, Y, T_save, ws, ws_bytes, stream);
}

int qlora_linear_bwd(const qlora_nf4_weight* W, const void* X, const void* A, const void* B,
                     const void* dY, const float* T_saved, int64_t M, int64_t r, float scale,
                     void* dX, void* dA, void* dB, void* ws, size_t ws_bytes, void* stream) {
  WView v;
  const int st = view_nf4(W, v);
  return st != QLORA_OK ? st : bwd_impl(v, X, A, B, dY, T_saved, M, r, scale, dX, dA, dB, ws, ws_bytes, stream);
}

int qlora_linear_bwd_4bit(const qlora_4bit_weight* W, const void* X, const void* A, const void* B,
                          const void* dY, const float* T_saved, int64_t M, int64_t r, float scale,
                          void* dX, void* dA, void* dB, void* ws, size_t ws_bytes, void* stream) {
  WView v;
  const int st = view_4bit(W, v);
  return st != QLORA_OK ? st : bwd_impl(v, X, A, B, dY, T_saved, M, r, scale, dX, dA, dB, ws, ws_bytes, stream);
}

}  // extern "C"
