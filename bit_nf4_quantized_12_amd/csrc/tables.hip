// Host construction of the level tables of the 4-bit data types and of the
// quantiser's search tables.
//
// Levels: "QLoRA: Efficient Finetuning of Quantized LLMs" (inquiringlines.com),
// section "Method", paragraph "4-bit NormalFloat Quantization": quantiles of
// the standard normal distribution, 2^(k-1)+1 = 9 on the positive side and
// 2^(k-1) = 8 on the negative side, unified with one of the two zeros
// removed, then scaled into [-1, 1]. The pages garble the quantile formula
// and omit the table, so the outermost quantile sits at the probability
// 1 - (1/32 + 1/30)/2 (a reading; the equally spaced probabilities between
// 1/2 and that value on each side follow the text's construction).
#include <cfloat>
#include <cmath>
#include <mutex>

#include "common.hpp"

namespace qlora {
namespace {

// Standard normal quantile for p in [1/2, 1) by Newton's method on
// Phi(x) = erfc(-x / sqrt 2) / 2. Phi is concave for x > 0, so Newton
// started at 0 approaches the root from below without overshooting.
double normal_quantile(double p) {
  if (p == 0.5) return 0.0;
  const double inv_sqrt2 = 0.70710678118654752440;
  const double inv_sqrt2pi = 0.39894228040143267794;
  double x = 0.0;
  for (int it = 0; it < 200; ++it) {
    const double f = 0.5 * std::erfc(-x * inv_sqrt2) - p;
    const double pdf = inv_sqrt2pi * std::exp(-0.5 * x * x);
    const double step = f / pdf;
    const double nx = x - step;
    if (nx == x) break;
    x = nx;
    if (std::fabs(step) <= 1e-17 * std::fabs(x)) break;
  }
  return x;
}

// Largest float32 not above v (v is a double).
float round_down_f32(double v) {
  float f = (float)v;
  if ((double)f > v) f = std::nextafter(f, -INFINITY);
  return f;
}

struct Tables {
  Levels lv[kNumCodebooks];
  QuantTable qt[kNumCodebooks];
  int status = 0;
};

// NF4 levels: quantiles of N(0, 1), 8 negative and 9 positive (one zero
// shared), divided by the outermost quantile.
Levels nf4_levels() {
  Levels lv;
  const double delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
  const double top = normal_quantile(delta);
  double v[16];
  int n = 0;
  for (int j = 7; j >= 1; --j) v[n++] = -normal_quantile(0.5 + j * (delta - 0.5) / 7.0) / top;
  v[n++] = 0.0;
  for (int j = 1; j <= 8; ++j) v[n++] = normal_quantile(0.5 + j * (delta - 0.5) / 8.0) / top;
  for (int i = 0; i < 16; ++i) lv.q[i] = (float)v[i];
  lv.q[0] = -1.0f;  // exact by construction (the same quantile on both sides)
  lv.q[15] = 1.0f;
  return lv;
}

// Int4: k / 7 for k = -7 .. 7 at code k + 7; code 15 repeats +1.
Levels int4_levels() {
  Levels lv;
  for (int k = -7; k <= 7; ++k) lv.q[k + 7] = (float)((double)k / 7.0);
  lv.q[15] = 1.0f;
  return lv;
}

// FP4: the E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} with both signs
// (one zero), ascending, over 6; code 15 repeats +1.
Levels fp4_levels() {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  Levels lv;
  for (int i = 0; i < 7; ++i) lv.q[i] = (float)(-mag[7 - i] / 6.0);
  for (int i = 0; i < 8; ++i) lv.q[7 + i] = (float)(mag[i] / 6.0);
  lv.q[15] = 1.0f;
  return lv;
}

// Search table for ascending levels (equal neighbours allowed only at the
// top). Returns nonzero if the cells of this scale cannot represent the
// thresholds exactly.
int build_search(const Levels& lv, double scale, QuantTable& qt) {
  // x goes to the nearest level, a tie to the lower code, so code > j exactly
  // when x is above the midpoint of q_j and q_{j+1}. As a float32
  // comparison: x > T_j with T_j = midpoint rounded down. A threshold at or
  // above 1 is never exceeded (|x| <= 1) and needs no cell.
  float T[15];
  for (int j = 0; j < 15; ++j) T[j] = round_down_f32(((double)lv.q[j] + (double)lv.q[j + 1]) * 0.5);
  const int cells = (int)std::lround(2.0 * scale);
  if (cells > kQuantCells || std::fabs(2.0 * scale - cells) > 0.0) return 1;
  int bad = 0;
  // entry `cells` is the cell of x = 1 alone (lo = 1)
  for (int c = 0; c <= cells; ++c) {
    const double lo = c / scale - 1.0, hi = (c + 1) / scale - 1.0;
    int base = 0, inside = 0;
    float thr = 2.0f;
    for (int j = 0; j < 15; ++j) {
      if ((double)T[j] >= 1.0) continue;
      if ((double)T[j] < lo) ++base;
      else if ((double)T[j] < hi) { ++inside; thr = T[j]; }
    }
    if (inside > 1) bad = 1;  // cell too coarse for this table
    qt.thr[c] = thr;
    qt.base[c] = base;
  }
  for (int c = cells + 1; c <= kQuantCells; ++c) { qt.thr[c] = 2.0f; qt.base[c] = 0; }
  // cell(x) is computed as trunc(fma(x, scale, scale)); its rounding can move
  // an x lying within ~2^-23 of a cell edge into the neighbouring cell. That
  // is harmless unless a threshold itself lies that close to an edge.
  for (int j = 0; j < 15; ++j) {
    if ((double)T[j] >= 1.0) continue;
    for (int k = 0; k <= cells; ++k)
      if (std::fabs((double)T[j] - (k / scale - 1.0)) <= 0x1p-20) bad = 1;
  }
  qt.scale = (float)scale;
  return bad;
}

int check_levels(const Levels& lv) {
  for (int i = 0; i < 14; ++i)
    if (!(lv.q[i] < lv.q[i + 1])) return 1;
  if (!(lv.q[14] <= lv.q[15])) return 1;
  if (lv.q[0] != -1.0f || lv.q[7] != 0.0f || lv.q[15] != 1.0f) return 1;
  return 0;
}

Tables build() {
  Tables t;
  t.lv[kNF4] = nf4_levels();
  t.lv[kInt4] = int4_levels();
  t.lv[kFP4] = fp4_levels();
  for (int cb = 0; cb < kNumCodebooks; ++cb) {
    if (check_levels(t.lv[cb])) t.status = 1;
    // the first cell scale (16, 15.5, 15, ...) that represents the thresholds
    int bad = 1;
    for (int h = 32; h >= 20 && bad; --h) bad = build_search(t.lv[cb], h * 0.5, t.qt[cb]);
    if (bad) t.status = 1;
  }
  return t;
}

const Tables& tables() {
  static const Tables t = build();
  return t;
}

}  // namespace

const Levels& host_levels(int codebook) { return tables().lv[codebook]; }
const QuantTable& host_quant_table(int codebook) { return tables().qt[codebook]; }
int tables_status() { return tables().status; }

}  // namespace qlora
