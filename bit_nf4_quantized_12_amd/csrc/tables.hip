// Host construction of the NF4 level table and the quantiser's search table.
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
  Levels lv;
  QuantTable qt;
  int status = 0;
};

Tables build() {
  Tables t;
  const double delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
  const double top = normal_quantile(delta);
  double v[16];
  int n = 0;
  for (int j = 7; j >= 1; --j) v[n++] = -normal_quantile(0.5 + j * (delta - 0.5) / 7.0) / top;
  v[n++] = 0.0;
  for (int j = 1; j <= 8; ++j) v[n++] = normal_quantile(0.5 + j * (delta - 0.5) / 8.0) / top;
  for (int i = 0; i < 16; ++i) t.lv.q[i] = (float)v[i];
  t.lv.q[0] = -1.0f;  // exact by construction (the same quantile on both sides)
  t.lv.q[15] = 1.0f;

  // Decision thresholds: x goes to the nearest level, a tie to the lower
  // code, so code > j exactly when x is above the midpoint of q_j and
  // q_{j+1}. As a float32 comparison: x > T_j with T_j = midpoint rounded down.
  float T[15];
  for (int j = 0; j < 15; ++j)
    T[j] = round_down_f32(((double)t.lv.q[j] + (double)t.lv.q[j + 1]) * 0.5);

  for (int c = 0; c < 32; ++c) {
    const double lo = c / 16.0 - 1.0, hi = (c + 1) / 16.0 - 1.0;
    int base = 0, inside = 0;
    float thr = 2.0f;
    for (int j = 0; j < 15; ++j) {
      if ((double)T[j] < lo) ++base;
      else if ((double)T[j] < hi) { ++inside; thr = T[j]; }
    }
    if (inside > 1) t.status = 1;  // cell too coarse for this table
    t.qt.thr[c] = thr;
    t.qt.base[c] = base;
  }
  // cell(x) is computed as trunc(fma(x, 16, 16)); its rounding can move an x
  // lying within 2^-24 of a cell edge into the neighbouring cell. That is
  // harmless unless a threshold itself lies that close to an edge.
  for (int j = 0; j < 15; ++j)
    for (int k = 0; k <= 32; ++k)
      if (std::fabs((double)T[j] - (k / 16.0 - 1.0)) <= 0x1p-20) t.status = 1;
  for (int i = 0; i < 15; ++i)
    if (!(t.lv.q[i] < t.lv.q[i + 1])) t.status = 1;
  return t;
}

const Tables& tables() {
  static const Tables t = build();
  return t;
}

}  // namespace

const Levels& host_levels() { return tables().lv; }
const QuantTable& host_quant_table() { return tables().qt; }
int tables_status() { return tables().status; }

}  // namespace qlora
