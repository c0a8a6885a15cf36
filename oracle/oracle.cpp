// Plain CPU oracle of the tile-based differentiable 2D-splat rasterizer.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may load, link or call this file's library: only the
// tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no code, header, constant table or
// helper with the HIP library; the two only meet through the seeded input generators.
//
// Every routine here is the plain definition of the step it follows, single-threaded, in the order the pages state
// it, with no skips, no tiling shortcuts and no fusion:
//   * binning  - one key per (splat, overlapped 16x16 tile), key = (tile id << 32) | depth bits, value = splat
//                index; a stable sort by key; per-tile [start, end) ranges.  [C0 resident arena + C1 pass skip page,
//                section 2 table, rows "C0" and "C1"]
//   * forward  - per pixel, front-to-back compositing over the tile's sorted splats with
//                alpha = min(0.999, color_a * exp(-sigma)), the sigma < 0 and alpha < 1/255 rejects, the
//                T < 1e-4 stop and last-contributor tracking.  [A.9 f16 forward page, implementation listing;
//                W1 warp sparse skip + exp-skip page, section 1 table row "W1b"]
//   * backward - replay of the forward per pixel up to the last contributor and the 9 per-splat gradients
//                (mean xy, conic 3, rgb 3, opacity) in the forward-order form after = C_final - acc - mine.
//                [M3 per-splat backward page, section 1, "brush's actual structure" and "differences" rows]
//   * Adam     - textbook Adam with bias correction over parameter groups.  [rasterize forward + adam kernel audit
//                page, section 2 "(f) bandwidth floor"]
//
// Conventions the pages leave open (each is listed with its reading in the design notes):
//   splat record  {x, y, a, b, c, r, g, b, o}: mean, conic [[a b][b c]] (inverse covariance), rgb, color_a.
//   pixel centre  (px + 0.5, py + 0.5); tiles are 16x16, tile id = ty * tiles_x + tx.
//   exp           the fp32 value of e^-sigma correctly rounded (evaluated in double, then rounded once).
//   stop rule     T' = T * (1 - alpha) < 1e-4 is tested before compositing; the stopping splat is not composited.
//   clamp         when o * G >= 0.999 alpha is the constant 0.999, so sigma, the conic, the mean and o get no
//                 gradient from that pixel (the page's "raw_alpha < 0.999" branch).
//   culling       a splat is not binned if any field or its depth is non-finite, depth <= 0, a <= 0,
//                 a*c - b*b <= 0, or o lies outside [0, 1].
//   overlap rule  the axis-aligned box of the 3-sigma ellipse: rx = 3 sqrt(c/det), ry = 3 sqrt(a/det); or, as an
//                 option, the tiles of that box which the 3-sigma ellipse itself meets (ellipse_meets_tile).
//
// Built with g++ -O2 -ffp-contract=off and no fast-math, so every float expression below rounds after each
// operation, in the order written.
//
// Parity pins for every function live in tests/test_oracle_*.py (closed forms, brute force, invariants,
// central finite differences, and the numbers the pages print).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr uint32_t kTile = 16;  // 16x16 pixel tiles: 2,500 tiles at 800x800 [M3 per-splat backward page, section 3]

template <typename R>
struct Consts {
  // fp32 constants of the method, carried exactly into R.
  static constexpr R alpha_max = R(0.999f);         // [A.9 f16 forward page, listing]
  static constexpr R alpha_min = R(1.0f / 255.0f);  // [W1 warp sparse skip + exp-skip page, summary]
  static constexpr R t_stop = R(1e-4f);             // stop threshold chosen for these workloads
  static constexpr R half = R(0.5f);
};

inline bool finite_f(float v) { return std::isfinite(v); }

// Per-splat record view.
template <typename R>
struct Splat {
  R x, y, a, b, c, r, g, bl, o;
};

template <typename R>
inline Splat<R> load_splat(const R* s, uint32_t i) {
  const R* p = s + size_t(i) * 9;
  return Splat<R>{p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8]};
}

// e^v rounded once to the precision R.
inline float exp_r(float v) { return float(std::exp(double(v))); }
inline double exp_r(double v) { return std::exp(v); }

// ---------------------------------------------------------------------------------------------------------------
// Binning
// ---------------------------------------------------------------------------------------------------------------

struct TileRect {
  bool empty;
  uint32_t tx0, tx1, ty0, ty1;
};

// Culling and the 3-sigma axis-aligned tile rectangle of one splat, in fp32, one rounding per operation.
TileRect tile_rect(const float* sp, float depth, uint32_t tiles_x, uint32_t tiles_y) {
  TileRect none{true, 0, 0, 0, 0};
  for (int k = 0; k < 9; ++k)
    if (!finite_f(sp[k])) return none;
  if (!finite_f(depth) || !(depth > 0.0f)) return none;
  const float x = sp[0], y = sp[1], a = sp[2], b = sp[3], c = sp[4], o = sp[8];
  if (!(o >= 0.0f && o <= 1.0f)) return none;
  if (!(a > 0.0f)) return none;
  const float ac = a * c;
  const float bb = b * b;
  const float det = ac - bb;
  if (!(det > 0.0f)) return none;
  // Covariance diagonal of the inverse conic, then 3 standard deviations per axis.
  const float sxx = c / det;
  const float syy = a / det;
  const float rx = 3.0f * std::sqrt(sxx);
  const float ry = 3.0f * std::sqrt(syy);
  const float fx0 = std::floor((x - rx) / 16.0f);
  const float fx1 = std::floor((x + rx) / 16.0f);
  const float fy0 = std::floor((y - ry) / 16.0f);
  const float fy1 = std::floor((y + ry) / 16.0f);
  // Clip to the tile grid in float, then convert.
  const float cx0 = std::max(0.0f, fx0);
  const float cx1 = std::min(float(tiles_x - 1), fx1);
  const float cy0 = std::max(0.0f, fy0);
  const float cy1 = std::min(float(tiles_y - 1), fy1);
  if (cx0 > cx1 || cy0 > cy1) return none;
  return TileRect{false, uint32_t(cx0), uint32_t(cx1), uint32_t(cy0), uint32_t(cy1)};
}

// The exact-ellipse rule: tile (tx, ty) of the box is kept when the 3-sigma ellipse
// q(p) = (p - mean)^T [[a b][b c]] (p - mean) <= 9 meets the tile's closed square [16 tx, 16 tx + 16] x
// [16 ty, 16 ty + 16], i.e. when the minimum of q over the square is at most 9. That minimum is 0 if the mean lies
// in the square; otherwise it is on the boundary, the least of the four edge minima, each at the vertex of the
// one-dimensional quadratic clamped to the edge. fp32, one rounding per operation, in the order written.
float conic_q(float a, float b, float c, float dx, float dy) {
  return ((a * dx) * dx + ((b + b) * dx) * dy) + (c * dy) * dy;
}

float clamp_f(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

bool ellipse_meets_tile(float x, float y, float a, float b, float c, uint32_t tx, uint32_t ty) {
  const float x0 = 16.0f * float(tx), x1 = x0 + 16.0f;
  const float y0 = 16.0f * float(ty), y1 = y0 + 16.0f;
  const float dx0 = x0 - x, dx1 = x1 - x;
  const float dy0 = y0 - y, dy1 = y1 - y;
  if (dx0 <= 0.0f && dx1 >= 0.0f && dy0 <= 0.0f && dy1 >= 0.0f) return true;
  const float ex[2] = {dx0, dx1}, ey[2] = {dy0, dy1};
  float best = INFINITY;
  for (int e = 0; e < 2; ++e) {  // the edges x = x0 and x = x1: q(dx, .) is least at dy = -b dx / c
    const float dx = ex[e];
    const float dy = clamp_f(-(b * dx) / c, dy0, dy1);
    best = std::min(best, conic_q(a, b, c, dx, dy));
  }
  for (int e = 0; e < 2; ++e) {  // the edges y = y0 and y = y1: q(., dy) is least at dx = -b dy / a
    const float dy = ey[e];
    const float dx = clamp_f(-(b * dy) / a, dx0, dx1);
    best = std::min(best, conic_q(a, b, c, dx, dy));
  }
  return best <= 9.0f;
}

// Whether rule `ellipse` keeps tile (tx, ty) of splat sp's box (every box tile under the box rule).
bool keep_tile(const float* sp, bool ellipse, uint32_t tx, uint32_t ty) {
  return !ellipse || ellipse_meets_tile(sp[0], sp[1], sp[2], sp[3], sp[4], tx, ty);
}

uint32_t float_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

struct Pair {
  uint64_t key;
  uint32_t val;
};

// Emission in splat order, tiles row-major inside each splat's rectangle (those the rule keeps).
std::vector<Pair> emit_pairs(const float* splats, const float* depths, uint32_t n, uint32_t tiles_x,
                             uint32_t tiles_y, bool ellipse) {
  std::vector<Pair> pairs;
  for (uint32_t i = 0; i < n; ++i) {
    TileRect r = tile_rect(splats + size_t(i) * 9, depths[i], tiles_x, tiles_y);
    if (r.empty) continue;
    for (uint32_t ty = r.ty0; ty <= r.ty1; ++ty)
      for (uint32_t tx = r.tx0; tx <= r.tx1; ++tx) {
        if (!keep_tile(splats + size_t(i) * 9, ellipse, tx, ty)) continue;
        const uint64_t tile = uint64_t(ty) * tiles_x + tx;
        pairs.push_back(Pair{(tile << 32) | uint64_t(float_bits(depths[i])), i});
      }
  }
  return pairs;
}

// ---------------------------------------------------------------------------------------------------------------
// Forward, per pixel
// ---------------------------------------------------------------------------------------------------------------

// Counters of what the forward examined; also the decision fingerprint used by the finite-difference pins.
struct FwdStats {
  uint64_t visited;        // list entries examined (the stopping entry included)
  uint64_t sigma_neg;      // rejected because sigma < 0
  uint64_t alpha_reject;   // rejected because alpha < 1/255
  uint64_t contrib;        // composited
  uint64_t stopped;        // pixels that stopped because T' < 1e-4
  uint64_t sigma_ge_skip;  // examined entries with sigma >= 5.55 (each of them must be an alpha reject)
  uint64_t clamped;        // composited entries whose o*G reached the 0.999 clamp
  uint64_t fingerprint;    // hash of every decision taken, pixel by pixel
};

inline uint64_t mix(uint64_t h, uint64_t v) {
  h ^= v + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
  return h;
}

enum Decision : uint32_t { kSigmaNeg = 1, kAlphaReject = 2, kStop = 3, kComposite = 4, kCompositeClamped = 5 };

// One evaluation of splat s at pixel centre (cx, cy): F1..F5 of the forward.
template <typename R>
struct Eval {
  R dx, dy, sigma, G, oG, alpha;
  Decision d;  // kSigmaNeg, kAlphaReject or kComposite (the stop test is applied by the caller)
};

template <typename R>
inline Eval<R> evaluate(const Splat<R>& s, R cx, R cy) {
  using C = Consts<R>;
  Eval<R> e{};
  e.dx = cx - s.x;
  e.dy = cy - s.y;
  // sigma = 0.5 (a dx^2 + c dy^2) + b dx dy, the Gaussian's quadratic form under the conic.
  const R t_a = s.a * e.dx * e.dx;
  const R t_c = s.c * e.dy * e.dy;
  const R t_b = s.b * e.dx * e.dy;
  e.sigma = C::half * (t_a + t_c) + t_b;
  if (e.sigma < R(0)) {
    e.d = kSigmaNeg;
    return e;
  }
  e.G = exp_r(-e.sigma);
  e.oG = s.o * e.G;
  e.alpha = std::min(C::alpha_max, e.oG);
  e.d = (e.alpha < C::alpha_min) ? kAlphaReject : kComposite;
  return e;
}

template <typename R>
struct PixelOut {
  R rgb[3];
  R T;
  uint32_t last;
};

// Front-to-back compositing of one pixel over its tile's list (F1..F8).
template <typename R>
PixelOut<R> forward_pixel(const R* splats, const uint32_t* vals, uint32_t start, uint32_t end, uint32_t px,
                          uint32_t py, FwdStats* st) {
  using C = Consts<R>;
  const R cx = R(px) + C::half;
  const R cy = R(py) + C::half;
  PixelOut<R> out{{R(0), R(0), R(0)}, R(1), 0};
  uint64_t h = mix(0, (uint64_t(py) << 32) | px);
  for (uint32_t k = start; k < end; ++k) {
    const uint32_t idx = vals[k];
    const Splat<R> s = load_splat(splats, idx);
    const Eval<R> e = evaluate(s, cx, cy);
    st->visited++;
    if (e.d == kSigmaNeg) {
      st->sigma_neg++;
      h = mix(h, (uint64_t(k - start) << 3) | kSigmaNeg);
      continue;
    }
    if (e.sigma >= R(5.55f)) st->sigma_ge_skip++;
    if (e.d == kAlphaReject) {
      st->alpha_reject++;
      h = mix(h, (uint64_t(k - start) << 3) | kAlphaReject);
      continue;
    }
    const R next_T = out.T * (R(1) - e.alpha);
    if (next_T < C::t_stop) {
      st->stopped++;
      h = mix(h, (uint64_t(k - start) << 3) | kStop);
      break;
    }
    const R w = e.alpha * out.T;
    out.rgb[0] = out.rgb[0] + s.r * w;
    out.rgb[1] = out.rgb[1] + s.g * w;
    out.rgb[2] = out.rgb[2] + s.bl * w;
    out.T = next_T;
    out.last = k - start + 1;
    st->contrib++;
    const bool clamped = !(e.oG < C::alpha_max);
    if (clamped) st->clamped++;
    h = mix(h, (uint64_t(k - start) << 3) | (clamped ? kCompositeClamped : kComposite));
  }
  st->fingerprint = mix(st->fingerprint, h);
  return out;
}

template <typename R>
void render_forward(const R* splats, const uint32_t* vals, const uint32_t* ranges, uint32_t width,
                    uint32_t row_begin, uint32_t row_end, R* out_rgba, R* final_T, uint32_t* last_contrib,
                    FwdStats* st) {
  const uint32_t tiles_x = (width + kTile - 1) / kTile;
  for (uint32_t py = row_begin; py < row_end; ++py)
    for (uint32_t px = 0; px < width; ++px) {
      const uint32_t t = (py / kTile) * tiles_x + (px / kTile);
      const PixelOut<R> o = forward_pixel(splats, vals, ranges[2 * t], ranges[2 * t + 1], px, py, st);
      const size_t p = size_t(py) * width + px;
      out_rgba[4 * p + 0] = o.rgb[0];
      out_rgba[4 * p + 1] = o.rgb[1];
      out_rgba[4 * p + 2] = o.rgb[2];
      out_rgba[4 * p + 3] = R(1) - o.T;
      final_T[p] = o.T;
      last_contrib[p] = o.last;
    }
}

// ---------------------------------------------------------------------------------------------------------------
// Backward, per pixel (B1..B9); per-splat sums in double, in a fixed order (pixels row-major, then list order).
// ---------------------------------------------------------------------------------------------------------------

// Counters of the backward's replay (entries before each pixel's last contributor).
struct BwdStats {
  uint64_t visited;        // sum over pixels of last_contrib
  uint64_t sigma_neg;      // rejected because sigma < 0
  uint64_t sigma_ge_skip;  // rejected with sigma >= 5.55 (a subset of alpha_reject)
  uint64_t alpha_reject;   // rejected because alpha < 1/255
  uint64_t contrib;        // composited, gradient terms formed
  uint64_t clamped;        // composited with o*G >= 0.999 (no opacity / geometry terms)
};

template <typename R>
void render_backward(const R* splats, uint32_t n, const uint32_t* vals, const uint32_t* ranges, uint32_t width,
                     uint32_t row_begin, uint32_t row_end, const R* out_rgba, const R* final_T,
                     const uint32_t* last_contrib, const R* v_out, double* acc_grad /* [n][9], accumulated */,
                     BwdStats* st) {
  using C = Consts<R>;
  (void)final_T;  // the forward-order form needs C_final and the replayed T, not the final T
  (void)n;
  const uint32_t tiles_x = (width + kTile - 1) / kTile;
  for (uint32_t py = row_begin; py < row_end; ++py)
    for (uint32_t px = 0; px < width; ++px) {
      const size_t p = size_t(py) * width + px;
      const uint32_t t = (py / kTile) * tiles_x + (px / kTile);
      const uint32_t start = ranges[2 * t];
      const uint32_t last = last_contrib[p];
      const R cx = R(px) + C::half;
      const R cy = R(py) + C::half;
      const R g[3] = {v_out[4 * p + 0], v_out[4 * p + 1], v_out[4 * p + 2]};
      const R Cf[3] = {out_rgba[4 * p + 0], out_rgba[4 * p + 1], out_rgba[4 * p + 2]};
      R T = R(1);
      R acc[3] = {R(0), R(0), R(0)};
      for (uint32_t k = start; k < start + last; ++k) {
        const uint32_t idx = vals[k];
        const Splat<R> s = load_splat(splats, idx);
        const Eval<R> e = evaluate(s, cx, cy);
        st->visited++;
        if (e.d == kSigmaNeg) st->sigma_neg++;
        if (e.d == kAlphaReject) {
          st->alpha_reject++;
          if (e.sigma >= R(5.55f)) st->sigma_ge_skip++;
        }
        if (e.d != kComposite) continue;
        st->contrib++;
        if (!(e.oG < C::alpha_max)) st->clamped++;
        double* gr = acc_grad + size_t(idx) * 9;
        const R rgb[3] = {s.r, s.g, s.bl};
        // B1: weight of this splat in the pixel, and the colour gradient.
        const R w = e.alpha * T;
        for (int ch = 0; ch < 3; ++ch) gr[5 + ch] += double(w * g[ch]);
        // B2..B3: what lies behind this splat, from the forward order, and dL/dalpha.
        const R one_m = R(1) - e.alpha;
        R my[3], dl_da = R(0);
        for (int ch = 0; ch < 3; ++ch) {
          my[ch] = rgb[ch] * w;
          const R after = Cf[ch] - acc[ch] - my[ch];
          dl_da = dl_da + g[ch] * (rgb[ch] * T - after / one_m);
        }
        // B4..B7: only where alpha is not clamped does alpha depend on o and sigma.
        if (e.oG < C::alpha_max) {
          gr[8] += double(dl_da * e.G);
          const R dl_ds = -(dl_da * e.oG);
          gr[2] += double(dl_ds * (C::half * e.dx * e.dx));
          gr[3] += double(dl_ds * (e.dx * e.dy));
          gr[4] += double(dl_ds * (C::half * e.dy * e.dy));
          gr[0] += double(dl_ds * -(s.a * e.dx + s.b * e.dy));
          gr[1] += double(dl_ds * -(s.b * e.dx + s.c * e.dy));
        }
        // B8: advance the replay.
        for (int ch = 0; ch < 3; ++ch) acc[ch] = acc[ch] + my[ch];
        T = T * one_m;
      }
    }
}

// The backward's exact values on its given inputs and the fp32 method's decisions: each pixel's decisions - which
// entries before last_contrib composite, and which of them reach the 0.999 clamp - are taken by the fp32
// evaluation above (the method's precision, the same decisions as the fp32 backward), and every value is then
// formed in fp64 from the same records: sigma, G, alpha (0.999 exactly where the fp32 evaluation clamped, o G
// elsewhere), the transmittance and the B1..B8 terms in the forward-order form, with C_final the forward output
// the backward is given (out_rgba, in double). The result is what the backward computes from its inputs, free of
// the fp32 rounding of its own values.
void render_backward_exact(const float* splats, const uint32_t* vals, const uint32_t* ranges, uint32_t width,
                           uint32_t row_begin, uint32_t row_end, const double* out_rgba,
                           const uint32_t* last_contrib, const float* v_out, double* acc_grad) {
  using Cf = Consts<float>;
  using C = Consts<double>;
  const uint32_t tiles_x = (width + kTile - 1) / kTile;
  for (uint32_t py = row_begin; py < row_end; ++py)
    for (uint32_t px = 0; px < width; ++px) {
      const size_t p = size_t(py) * width + px;
      const uint32_t t = (py / kTile) * tiles_x + (px / kTile);
      const uint32_t start = ranges[2 * t];
      const uint32_t last = last_contrib[p];
      const float cxf = float(px) + Cf::half, cyf = float(py) + Cf::half;
      const double cx = double(cxf), cy = double(cyf);
      const double g[3] = {v_out[4 * p + 0], v_out[4 * p + 1], v_out[4 * p + 2]};
      const double Cfin[3] = {out_rgba[4 * p + 0], out_rgba[4 * p + 1], out_rgba[4 * p + 2]};
      double acc[3] = {0.0, 0.0, 0.0}, T = 1.0;
      for (uint32_t k = start; k < start + last; ++k) {
        const uint32_t idx = vals[k];
        const Eval<float> ef = evaluate(load_splat(splats, idx), cxf, cyf);  // the decision, in fp32
        if (ef.d != kComposite) continue;
        const bool clamped = !(ef.oG < Cf::alpha_max);
        const float* sp = splats + size_t(idx) * 9;
        const Splat<double> sd{sp[0], sp[1], sp[2], sp[3], sp[4], sp[5], sp[6], sp[7], sp[8]};
        const Eval<double> e = evaluate(sd, cx, cy);  // the values, in fp64
        const double alpha = clamped ? C::alpha_max : e.oG;
        const double rgb[3] = {sd.r, sd.g, sd.bl};
        double* gr = acc_grad + size_t(idx) * 9;
        const double w = alpha * T;  // B1
        for (int ch = 0; ch < 3; ++ch) gr[5 + ch] += w * g[ch];
        const double one_m = 1.0 - alpha;  // B2..B3
        double my[3], dl_da = 0.0;
        for (int ch = 0; ch < 3; ++ch) {
          my[ch] = rgb[ch] * w;
          const double after = Cfin[ch] - acc[ch] - my[ch];
          dl_da += g[ch] * (rgb[ch] * T - after / one_m);
        }
        if (!clamped) {  // B4..B7
          gr[8] += dl_da * e.G;
          const double dl_ds = -(dl_da * e.oG);
          gr[2] += dl_ds * (0.5 * e.dx * e.dx);
          gr[3] += dl_ds * (e.dx * e.dy);
          gr[4] += dl_ds * (0.5 * e.dy * e.dy);
          gr[0] += dl_ds * -(sd.a * e.dx + sd.b * e.dy);
          gr[1] += dl_ds * -(sd.b * e.dx + sd.c * e.dy);
        }
        for (int ch = 0; ch < 3; ++ch) acc[ch] += my[ch];  // B8
        T *= one_m;
      }
    }
}

// Runs fn(thread, row_begin, row_end) over bands of 16 pixel rows dealt round-robin to `threads` threads.
template <typename Fn>
void run_bands(uint32_t height, uint32_t threads, Fn fn) {
  const uint32_t bands = (height + kTile - 1) / kTile;
  std::vector<std::thread> pool;
  for (uint32_t t = 0; t < threads; ++t)
    pool.emplace_back([=] {
      for (uint32_t b = t; b < bands; b += threads) fn(t, b * kTile, std::min(height, (b + 1) * kTile));
    });
  for (auto& th : pool) th.join();
}

}  // namespace

// ===============================================================================================================
// C entry points (host pointers; row-major layouts as documented per function). Return 0 on success, -1 on a bad
// argument.
// ===============================================================================================================

extern "C" {

// Number of (splat, tile) pairs the binning emits (rule 0: box, 1: exact ellipse).
int oracle_bin_count_rule(const float* splats, const float* depths, uint32_t n, uint32_t width, uint32_t height,
                          int rule, uint64_t* num_pairs) {
  if (!num_pairs || (n && (!splats || !depths)) || width == 0 || height == 0 || (rule != 0 && rule != 1)) return -1;
  const uint32_t tiles_x = (width + kTile - 1) / kTile, tiles_y = (height + kTile - 1) / kTile;
  uint64_t total = 0;
  for (uint32_t i = 0; i < n; ++i) {
    TileRect r = tile_rect(splats + size_t(i) * 9, depths[i], tiles_x, tiles_y);
    if (r.empty) continue;
    for (uint32_t ty = r.ty0; ty <= r.ty1; ++ty)
      for (uint32_t tx = r.tx0; tx <= r.tx1; ++tx) total += keep_tile(splats + size_t(i) * 9, rule == 1, tx, ty);
  }
  *num_pairs = total;
  return 0;
}

int oracle_bin_count(const float* splats, const float* depths, uint32_t n, uint32_t width, uint32_t height,
                     uint64_t* num_pairs) {
  return oracle_bin_count_rule(splats, depths, n, width, height, 0, num_pairs);
}

// The exact-ellipse test of one splat {x, y, a, b, c} against tile (tx, ty): 1 kept, 0 not.
int oracle_ellipse_meets_tile(const float* splat, uint32_t tx, uint32_t ty) {
  return ellipse_meets_tile(splat[0], splat[1], splat[2], splat[3], splat[4], tx, ty) ? 1 : 0;
}

// Tile rectangle of one splat: rect = {tx0, tx1, ty0, ty1}; returns 1 if the splat is culled or off the grid.
int oracle_tile_rect(const float* splat, float depth, uint32_t width, uint32_t height, uint32_t* rect) {
  const uint32_t tiles_x = (width + kTile - 1) / kTile, tiles_y = (height + kTile - 1) / kTile;
  TileRect r = tile_rect(splat, depth, tiles_x, tiles_y);
  rect[0] = r.tx0;
  rect[1] = r.tx1;
  rect[2] = r.ty0;
  rect[3] = r.ty1;
  return r.empty ? 1 : 0;
}

// Sorted keys [capacity], values [capacity] and per-tile ranges [2 * tiles] (start, end) for the pair list
// (rule 0: box, 1: exact ellipse).
int oracle_bin_rule(const float* splats, const float* depths, uint32_t n, uint32_t width, uint32_t height, int rule,
                    uint64_t* keys, uint32_t* vals, uint32_t* ranges, uint64_t capacity) {
  if ((n && (!splats || !depths)) || width == 0 || height == 0 || !ranges || (rule != 0 && rule != 1)) return -1;
  const uint32_t tiles_x = (width + kTile - 1) / kTile, tiles_y = (height + kTile - 1) / kTile;
  std::vector<Pair> pairs = emit_pairs(splats, depths, n, tiles_x, tiles_y, rule == 1);
  if (pairs.size() > capacity || (!pairs.empty() && (!keys || !vals))) return -1;
  std::stable_sort(pairs.begin(), pairs.end(), [](const Pair& l, const Pair& r) { return l.key < r.key; });
  for (size_t k = 0; k < pairs.size(); ++k) {
    keys[k] = pairs[k].key;
    vals[k] = pairs[k].val;
  }
  // ranges[t] = [first pair with tile >= t, first pair with tile >= t + 1)
  const uint64_t num_tiles = uint64_t(tiles_x) * tiles_y;
  for (uint64_t t = 0; t < num_tiles; ++t) {
    auto lo = std::lower_bound(pairs.begin(), pairs.end(), t << 32,
                               [](const Pair& p, uint64_t k) { return p.key < k; });
    auto hi = std::lower_bound(pairs.begin(), pairs.end(), (t + 1) << 32,
                               [](const Pair& p, uint64_t k) { return p.key < k; });
    ranges[2 * t] = uint32_t(lo - pairs.begin());
    ranges[2 * t + 1] = uint32_t(hi - pairs.begin());
  }
  return 0;
}

int oracle_bin(const float* splats, const float* depths, uint32_t n, uint32_t width, uint32_t height,
               uint64_t* keys, uint32_t* vals, uint32_t* ranges, uint64_t capacity) {
  return oracle_bin_rule(splats, depths, n, width, height, 0, keys, vals, ranges, capacity);
}

// Stable sort of (key, value) pairs by key; the reference for the radix sort alone.
int oracle_sort_pairs(const uint64_t* keys_in, const uint32_t* vals_in, uint64_t n, uint64_t* keys_out,
                      uint32_t* vals_out) {
  if (n && (!keys_in || !vals_in || !keys_out || !vals_out)) return -1;
  std::vector<Pair> pairs(n);
  for (uint64_t k = 0; k < n; ++k) pairs[k] = Pair{keys_in[k], vals_in[k]};
  std::stable_sort(pairs.begin(), pairs.end(), [](const Pair& l, const Pair& r) { return l.key < r.key; });
  for (uint64_t k = 0; k < n; ++k) {
    keys_out[k] = pairs[k].key;
    vals_out[k] = pairs[k].val;
  }
  return 0;
}

// stats[8] = {visited, sigma_neg, alpha_reject, contrib, stopped, sigma_ge_skip, clamped, fingerprint}
int oracle_render_forward_f32(const float* splats, const uint32_t* vals, const uint32_t* ranges, uint32_t width,
                              uint32_t height, float* out_rgba, float* final_T, uint32_t* last_contrib,
                              uint64_t* stats) {
  if (!ranges || !out_rgba || !final_T || !last_contrib || width == 0 || height == 0) return -1;
  FwdStats st{};
  render_forward<float>(splats, vals, ranges, width, 0, height, out_rgba, final_T, last_contrib, &st);
  if (stats) std::memcpy(stats, &st, sizeof st);
  return 0;
}

int oracle_render_forward_f64(const double* splats, const uint32_t* vals, const uint32_t* ranges, uint32_t width,
                              uint32_t height, double* out_rgba, double* final_T, uint32_t* last_contrib,
                              uint64_t* stats) {
  if (!ranges || !out_rgba || !final_T || !last_contrib || width == 0 || height == 0) return -1;
  FwdStats st{};
  render_forward<double>(splats, vals, ranges, width, 0, height, out_rgba, final_T, last_contrib, &st);
  if (stats) std::memcpy(stats, &st, sizeof st);
  return 0;
}

// splats_grad [n][9] in the record order {x, y, a, b, c, r, g, b, o}; sums kept in double, rounded once.
// stats[6] (optional) = {visited, sigma_neg, sigma_ge_skip, alpha_reject, contrib, clamped} of the replay.
int oracle_render_backward_f32(const float* splats, uint32_t n, const uint32_t* vals, const uint32_t* ranges,
                               uint32_t width, uint32_t height, const float* out_rgba, const float* final_T,
                               const uint32_t* last_contrib, const float* v_out, float* splats_grad,
                               uint64_t* stats) {
  if (!ranges || !out_rgba || !last_contrib || !v_out || (n && !splats_grad) || width == 0 || height == 0)
    return -1;
  std::vector<double> acc(size_t(n) * 9, 0.0);
  BwdStats st{};
  render_backward<float>(splats, n, vals, ranges, width, 0, height, out_rgba, final_T, last_contrib, v_out,
                         acc.data(), &st);
  if (stats) std::memcpy(stats, &st, sizeof st);
  for (size_t k = 0; k < acc.size(); ++k) splats_grad[k] = float(acc[k]);
  return 0;
}

int oracle_render_backward_f64(const double* splats, uint32_t n, const uint32_t* vals, const uint32_t* ranges,
                               uint32_t width, uint32_t height, const double* out_rgba, const double* final_T,
                               const uint32_t* last_contrib, const double* v_out, double* splats_grad) {
  if (!ranges || !out_rgba || !last_contrib || !v_out || (n && !splats_grad) || width == 0 || height == 0)
    return -1;
  BwdStats st{};
  std::fill(splats_grad, splats_grad + size_t(n) * 9, 0.0);
  render_backward<double>(splats, n, vals, ranges, width, 0, height, out_rgba, final_T, last_contrib, v_out,
                          splats_grad, &st);
  return 0;
}

// The backward's exact values on its given inputs and the fp32 method's decisions (render_backward_exact), over
// `threads` host threads (bands of 16 pixel rows; per-thread sums in double added in thread order). out_rgba is the
// forward output the backward is given, in double.
int oracle_render_backward_exact(const float* splats, uint32_t n, const uint32_t* vals, const uint32_t* ranges,
                                 uint32_t width, uint32_t height, const double* out_rgba,
                                 const uint32_t* last_contrib, const float* v_out, double* splats_grad,
                                 uint32_t threads) {
  if (!ranges || !out_rgba || !last_contrib || !v_out || (n && !splats_grad) || width == 0 || height == 0 ||
      threads == 0)
    return -1;
  std::vector<std::vector<double>> acc(threads, std::vector<double>(size_t(n) * 9, 0.0));
  run_bands(height, threads, [&](uint32_t t, uint32_t y0, uint32_t y1) {
    render_backward_exact(splats, vals, ranges, width, y0, y1, out_rgba, last_contrib, v_out, acc[t].data());
  });
  std::fill(splats_grad, splats_grad + size_t(n) * 9, 0.0);
  for (uint32_t t = 0; t < threads; ++t)
    for (size_t k = 0; k < size_t(n) * 9; ++k) splats_grad[k] += acc[t][k];
  return 0;
}

// The same forward and backward spread over `threads` host threads for timing on all cores: bands of 16 pixel
// rows (one tile row) are dealt round-robin to the threads, which run the per-pixel functions above unchanged.
// The forward's outputs are identical to the single-threaded call; the backward's per-splat sums are kept per
// thread in double and added in thread order, so they may differ from the single-threaded sums in the last bits
// of the double before the one rounding to fp32.
int oracle_render_forward_f32_mt(const float* splats, const uint32_t* vals, const uint32_t* ranges, uint32_t width,
                                 uint32_t height, float* out_rgba, float* final_T, uint32_t* last_contrib,
                                 uint32_t threads) {
  if (!ranges || !out_rgba || !final_T || !last_contrib || width == 0 || height == 0 || threads == 0) return -1;
  std::vector<FwdStats> st(threads);
  run_bands(height, threads, [&](uint32_t t, uint32_t y0, uint32_t y1) {
    render_forward<float>(splats, vals, ranges, width, y0, y1, out_rgba, final_T, last_contrib, &st[t]);
  });
  return 0;
}

int oracle_render_backward_f32_mt(const float* splats, uint32_t n, const uint32_t* vals, const uint32_t* ranges,
                                  uint32_t width, uint32_t height, const float* out_rgba, const float* final_T,
                                  const uint32_t* last_contrib, const float* v_out, float* splats_grad,
                                  uint32_t threads) {
  if (!ranges || !out_rgba || !last_contrib || !v_out || (n && !splats_grad) || width == 0 || height == 0 ||
      threads == 0)
    return -1;
  std::vector<std::vector<double>> acc(threads, std::vector<double>(size_t(n) * 9, 0.0));
  std::vector<BwdStats> st(threads);
  run_bands(height, threads, [&](uint32_t t, uint32_t y0, uint32_t y1) {
    render_backward<float>(splats, n, vals, ranges, width, y0, y1, out_rgba, final_T, last_contrib, v_out,
                           acc[t].data(), &st[t]);
  });
  for (size_t k = 0; k < size_t(n) * 9; ++k) {
    double sum = 0.0;
    for (uint32_t t = 0; t < threads; ++t) sum += acc[t][k];
    splats_grad[k] = float(sum);
  }
  return 0;
}

// One Adam step over `count` elements of one parameter group:
//   m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;  p <- p - lr (m / bc1) / (sqrt(v / bc2) + eps)
// with bc1 = 1 - b1^t and bc2 = 1 - b2^t supplied by the caller.
int oracle_adam_step(float* param, const float* grad, float* m, float* v, uint64_t count, float lr, float beta1,
                     float beta2, float eps, float bc1, float bc2) {
  if (count && (!param || !grad || !m || !v)) return -1;
  const float one_m_b1 = 1.0f - beta1;
  const float one_m_b2 = 1.0f - beta2;
  for (uint64_t i = 0; i < count; ++i) {
    const float g = grad[i];
    const float m_new = beta1 * m[i] + one_m_b1 * g;
    const float v_new = beta2 * v[i] + one_m_b2 * (g * g);
    const float m_hat = m_new / bc1;
    const float v_hat = v_new / bc2;
    const float denom = std::sqrt(v_hat) + eps;
    param[i] = param[i] - (lr * m_hat) / denom;
    m[i] = m_new;
    v[i] = v_new;
  }
  return 0;
}

// Per-entry trace of one pixel's forward, for the invariant pins. For each examined list entry j < max_len:
// code[j] in {1 sigma<0, 2 alpha reject, 3 stop, 4 composite, 5 composite clamped}, sigma[j], alpha[j] (0 when
// sigma < 0), T_before[j], T_after[j]. Returns the number of entries written.
int oracle_trace_pixel_f32(const float* splats, const uint32_t* vals, const uint32_t* ranges, uint32_t width,
                           uint32_t height, uint32_t px, uint32_t py, uint32_t max_len, uint32_t* code,
                           float* sigma, float* alpha, float* T_before, float* T_after) {
  if (px >= width || py >= height) return -1;
  using C = Consts<float>;
  const uint32_t tiles_x = (width + kTile - 1) / kTile;
  const uint32_t t = (py / kTile) * tiles_x + (px / kTile);
  const float cx = float(px) + C::half, cy = float(py) + C::half;
  float T = 1.0f;
  uint32_t j = 0;
  for (uint32_t k = ranges[2 * t]; k < ranges[2 * t + 1] && j < max_len; ++k, ++j) {
    const Splat<float> s = load_splat(splats, vals[k]);
    const Eval<float> e = evaluate(s, cx, cy);
    sigma[j] = e.sigma;
    alpha[j] = e.d == kSigmaNeg ? 0.0f : e.alpha;
    T_before[j] = T;
    if (e.d != kComposite) {
      code[j] = e.d;
      T_after[j] = T;
      continue;
    }
    const float next_T = T * (1.0f - e.alpha);
    if (next_T < C::t_stop) {
      code[j] = kStop;
      T_after[j] = T;
      ++j;
      break;
    }
    code[j] = (e.oG < C::alpha_max) ? kComposite : kCompositeClamped;
    T = next_T;
    T_after[j] = T;
  }
  return int(j);
}

// One pixel's compositing candidates with the stop test left out, for judging stop decisions taken on a transmittance
// that carries rounding error: every entry of the tile's list that passes the sigma and alpha tests, in list order,
// composited as the forward composites (T' = T (1 - alpha), colour += rgb alpha T) whatever T' is. For candidate
// j < max_len: pos[j] (its 1-based list position, the value last_contrib takes when it is the last one composited),
// alpha[j], T_next[j] = T' and rgb[3 j .. 3 j + 2], the colour once it is composited. The forward stops at the first
// candidate whose T_next is below 1e-4. Returns the number of candidates written.
int oracle_trace_candidates_f32(const float* splats, const uint32_t* vals, const uint32_t* ranges, uint32_t width,
                                uint32_t height, uint32_t px, uint32_t py, uint32_t max_len, uint32_t* pos,
                                float* alpha, float* T_next, float* rgb) {
  if (px >= width || py >= height) return -1;
  using C = Consts<float>;
  const uint32_t tiles_x = (width + kTile - 1) / kTile;
  const uint32_t t = (py / kTile) * tiles_x + (px / kTile);
  const float cx = float(px) + C::half, cy = float(py) + C::half;
  float T = 1.0f, cr = 0.0f, cg = 0.0f, cb = 0.0f;
  uint32_t j = 0;
  for (uint32_t k = ranges[2 * t]; k < ranges[2 * t + 1] && j < max_len; ++k) {
    const Splat<float> s = load_splat(splats, vals[k]);
    const Eval<float> e = evaluate(s, cx, cy);
    if (e.d != kComposite) continue;
    const float next_T = T * (1.0f - e.alpha);
    const float w = e.alpha * T;
    cr = cr + s.r * w;
    cg = cg + s.g * w;
    cb = cb + s.bl * w;
    T = next_T;
    pos[j] = k - ranges[2 * t] + 1;
    alpha[j] = e.alpha;
    T_next[j] = next_T;
    rgb[3 * j] = cr;
    rgb[3 * j + 1] = cg;
    rgb[3 * j + 2] = cb;
    ++j;
  }
  return int(j);
}

}  // extern "C"
