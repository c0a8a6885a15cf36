// Device helpers shared by the forward and backward raster kernels. Both kernels must take exactly the same
// decisions for every (pixel, splat), so the evaluation below is the only place sigma, exp(-sigma) and alpha are
// computed. The file is compiled without floating-point contraction: every float expression rounds once per
// operation, in the order written, which makes each decision equal to a plain fp32 evaluation of the definition.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gsr {

// Method constants (fp32). [A.9 f16 forward page, listing: alpha clamp 0.999; W1 warp sparse skip + exp-skip page,
// summary: alpha < 1/255 reject and the sigma >= 5.55 skip]
constexpr float kAlphaMax = 0.999f;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kTStop = 1e-4f;
constexpr float kSigmaSkip = 5.55f;
// A certain alpha reject: o * exp(-sigma) evaluated with the hardware exp2 (relative error below 1e-6 here) under
// 1/255 by a relative margin of 2^-12 cannot reach 1/255 when evaluated exactly.
constexpr float kAlphaMinCertain = kAlphaMin * (1.0f - 1.0f / 4096.0f);

// e^x rounded to fp32, for |x| below 80. Cody-Waite reduction x = k ln2 + r with |r| <= ln2 / 2 (ln2 split into a
// 32-bit head, exact in k * head for |k| < 2^20, and a tail), the Taylor series of e^r to degree 11 in fp64
// (truncation below 7e-15 relative) evaluated by Estrin's scheme (pairs, then powers r^2, r^4, r^8: every fma adds
// a temporary, so no coefficient register is overwritten), then scaling by 2^k and one rounding to fp32. The fp64
// value is within about 2^-46 of e^x, so the fp32 result is the correctly rounded one except when e^x lies within
// 2^-46 (relative) of the midpoint between two floats, i.e. about one argument in 2^22.
__host__ __device__ __forceinline__ float exp_rn(float x) {
  const double xd = double(x);
  const double k = rint(xd * 1.4426950408889634074);
  double r = fma(-k, 6.93147180369123816490e-01, xd);
  r = fma(-k, 1.90821492927058770002e-10, r);
  const double r2 = r * r, r4 = r2 * r2, r8 = r4 * r4;
  const double q0 = r + 1.0;                                  // 1 + r
  const double q1 = fma(1.0 / 6.0, r, 0.5);                   // 1/2! + r/3!
  const double q2 = fma(1.0 / 120.0, r, 1.0 / 24.0);          // 1/4! + r/5!
  const double q3 = fma(1.0 / 5040.0, r, 1.0 / 720.0);        // 1/6! + r/7!
  const double q4 = fma(1.0 / 362880.0, r, 1.0 / 40320.0);    // 1/8! + r/9!
  const double q5 = fma(1.0 / 39916800.0, r, 1.0 / 3628800.0);  // 1/10! + r/11!
  const double s0 = fma(q1, r2, q0);
  const double s1 = fma(q3, r2, q2);
  const double s2 = fma(q5, r2, q4);
  const double p = fma(s2, r8, fma(s1, r4, s0));
  return float(ldexp(p, int(k)));
}

// One splat as staged in LDS for a batch: 48 bytes, read by every lane of a wavefront at the same address.
struct alignas(16) StagedSplat {
  float x, y, ha, b;  // mean, a / 2, b
  float hc, o, r, g;  // c / 2, opacity, red, green
  float bl, a, c;     // blue, a, c (the backward's mean gradient needs the full conic)
  uint32_t idx;       // splat index, or 0xFFFFFFFF for a slot that must not contribute
};

__device__ __forceinline__ StagedSplat stage_splat(const float* __restrict__ splats, uint32_t idx, uint32_t n) {
  StagedSplat s;
  if (idx < n) {
    const float* p = splats + size_t(idx) * 9;
    s.x = p[0];
    s.y = p[1];
    s.a = p[2];
    s.b = p[3];
    s.c = p[4];
    s.r = p[5];
    s.g = p[6];
    s.bl = p[7];
    s.o = p[8];
    s.ha = 0.5f * s.a;  // exact: scaling by a power of two
    s.hc = 0.5f * s.c;
    s.idx = idx;
  } else {
    // o = 0 makes every evaluation a reject
    s.x = s.y = s.a = s.b = s.c = s.r = s.g = s.bl = s.o = s.ha = s.hc = 0.0f;
    s.idx = 0xFFFFFFFFu;
  }
  return s;
}

// Pixel of lane `lane` of wave `w` in a 16x16 tile: each wave covers one 8x8 quarter (waves 0..3 = top-left,
// top-right, bottom-left, bottom-right), lanes row-major inside it.
__device__ __forceinline__ uint32_t lane_px(uint32_t w, uint32_t lane) { return 8u * (w & 1u) + (lane & 7u); }
__device__ __forceinline__ uint32_t lane_py(uint32_t w, uint32_t lane) { return 8u * (w >> 1) + (lane >> 3); }

// Which of the tile's four 8x8 wave blocks splat s can reach with alpha >= 1/255: bit q set unless the splat is
// provably a reject at every pixel centre of block q. (x0, y0) is the first pixel centre of the tile.
// alpha <= o exp(-sigma) reaches 1/255 only where sigma <= L = ln(255 o), an ellipse whose bounding box has
// half-widths sqrt(2 L c / det) and sqrt(2 L a / det). Evaluated in fp32 and widened for every rounding involved:
// the fp32 sigma of the per-lane test (relative error below 4.5 eps kappa, where kappa = (a + c)^2 / det bounds the
// conic's condition number), the fp32 det here (relative error below 2 eps kappa), the fast log (absolute error
// below 1e-5), sqrt and the products (a few ulp): L gets +1e-3 and the factor 1 + 1e-6 kappa, the half-widths
// x1.001 + 0.01 px. A splat that is not finite, not positive definite or worse conditioned than kappa = 1e5 is never
// culled: the per-lane evaluation then decides, exactly as without the cull. Skipping a certain reject changes no
// result.
__device__ __forceinline__ uint32_t reach_mask(const StagedSplat& s, float x0, float y0) {
  if (s.o < 0.99f / 255.0f) return 0u;  // alpha <= o < 1/255 everywhere (a NaN o falls through)
  const float det = s.a * s.c - s.b * s.b;
  if (!(det > 0.0f && s.a > 0.0f)) return 0xFu;
  const float apc = s.a + s.c;
  const float kappa = apc * apc / det;
  if (!(kappa <= 1e5f)) return 0xFu;
  const float L = __logf(255.0f * s.o);
  const float Lm = (fmaxf(L, 0.0f) + 1e-3f) * (1.0f + 1e-6f * kappa);
  const float two_l_det = 2.0f * Lm / det;
  const float rx = __builtin_sqrtf(two_l_det * s.c) * 1.001f + 0.01f;
  const float ry = __builtin_sqrtf(two_l_det * s.a) * 1.001f + 0.01f;
  uint32_t m = 0;
#pragma unroll
  for (uint32_t q = 0; q < 4; ++q) {
    const float xl = x0 + 8.0f * float(q & 1u), xh = xl + 7.0f;
    const float yl = y0 + 8.0f * float(q >> 1), yh = yl + 7.0f;
    const bool disjoint = (s.x - rx > xh) || (s.x + rx < xl) || (s.y - ry > yh) || (s.y + ry < yl);
    if (!disjoint) m |= 1u << q;
  }
  return m;
}

// Workgroup barrier that orders LDS accesses only: it waits for the wave's own LDS operations, not for its
// outstanding global memory operations (unlike __syncthreads, whose fence also drains every pending global store and
// atomic). For loops whose barriers protect LDS buffers while global atomics, which nothing in the workgroup reads
// back, may complete later.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave-uniform 64-bit value held in scalar registers.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return (uint64_t(hi) << 32) | lo;
}

struct Eval {
  float dx, dy, G, oG, alpha;
};

// Evaluates splat s at pixel centre (cx, cy). Returns true when the splat passes every reject (sigma >= 0,
// alpha >= 1/255); then e holds dx, dy, G = exp(-sigma), o G and alpha = min(0.999, o G).
// sigma = 0.5 (a dx dx + c dy dy) + b dx dy is formed as (ha dx) dx + (hc dy) dy + (b dx) dy, which rounds to the
// same fp32 value because halving is exact. Splats with sigma >= 5.55 are rejected before any exponential (their
// alpha is at most e^-5.55 < 1/255 since o <= 1), and most other rejects are settled by the hardware exp2 before
// the fp64 evaluation.
//
// kExactValues = true (forward): every splat that passes is evaluated with the correctly rounded G, so alpha and the
// transmittance chain are exactly those of a plain fp32 evaluation - the stop test T' < 1e-4 depends on them.
// kExactValues = false (backward): the decisions must still be exact (reject or composite, clamped or not), but the
// values only feed gradient terms. G comes from the hardware exp2 (relative error below 3e-7 for sigma < 5.55) and
// the fp64 value is computed only when o G lies within 2^-18 (relative) of 1/255 or of 0.999, where the fast value
// could fall on the other side of a threshold.
constexpr float kBand = 1.0f / 262144.0f;
constexpr float kAlphaMinLo = kAlphaMin * (1.0f - kBand), kAlphaMinHi = kAlphaMin * (1.0f + kBand);
constexpr float kAlphaMaxLo = kAlphaMax * (1.0f - kBand), kAlphaMaxHi = kAlphaMax * (1.0f + kBand);

template <bool kExactValues>
__device__ __forceinline__ bool evaluate(const StagedSplat& s, float cx, float cy, Eval& e) {
  e.dx = cx - s.x;
  e.dy = cy - s.y;
  const float t_a = (s.ha * e.dx) * e.dx;
  const float t_c = (s.hc * e.dy) * e.dy;
  const float t_b = (s.b * e.dx) * e.dy;
  const float sigma = (t_a + t_c) + t_b;
  if (!(sigma >= 0.0f && sigma < kSigmaSkip)) return false;
  const float g_fast = __builtin_amdgcn_exp2f(sigma * -1.44269504088896341f);
  const float og_fast = s.o * g_fast;
  if (kExactValues) {
    if (og_fast < kAlphaMinCertain) return false;
    e.G = exp_rn(-sigma);
  } else {
    if (og_fast < kAlphaMinLo) return false;
    const bool near = og_fast < kAlphaMinHi || (og_fast > kAlphaMaxLo && og_fast < kAlphaMaxHi);
    e.G = near ? exp_rn(-sigma) : g_fast;
  }
  e.oG = s.o * e.G;
  e.alpha = (e.oG < kAlphaMax) ? e.oG : kAlphaMax;
  return !(e.alpha < kAlphaMin);
}

}  // namespace gsr
