// Device helpers shared by the forward and backward raster kernels. Both kernels must take exactly the same
// decisions for every (pixel, splat), so the evaluation below is the only place sigma, exp(-sigma) and alpha are
// computed. The file is compiled without floating-point contraction: every float expression rounds once per
// operation, in the order written, which makes each decision equal to a plain fp32 evaluation of the definition.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gsr {

// Method constants (fp32). [A.9 f16 forward page, listing: alpha clamp 0.999; W1 warp sparse skip + exp-skip page,
// summary: alpha < 1/255 reject and the sigma >= 5.55 skip, which the per-splat bound lr below contains]
constexpr float kAlphaMax = 0.999f;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kTStop = 1e-4f;

// 2^(j/32) for j = 0..31 as pairs (hi, lo) of doubles: hi is the value rounded to double, lo the rounded
// remainder, so hi + lo carries it to about 2^-106.
constexpr double kExp2Tab[64] = {
    0x1.0000000000000p+0, 0x0.0p+0,  // j = 0
    0x1.059b0d3158574p+0, 0x1.d73e2a475b465p-55,  // j = 1
    0x1.0b5586cf9890fp+0, 0x1.8a62e4adc610bp-54,  // j = 2
    0x1.11301d0125b51p+0, -0x1.6c51039449b3ap-54,  // j = 3
    0x1.172b83c7d517bp+0, -0x1.19041b9d78a76p-55,  // j = 4
    0x1.1d4873168b9aap+0, 0x1.e016e00a2643cp-54,  // j = 5
    0x1.2387a6e756238p+0, 0x1.9b07eb6c70573p-54,  // j = 6
    0x1.29e9df51fdee1p+0, 0x1.612e8afad1255p-55,  // j = 7
    0x1.306fe0a31b715p+0, 0x1.6f46ad23182e4p-55,  // j = 8
    0x1.371a7373aa9cbp+0, -0x1.63aeabf42eae2p-54,  // j = 9
    0x1.3dea64c123422p+0, 0x1.ada0911f09ebcp-55,  // j = 10
    0x1.44e086061892dp+0, 0x1.89b7a04ef80d0p-59,  // j = 11
    0x1.4bfdad5362a27p+0, 0x1.d4397afec42e2p-56,  // j = 12
    0x1.5342b569d4f82p+0, -0x1.07abe1db13cadp-55,  // j = 13
    0x1.5ab07dd485429p+0, 0x1.6324c054647adp-54,  // j = 14
    0x1.6247eb03a5585p+0, -0x1.383c17e40b497p-54,  // j = 15
    0x1.6a09e667f3bcdp+0, -0x1.bdd3413b26456p-54,  // j = 16
    0x1.71f75e8ec5f74p+0, -0x1.16e4786887a99p-55,  // j = 17
    0x1.7a11473eb0187p+0, -0x1.41577ee04992fp-55,  // j = 18
    0x1.82589994cce13p+0, -0x1.d4c1dd41532d8p-54,  // j = 19
    0x1.8ace5422aa0dbp+0, 0x1.6e9f156864b27p-54,  // j = 20
    0x1.93737b0cdc5e5p+0, -0x1.75fc781b57ebcp-57,  // j = 21
    0x1.9c49182a3f090p+0, 0x1.c7c46b071f2bep-56,  // j = 22
    0x1.a5503b23e255dp+0, -0x1.d2f6edb8d41e1p-54,  // j = 23
    0x1.ae89f995ad3adp+0, 0x1.7a1cd345dcc81p-54,  // j = 24
    0x1.b7f76f2fb5e47p+0, -0x1.5584f7e54ac3bp-56,  // j = 25
    0x1.c199bdd85529cp+0, 0x1.11065895048ddp-55,  // j = 26
    0x1.cb720dcef9069p+0, 0x1.503cbd1e949dbp-56,  // j = 27
    0x1.d5818dcfba487p+0, 0x1.2ed02d75b3707p-55,  // j = 28
    0x1.dfc97337b9b5fp+0, -0x1.1a5cd4f184b5cp-54,  // j = 29
    0x1.ea4afa2a490dap+0, -0x1.e9c23179c2893p-54,  // j = 30
    0x1.f50765b6e4540p+0, 0x1.9d3e12dd8a18bp-54,  // j = 31
};

// e^x rounded to fp32, for |x| below 80, with `tab` holding kExp2Tab (an LDS copy on the device). The method is
// P. T. P. Tang's table-driven exponential (ACM Transactions on Mathematical Software 15(2), 1989): reduction
// x = k ln2/32 + r with |r| <= ln2/64 (ln2/32 split into a 32-bit head, exact in k * head for |k| < 2^21, and a
// tail), e^r - 1 by its Taylor series to degree 6 (truncation below 4e-18), then
// 2^(k/32) e^r = 2^floor(k/32) (hi + (hi (e^r - 1) + lo)) with one rounding to double and one to fp32. The double
// is within about 1.2e-16 (relative) of e^x; over every float x in [-5.55, 0] (the arguments the raster kernels
// evaluate) the fp32 result equals the correctly rounded e^x, which a host test checks exhaustively.
__host__ __device__ __forceinline__ float exp_rn(float x, const double* tab) {
  const double xd = double(x);
  const double k = rint(xd * 46.166241308446828384);  // 32 / ln 2
  double r = fma(-k, 0x1.62e42fee00000p-6, xd);
  r = fma(-k, 0x1.a39ef35793c76p-38, r);
  const double r2 = r * r;
  double q = fma(r, 1.0 / 720.0, 1.0 / 120.0);
  q = fma(q, r, 1.0 / 24.0);
  q = fma(q, r, 1.0 / 6.0);
  q = fma(q, r, 0.5);
  q = fma(q, r2, r);  // e^r - 1
  const int ki = int(k);
  const double hi = tab[2 * (ki & 31)], lo = tab[2 * (ki & 31) + 1];
  return float(ldexp(hi + fma(hi, q, lo), ki >> 5));
}

// The forward's form of exp_rn: e^-s for s in [0, 5.70] with `tab` holding kExpTabN pairs (hi, lo), entry k being
// 2^(-k/32): kExp2Tab's pair for the residue of -k scaled by 2^floor(-k/32), which is exact. With k = round(32 s /
// ln 2) the table entry already carries the power of two, so no ldexp or index masking follows the series; k is
// found by one rounding of s 32 / ln 2 (adding 1.5 2^52 leaves it in the low word, so no conversion follows
// either), where exp_rn rounds the product first, which can pick the neighbouring k at a tie: either residue lies
// in the series' range. Both functions are correctly rounded on every argument, so they agree bit for bit - the
// host test checks both exhaustively. The caller keeps s <= kSigmaCap (the kernels evaluate s <= lr <= kSigmaCap,
// see StagedSplat), which keeps k below kExpTabN: the table index needs no clamp.
constexpr uint32_t kExpTabN = 264;
constexpr float kSigmaCap = 5.70f;  // round(5.70 * 32 / ln 2) = 263 = kExpTabN - 1

__host__ __device__ __forceinline__ void exp_neg_entry(uint32_t kp, double* hi_lo) {
  const int k = -int(kp);
  hi_lo[0] = ldexp(kExp2Tab[2 * (k & 31)], k >> 5);
  hi_lo[1] = ldexp(kExp2Tab[2 * (k & 31) + 1], k >> 5);
}

// fma(a, b, c) for a wave-uniform constant c, taken from scalar registers: the compiler's own choice, the tied
// v_fmac form, would copy the constant into the destination register before every use.
__host__ __device__ __forceinline__ double fma_uniform_c(double a, double b, double c) {
#if defined(__HIP_DEVICE_COMPILE__)
  double d;
  asm("v_fma_f64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "s"(c));
  return d;
#else
  return fma(a, b, c);
#endif
}

__host__ __device__ __forceinline__ float exp_neg_rn(float s, const double* tab) {
  const double sd = double(s);
  // k = the integer nearest sd 32 / ln 2, by adding 1.5 2^52 (one rounding to an integer, left in the low word)
  const double t = fma(sd, 46.166241308446828384, 0x1.8p52);
  const double k = t - 0x1.8p52;
  uint64_t tbits;
  __builtin_memcpy(&tbits, &t, sizeof tbits);
  double r = fma(k, 0x1.62e42fee00000p-6, -sd);
  r = fma(k, 0x1.a39ef35793c76p-38, r);
  const double r2 = r * r;
  double q = fma_uniform_c(r, 1.0 / 720.0, 1.0 / 120.0);
  q = fma_uniform_c(q, r, 1.0 / 24.0);
  q = fma_uniform_c(q, r, 1.0 / 6.0);
  q = fma(q, r, 0.5);
  q = fma(q, r2, r);  // e^r - 1
  const uint32_t ki = uint32_t(tbits);  // k, below kExpTabN for 0 <= s <= kSigmaCap
  const double hi = tab[2 * ki], lo = tab[2 * ki + 1];
  return float(hi + fma(hi, q, lo));
}

// One splat as staged in LDS for a batch: 48 bytes, read by every lane of a wavefront at the same address. The
// conic is kept as a / 2 and c / 2 (what sigma uses) beside b and b / 2; a and c are ha + ha and hc + hc, exactly.
// lr bounds sigma: alpha <= o e^-sigma < 1/255 wherever sigma > lr, so those evaluations are certain rejects.
// lr is ln(255 o) from the fast log, raised by 2^-16 relative and 2^-16 absolute (far more than the log's and the
// product's rounding), then clamped to [0, kSigmaCap]. For 0 <= o <= 1 (every splat the binning keeps) it lies in
// [0, 5.55): the clamp at 0 only lets sigma = 0 through where o < 1/255, which alpha then rejects, and the one at
// kSigmaCap never binds; the bound contains the sigma >= 5.55 skip. A NaN log (o < 0 or NaN, never binned) gives
// kSigmaCap, and the exact evaluation decides.
struct alignas(16) StagedSplat {
  float x, y, ha, b;  // mean, a / 2, b
  float hc, o, r, g;  // c / 2, opacity, red, green
  float bl, lr, hb;   // blue, the sigma bound, b / 2
  uint32_t idx;       // splat index, or 0xFFFFFFFF for a slot that must not contribute
};

__device__ __forceinline__ StagedSplat stage_splat(const float* __restrict__ splats, uint32_t idx, uint32_t n) {
  StagedSplat s;
  if (idx < n) {
    const float* p = splats + size_t(idx) * 9;
    s.x = p[0];
    s.y = p[1];
    s.ha = 0.5f * p[2];  // exact: scaling by a power of two
    s.b = p[3];
    s.hb = 0.5f * s.b;
    s.hc = 0.5f * p[4];
    s.r = p[5];
    s.g = p[6];
    s.bl = p[7];
    s.o = p[8];
    const float L = __logf(255.0f * s.o);
    const float lr = L == L ? (L + __builtin_fabsf(L) * (1.0f / 65536.0f)) + (1.0f / 65536.0f) : kSigmaCap;
    s.lr = __builtin_fminf(__builtin_fmaxf(lr, 0.0f), kSigmaCap);
    s.idx = idx;
  } else {
    // o = 0 makes every evaluation a reject
    s.x = s.y = s.ha = s.b = s.hb = s.hc = s.r = s.g = s.bl = s.o = 0.0f;
    s.lr = 0.0f;
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
// alpha <= o exp(-sigma) reaches 1/255 only where sigma <= L = ln(255 o), an ellipse. A block is dropped when a
// separating axis shows the ellipse misses the rectangle spanned by the block's pixel centres: the x and y axes
// (the ellipse's bounding box, half-widths sqrt(2 L c / det) and sqrt(2 L a / det)) and the two diagonals (half-
// ranges of x + y and x - y: sqrt(2 L (a + c -+ 2 b) / det)), an octagon around the ellipse that also drops the
// blocks beside a thin tilted splat which its bounding box still meets. Evaluated in fp32 and widened for every
// rounding involved: the fp32 sigma of the per-lane test (relative error below 4.5 eps kappa, where
// kappa = (a + c)^2 / det bounds the conic's condition number), det here and a + c -+ 2 b (relative errors below
// 2 eps kappa and eps kappa / 2 + eps, as a + c -+ 2 b >= 2 det / (a + c)), the fast log (absolute error below 1e-5),
// the reciprocal, square roots and products (a few ulp): L gets +1e-3 and the factor 1 + 1e-6 kappa, the half-widths
// x1.001 + 0.01 px. A splat that is not finite, not positive definite or worse conditioned than kappa = 1e5 is never
// culled: the per-lane evaluation then decides, exactly as without the cull. Skipping a certain reject changes no
// result.
__device__ __forceinline__ uint32_t reach_mask(const StagedSplat& s, float x0, float y0) {
  if (s.o < 0.99f / 255.0f) return 0u;  // alpha <= o < 1/255 everywhere (a NaN o falls through)
  const float a = s.ha + s.ha, c = s.hc + s.hc;
  const float det = a * c - s.b * s.b;
  if (!(det > 0.0f && a > 0.0f)) return 0xFu;
  const float apc = a + c, b2 = s.b + s.b;
  const float inv_det = __builtin_amdgcn_rcpf(det);
  const float kappa = apc * apc * inv_det;
  if (!(kappa <= 1e5f)) return 0xFu;
  const float L = s.lr;  // at least ln(255 o)
  const float Lm = (fmaxf(L, 0.0f) + 1e-3f) * (1.0f + 1e-6f * kappa);
  const float two_l_det = 2.0f * Lm * inv_det;
  // Blocks q = 0..3: columns q & 1 and rows q >> 1 of the 2 x 2 grid; each axis test clears the blocks it separates.
  // Over a block's pixel centres x - x0 spans [0, 7] or [8, 15] (likewise y - y0), (x + y) - (x0 + y0) spans [0, 14],
  // [8, 22] (q = 1, 2) or [16, 30], and (x - y) - (x0 - y0) spans [-7, 7] (q = 0, 3), [1, 15] or [-15, -1].
  uint32_t m = 0xFu;
  {
    const float r = __builtin_amdgcn_sqrtf(two_l_det * c) * 1.001f + 0.01f;
    const float lo = s.x - r, hi = s.x + r;
    if (lo > x0 + 7.0f || hi < x0) m &= ~0x5u;
    if (lo > x0 + 15.0f || hi < x0 + 8.0f) m &= ~0xAu;
  }
  {
    const float r = __builtin_amdgcn_sqrtf(two_l_det * a) * 1.001f + 0.01f;
    const float lo = s.y - r, hi = s.y + r;
    if (lo > y0 + 7.0f || hi < y0) m &= ~0x3u;
    if (lo > y0 + 15.0f || hi < y0 + 8.0f) m &= ~0xCu;
  }
  {
    const float r = __builtin_amdgcn_sqrtf(two_l_det * (apc - b2)) * 1.001f + 0.01f;  // x + y
    const float v = s.x + s.y, o = x0 + y0;
    const float lo = v - r, hi = v + r;
    if (lo > o + 14.0f || hi < o) m &= ~0x1u;
    if (lo > o + 22.0f || hi < o + 8.0f) m &= ~0x6u;
    if (lo > o + 30.0f || hi < o + 16.0f) m &= ~0x8u;
  }
  {
    const float r = __builtin_amdgcn_sqrtf(two_l_det * (apc + b2)) * 1.001f + 0.01f;  // x - y
    const float v = s.x - s.y, o = x0 - y0;
    const float lo = v - r, hi = v + r;
    if (lo > o + 7.0f || hi < o - 7.0f) m &= ~0x9u;
    if (lo > o + 15.0f || hi < o + 1.0f) m &= ~0x2u;
    if (lo > o - 1.0f || hi < o - 15.0f) m &= ~0x4u;
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

// Copies kExp2Tab into the workgroup's LDS table (threads 0..63); a barrier must follow before its first use.
__device__ __forceinline__ void load_exp_table(double* s_tab) {
  if (threadIdx.x < 64) s_tab[threadIdx.x] = kExp2Tab[threadIdx.x];
}

// Fills the workgroup's LDS table of exp_neg_rn (kExpTabN pairs); a barrier must follow before its first use.
__device__ __forceinline__ void load_exp_neg_table(double* s_tab) {
  for (uint32_t k = threadIdx.x; k < kExpTabN; k += blockDim.x) exp_neg_entry(k, s_tab + 2 * k);
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
// same fp32 value because halving is exact. Evaluations with sigma > lr (the splat's bound, at least ln(255 o)) are
// rejected before any exponential: their alpha is below 1/255 by a margin no rounding can close. This contains the
// pages' sigma >= 5.55 skip (lr < 5.55 for o <= 1) and is exact for 0 <= o <= 1. Both ends are tested at once on
// the bit patterns: for a, c > 0 (binned splats) the fp32 sigma is +0 or more, never -0 (the two squares are +0 or
// positive and +0 + -0 = +0), and lr lies in [+0, kSigmaCap], where unsigned order is float order; a negative or NaN
// sigma has a larger pattern than any such lr.
//
// kExactValues = true (forward, `tab` = the exp_neg_rn table): every splat that passes is evaluated with the correctly
// rounded G, so alpha and the transmittance chain are exactly those of a plain fp32 evaluation - the stop test
// T' < 1e-4 depends on them.
// kExactValues = false (backward, `tab` = kExp2Tab): the decisions must still be exact (reject or composite, clamped or not), but the
// values only feed gradient terms. G comes from the hardware exp2 (relative error below 5.2e-7 for sigma < 5.55) and
// the fp64 value is computed only when o G lies within 2^-18 (relative) of 1/255 or of 0.999, where the fast value
// could fall on the other side of a threshold.
constexpr float kBand = 1.0f / 262144.0f;
constexpr float kAlphaMinLo = kAlphaMin * (1.0f - kBand), kAlphaMinHi = kAlphaMin * (1.0f + kBand);
constexpr float kAlphaMaxLo = kAlphaMax * (1.0f - kBand), kAlphaMaxHi = kAlphaMax * (1.0f + kBand);

// kClampBand = false (the forward's fast form): only the reject threshold gets the exact value. A fast o G on the
// wrong side of 0.999 changes alpha by less than the fast value's own error (the clamp's choice is between o G and
// 0.999, which then differ by less than that), and the forward's alpha only feeds T; the backward decides the clamp
// exactly, since its gradient terms differ in kind on either side.
template <bool kExactValues, bool kClampBand = true>
__device__ __forceinline__ bool evaluate(const StagedSplat& s, float cx, float cy, Eval& e, const double* tab) {
  e.dx = cx - s.x;
  e.dy = cy - s.y;
  const float t_a = (s.ha * e.dx) * e.dx;
  const float t_c = (s.hc * e.dy) * e.dy;
  const float t_b = (s.b * e.dx) * e.dy;
  const float sigma = (t_a + t_c) + t_b;
  const bool in_range = __float_as_uint(sigma) <= __float_as_uint(s.lr);  // not sigma < 0, NaN, or above lr
  if constexpr (kExactValues) {
    if (!in_range) return false;
    e.G = exp_neg_rn(sigma, tab);
    e.oG = s.o * e.G;
  } else {
    // Without branches but for the rare wave in which some lane lies near a threshold: there every lane takes the
    // exact value through exp_rn (lanes not near keep the fast one; for the others exp_rn's result is unused, and
    // its table index is masked, so any argument reads in bounds). A fast o G below kAlphaMinLo is a certain reject
    // and gives alpha < 1/255 as it stands.
    float g = __builtin_amdgcn_exp2f(sigma * -1.44269504088896341f);
    float og = s.o * g;
    // (bitwise operators: no short-circuit branches, the masks combine in scalar registers)
    const bool near_max = kClampBand && ((og > kAlphaMaxLo) & (og < kAlphaMaxHi));
    const bool near = in_range & (og >= kAlphaMinLo) & ((og < kAlphaMinHi) | near_max);
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
      const float g_exact = exp_rn(-sigma, tab);
      g = near ? g_exact : g;
      og = near ? s.o * g_exact : og;
    }
    e.G = g;
    e.oG = og;
  }
  if constexpr (kExactValues) {
    e.alpha = (e.oG < kAlphaMax) ? e.oG : kAlphaMax;
  } else {
    // the same value as the select (o G is a product of finite values, never NaN), in one instruction: the
    // compiler's min would first canonicalise its operand; the constant is the instruction's literal (in a register
    // operand it is materialised on every evaluation)
    static_assert(__builtin_bit_cast(uint32_t, kAlphaMax) == 0x3f7fbe77u, "the literal below is 0.999f");
    asm("v_min_f32 %0, 0x3f7fbe77, %1" : "=v"(e.alpha) : "v"(e.oG));
  }
  return in_range & !(e.alpha < kAlphaMin);
}

}  // namespace gsr
