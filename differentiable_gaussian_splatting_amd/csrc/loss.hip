// L1 + SSIM training loss and its gradient with respect to the rendered image, for gfx950.
//
// The pages name a fused L1 + SSIM loss and its backward (M3 per-splat backward page: the brush change it ports is a
// per-splat backward "+ fused L1+SSIM loss"), the SSIM kernel's share of the iteration, and its window sizes K = 7
// and 11 (SSIM float4 finding); the formula is the usual one:
//   L = (1 - lam) mean|x - y| + lam (1 - mean S),  S = ((2 mx my + C1)(2 sxy + C2)) / ((mx^2 + my^2 + C1)(sx + sy + C2))
// with mx = G * x, sx = G * x^2 - mx^2, sxy = G * xy - mx my per channel, G * the correlation with the normalised
// 11-tap Gaussian (sigma 1.5) in x and in y over the zero-padded image, C1 = 0.01^2, C2 = 0.03^2, lam = 0.2.
// With f = N / M, N = A B, M = C D (A = 2 mx my + C1, B = 2 sxy + C2, C = mx^2 + my^2 + C1, D = sx + sy + C2),
// holding G * y and G * y^2 fixed:
//   df/dmx = (2 my (B - A) - f 2 mx (D - C)) / M,  df/d(G * x^2) = -f / D,  df/d(G * xy) = 2 A / M,
//   dL/dx(q) = (1 - lam) sign(x - y) / (3 H W) - lam / (3 H W) [G * df/dmx + 2 x G * df/d(G*x^2) + y G * df/d(G*xy)](q)
// (G is symmetric, so its transpose is the same correlation).
//
// One workgroup per 16x16 tile and per image, all in LDS: the tile's pixels need the derivative maps on the tile
// grown by 5 (26 x 26), which need the images on the tile grown by 10 (36 x 36). Per channel: load x and y (zeros
// outside the image), a horizontal then a vertical 11-tap pass of the five products, the map values and their three
// derivatives (zero outside the image), a horizontal and a vertical pass of those, and the gradient. Each tile writes
// its sums of S and |x - y| (fp64) to its own slot; one workgroup adds the slots in order, so the loss is the same on
// every run.
#include <cmath>

#include "gsr_internal.hpp"

namespace gsr {
namespace {

constexpr uint32_t kThreads = 256;
constexpr int kT = 16;              // output tile
constexpr int kR = 5;               // window radius
constexpr int kP = kT + 2 * kR;     // 26: derivative maps
constexpr int kI = kT + 4 * kR;     // 36: images
constexpr float kC1 = 0.01f * 0.01f;
constexpr float kC2 = 0.03f * 0.03f;

struct Taps {
  float g[2 * kR + 1];
};

__device__ __forceinline__ double block_sum(double v, double* s_red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
  if (lane == 0) s_red[w] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0)
    for (uint32_t q = 0; q < kThreads / 64; ++q) t += s_red[q];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kThreads) void k_l1_ssim(Taps taps, uint32_t width, uint32_t height, uint32_t tiles_x,
                                                      float lam, float inv_n, const float4* __restrict__ out_rgba,
                                                      const float* __restrict__ target, float4* __restrict__ v_out,
                                                      double* __restrict__ part) {
  __shared__ float s_x[kI][kI], s_y[kI][kI];
  __shared__ float s_h[5][kI][kP];   // horizontal sums of x, y, xx, yy, xy
  __shared__ float s_d[3][kP][kP];   // df/dmx, df/dSxx, df/dSxy (0 outside the image)
  __shared__ float s_h2[3][kP][kT];  // their horizontal sums
  __shared__ double s_red[kThreads / 64];
  const uint32_t tid = threadIdx.x;
  const int tx0 = int(blockIdx.x % tiles_x) * kT, ty0 = int(blockIdx.x / tiles_x) * kT;
  const int W = int(width), H = int(height);
  const int ox = tid % kT, oy = tid / kT;  // this thread's output pixel in the tile
  const int px = tx0 + ox, py = ty0 + oy;
  const bool inside = px < W && py < H;
  const size_t pix = inside ? size_t(py) * W + px : 0;
  float g_out[3];
  double ssim_sum = 0.0, l1_sum = 0.0;

  for (int c = 0; c < 3; ++c) {
    // images on the tile grown by 10, zero outside
    for (int e = tid; e < kI * kI; e += kThreads) {
      const int r = e / kI, q = e % kI;
      const int gx = tx0 - 2 * kR + q, gy = ty0 - 2 * kR + r;
      float xv = 0.0f, yv = 0.0f;
      if (gx >= 0 && gy >= 0 && gx < W && gy < H) {
        const size_t p = size_t(gy) * W + gx;
        xv = reinterpret_cast<const float*>(out_rgba)[4 * p + c];
        yv = target[3 * p + c];
      }
      s_x[r][q] = xv;
      s_y[r][q] = yv;
    }
    __syncthreads();
    // horizontal pass: rows 0..35, columns of the 26-wide region
    for (int e = tid; e < kI * kP; e += kThreads) {
      const int r = e / kP, q = e % kP;
      float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f, a4 = 0.0f;
#pragma unroll
      for (int t = 0; t < 2 * kR + 1; ++t) {
        const float xv = s_x[r][q + t], yv = s_y[r][q + t], g = taps.g[t];
        a0 = fmaf(g, xv, a0);
        a1 = fmaf(g, yv, a1);
        a2 = fmaf(g, xv * xv, a2);
        a3 = fmaf(g, yv * yv, a3);
        a4 = fmaf(g, xv * yv, a4);
      }
      s_h[0][r][q] = a0;
      s_h[1][r][q] = a1;
      s_h[2][r][q] = a2;
      s_h[3][r][q] = a3;
      s_h[4][r][q] = a4;
    }
    __syncthreads();
    // vertical pass on the 26 x 26 region: the map and its three derivatives
    for (int e = tid; e < kP * kP; e += kThreads) {
      const int r = e / kP, q = e % kP;
      const int gx = tx0 - kR + q, gy = ty0 - kR + r;
      float d0 = 0.0f, d1 = 0.0f, d2 = 0.0f, S = 0.0f;
      if (gx >= 0 && gy >= 0 && gx < W && gy < H) {
        float mx = 0.0f, my = 0.0f, xx = 0.0f, yy = 0.0f, xy = 0.0f;
#pragma unroll
        for (int t = 0; t < 2 * kR + 1; ++t) {
          const float g = taps.g[t];
          mx = fmaf(g, s_h[0][r + t][q], mx);
          my = fmaf(g, s_h[1][r + t][q], my);
          xx = fmaf(g, s_h[2][r + t][q], xx);
          yy = fmaf(g, s_h[3][r + t][q], yy);
          xy = fmaf(g, s_h[4][r + t][q], xy);
        }
        const float sx = xx - mx * mx, sy = yy - my * my, sxy = xy - mx * my;
        const float A = 2.0f * mx * my + kC1, B = 2.0f * sxy + kC2;
        const float C = mx * mx + my * my + kC1, D = sx + sy + kC2;
        const float iM = 1.0f / (C * D);
        S = (A * B) * iM;
        d0 = (2.0f * my * (B - A) - S * (2.0f * mx) * (D - C)) * iM;
        d1 = -S / D;
        d2 = 2.0f * A * iM;
      }
      s_d[0][r][q] = d0;
      s_d[1][r][q] = d1;
      s_d[2][r][q] = d2;
      if (r >= kR && r < kR + kT && q >= kR && q < kR + kT) ssim_sum += double(S);  // the tile's own pixels
    }
    __syncthreads();
    // horizontal pass of the derivative maps: rows 0..25, the tile's 16 columns
    for (int e = tid; e < kP * kT; e += kThreads) {
      const int r = e / kT, q = e % kT;
      float b0 = 0.0f, b1 = 0.0f, b2 = 0.0f;
#pragma unroll
      for (int t = 0; t < 2 * kR + 1; ++t) {
        const float g = taps.g[t];
        b0 = fmaf(g, s_d[0][r][q + t], b0);
        b1 = fmaf(g, s_d[1][r][q + t], b1);
        b2 = fmaf(g, s_d[2][r][q + t], b2);
      }
      s_h2[0][r][q] = b0;
      s_h2[1][r][q] = b1;
      s_h2[2][r][q] = b2;
    }
    __syncthreads();
    // vertical pass at this thread's pixel, and the gradient
    {
      float b0 = 0.0f, b1 = 0.0f, b2 = 0.0f;
#pragma unroll
      for (int t = 0; t < 2 * kR + 1; ++t) {
        const float g = taps.g[t];
        b0 = fmaf(g, s_h2[0][oy + t][ox], b0);
        b1 = fmaf(g, s_h2[1][oy + t][ox], b1);
        b2 = fmaf(g, s_h2[2][oy + t][ox], b2);
      }
      const float xv = s_x[oy + 2 * kR][ox + 2 * kR], yv = s_y[oy + 2 * kR][ox + 2 * kR];
      const float dssim = fmaf(yv, b2, fmaf(2.0f * xv, b1, b0));
      const float diff = xv - yv;
      const float sgn = diff > 0.0f ? 1.0f : (diff < 0.0f ? -1.0f : 0.0f);
      g_out[c] = ((1.0f - lam) * sgn - lam * dssim) * inv_n;
      if (inside) l1_sum += double(fabsf(diff));
    }
    __syncthreads();  // the next channel overwrites the LDS images
  }
  if (inside) v_out[pix] = make_float4(g_out[0], g_out[1], g_out[2], 0.0f);
  const double s_tot = block_sum(ssim_sum, s_red);
  const double l_tot = block_sum(l1_sum, s_red);
  if (tid == 0) {
    part[2 * size_t(blockIdx.x)] = s_tot;
    part[2 * size_t(blockIdx.x) + 1] = l_tot;
  }
}

// out[0] = loss, out[1] = mean |x - y|, out[2] = mean S: the tiles' sums added in tile order by one workgroup.
__global__ __launch_bounds__(kThreads) void k_l1_ssim_total(const double* __restrict__ part, uint32_t num_tiles,
                                                            double inv_n, float lam, float* __restrict__ out) {
  __shared__ double s_red[kThreads / 64];
  // fixed assignment of tiles to threads and a fixed reduction tree: the same sum on every run
  double s = 0.0, l = 0.0;
  for (uint32_t t = threadIdx.x; t < num_tiles; t += kThreads) {
    s += part[2 * size_t(t)];
    l += part[2 * size_t(t) + 1];
  }
  const double S = block_sum(s, s_red);
  const double L1 = block_sum(l, s_red);
  if (threadIdx.x == 0) {
    const double l1m = L1 * inv_n, sm = S * inv_n;
    out[0] = float((1.0 - double(lam)) * l1m + double(lam) * (1.0 - sm));
    out[1] = float(l1m);
    out[2] = float(sm);
  }
}

Taps make_taps() {
  Taps t;
  double g[2 * kR + 1], sum = 0.0;
  for (int i = 0; i <= 2 * kR; ++i) {
    const double d = i - kR;
    g[i] = std::exp(-d * d / (2.0 * 1.5 * 1.5));
    sum += g[i];
  }
  for (int i = 0; i <= 2 * kR; ++i) t.g[i] = float(g[i] / sum);
  return t;
}

}  // namespace
}  // namespace gsr

using namespace gsr;

extern "C" gsr_status gsr_loss_l1_ssim(gsr_ctx* ctx, void* stream, uint32_t width, uint32_t height,
                                       const float* out_rgba, const float* target, float* v_out, float* loss) {
  if (!ctx) return GSR_EINVAL;
  if (width == 0 || height == 0) return fail(ctx, GSR_EINVAL, "gsr_loss_l1_ssim: empty image");
  if (!out_rgba || !target || !v_out || !loss) return fail(ctx, GSR_EINVAL, "gsr_loss_l1_ssim: null pointer");
  if (reinterpret_cast<uintptr_t>(out_rgba) % 16 || reinterpret_cast<uintptr_t>(v_out) % 16)
    return fail(ctx, GSR_EINVAL, "gsr_loss_l1_ssim: out_rgba and v_out must be 16-byte aligned");
  const uint64_t tiles_x = (width + kT - 1) / kT, tiles_y = (height + kT - 1) / kT;
  const uint64_t num_tiles = tiles_x * tiles_y;
  if (num_tiles >= (uint64_t(1) << 31)) return fail(ctx, GSR_EINVAL, "gsr_loss_l1_ssim: image too large");
  gsr_status st = enter(ctx);
  if (st) return st;
  if ((st = grow(ctx, ctx->arena.loss_part, size_t(num_tiles) * 16))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* part = static_cast<double*>(ctx->arena.loss_part.ptr);
  const double n = 3.0 * double(width) * double(height);
  hipLaunchKernelGGL(k_l1_ssim, dim3(uint32_t(num_tiles)), dim3(kThreads), 0, s, make_taps(), width, height,
                     uint32_t(tiles_x), 0.2f, float(1.0 / n), reinterpret_cast<const float4*>(out_rgba), target,
                     reinterpret_cast<float4*>(v_out), part);
  hipLaunchKernelGGL(k_l1_ssim_total, dim3(1), dim3(kThreads), 0, s, part, uint32_t(num_tiles), 1.0 / n, 0.2f, loss);
  return check_launch(ctx, "gsr_loss_l1_ssim");
}
