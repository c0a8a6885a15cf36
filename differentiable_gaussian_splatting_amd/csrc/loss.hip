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
// Two passes over 16x16 tiles (see k_ssim_maps and k_ssim_grad), with every window sum in LDS; each of the chip's
// eight dies takes one band of tiles (band_tile), so that neighbouring tiles read their shared halos through the
// same L2. Each tile of the first
// pass writes its sums of S and |x - y| (fp64) to its own slot; the second pass's first workgroup adds the slots in
// order, so the loss is the same on every run.
#include <cmath>

#include "gsr_internal.hpp"

namespace gsr {
namespace {

constexpr uint32_t kThreads = 256;
constexpr int kT = 16;              // output tile
constexpr int kR = 5;               // window radius
constexpr int kP = kT + 2 * kR;     // 26: the tile grown by the window radius
constexpr int kLoads = (kP * kP + 255) / 256;  // positions of the 26 x 26 region per thread (256 threads)
constexpr float kC1 = 0.01f * 0.01f;
constexpr float kC2 = 0.03f * 0.03f;

struct Taps {
  float g[2 * kR + 1];
};

// Tile of workgroup b: workgroups go to the eight dies (XCDs) in turn, b to die b % 8, so die x takes the tiles of
// one contiguous band [x band, (x + 1) band) of the image in raster order, and the halos that neighbouring tiles
// share are read through that die's L2. Workgroups past the last tile return.
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t band_tile(uint32_t num_tiles) {
  const uint32_t band = (num_tiles + kXcds - 1) / kXcds;
  return (blockIdx.x % kXcds) * band + blockIdx.x / kXcds;
}

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

// Pass 1 (k_ssim_maps), per 16x16 tile: both images on the tile grown by 5 (26 x 26, all channels, zeros outside),
// a horizontal 11-tap pass of the five products on 26 rows x the tile's 16 columns, a vertical pass at the tile's
// pixels, then S and its three derivatives there, written to nine planes [map][channel][H][W]; the tile's sums of S
// and |x - y| go to its slot. Pass 2 (k_ssim_grad), per tile: the nine planes on the tile grown by 5, a horizontal
// and a vertical pass, and the gradient at the tile's pixels. Splitting at the derivative maps costs their 9 x 4 B
// per pixel of traffic but halves the recomputed halo (a fused pass needs the images on the tile grown by 10).
__global__ __launch_bounds__(kThreads) void k_ssim_maps(Taps taps, uint32_t width, uint32_t height, uint32_t tiles_x,
                                                        uint32_t num_tiles,
                                                        const float4* __restrict__ out_rgba,
                                                        const float* __restrict__ target, float* __restrict__ maps,
                                                        double* __restrict__ part) {
  __shared__ float s_x[3][kP][kP], s_y[3][kP][kP];
  __shared__ float s_h[5][kP][kT];
  __shared__ double s_red[kThreads / 64];
  const int tid = int(threadIdx.x);
  const uint32_t tile = band_tile(num_tiles);
  if (tile >= num_tiles) return;
  const int tx0 = int(tile % tiles_x) * kT, ty0 = int(tile / tiles_x) * kT;
  const int W = int(width), H = int(height);
  const size_t plane = size_t(W) * H;
  {
    // every load of the thread's (at most kLoads) positions is issued before the first store to LDS
    float4 xv[kLoads];
    float yv[kLoads][3];
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int e = tid + it * int(kThreads);
      const int r = e / kP, q = e % kP;
      const int gx = tx0 - kR + q, gy = ty0 - kR + r;
      xv[it] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      yv[it][0] = yv[it][1] = yv[it][2] = 0.0f;
      if (e < kP * kP && gx >= 0 && gy >= 0 && gx < W && gy < H) {
        const size_t p = size_t(gy) * W + gx;
        xv[it] = out_rgba[p];
        yv[it][0] = target[3 * p];
        yv[it][1] = target[3 * p + 1];
        yv[it][2] = target[3 * p + 2];
      }
    }
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int e = tid + it * int(kThreads);
      if (e >= kP * kP) break;
      const int r = e / kP, q = e % kP;
      s_x[0][r][q] = xv[it].x;
      s_x[1][r][q] = xv[it].y;
      s_x[2][r][q] = xv[it].z;
      s_y[0][r][q] = yv[it][0];
      s_y[1][r][q] = yv[it][1];
      s_y[2][r][q] = yv[it][2];
    }
  }
  __syncthreads();
  const int ox = tid % kT, oy = tid / kT;
  const int px = tx0 + ox, py = ty0 + oy;
  const bool inside = px < W && py < H;
  double ssim_sum = 0.0, l1_sum = 0.0;
  for (int c = 0; c < 3; ++c) {
    // horizontal: rows 0..25, the tile's 16 columns; a thread takes two neighbouring columns and slides the window
    // over the 12 values they share (208 threads, one pass)
    if (tid < kP * (kT / 2)) {
      const int r = tid % kP, q0 = 2 * (tid / kP);
      float a[5][2];
#pragma unroll
      for (int o = 0; o < 2; ++o) a[0][o] = a[1][o] = a[2][o] = a[3][o] = a[4][o] = 0.0f;
#pragma unroll
      for (int j = 0; j <= 2 * kR + 1; ++j) {
        const float xv = s_x[c][r][q0 + j], yv = s_y[c][r][q0 + j];
        const float xx = xv * xv, yy = yv * yv, xy = xv * yv;
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          const int t = j - o;
          if (t >= 0 && t <= 2 * kR) {
            const float g = taps.g[t];
            a[0][o] = fmaf(g, xv, a[0][o]);
            a[1][o] = fmaf(g, yv, a[1][o]);
            a[2][o] = fmaf(g, xx, a[2][o]);
            a[3][o] = fmaf(g, yy, a[3][o]);
            a[4][o] = fmaf(g, xy, a[4][o]);
          }
        }
      }
#pragma unroll
      for (int o = 0; o < 2; ++o)
#pragma unroll
        for (int k = 0; k < 5; ++k) s_h[k][r][q0 + o] = a[k][o];
    }
    __syncthreads();
    float mx = 0.0f, my = 0.0f, xx = 0.0f, yy = 0.0f, xy = 0.0f;
#pragma unroll
    for (int t = 0; t <= 2 * kR; ++t) {
      const float g = taps.g[t];
      mx = fmaf(g, s_h[0][oy + t][ox], mx);
      my = fmaf(g, s_h[1][oy + t][ox], my);
      xx = fmaf(g, s_h[2][oy + t][ox], xx);
      yy = fmaf(g, s_h[3][oy + t][ox], yy);
      xy = fmaf(g, s_h[4][oy + t][ox], xy);
    }
    __syncthreads();  // the next channel overwrites s_h
    if (inside) {
      const float sx = xx - mx * mx, sy = yy - my * my, sxy = xy - mx * my;
      const float A = 2.0f * mx * my + kC1, B = 2.0f * sxy + kC2;
      const float C = mx * mx + my * my + kC1, D = sx + sy + kC2;
      const float iM = 1.0f / (C * D);
      const float S = (A * B) * iM;
      const size_t p = size_t(py) * W + px;
      maps[(0 * 3 + c) * plane + p] = (2.0f * my * (B - A) - S * (2.0f * mx) * (D - C)) * iM;
      maps[(1 * 3 + c) * plane + p] = -S / D;
      maps[(2 * 3 + c) * plane + p] = 2.0f * A * iM;
      ssim_sum += double(S);
      l1_sum += double(fabsf(s_x[c][oy + kR][ox + kR] - s_y[c][oy + kR][ox + kR]));
    }
  }
  const double s_tot = block_sum(ssim_sum, s_red);
  const double l_tot = block_sum(l1_sum, s_red);
  if (tid == 0) {
    part[2 * size_t(tile)] = s_tot;
    part[2 * size_t(tile) + 1] = l_tot;
  }
}

// The loss from the tiles' sums (written by k_ssim_maps, so complete when this kernel starts), added in tile order
// with a fixed reduction tree by one workgroup: out[0] = loss, out[1] = mean |x - y|, out[2] = mean S.
__device__ __forceinline__ void loss_total(const double* __restrict__ part, uint32_t num_tiles, double inv_n,
                                           float lam, float* __restrict__ out, double* s_red) {
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

__global__ __launch_bounds__(kThreads) void k_ssim_grad(Taps taps, uint32_t width, uint32_t height, uint32_t tiles_x,
                                                        uint32_t num_tiles,
                                                        float lam, float inv_n, const float4* __restrict__ out_rgba,
                                                        const float* __restrict__ target,
                                                        const float* __restrict__ maps, float4* __restrict__ v_out,
                                                        const double* __restrict__ part, double inv_nd,
                                                        float* __restrict__ loss) {
  __shared__ float s_d[9][kP][kP];   // the nine planes on the tile grown by 5 (0 outside the image)
  __shared__ float s_h[9][kP][kT];   // their horizontal sums
  __shared__ double s_red[kThreads / 64];
  const int tid = int(threadIdx.x);
  if (blockIdx.x == 0) loss_total(part, num_tiles, inv_nd, lam, loss, s_red);
  const uint32_t tile = band_tile(num_tiles);
  if (tile >= num_tiles) return;
  const int tx0 = int(tile % tiles_x) * kT, ty0 = int(tile / tiles_x) * kT;
  const int W = int(width), H = int(height);
  const size_t plane = size_t(W) * H;
  {
    float v[kLoads][9];
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int e = tid + it * int(kThreads);
      const int r = e / kP, q = e % kP;
      const int gx = tx0 - kR + q, gy = ty0 - kR + r;
      const bool in = e < kP * kP && gx >= 0 && gy >= 0 && gx < W && gy < H;
      const size_t p = in ? size_t(gy) * W + gx : 0;
#pragma unroll
      for (int k = 0; k < 9; ++k) v[it][k] = in ? maps[k * plane + p] : 0.0f;
    }
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int e = tid + it * int(kThreads);
      if (e >= kP * kP) break;
      const int r = e / kP, q = e % kP;
#pragma unroll
      for (int k = 0; k < 9; ++k) s_d[k][r][q] = v[it][k];
    }
  }
  __syncthreads();
  if (tid < kP * (kT / 2)) {  // two neighbouring columns per thread, as in k_ssim_maps
    const int r = tid % kP, q0 = 2 * (tid / kP);
    float b[9][2];
#pragma unroll
    for (int k = 0; k < 9; ++k) b[k][0] = b[k][1] = 0.0f;
#pragma unroll
    for (int j = 0; j <= 2 * kR + 1; ++j) {
      float v[9];
#pragma unroll
      for (int k = 0; k < 9; ++k) v[k] = s_d[k][r][q0 + j];
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const int t = j - o;
        if (t >= 0 && t <= 2 * kR) {
          const float g = taps.g[t];
#pragma unroll
          for (int k = 0; k < 9; ++k) b[k][o] = fmaf(g, v[k], b[k][o]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      s_h[k][r][q0] = b[k][0];
      s_h[k][r][q0 + 1] = b[k][1];
    }
  }
  __syncthreads();
  const int ox = tid % kT, oy = tid / kT;
  const int px = tx0 + ox, py = ty0 + oy;
  if (px >= W || py >= H) return;
  float b[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) b[k] = 0.0f;
#pragma unroll
  for (int t = 0; t <= 2 * kR; ++t) {
    const float g = taps.g[t];
#pragma unroll
    for (int k = 0; k < 9; ++k) b[k] = fmaf(g, s_h[k][oy + t][ox], b[k]);
  }
  const size_t p = size_t(py) * W + px;
  const float4 x4 = out_rgba[p];
  const float xs[3] = {x4.x, x4.y, x4.z};
  float g[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const float xv = xs[c], yv = target[3 * p + c];
    const float dssim = fmaf(yv, b[6 + c], fmaf(2.0f * xv, b[3 + c], b[c]));
    const float diff = xv - yv;
    const float sgn = diff > 0.0f ? 1.0f : (diff < 0.0f ? -1.0f : 0.0f);
    g[c] = ((1.0f - lam) * sgn - lam * dssim) * inv_n;
  }
  v_out[p] = make_float4(g[0], g[1], g[2], 0.0f);
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
  if ((st = grow(ctx, ctx->arena.loss_maps, size_t(width) * height * 9 * sizeof(float)))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* part = static_cast<double*>(ctx->arena.loss_part.ptr);
  float* maps = static_cast<float*>(ctx->arena.loss_maps.ptr);
  const double n = 3.0 * double(width) * double(height);
  const Taps taps = make_taps();
  timing_mark(ctx, GSR_STAGE_LOSS, s, false);
  const uint32_t grid = uint32_t((num_tiles + kXcds - 1) / kXcds * kXcds);
  hipLaunchKernelGGL(k_ssim_maps, dim3(grid), dim3(kThreads), 0, s, taps, width, height, uint32_t(tiles_x),
                     uint32_t(num_tiles), reinterpret_cast<const float4*>(out_rgba), target, maps, part);
  hipLaunchKernelGGL(k_ssim_grad, dim3(grid), dim3(kThreads), 0, s, taps, width, height, uint32_t(tiles_x),
                     uint32_t(num_tiles), 0.2f, float(1.0 / n), reinterpret_cast<const float4*>(out_rgba), target, maps,
                     reinterpret_cast<float4*>(v_out), part, 1.0 / n, loss);
  timing_mark(ctx, GSR_STAGE_LOSS, s, true);
  return check_launch(ctx, "gsr_loss_l1_ssim");
}
