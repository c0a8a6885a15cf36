// Projection of 3D Gaussians to the rasterizer's 2D splat records, and its backward pass, for gfx950.
//
// The pages fix the five parameter groups of a Gaussian (means 3, log_scales 3, rot_quats 4, raw_opacities 1,
// sh_coeffs 16 x 3 for SH degree 3: 59 floats; M3 per-splat backward page, full-scale parity table; forward/Adam
// audit page, section 2 "(f)") and that the record's opacity is the sigmoid of the raw opacity (W1 warp sparse skip
// + exp-skip page, section 1). The projection itself is the pinhole EWA projection:
//   t = R p + tv (culled when t.z <= near); Sigma = Rq diag(exp(2 log_s)) Rq^T, Rq from the normalised quaternion
//   (w, x, y, z); J = d(pixel mean)/dt; Sigma' = J R Sigma R^T J^T + 0.3 I; conic = Sigma'^-1;
//   mean = (fx tx / tz + cx, fy ty / tz + cy); rgb = max(sum_k sh_k Y_k(d) + 0.5, 0) with d the unit vector from the
//   camera centre to p and Y_k the real spherical harmonics of degrees 0..3; o = sigmoid(raw); depth = tz.
// One thread per Gaussian, fp32. The 2x2 determinant is formed as det(T T^T) + 0.3 trace(T T^T) + 0.09 with
// T = J R Rq diag(s) and det(T T^T) as the sum of the squared 2x2 minors of T (Cauchy-Binet): every term is a sum
// of squares, so the conic of a thin Gaussian keeps its relative accuracy where a c - b^2 would cancel.
// The backward recomputes the forward's intermediates and applies the chain rule in reverse, with
// dL/dSigma' = -C G C (C the conic, G = [[ga, gb / 2], [gb / 2, gc]]) and dL/dT = 2 dL/dSigma' T.
#include "gsr_internal.hpp"

namespace gsr {
namespace {

constexpr uint32_t kThreads = 256;
constexpr float kLowPass = 0.3f;

struct Cam {
  float R[9], tv[3], fx, fy, cx, cy, near, centre[3];
};

// Real spherical harmonics of degrees 0..3 (orthonormal on the sphere, Condon-Shortley signs), at unit d.
struct ShConst {
  static constexpr float c0 = 0.28209479177387814f;   // 1 / (2 sqrt(pi))
  static constexpr float c1 = 0.48860251190291992f;   // sqrt(3 / (4 pi))
  static constexpr float c2a = 1.0925484305920792f;   // sqrt(15 / (4 pi))
  static constexpr float c2b = 0.31539156525252005f;  // sqrt(5 / (16 pi))
  static constexpr float c2c = 0.54627421529603959f;  // sqrt(15 / (16 pi))
  static constexpr float c3a = 0.59004358992664352f;  // sqrt(35 / (32 pi))
  static constexpr float c3b = 2.8906114426405538f;   // sqrt(105 / (4 pi))
  static constexpr float c3c = 0.45704579946446572f;  // sqrt(21 / (32 pi))
  static constexpr float c3d = 0.3731763325901154f;   // sqrt(7 / (16 pi))
  static constexpr float c3e = 1.4453057213202769f;   // sqrt(105 / (16 pi))
};

__device__ __forceinline__ void sh_basis(float x, float y, float z, float (&Y)[16]) {
  using C = ShConst;
  const float xx = x * x, yy = y * y, zz = z * z;
  Y[0] = C::c0;
  Y[1] = -C::c1 * y;
  Y[2] = C::c1 * z;
  Y[3] = -C::c1 * x;
  Y[4] = C::c2a * (x * y);
  Y[5] = -C::c2a * (y * z);
  Y[6] = C::c2b * (2.0f * zz - xx - yy);
  Y[7] = -C::c2a * (x * z);
  Y[8] = C::c2c * (xx - yy);
  Y[9] = -C::c3a * (y * (3.0f * xx - yy));
  Y[10] = C::c3b * (x * y * z);
  Y[11] = -C::c3c * (y * (4.0f * zz - xx - yy));
  Y[12] = C::c3d * (z * (2.0f * zz - 3.0f * xx - 3.0f * yy));
  Y[13] = -C::c3c * (x * (4.0f * zz - xx - yy));
  Y[14] = C::c3e * (z * (xx - yy));
  Y[15] = -C::c3a * (x * (xx - 3.0f * yy));
}

// sum_k dY_k grad(Y_k) at d: the gradient of the polynomials above, each differentiated term by term.
__device__ __forceinline__ void sh_basis_vjp(float x, float y, float z, const float (&dY)[16], float& gx, float& gy,
                                             float& gz) {
  using C = ShConst;
  const float xx = x * x, yy = y * y, zz = z * z;
  gx = -C::c1 * dY[3];
  gy = -C::c1 * dY[1];
  gz = C::c1 * dY[2];
  gx += C::c2a * (y * dY[4]) - C::c2a * (z * dY[7]) - 2.0f * C::c2b * (x * dY[6]) + 2.0f * C::c2c * (x * dY[8]);
  gy += C::c2a * (x * dY[4]) - C::c2a * (z * dY[5]) - 2.0f * C::c2b * (y * dY[6]) - 2.0f * C::c2c * (y * dY[8]);
  gz += -C::c2a * (y * dY[5]) + 4.0f * C::c2b * (z * dY[6]) - C::c2a * (x * dY[7]);
  // degree 3
  gx += -C::c3a * (6.0f * x * y) * dY[9] + C::c3b * (y * z) * dY[10] + C::c3c * (2.0f * x * y) * dY[11] +
        C::c3d * (-6.0f * x * z) * dY[12] - C::c3c * (4.0f * zz - 3.0f * xx - yy) * dY[13] +
        C::c3e * (2.0f * x * z) * dY[14] - C::c3a * (3.0f * xx - 3.0f * yy) * dY[15];
  gy += -C::c3a * (3.0f * xx - 3.0f * yy) * dY[9] + C::c3b * (x * z) * dY[10] -
        C::c3c * (4.0f * zz - xx - 3.0f * yy) * dY[11] + C::c3d * (-6.0f * y * z) * dY[12] +
        C::c3c * (2.0f * x * y) * dY[13] - C::c3e * (2.0f * y * z) * dY[14] + C::c3a * (6.0f * x * y) * dY[15];
  gz += C::c3b * (x * y) * dY[10] - C::c3c * (8.0f * y * z) * dY[11] + C::c3d * (6.0f * zz - 3.0f * xx - 3.0f * yy) * dY[12] -
        C::c3c * (8.0f * x * z) * dY[13] + C::c3e * (xx - yy) * dY[14];
}

// Everything the forward computes for one Gaussian that the backward needs again.
struct Proj {
  float t[3], s[3], qn[4], qinv, Rq[9], RM[9];
  float j00, j02, j11, j12, T[6];  // T row-major 2x3
  float sxx, sxy, syy, det, a, b, c;
  float dir[3], vinv;
};

__device__ __forceinline__ void project_one(const Cam& cam, const float* p, const float* ls, const float* q, Proj& P) {
  const float* R = cam.R;
#pragma unroll
  for (int r = 0; r < 3; ++r) P.t[r] = fmaf(R[3 * r + 2], p[2], fmaf(R[3 * r + 1], p[1], fmaf(R[3 * r], p[0], cam.tv[r])));
#pragma unroll
  for (int k = 0; k < 3; ++k) P.s[k] = expf(ls[k]);
  const float qq = fmaf(q[3], q[3], fmaf(q[2], q[2], fmaf(q[1], q[1], q[0] * q[0])));
  P.qinv = 1.0f / sqrtf(qq);
#pragma unroll
  for (int k = 0; k < 4; ++k) P.qn[k] = q[k] * P.qinv;
  const float w = P.qn[0], x = P.qn[1], y = P.qn[2], z = P.qn[3];
  P.Rq[0] = 1.0f - 2.0f * (y * y + z * z);
  P.Rq[1] = 2.0f * (x * y - w * z);
  P.Rq[2] = 2.0f * (x * z + w * y);
  P.Rq[3] = 2.0f * (x * y + w * z);
  P.Rq[4] = 1.0f - 2.0f * (x * x + z * z);
  P.Rq[5] = 2.0f * (y * z - w * x);
  P.Rq[6] = 2.0f * (x * z - w * y);
  P.Rq[7] = 2.0f * (y * z + w * x);
  P.Rq[8] = 1.0f - 2.0f * (x * x + y * y);
  // RM = R (Rq diag(s))
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int k = 0; k < 3; ++k)
      P.RM[3 * r + k] =
          fmaf(R[3 * r + 2], P.Rq[6 + k], fmaf(R[3 * r + 1], P.Rq[3 + k], R[3 * r] * P.Rq[k])) * P.s[k];
  const float tz = P.t[2], iz = 1.0f / tz;
  P.j00 = cam.fx * iz;
  P.j11 = cam.fy * iz;
  P.j02 = -P.j00 * (P.t[0] * iz);
  P.j12 = -P.j11 * (P.t[1] * iz);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    P.T[k] = fmaf(P.j00, P.RM[k], P.j02 * P.RM[6 + k]);
    P.T[3 + k] = fmaf(P.j11, P.RM[3 + k], P.j12 * P.RM[6 + k]);
  }
  const float* T = P.T;
  const float txx = fmaf(T[2], T[2], fmaf(T[1], T[1], T[0] * T[0]));
  const float tyy = fmaf(T[5], T[5], fmaf(T[4], T[4], T[3] * T[3]));
  P.sxy = fmaf(T[2], T[5], fmaf(T[1], T[4], T[0] * T[3]));
  P.sxx = txx + kLowPass;
  P.syy = tyy + kLowPass;
  const float m01 = fmaf(T[0], T[4], -(T[1] * T[3]));
  const float m02 = fmaf(T[0], T[5], -(T[2] * T[3]));
  const float m12 = fmaf(T[1], T[5], -(T[2] * T[4]));
  const float detTT = fmaf(m12, m12, fmaf(m02, m02, m01 * m01));
  P.det = fmaf(kLowPass, txx + tyy, detTT) + kLowPass * kLowPass;
  const float idet = 1.0f / P.det;
  P.a = P.syy * idet;
  P.b = -P.sxy * idet;
  P.c = P.sxx * idet;
  const float v0 = p[0] - cam.centre[0], v1 = p[1] - cam.centre[1], v2 = p[2] - cam.centre[2];
  P.vinv = 1.0f / sqrtf(fmaf(v2, v2, fmaf(v1, v1, v0 * v0)));
  P.dir[0] = v0 * P.vinv;
  P.dir[1] = v1 * P.vinv;
  P.dir[2] = v2 * P.vinv;
}

__device__ __forceinline__ void load3(const float* __restrict__ a, uint32_t i, float (&v)[3]) {
  v[0] = a[3 * size_t(i)];
  v[1] = a[3 * size_t(i) + 1];
  v[2] = a[3 * size_t(i) + 2];
}

// The SH blocks of a workgroup's 256 Gaussians are contiguous (256 x 192 B). The backward moves them between HBM and
// LDS with 16-byte accesses of consecutive threads to consecutive addresses, and each thread reads or writes its own
// 48 values in LDS (a thread storing its own 192 bytes makes every wave-wide store touch 64 lines); the forward
// loads them directly, which measured faster there (no 48 KB of LDS per workgroup, twice the resident waves).
constexpr uint32_t kShVec = 12;  // float4 per Gaussian

__device__ __forceinline__ void stage_sh_in(const float* __restrict__ sh, uint32_t n, float4* s_sh) {
  const uint32_t g0 = blockIdx.x * kThreads;
  const uint32_t count = min(kThreads, n - g0) * kShVec;
  const float4* src = reinterpret_cast<const float4*>(sh) + size_t(g0) * kShVec;
#pragma unroll
  for (uint32_t j = 0; j < kShVec; ++j) {
    const uint32_t e = threadIdx.x + j * kThreads;
    if (e < count) s_sh[e] = src[e];
  }
  __syncthreads();
}

__device__ __forceinline__ void stage_sh_out(float* __restrict__ out, uint32_t n, const float4* s_sh) {
  __syncthreads();
  const uint32_t g0 = blockIdx.x * kThreads;
  const uint32_t count = min(kThreads, n - g0) * kShVec;
  float4* dst = reinterpret_cast<float4*>(out) + size_t(g0) * kShVec;
#pragma unroll
  for (uint32_t j = 0; j < kShVec; ++j) {
    const uint32_t e = threadIdx.x + j * kThreads;
    if (e < count) dst[e] = s_sh[e];
  }
}

__device__ __forceinline__ void load_sh(const float* __restrict__ sh, uint32_t i, float (&c)[48]) {
  const float4* s4 = reinterpret_cast<const float4*>(sh + 48 * size_t(i));
#pragma unroll
  for (uint32_t k = 0; k < kShVec; ++k) {
    const float4 v = s4[k];
    c[4 * k] = v.x;
    c[4 * k + 1] = v.y;
    c[4 * k + 2] = v.z;
    c[4 * k + 3] = v.w;
  }
}

__device__ __forceinline__ void read_sh(const float4* s_sh, float (&c)[48]) {
#pragma unroll
  for (uint32_t k = 0; k < kShVec; ++k) {
    const float4 v = s_sh[threadIdx.x * kShVec + k];
    c[4 * k] = v.x;
    c[4 * k + 1] = v.y;
    c[4 * k + 2] = v.z;
    c[4 * k + 3] = v.w;
  }
}

__global__ __launch_bounds__(kThreads) void k_project_forward(Cam cam, uint32_t n, const float* __restrict__ means,
                                                              const float* __restrict__ log_scales,
                                                              const float* __restrict__ quats,
                                                              const float* __restrict__ raw_op,
                                                              const float* __restrict__ sh, float* __restrict__ splats,
                                                              float* __restrict__ depths) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  float p[3], ls[3], q[4];
  load3(means, i, p);
  load3(log_scales, i, ls);
  const float4 q4 = reinterpret_cast<const float4*>(quats)[i];
  q[0] = q4.x, q[1] = q4.y, q[2] = q4.z, q[3] = q4.w;
  float* rec = splats + 9 * size_t(i);
  const float tz = fmaf(cam.R[8], p[2], fmaf(cam.R[7], p[1], fmaf(cam.R[6], p[0], cam.tv[2])));
  if (!(tz > cam.near)) {  // culled (also a NaN depth): a zero record that binning skips
#pragma unroll
    for (int k = 0; k < 9; ++k) rec[k] = 0.0f;
    depths[i] = 0.0f;
    return;
  }
  Proj P;
  project_one(cam, p, ls, q, P);
  float c[48];
  load_sh(sh, i, c);  // direct 16-byte loads: staging through LDS (as the backward does) measured slower here
  float Y[16];
  sh_basis(P.dir[0], P.dir[1], P.dir[2], Y);
  float rgb[3];
#pragma unroll
  for (int ch = 0; ch < 3; ++ch) {
    float acc = 0.5f;
#pragma unroll
    for (int k = 0; k < 16; ++k) acc = fmaf(Y[k], c[3 * k + ch], acc);
    rgb[ch] = acc > 0.0f ? acc : 0.0f;
  }
  const float iz = 1.0f / P.t[2];
  rec[0] = fmaf(cam.fx, P.t[0] * iz, cam.cx);
  rec[1] = fmaf(cam.fy, P.t[1] * iz, cam.cy);
  rec[2] = P.a;
  rec[3] = P.b;
  rec[4] = P.c;
  rec[5] = rgb[0];
  rec[6] = rgb[1];
  rec[7] = rgb[2];
  rec[8] = 1.0f / (1.0f + expf(-raw_op[i]));
  depths[i] = P.t[2];
}

__device__ __forceinline__ void backward_one(const Cam& cam, uint32_t i, const float* __restrict__ means,
                                             const float* __restrict__ log_scales, const float* __restrict__ quats,
                                             const float* __restrict__ raw_op, const float* __restrict__ splats_grad,
                                             float* __restrict__ g_means, float* __restrict__ g_log_scales,
                                             float* __restrict__ g_quats, float* __restrict__ g_raw_op,
                                             float4* s_sh) {
  float p[3], ls[3], q[4];
  load3(means, i, p);
  load3(log_scales, i, ls);
  const float4 q4 = reinterpret_cast<const float4*>(quats)[i];
  q[0] = q4.x, q[1] = q4.y, q[2] = q4.z, q[3] = q4.w;
  const float tz0 = fmaf(cam.R[8], p[2], fmaf(cam.R[7], p[1], fmaf(cam.R[6], p[0], cam.tv[2])));
  float4* gsh4 = s_sh + threadIdx.x * kShVec;  // the thread's coefficients, overwritten by their gradients
  if (!(tz0 > cam.near)) {
#pragma unroll
    for (int k = 0; k < 3; ++k) g_means[3 * size_t(i) + k] = g_log_scales[3 * size_t(i) + k] = 0.0f;
    reinterpret_cast<float4*>(g_quats)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    g_raw_op[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < 12; ++k) gsh4[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    return;
  }
  float g[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) g[k] = splats_grad[9 * size_t(i) + k];
  Proj P;
  project_one(cam, p, ls, q, P);

  // opacity
  const float o = 1.0f / (1.0f + expf(-raw_op[i]));
  g_raw_op[i] = g[8] * (o * (1.0f - o));

  // colour: d sh, and d dir through the basis
  float c[48];
  read_sh(s_sh, c);
  float Y[16];
  sh_basis(P.dir[0], P.dir[1], P.dir[2], Y);
  float gc[3];
#pragma unroll
  for (int ch = 0; ch < 3; ++ch) {
    float acc = 0.5f;
#pragma unroll
    for (int k = 0; k < 16; ++k) acc = fmaf(Y[k], c[3 * k + ch], acc);
    gc[ch] = acc > 0.0f ? g[5 + ch] : 0.0f;
  }
  float dY[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) dY[k] = fmaf(gc[2], c[3 * k + 2], fmaf(gc[1], c[3 * k + 1], gc[0] * c[3 * k]));
#pragma unroll
  for (int k = 0; k < 12; ++k) {
    const int e = 4 * k;  // elements e..e+3 of the [16][3] block: coefficient e / 3, channel e % 3, ...
    gsh4[k] = make_float4(gc[e % 3] * Y[e / 3], gc[(e + 1) % 3] * Y[(e + 1) / 3], gc[(e + 2) % 3] * Y[(e + 2) / 3],
                          gc[(e + 3) % 3] * Y[(e + 3) / 3]);
  }
  float gdx, gdy, gdz;
  sh_basis_vjp(P.dir[0], P.dir[1], P.dir[2], dY, gdx, gdy, gdz);
  // d = v / |v|: dL/dv = (dL/dd - d (d . dL/dd)) / |v|
  const float dd = fmaf(P.dir[2], gdz, fmaf(P.dir[1], gdy, P.dir[0] * gdx));
  float gp[3] = {(gdx - P.dir[0] * dd) * P.vinv, (gdy - P.dir[1] * dd) * P.vinv, (gdz - P.dir[2] * dd) * P.vinv};

  // conic -> Sigma': dS = -C G C with G = [[ga, gb / 2], [gb / 2, gc]]
  const float ga = g[2], gbh = 0.5f * g[3], gcc = g[4];
  const float x00 = fmaf(P.a, ga, P.b * gbh), x01 = fmaf(P.a, gbh, P.b * gcc);
  const float x10 = fmaf(P.b, ga, P.c * gbh), x11 = fmaf(P.b, gbh, P.c * gcc);
  const float dSxx = -fmaf(x00, P.a, x01 * P.b);
  const float dSxy = -fmaf(x00, P.b, x01 * P.c);
  const float dSyy = -fmaf(x10, P.b, x11 * P.c);
  // Sigma' = T T^T + 0.3 I: dT = 2 dS T
  float dT[6];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    dT[k] = 2.0f * fmaf(dSxx, P.T[k], dSxy * P.T[3 + k]);
    dT[3 + k] = 2.0f * fmaf(dSxy, P.T[k], dSyy * P.T[3 + k]);
  }
  // T = J RM
  const float dj00 = fmaf(dT[2], P.RM[2], fmaf(dT[1], P.RM[1], dT[0] * P.RM[0]));
  const float dj02 = fmaf(dT[2], P.RM[8], fmaf(dT[1], P.RM[7], dT[0] * P.RM[6]));
  const float dj11 = fmaf(dT[5], P.RM[5], fmaf(dT[4], P.RM[4], dT[3] * P.RM[3]));
  const float dj12 = fmaf(dT[5], P.RM[8], fmaf(dT[4], P.RM[7], dT[3] * P.RM[6]));
  float dRM[9];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    dRM[k] = P.j00 * dT[k];
    dRM[3 + k] = P.j11 * dT[3 + k];
    dRM[6 + k] = fmaf(P.j02, dT[k], P.j12 * dT[3 + k]);
  }
  // RM = R M: dM = R^T dRM; M = Rq diag(s): dRq = dM diag(s), ds_k = sum_j dM_jk Rq_jk
  const float* R = cam.R;
  float dRq[9], gls[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    float ds = 0.0f;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const float dM = fmaf(R[6 + j], dRM[6 + k], fmaf(R[3 + j], dRM[3 + k], R[j] * dRM[k]));
      dRq[3 * j + k] = dM * P.s[k];
      ds = fmaf(dM, P.Rq[3 * j + k], ds);
    }
    gls[k] = ds * P.s[k];
  }
  // rotation matrix of the unit quaternion (w, x, y, z)
  const float w = P.qn[0], x = P.qn[1], y = P.qn[2], z = P.qn[3];
  const float dw = 2.0f * (-z * dRq[1] + y * dRq[2] + z * dRq[3] - x * dRq[5] - y * dRq[6] + x * dRq[7]);
  const float dx = 2.0f * (y * dRq[1] + z * dRq[2] + y * dRq[3] - 2.0f * x * dRq[4] - w * dRq[5] + z * dRq[6] +
                           w * dRq[7] - 2.0f * x * dRq[8]);
  const float dy = 2.0f * (-2.0f * y * dRq[0] + x * dRq[1] + w * dRq[2] + x * dRq[3] + z * dRq[5] - w * dRq[6] +
                           z * dRq[7] - 2.0f * y * dRq[8]);
  const float dz = 2.0f * (-2.0f * z * dRq[0] - w * dRq[1] + x * dRq[2] + w * dRq[3] - 2.0f * z * dRq[4] +
                           y * dRq[5] + x * dRq[6] + y * dRq[7]);
  // q_n = q / |q|: dq = (dqn - qn (qn . dqn)) / |q|
  const float qd = fmaf(z, dz, fmaf(y, dy, fmaf(x, dx, w * dw)));
  reinterpret_cast<float4*>(g_quats)[i] =
      make_float4((dw - w * qd) * P.qinv, (dx - x * qd) * P.qinv, (dy - y * qd) * P.qinv, (dz - z * qd) * P.qinv);
#pragma unroll
  for (int k = 0; k < 3; ++k) g_log_scales[3 * size_t(i) + k] = gls[k];

  // mean and J through t
  const float iz = 1.0f / P.t[2], iz2 = iz * iz;
  const float fxz2 = cam.fx * iz2, fyz2 = cam.fy * iz2;
  const float dtx = fmaf(g[0], cam.fx * iz, -dj02 * fxz2);
  const float dty = fmaf(g[1], cam.fy * iz, -dj12 * fyz2);
  const float dtz = -(g[0] * fxz2) * P.t[0] - (g[1] * fyz2) * P.t[1] - dj00 * fxz2 - dj11 * fyz2 +
                    2.0f * (dj02 * fxz2) * (P.t[0] * iz) + 2.0f * (dj12 * fyz2) * (P.t[1] * iz);
  // t = R p + tv: dp = R^T dt
#pragma unroll
  for (int k = 0; k < 3; ++k)
    g_means[3 * size_t(i) + k] = gp[k] + fmaf(R[6 + k], dtz, fmaf(R[3 + k], dty, R[k] * dtx));
}

__global__ __launch_bounds__(kThreads) void k_project_backward(
    Cam cam, uint32_t n, const float* __restrict__ means, const float* __restrict__ log_scales,
    const float* __restrict__ quats, const float* __restrict__ raw_op, const float* __restrict__ sh,
    const float* __restrict__ splats_grad, float* __restrict__ g_means, float* __restrict__ g_log_scales,
    float* __restrict__ g_quats, float* __restrict__ g_raw_op, float* __restrict__ g_sh) {
  __shared__ float4 s_sh[kThreads * kShVec];  // the coefficients in, then their gradients out
  stage_sh_in(sh, n, s_sh);
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  // every thread of the workgroup reaches the barrier of stage_sh_out, so the work below runs under a condition
  if (i < n) backward_one(cam, i, means, log_scales, quats, raw_op, splats_grad, g_means, g_log_scales, g_quats,
                          g_raw_op, s_sh);
  stage_sh_out(g_sh, n, s_sh);
}

Cam make_cam(const gsr_camera& c) {
  Cam k;
  for (int j = 0; j < 9; ++j) k.R[j] = c.R[j];
  for (int j = 0; j < 3; ++j) k.tv[j] = c.tv[j];
  k.fx = c.fx, k.fy = c.fy, k.cx = c.cx, k.cy = c.cy, k.near = c.near;
  for (int j = 0; j < 3; ++j) {  // centre = -R^T tv, in double then rounded
    double s = 0.0;
    for (int r = 0; r < 3; ++r) s -= double(c.R[3 * r + j]) * double(c.tv[r]);
    k.centre[j] = float(s);
  }
  return k;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace gsr

using namespace gsr;

extern "C" gsr_status gsr_project_forward(gsr_ctx* ctx, void* stream, const gsr_camera* cam, uint32_t n,
                                          const float* means, const float* log_scales, const float* quats,
                                          const float* raw_opacities, const float* sh, float* splats,
                                          float* depths) {
  if (!ctx) return GSR_EINVAL;
  if (!cam) return fail(ctx, GSR_EINVAL, "gsr_project_forward: null camera");
  if (n == 0) return GSR_OK;
  if (uint64_t(n) * 48 >= (uint64_t(1) << 32)) return fail(ctx, GSR_EOVERFLOW, "gsr_project_forward: n * 48 >= 2^32");
  if (!means || !log_scales || !quats || !raw_opacities || !sh || !splats || !depths)
    return fail(ctx, GSR_EINVAL, "gsr_project_forward: null pointer");
  if (!aligned16(quats) || !aligned16(sh))
    return fail(ctx, GSR_EINVAL, "gsr_project_forward: quats and sh must be 16-byte aligned");
  gsr_status st = enter(ctx);
  if (st) return st;
  timing_mark(ctx, GSR_STAGE_PROJECT_FORWARD, static_cast<hipStream_t>(stream), false);
  hipLaunchKernelGGL(k_project_forward, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), make_cam(*cam), n, means, log_scales, quats, raw_opacities, sh,
                     splats, depths);
  timing_mark(ctx, GSR_STAGE_PROJECT_FORWARD, static_cast<hipStream_t>(stream), true);
  return check_launch(ctx, "gsr_project_forward");
}

extern "C" gsr_status gsr_project_backward(gsr_ctx* ctx, void* stream, const gsr_camera* cam, uint32_t n,
                                           const float* means, const float* log_scales, const float* quats,
                                           const float* raw_opacities, const float* sh, const float* splats_grad,
                                           float* means_grad, float* log_scales_grad, float* quats_grad,
                                           float* raw_opacities_grad, float* sh_grad) {
  if (!ctx) return GSR_EINVAL;
  if (!cam) return fail(ctx, GSR_EINVAL, "gsr_project_backward: null camera");
  if (n == 0) return GSR_OK;
  if (uint64_t(n) * 48 >= (uint64_t(1) << 32))
    return fail(ctx, GSR_EOVERFLOW, "gsr_project_backward: n * 48 >= 2^32");
  if (!means || !log_scales || !quats || !raw_opacities || !sh || !splats_grad || !means_grad || !log_scales_grad ||
      !quats_grad || !raw_opacities_grad || !sh_grad)
    return fail(ctx, GSR_EINVAL, "gsr_project_backward: null pointer");
  if (!aligned16(quats) || !aligned16(sh) || !aligned16(quats_grad) || !aligned16(sh_grad))
    return fail(ctx, GSR_EINVAL, "gsr_project_backward: quats, sh and their gradients must be 16-byte aligned");
  gsr_status st = enter(ctx);
  if (st) return st;
  timing_mark(ctx, GSR_STAGE_PROJECT_BACKWARD, static_cast<hipStream_t>(stream), false);
  hipLaunchKernelGGL(k_project_backward, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), make_cam(*cam), n, means, log_scales, quats, raw_opacities, sh,
                     splats_grad, means_grad, log_scales_grad, quats_grad, raw_opacities_grad, sh_grad);
  timing_mark(ctx, GSR_STAGE_PROJECT_BACKWARD, static_cast<hipStream_t>(stream), true);
  return check_launch(ctx, "gsr_project_backward");
}
