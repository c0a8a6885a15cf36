// Fused Adam: every parameter group in one launch, eight elements per thread (two 16-byte non-temporal loads per
// array, all issued before any arithmetic) where the group's arrays allow it. 28 bytes move per element (read grad,
// m, v, param; write m, v, param), so the kernel is bound by HBM bandwidth. [rasterize forward + adam kernel audit
// page, section 2 "(f)": 5 groups, 59 elements per splat, 28 B per element, 1,652 B per splat]
//
// Every operation is one IEEE fp32 operation in the order written (the file is compiled without contraction; HIP's
// default division and square root are correctly rounded), so the step equals a plain fp32 evaluation.
#include "gsr_internal.hpp"

namespace gsr {
namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kVec = 2;                     // float4 loads per array and thread
constexpr uint32_t kPerThread = 4 * kVec;        // elements per thread
constexpr uint32_t kPerBlock = kThreads * kPerThread;

struct AdamArgs {
  float* param[GSR_ADAM_MAX_GROUPS];
  const float* grad[GSR_ADAM_MAX_GROUPS];
  float* m[GSR_ADAM_MAX_GROUPS];
  float* v[GSR_ADAM_MAX_GROUPS];
  uint64_t count[GSR_ADAM_MAX_GROUPS];
  float lr[GSR_ADAM_MAX_GROUPS];
  uint32_t vec4[GSR_ADAM_MAX_GROUPS];               // all four arrays 16-byte aligned
  uint32_t block_start[GSR_ADAM_MAX_GROUPS + 1];    // first workgroup of each group
  uint32_t n_groups;
  float beta1, beta2, eps, bc1, bc2;
  // visible-only step: splat i is visible when pairs[i] != 0; group q has per_splat[q] elements per splat, and
  // magic[q] = floor(2^32 / per_splat[q]) + 1 divides the small offsets inside a block by it exactly
  const uint32_t* pairs;
  uint32_t per_splat[GSR_ADAM_MAX_GROUPS];
  uint64_t magic[GSR_ADAM_MAX_GROUPS];
};

struct Hyper {
  float b1, b2, omb1, omb2, eps, bc1, bc2, lr;
};

__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v, const Hyper& h) {
  const float m_new = h.b1 * m + h.omb1 * g;
  const float v_new = h.b2 * v + h.omb2 * (g * g);
  const float m_hat = m_new / h.bc1;
  const float v_hat = v_new / h.bc2;
  const float denom = sqrtf(v_hat) + h.eps;
  p = p - (h.lr * m_hat) / denom;
  m = m_new;
  v = v_new;
}

// Streaming loads and stores (no reuse): non-temporal, so they do not displace anything in the caches.
using f4 = float __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f4 ld_stream(const float* p) { return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p)); }
__device__ __forceinline__ void st_stream(float* p, f4 v) { __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p)); }

// Visibility of the elements of one block of a group: element blk0 + o (o < kPerBlock) belongs to splat
// s0 + (r0 + o) / k, where blk0 = s0 k + r0; the small offset x = r0 + o < 2^12 is divided by multiplying with
// m = floor(2^32 / k) + 1 and keeping the bits above 32: x m / 2^32 = x / k + x (m - 2^32 / k) / 2^32, and the
// second term is below 1 / k for x < 2^32 / k, so the floor is exact.
struct BlockSplats {
  const uint32_t* pairs;
  uint64_t s0, magic;
  uint32_t r0;
  __device__ bool visible(uint32_t o) const { return pairs[s0 + ((uint64_t(r0 + o) * magic) >> 32)] != 0u; }
};

// kVisible: only elements of visible splats are read, updated and written; a float4 with no visible element is
// neither loaded nor stored, and one with some is stored back whole (its invisible elements with their own bits).
template <bool kVisible>
__global__ __launch_bounds__(kThreads) void k_adam(AdamArgs a) {
  uint32_t q = 0;
  while (q + 1 < a.n_groups && a.block_start[q + 1] <= blockIdx.x) ++q;
  const uint64_t count = a.count[q];
  // a block covers kPerBlock consecutive elements; thread t takes float4 number t and t + kThreads (coalesced)
  const uint64_t blk0 = uint64_t(blockIdx.x - a.block_start[q]) * kPerBlock;
  if (blk0 >= count) return;
  const Hyper h{a.beta1, a.beta2, 1.0f - a.beta1, 1.0f - a.beta2, a.eps, a.bc1, a.bc2, a.lr[q]};
  float* __restrict__ P = a.param[q];
  const float* __restrict__ G = a.grad[q];
  float* __restrict__ M = a.m[q];
  float* __restrict__ V = a.v[q];
  BlockSplats bs{};
  if constexpr (kVisible) {
    const uint32_t k = a.per_splat[q];
    bs = {a.pairs, blk0 / k, a.magic[q], 0u};
    bs.r0 = uint32_t(blk0 - bs.s0 * k);
  }
  if (a.vec4[q] && blk0 + kPerBlock <= count) {
    f4 p[kVec], g[kVec], m[kVec], v[kVec];
    uint32_t vis[kVec];  // bit e: element e of the float4 is visible
#pragma unroll
    for (uint32_t c = 0; c < kVec; ++c) {
      const uint32_t o = 4 * (c * kThreads + threadIdx.x);
      vis[c] = 0xFu;
      if constexpr (kVisible) {
        vis[c] = 0u;
#pragma unroll
        for (uint32_t e = 0; e < 4; ++e) vis[c] |= uint32_t(bs.visible(o + e)) << e;
      }
      if (vis[c]) {
        p[c] = ld_stream(P + blk0 + o);
        g[c] = ld_stream(G + blk0 + o);
        m[c] = ld_stream(M + blk0 + o);
        v[c] = ld_stream(V + blk0 + o);
      }
    }
#pragma unroll
    for (uint32_t c = 0; c < kVec; ++c) {
      if (!vis[c]) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pe = p[c][e], me = m[c][e], ve = v[c][e];
        adam_one(pe, g[c][e], me, ve, h);
        if (!kVisible || ((vis[c] >> e) & 1u)) {
          p[c][e] = pe;
          m[c][e] = me;
          v[c][e] = ve;
        }
      }
      const uint64_t i = blk0 + 4 * (uint64_t(c) * kThreads + threadIdx.x);
      st_stream(P + i, p[c]);
      st_stream(M + i, m[c]);
      st_stream(V + i, v[c]);
    }
  } else {
    // tail block or unaligned arrays: element by element
    for (uint64_t i = blk0 + threadIdx.x; i < count && i < blk0 + kPerBlock; i += kThreads) {
      if (kVisible && !bs.visible(uint32_t(i - blk0))) continue;
      float p = P[i], m = M[i], v = V[i];
      adam_one(p, G[i], m, v, h);
      P[i] = p;
      M[i] = m;
      V[i] = v;
    }
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace gsr

using namespace gsr;

namespace {

constexpr uint32_t kMaxPerSplat = 1024;

// visible: null for the dense step; else the per-splat pair counts of n splats.
gsr_status adam_launch(gsr_ctx* ctx, void* stream, const gsr_adam_group* groups, uint32_t n_groups, float beta1,
                       float beta2, float eps, float bc1, float bc2, bool sparse, const uint32_t* visible, uint32_t n,
                       const char* what) {
  if (!ctx) return GSR_EINVAL;
  if (n_groups > GSR_ADAM_MAX_GROUPS)
    return fail(ctx, GSR_EINVAL, "%s: %u groups, at most %d", what, n_groups, GSR_ADAM_MAX_GROUPS);
  if (n_groups && !groups) return fail(ctx, GSR_EINVAL, "%s: null groups", what);
  if (!(bc1 > 0.0f) || !(bc2 > 0.0f)) return fail(ctx, GSR_EINVAL, "%s: bias corrections must be > 0", what);
  if (sparse && n && !visible) return fail(ctx, GSR_EINVAL, "%s: null splat_pairs", what);
  AdamArgs a{};
  uint64_t blocks = 0;
  a.n_groups = n_groups;
  a.pairs = visible;
  for (uint32_t q = 0; q < n_groups; ++q) {
    const gsr_adam_group& g = groups[q];
    if (g.count && (!g.param || !g.grad || !g.m || !g.v))
      return fail(ctx, GSR_EINVAL, "%s: group %u has a null array", what, q);
    if (sparse) {
      const uint64_t k = n ? g.count / n : 0;
      if (n ? (g.count % n != 0) : (g.count != 0))
        return fail(ctx, GSR_EINVAL, "%s: group %u has %llu elements, not a multiple of %u splats", what, q,
                    (unsigned long long)g.count, n);
      if (k > kMaxPerSplat)
        return fail(ctx, GSR_EINVAL, "%s: group %u has %llu elements per splat, at most %u", what, q,
                    (unsigned long long)k, kMaxPerSplat);
      a.per_splat[q] = uint32_t(k ? k : 1);
      a.magic[q] = (uint64_t(1) << 32) / a.per_splat[q] + 1;
    }
    a.param[q] = g.param;
    a.grad[q] = g.grad;
    a.m[q] = g.m;
    a.v[q] = g.v;
    a.count[q] = g.count;
    a.lr[q] = g.lr;
    a.vec4[q] = aligned16(g.param) && aligned16(g.grad) && aligned16(g.m) && aligned16(g.v);
    a.block_start[q] = uint32_t(blocks);
    blocks += (g.count + kPerBlock - 1) / kPerBlock;
    if (blocks >= (uint64_t(1) << 31)) return fail(ctx, GSR_EOVERFLOW, "%s: too many elements", what);
  }
  a.block_start[n_groups] = uint32_t(blocks);
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  a.bc1 = bc1;
  a.bc2 = bc2;
  if (blocks == 0) return GSR_OK;
  gsr_status st = enter(ctx);
  if (st) return st;
  timing_mark(ctx, GSR_STAGE_ADAM, static_cast<hipStream_t>(stream), false);
  hipLaunchKernelGGL(sparse ? k_adam<true> : k_adam<false>, dim3(uint32_t(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  timing_mark(ctx, GSR_STAGE_ADAM, static_cast<hipStream_t>(stream), true);
  return check_launch(ctx, what);
}

}  // namespace

extern "C" gsr_status gsr_adam_step(gsr_ctx* ctx, void* stream, const gsr_adam_group* groups, uint32_t n_groups,
                                    float beta1, float beta2, float eps, float bc1, float bc2) {
  return adam_launch(ctx, stream, groups, n_groups, beta1, beta2, eps, bc1, bc2, false, nullptr, 0, "gsr_adam_step");
}

extern "C" gsr_status gsr_adam_step_visible(gsr_ctx* ctx, void* stream, const gsr_adam_group* groups,
                                            uint32_t n_groups, float beta1, float beta2, float eps, float bc1,
                                            float bc2, const uint32_t* splat_pairs, uint32_t n) {
  return adam_launch(ctx, stream, groups, n_groups, beta1, beta2, eps, bc1, bc2, true, splat_pairs, n,
                     "gsr_adam_step_visible");
}
