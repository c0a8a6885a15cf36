// Context, arena and error plumbing of libgsr.
#include <algorithm>
#include <cstring>

#include "gsr_internal.hpp"

namespace gsr {

gsr_status fail(gsr_ctx* ctx, gsr_status st, const char* fmt, ...) {
  if (ctx) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    ctx->error = buf;
  }
  return st;
}

gsr_status hip_fail(gsr_ctx* ctx, hipError_t e, const char* what) {
  return fail(ctx, GSR_EHIP, "%s: HIP error %d (%s)", what, int(e), hipGetErrorName(e));
}

gsr_status enter(gsr_ctx* ctx) {
  hipError_t e = hipSetDevice(ctx->device);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipSetDevice");
  return GSR_OK;
}

// Calls f on every buffer of the arena.
template <typename F>
static void for_each_buffer(Arena& a, F f) {
  for (DevBuf* b : {&a.keys[0], &a.keys[1], &a.vals[0], &a.vals[1], &a.counts, &a.offsets, &a.order, &a.order_alt,
                    &a.order_vals, &a.order_vals_alt, &a.scan_part, &a.hist, &a.digit_tot,
                    &a.ranges, &a.rects,
                    &a.tile_order_ext, &a.tile_cost, &a.tile_rows, &a.tile_scratch, &a.loss_part, &a.loss_maps, &a.grad_fixed})
    f(*b);
}

size_t arena_bytes(const Arena& a) {
  size_t total = 0;
  for_each_buffer(const_cast<Arena&>(a), [&](DevBuf& b) { total += b.bytes; });
  return total;
}

gsr_status grow(gsr_ctx* ctx, DevBuf& b, size_t bytes) {
  if (bytes <= b.bytes) return GSR_OK;
  size_t want = std::max<size_t>({bytes, b.bytes + b.bytes / 2, size_t(1) << 16});
  if (ctx->arena.limit) {
    const size_t others = arena_bytes(ctx->arena) - b.bytes;
    if (others + bytes > ctx->arena.limit)
      return fail(ctx, GSR_ENOMEM, "device arena: growing a buffer to %zu bytes would pass the arena limit of %zu "
                  "bytes (%zu held by the other buffers)", bytes, ctx->arena.limit, others);
    want = std::min(want, ctx->arena.limit - others);
  }
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, want);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky allocation error; the old buffer stays valid
    if (want > bytes) {       // retry at the exact size before giving up
      want = bytes;
      e = hipMalloc(&p, want);
      if (e != hipSuccess) (void)hipGetLastError();
    }
    if (e != hipSuccess)
      return fail(ctx, GSR_ENOMEM, "device arena: could not grow a buffer to %zu bytes (%s)", bytes,
                  hipGetErrorName(e));
  }
  if (b.ptr) {
    // The old buffer may still be read by queued work on some stream: wait for the device before freeing it.
    hipError_t se = hipDeviceSynchronize();
    if (se != hipSuccess) {
      (void)hipFree(p);
      return hip_fail(ctx, se, "device arena: synchronize before growing");
    }
    (void)hipFree(b.ptr);
  }
  b.ptr = p;
  b.bytes = want;
  return GSR_OK;
}

gsr_status check_launch(gsr_ctx* ctx, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(ctx, e, what);
  return GSR_OK;
}

void timing_mark(gsr_ctx* ctx, int stage, hipStream_t s, bool end) {
  if (!ctx->timing_cap) return;
  const uint64_t slot = ctx->timing_count[stage] % ctx->timing_cap;
  // a failed record shows up as an error of gsr_kernel_times, not of the call being timed
  (void)hipEventRecord(ctx->timing_events[(size_t(stage) * ctx->timing_cap + slot) * 2 + (end ? 1 : 0)], s);
  if (end) ++ctx->timing_count[stage];
}

static void timing_release(gsr_ctx* ctx) {
  for (hipEvent_t e : ctx->timing_events) (void)hipEventDestroy(e);
  ctx->timing_events.clear();
  ctx->timing_cap = 0;
  for (uint64_t& c : ctx->timing_count) c = 0;
}

static gsr_status timing_setup(gsr_ctx* ctx, uint32_t cap) {
  timing_release(ctx);
  if (!cap) return GSR_OK;
  gsr_status st = enter(ctx);
  if (st) return st;
  ctx->timing_events.reserve(size_t(cap) * GSR_NUM_STAGES * 2);
  for (size_t i = 0; i < size_t(cap) * GSR_NUM_STAGES * 2; ++i) {
    hipEvent_t e = nullptr;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      timing_release(ctx);
      return hip_fail(ctx, err, "gsr_set_option: creating timing events");
    }
    ctx->timing_events.push_back(e);
  }
  ctx->timing_cap = cap;
  return GSR_OK;
}

static void release(DevBuf& b) {
  if (b.ptr) (void)hipFree(b.ptr);
  b.ptr = nullptr;
  b.bytes = 0;
}

void note_pair_count(gsr_ctx* ctx) {
  ctx->last_pairs = *static_cast<volatile uint64_t*>(ctx->arena.host_total);
  ctx->pair_hint = std::max(ctx->pair_hint, ctx->last_pairs);
  ctx->pairs_pending = false;
}

}  // namespace gsr

using namespace gsr;

extern "C" {

gsr_status gsr_create(gsr_ctx** out, int hip_device) {
  if (!out) return GSR_EINVAL;
  *out = nullptr;
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess) return GSR_EHIP;
  if (hip_device < 0 || hip_device >= count) return GSR_EINVAL;
  gsr_ctx* ctx = new (std::nothrow) gsr_ctx();
  if (!ctx) return GSR_ENOMEM;
  ctx->device = hip_device;
  if (enter(ctx) != GSR_OK) {
    delete ctx;
    return GSR_EHIP;
  }
  Arena& a = ctx->arena;
  // coherent: k_prep's store of the pair count is visible to the host once the launch has completed
  e = hipHostMalloc(reinterpret_cast<void**>(&a.host_total), sizeof(uint64_t),
                    hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess) {
    delete ctx;
    return GSR_ENOMEM;
  }
  *a.host_total = 0;
  e = hipHostGetDevicePointer(reinterpret_cast<void**>(&a.host_total_dev), a.host_total, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(a.host_total);
    delete ctx;
    return GSR_EHIP;
  }
  // the count scan's last-block-done counter, zero between launches
  e = hipMalloc(reinterpret_cast<void**>(&a.done), sizeof(uint32_t));
  if (e == hipSuccess) e = hipMemset(a.done, 0, sizeof(uint32_t));
  if (e == hipSuccess) e = hipEventCreateWithFlags(&a.total_ready, hipEventDisableTiming);
  if (e == hipSuccess && noalloc_setup(ctx) != GSR_OK) e = hipErrorInvalidSymbol;
  if (e != hipSuccess) {
    if (a.total_ready) (void)hipEventDestroy(a.total_ready);
    if (a.done) (void)hipFree(a.done);
    (void)hipHostFree(a.host_total);
    delete ctx;
    return GSR_EHIP;
  }
  *out = ctx;
  return GSR_OK;
}

void gsr_destroy(gsr_ctx* ctx) {
  if (!ctx) return;
  (void)hipSetDevice(ctx->device);
  Arena& a = ctx->arena;
  for_each_buffer(a, [](DevBuf& b) { release(b); });
  if (a.host_total) (void)hipHostFree(a.host_total);
  if (a.done) (void)hipFree(a.done);
  if (a.total_ready) (void)hipEventDestroy(a.total_ready);
  timing_release(ctx);
  delete ctx;
}

const char* gsr_last_error(const gsr_ctx* ctx) { return ctx ? ctx->error.c_str() : "null context"; }

gsr_status gsr_set_option(gsr_ctx* ctx, int32_t option, int64_t value) {
  if (!ctx) return GSR_EINVAL;
  switch (option) {
    case GSR_OPT_BIN_SCHEME:
      if (value != GSR_BIN_PRESORT && value != GSR_BIN_KEY64 && value != GSR_BIN_TILE_DEPTH)
        return fail(ctx, GSR_EINVAL, "gsr_set_option: unknown bin scheme %lld", (long long)value);
      ctx->bin_scheme = int32_t(value);
      return GSR_OK;
    case GSR_OPT_BIN_RULE:
      if (value != GSR_BIN_BOX && value != GSR_BIN_ELLIPSE)
        return fail(ctx, GSR_EINVAL, "gsr_set_option: unknown overlap rule %lld", (long long)value);
      ctx->bin_rule = int32_t(value);
      return GSR_OK;
    case GSR_OPT_BIN_KEYS:
      if (value != 0 && value != 1) return fail(ctx, GSR_EINVAL, "gsr_set_option: bin keys must be 0 or 1");
      ctx->bin_keys = value != 0;
      return GSR_OK;
    case GSR_OPT_RASTER_SKIP:
      if (value != 0 && value != 1) return fail(ctx, GSR_EINVAL, "gsr_set_option: raster skip must be 0 or 1");
      ctx->raster_skip = value != 0;
      return GSR_OK;
    case GSR_OPT_DETERMINISTIC:
      if (value != 0 && value != 1) return fail(ctx, GSR_EINVAL, "gsr_set_option: deterministic must be 0 or 1");
      ctx->deterministic = value != 0;
      return GSR_OK;
    case GSR_OPT_BACKWARD_SCHEME:
      if (value != GSR_BACKWARD_PER_PIXEL && value != GSR_BACKWARD_PER_SPLAT)
        return fail(ctx, GSR_EINVAL, "gsr_set_option: unknown backward scheme %lld", (long long)value);
      ctx->backward_scheme = int32_t(value);
      return GSR_OK;
    case GSR_OPT_TILE_ORDER:
      if (value != GSR_ORDER_COST && value != GSR_ORDER_LENGTH && value != GSR_ORDER_NONE)
        return fail(ctx, GSR_EINVAL, "gsr_set_option: unknown tile order %lld", (long long)value);
      ctx->tile_order = int32_t(value);
      ctx->order_ranges = nullptr;  // rank again at the next raster launch
      return GSR_OK;
    case GSR_OPT_ARENA_LIMIT:
      if (value < 0) return fail(ctx, GSR_EINVAL, "gsr_set_option: the arena limit must be >= 0");
      ctx->arena.limit = size_t(value);
      return GSR_OK;
    case GSR_OPT_FORWARD_EXP:
      if (value != GSR_EXP_EXACT && value != GSR_EXP_FAST)
        return fail(ctx, GSR_EINVAL, "gsr_set_option: unknown forward exponential %lld", (long long)value);
      ctx->forward_exp = int32_t(value);
      return GSR_OK;
    case GSR_OPT_BIN_SYNC_FREE:
      if (value != 0 && value != 1) return fail(ctx, GSR_EINVAL, "gsr_set_option: bin sync-free must be 0 or 1");
      ctx->bin_sync_free = value != 0;
      return GSR_OK;
    case GSR_OPT_KERNEL_TIMING:
      if (value < 0 || value > 4096)
        return fail(ctx, GSR_EINVAL, "gsr_set_option: kernel timing ring must hold 0..4096 launches");
      return timing_setup(ctx, uint32_t(value));
    default:
      return fail(ctx, GSR_EINVAL, "gsr_set_option: unknown option %d", int(option));
  }
}

gsr_status gsr_kernel_times(gsr_ctx* ctx, int32_t stage, float* ms, uint32_t max, uint32_t* count) {
  if (!ctx || !count || (max && !ms)) return GSR_EINVAL;
  *count = 0;
  if (stage < 0 || stage >= GSR_NUM_STAGES) return fail(ctx, GSR_EINVAL, "gsr_kernel_times: no stage %d", stage);
  if (!ctx->timing_cap) return fail(ctx, GSR_EINVAL, "gsr_kernel_times: kernel timing is off");
  gsr_status st = enter(ctx);
  if (st) return st;
  const uint64_t rec = ctx->timing_count[stage];
  const uint64_t n = std::min<uint64_t>({rec, ctx->timing_cap, max});
  for (uint64_t i = rec - n, j = 0; i < rec; ++i, ++j) {
    const size_t at = (size_t(stage) * ctx->timing_cap + i % ctx->timing_cap) * 2;
    hipError_t e = hipEventSynchronize(ctx->timing_events[at + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[j], ctx->timing_events[at], ctx->timing_events[at + 1]);
    if (e != hipSuccess) return hip_fail(ctx, e, "gsr_kernel_times");
  }
  *count = uint32_t(n);
  return GSR_OK;
}

gsr_status gsr_reserve(gsr_ctx* ctx, uint64_t max_pairs, uint32_t max_splats) {
  if (!ctx) return GSR_EINVAL;
  if (max_pairs >= (uint64_t(1) << 32)) return fail(ctx, GSR_EOVERFLOW, "gsr_reserve: max_pairs >= 2^32");
  gsr_status st = enter(ctx);
  if (st) return st;
  Arena& a = ctx->arena;
  const uint64_t ns = uint64_t(max_splats) + 1;
  const uint64_t nb = std::max<uint64_t>({sort_blocks(max_pairs), sort_blocks(ns), 1});
  struct {
    DevBuf* b;
    size_t bytes;
  } plan[] = {
      {&a.keys[0], size_t(max_pairs) * 8}, {&a.keys[1], size_t(max_pairs) * 8},
      {&a.vals[0], size_t(max_pairs) * 4}, {&a.vals[1], size_t(max_pairs) * 4},
      {&a.counts, size_t(ns) * 4},         {&a.offsets, size_t(ns + 1) * 8},
      {&a.order, size_t(ns) * 8},
      {&a.order_alt, size_t(std::max<uint64_t>(ns, max_pairs)) * 8},  // also the presort scheme's 64-bit keys
      {&a.order_vals, size_t(ns) * 4},
      {&a.order_vals_alt, size_t(std::max<uint64_t>(ns, max_pairs)) * 4},  // also the tile-first scheme's scratch
      {&a.tile_scratch, size_t(max_pairs) * 8},
      {&a.scan_part, size_t(std::max<uint64_t>(nb, ns / 256 + 1) + 1) * 8},
      {&a.hist, size_t(nb) * 256 * 4},     {&a.digit_tot, 256 * 4},
      {&a.rects, size_t(ns) * 16},
  };
  for (auto& p : plan)
    if ((st = grow(ctx, *p.b, p.bytes))) return st;
  ctx->pair_reserved = std::max(ctx->pair_reserved, max_pairs);
  return GSR_OK;
}


gsr_status gsr_bins_copy(gsr_ctx* ctx, void* stream, const gsr_bins* bins, uint64_t* keys, uint32_t* vals,
                         uint32_t* ranges, uint32_t* splat_pairs) {
  if (!ctx || !bins) return GSR_EINVAL;
  gsr_status st = enter(ctx);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t P = bins->num_pairs;
  const size_t T = size_t(bins->tiles_x) * bins->tiles_y;
  if (keys && P) {
    if (!bins->keys) return fail(ctx, GSR_EINVAL, "gsr_bins_copy: the bins carry no keys");
    hipError_t e = hipMemcpyAsync(keys, bins->keys, P * 8, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "gsr_bins_copy keys");
  }
  if (vals && P) {
    hipError_t e = hipMemcpyAsync(vals, bins->vals, P * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "gsr_bins_copy vals");
  }
  if (ranges && T) {
    hipError_t e = hipMemcpyAsync(ranges, bins->ranges, T * 8, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "gsr_bins_copy ranges");
  }
  if (splat_pairs && bins->num_splats) {
    if (!bins->splat_pairs) return fail(ctx, GSR_EINVAL, "gsr_bins_copy: the bins carry no splat_pairs");
    hipError_t e = hipMemcpyAsync(splat_pairs, bins->splat_pairs, size_t(bins->num_splats) * 4,
                                  hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "gsr_bins_copy splat_pairs");
  }
  return GSR_OK;
}

uint32_t gsr_radix_pass_count(uint64_t num_tiles, uint32_t digit_bits) {
  if (digit_bits != 4 && digit_bits != 8) return 0;
  uint32_t tile_bits = 0;
  for (uint64_t v = num_tiles ? num_tiles - 1 : 0; v; v >>= 1) ++tile_bits;
  const uint32_t all = 64 / digit_bits, depth = 32 / digit_bits;
  const uint32_t p = depth + (tile_bits + digit_bits - 1) / digit_bits;
  return p < all ? p : all;
}

}  // extern "C"
