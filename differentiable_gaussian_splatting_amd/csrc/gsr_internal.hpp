// Internal declarations shared by the libgsr translation units: the context, its grow-only device arena, error
// reporting, and the launch helpers one file provides to another.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "gsr.h"

namespace gsr {

constexpr uint32_t kTile = 16;          // 16x16 pixel tiles
constexpr uint32_t kTilePixels = 256;   // one workgroup of 4 wave64 per tile in the raster kernels
constexpr uint32_t kWave = 64;

// One device allocation that only ever grows. Contents are not preserved across growth.
struct DevBuf {
  void* ptr = nullptr;
  size_t bytes = 0;
};

// Everything gsr_bin and gsr_radix_sort keep between calls. Sized by the largest call seen so far (C0 resident
// arena: capacity only grows, so steady-state iterations allocate nothing).
struct Arena {
  DevBuf keys[2];     // uint64 [pair capacity], ping-pong
  DevBuf vals[2];     // uint32 [pair capacity], ping-pong
  DevBuf counts;      // uint32 [splat capacity] pairs per splat (in emission order)
  DevBuf offsets;     // uint64 [splat capacity + 1] exclusive scan of counts
  DevBuf order;       // uint64 [splat capacity] depth keys / splat order for the presort scheme (x2 for ping-pong)
  DevBuf order_alt;   // uint64 [max(splat, pair capacity)]: depth sort scratch, then the presort scheme's 64-bit keys
  DevBuf order_vals;  // uint32 [splat capacity]
  DevBuf order_vals_alt;
  DevBuf scan_part;   // uint64 [scan blocks] partial sums of the count scan
  DevBuf hist;        // uint32 [256 * sort blocks] per-block digit counts, then their per-digit scan
  DevBuf digit_tot;   // uint32 [256] per-digit totals of the current pass
  DevBuf ranges;      // uint32 [2 * tiles]
  DevBuf rects;       // uint32x4 [splat capacity] tile rectangle (tx0, ty0, w, h) of each splat, natural order
  DevBuf tile_scratch;  // uint64 [pair capacity] the tile-first per-tile order's entries for lists longer than LDS
  DevBuf tile_rows;   // uint32 [splat blocks + 2][tiles] tile-first counting sort: block offsets, tile totals, starts
  DevBuf tile_order_ext;  // uint32 [tiles] raster launch order: the slowest expected tiles first
  DevBuf tile_cost;   // uint32 [4 tiles] splats each wavefront of the last forward walked (launch-order hint)
  DevBuf loss_part;   // double [2 tiles] per-tile sums of the SSIM map and |x - y| (the loss)
  DevBuf loss_maps;   // float [9][H][W] the SSIM map's three derivatives per channel, between the loss's passes
  DevBuf grad_fixed;  // the deterministic backward's sums: uint64 [n][9][2] fixed point, then uint32 [n] flags
  size_t limit = 0;                // GSR_OPT_ARENA_LIMIT: most bytes the buffers above may hold together (0: none)
  uint64_t* host_total = nullptr;  // pinned host word for the one pair-count readback (written by a kernel)
  uint64_t* host_total_dev = nullptr;  // its device-side address
  uint32_t* done = nullptr;        // last-block-done counter of the count scan (0 between launches)
  hipEvent_t total_ready = nullptr;  // recorded after the readback is queued
};

}  // namespace gsr

struct gsr_ctx {
  int device = 0;
  std::string error;
  gsr::Arena arena;
  int32_t bin_scheme = GSR_BIN_TILE_DEPTH;
  int32_t bin_rule = GSR_BIN_BOX;
  bool bin_keys = true;
  bool raster_skip = true;  // per-wave cull and the backward's all-lanes-rejected skip
  bool deterministic = false;  // backward sums independent of scheduling (fixed-point atomics)
  int32_t backward_scheme = GSR_BACKWARD_PER_PIXEL;
  int32_t tile_order = GSR_ORDER_COST;  // how raster_tile_order ranks the tiles
  int32_t forward_exp = GSR_EXP_EXACT;  // the forward's exponential (GSR_OPT_FORWARD_EXP)
  // GSR_OPT_BIN_SYNC_FREE, and the pair counts it sizes its buffers from
  bool bin_sync_free = false;
  bool pairs_pending = false;  // the last gsr_bin's count is still on its way to the pinned word
  uint64_t pair_hint = 0;      // the largest pair count the host has read
  uint64_t pair_reserved = 0;  // the largest gsr_reserve
  uint64_t last_pairs = 0;     // the last count read
  uint64_t last_cap = 0;       // pairs the last gsr_bin's launches were sized for (its count, when it waited)
  uint64_t cost_tiles = 0;  // tile count of the grid tile_cost describes (0: none yet)
  const uint32_t* order_ranges = nullptr;  // the ranges tile_order_ext was last ranked for (by a forward)
  uint64_t order_tiles = 0;
  // gsr_render_forward_noalloc's scratch on this context's device: the device address of a file-scope array
  // (looked up once, when the context is created)
  uint32_t* noalloc_scratch = nullptr;
  // GSR_OPT_KERNEL_TIMING: events [stage][slot][begin, end], a ring of timing_cap launches per stage
  std::vector<hipEvent_t> timing_events;
  uint32_t timing_cap = 0;
  uint64_t timing_count[GSR_NUM_STAGES] = {};
};

namespace gsr {

// Records a message on ctx and returns `st`.
gsr_status fail(gsr_ctx* ctx, gsr_status st, const char* fmt, ...);

// Maps a HIP error (this call's or an earlier asynchronous one) to GSR_EHIP with its name.
gsr_status hip_fail(gsr_ctx* ctx, hipError_t e, const char* what);

// Makes ctx's device current for this thread.
gsr_status enter(gsr_ctx* ctx);

// Bytes held by the arena's buffers.
size_t arena_bytes(const Arena& a);

// Grows `b` to at least `bytes` (grow-only; factor 1.5 over the previous size, floor 64 KiB, neither beyond the
// arena limit). GSR_ENOMEM when the allocation fails or the arena would pass its limit; `b` then keeps its size.
gsr_status grow(gsr_ctx* ctx, DevBuf& b, size_t bytes);

// Checks for launch errors after queuing kernels.
gsr_status check_launch(gsr_ctx* ctx, const char* what);

// With kernel timing on, records the begin (end = false) or end event of the stage's current launch on `s`.
void timing_mark(gsr_ctx* ctx, int stage, hipStream_t s, bool end);

// Reads the pair count the last gsr_bin left in the pinned word (its launch must have completed) into
// ctx->last_pairs and raises ctx->pair_hint to it.
void note_pair_count(gsr_ctx* ctx);

// Looks up the device address of gsr_render_forward_noalloc's scratch array on the current device into
// ctx->noalloc_scratch (raster_fwd.hip; called by gsr_create with ctx's device current).
gsr_status noalloc_setup(gsr_ctx* ctx);

// Raster launch order (bin.hip): writes into `order` the tiles 0..num_tiles-1 with the longest pair lists first
// (64 length classes; any order inside a class), on stream s. One workgroup.
// With `cost` ([4 tiles], per-wavefront walk lengths of an earlier forward on the same grid), tiles are ranked by
// their summed cost instead of their list length.
// With `identity`, order[t] = t (no ranking).
void launch_tile_order(hipStream_t s, const uint32_t* ranges, const uint32_t* cost, uint32_t num_tiles,
                       uint32_t num_pairs, uint32_t* order, bool identity = false);
// The launch order of the raster kernels for `bins`, computed now into the arena: by the last forward's measured
// per-tile cost when it ran on the same tile grid, else by list length. Results never depend on the order; it only
// lets the slowest tiles start first. Null on failure (the error is recorded on ctx).
// The backward reuses the order the forward ranked for the same ranges pointer and grid (gsr_bin clears it).
const uint32_t* raster_tile_order(gsr_ctx* ctx, hipStream_t s, const gsr_bins* bins, bool backward,
                                  gsr_status* st);

// Radix sort (sort.hip). Sorts n (key, value) pairs stably by the low key_bits bits, 6 or 8 bits per pass
// (sort_passes). The result lands in (keys_out, vals_out); (tmp_keys, tmp_vals) are scratch of n elements. The
// first pass must not write over keys_in: keys_in may equal keys_out when the pass count is even and tmp_keys when
// it is odd. Uses the arena's histogram buffers (grown as needed).
// With n_dev (here and in the two tile sorts below), n is a capacity: the launches are sized for n keys and sort
// the first *n_dev of them, a count earlier launches on the stream leave in device memory (none when it exceeds n).
uint32_t sort_blocks(uint64_t n);
uint32_t sort_passes(uint32_t key_bits);
template <typename K>
gsr_status radix_sort_launch(gsr_ctx* ctx, hipStream_t s, const K* keys_in, const uint32_t* vals_in, uint64_t n,
                             uint32_t key_bits, K* keys_out, uint32_t* vals_out, K* tmp_keys, uint32_t* tmp_vals,
                             const uint64_t* n_dev = nullptr);

// Per-tile depth order of the tile-first scheme (tile_depth.hip): one workgroup per tile puts the tile's list
// list[start..end) (ranges clamped to the pair count, *pairs_dev when not null) in (depth bits, splat) order. The
// list holds packed words (tile << idx_bits) | splat when list_vals is null, else list_vals holds the splats;
// `ordered` says it is in ascending splat order (otherwise any order). The result is written to vals_out[start..end)
// and, when keys_out is not null, keys_out = (tile << 32) | depth bits. Lists longer than tile_depth_capacity() are
// sorted through gent (a 64-bit pair-count array) and gk0, gk1, gp0, gp1 (32-bit pair-count arrays), each tile using
// its own stretch; gent shares no memory with the other five.
void launch_tile_depth(hipStream_t s, const uint32_t* list, const uint32_t* list_vals, uint32_t idx_bits,
                       bool ordered, const uint32_t* ranges, uint64_t pairs_cap, const uint64_t* pairs_dev,
                       uint32_t num_tiles, const float* depths, uint32_t n, uint32_t* vals_out, uint64_t* keys_out,
                       uint64_t* gent, uint32_t* gk0, uint32_t* gk1, uint32_t* gp0, uint32_t* gp1);
uint32_t tile_depth_capacity();

// Per-super-tile order of the fused counting sort (tile_depth.hip): one workgroup per super-tile (2 x 2 tiles,
// row-major over a grid of ceil(tiles_x / 2) columns) sorts its list list[sup_start .. + sup_total) (clamped to the
// pair count) of entries (depth bits << 32) | (cover << 28) | splat, in any order, by (depth bits, splat) and writes
// each of its tiles' lists from the tile's start (ranges) on: vals_out = the splats, keys_out (if not null) =
// (tile << 32) | depth bits. Cover bit 2 dy + dx says the splat belongs to tile (dx, dy) of the super-tile. Lists
// longer than LDS holds are partitioned through gk0, gk1 and ordered in chunks; lists or chunks with many equal
// depths are sorted through gk0, gk1, gp0, gp1 (32-bit pair-count arrays, each super-tile using its own stretch)
// and the list's own stretch, which the call overwrites.
void launch_super_order(hipStream_t s, uint64_t* list, const uint32_t* sup_start, const uint32_t* sup_total,
                        uint32_t num_sup, uint32_t tiles_x, uint32_t tiles_y, const uint32_t* ranges,
                        uint64_t pairs_cap, const uint64_t* pairs_dev, const float* depths, uint32_t n,
                        uint32_t* vals_out, uint64_t* keys_out, uint32_t* gk0, uint32_t* gk1, uint32_t* gp0,
                        uint32_t* gp1);

// The same sort of 32-bit tile ids whose last pass also writes keys_final[g] = (key << 32) | bits(depths[val]) for
// every output position g (values below n_depths; others get depth bits 0). Requires key_bits > 0.
gsr_status radix_sort_tiles_final(gsr_ctx* ctx, hipStream_t s, const uint32_t* keys_in, const uint32_t* vals_in,
                                  uint64_t n, uint32_t key_bits, uint32_t* keys_out, uint32_t* vals_out,
                                  uint32_t* tmp_keys, uint32_t* tmp_vals, uint64_t* keys_final,
                                  const float* depths, uint32_t n_depths, const uint64_t* n_dev = nullptr);

// The tile sort on packed keys (tile << idx_bits) | value (idx_bits + tile_bits <= 32): sorts stably by the tile
// field, keys only; the last pass writes the sorted keys to keys_out, the values to vals_out and, when keys_final
// is not null, keys_final[g] = (tile << 32) | bits(depths[value]). With vals_out null the keys stay packed (the
// last pass writes keys only). Same pass-parity rule as radix_sort_launch.
gsr_status radix_sort_tiles_packed(gsr_ctx* ctx, hipStream_t s, const uint32_t* keys_in, uint64_t n,
                                   uint32_t idx_bits, uint32_t tile_bits, uint32_t* keys_out, uint32_t* tmp_keys,
                                   uint32_t* vals_out, uint64_t* keys_final, const float* depths,
                                   uint32_t n_depths, const uint64_t* n_dev = nullptr);

}  // namespace gsr
