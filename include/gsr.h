/* gsr.h - C ABI of libgsr, a tile-based differentiable 2D-splat rasterizer for AMD MI355X (gfx950).
 *
 * The library runs the hot path of a Gaussian-splatting training step on one GPU:
 *   gsr_bin             (tile | depth) keys per splat-tile overlap, a stable LSD radix sort, per-tile ranges
 *   gsr_render_forward  per-pixel front-to-back alpha compositing over each 16x16 tile's depth-sorted splats
 *   gsr_render_backward the 9 per-splat 2D gradients of that compositing
 *   gsr_adam_step       one fused Adam step over every parameter group (gsr_adam_step_visible: only the splats
 *                       binned in the view)
 * and, on either side of it, the projection of 3D Gaussians to those splats and the projection's backward pass
 * (gsr_project_forward / gsr_project_backward), and the L1 + SSIM loss that gives the backward its v_out
 * (gsr_loss_l1_ssim).
 *
 * Conventions shared by every entry point
 *   - Pointers named as device pointers must point to memory allocated on the context's device (hipMalloc or a
 *     caching allocator on top of it, such as PyTorch's). The caller owns them and keeps them alive until the work
 *     queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void*; NULL means the device's null stream. Every call queues its work on
 *     that stream and returns without waiting, except gsr_bin, which waits once for a 4-byte count (see there).
 *   - Arguments are checked before any work is queued; a rejected call queues nothing. An error raised by the HIP
 *     runtime (including a fault of earlier asynchronous work found by this call) is reported as GSR_EHIP.
 *     gsr_last_error() then holds a message for the last failing call on that context.
 *   - One context serves one host thread and one stream at a time; it is not thread-safe.
 *   - Splat records are 9 float32 values {x, y, a, b, c, r, g, b, o}, row-major [n][9]: the mean in pixels, the
 *     conic [[a, b], [b, c]] (inverse 2D covariance), the colour, and the opacity color_a in [0, 1]. Pixel (px, py)
 *     has its centre at (px + 0.5, py + 0.5). Tiles are 16x16 pixels; tiles_x = ceil(width / 16),
 *     tiles_y = ceil(height / 16), tile id = ty * tiles_x + tx. Images are row-major.
 */
#ifndef GSR_H
#define GSR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gsr_status;
#define GSR_OK 0
#define GSR_EINVAL (-1)    /* bad pointer, size or option; nothing was queued                                   */
#define GSR_ENOMEM (-2)    /* growing the device arena failed; the arena keeps its previous size and stays usable */
#define GSR_EHIP (-3)      /* the HIP runtime reported an error; gsr_last_error() has its name                   */
#define GSR_EOVERFLOW (-4) /* a count does not fit its 32-bit field (pairs >= 2^32, n * 9 >= 2^32)               */

typedef struct gsr_ctx gsr_ctx;

/* Creates a context on HIP device `hip_device`. The context owns a grow-only device arena for the binning
 * (keys, values, per-splat counts and offsets, radix histograms, tile ranges), reused across calls: only a call
 * that needs more room reallocates it. [C0 resident arena + C1 pass skip page, section 2 table, row "C0 resident
 * arena"] Returns GSR_EINVAL for a null `out` or a device index out of range, GSR_EHIP or GSR_ENOMEM otherwise. */
gsr_status gsr_create(gsr_ctx** out, int hip_device);

/* Frees the arena and the context. Waits for nothing: the caller must have finished using every gsr_bins view. */
void gsr_destroy(gsr_ctx* ctx);

/* Message for the last failing call on `ctx` ("" if none). The pointer stays valid until the next call on ctx. */
const char* gsr_last_error(const gsr_ctx* ctx);

/* Grows the arena so that later gsr_bin calls with up to `max_pairs` pairs and `max_splats` splats allocate
 * nothing (first-touch and allocation stay out of timed loops). [C0 resident arena + C1 pass skip page, section 1,
 * "Day 0 attribution": fresh allocation 26.50 ms vs reused buffers 0.61 ms] */
gsr_status gsr_reserve(gsr_ctx* ctx, uint64_t max_pairs, uint32_t max_splats);

/* Context options (gsr_set_option). */
#define GSR_OPT_BIN_SCHEME 1 /* how gsr_bin orders the pairs; all schemes give bit-identical results:            */
#define GSR_BIN_PRESORT 0    /*   radix-sort splats by depth, emit pairs in that order, then a stable radix sort  */
                             /*   of the pairs by tile id only                                                    */
#define GSR_BIN_KEY64 1      /*   emit pairs splat by splat and radix-sort the full 64-bit keys                   */
#define GSR_BIN_TILE_DEPTH 2 /*   default: tile order first, then each list by (depth, splat) in one workgroup.   */
                             /*   Under the box rule with at most 8192 tiles and fewer than 2^28 splats, a        */
                             /*   counting sort into the lists of 2x2-tile super-tiles, each of which is sorted   */
                             /*   once on chip (longer lists than 4608 entries in chunks of consecutive depths)   */
                             /*   and filtered into its four tiles' lists; otherwise emission in splat order, a   */
                             /*   radix sort by tile id and a sort of each tile's list (on chip up to 3456        */
                             /*   pairs, longer lists through the arena), and when the last pair count seen       */
                             /*   averages more than 3072 pairs per tile, a call runs the presort scheme instead  */
#define GSR_OPT_BIN_KEYS 2   /* 1 (default): gsr_bin materialises the sorted 64-bit keys; 0: keys = NULL          */
#define GSR_OPT_RASTER_SKIP 3 /* 1 (default): the raster kernels skip work that provably changes nothing - splats   */
                              /*   that cannot reach alpha >= 1/255 in a wavefront's 8x8 block, and, in the        */
                              /*   backward, splats no lane of a wavefront composited; 0: every lane evaluates    */
                              /*   every splat up to its bound. Results are identical either way (the A/B switch  */
                              /*   of the W1 warp sparse skip + exp-skip page, section 1, "raster_backward_sparse")*/
#define GSR_OPT_BIN_RULE 4    /* which tiles a splat is binned to (the pages never state the rule; the 1M-splat    */
                             /*   stress count of about 16M keys fits the ellipse rule):                          */
#define GSR_BIN_BOX 0        /*   default: every tile of the axis-aligned box of the 3-sigma ellipse              */
#define GSR_BIN_ELLIPSE 1    /*   the box's tiles whose closed 16x16 square the 3-sigma ellipse                   */
                             /*   (p - mean)^T [[a b][b c]] (p - mean) <= 9 meets, decided in fp32 from the       */
                             /*   minimum of the quadratic over the square (0 if the mean is inside, else the     */
                             /*   least edge minimum at the clamped vertex)                                       */
#define GSR_OPT_DETERMINISTIC 5 /* 0 (default): the backward adds its per-tile sums with float atomics, so the     */
                              /*   last bits of splats_grad depend on scheduling; 1: the same bits on every run.   */
                              /*   Within a tile, each pair of wavefronts adds into a per-batch sum of its own     */
                              /*   (two additions to a zeroed cell commute exactly) and the two are added at the  */
                              /*   end of the batch; the tiles' totals are summed as 128-bit fixed-point integers  */
                              /*   (each rounded to a multiple of 2^-48) and rounded to float once. A tile total   */
                              /*   that is not finite, or of magnitude 2^79 or more, gives NaN or +-inf as a      */
                              /*   float sum would. Costs an arena buffer of 148 bytes per splat and about a fifth */
                              /*   of the backward's speed. (The per-splat backward page shrinks, but does not    */
                              /*   remove, the run-to-run noise by changing the loop order; its determinism note.) */
#define GSR_OPT_BACKWARD_SCHEME 7 /* the backward's loop order; both give the same terms, summed in other orders:   */
#define GSR_BACKWARD_PER_PIXEL 0  /*   default: a lane per pixel walks the splats; the 64 lanes' terms are reduced   */
                                  /*   across the wave for every splat some lane composited                          */
#define GSR_BACKWARD_PER_SPLAT 1  /*   a lane per splat sweeps the 64 pixels of its wave's 8x8 block in a diagonal  */
                                  /*   schedule, the pixel state passed lane to lane (the M3 per-splat backward     */
                                  /*   page's order); no cross-lane reduction, each splat's sums in pixel order     */
#define GSR_OPT_KERNEL_TIMING 6 /* 0 (default): off; n in 1..4096: every entry point records a pair of HIP events   */
                              /*   on its stream around its main kernel(s), in a ring of the last n launches per  */
                              /*   stage (read with gsr_kernel_times); setting the option clears the rings        */
#define GSR_OPT_TILE_ORDER 9    /* the order in which the raster kernels start their tiles (results never depend on */
#define GSR_ORDER_COST 0        /*   it): default: slowest first by the per-wavefront walk counts of the last       */
                                /*   forward on the same tile grid (a stand-in for this view's costs; list length  */
                                /*   before any forward);                                                          */
#define GSR_ORDER_LENGTH 1      /*   longest tile list first;                                                      */
#define GSR_ORDER_NONE 2        /*   tile index order                                                              */
#define GSR_OPT_ARENA_LIMIT 8  /* 0 (default): none; b > 0: the arena's buffers together never hold more than b   */
                              /*   bytes - a call that would grow it further fails with GSR_ENOMEM before queuing */
                              /*   anything that needs the growth, and the arena keeps its buffers and contents   */
                              /*   (a device-memory budget; also how failure handling is tested from the host).   */
                              /*   Lowering it frees nothing already held.                                       */
#define GSR_OPT_BIN_SYNC_FREE 10 /* 0 (default): gsr_bin waits once for the pair count and sizes its buffers to it;   */
                                /*   1: gsr_bin queues everything without waiting, its buffers sized for a capacity  */
                                /*   (the largest of 2^16, 16 n, 1.5 times the largest count seen and gsr_reserve's */
                                /*   pairs [C0 resident arena + C1 pass skip page, section 2 table, row "C0"]); its */
                                /*   kernels read the count from device memory. Identical results when the pairs    */
                                /*   fit; when they do not, nothing is emitted, every tile's range is empty and     */
                                /*   gsr_bin_pair_count reports the overflow (binning again then fits). A call with */
                                /*   no count seen yet and no reservation still waits once.                         */
#define GSR_OPT_FORWARD_EXP 11  /* the forward's exp(-sigma):                                                         */
#define GSR_EXP_EXACT 0         /*   (default) correctly rounded: T and every stop decision are those of a plain    */
                                /*   fp32 evaluation of the definition;                                               */
#define GSR_EXP_FAST 1          /*   the hardware exponential (relative error below 1e-6), the exact value only    */
                                /*   within 2^-18 of the 1/255 threshold: reject decisions stay exact, alpha and T  */
                                /*   carry the fast value's error, and a pixel whose exact T' falls that close to    */
                                /*   1e-4 may stop one splat apart. About 15 % faster.                               */
gsr_status gsr_set_option(gsr_ctx* ctx, int32_t option, int64_t value);

/* Stages timed by GSR_OPT_KERNEL_TIMING, each the kernels between its pair of events. */
#define GSR_STAGE_BIN 0              /* gsr_bin, first launch to last (its wait for the pair count included)      */
#define GSR_STAGE_FORWARD 1          /* the forward raster kernel                                                */
#define GSR_STAGE_BACKWARD 2         /* the backward raster kernel (not its zero fill, tile ranking or, with     */
                                     /*   GSR_OPT_DETERMINISTIC, the clearing and conversion of the fixed sums)  */
#define GSR_STAGE_ADAM 3             /* the Adam kernel, dense or visible-only                                   */
#define GSR_STAGE_PROJECT_FORWARD 4  /* the projection kernel                                                    */
#define GSR_STAGE_PROJECT_BACKWARD 5 /* the projection's backward kernel                                         */
#define GSR_STAGE_LOSS 6             /* both passes of the L1 + SSIM loss                                        */
#define GSR_STAGE_DEPTH_SORT 7       /* inside gsr_bin: the radix sort of the splats by depth (presort scheme)   */
#define GSR_STAGE_TILE_SORT 8        /* inside gsr_bin: the radix sort of the pairs (by tile, or by the 64-bit   */
                                     /*   key with GSR_BIN_KEY64), or the counting sort's scatter to super-tiles */
#define GSR_STAGE_TILE_DEPTH 9       /* inside gsr_bin: the per-tile (or per-super-tile) depth order of the      */
                                     /*   tile-first scheme                                                      */
#define GSR_STAGE_TILE_SCAN 10       /* inside gsr_bin: the column scan and list starts of the tile-first        */
                                     /*   scheme's counting sort (its scatter is GSR_STAGE_TILE_SORT)            */
#define GSR_NUM_STAGES 11

/* GPU durations in milliseconds of the recorded launches of `stage`, oldest first: the last min(recorded, ring
 * size, max) of them. Waits for the newest one to finish. *count = the number written.
 * Errors: GSR_EINVAL (null ctx, ms with max > 0, or count; stage out of range; timing off), GSR_EHIP. */
gsr_status gsr_kernel_times(gsr_ctx* ctx, int32_t stage, float* ms, uint32_t max, uint32_t* count);

/* Views into the context's arena, valid until the next gsr_bin or gsr_reserve on the same context. A caller may
 * also fill one with its own device buffers of the same layout (for example bins computed elsewhere). */
typedef struct gsr_bins {
  const uint64_t* keys;   /* [num_pairs] (tile id << 32) | float bits of the splat's depth, ascending; NULL     */
                          /*   with GSR_OPT_BIN_KEYS = 0, and it may be NULL when num_pairs is 0               */
  const uint32_t* vals;   /* [num_pairs] splat index of each key (may be NULL when num_pairs is 0)             */
  const uint32_t* ranges; /* [2 * tiles_x * tiles_y] (start, end) of each tile's run in keys / vals            */
  uint32_t num_pairs;
  uint32_t tiles_x;
  uint32_t tiles_y;
  const uint32_t* splat_pairs; /* [num_splats] pairs of each splat (0: not binned), or NULL; filled by gsr_bin   */
  uint32_t num_splats;
} gsr_bins;

/* Binning. For every splat that passes the validity test, one pair per 16x16 tile that its 3-sigma axis-aligned
 * box overlaps: key = (tile id << 32) | float bits of depths[i], value = i. The pairs are sorted stably by key
 * (ties in depth keep splat order) and each tile gets the [start, end) range of its pairs; tiles without pairs get
 * start = end = the position where their pairs would be. [C0 resident arena + C1 pass skip page, section 2 table,
 * rows "C0" and "C1"; tile size and range count from the M3 per-splat backward page, section 3 table]
 *   splats  device [n][9] float32;  depths  device [n] float32
 *   A splat emits nothing if any of its values or its depth is not finite, depth <= 0, a <= 0, a*c - b*b <= 0, or
 *   o is outside [0, 1]. The box is x +- 3 sqrt(c / det), y +- 3 sqrt(a / det), det = a*c - b*b, in fp32.
 *   out     host struct filled with views into the arena (valid until the context's next gsr_bin), including
 *           splat_pairs: the number of pairs each splat emitted (0 for a culled or off-image splat).
 * Synchronisation: waits on `stream` once, to read the pair count before sizing the arena; the rest is queued.
 *   With GSR_OPT_BIN_SYNC_FREE it does not wait: out->num_pairs is then the capacity the buffers were sized for
 *   (the ranges hold the exact runs; keys and vals past the last pair are unspecified), and gsr_bin_pair_count
 *   gives the count.
 * Errors: GSR_EINVAL (null pointers with n > 0, width or height 0, tiles_x * tiles_y >= 2^32),
 * GSR_EOVERFLOW (2^32 or more pairs), GSR_ENOMEM, GSR_EHIP. */
gsr_status gsr_bin(gsr_ctx* ctx, void* stream, const float* splats, const float* depths, uint32_t n,
                   uint32_t width, uint32_t height, gsr_bins* out);

/* The pair count of the context's last gsr_bin, waiting for it when that call did not (GSR_OPT_BIN_SYNC_FREE).
 * *overflowed = 1 when those pairs exceeded the capacity that call was sized for (it then emitted nothing; the
 * next gsr_bin sizes its buffers for at least this count), else 0. [C0 resident arena + C1 pass skip page,
 * section 2 table, row "C0": overflow means growing the arena and emitting again]
 * Errors: GSR_EINVAL (null pointers), GSR_EHIP. */
gsr_status gsr_bin_pair_count(gsr_ctx* ctx, uint64_t* num_pairs, int32_t* overflowed);

/* Copies the contents of `bins` into caller buffers (device pointers; any of them may be NULL to skip it):
 * keys [num_pairs] uint64, vals [num_pairs] uint32, ranges [2 * tiles] uint32, splat_pairs [num_splats] uint32.
 * Queued on stream. GSR_EINVAL when keys (with num_pairs > 0) or splat_pairs (with num_splats > 0) is asked for
 * and the bins carry none. */
gsr_status gsr_bins_copy(gsr_ctx* ctx, void* stream, const gsr_bins* bins, uint64_t* keys, uint32_t* vals,
                         uint32_t* ranges, uint32_t* splat_pairs);

/* The sort gsr_bin uses, on its own: a stable LSD radix sort by the low `key_bits` bits of 64-bit keys carrying
 * 32-bit values, 8 bits per pass; digits above key_bits are not looked at (a key with bits set above key_bits
 * sorts as if they were zero). The pass count is ceil(key_bits / 8): digits that the key range makes constant are
 * skipped, the same identity-pass argument as [C0 resident arena + C1 pass skip page, section 2 table, row "C1
 * radix pass skip"]. keys_in / vals_in / keys_out / vals_out: device [n]; in and out must not overlap.
 * Uses the context arena as scratch. Errors: GSR_EINVAL (null pointers with n > 0, key_bits 0 or > 64),
 * GSR_EOVERFLOW (n >= 2^32), GSR_ENOMEM, GSR_EHIP. */
gsr_status gsr_radix_sort(gsr_ctx* ctx, void* stream, const uint64_t* keys_in, const uint32_t* vals_in, uint64_t n,
                          uint32_t key_bits, uint64_t* keys_out, uint32_t* vals_out);

/* Number of 4-bit LSD passes that are not identity passes for keys (tile id << 32) | depth bits with tile ids
 * below num_tiles: min(16, 8 + ceil(bits(num_tiles - 1) / 4)). With digit_bits = 8 the same rule at 8-bit
 * digits: min(8, 4 + ceil(bits(num_tiles - 1) / 8)). [C0 resident arena + C1 pass skip page, section 2 table, row
 * "C1 radix pass skip"] Host only; returns 0 for digit_bits other than 4 or 8. */
uint32_t gsr_radix_pass_count(uint64_t num_tiles, uint32_t digit_bits);

/* Forward rasterization. For each pixel, walks its tile's pairs front to back with T = 1, C = 0:
 *   sigma = 0.5 (a dx^2 + c dy^2) + b dx dy, (dx, dy) = pixel centre - mean; skip if sigma < 0;
 *   alpha = min(0.999, o exp(-sigma)); skip if alpha < 1/255;
 *   T' = T (1 - alpha); if T' < 1e-4 the pixel stops here without compositing this splat;
 *   C += rgb (alpha T); T = T'; last = list position + 1.
 * exp(-sigma) is the correctly rounded fp32 value of e^-sigma (on every float sigma in [0, 5.55] it equals the
 * double-precision exp rounded to fp32; GSR_OPT_FORWARD_EXP selects the hardware exponential instead), and the
 * transmittance's operations are IEEE fp32 operations in the order written (no fused multiply-add), so results
 * match a plain fp32 evaluation of the definition. Splats with sigma >= 5.55 are skipped before the exponential,
 * which cannot change a result because o <= 1 makes their alpha at most e^-5.55 < 1/255. [A.9 f16 forward page,
 * implementation listing; W1 warp sparse skip + exp-skip page, summary and section 1 row "W1b"; rasterize
 * forward + adam kernel audit page, section 1 rows (a) and (b)]
 *   splats        device [n][9] float32 (the records the bins were built from; the result is defined for the
 *                 splats gsr_bin keeps - finite, a > 0, det > 0, 0 <= o <= 1 - whatever else the bins hold)
 *   bins          host struct of device views, tiles_x / tiles_y matching width / height; pairs whose value is
 *                 >= n are ignored, and ranges are clamped to [0, num_pairs]
 *   out_rgba      device [height][width][4] float32: (C.r, C.g, C.b, 1 - T_final)
 *   final_T       device [height][width] float32;  last_contrib  device [height][width] uint32 (0: none)
 * Errors: GSR_EINVAL (null pointers, size mismatch), GSR_EHIP. */
gsr_status gsr_render_forward(gsr_ctx* ctx, void* stream, const float* splats, uint32_t n, const gsr_bins* bins,
                              uint32_t width, uint32_t height, float* out_rgba, float* final_T,
                              uint32_t* last_contrib);

/* gsr_render_forward for callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, hosts that forbid allocation. The same results, bit for bit, and the same arguments and errors; it never
 * calls hipMalloc or hipFree (gsr_render_forward may grow the context's arena on its first call on a grid).
 * Its scratch - the tiles' launch order and the per-tile walk counts that rank the next call's order, 20 bytes per
 * tile - is a fixed array of 1.25 MiB in device memory, one copy per device, held until the process ends; images of
 * more than 65536 tiles (4096 x 4096 pixels) are refused with GSR_EINVAL. Every call on a device shares that
 * device's array and leaves its walk counts there for the next call (any contents give a valid order; the order
 * changes no result): calls that overlap on one device, on different streams or host threads, race. */
gsr_status gsr_render_forward_noalloc(gsr_ctx* ctx, void* stream, const float* splats, uint32_t n,
                                      const gsr_bins* bins, uint32_t width, uint32_t height, float* out_rgba,
                                      float* final_T, uint32_t* last_contrib);

/* Backward rasterization: dL/d(splat record) for the loss whose gradient with respect to out_rgba.rgb is v_out.rgb
 * (v_out.w is ignored). Each pixel replays its forward decisions up to last_contrib and, for each splat it
 * composited, with w = alpha T, mine = rgb w, after = C_final - acc - mine (acc = colour composited in front):
 *   d rgb += w g;  dL/dalpha = sum_ch g_ch (rgb_ch T - after_ch / (1 - alpha));
 *   only if o exp(-sigma) < 0.999 (alpha not clamped): d o += dL/dalpha exp(-sigma),
 *   dL/dsigma = -dL/dalpha o exp(-sigma), d(a, b, c) += dL/dsigma (dx^2 / 2, dx dy, dy^2 / 2),
 *   d(x, y) -= dL/dsigma (a dx + b dy, b dx + c dy).
 * Splats no pixel of a wavefront composites are skipped before any reduction; the per-pixel terms are summed
 * across the wavefront and the tile on chip and added to splats_grad with one atomic per (splat, tile, value).
 * [M3 per-splat backward page, section 1 rows "brush's actual structure" and "differences"; W1 warp sparse skip +
 * exp-skip page, section 1 row "W1a"]
 *   splats, bins, out_rgba, final_T, last_contrib: as produced by gsr_render_forward for the same inputs
 *   v_out         device [height][width][4] float32
 *   splats_grad   device [n][9] float32, overwritten (record order {x, y, a, b, c, r, g, b, o}); the summation
 *                 order across tiles is not fixed, so results may differ in the last bits between runs
 * Errors: GSR_EINVAL, GSR_EOVERFLOW (n * 9 >= 2^32), GSR_EHIP. */
gsr_status gsr_render_backward(gsr_ctx* ctx, void* stream, const float* splats, uint32_t n, const gsr_bins* bins,
                               uint32_t width, uint32_t height, const float* out_rgba, const float* final_T,
                               const uint32_t* last_contrib, const float* v_out, float* splats_grad);

/* One Adam parameter group: `count` float32 elements at device pointers param, grad, m, v, with its step size. */
typedef struct gsr_adam_group {
  float* param;
  const float* grad;
  float* m;
  float* v;
  uint64_t count;
  float lr;
} gsr_adam_group;

#define GSR_ADAM_MAX_GROUPS 8

/* One Adam step over up to GSR_ADAM_MAX_GROUPS groups in a single launch, element by element:
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2;  param -= lr (m / bc1) / (sqrt(v / bc2) + eps)
 * with the bias corrections bc1 = 1 - beta1^t and bc2 = 1 - beta2^t supplied by the caller. Each operation is one
 * IEEE fp32 operation in the order written (correctly rounded division and square root, no fused multiply-add).
 * [rasterize forward + adam kernel audit page, section 2 "(f)": 5 groups, 59 elements per splat, 28 B per element]
 *   groups     host array [n_groups]; groups with count 0 are allowed; arrays of different groups must not overlap
 * Errors: GSR_EINVAL (null pointers with count > 0, n_groups > GSR_ADAM_MAX_GROUPS, bc1 or bc2 not > 0), GSR_EHIP. */
gsr_status gsr_adam_step(gsr_ctx* ctx, void* stream, const gsr_adam_group* groups, uint32_t n_groups, float beta1,
                         float beta2, float eps, float bc1, float bc2);

/* Visible-only Adam: the step of gsr_adam_step for the splats that were binned in this view, and no change at all
 * (param, m and v keep their bits; the gradient is not read) for the others, whose moments dense Adam would decay
 * and whose parameters it would still move. Each group holds n splats' worth of elements, k = count / n consecutive
 * elements per splat (3, 3, 4, 1, 48 for the Gaussians' groups). Skipping the invisible splats' bytes is the only
 * saving left to a bandwidth-bound Adam; the result differs from dense Adam by design. [rasterize forward + adam
 * kernel audit page, section 2 "(h)": the visible-only skip, gsplat's sparse-gradient Adam]
 *   splat_pairs  device [n] uint32; splat i is visible when splat_pairs[i] != 0 (gsr_bins.splat_pairs of the
 *                view's bins, or any caller mask of that type)
 * Visible splats get exactly gsr_adam_step's bits.
 * Errors: as gsr_adam_step; GSR_EINVAL also when a group's count is not a multiple of n (or not 0 when n = 0), or
 * k > 1024, or splat_pairs is NULL with n > 0. */
gsr_status gsr_adam_step_visible(gsr_ctx* ctx, void* stream, const gsr_adam_group* groups, uint32_t n_groups,
                                 float beta1, float beta2, float eps, float bc1, float bc2,
                                 const uint32_t* splat_pairs, uint32_t n);

/* Pinhole camera of the projection. World point p has camera coordinates t = R p + tv; pixel coordinates are
 * (fx tx / tz + cx, fy ty / tz + cy) in the frame where pixel (px, py) has its centre at (px + 0.5, py + 0.5). */
typedef struct gsr_camera {
  float R[9];  /* world-to-camera rotation, row-major */
  float tv[3];
  float fx, fy, cx, cy;
  float near;  /* Gaussians with tz <= near (or a NaN tz) are culled */
} gsr_camera;

/* Projection of n 3D Gaussians to splat records and depths. The parameter groups are those of the pages' trainer
 * (means 3, log_scales 3, rot_quats 4, raw_opacities 1, sh_coeffs 16 x 3: SH degree 3, 59 floats per Gaussian;
 * M3 per-splat backward page, full-scale parity table; rasterize forward + adam kernel audit page, section 2 "(f)"),
 * and the record's opacity is the sigmoid of the raw opacity (W1 warp sparse skip + exp-skip page, section 1). The
 * pages print no projection formula; this is the pinhole EWA projection:
 *   t = R p + tv;  Sigma = Rq diag(exp(log_s))^2 Rq^T with Rq the rotation of the normalised quaternion (w, x, y, z);
 *   J = d(pixel mean)/dt = [[fx / tz, 0, -fx tx / tz^2], [0, fy / tz, -fy ty / tz^2]];
 *   Sigma' = J R Sigma R^T J^T + 0.3 I (a 0.3 px^2 low-pass); [[a, b], [b, c]] = Sigma'^-1;
 *   (x, y) = (fx tx / tz + cx, fy ty / tz + cy);  o = 1 / (1 + exp(-raw));  depth = tz;
 *   rgb = max(sum_k sh[k] Y_k(d) + 0.5, 0), d = (p - camera centre) / |p - camera centre|, Y_0..Y_15 the real
 *   spherical harmonics of degrees 0..3 (orthonormal, Condon-Shortley signs, ordered by degree, then m = -l..l).
 * A culled Gaussian gets the record 0 and depth 0, which gsr_bin skips. fp32 throughout; results agree with an
 * exact evaluation to about 1e-6 relative (the 2x2 determinant is a sum of squares, see project.hip).
 *   cam            host pointer
 *   means, log_scales  device [n][3];  quats device [n][4] (16-byte aligned);  raw_opacities device [n]
 *   sh             device [n][16][3] (coefficient-major, channel fastest; 16-byte aligned)
 *   splats         device [n][9] float32, written;  depths device [n] float32, written
 * Errors: GSR_EINVAL (null pointers, misalignment), GSR_EOVERFLOW (n * 48 >= 2^32), GSR_EHIP. */
gsr_status gsr_project_forward(gsr_ctx* ctx, void* stream, const gsr_camera* cam, uint32_t n, const float* means,
                               const float* log_scales, const float* quats, const float* raw_opacities,
                               const float* sh, float* splats, float* depths);

/* Backward pass of gsr_project_forward: given dL/d(record) for each Gaussian, the gradients of its five parameter
 * groups, by the chain rule through the same formulas (recomputed, nothing is cached between the two calls);
 * the clamp of a colour channel at 0 passes no gradient, and a culled Gaussian gets zero gradients.
 *   cam, n, means .. sh  as given to gsr_project_forward
 *   splats_grad    device [n][9] float32 (as written by gsr_render_backward)
 *   *_grad         device arrays shaped like their parameters (quats_grad and sh_grad 16-byte aligned), overwritten
 * Errors: GSR_EINVAL, GSR_EOVERFLOW, GSR_EHIP. */
gsr_status gsr_project_backward(gsr_ctx* ctx, void* stream, const gsr_camera* cam, uint32_t n, const float* means,
                                const float* log_scales, const float* quats, const float* raw_opacities,
                                const float* sh, const float* splats_grad, float* means_grad,
                                float* log_scales_grad, float* quats_grad, float* raw_opacities_grad,
                                float* sh_grad);

/* The training loss on the rendered image and its gradient, which is the v_out of gsr_render_backward:
 *   L = (1 - 0.2) mean|x - y| + 0.2 (1 - mean S),
 *   S = ((2 mx my + C1)(2 sxy + C2)) / ((mx^2 + my^2 + C1)(sx + sy + C2)),  C1 = 0.01^2,  C2 = 0.03^2,
 * per channel with mx = G * x, sx = G * x^2 - mx^2, sxy = G * (x y) - mx my, G * the correlation with the normalised
 * 11-tap Gaussian window (sigma 1.5) in each direction over the zero-padded image; means over the 3 W H values.
 * The pages name a fused L1 + SSIM loss and its backward (M3 per-splat backward page, the brush change it ports) and
 * the SSIM window sizes 7 and 11 (SSIM float4 finding); the constants and the weight 0.2 are the usual ones.
 * fp32 arithmetic; the loss adds per-tile fp64 partial sums in a fixed order (the same value on every run).
 *   out_rgba   device [height][width][4] float32 (x = its first three channels; 16-byte aligned)
 *   target     device [height][width][3] float32 (y)
 *   v_out      device [height][width][4] float32, written: dL/dx in .xyz, 0 in .w (16-byte aligned)
 *   loss       device [3] float32, written: L, mean|x - y|, mean S
 * Errors: GSR_EINVAL (null pointers, empty image, misalignment), GSR_ENOMEM, GSR_EHIP. */
gsr_status gsr_loss_l1_ssim(gsr_ctx* ctx, void* stream, uint32_t width, uint32_t height, const float* out_rgba,
                            const float* target, float* v_out, float* loss);

#ifdef __cplusplus
}
#endif

#endif /* GSR_H */
