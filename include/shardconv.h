/*
 * shardconv.h - C-ABI of the halo-sharded conv + GroupNorm library (gfx950).
 *
 * One GPU's share of a domain-sharded spatial layer, after "Technical summary:
 * ShardTensor - domain parallelism for scientific machine learning"
 * (gist.science paper 2605.11111):
 *   - section 2, "Design principles": a batch-1 volume is split along its
 *     spatial axes into chunks whose per-chunk shapes ("sharding shapes") may
 *     be uneven;
 *   - section 2, "Implementation details", "Communication": neighbouring
 *     cells are exchanged as halos and statistics are combined with
 *     collectives so that convolution and normalisation give the unsharded
 *     result.
 * On one GPU every shard is its own HBM buffer: the halo exchange is a pack
 * into a message buffer and an unpack into the neighbours' margins, and the
 * statistics combine is an on-device reduction over the per-shard partials.
 *
 * Conventions for every entry point
 *   - Buffers are device pointers owned by the caller; the library never frees
 *     or retains them.  The library owns only plans (st_plan_destroy).
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream) with no host synchronisation.  Results are defined once the
 *     stream reaches that point.
 *   - Every call returns an st_status.  Nothing throws or aborts across the
 *     ABI.  On failure st_last_error() returns a thread-local message; all
 *     argument, shape and alignment checks run on the host before any launch,
 *     so a failed check enqueues nothing.  Launch failures map to ST_ERR_HIP.
 *   - Layout: channels-last.  A shard buffer holds [N][Dp][Hp][Wp][C] (3D) or
 *     [N][Hp][Wp][C] (2D), where each padded extent is the shard's extent plus
 *     2*halo on that axis.  Every spatial axis is padded, also where the shard
 *     touches the global boundary (those margins hold zeros after
 *     st_halo_unpack with zero_global_margins != 0).
 *   - Device pointers must be 16-byte aligned.
 *   - Shards are numbered row-major over the shard grid (axis 0 outermost);
 *     along each axis the first size is the lowest-index shard.
 */
#ifndef SHARDCONV_H
#define SHARDCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ST_MAX_SHARDS 64   /* shards per plan */
#define ST_MAX_NDIM 3

typedef enum st_status {
  ST_OK = 0,
  ST_ERR_INVALID_ARG = 1,      /* null pointer, bad enum, negative size */
  ST_ERR_BAD_SHAPE = 2,        /* sizes that do not add up or plans that do not match */
  ST_ERR_SHARD_TOO_SMALL = 3,  /* a shard thinner than the halo along a split axis */
  ST_ERR_UNSUPPORTED = 4,      /* ndim not 2/3, even kernel, too many shards, ... */
  ST_ERR_WORKSPACE = 5,        /* workspace missing or too small */
  ST_ERR_HIP = 6,              /* a HIP runtime call or kernel launch failed */
  ST_ERR_ALIGNMENT = 7         /* a device pointer is not 16-byte aligned */
} st_status;

typedef enum st_dtype { ST_F32 = 0, ST_BF16 = 1 } st_dtype;

typedef struct st_plan st_plan; /* opaque, library-owned */

typedef struct st_shard_info {
  int32_t index;          /* linear shard index */
  int32_t grid[3];        /* coordinate in the shard grid per spatial axis (unused axes: 0) */
  int64_t offset[3];      /* global start of the interior per spatial axis */
  int64_t extent[3];      /* interior extent per spatial axis (unused axes: 1) */
  int64_t padded[3];      /* extent + 2*halo per spatial axis (unused axes: 1) */
  int64_t elems;          /* elements of the padded buffer: N * prod(padded) * C */
  int64_t bytes;          /* elems * element size */
} st_shard_info;

typedef struct st_halo_box {
  int32_t src_shard;      /* shard whose interior cells are sent; -1 for a zero box */
  int32_t dst_shard;      /* shard whose margin receives them */
  int32_t dir[3];         /* direction from src to dst (from dst outwards for zero boxes) */
  int64_t dst_lo[3];      /* box origin in the receiver's padded coordinates */
  int64_t src_lo[3];      /* box origin in the sender's padded coordinates (zero box: unused) */
  int64_t ext[3];         /* box extent per spatial axis */
  int64_t msg_offset;     /* byte offset of the box in the message (zero box: -1) */
} st_halo_box;

/* ------------------------------------------------------------------ misc */

const char* st_version(void);
/* Message of the last failed call on this thread ("" if none). */
const char* st_last_error(void);
const char* st_status_string(st_status s);

/* ------------------------------------------------------------ planning */

/*
 * st_plan_shards - sharding shapes and halo geometry (host only, no GPU call).
 *
 * Section 2 ("Design principles") of the ShardTensor summary: a per-chunk
 * local shape along each sharded axis, allowing uneven chunks.
 *
 *   ndim              2 or 3 spatial axes (else ST_ERR_UNSUPPORTED)
 *   batch, channels   N >= 1 and C >= 1
 *   spatial[ndim]     global extents, axis 0 outermost ((H, W) or (D, H, W))
 *   nshards_per_axis[ndim]  number of shards along each axis (>= 1); their
 *                     product is at most ST_MAX_SHARDS
 *   sizes_concat      the per-axis shard sizes concatenated: axis 0's
 *                     nshards_per_axis[0] sizes, then axis 1's, ...; each
 *                     axis must sum to spatial[axis]
 *   halo_per_axis[ndim]  margin width h per axis (>= 0); a conv with odd
 *                     kernel k needs h >= k/2.  Along an axis with more than
 *                     one shard every shard must be at least h thick
 *                     (ST_ERR_SHARD_TOO_SMALL)
 *   dtype             element type of the shard buffers
 *   out               receives the plan; release it with st_plan_destroy
 *
 * The plan enumerates, for every shard and every neighbour direction in
 * {-1,0,1}^ndim \ {0}, either a halo box (the neighbour exists: its interior
 * cells are sent) or a zero box (global face: the margin is zero padding).
 * Message layout: boxes ordered by sending shard, then by direction
 * (lexicographic, -1 < 0 < 1), each box channels-last and starting at a
 * 16-byte-aligned byte offset.
 */
st_status st_plan_shards(int32_t ndim, int64_t batch, int64_t channels, const int64_t* spatial,
                         const int32_t* nshards_per_axis, const int64_t* sizes_concat,
                         const int32_t* halo_per_axis, st_dtype dtype, st_plan** out);

/* Frees the plan and its device descriptor table (if one was uploaded). */
st_status st_plan_destroy(st_plan* plan);

/*
 * st_plan_upload - put the plan's halo descriptor table on the current device
 * now (one allocation owned by the plan, filled on `stream`; returns after
 * the stream has drained).  The halo calls do this themselves on first use,
 * except inside a HIP graph capture, where a plan not uploaded yet makes them
 * fail with ST_ERR_UNSUPPORTED and enqueue nothing: call this before
 * capturing.  Repeated calls on the same device do nothing; on another
 * device: ST_ERR_INVALID_ARG.
 */
st_status st_plan_upload(st_plan* plan, void* stream);

/* Plan queries; return -1 for a null plan. */
int64_t st_plan_num_shards(const st_plan* plan);
int64_t st_plan_msg_bytes(const st_plan* plan);
int64_t st_plan_num_halo_boxes(const st_plan* plan);  /* boxes sent */
int64_t st_plan_num_zero_boxes(const st_plan* plan);  /* global-face margins */
st_status st_plan_shard_info(const st_plan* plan, int32_t shard, st_shard_info* out);
/* i in [0, halo boxes): sent boxes in message order; then the zero boxes. */
st_status st_plan_halo_box(const st_plan* plan, int32_t i, st_halo_box* out);

/* ---------------------------------------------------------- halo exchange */

/*
 * st_halo_pack - copy every sent box out of its shard's interior into `msg`.
 * Section 2, "Implementation details", "Communication" (halo exchange: the
 * cells next to a chunk's boundary are fetched from the adjacent chunk).
 *
 *   shard_bufs[num_shards]  padded shard buffers (read)
 *   msg                      st_plan_msg_bytes(plan) bytes (written; gaps
 *                            between boxes are not touched)
 * Raw bit copy.  The first device call on a plan uploads its descriptor table
 * (one small allocation owned by the plan, on the current device).
 */
st_status st_halo_pack(st_plan* plan, const void* const* shard_bufs, void* msg, void* stream);

/*
 * st_halo_unpack - copy every box of `msg` into the receiving shard's margin;
 * with zero_global_margins != 0 also write zeros into the margins on the
 * global faces (the conv's zero padding).  Same section as st_halo_pack.
 *   msg                      as written by st_halo_pack (read)
 *   shard_bufs[num_shards]  padded shard buffers (margins written, interiors
 *                            untouched)
 */
st_status st_halo_unpack(st_plan* plan, const void* msg, void* const* shard_bufs,
                         int32_t zero_global_margins, void* stream);

/*
 * st_halo_exchange - st_halo_pack followed by st_halo_unpack, fused into one
 * copy for shards that share one device: every sent box goes from the
 * sender's interior straight into the receiver's margin, with no message
 * buffer (half the bytes of the two-copy form).  Same section as
 * st_halo_pack; the same bits land in every margin.
 *   shard_bufs[num_shards]  padded shard buffers: interiors read, margins
 *                            written (with zero_global_margins != 0 also the
 *                            global-face margins, as zeros)
 * Every shard buffer must be a distinct allocation (no two shards overlap).
 */
st_status st_halo_exchange(st_plan* plan, void* const* shard_bufs, int32_t zero_global_margins,
                           void* stream);

/* ------------------------------------------------------------------ conv */

/*
 * Packed weights, for st_conv_sharded_packed.  Weights are given as
 * [Cout][Cin][k]^ndim (PyTorch's logical order) in `dtype` and repacked into
 * the layout the kernel for that shape reads.  st_conv_weight_bytes returns 0
 * for unsupported arguments.  st_conv_sharded does this packing itself, into
 * its workspace, on every call.
 */
size_t st_conv_weight_bytes(int32_t ndim, int32_t cin, int32_t cout, int32_t ksize, st_dtype dtype);
st_status st_conv_pack_weights(int32_t ndim, int32_t cin, int32_t cout, int32_t ksize,
                               st_dtype dtype, const void* weight, void* packed, void* stream);

/*
 * st_conv_dgrad_weights - the weights of the input-gradient convolution.
 * Training at native resolution needs the backward pass ("Technical
 * summary: ShardTensor", section 1 "Problem statement"; section 4 "Results
 * and benchmarks", the ViT and StormScope training runs).  For the 'same',
 * stride-1 cross-correlation y = conv(x, w), the gradient with respect to x is
 * dx = conv(dy, w') with w'[c][o][t] = w[o][c][flip(t)] (channels swapped,
 * every tap axis reversed), so the sharded input gradient is: exchange the
 * halos of dy, then st_conv_sharded with cin' = Cout, cout' = Cin and
 * weight w' (or st_conv_sharded_packed with w' packed by
 * st_conv_pack_weights).
 *   weight   [Cout][Cin][k]^ndim in `dtype` (read)
 *   out      [Cin][Cout][k]^ndim in `dtype` (written; must not alias weight)
 * Pure bit permutation.  Errors: ST_ERR_UNSUPPORTED (ndim, even k, dtype),
 * ST_ERR_INVALID_ARG (NULL or aliased pointers).
 */
st_status st_conv_dgrad_weights(int32_t ndim, int32_t cin, int32_t cout, int32_t ksize, st_dtype dtype,
                                const void* weight, void* out, void* stream);

/*
 * st_conv_sharded - per-shard convolution on the halo-padded chunks.
 * Section 2, "Implementation details", "Communication": with the halo in
 * place every shard's output equals the matching slice of the unsharded
 * convolution.
 *
 * Cross-correlation, stride 1, dilation 1, odd cubic kernel `ksize`, zero
 * padding ksize/2 supplied by the shard margins:
 *   y[n, i, o] = bias[o] + sum_t sum_c W[o, c, t] * x[n, i + t - ksize/2, c]
 *
 *   in_plan, in_bufs   padded input shards, C = Cin, halo >= ksize/2 per
 *                      spatial axis (read; only cells within ksize/2 of an
 *                      interior are touched)
 *   weight             [Cout][Cin][ksize]^ndim in in_plan's dtype (PyTorch's
 *                      order; read)
 *   bias_or_null       Cout floats or NULL (zero bias)
 *   y_bufs             fp32 outputs, one per shard: unpadded channels-last
 *                      [N][extent...][Cout] over that shard's interior
 *                      (written)
 *   ymax_or_null       if not NULL: [N][groups] uint32 receiving the bit
 *                      pattern of max |y| per (n, group) over all shards
 *                      (groups: contiguous blocks of Cout/groups channels)
 *   workspace          >= st_conv_workspace_bytes(in_plan, cout, ksize)
 *                      bytes, 16-byte aligned: the weights packed for the
 *                      kernel that runs this shape (overwritten each call)
 * bf16 operands accumulate in fp32 on the matrix cores; fp32 operands use
 * fp32 FMA.  Each output's accumulation order depends only on its kernel
 * taps, so a shard's output is bitwise independent of the shard plan.
 * Errors: ST_ERR_UNSUPPORTED (even ksize, unsupported dtype), ST_ERR_BAD_SHAPE
 * (halo narrower than ksize/2), ST_ERR_WORKSPACE, ST_ERR_ALIGNMENT,
 * ST_ERR_INVALID_ARG (NULL pointers, groups not dividing Cout), ST_ERR_HIP.
 */
size_t st_conv_workspace_bytes(const st_plan* in_plan, int32_t cout, int32_t ksize);
st_status st_conv_sharded(const st_plan* in_plan, const void* const* in_bufs, const void* weight,
                          const float* bias_or_null, int32_t cout, int32_t ksize, float* const* y_bufs,
                          uint32_t* ymax_or_null, int32_t groups, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * st_conv_sharded_packed - st_conv_sharded from weights packed beforehand by
 * st_conv_pack_weights (same ndim, Cin, Cout, ksize and dtype), for callers
 * that keep one set of weights over many calls; no workspace.  Same
 * passage, arguments, outputs and errors as st_conv_sharded.
 */
st_status st_conv_sharded_packed(const st_plan* in_plan, const void* const* in_bufs, const void* packed_weight,
                                 const float* bias_or_null, int32_t cout, int32_t ksize, float* const* y_bufs,
                                 uint32_t* ymax_or_null, int32_t groups, void* stream);

/*
 * st_conv_wgrad - weight gradient of st_conv_sharded, summed over all shards.
 * The weight half of the backward pass (same passages as
 * st_conv_dgrad_weights); every shard contributes a partial sum from its own
 * halo-padded input, and the partials are reduced in a fixed order (the
 * all-reduce of section 2, "Implementation details", "Communication"):
 *   dw[o, c, t] = sum_n sum_i dy[n, i, o] * x[n, i + t - ksize/2, c]
 *
 *   x_plan, x_bufs     the forward call's padded inputs (halo >= ksize/2 per
 *                      axis, margins filled by the halo exchange) (read)
 *   dy_plan, dy_bufs   gradient at y: same ndim, batch, dtype and shard sizes,
 *                      C = Cout, any halo (only interiors are read)
 *   dweight            [Cout][Cin][ksize]^ndim fp32 (written)
 *   workspace          >= st_conv_wgrad_workspace_bytes(x_plan, cout, ksize)
 *                      bytes: per-partition partial sums
 * bf16 operands run on the matrix cores (fp32 accumulation) for the shapes
 * with a tuned instance, every other shape and fp32 on fp32 FMA.  The
 * result does not depend on timing or the device, only on the shard plan.
 */
size_t st_conv_wgrad_workspace_bytes(const st_plan* x_plan, int32_t cout, int32_t ksize);
st_status st_conv_wgrad(const st_plan* x_plan, const void* const* x_bufs, const st_plan* dy_plan,
                        const void* const* dy_bufs, int32_t ksize, float* dweight, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ------------------------------------------------------ shape-changing ops */

/*
 * st_plan_pooled - the output plan of a 'valid' pooling of in_plan's shards.
 * Section 2, "Design principles" of the ShardTensor summary: each local chunk
 * carries its own shape ("sharding shapes"), so an op that changes shapes
 * derives the output chunks from the input ones.  Window ksize, stride on
 * every spatial axis; output j along an axis of extent n covers inputs
 * [j*stride, j*stride + ksize), j = 0 .. (n - ksize) / stride, and belongs to
 * the shard whose interior holds j*stride.
 *   out_halo_or_null   ndim halo widths of the output plan (NULL: 0)
 *   out_dtype          element type of the output shards
 *   out                receives the plan (release with st_plan_destroy)
 * Errors: ST_ERR_BAD_SHAPE (window larger than the volume),
 * ST_ERR_SHARD_TOO_SMALL (a shard holds no window start: it would own no
 * output), ST_ERR_INVALID_ARG.
 */
st_status st_plan_pooled(const st_plan* in_plan, int32_t ksize, int32_t stride, const int32_t* out_halo_or_null,
                         st_dtype out_dtype, st_plan** out);

/*
 * st_pool_sharded - 'valid' pooling of every shard from its halo-padded chunk.
 * Same passage as st_plan_pooled.
 *   in_plan, in_bufs   input shards after their halo exchange; halo >= ksize - 1
 *                      along every split axis (ST_ERR_BAD_SHAPE otherwise)
 *   mode               0: average of the ksize^d window, 1: maximum
 *   out_plan, out_bufs the plan st_plan_pooled returned for (in_plan, ksize,
 *                      stride) (any output halo; only interiors are written)
 *                      and its shards; dtype the input's or ST_F32
 * Windows are read in lexicographic order and accumulated in fp32 (bf16
 * outputs rounded to nearest even), so an output's bits do not depend on the
 * shard plan.
 */
st_status st_pool_sharded(const st_plan* in_plan, const void* const* in_bufs, int32_t ksize, int32_t stride,
                          int32_t mode, const st_plan* out_plan, void* const* out_bufs, void* stream);

/*
 * st_plan_strided - the output plan of a strided 'same'-padded convolution of
 * in_plan's shards (the downsampling conv).  Same passage as st_plan_pooled.
 * Odd window ksize, padding ksize/2, stride on every spatial axis: output j
 * along an axis of extent n reads inputs [j*stride - ksize/2, j*stride +
 * ksize/2], j = 0 .. (n + 2*(ksize/2) - ksize) / stride, and belongs to the
 * shard whose interior holds the window's centre j*stride.
 *   cout               channels of the output plan
 *   out_halo_or_null   ndim halo widths of the output plan (NULL: 0)
 *   out                receives the fp32 output plan (st_plan_destroy)
 * Errors: ST_ERR_SHARD_TOO_SMALL (a shard holds no window centre: it would
 * own no output), ST_ERR_BAD_SHAPE, ST_ERR_UNSUPPORTED (even ksize),
 * ST_ERR_INVALID_ARG.
 */
st_status st_plan_strided(const st_plan* in_plan, int32_t ksize, int32_t stride, int32_t cout,
                          const int32_t* out_halo_or_null, st_plan** out);

/*
 * st_conv_strided_sharded - strided convolution of every shard from its
 * halo-padded chunk (after the halo exchange; halo >= ksize/2 per split axis):
 *   y[n, j, o] = bias[o] + sum_t sum_c W[o, c, t] * x[n, j*stride + t - ksize/2, c]
 *   in_plan, in_bufs   padded input shards (fp32 or bf16 operands; read)
 *   weight             W as [Cout][Cin][ksize]^ndim in in_plan's dtype
 *                      (PyTorch's conv order; read)
 *   bias_or_null       Cout floats or NULL
 *   out_plan, out_bufs the plan st_plan_strided returned for (in_plan, ksize,
 *                      stride, Cout) and its fp32 shards (only interiors written)
 *   workspace          >= st_conv_strided_workspace_bytes(in_plan, Cout,
 *                      ksize) bytes, 16-byte aligned: the weights widened to
 *                      fp32 and reordered [taps][Cin][Cout] (overwritten)
 * bf16 input shards with Cin % 16 == 0, Cout % 16 == 0 and the weights of
 * a 64- (or 32-) channel output block within 160 KiB run on the matrix cores
 * (bf16 products, fp32 accumulation); every other case on fp32 FMA.  Either
 * way each output sums bias, then taps lexicographic, input channels
 * ascending, in an order fixed by the layer shape, so its bits do not depend
 * on the shard plan.
 * Errors: ST_ERR_BAD_SHAPE (out_plan is not the strided plan, halo too small),
 * ST_ERR_WORKSPACE, ST_ERR_ALIGNMENT, ST_ERR_INVALID_ARG, ST_ERR_UNSUPPORTED.
 */
size_t st_conv_strided_workspace_bytes(const st_plan* in_plan, int32_t cout, int32_t ksize);
st_status st_conv_strided_sharded(const st_plan* in_plan, const void* const* in_bufs, const void* weight,
                                  const float* bias_or_null, int32_t ksize, int32_t stride,
                                  const st_plan* out_plan, float* const* out_bufs, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * st_plan_transposed - the output plan of a transposed (upsampling)
 * convolution of in_plan's shards, the adjoint of the strided convolution.
 * Same passage as st_plan_pooled: input cell i scatters onto outputs
 * i*stride + t - ksize/2, the output has stride times the input's extent on
 * every spatial axis, and the shard with interior [a, a + e) owns outputs
 * [a*stride, (a + e)*stride).
 *   stride             1 .. 8
 *   cout               channels of the output plan
 *   out_halo_or_null   ndim halo widths of the output plan (NULL: 0)
 *   out                receives the fp32 output plan (st_plan_destroy)
 * Errors: ST_ERR_UNSUPPORTED (even ksize), ST_ERR_INVALID_ARG.
 */
st_status st_plan_transposed(const st_plan* in_plan, int32_t ksize, int32_t stride, int32_t cout,
                             const int32_t* out_halo_or_null, st_plan** out);

/*
 * st_conv_transposed_sharded - transposed convolution of every shard from its
 * halo-padded chunk (after the halo exchange).  Output q*stride + r reads the
 * input cells q + (r + ksize/2 - t)/stride over the taps t = r + ksize/2
 * (mod stride); the halo must cover that reach on both sides (ksize/2 always
 * does; stride 2 with ksize 3 or 5 needs 1):
 *   x[n, j, c] = bias[c] + sum over (i, t) with i*stride + t - ksize/2 = j of
 *                sum_o W[o, c, t] * y[n, i, o]
 * so that <conv_strided(x, W), y> = <x, conv_transposed(y, W)> without bias.
 *   in_plan, in_bufs   padded input shards y (fp32 or bf16 operands; read),
 *                      in_plan channels = the strided conv's output channels
 *   weight             W as [Cin][Cout][ksize]^ndim in in_plan's dtype, Cin =
 *                      in_plan channels (PyTorch's conv_transpose order: the
 *                      same array as the matching strided conv's weight; read)
 *   bias_or_null       Cout floats or NULL
 *   out_plan, out_bufs the plan st_plan_transposed returned for (in_plan,
 *                      ksize, stride, Cout) and its fp32 shards (only
 *                      interiors written)
 *   workspace          >= st_conv_transposed_workspace_bytes(in_plan, Cout,
 *                      ksize) bytes, 16-byte aligned: the weights widened to
 *                      fp32 and reordered [taps][Cin][Cout] (overwritten)
 * Matrix cores or fp32 FMA under the same conditions as the strided conv;
 * each output sums bias, then its phase's taps lexicographic, input channels
 * ascending, so its bits do not depend on the shard plan.
 * Errors: ST_ERR_BAD_SHAPE (out_plan is not the transposed plan, halo too
 * small), ST_ERR_WORKSPACE, ST_ERR_ALIGNMENT, ST_ERR_INVALID_ARG,
 * ST_ERR_UNSUPPORTED.
 */
size_t st_conv_transposed_workspace_bytes(const st_plan* in_plan, int32_t cout, int32_t ksize);
st_status st_conv_transposed_sharded(const st_plan* in_plan, const void* const* in_bufs, const void* weight,
                                     const float* bias_or_null, int32_t ksize, int32_t stride,
                                     const st_plan* out_plan, float* const* out_bufs, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------- GroupNorm */

/*
 * Workspace of st_groupnorm_sharded.  Leading regions (byte offsets from
 * st_groupnorm_workspace_layout):
 *   partials  [S][N][G][2] double: per-shard (sum q1, sum q2), exact integers
 *   stats     [N][G][2]   float:  (mean, rstd) after the combine
 *   scales    [N][G][2]   int32:  fixed-point exponents (e1, e2)
 *   ymax      [N][G]      uint32: max |y| when the caller passes no ymax
 */
typedef struct st_gn_layout {
  size_t partials_offset, stats_offset, scales_offset, ymax_offset, chan_offset, total_bytes;
} st_gn_layout;
size_t st_groupnorm_workspace_bytes(const st_plan* y_plan, int32_t groups);
st_status st_groupnorm_workspace_layout(const st_plan* y_plan, int32_t groups, st_gn_layout* out);

/*
 * st_groupnorm_sharded - split-statistics GroupNorm over all shards.
 * Section 2, "Implementation details", "Communication": normalisation stays
 * consistent with the unsharded model by combining per-chunk statistics with
 * a collective.  GroupNorm itself is not defined on the pages; this is the
 * standard one: contiguous channel groups, biased variance, eps inside the
 * square root, per-channel affine:
 *   z = (y - mean_g) / sqrt(var_g + eps) * gamma_c + beta_c
 *
 * Statistics are exact: every y contributes q1 = rint(y * 2^e1) and
 * q2 = rint(y^2 * 2^e2), with e1, e2 chosen from the global max |y| and the
 * element count so that every partial sum is an integer below 2^53; sums of
 * such integers do not depend on their order, so the per-shard partials and
 * their combine give the same bits for any shard plan.  mean, the biased
 * variance and rstd are then formed in fp64 and rounded once to fp32.
 *
 *   y_plan, y_bufs      fp32 conv outputs (halo-0 plan, C = Cout)
 *   ymax_or_null        max |y| bits from st_conv_sharded, or NULL to have
 *                       this call compute it (one more read of y)
 *   groups              divides C
 *   eps                 added to the variance
 *   gamma/beta_or_null  C floats or NULL (1 and 0)
 *   z_bufs              fp32 outputs, same layout as y; may alias y_bufs
 *   workspace           >= st_groupnorm_workspace_bytes(y_plan, groups) bytes
 */
st_status st_groupnorm_sharded(const st_plan* y_plan, const float* const* y_bufs,
                               const uint32_t* ymax_or_null, int32_t groups, float eps,
                               const float* gamma_or_null, const float* beta_or_null,
                               float* const* z_bufs, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * st_groupnorm_sharded_noalloc - st_groupnorm_sharded for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (without the
 * workspace), semantics and output bits as st_groupnorm_sharded.  The
 * workspace is a static device array of ST_GN_NOALLOC_SCRATCH_BYTES that each
 * GPU the library runs on holds until the process ends; the call makes no
 * hipMalloc, hipFree or other allocation.  The first call on a device looks
 * up that device's scratch address once.
 * Errors: those of st_groupnorm_sharded, and ST_ERR_WORKSPACE (returned
 * before any GPU call) when st_groupnorm_workspace_bytes(y_plan, groups)
 * exceeds ST_GN_NOALLOC_SCRATCH_BYTES.
 * Every call on one GPU uses that GPU's one scratch array, which keeps the
 * last call's contents (the partial sums are cleared at the start of each
 * call): calls that overlap on one GPU (several streams or host threads)
 * race, and the caller must serialise them.
 */
#define ST_GN_NOALLOC_SCRATCH_BYTES (1u << 20)
st_status st_groupnorm_sharded_noalloc(const st_plan* y_plan, const float* const* y_bufs,
                                       const uint32_t* ymax_or_null, int32_t groups, float eps,
                                       const float* gamma_or_null, const float* beta_or_null,
                                       float* const* z_bufs, void* stream);

/*
 * The three steps of st_groupnorm_sharded as separate calls, in this order
 * on one stream (same plan, groups and workspace).  Between partials and
 * combine is where a multi-device run would all-reduce the per-shard
 * partials (section 2, "Implementation details", "Communication").
 *
 * st_groupnorm_partials  clears the partials, computes max |y| into the
 *                        workspace when ymax_or_null is NULL, then writes
 *                        the per-shard exact (sum q1, sum q2) and the
 *                        exponents (e1, e2) into the workspace.
 * st_groupnorm_combine   sums the partials over shards and writes (mean,
 *                        rstd) per (n, group) and the per-channel
 *                        (mean, rstd*gamma, beta) the apply reads.
 * st_groupnorm_apply     z = (y - mean) * rstd * gamma + beta; z may alias y.
 *
 * st_groupnorm_combine_apply does combine and apply in one call (arguments
 * of both; same outputs and bits, including the (mean, rstd) written to the
 * workspace).  When every workgroup of the apply can form its channels'
 * coefficients itself (the apply's per-lane coefficient layout: 1024 (C % 4
 * == 0) or 256 values per workgroup pass, a multiple of C) and N * groups
 * <= 256, the combine runs in the apply kernel's prologue and the call is
 * one launch; otherwise it launches both kernels.  st_groupnorm_sharded is
 * st_groupnorm_partials followed by this call.
 */
st_status st_groupnorm_partials(const st_plan* y_plan, const float* const* y_bufs,
                                const uint32_t* ymax_or_null, int32_t groups, void* workspace,
                                size_t workspace_bytes, void* stream);
st_status st_groupnorm_combine(const st_plan* y_plan, int32_t groups, float eps,
                               const float* gamma_or_null, const float* beta_or_null,
                               void* workspace, size_t workspace_bytes, void* stream);
st_status st_groupnorm_apply(const st_plan* y_plan, const float* const* y_bufs, int32_t groups,
                             float* const* z_bufs, void* workspace, size_t workspace_bytes,
                             void* stream);
st_status st_groupnorm_combine_apply(const st_plan* y_plan, const float* const* y_bufs, int32_t groups,
                                     float eps, const float* gamma_or_null, const float* beta_or_null,
                                     float* const* z_bufs, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * st_groupnorm_backward - gradients of st_groupnorm_sharded for an upstream
 * gradient dz: dy (the gradient at the conv output y), dgamma and dbeta.
 * Training at native resolution needs the backward pass ("Technical summary:
 * ShardTensor", section 1 "Problem statement"; section 4 "Results and
 * benchmarks", the training runs); like the forward statistics, the two
 * per-group reductions of the backward pass are combined over all shards
 * (section 2, "Implementation details", "Communication").  Per (n, group),
 * with r = rstd, yhat = (y - mean) * r and g = gamma_c * dz:
 *   dy     = r * (g - mean_group(g) - yhat * mean_group(g * yhat))
 *   dgamma = sum over n and positions of dz * yhat   (per channel)
 *   dbeta  = sum over n and positions of dz          (per channel)
 * The per-(n, channel) sums of dz and dz * yhat are exact fixed-point sums
 * (scaled by max |dz| and a bound on |yhat| from the forward pass), so dy,
 * dgamma and dbeta are the same bits for every shard plan.
 *
 *   y_plan, y_bufs     the forward call's plan and input y (read)
 *   dz_bufs            upstream gradient, same layout as y (read)
 *   ymax_or_null       the ymax pointer the forward call got (NULL: the forward
 *                      computed it into its workspace)
 *   dzmax_or_null      [N][groups] bits of max |dz| per (n, group), e.g. from
 *                      st_conv_sharded's fused max; NULL: computed here (one
 *                      more read of dz)
 *   groups, gamma_or_null   as in the forward call
 *   fwd_workspace      the forward call's workspace, holding its (mean, rstd)
 *                      (read; must not have been reused since)
 *   dy_plan_or_null    NULL: dy_bufs are fp32 in y's layout (may alias dz_bufs or
 *                      y_bufs).  Else the layout dy is written in, e.g. the
 *                      padded bf16 plan the input-gradient conv reads: same
 *                      ndim, batch, channels and shard sizes as y_plan, any
 *                      halo, ST_F32 or ST_BF16 (rounded to nearest even; C
 *                      divisible by 4); only interiors are written and dy must
 *                      not alias y or dz
 *   dy_bufs            dy output shards
 *   dgamma_or_null, dbeta_or_null   C floats each, or NULL (not computed)
 *   workspace          >= st_groupnorm_backward_workspace_bytes(y_plan, groups)
 *                      bytes, distinct from fwd_workspace
 * The forward variance must be finite and var + eps > 0.
 */
size_t st_groupnorm_backward_workspace_bytes(const st_plan* y_plan, int32_t groups);
st_status st_groupnorm_backward(const st_plan* y_plan, const float* const* y_bufs, const float* const* dz_bufs,
                                const uint32_t* ymax_or_null, const uint32_t* dzmax_or_null, int32_t groups,
                                const float* gamma_or_null, const void* fwd_workspace,
                                size_t fwd_workspace_bytes, const st_plan* dy_plan_or_null, void* const* dy_bufs,
                                float* dgamma_or_null, float* dbeta_or_null, void* workspace, size_t workspace_bytes,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SHARDCONV_H */
