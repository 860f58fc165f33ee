// Internal declarations shared by the library's translation units.
// Not part of the ABI: callers use include/shardconv.h only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/shardconv.h"

namespace st {

// Error reporting: a thread-local message plus the status code.
st_status fail(st_status s, const std::string& msg);
st_status ok();
st_status hip_check(hipError_t e, const char* what);
// Reports the launch status of the kernels just enqueued.
st_status launch_check(const char* what);
bool aligned16(const void* p);

// Geometry is held with three spatial axes; a 2D plan has a leading axis of
// extent 1, halo 0 and one shard.
constexpr int kAxes = 3;

struct Shard {
  int32_t grid[kAxes];
  int64_t off[kAxes];
  int64_t ext[kAxes];
  int64_t pad[kAxes];     // ext + 2*halo
  int64_t elems;          // N * prod(pad) * C
};

// One row-structured box copy of the halo exchange, in units of `vec`-byte
// words.  A box spans N x rows_d x rows_h rows of `upr` contiguous words.
struct HaloDesc {
  int32_t src;            // sending shard, -1 for a zero box
  int32_t dst;            // receiving shard
  int32_t rows_h;         // box extent along H
  int32_t rows_dh;        // rows per batch item = rows_d * rows_h
  int32_t upr;            // words per row
  int32_t pad0;
  // multiply-shift dividers by upr, rows_dh and rows_h: q = (n * m) >> p for
  // n < 2^31, with p = 31 + ceil(log2 d) and m = ceil(2^p / d)
  uint32_t m_upr, m_rdh, m_rh;
  int32_t p_upr, p_rdh, p_rh;
  int64_t units;          // words in the box: N * rows_dh * upr
  int64_t src_base, src_sn, src_sd, src_sh;   // word offsets/strides in the sender
  int64_t dst_base, dst_sn, dst_sd, dst_sh;   // word offsets/strides in the receiver
  int64_t msg_base;       // word offset in the message
  int64_t block_begin;    // first block of this box in a launch
};

struct PublicBox {        // st_halo_box in internal axis order
  int32_t src, dst;
  int32_t dir[kAxes];
  int64_t dst_lo[kAxes], src_lo[kAxes], ext[kAxes];
  int64_t msg_offset;
};

}  // namespace st

struct st_plan {
  int32_t ndim;
  int64_t batch;
  int64_t channels;
  st_dtype dtype;
  int32_t esize;
  int64_t spatial[st::kAxes];
  int32_t nshards[st::kAxes];
  int32_t halo[st::kAxes];
  std::vector<std::vector<int64_t>> sizes;   // per internal axis
  std::vector<st::Shard> shards;
  std::vector<st::PublicBox> boxes;          // sent boxes (message order), then zero boxes
  int64_t n_real = 0, n_zero = 0;
  int32_t vec = 16;                          // bytes per copy word
  int64_t msg_bytes = 0;
  std::vector<st::HaloDesc> descs;           // same order as boxes
  int64_t blocks_real = 0, blocks_all = 0;
  // device copy of `descs`, created on first use
  std::mutex dev_mu;
  st::HaloDesc* d_descs = nullptr;
  int dev_id = -1;
};

namespace st {
constexpr int kHaloThreads = 256;
constexpr int kHaloWordsPerThread = 2;
constexpr int64_t kHaloWordsPerBlock = kHaloThreads * kHaloWordsPerThread;

// Every kernel receives its per-shard table by value, sized for
// ST_MAX_SHARDS whatever the plan's shard count, so each argument struct has
// one fixed size, checked at compile time against this bound.  The largest,
// the weight gradient's (~8.2 KB), is what every launch of that kernel
// passes, at any shard count, so the GPU tests exercise the full sizes.
constexpr size_t kMaxKernargBytes = 12 * 1024;

// Weights [B][A][taps] (a_major false: [Cout][Cin], PyTorch's conv order) or
// [A][B][taps] (a_major true) in `dtype` -> fp32 [taps][A][B]; the same
// launch zeroes clr[0, nclr).  (strided.hip)
st_status pack_tab_launch(const void* weight, st_dtype dtype, float* out, int a_ch, int b_ch, int taps, bool a_major,
                          uint32_t* clr, int nclr, hipStream_t st, const char* who);
// The stride-1 'same' conv of bf16 shards on the matrix cores (strided.hip's
// implicit GEMM at stride 1) for shapes without a tuned kernel: Cin % 16 ==
// 0, Cout % 16 == 0 and one channel block of weights within LDS.  Weights
// fp32 [taps][Cin][Cout] (bf16 values); y unpadded channels-last fp32.
bool sx_same_fits(int ndim, int cin, int cout, int ksize);
st_status sx_same_conv(const st_plan* in_plan, const void* const* in_bufs, const float* w_tco, const float* bias,
                       int cout, int ksize, float* const* y_bufs, hipStream_t st);

// Uploads the descriptor table on first use (on the current device).
st_status plan_device_table(st_plan* p, hipStream_t stream);
// Public axis a of an ndim plan maps to internal axis a + (3 - ndim).
inline int axis_of(const st_plan* p, int a) { return a + (kAxes - p->ndim); }
}  // namespace st
