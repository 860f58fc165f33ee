// Per-shard convolution on halo-padded chunks (one grouped launch).
//
// "Technical summary: ShardTensor - domain parallelism for scientific machine
// learning", section 2, "Implementation details", "Communication": once the
// halo is in place a shard's convolution output equals the matching slice of
// the unsharded one.  The pages do not define the convolution; it is the
// PyTorch one (ShardTensor extends PyTorch's DTensor, section 2):
// cross-correlation, stride 1, dilation 1, zero 'same' padding, bias.
//
// bf16 path: implicit GEMM on the gfx950 matrix cores,
//   M = output channels (A = packed weights)
//   N = output positions (B = input cells staged in LDS)
//   K = kernel taps x input channels,
// with fp32 accumulation.  Three kernel families, one instance per supported
// layer shape (the instance table at the end):
//   conv_rows  streams a strip of the shard along its outermost axis with the
//              weights resident in LDS; 32x32x16 MFMA (64->64 and 32->32 k3)
//   conv_taps  streams a 3D strip over the whole shard depth with two
//              in-plane taps per K step of 16x16x32 MFMA and the weights
//              streamed in five segments of tap pairs (3D 16->16 k5)
//   conv_gemm  tiles with the weights streamed through LDS per 16-channel K
//              chunk, for layers whose weights do not fit in LDS (2D 256->256)
// Each output accumulates its K-steps in an order fixed by the layer shape
// alone (taps in one fixed order, channels ascending), so its bits do not
// depend on which tile, job, shard or plan it belongs to.  Workgroups are persistent and deal
// out their work per XCD, so neighbouring tiles share halo rows in one L2.
//
// fp32 path (and bf16 shapes without a matrix-core instance): a direct
// kernel, one thread per output position, fp32 FMA in the same fixed order.
//
// Epilogue: optional bias, fp32 store, and max |y| per (n, group) via
// integer atomicMax on the float bits (order-free).
#include <algorithm>
#include <type_traits>
#include <utility>

#include "internal.h"

namespace st {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ConvShardArg {
  const uint16_t* in;    // padded input, [N][Pd][Ph][Pw][Cin] (bf16 bits or f32 via cast)
  float* out;            // [N][Ed][Eh][Ew][Cout]
  int32_t tile_begin;
  int32_t tiles_d, tiles_h, tiles_w;
  int32_t ext[3];
  int32_t pad[3];
};

struct ConvArgs {
  int32_t nshards;
  int32_t total_tiles;
  int32_t groups;
  int32_t batch;
  int32_t origin[3];          // halo - ksize/2 per axis
  const uint16_t* w;          // packed weights
  const float* bias;          // or null
  uint32_t* ymax;             // or null
  int32_t xcd_begin[9];       // conv_taps: first job of each XCD's range, [8] = total_tiles
  ConvShardArg sh[ST_MAX_SHARDS];
};
static_assert(sizeof(ConvArgs) <= kMaxKernargBytes, "kernel argument struct too large");

__global__ void fill_u32(uint32_t* __restrict__ p, uint32_t v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// --------------------------------------------------------------------------
// direct kernel (fp32 operands, or bf16 shapes without a matrix-core instance)
// --------------------------------------------------------------------------

struct DirectShardArg {
  const void* in;
  float* out;
  int64_t pos_begin;        // first output position (over N and space) of this shard
  int32_t ext[3];
  int32_t pad[3];
};

struct DirectArgs {
  int32_t nshards, cin, cout, ks, taps, groups;
  int32_t origin[3];
  int64_t total_pos;
  const float* w;           // [taps][Cin][Cout] fp32
  const float* bias;
  uint32_t* ymax;
  DirectShardArg sh[ST_MAX_SHARDS];
};
static_assert(sizeof(DirectArgs) <= kMaxKernargBytes, "kernel argument struct too large");

// CV consecutive input channels of one cell as fp32 (one 16-byte load when CV > 1)
template <typename T, int CV> __device__ __forceinline__ void ld_cells(const T* p, float (&x)[CV]);
template <> __device__ __forceinline__ void ld_cells<float, 1>(const float* p, float (&x)[1]) { x[0] = *p; }
template <> __device__ __forceinline__ void ld_cells<float, 4>(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <> __device__ __forceinline__ void ld_cells<uint16_t, 1>(const uint16_t* p, float (&x)[1]) {
  x[0] = __uint_as_float((uint32_t)*p << 16);
}
template <> __device__ __forceinline__ void ld_cells<uint16_t, 8>(const uint16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

// Direct kernel (fp32 operands, and bf16 shapes off the matrix-core grid): a
// thread owns one output position and OB consecutive output channels, reads
// CV input channels per load and the weights [taps][Cin][Cout] from LDS (WL)
// or from L1/L2 (larger layers).  Each output sums its taps lexicographic,
// channels ascending, one fp32 FMA at a time, whatever thread, tile or shard
// computes it.
template <typename T, int OB, int CV, bool WL>
__global__ __launch_bounds__(256) void conv_direct(const DirectArgs a) {
  extern __shared__ __attribute__((aligned(16))) float dsm[];   // [taps * cin * cout] (WL), then cout max slots
  const int tid = threadIdx.x;
  const int wn = WL ? a.taps * a.cin * a.cout : 0;
  uint32_t* dmax = reinterpret_cast<uint32_t*>(dsm + wn);
  if (WL)
    for (int i = tid; i < wn; i += 256) dsm[i] = a.w[i];
  for (int i = tid; i < a.cout; i += 256) dmax[i] = 0u;
  __syncthreads();
  const float* wsrc = WL ? dsm : a.w;
  const int ncb = a.cout / OB;
  const int64_t gid = (int64_t)blockIdx.x * 256 + tid;
  const int64_t pos = gid / ncb;
  const int ob0 = (int)(gid - pos * ncb) * OB;
  if (pos < a.total_pos) {
    int s = 0;
    while (s + 1 < a.nshards && a.sh[s + 1].pos_begin <= pos) ++s;
    const DirectShardArg& sh = a.sh[s];
    int64_t r = pos - sh.pos_begin;
    const int64_t per_n = (int64_t)sh.ext[0] * sh.ext[1] * sh.ext[2];
    const int n = (int)(r / per_n);
    r -= n * per_n;
    const int od = (int)(r / ((int64_t)sh.ext[1] * sh.ext[2]));
    r -= (int64_t)od * sh.ext[1] * sh.ext[2];
    const int oh = (int)(r / sh.ext[2]);
    const int ow = (int)(r - (int64_t)oh * sh.ext[2]);
    const T* in = static_cast<const T*>(sh.in);
    const int kd_n = a.taps / (a.ks * a.ks);
    float acc[OB];
#pragma unroll
    for (int j = 0; j < OB; ++j) acc[j] = 0.f;
    for (int kd = 0; kd < kd_n; ++kd)
      for (int kh = 0; kh < a.ks; ++kh)
        for (int kw = 0; kw < a.ks; ++kw) {
          const int t = (kd * a.ks + kh) * a.ks + kw;
          const size_t cell = (((size_t)n * sh.pad[0] + od + kd + a.origin[0]) * sh.pad[1] + oh + kh + a.origin[1]) *
                                  sh.pad[2] + ow + kw + a.origin[2];
          const T* xp = in + cell * a.cin;
          const float* wt = wsrc + (size_t)t * a.cin * a.cout + ob0;
          for (int c = 0; c < a.cin; c += CV) {
            float xv[CV];
            ld_cells<T, CV>(xp + c, xv);
#pragma unroll
            for (int v = 0; v < CV; ++v) {
              const float* wc = wt + (size_t)(c + v) * a.cout;
              if (OB == 4) {
                const float4 w4 = *reinterpret_cast<const float4*>(wc);
                acc[0] = fmaf(w4.x, xv[v], acc[0]);
                acc[1] = fmaf(w4.y, xv[v], acc[1]);
                acc[2] = fmaf(w4.z, xv[v], acc[2]);
                acc[3] = fmaf(w4.w, xv[v], acc[3]);
              } else {
#pragma unroll
                for (int j = 0; j < OB; ++j) acc[j] = fmaf(wc[j], xv[v], acc[j]);
              }
            }
          }
        }
    const size_t cell_out = (((size_t)n * sh.ext[0] + od) * sh.ext[1] + oh) * sh.ext[2] + ow;
    float* yp = sh.out + cell_out * a.cout + ob0;
#pragma unroll
    for (int j = 0; j < OB; ++j) {
      if (a.bias) acc[j] += a.bias[ob0 + j];
      if (a.ymax) atomicMax(&dmax[ob0 + j], __float_as_uint(fabsf(acc[j])));
    }
    if (OB == 4) *reinterpret_cast<float4*>(yp) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    else
#pragma unroll
      for (int j = 0; j < OB; ++j) yp[j] = acc[j];
  }
  if (!a.ymax) return;
  __syncthreads();
  // one atomic per (block, group); a block may straddle two batch items or
  // shards, so the batch index is resolved per position below
  const int64_t first = (int64_t)blockIdx.x * 256 / ncb;
  const int64_t last = min(((int64_t)blockIdx.x * 256 + 255) / ncb, a.total_pos - 1);
  auto batch_of = [&](int64_t g) {
    int s = 0;
    while (s + 1 < a.nshards && a.sh[s + 1].pos_begin <= g) ++s;
    const int64_t per_n = (int64_t)a.sh[s].ext[0] * a.sh[s].ext[1] * a.sh[s].ext[2];
    return (int)((g - a.sh[s].pos_begin) / per_n);
  };
  const int n0 = batch_of(first), n1 = batch_of(last);
  const int gs = a.cout / a.groups;
  if (n0 == n1) {
    for (int g = tid; g < a.groups; g += 256) {
      uint32_t m = 0;
      for (int c = g * gs; c < (g + 1) * gs; ++c) m = max(m, dmax[c]);
      atomicMax(&a.ymax[n0 * a.groups + g], m);
    }
  } else if (pos < a.total_pos) {
    // rare (a block spanning two batch items): attribute each output
    // directly, from the values just stored by this thread
    const int n = batch_of(pos);
    int s = 0;
    while (s + 1 < a.nshards && a.sh[s + 1].pos_begin <= pos) ++s;
    const int64_t per_n = (int64_t)a.sh[s].ext[0] * a.sh[s].ext[1] * a.sh[s].ext[2];
    const int64_t r = pos - a.sh[s].pos_begin - (int64_t)n * per_n;
    const float* y = a.sh[s].out + (((size_t)n * per_n) + r) * a.cout + ob0;
    for (int j = 0; j < OB; ++j) atomicMax(&a.ymax[n * a.groups + (ob0 + j) / gs], __float_as_uint(fabsf(y[j])));
  }
}

// max |y| per (n, group) over every shard's fp32 output, for the conv path
// that does not fuse it (the matrix-core 'same' conv of shapes without a
// tuned kernel).  blockIdx.y = shard * batch + n; a thread keeps the running
// max of its 4 channels (cout % 4 == 0) over the positions it visits.
struct YmaxArgs {
  int32_t nshards, batch, cout, groups;
  uint32_t* ymax;
  const float* y[ST_MAX_SHARDS];
  int64_t positions[ST_MAX_SHARDS];   // per sample
};
static_assert(sizeof(YmaxArgs) <= kMaxKernargBytes, "kernel argument struct too large");

__global__ __launch_bounds__(256) void ymax_pass(const YmaxArgs a) {
  const int s = blockIdx.y / a.batch, n = blockIdx.y - s * a.batch;
  const int cq = a.cout / 4;
  const int per_block = 256 / cq;                  // positions per block row
  const int q = threadIdx.x % cq, pr = threadIdx.x / cq;
  if (pr >= per_block) return;
  const int64_t P = a.positions[s];
  const float4* y = reinterpret_cast<const float4*>(a.y[s] + (size_t)n * P * a.cout);
  float m[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t p = (int64_t)blockIdx.x * per_block + pr; p < P; p += (int64_t)gridDim.x * per_block) {
    const float4 v = y[p * cq + q];
    m[0] = fmaxf(m[0], fabsf(v.x));
    m[1] = fmaxf(m[1], fabsf(v.y));
    m[2] = fmaxf(m[2], fabsf(v.z));
    m[3] = fmaxf(m[3], fabsf(v.w));
  }
  const int gs = a.cout / a.groups;
#pragma unroll
  for (int j = 0; j < 4; ++j) atomicMax(&a.ymax[n * a.groups + (4 * q + j) / gs], __float_as_uint(m[j]));
}

// --------------------------------------------------------------------------
// weight packing
// --------------------------------------------------------------------------

// [Cout][Cin][taps] -> [Cin/CK][Cout][KVP], k index = tap*CK + (cin % CK)
// Every packing kernel also zeroes clr[0, nclr) (the max |y| accumulator of
// the conv that follows), so packing and that clear take one launch.
__global__ void pack_w_mfma(const uint16_t* __restrict__ w, uint16_t* __restrict__ out, int cin,
                            int cout, int taps, int ck, int kvp, int64_t total, uint32_t* clr, int nclr) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nclr) clr[i] = 0u;
  if (i >= total) return;
  const int vk = (int)(i % kvp);
  const int64_t r = i / kvp;
  const int o = (int)(r % cout);
  const int cc = (int)(r / cout);
  uint16_t v = 0;
  if (vk < taps * ck) {
    const int t = vk / ck, c = cc * ck + vk % ck;
    v = w[((int64_t)o * cin + c) * taps + t];
  }
  out[i] = v;
}

// [Cout][Cin][taps] -> [Cout/bn][Cin/ck][taps][bn][ck]: each (cout block, K chunk)
// slab is contiguous and already in the order its LDS stage holds it
__global__ void pack_w_gemm(const uint16_t* __restrict__ w, uint16_t* __restrict__ out, int cin, int cout,
                            int taps, int ck, int bn, int64_t total, uint32_t* clr, int nclr) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nclr) clr[i] = 0u;
  if (i >= total) return;
  const int c = (int)(i % ck);
  int64_t r = i / ck;
  const int m = (int)(r % bn);
  r /= bn;
  const int t = (int)(r % taps);
  r /= taps;
  const int cc = (int)(r % (cin / ck));
  const int cb = (int)(r / (cin / ck));
  out[i] = w[((int64_t)(cb * bn + m) * cin + cc * ck + c) * taps + t];
}

// Tap pairs of the 3D k5 tap-pair kernel: in-plane tap dy * 5 + dx in half h
// of pair p (-1: the empty half).  Pairs 0-1 hold the taps (0, 0..3), pairs
// 11-12 the taps (4, 0..3), pairs 2-9 the rest in lexicographic order and
// pair 10 the tap (4, 4) alone.
__host__ __device__ constexpr int k5_pair_tap(int p, int h) {
  return p < 10 ? 2 * p + h : p == 10 ? (h ? -1 : 24) : 20 + 2 * (p - 11) + h;
}
// weight segments of 2, 3, 3, 3 and 2 pairs: first pair, count, and the
// segment of a pair
__host__ __device__ constexpr int k5_seg_first(int s) { return s == 0 ? 0 : s == 4 ? 11 : 3 * s - 1; }
__host__ __device__ constexpr int k5_seg_pairs(int s) { return s == 0 || s == 4 ? 2 : 3; }
__host__ __device__ constexpr int k5_seg_of(int p) { return p < 2 ? 0 : p < 5 ? 1 : p < 8 ? 2 : p < 11 ? 3 : 4; }
// the tables' contract: every in-plane tap in exactly one half; pairs 0-1
// read kernel row 0 only and pairs 11-12 kernel row 4 only (the ring
// protocol); the segments tile the 13 pairs in order
constexpr bool k5_tables_ok() {
  int seen[25] = {};
  for (int p = 0; p < 13; ++p)
    for (int h = 0; h < 2; ++h) {
      const int t = k5_pair_tap(p, h);
      if (t < -1 || t > 24) return false;
      if (t >= 0) ++seen[t];
      if (t >= 0 && p < 2 && t / 5 != 0) return false;
      if (t >= 0 && p > 10 && t / 5 != 4) return false;
    }
  for (int t = 0; t < 25; ++t)
    if (seen[t] != 1) return false;
  for (int s = 0, p = 0; s < 5; p += k5_seg_pairs(s), ++s) {
    if (k5_seg_first(s) != p) return false;
    for (int q = p; q < p + k5_seg_pairs(s); ++q)
      if (k5_seg_of(q) != s) return false;
  }
  return k5_seg_first(4) + k5_seg_pairs(4) == 13;
}
static_assert(k5_tables_ok(), "tap-pair and segment tables");

// [16][16][5][5][5] -> [segment 5][pair slot 3][dz 5][lane 64][8]: the 16x32 A
// fragment of (pair, dz) in lane order, lane 16 kg + cout holding input
// channels 8 (kg >> 1) .. + 7 of the pair's tap kg & 1; the empty half and
// the unused slots of two-pair segments are zero
__global__ void pack_w_taps(const uint16_t* __restrict__ w, uint16_t* __restrict__ out, int64_t total, uint32_t* clr,
                            int nclr) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nclr) clr[i] = 0u;
  if (i >= total) return;
  const int e = (int)(i & 7);
  const int lane = (int)((i >> 3) & 63);
  int r = (int)(i >> 9);
  const int dz = r % 5;
  r /= 5;
  const int slot = r % 3, seg = r / 3;
  const int kg = lane >> 4, o = lane & 15, c = 8 * (kg >> 1) + e;
  const int t = slot < k5_seg_pairs(seg) ? k5_pair_tap(k5_seg_first(seg) + slot, kg & 1) : -1;
  out[i] = t < 0 ? (uint16_t)0 : w[((int64_t)o * 16 + c) * 125 + dz * 25 + t];
}

// [Cout][Cin][taps] -> [Cout][taps][Cin]
// Input gradient: the convolution that maps dy (Cout channels) to dx (Cin
// channels) has weights w'[c][o][t] = w[o][c][flip(t)], every tap axis
// reversed; for taps in lexicographic order flip(t) = taps - 1 - t.
template <typename T>
__global__ void dgrad_weights(const T* __restrict__ w, T* __restrict__ out, int cin, int cout, int taps,
                              int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int t = (int)(i % taps);
  const int64_t co = i / taps;
  const int o = (int)(co % cout), c = (int)(co / cout);
  out[i] = w[((int64_t)o * cin + c) * taps + (taps - 1 - t)];
}


// --------------------------------------------------------------------------
// helpers of the v_mfma_f32_32x32x16_bf16 kernels
// --------------------------------------------------------------------------
//
// All global traffic of these kernels uses range-checked buffer instructions:
// a lane whose cell lies outside the shard gets an out-of-range offset, so
// its load returns 0 and its store is dropped, and the loop bodies carry no
// branches around memory operations.
//
// Output layout of a 32x32 block in a lane: column (position) = lane % 32,
// rows (channels) 8j + 4*(lane/32) + i for accumulator element 4j + i.
//
// Stores of conv_rows: the quads j = 2c and 2c + 1 of a block
// (channels 16c .. 16c + 15) go out as one pair.  Stored as they are (as
// conv_gemm does: its epilogue is a small part of a tile, and the swap's
// extra registers made it spill), each store instruction would
// write 32 bytes into each of 32 cells; swap16 first trades the odd 16-lane
// rows of the first quad with the even rows of the second (one
// v_permlane16_swap per element), after which lane 16 r + t holds channels
// 16c + 4 SWAP_QUAD(r) .. + 3 of position t (first quad) and of position
// 16 + t (second quad), so each instruction writes 16 whole 64-byte runs.

typedef float f32x16 __attribute__((ext_vector_type(16)));
#define SWAP_QUAD(r) ((((r) & 1) << 1) | ((r) >> 1))

__device__ __forceinline__ void swap16(f32x4& x, f32x4& y) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]), __float_as_uint(y[i]), false, false);
    x[i] = __uint_as_float(r[0]);
    y[i] = __uint_as_float(r[1]);
  }
}
constexpr uint32_t kOob = 0x80000000u;        // offset beyond every num_records used
constexpr uint32_t kBufFlags = 0x00020000u;   // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, (int)kBufFlags);
}

// Swizzle of input cells: chunk j of the cell in strip column qc sits at
// chunk j ^ key(qc).  16 lanes reading 16 consecutive columns at one chunk
// then hit 16 distinct 16-byte slots of a 256-byte LDS window.
template <class C>
__device__ __forceinline__ int cell_key(int qc) { return (qc / C::KD) % C::NCH; }

// --------------------------------------------------------------------------
// instance table
// --------------------------------------------------------------------------

struct Instance {
  int ndim, cin, cout, ks;
  int ck, kvp, nt;
  int td, th, tw, ncb;
  int lds;
  st_status (*run)(ConvArgs&, const st_plan*, hipStream_t);
  int bn = 0;                 // cout block of the streamed-weight layout
  int kind = 0;               // weight layout: 0 [Cin/ck][Cout][kvp]; 1 [Cout/bn][Cin/ck][tap][bn][ck];
                              // 3 [segment][pair slot][dz][lane][8] (tap pairs)
};

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus[dev] = prop.multiProcessorCount;
    else cus[dev] = 256;
  }
  return cus[dev];
}



// --------------------------------------------------------------------------
// streaming implicit GEMM with operand reuse along the streamed axis
// --------------------------------------------------------------------------
//
// A wave owns RW consecutive output slices (rows in 2D, planes in 3D) of one
// 32-position run along W, for every output channel.  Along the streamed axis
// the kernel's taps shift by whole slices, so for one in-slice tap and one
// 16-channel K chunk the wave reads the RW + k - 1 input fragments of its
// slices once and the k weight fragments of the streamed-axis taps once, and
// issues RW * k matrix instructions per 32 output channels from them:
// (RW + k - 1 + k * MB) LDS reads per RW * k * MB MFMAs instead of
// (MB + 1) per MB.
//
// The ring holds exactly the TS + k - 1 input slices one step reads.  The
// TS slices of the next step are fetched into registers while the step
// computes and written over the TS oldest slices between two barriers; the
// next job's first TS + k - 1 slices travel the same way during a job's last
// step, so a block never waits on HBM latency between jobs.

template <int NDIM_, int CIN_, int COUT_, int KS_, int BH_, int BW_, int TS_, int RC_, int RW_, int NH_>
struct RowsCfg {
  static constexpr int NDIM = NDIM_, CIN = CIN_, COUT = COUT_, KS = KS_;
  static constexpr int NH = NH_;                      // passes over K per step (output-channel groups)
  static constexpr int BH = NDIM == 3 ? BH_ : 1;
  static constexpr int BW = BW_, TS = TS_, RC = RC_, RW = RW_;
  static constexpr int KH = NDIM == 3 ? KS : 1;
  static constexpr int SH = BH + KH - 1, SW = BW + KS - 1, SLICE = SH * SW;
  static constexpr int RING = TS + KS - 1;
  static constexpr int PG = BH * BW / 32;             // 32-position runs per slice
  static constexpr int RG = TS / RW;                  // slice groups per step
  static constexpr int NWAVES = PG * RG, NT = NWAVES * 64;
  static constexpr int MB = COUT / 32;
  static constexpr int NIN = RW + KS - 1;             // input fragments per K chunk
  static constexpr int TAPS = KS * KH * KS;
  static constexpr int CK = CIN, KV = TAPS * CK;
  static constexpr int KCS = CK / 16;
  static constexpr int KVP = ((KV + 63) / 64) % 2 == 1 ? (KV + 63) / 64 * 64 : (KV + 63) / 64 * 64 + 64;
  static constexpr int NCH = CK / 8, CB = CK * 2, KD = 16 / NCH;
  static constexpr int LDS_W = COUT * KVP * 2;
  static constexpr int LDS_X = RING * SLICE * CB;
  static constexpr int STEP_CHUNKS = TS * SLICE * NCH;
  static constexpr int PRO_CHUNKS = RING * SLICE * NCH;
  static constexpr int PF = (PRO_CHUNKS + NT - 1) / NT;
  static constexpr int PFS = (STEP_CHUNKS + NT - 1) / NT;
  static constexpr int NCHUNK = 1, NCB = 1, TD = 1, TH = 1, TW = BW, BN = COUT;
  static_assert(CIN % 16 == 0 && NCH <= 16 && COUT % 32 == 0, "shape");
  static_assert(BW % 32 == 0 && TS % RW == 0 && RC % TS == 0 && MB % NH == 0, "tiling");
  static_assert(NT <= 1024, "block size");
  static_assert(LDS_W + LDS_X + COUT * 8 <= 160 * 1024, "LDS budget");
};

// MAXG: the running max|y| is kept per 4, 2 or 1 channels (a divisor of the
// group size), or not at all (0)
template <class C, bool BIAS, int MAXG>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::NT / 256, C::NT / 256))) void conv_rows(const ConvArgs args) {
  __shared__ __attribute__((aligned(16))) uint16_t sw[C::LDS_W / 2];
  __shared__ __attribute__((aligned(16))) uint16_t sx[C::LDS_X / 2];
  __shared__ __attribute__((aligned(16))) float sbias[C::COUT];
  __shared__ uint32_t smax[C::COUT];
  char* const swb = reinterpret_cast<char*>(sw);
  char* const sxb = reinterpret_cast<char*>(sx);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int pg = wave % C::PG;
  const int t0 = (wave / C::PG) * C::RW;            // first output slice of this wave within a step
  const int l32 = lane & 31;
  const int g2 = lane >> 5;
  constexpr int RA = C::NDIM == 3 ? 0 : 1;
  constexpr int RSB = C::KVP * 2;
  constexpr bool MAXV = MAXG > 0;
  constexpr int MG = MAXG > 0 ? MAXG : 1;
  constexpr int NMX = 16 / MG;                      // running-max slots per 32-channel block

  for (int i = tid; i < C::COUT; i += C::NT) {
    smax[i] = 0u;
    sbias[i] = BIAS ? args.bias[i] : 0.f;
  }
  {  // resident weights: chunk j of row m at chunk (j & ~7) | ((j & 7) ^ ((m >> 1) & 7))
    constexpr int CPR = C::KVP / 8;
    for (int i = tid; i < C::COUT * CPR; i += C::NT) {
      const int m = i / CPR, j = i - m * CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(args.w + (size_t)m * C::KVP + 8 * j);
      *reinterpret_cast<uint4*>(swb + m * RSB + 16 * ((j & ~7) | ((j & 7) ^ ((m >> 1) & 7)))) = v;
    }
  }

  int ybase[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    const int m = mb * 32 + l32;
    ybase[mb] = (m * RSB + 16 * ((m >> 1) & 7)) ^ (16 * g2);
  }
  const int p = pg * 32 + l32;
  const int ph = p / C::BW, pw = p % C::BW;
  int lcol[C::KS];
#pragma unroll
  for (int tw = 0; tw < C::KS; ++tw) {
    const int qc = pw + tw;
    lcol[tw] = ((ph * C::SW + qc) * C::CB + 16 * cell_key<C>(qc)) ^ (16 * g2);
  }
  const int co_lane = 4 * g2;

  const int total = args.total_tiles;
  int j0 = blockIdx.x, jstride = gridDim.x, j_end = total;
  if (gridDim.x >= 8 && (gridDim.x & 7) == 0) {
    const int xcd = blockIdx.x & 7;
    j0 = (int)((int64_t)total * xcd / 8) + (blockIdx.x >> 3);
    jstride = gridDim.x >> 3;
    j_end = (int)((int64_t)total * (xcd + 1) / 8);
  }

  // slot i covers accumulator elements i*MG .. i*MG+MG-1: channels
  // co_lane + 32*mb + 8*((i*MG)/4) + (i*MG)%4 and the next MG-1
  float runmax[C::MB][NMX];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int i = 0; i < NMX; ++i) runmax[mb][i] = 0.f;
  int cur_n = -1;

  auto flush = [&](int n) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int i = 0; i < NMX; ++i) {
        float v = runmax[mb][i];
        v = fmaxf(v, __shfl_xor(v, 1));
        v = fmaxf(v, __shfl_xor(v, 2));
        v = fmaxf(v, __shfl_xor(v, 4));
        v = fmaxf(v, __shfl_xor(v, 8));
        v = fmaxf(v, __shfl_xor(v, 16));
        runmax[mb][i] = 0.f;
        const int e = i * MG;
        if (l32 == 0) atomicMax(&smax[co_lane + mb * 32 + 8 * (e >> 2) + (e & 3)], __float_as_uint(v));
      }
    __syncthreads();
    const int gs = C::COUT / args.groups;
    for (int g = tid; g < args.groups; g += C::NT) {
      uint32_t m = 0;
      for (int c = g * gs; c < (g + 1) * gs; ++c) m = max(m, smax[c]);
      atomicMax(&args.ymax[n * args.groups + g], m);
    }
    __syncthreads();
    for (int i = tid; i < C::COUT; i += C::NT) smax[i] = 0u;
  };

  // A job is one strip (h0, w0) of one shard and sample, rows [s_begin, s_end)
  // of the streamed axis.  Uniform across the workgroup.
  struct Job {
    int valid, n, s_begin, s_end, h0, w0, o_ring, o_h, o_w, p1, p2, e1, e2, a_lim, ring_pad;
    uint32_t in_slice_b;
    int64_t out_cells;
    __amdgpu_buffer_rsrc_t rin, rout;
  };
  auto make_job = [&](int job) __attribute__((always_inline)) {
    Job J;
    J.valid = job < j_end;
    const int jj = J.valid ? job : j0;
    int s = 0;
    while (s + 1 < args.nshards && args.sh[s + 1].tile_begin <= jj) ++s;
    const ConvShardArg& sh = args.sh[s];
    const int strips = sh.tiles_h * sh.tiles_w;
    int r = jj - sh.tile_begin;
    const int per_n = sh.tiles_d * strips;
    J.n = r / per_n;
    r -= J.n * per_n;
    const int chunk = r / strips;
    r -= chunk * strips;
    const int sth = r / sh.tiles_w;
    const int stw = r - sth * sh.tiles_w;
    J.s_begin = chunk * C::RC;
    J.s_end = min(J.s_begin + C::RC, sh.ext[RA]);
    J.h0 = sth * C::BH;
    J.w0 = stw * C::BW;
    J.o_ring = args.origin[RA];
    J.o_h = args.origin[1];
    J.o_w = args.origin[2];
    const int p0 = sh.pad[0];
    J.p1 = sh.pad[1];
    J.p2 = sh.pad[2];
    J.e1 = sh.ext[1];
    J.e2 = sh.ext[2];
    J.a_lim = J.s_end + C::KS - 1;
    J.ring_pad = C::NDIM == 3 ? p0 : J.p1;
    const int64_t in_slice = C::NDIM == 3 ? (int64_t)J.p1 * J.p2 * C::CIN : (int64_t)J.p2 * C::CIN;
    const int64_t in_base = C::NDIM == 3 ? ((int64_t)J.n * p0 + J.s_begin + J.o_ring) * in_slice
                                         : ((int64_t)J.n * J.p1 + J.s_begin + J.o_ring) * in_slice;
    const int64_t in_total = (int64_t)args.batch * p0 * J.p1 * J.p2 * C::CIN;
    J.rin = make_rsrc(sh.in + in_base, J.valid ? (in_total - in_base) * 2 : 0);
    J.out_cells = C::NDIM == 3 ? (int64_t)J.e1 * J.e2 : (int64_t)J.e2;
    const int64_t out_base = (C::NDIM == 3 ? ((int64_t)J.n * sh.ext[0] + J.s_begin)
                                           : ((int64_t)J.n * J.e1 + J.s_begin)) * J.out_cells * C::COUT;
    const int64_t out_total = (int64_t)args.batch * sh.ext[0] * J.e1 * J.e2 * C::COUT;
    J.rout = make_rsrc(sh.out + out_base, J.valid ? (out_total - out_base) * 4 : 0);
    J.in_slice_b = (uint32_t)(in_slice * 2);
    return J;
  };
  // global byte offset of 16-byte piece u of the slice run starting at row a0,
  // or kOob outside the padded shard, the job's rows or the first lim pieces
  auto piece_off = [&](const Job& J, int u, int lim, int a0) __attribute__((always_inline)) -> uint32_t {
    const int rel = u / (C::SLICE * C::NCH);
    const int pc = u - rel * C::SLICE * C::NCH;
    const int q = pc / C::NCH;
    const int j = pc - q * C::NCH;
    const int qr = q / C::SW, qc = q - qr * C::SW;
    const int gh = J.h0 + qr + J.o_h, gw = J.w0 + qc + J.o_w;
    const int a = a0 + rel;
    const bool ok = u < lim && (C::NDIM == 2 || gh < J.p1) && gw < J.p2 && a < J.a_lim && a + J.o_ring < J.ring_pad;
    const uint32_t goff = (uint32_t)((((C::NDIM == 3 ? (int64_t)gh * J.p2 : 0) + gw) * C::CIN + 8 * j) * 2);
    return ok ? goff + (uint32_t)(a - J.s_begin) * J.in_slice_b : kOob;
  };
  // LDS byte offset of piece u of the slice run starting at row a0
  auto piece_lds = [&](int u, int a0) __attribute__((always_inline)) -> int {
    const int rel = u / (C::SLICE * C::NCH);
    const int pc = u - rel * C::SLICE * C::NCH;
    const int q = pc / C::NCH;
    const int j = pc - q * C::NCH;
    const int qc = q % C::SW;
    return ((a0 + rel) % C::RING) * (C::SLICE * C::CB) + q * C::CB + 16 * (j ^ cell_key<C>(qc));
  };

  Job J = make_job(j0);
  if (!J.valid) return;
  {  // first job's first TS + k - 1 slices, every load in flight before the first store
    uint4 v[C::PF];
#pragma unroll
    for (int k = 0; k < C::PF; ++k)
      v[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                          J.rin, piece_off(J, tid + k * C::NT, C::PRO_CHUNKS, J.s_begin), 0, 0));
#pragma unroll
    for (int k = 0; k < C::PF; ++k)
      if (tid + k * C::NT < C::PRO_CHUNKS)
        *reinterpret_cast<uint4*>(sxb + piece_lds(tid + k * C::NT, J.s_begin)) = v[k];
  }
  if (MAXV) cur_n = J.n;
  __syncthreads();

  f32x16 acc[C::RW][C::MB];
  int job = j0;
  int cur = J.s_begin;
  int base = J.s_begin % C::RING;
  auto step = [&]() __attribute__((always_inline)) -> bool {
    const bool more = cur + C::TS < J.s_end;
    Job N = J;
    if (!more) N = make_job(job + jstride);
    // 1. the next step's TS slices, or the next job's first TS + k - 1, -> registers;
    // the loads issue during the first half of the K loop, between MFMAs
    const int pf_a0 = more ? cur + C::RING : N.s_begin;
    const int pf_lim = more ? C::STEP_CHUNKS : (N.valid ? C::PRO_CHUNKS : 0);
    uint4 pf[C::PF];
    auto issue_pf = [&](int k) __attribute__((always_inline)) {
      const int u = tid + k * C::NT;
      const uint32_t off = piece_off(N, u, (more && k >= C::PFS) ? 0 : pf_lim, pf_a0);
      pf[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(N.rin, off, 0, 0));
    };

    // 2. matrix-core work in NH passes over K, one per group of MH 32-channel
    // output blocks.  A pass's results are stored during the next pass, so
    // the stores run under the matrix instructions and an accumulator is
    // rewritten only half a step after its stores were issued.  The operands
    // of K chunk i+1 are read during chunk i.
    int sbase[C::NIN];                                // ring slice byte base of input slice t0 + r
#pragma unroll
    for (int r = 0; r < C::NIN; ++r) {
      int sl = base + t0 + r;
      sl -= sl >= C::RING ? C::RING : 0;
      sl -= sl >= C::RING ? C::RING : 0;
      sbase[r] = sl * (C::SLICE * C::CB);
    }
    constexpr int NK = C::KH * C::KS * C::KCS;        // in-slice taps x K chunks
    constexpr int NH = C::NH, MH = C::MB / C::NH;
    constexpr int NKT = NH * NK;
    auto load_ops = [&](int ii, bf16x8 (&a)[C::KS][MH], bf16x8 (&b)[C::NIN]) __attribute__((always_inline)) {
      const int hh = ii / NK, i = ii % NK;
      const int cs = i % C::KCS;
      const int tw = (i / C::KCS) % C::KS;
      const int th = i / (C::KCS * C::KS);
#pragma unroll
      for (int r = 0; r < C::NIN; ++r)
        b[r] = *reinterpret_cast<const bf16x8*>(sxb + (((sbase[r] + lcol[tw]) ^ (32 * cs)) + th * C::SW * C::CB));
#pragma unroll
      for (int tr = 0; tr < C::KS; ++tr) {
        const int tap = (tr * C::KH + th) * C::KS + tw;
        const int jw = tap * C::NCH + 2 * cs;
#pragma unroll
        for (int mm = 0; mm < MH; ++mm)
          a[tr][mm] = *reinterpret_cast<const bf16x8*>(swb + ((ybase[hh * MH + mm] ^ (16 * (jw & 7))) + 128 * (jw >> 3)));
      }
    };

    // epilogue pairs: output row t, channel block mb, channel half jp (quads
    // 2 jp and 2 jp + 1), stored after swap16 as 16 positions each
    const int oh = C::NDIM == 3 ? J.h0 + ph : 0;
    const int ow = J.w0 + pw;
    const bool row_in = C::NDIM == 2 || oh < J.e1;
    const bool in_plane = row_in && ow < J.e2;          // this lane's position before the swap
    const int t16 = lane & 15;
    const int owx = ow - l32 + t16;                    // positions after the swap: owx, owx + 16
    const bool okx_plane = row_in && owx < J.e2, oky_plane = row_in && owx + 16 < J.e2;
    const int co_sw = 4 * SWAP_QUAD(lane >> 4);
    auto store_pair = [&](int t, int mb, int jp) __attribute__((always_inline)) {
      const int osl = cur + t0 + t;
      const bool live = osl < J.s_end;
      const bool ok = in_plane && live;
      const int64_t row_cell = (int64_t)(osl - J.s_begin) * J.out_cells + (C::NDIM == 3 ? (int64_t)oh * J.e2 : 0);
      f32x4 v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int jj = 2 * jp + h;
        const int co = mb * 32 + 8 * jj;              // relative to co_lane
#pragma unroll
        for (int i = 0; i < 4; ++i) v[h][i] = acc[t][mb][4 * jj + i];
        if (BIAS) {
          const float4 bv4 = *reinterpret_cast<const float4*>(&sbias[co_lane + co]);
          v[h][0] += bv4.x; v[h][1] += bv4.y; v[h][2] += bv4.z; v[h][3] += bv4.w;
        }
        if (MAXV) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            runmax[mb][(4 * jj + i) / MG] = fmaxf(runmax[mb][(4 * jj + i) / MG], ok ? fabsf(v[h][i]) : 0.f);
        }
      }
      swap16(v[0], v[1]);
      const uint32_t cx = (uint32_t)(((row_cell + owx) * C::COUT + co_sw) * 4);
      const uint32_t co4 = (uint32_t)((mb * 32 + 16 * jp) * 4);       // kOob + co4 stays out of range
      const uint32_t ox = live && okx_plane ? cx : kOob;
      const uint32_t oy = live && oky_plane ? cx + 16 * C::COUT * 4 : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(v[0], J.rout, ox + co4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(v[1], J.rout, oy + co4, 0, 0);
    };
    constexpr int NSP = C::RW * MH * 2;               // store pairs of one pass
    auto store_pass = [&](int hh, int q0, int q1) __attribute__((always_inline)) {
#pragma unroll
      for (int q = q0; q < q1; ++q) store_pair(q / (MH * 2), hh * MH + (q / 2) % MH, q % 2);
    };

    bf16x8 av[2][C::KS][MH], bv[2][C::NIN];
    load_ops(0, av[0], bv[0]);
    constexpr int NRD = C::NIN + C::KS * MH;          // LDS reads per K chunk
    constexpr int NMF = C::RW * C::KS * MH;           // matrix instructions per K chunk
    constexpr int PF_CHUNKS = NK / 2 > 0 ? NK / 2 : 1;   // K chunks that carry the prefetch loads
#pragma unroll
    for (int ii = 0; ii < NKT; ++ii) {
      const int hh = ii / NK, i = ii % NK;
      const int cb = ii & 1;
      __builtin_amdgcn_sched_barrier(0);
      if (i == 0) {
#pragma unroll
        for (int t = 0; t < C::RW; ++t)
#pragma unroll
          for (int mm = 0; mm < MH; ++mm) acc[t][hh * MH + mm] = f32x16{};
      }
      if (hh == 0 && i < PF_CHUNKS) {
#pragma unroll
        for (int k = i * C::PF / PF_CHUNKS; k < (i + 1) * C::PF / PF_CHUNKS; ++k) issue_pf(k);
      }
      if (hh > 0) store_pass(hh - 1, i * NSP / NK, (i + 1) * NSP / NK);
      if (ii + 1 < NKT) load_ops(ii + 1, av[cb ^ 1], bv[cb ^ 1]);
#pragma unroll
      for (int tr = 0; tr < C::KS; ++tr)
#pragma unroll
        for (int t = 0; t < C::RW; ++t)
#pragma unroll
          for (int mm = 0; mm < MH; ++mm)
            acc[t][hh * MH + mm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cb][tr][mm], bv[cb][t + tr],
                                                                           acc[t][hh * MH + mm], 0, 0, 0);
      // interleave: the next chunk's reads (and the previous pass's stores)
      // spread over this chunk's MFMAs
      if (ii + 1 < NKT) {
        const int nst = hh > 0 ? 2 * ((i + 1) * NSP / NK - i * NSP / NK) : 0;
#pragma unroll
        for (int g = 0; g < NRD; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                 // one LDS read
          const int nm = (g + 1) * NMF / NRD - g * NMF / NRD;
          if (nm == 1) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMAs
          else if (nm == 2) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          else if (nm == 3) __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
          else if (nm >= 4) __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          if (g < nst) __builtin_amdgcn_sched_group_barrier(0x040, 1, 0);    // one store
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // 3. the last pass's results: bias, range-checked fp32 stores, running max
    store_pass(NH - 1, 0, NSP);

    // 4. every wave is done with the ring: the fetched slices replace the TS
    // oldest ones (or the whole ring for the next job)
    __syncthreads();
    if (more) {
#pragma unroll
      for (int k = 0; k < C::PFS; ++k) {
        const int u = tid + k * C::NT;
        if (u < C::STEP_CHUNKS) *reinterpret_cast<uint4*>(sxb + piece_lds(u, cur + C::RING)) = pf[k];
      }
      __syncthreads();
      cur += C::TS;
      base += C::TS;
      base -= base >= C::RING ? C::RING : 0;
    } else {
      if (!N.valid) return false;
#pragma unroll
      for (int k = 0; k < C::PF; ++k) {
        const int u = tid + k * C::NT;
        if (u < C::PRO_CHUNKS) *reinterpret_cast<uint4*>(sxb + piece_lds(u, N.s_begin)) = pf[k];
      }
      if (MAXV && N.n != cur_n) {
        flush(cur_n);
        cur_n = N.n;
      }
      __syncthreads();
      job += jstride;
      J = N;
      cur = J.s_begin;
      base = J.s_begin % C::RING;
    }
    return true;
  };
  for (;;) {
    if (!step()) break;
  }
  if (MAXV) flush(cur_n);
}

template <class C>
st_status run_rows(ConvArgs& a, const st_plan* in_plan, hipStream_t stream) {
  constexpr int RA = C::NDIM == 3 ? 0 : 1;
  int jobs = 0;
  for (size_t s = 0; s < in_plan->shards.size(); ++s) {
    const Shard& sd = in_plan->shards[s];
    ConvShardArg& sh = a.sh[s];
    // the buffer views of one job must stay below 2 GiB
    const int64_t in_slice = C::NDIM == 3 ? sd.pad[1] * sd.pad[2] * C::CIN : sd.pad[2] * C::CIN;
    const int64_t out_slice = C::NDIM == 3 ? sd.ext[1] * sd.ext[2] * C::COUT : sd.ext[2] * C::COUT;
    if ((C::RC + C::TS + C::KS) * in_slice * 2 >= 0x7FFFFFFF || C::RC * out_slice * 4 >= 0x7FFFFFFF)
      return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: slices too large for the streaming kernel");
    sh.tiles_d = (int)((sd.ext[RA] + C::RC - 1) / C::RC);
    sh.tiles_h = C::NDIM == 3 ? (int)((sd.ext[1] + C::BH - 1) / C::BH) : 1;
    sh.tiles_w = (int)((sd.ext[2] + C::BW - 1) / C::BW);
    sh.tile_begin = jobs;
    const int64_t t = (int64_t)in_plan->batch * sh.tiles_d * sh.tiles_h * sh.tiles_w;
    if ((int64_t)jobs + t > INT32_MAX) return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: too many jobs");
    jobs += (int)t;
  }
  a.total_tiles = jobs;
  if (jobs == 0) return ST_OK;
  // one workgroup per CU: the LDS footprint allows no more
  int grid = std::min(jobs, device_cus());
  if (grid >= 8) grid &= ~7;
  // running max per 4 / 2 / 1 channels, whichever divides the group size
  const int gs = a.ymax ? C::COUT / a.groups : 0;
  const int g = a.ymax == nullptr ? 0 : gs % 4 == 0 ? 4 : gs % 2 == 0 ? 2 : 1;
  const dim3 gd(grid), bd(C::NT);
  if (a.bias) {
    if (g == 4) hipLaunchKernelGGL((conv_rows<C, true, 4>), gd, bd, 0, stream, a);
    else if (g == 2) hipLaunchKernelGGL((conv_rows<C, true, 2>), gd, bd, 0, stream, a);
    else if (g == 1) hipLaunchKernelGGL((conv_rows<C, true, 1>), gd, bd, 0, stream, a);
    else hipLaunchKernelGGL((conv_rows<C, true, 0>), gd, bd, 0, stream, a);
  } else {
    if (g == 4) hipLaunchKernelGGL((conv_rows<C, false, 4>), gd, bd, 0, stream, a);
    else if (g == 2) hipLaunchKernelGGL((conv_rows<C, false, 2>), gd, bd, 0, stream, a);
    else if (g == 1) hipLaunchKernelGGL((conv_rows<C, false, 1>), gd, bd, 0, stream, a);
    else hipLaunchKernelGGL((conv_rows<C, false, 0>), gd, bd, 0, stream, a);
  }
  return launch_check("st_conv_sharded: conv_rows launch");
}

template <class C>
constexpr Instance inst_rows() {
  return Instance{C::NDIM, C::CIN, C::COUT, C::KS, C::CK, C::KVP, C::NT,
                  1, C::BH, C::BW, 1, C::LDS_W + C::LDS_X, &run_rows<C>};
}




// --------------------------------------------------------------------------
// tiled implicit GEMM with streamed weights (wide 2D layers)
// --------------------------------------------------------------------------
//
// For layers whose weights do not fit in LDS (2D 256->256 k3: 1.2 MB).  A
// workgroup owns TR rows x TW columns of output positions and BN output
// channels; wave w owns row w (TW/32 runs of 32 positions) and all BN
// channels (BN/32 blocks), so one K step reads BN/32 + TW/32 fragments for
// (BN/32)*(TW/32) MFMAs.  K is streamed in 16-channel chunks: per chunk the
// input box (TR + k - 1) x (TW + k - 1) cells x 16 channels and the chunk's
// weights (BN x k^2 x 16) sit in one of two LDS stages.  The next chunk's
// pieces (or the next tile's first chunk) are loaded into registers at the
// start of a chunk and written to the other stage in its middle; one barrier
// per chunk.  Cout blocks are the innermost tile index, so the tiles that
// share an input box run side by side on one XCD and read it from its L2.

template <int CIN_, int COUT_, int KS_, int TR_, int TW_, int BN_>
struct GemmCfg {
  static constexpr int NDIM = 2, CIN = CIN_, COUT = COUT_, KS = KS_;
  static constexpr int TR = TR_, TW = TW_, BN = BN_;
  static constexpr int CK = 16;                       // channels per K chunk (one 32x32x16 K step per tap)
  static constexpr int TAPS = KS * KS;
  static constexpr int KVP = TAPS * CK;               // packed weight row: [tap][16 channels]
  static constexpr int NCHUNK = CIN / CK, NCB = COUT / BN;
  static constexpr int BOXH = TR + KS - 1, BOXW = TW + KS - 1;
  static constexpr int MB = BN / 32, NB = TW / 32;
  static constexpr int NWAVES = TR, NT = NWAVES * 64;
  static constexpr int X_CELLS = BOXH * BOXW;         // cells of a chunk's input box
  static constexpr int STAGE_W = BN * TAPS * 32;                  // bytes of a chunk's weights
  static constexpr int STAGE_X = (BOXH * BOXW * 32 + 1023) / 1024 * 1024;   // input box, whole KiB
  static constexpr int STAGE = STAGE_W + STAGE_X;
  static constexpr int NJ = STAGE / 1024, NJW = STAGE_W / 1024;   // 1 KiB LDS-DMA transfers per stage
  static constexpr int JPW = (NJ + TR - 1) / TR;                  // transfers per wave
  static constexpr int LDS = 2 * STAGE;
  static constexpr int CK_ = CK, TD = 1, TH = TR;
  static_assert(CIN % CK == 0 && COUT % BN == 0 && BN % 32 == 0 && TW % 32 == 0, "shape");
  static_assert(STAGE_W % 1024 == 0, "weight slab in whole KiB");
  static_assert(LDS + BN * 8 <= 160 * 1024, "LDS budget");
  static_assert(NT <= 1024, "block size");
};

template <class C, bool BIAS, int MAXG>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void conv_gemm(const ConvArgs args) {
  // two LDS stages, separate objects so the compiler can tell the stage being
  // read from the one being filled
  __shared__ __attribute__((aligned(1024))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[C::STAGE];
  __shared__ __attribute__((aligned(16))) float sbias[C::BN];
  __shared__ uint32_t smax[C::BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;                             // output row of the tile
  const int l32 = lane & 31;
  const int g2 = lane >> 5;
  constexpr bool MAXV = MAXG > 0;
  constexpr int MG = MAXG > 0 ? MAXG : 1;
  constexpr int NMX = 16 / MG;

  for (int i = tid; i < C::BN; i += C::NT) smax[i] = 0u;

  // fragment addresses within a stage.  A: [tap][BN][16 ch], B: box cells of
  // 16 channels; the two 16-byte halves of a 32-byte row are swapped when bit
  // 3 of the row (channel / column) is set, so 16 consecutive rows read by 16
  // lanes cover all 64 banks.
  int aoff[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    const int m = mb * 32 + l32;
    aoff[mb] = m * 32 + 16 * (g2 ^ ((m >> 3) & 1));
  }
  int boff[C::NB][C::KS];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int dx = 0; dx < C::KS; ++dx) {
      const int c = nb * 32 + l32 + dx;
      boff[nb][dx] = C::STAGE_W + (w * C::BOXW + c) * 32 + 16 * (g2 ^ ((c >> 3) & 1));
    }

  const int total = args.total_tiles;
  int t0 = blockIdx.x, tstride = gridDim.x, t_end = total;
  if (gridDim.x >= 8 && (gridDim.x & 7) == 0) {
    const int xcd = blockIdx.x & 7;
    t0 = (int)((int64_t)total * xcd / 8) + (blockIdx.x >> 3);
    tstride = gridDim.x >> 3;
    t_end = (int)((int64_t)total * (xcd + 1) / 8);
  }

  // A tile: shard s, sample n, cout block cb, top-left output (h0, w0).
  // Buffer descriptors and extents are rebuilt from the shard table when used.
  struct Tile {
    int valid, s, n, cb, h0, w0;
  };
  auto make_tile = [&](int t) __attribute__((always_inline)) {
    Tile T;
    T.valid = t < t_end;
    const int tt = T.valid ? t : t0;
    int s = 0;
    while (s + 1 < args.nshards && args.sh[s + 1].tile_begin <= tt) ++s;
    const ConvShardArg& sh = args.sh[s];
    const int tiles_sp = sh.tiles_h * sh.tiles_w;
    int r = tt - sh.tile_begin;
    T.s = s;
    T.cb = r % C::NCB;
    r /= C::NCB;
    T.n = r / tiles_sp;
    r -= T.n * tiles_sp;
    const int th = r / sh.tiles_w;
    T.h0 = th * C::TR;
    T.w0 = (r - th * sh.tiles_w) * C::TW;
    return T;
  };
  auto rsrc_in = [&](const Tile& T) __attribute__((always_inline)) {
    const ConvShardArg& sh = args.sh[T.s];
    const int64_t in_n = (int64_t)sh.pad[1] * sh.pad[2] * C::CIN;
    return make_rsrc(sh.in + T.n * in_n, T.valid ? in_n * 2 : 0);
  };
  auto rsrc_w = [&](const Tile& T) __attribute__((always_inline)) {
    return make_rsrc(args.w + (size_t)T.cb * C::NCHUNK * C::STAGE_W / 2, T.valid ? (int64_t)C::NCHUNK * C::STAGE_W : 0);
  };

  constexpr uint32_t W_CHUNK = C::STAGE_W;            // bytes between chunks in the packed weights
  // Stage filling by LDS-DMA: transfer j of a stage moves 1 KiB; lane l writes
  // 16-byte slot s = 64 j + l.  Weights (j < NJW): slot s holds row s / 2
  // (tap * BN + m), half (s & 1) ^ bit 3 of m.  Input (j >= NJW): slot s holds
  // box cell q = s / 2 - 32 NJW, half (s & 1) ^ bit 3 of its column.  Lanes
  // outside the box or the padded shard get an out-of-range offset: the
  // transfer writes zeros there.  Wave w moves transfers w, w + TR, ...
  auto fetch = [&](char* dst, int i, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rin, int gh0, int gw0,
                   int p1, int p2, int cc) __attribute__((always_inline)) {
    const int j = w + i * C::TR;
    if (j >= C::NJ) return;
    typedef __attribute__((address_space(3))) void* lds_ptr;
    lds_ptr ldst = (lds_ptr)(dst + j * 1024);
    const int slot = 64 * j + lane;
    if (j < C::NJW) {
      const int row = slot >> 1, m = row % C::BN;
      const uint32_t off = (uint32_t)(row * 2 + ((slot & 1) ^ ((m >> 3) & 1))) * 16 + (uint32_t)cc * W_CHUNK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, ldst, 16, off, 0, 0, 0);
    } else {
      const int q = (slot >> 1) - 32 * C::NJW;
      const int r = q / C::BOXW, c = q - r * C::BOXW;
      const int h = (slot & 1) ^ ((c >> 3) & 1);
      const int gh = gh0 + r, gw = gw0 + c;
      const bool ok = q < C::X_CELLS && gh < p1 && gw < p2;
      const uint32_t off = ok ? (uint32_t)((gh * p2 + gw) * C::CIN * 2 + 16 * h + cc * 32) : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rin, ldst, 16, off, 0, 0, 0);
    }
  };
  auto wait_fetches = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0): this wave's transfers are in LDS
    __syncthreads();
  };


  Tile T = make_tile(t0);
  if (!T.valid) return;
  for (int i = tid; i < C::BN; i += C::NT) sbias[i] = BIAS ? args.bias[T.cb * C::BN + i] : 0.f;
#pragma unroll
  for (int i = 0; i < C::JPW; ++i)
    fetch(stage0, i, rsrc_w(T), rsrc_in(T), T.h0 + args.origin[1], T.w0 + args.origin[2], args.sh[T.s].pad[1],
          args.sh[T.s].pad[2], 0);
  wait_fetches();
  int cur_key = MAXV ? T.n * C::NCB + T.cb : -1;

  // per-(n, cout block) maxima collect in smax (one LDS atomic per slot and
  // tile) and go to ymax when the block moves to another (n, cout block)
  auto flush = [&](int n, int cb) __attribute__((always_inline)) {
    __syncthreads();
    const int gs = C::COUT / args.groups;
    const int c_lo = cb * C::BN;
    const int g_lo = c_lo / gs, g_hi = (c_lo + C::BN - 1) / gs;
    for (int g = g_lo + tid; g <= g_hi; g += C::NT) {
      uint32_t m = 0;
      const int a = max(g * gs, c_lo), b = min((g + 1) * gs, c_lo + C::BN);
      for (int c = a; c < b; ++c) m = max(m, smax[c - c_lo]);
      atomicMax(&args.ymax[n * args.groups + g], m);
    }
    __syncthreads();
    for (int i = tid; i < C::BN; i += C::NT) smax[i] = 0u;
  };

  int t = t0;
  for (;;) {
    f32x16 acc[C::MB][C::NB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = f32x16{};
    // the current tile's transfer parameters (the last chunk fetches the next tile's first)
    const __amdgpu_buffer_rsrc_t rwT = rsrc_w(T), rinT = rsrc_in(T);
    const int gh0T = T.h0 + args.origin[1], gw0T = T.w0 + args.origin[2];
    const int p1T = args.sh[T.s].pad[1], p2T = args.sh[T.s].pad[2];
    Tile N = T;
    // Per chunk: a barrier (every wave is done with the previous chunk, which
    // read the other stage), the next chunk's transfers into the other stage
    // during taps 0-2, and before the last tap a wait for them and a barrier;
    // the last tap reads the next chunk's first operands.  Tap 0 runs on
    // operands already in registers, so neither barrier stalls the matrix
    // cores for an LDS round trip.  A tile has an even number of chunks and
    // starts in stage 0; chunk cc reads stage cc & 1.
    constexpr int TI1 = 3;                            // transfers issued during taps [0, TI1)
    bf16x8 av[2][C::MB], bv[2][C::NB];
    auto load_ops = [&](const char* sb, int tap, bf16x8 (&a)[C::MB], bf16x8 (&b)[C::NB]) __attribute__((always_inline)) {
      const int dy = tap / C::KS, dx = tap - dy * C::KS;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
        a[mb] = *reinterpret_cast<const bf16x8*>(sb + tap * (C::BN * 32) + aoff[mb]);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
        b[nb] = *reinterpret_cast<const bf16x8*>(sb + dy * (C::BOXW * 32) + boff[nb][dx]);
    };
    load_ops(stage0, 0, av[0], bv[0]);
    auto chunk = [&](int cc, auto P) __attribute__((always_inline)) {
      constexpr int par = decltype(P)::value;
      char* const cur = par ? stage1 : stage0;
      char* const nxt = par ? stage0 : stage1;
      const bool last = cc + 1 == C::NCHUNK;
      __amdgpu_buffer_rsrc_t rw = rwT, rin = rinT;
      int gh0 = gh0T, gw0 = gw0T, p1 = p1T, p2 = p2T;
      if (last) {
        N = make_tile(t + tstride);
        rw = rsrc_w(N);
        rin = rsrc_in(N);
        gh0 = N.h0 + args.origin[1];
        gw0 = N.w0 + args.origin[2];
        p1 = args.sh[N.s].pad[1];
        p2 = args.sh[N.s].pad[2];
      }
      const int cn = last ? 0 : cc + 1;
      constexpr int NRD = C::MB + C::NB, NMF = C::MB * C::NB;
#pragma unroll
      for (int tap = 0; tap < C::TAPS; ++tap) {
        const int cb = (tap + par) & 1;
        __builtin_amdgcn_sched_barrier(0);
        if (tap == 0) __syncthreads();
        if (tap < TI1) {
#pragma unroll
          for (int i = tap * C::JPW / TI1; i < (tap + 1) * C::JPW / TI1; ++i)
            fetch(nxt, i, rw, rin, gh0, gw0, p1, p2, cn);
        }
        if (tap + 1 == C::TAPS) wait_fetches();
        // operands of the next tap; after the last tap, the next chunk's first
        load_ops(tap + 1 < C::TAPS ? cur : nxt, tap + 1 < C::TAPS ? tap + 1 : 0, av[cb ^ 1], bv[cb ^ 1]);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cb][mb], bv[cb][nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
        for (int g = 0; g < NRD; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NMF / NRD > 0 ? NMF / NRD : 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    static_assert(C::NCHUNK % 2 == 0 && C::TAPS % 2 == 1, "chunks pair up: stages and operand buffers alternate");
#pragma unroll 1
    for (int cc = 0; cc < C::NCHUNK; cc += 2) {
      chunk(cc, std::integral_constant<int, 0>{});
      chunk(cc + 1, std::integral_constant<int, 1>{});
    }

    // epilogue: bias, range-checked fp32 stores, running max
    const int e1 = args.sh[T.s].ext[1], e2 = args.sh[T.s].ext[2];
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(args.sh[T.s].out + (int64_t)T.n * e1 * e2 * C::COUT,
                                                  (int64_t)e1 * e2 * C::COUT * 4);
    const int oh = T.h0 + w;
    const bool row_ok = oh < e1;
    float tmax[C::MB][NMX];                           // this tile's max|y| per slot of MG channels
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int i = 0; i < NMX; ++i) tmax[mb][i] = 0.f;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      const int ow = T.w0 + nb * 32 + l32;
      const bool ok = row_ok && ow < e2;
      const uint32_t cbase = ok ? (uint32_t)((((int64_t)oh * e2 + ow) * C::COUT + T.cb * C::BN + 4 * g2) * 4) : kOob;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int co = mb * 32 + 8 * jj;
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[mb][nb][4 * jj + i];
          if (BIAS) {
            const float4 bv4 = *reinterpret_cast<const float4*>(&sbias[4 * g2 + co]);
            v[0] += bv4.x; v[1] += bv4.y; v[2] += bv4.z; v[3] += bv4.w;
          }
          __builtin_amdgcn_raw_buffer_store_b128(v, rout, cbase + (uint32_t)(co * 4), 0, 0);
          if (MAXV) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              tmax[mb][(4 * jj + i) / MG] = fmaxf(tmax[mb][(4 * jj + i) / MG], ok ? fabsf(v[i]) : 0.f);
          }
        }
    }
    if (MAXV) {
      // over the 32 lanes that share the channels, then one LDS atomic per slot
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int i = 0; i < NMX; ++i) {
          float v = tmax[mb][i];
          v = fmaxf(v, __shfl_xor(v, 1));
          v = fmaxf(v, __shfl_xor(v, 2));
          v = fmaxf(v, __shfl_xor(v, 4));
          v = fmaxf(v, __shfl_xor(v, 8));
          v = fmaxf(v, __shfl_xor(v, 16));
          const int e = i * MG;
          if (l32 == 0) atomicMax(&smax[4 * g2 + mb * 32 + 8 * (e >> 2) + (e & 3)], __float_as_uint(v));
        }
    }
    if (!N.valid) break;
    if (MAXV && N.n * C::NCB + N.cb != cur_key) {
      flush(cur_key / C::NCB, cur_key % C::NCB);
      cur_key = N.n * C::NCB + N.cb;
    }
    if (BIAS && N.cb != T.cb) {
      __syncthreads();
      for (int i = tid; i < C::BN; i += C::NT) sbias[i] = args.bias[N.cb * C::BN + i];
      __syncthreads();
    }
    t += tstride;
    T = N;
  }
  if (MAXV) flush(cur_key / C::NCB, cur_key % C::NCB);
}

template <class C>
st_status run_gemm(ConvArgs& a, const st_plan* in_plan, hipStream_t stream) {
  int tiles = 0;
  for (size_t s = 0; s < in_plan->shards.size(); ++s) {
    const Shard& sd = in_plan->shards[s];
    ConvShardArg& sh = a.sh[s];
    const int64_t in_n = (int64_t)sd.pad[1] * sd.pad[2] * C::CIN;
    const int64_t out_n = (int64_t)sd.ext[1] * sd.ext[2] * C::COUT;
    if (in_n * 2 >= 0x7FFFFFFF || out_n * 4 >= 0x7FFFFFFF)
      return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: shard too large for the tiled kernel");
    sh.tiles_d = 1;
    sh.tiles_h = (int)((sd.ext[1] + C::TR - 1) / C::TR);
    sh.tiles_w = (int)((sd.ext[2] + C::TW - 1) / C::TW);
    sh.tile_begin = tiles;
    const int64_t t = (int64_t)in_plan->batch * sh.tiles_h * sh.tiles_w * C::NCB;
    if ((int64_t)tiles + t > INT32_MAX) return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: too many tiles");
    tiles += (int)t;
  }
  a.total_tiles = tiles;
  if (tiles == 0) return ST_OK;
  int grid = std::min(tiles, device_cus());
  if (grid >= 8) grid &= ~7;
  const int gs = a.ymax ? C::COUT / a.groups : 0;
  const int g = a.ymax == nullptr ? 0 : gs % 4 == 0 ? 4 : gs % 2 == 0 ? 2 : 1;
  const dim3 gd(grid), bd(C::NT);
  if (a.bias) {
    if (g == 4) hipLaunchKernelGGL((conv_gemm<C, true, 4>), gd, bd, 0, stream, a);
    else if (g == 2) hipLaunchKernelGGL((conv_gemm<C, true, 2>), gd, bd, 0, stream, a);
    else if (g == 1) hipLaunchKernelGGL((conv_gemm<C, true, 1>), gd, bd, 0, stream, a);
    else hipLaunchKernelGGL((conv_gemm<C, true, 0>), gd, bd, 0, stream, a);
  } else {
    if (g == 4) hipLaunchKernelGGL((conv_gemm<C, false, 4>), gd, bd, 0, stream, a);
    else if (g == 2) hipLaunchKernelGGL((conv_gemm<C, false, 2>), gd, bd, 0, stream, a);
    else if (g == 1) hipLaunchKernelGGL((conv_gemm<C, false, 1>), gd, bd, 0, stream, a);
    else hipLaunchKernelGGL((conv_gemm<C, false, 0>), gd, bd, 0, stream, a);
  }
  return launch_check("st_conv_sharded: conv_gemm launch");
}

template <class C>
constexpr Instance inst_gemm() {
  return Instance{C::NDIM, C::CIN, C::COUT, C::KS, C::CK, C::KVP, C::NT,
                  1, C::TR, C::TW, C::NCB, C::LDS, &run_gemm<C>, C::BN, 1};
}

// --------------------------------------------------------------------------
// 3D layers with 16 input and 16 output channels: tap pairs on 16x16x32 MFMA
// --------------------------------------------------------------------------
//
// A K step of v_mfma_f32_16x16x32_bf16 holds two in-plane taps (dy, dx) x 16
// input channels; its 16 rows are the 16 output channels and its 16 columns
// 16 positions along W.  A wave owns one row of a BH x 32 strip (two column
// blocks) and RW consecutive output planes.  For one tap pair it reads the
// fragments of the RW + k - 1 input planes (B, per column block) and one
// weight fragment per depth tap dz (A), and issues one MFMA per (output
// plane, dz, column block): each input fragment feeds the up to k output
// planes it reaches and each weight fragment all RW of them.  The k^2
// in-plane taps make ceil(k^2 / 2) pairs, one with an empty half (zero
// weights): for k = 5, 13 pairs x 80 = 1040 MFMAs of 16 cycles per step,
// 96% of their products useful.
//
// Every output accumulates the pairs in one fixed order (a pair's two taps
// inside one MFMA, then dz upwards), wherever it lies, so sharded and
// unsharded outputs agree bit for bit.  The pair order serves the ring: the
// first two pairs hold the taps (0, 0..3), the last two (4, 0..3), and the
// nine between them the rest in lexicographic order, (4, 4) last and alone.
//
// The ring in LDS holds the TS + k - 1 input planes of one step (TS = RW, all
// waves on the same planes).  The next step's TS planes are fetched into
// registers during the step in two halves of slice rows and written over the
// oldest planes: rows 0-3 once the pairs left in the step read kernel row 4
// only, rows 4-7 at the step's end.  The weights (the same for every job)
// stream from L2 into three LDS stages by LDS-DMA in five segments of 2, 3,
// 3, 3 and 2 pairs, segments 0-4 of every step in stages 0, 1, 2, 0, 1, each
// fetched one or two segments ahead of its use.  A job is one strip of a
// shard over its whole depth.

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>) in order:
// a loop whose body must see its index as a constant (the pair loop below is
// too large for the unroller's threshold)
template <class F, int... P>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, P...>) {
  (f(std::integral_constant<int, P>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int BH_, int RW_>
struct TapsCfg {
  static constexpr int NDIM = 3, CIN = 16, COUT = 16, KS = 5;
  static constexpr int BH = BH_, BW = 32, RW = RW_, TS = RW;
  static constexpr int SH = BH + KS - 1, SW = BW + KS - 1, SLICE = SH * SW;
  static constexpr int CB = CIN * 2;                  // bytes per input cell
  static constexpr int SLICE_B = SLICE * CB;
  static constexpr int RING = TS + KS - 1;
  static constexpr int NIN = RW + KS - 1;             // input planes of one step
  static constexpr int NWAVES = BH, NT = NWAVES * 64;
  static constexpr int NPAIRS = (KS * KS + 1) / 2, NSEG = 5, SLOTS = 3;
  static constexpr int FRAG = 1024;                   // one A fragment: 64 lanes x 16 bytes
  static constexpr int WSTAGE = SLOTS * KS * FRAG;    // a segment's weights, [pair][dz][lane][8]
  static constexpr int LDS_X = RING * SLICE_B;
  static constexpr int LDS = LDS_X + 3 * WSTAGE;
  static constexpr int STEP_CHUNKS = TS * SLICE * 2;  // 16-byte pieces of a step's new planes
  static constexpr int PF = (STEP_CHUNKS + NT - 1) / NT;
  static constexpr int PFH = PF / 2;                  // loads per half: slice rows 0-3, then rows 4-7
  static constexpr int CK = CIN, KVP = NSEG * WSTAGE / (COUT * 2), TD = 1, TH = BH, TW = BW, NCB = 1;
  static_assert(SH == 8 && NWAVES == 4 && STEP_CHUNKS == 2 * PFH * NT, "halves of whole slice rows");
  static_assert(k5_seg_first(NSEG - 1) + k5_seg_pairs(NSEG - 1) == NPAIRS, "segments cover the pairs");
  static_assert(RW >= 1 && NT <= 1024 && LDS + COUT * 8 <= 160 * 1024, "resources");
};

template <class C, bool BIAS, int MAXG>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void conv_taps(const ConvArgs args) {
  __shared__ __attribute__((aligned(1024))) char sring[C::LDS_X];
  __shared__ __attribute__((aligned(1024))) char sw0[C::WSTAGE];
  __shared__ __attribute__((aligned(1024))) char sw1[C::WSTAGE];
  __shared__ __attribute__((aligned(1024))) char sw2[C::WSTAGE];
  __shared__ __attribute__((aligned(16))) float sbias[C::COUT];
  __shared__ uint32_t smax[C::COUT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // the wave's row in the strip
  const int l16 = lane & 15;                          // position within a 16-column block
  // K group: tap kg & 1 of a pair, input channels 8 (kg >> 1) .. + 7 (lanes
  // 0-31 read the first halves of both taps' cells: 6.5x fewer LDS bank
  // conflict cycles than tap-major K groups); output channels 4 kg .. + 3
  const int kg = lane >> 4;
  constexpr bool MAXV = MAXG > 0;
  constexpr int MG = MAXG > 0 ? MAXG : 1;
  constexpr int NMX = 4 / MG;                         // running-max slots per lane (4 channels)

  for (int i = tid; i < C::COUT; i += C::NT) {
    smax[i] = 0u;
    sbias[i] = BIAS ? args.bias[i] : 0.f;
  }

  // B: this lane's cell column in a slice row for each dx, and the half of
  // the cell it reads (the 16-byte halves swap when bit 3 of the column is set)
  int bcol[C::KS];
#pragma unroll
  for (int dx = 0; dx < C::KS; ++dx) {
    const int c = l16 + dx;
    bcol[dx] = c * 32 + 16 * ((kg >> 1) ^ ((c >> 3) & 1));
  }
  const bool second = (kg & 1) != 0;                  // the lane reads the pair's second tap
  // this lane's B offset from slice row w for pair p; the empty half reads
  // the first tap's cells (finite values times zero weights)
  auto pair_off = [&](int p) __attribute__((always_inline)) -> int {
    const int ta = k5_pair_tap(p, 0), t1 = k5_pair_tap(p, 1);
    const int tb = t1 < 0 ? ta : t1;
    const int oa = (ta / C::KS) * (C::SW * 32) + bcol[ta % C::KS];
    const int ob = (tb / C::KS) * (C::SW * 32) + bcol[tb % C::KS];
    return second ? ob : oa;
  };

  // jobs are dealt per XCD (workgroup b runs on XCD b mod 8): XCD x takes the
  // contiguous range [xcd_begin[x], xcd_begin[x + 1]), which the host cuts at
  // equal cost (a job streams its shard's whole depth, and shards differ in
  // depth), strided over that XCD's workgroups
  int j0 = blockIdx.x, jstride = gridDim.x, j_end = args.total_tiles;
  if (gridDim.x >= 8 && (gridDim.x & 7) == 0) {
    const int xcd = blockIdx.x & 7;
    j0 = args.xcd_begin[xcd] + (blockIdx.x >> 3);
    jstride = gridDim.x >> 3;
    j_end = args.xcd_begin[xcd + 1];
  }

  float runmax[NMX];
#pragma unroll
  for (int i = 0; i < NMX; ++i) runmax[i] = 0.f;
  int cur_n = -1;
  auto flush = [&](int n) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NMX; ++i) {
      float v = runmax[i];
      v = fmaxf(v, __shfl_xor(v, 1));
      v = fmaxf(v, __shfl_xor(v, 2));
      v = fmaxf(v, __shfl_xor(v, 4));
      v = fmaxf(v, __shfl_xor(v, 8));
      runmax[i] = 0.f;
      // slot i: channels 4 kg + i MG .. + MG - 1, all in one group
      if (l16 == 0) atomicMax(&smax[4 * kg + i * MG], __float_as_uint(v));
    }
    __syncthreads();
    const int gs = C::COUT / args.groups;
    for (int g = tid; g < args.groups; g += C::NT) {
      uint32_t m = 0;
      for (int c = g * gs; c < (g + 1) * gs; ++c) m = max(m, smax[c]);
      atomicMax(&args.ymax[n * args.groups + g], m);
    }
    __syncthreads();
    for (int i = tid; i < C::COUT; i += C::NT) smax[i] = 0u;
  };


  // A job: shard s, sample n, strip (h0, w0), all planes of the shard
  // job's buffers start at its sample's first plane; each step rebases them
  // at its own first plane so that in-step offsets stay below 2^31
  struct Job {
    int valid, n, h0, w0, depth, e1, e2, p1, p2, gh0, gw0;
    uint32_t in_plane_b, out_plane_b;
    int64_t out_cells, in_bytes, out_bytes;
    const char* in;
    char* out;
  };
  auto make_job = [&](int job) __attribute__((always_inline)) {
    Job J;
    J.valid = job < j_end;
    const int jj = J.valid ? job : j0;
    int s = 0;
    while (s + 1 < args.nshards && args.sh[s + 1].tile_begin <= jj) ++s;
    const ConvShardArg& sh = args.sh[s];
    const int strips = sh.tiles_h * sh.tiles_w;
    int r = jj - sh.tile_begin;
    J.n = r / strips;
    r -= J.n * strips;
    const int sth = r / sh.tiles_w;
    J.h0 = sth * C::BH;
    J.w0 = (r - sth * sh.tiles_w) * C::BW;
    J.depth = sh.ext[0];
    J.e1 = sh.ext[1];
    J.e2 = sh.ext[2];
    const int p0 = sh.pad[0];
    J.p1 = sh.pad[1];
    J.p2 = sh.pad[2];
    J.gh0 = J.h0 + args.origin[1];
    J.gw0 = J.w0 + args.origin[2];
    const int64_t in_plane = (int64_t)J.p1 * J.p2 * C::CIN;
    const int64_t in_base = ((int64_t)J.n * p0 + args.origin[0]) * in_plane;
    const int64_t in_total = (int64_t)args.batch * p0 * in_plane;
    J.in_plane_b = (uint32_t)(in_plane * 2);
    J.in = reinterpret_cast<const char*>(sh.in + in_base);
    J.in_bytes = J.valid ? (in_total - in_base) * 2 : 0;
    J.out_cells = (int64_t)J.e1 * J.e2;
    J.out_plane_b = (uint32_t)(J.out_cells * C::COUT * 4);
    const int64_t out_base = (int64_t)J.n * J.depth * J.out_cells * C::COUT;
    J.out = reinterpret_cast<char*>(sh.out + out_base);
    J.out_bytes = J.valid ? (int64_t)J.depth * J.out_cells * C::COUT * 4 : 0;
    return J;
  };
  // input planes from c0 up to the shard's last padded plane (depth + k - 2):
  // reads past it return zeros, so plane bounds need no per-lane test
  auto in_rsrc = [&](const Job& J, int c0, bool any = true) __attribute__((always_inline)) {
    const int64_t left = (int64_t)(J.depth + C::KS - 1 - c0) * J.in_plane_b;
    const int64_t rest = J.in_bytes - (int64_t)c0 * J.in_plane_b;
    return make_rsrc(J.in + (int64_t)c0 * J.in_plane_b, any ? (left < rest ? left : rest) : 0);
  };
  // 16-byte piece u of a step's TS new planes, ordered (row, plane, column,
  // half) so that the first half of the pieces holds slice rows 0-3: those
  // rows of the ring are free once row 3 of the kernel is done, rows 4-7 only
  // at the end of the step.  Offset from the step's first plane (kOob outside
  // the strip's padded rows and columns), and LDS position for ring slot
  // base + plane.
  auto step_off = [&](const Job& J, int u) __attribute__((always_inline)) -> uint32_t {
    const int h = u & 1;
    int t = u >> 1;
    const int qc = t % C::SW;
    t /= C::SW;
    const int rel = t % C::TS, qr = t / C::TS;
    const int gh = J.gh0 + qr, gw = J.gw0 + qc;
    const bool ok = gh < J.p1 && gw < J.p2;
    return ok ? (uint32_t)(C::RING + rel) * J.in_plane_b + (uint32_t)((gh * J.p2 + gw) * C::CB + 16 * h) : kOob;
  };
  auto step_lds = [&](int u, int base) __attribute__((always_inline)) -> int {
    const int h = u & 1;
    int t = u >> 1;
    const int qc = t % C::SW;
    t /= C::SW;
    const int rel = t % C::TS, qr = t / C::TS;
    int sl = base + rel;
    sl -= sl >= C::RING ? C::RING : 0;
    return sl * C::SLICE_B + (qr * C::SW + qc) * 32 + 16 * (h ^ ((qc >> 3) & 1));
  };
  // weights of segment s -> a stage, by LDS-DMA: the packed segments lie
  // WSTAGE apart, already in LDS order
  auto fetch_w = [&](char* dst, int s) __attribute__((always_inline)) {
    const int nj = k5_seg_pairs(s) * C::KS;           // 1 KiB transfers
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(reinterpret_cast<const char*>(args.w) + s * C::WSTAGE, nj * 1024);
    typedef __attribute__((address_space(3))) void* lds_ptr;
#pragma unroll
    for (int i = 0; i < (C::SLOTS * C::KS + C::NWAVES - 1) / C::NWAVES; ++i) {
      const int j = w + i * C::NWAVES;
      if (j < nj)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(dst + j * 1024), 16, (uint32_t)(j * 1024 + lane * 16),
                                                 0, 0, 0);
    }
  };

  // a job's first RING planes -> ring slots 0 .. RING-1 by LDS-DMA: the ring
  // is RING * SLICE_B = whole KiB, and transfer j of 1 KiB fills LDS bytes
  // [j KiB, (j+1) KiB); each lane fetches the 16 bytes its position holds
  // (the swizzled half of its cell), out-of-strip lanes read zeros
  auto prologue = [&](const Job& Jb) __attribute__((always_inline)) {
    static_assert(C::LDS_X % 1024 == 0, "ring in whole KiB");
    constexpr int NCH = C::LDS_X / 1024;
    const __amdgpu_buffer_rsrc_t rin0 = in_rsrc(Jb, 0);
    typedef __attribute__((address_space(3))) void* lds_ptr;
#pragma unroll
    for (int k = 0; k < (NCH + C::NWAVES - 1) / C::NWAVES; ++k) {
      const int j = w + k * C::NWAVES;
      if (j < NCH) {
        const int p = 64 * j + lane;                  // 16-byte position in the ring
        const int sl = p / (C::SLICE * 2), pc = p - sl * C::SLICE * 2;
        const int q = pc >> 1, qr = q / C::SW, qc = q - qr * C::SW;
        const int h = (pc & 1) ^ ((qc >> 3) & 1);
        const int gh = Jb.gh0 + qr, gw = Jb.gw0 + qc;
        const uint32_t off = (gh < Jb.p1 && gw < Jb.p2)
                                 ? (uint32_t)sl * Jb.in_plane_b + (uint32_t)((gh * Jb.p2 + gw) * C::CB + 16 * h)
                                 : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rin0, (lds_ptr)(sring + j * 1024), 16, off, 0, 0, 0);
      }
    }
  };


  Job J = make_job(j0);
  if (!J.valid) return;
  fetch_w(sw0, 0);                                    // segments 0-2 of the first step; later ones
  fetch_w(sw1, 1);                                    // are fetched one or two segments ahead
  fetch_w(sw2, 2);
  prologue(J);                                        // first job's first TS + k - 1 planes
  __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0)
  if (MAXV) cur_n = J.n;
  __syncthreads();

  f32x4 acc[C::RW][2];                                // [output plane][column block]
  bf16x8 av[2][C::KS];                                // weights per dz, double-buffered by pair parity
  bf16x8 bv[C::NIN][2];                               // input fragments, each reloaded after its last use
  uint4 pf[C::PFH];                                   // half of the next step's planes
  uint32_t pfo[C::PF];                                // their offsets from the step's first plane
#pragma unroll
  for (int k = 0; k < C::PF; ++k) pfo[k] = step_off(J, tid + k * C::NT);
  int job = j0;
  int cur = 0;                                        // first output plane of the step
  constexpr int NS = 2 * C::RW;                       // stores of one step's epilogue
  for (;;) {
    const bool more = cur + C::TS < J.depth;
    const __amdgpu_buffer_rsrc_t rin = in_rsrc(J, cur, more);   // no planes to fetch in a job's last step
    const __amdgpu_buffer_rsrc_t rout =
        make_rsrc(J.out + (int64_t)cur * J.out_plane_b, J.out_bytes - (int64_t)cur * J.out_plane_b);
    const int base = cur % C::RING;
    int sbase[C::NIN];
#pragma unroll
    for (int r = 0; r < C::NIN; ++r) {
      int sl = base + r;
      sl -= sl >= C::RING ? C::RING : 0;
      sbase[r] = sl * C::SLICE_B + w * (C::SW * 32);
    }
    // segment -> weight stage, the same in every step, so that every LDS
    // address below names its stage at compile time
    auto stage = [&](int s) __attribute__((always_inline)) -> char* {
      return s % 3 == 0 ? sw0 : s % 3 == 1 ? sw1 : sw2;
    };
    auto load_a = [&](int buf, int p, int dz) __attribute__((always_inline)) {
      const int s = k5_seg_of(p);
      const int off = ((p - k5_seg_first(s)) * C::KS + dz) * C::FRAG + lane * 16;
      av[buf][dz] = *reinterpret_cast<const bf16x8*>(stage(s) + off);
    };
    // the plane base goes through an opaque scalar so that the compiler forms
    // each address right before its read instead of keeping one register per
    // (plane, pair) alive across the whole step
    auto load_b = [&](int i, int nb, int po) __attribute__((always_inline)) {
      int rb = sbase[i];
      asm volatile("" : "+s"(rb));
      bv[i][nb] = *reinterpret_cast<const bf16x8*>(sring + rb + po + nb * 512);
    };

    // step start (segment 1's weights are on their way): rows 0-3 of the
    // next step's planes, then pair 0's operands
#pragma unroll
    for (int k = 0; k < C::PFH; ++k)
      pf[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rin, pfo[k], 0, 0));
    {
      const int po = pair_off(0);
#pragma unroll
      for (int dz = 0; dz < C::KS; ++dz) load_a(0, 0, dz);
#pragma unroll
      for (int i = 0; i < C::NIN; ++i) {
        load_b(i, 0, po);
        load_b(i, 1, po);
      }
    }

    // pair p issues the LDS reads of pair p + 1 between its MFMAs: input
    // fragment (i, nb) right after its last use, the weights into the other
    // buffer.  Inside a pair the compiler schedules freely (a scheduling
    // barrier per input plane, as the 32x32 kernels keep, cost 3.5% here).
    static_for<C::NPAIRS>([&](auto pc) __attribute__((always_inline)) {
      constexpr int p = decltype(pc)::value;
      const int cb = p & 1;
      const bool last = p == C::NPAIRS - 1;
      __builtin_amdgcn_sched_barrier(0);
      const int s = k5_seg_of(p);
      if (s < C::NSEG - 1 && p == k5_seg_first(s) + k5_seg_pairs(s) - 1) {
        // the last pair of segment s: segment s + 1 must be complete on every
        // wave before this pair reads the next pair's weights, and past the
        // barrier every wave's reads of segment s's stage are done (this
        // pair's operands are in registers), so that stage takes the next
        // segment that uses it:
        //   s 0: segment 3 -> stage 0     s 1: segment 4 -> stage 1
        //   s 2: next step's segment 2 -> stage 2
        //   s 3: next step's segment 0 -> stage 0 (segment 1 follows at step end)
        // Waits: segment 1 was fetched just before the previous step's NS
        // stores and this step's PFH plane loads; segment 2 is older than
        // segment 1; segments 3 and 4 each have one later fetch (segment 4's
        // or the next segment 2's, nj / 4 transfers per wave or more) behind them.
        // These are the waits the schedule needs; after segments 1-3 the
        // barrier's workgroup fence makes the compiler wait for every transfer
        // in flight as well (a raw barrier behind these waits alone measured
        // 0.4% faster: not worth a barrier the compiler does not see as one).
        constexpr int W0 = NS + C::PFH;
        constexpr int W3 = k5_seg_pairs(4) * C::KS / C::NWAVES;
        constexpr int W4 = k5_seg_pairs(2) * C::KS / C::NWAVES;
        if (s == 0) __builtin_amdgcn_s_waitcnt(0x0F70 | (W0 & 15) | ((W0 >> 4) << 14));
        else if (s == 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (W3 & 15) | ((W3 >> 4) << 14));
        else if (s == 3) __builtin_amdgcn_s_waitcnt(0x0F70 | (W4 & 15) | ((W4 >> 4) << 14));
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        if (s == 0) fetch_w(sw0, 3);
        else if (s == 1) fetch_w(sw1, 4);
        else if (s == 2) fetch_w(sw2, 2);
        else {
          // only kernel row 4 is left (slice rows w + 4): the fetched rows
          // 0-3 of the next step's planes go over the oldest planes, and rows
          // 4-7 start
          if (more) {
#pragma unroll
            for (int k = 0; k < C::PFH; ++k)
              *reinterpret_cast<uint4*>(sring + step_lds(tid + k * C::NT, base)) = pf[k];
          }
          fetch_w(sw0, 0);
#pragma unroll
          for (int k = 0; k < C::PFH; ++k)
            pf[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rin, pfo[C::PFH + k], 0, 0));
        }
      }
      const int po = last ? 0 : pair_off(p + 1);
#pragma unroll
      for (int i = 0; i < C::NIN; ++i) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
          for (int dz = 0; dz < C::KS; ++dz) {
            const int o = i - dz;
            if (o >= 0 && o < C::RW) {
              if (p == 0 && dz == 0)
                acc[o][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[cb][dz], bv[i][nb], f32x4{}, 0, 0, 0);
              else
                acc[o][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[cb][dz], bv[i][nb], acc[o][nb], 0, 0, 0);
            }
          }
          if (!last) load_b(i, nb, po);
        }
        if (!last && i < C::KS) load_a(cb ^ 1, p + 1, i);
      }
    });

    // every wave is done with segment 4's stage and with slice rows 4-7 of
    // the ring, and the next step's segment 0 (fetched at segment 3) and
    // planes are complete: segment 1 goes to stage 1 ahead of the stores, so
    // that waiting for it never waits for them, and rows 4-7 of the fetched
    // planes go over the oldest TS before the stores too (after them, the LDS
    // writes wait behind the stores' data: 1.1% on the 512^3 volume).  No
    // barrier follows: until its first barrier the next step reads only
    // slice rows 0-3 (its first two pairs are kernel row 0: wave w reads row
    // w), and every wave's writes are complete (lgkmcnt(0)) before that
    // barrier.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    fetch_w(sw1, 1);
    if (more) {
#pragma unroll
      for (int k = 0; k < C::PFH; ++k)
        *reinterpret_cast<uint4*>(sring + step_lds(tid + (C::PFH + k) * C::NT, base)) = pf[k];
    }

    // epilogue: lane (kg, l16) of acc[o][nb] holds output channels 4 kg .. + 3
    // of position 16 nb + l16 in plane cur + o, so each store writes 16 whole
    // 64-byte cells (1 KiB in a row); planes past the shard fall outside the
    // output descriptor's range
    {
      const int oh = J.h0 + w;
      const int64_t row_cell = (int64_t)oh * J.e2 + J.w0;
      const bool row_in = oh < J.e1;
      float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (BIAS) b4 = *reinterpret_cast<const float4*>(&sbias[4 * kg]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const bool col_in = row_in && J.w0 + 16 * nb + l16 < J.e2;
        const uint32_t cell_b = (uint32_t)((row_cell + 16 * nb + l16) * (C::COUT * 4)) + 16 * kg;
#pragma unroll
        for (int o = 0; o < C::RW; ++o) {
          f32x4 v = acc[o][nb];
          if (BIAS) {
            v[0] += b4.x; v[1] += b4.y; v[2] += b4.z; v[3] += b4.w;
          }
          if (MAXV) {
            const bool real = col_in && cur + o < J.depth;
#pragma unroll
            for (int e = 0; e < 4; ++e) runmax[e / MG] = fmaxf(runmax[e / MG], real ? fabsf(v[e]) : 0.f);
          }
          const uint32_t off = col_in ? (uint32_t)o * J.out_plane_b + cell_b : kOob;
          // non-temporal (cache policy NT), as the streamed outputs elsewhere
          __builtin_amdgcn_raw_buffer_store_b128(v, rout, off, 0, 2);
        }
      }
    }

    if (more) {
      cur += C::TS;
    } else {
      job += jstride;
      const Job N = make_job(job);
      if (!N.valid) break;
      if (MAXV && N.n != cur_n) {
        flush(cur_n);
        cur_n = N.n;
      }
      J = N;
      cur = 0;
#pragma unroll
      for (int k = 0; k < C::PF; ++k) pfo[k] = step_off(J, tid + k * C::NT);
      // the new job's first planes go over the whole ring (every wave is
      // past the step's last reads: the barrier after the pairs)
      prologue(J);
      __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt(0)
      __syncthreads();
    }
  }
  if (MAXV && cur_n >= 0) flush(cur_n);
}

template <class C>
st_status run_taps(ConvArgs& a, const st_plan* in_plan, hipStream_t stream) {
  int jobs = 0;
  for (size_t s = 0; s < in_plan->shards.size(); ++s) {
    const Shard& sd = in_plan->shards[s];
    ConvShardArg& sh = a.sh[s];
    // in-step offsets span RING + TS input planes and TS output planes
    const int64_t in_plane_b = (int64_t)sd.pad[1] * sd.pad[2] * C::CIN * 2;
    const int64_t out_plane_b = (int64_t)sd.ext[1] * sd.ext[2] * C::COUT * 4;
    if (in_plane_b * (C::RING + C::TS) >= 0x7FFFFFFF || out_plane_b * C::TS >= 0x7FFFFFFF)
      return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: shard planes too large for the tap-pair kernel");
    sh.tiles_d = 1;
    sh.tiles_h = (int)((sd.ext[1] + C::BH - 1) / C::BH);
    sh.tiles_w = (int)((sd.ext[2] + C::BW - 1) / C::BW);
    sh.tile_begin = jobs;
    const int64_t t = (int64_t)in_plan->batch * sh.tiles_h * sh.tiles_w;
    if ((int64_t)jobs + t > INT32_MAX) return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: too many jobs");
    jobs += (int)t;
  }
  a.total_tiles = jobs;
  if (jobs == 0) return ST_OK;
  int grid = std::min(jobs, device_cus());
  if (grid >= 8) grid &= ~7;
  // cut the job list into 8 contiguous ranges of equal cost: a job costs its
  // steps (its shard's depth over TS, rounded up) plus about a quarter step
  // for the job switch; with the 512^3 volume's eight depth shards (54-79
  // planes) equal job counts left the XCD of the deepest shard 19% above the
  // mean
  {
    auto cost = [&](size_t s) { return 4 * (((int64_t)in_plan->shards[s].ext[0] + C::TS - 1) / C::TS) + 1; };
    int64_t total_cost = 0;
    for (size_t s = 0; s < in_plan->shards.size(); ++s)
      total_cost += cost(s) * ((int64_t)in_plan->batch * a.sh[s].tiles_h * a.sh[s].tiles_w);
    a.xcd_begin[0] = 0;
    a.xcd_begin[8] = jobs;
    for (int x = 1; x < 8; ++x) {
      const int64_t target = total_cost * x / 8;
      int64_t cum = 0;
      int32_t at = jobs;
      for (size_t s = 0; s < in_plan->shards.size(); ++s) {
        const int64_t n = (int64_t)in_plan->batch * a.sh[s].tiles_h * a.sh[s].tiles_w, c = cost(s);
        if (cum + n * c >= target) {
          at = a.sh[s].tile_begin + (int32_t)std::min<int64_t>(n, (target - cum + c - 1) / c);
          break;
        }
        cum += n * c;
      }
      a.xcd_begin[x] = std::max(a.xcd_begin[x - 1], std::min(at, jobs));
    }
  }
  const int gs = a.ymax ? C::COUT / a.groups : 0;
  const int g = a.ymax == nullptr ? 0 : gs % 4 == 0 ? 4 : gs % 2 == 0 ? 2 : 1;
  const dim3 gd(grid), bd(C::NT);
  if (a.bias) {
    if (g == 4) hipLaunchKernelGGL((conv_taps<C, true, 4>), gd, bd, 0, stream, a);
    else if (g == 2) hipLaunchKernelGGL((conv_taps<C, true, 2>), gd, bd, 0, stream, a);
    else if (g == 1) hipLaunchKernelGGL((conv_taps<C, true, 1>), gd, bd, 0, stream, a);
    else hipLaunchKernelGGL((conv_taps<C, true, 0>), gd, bd, 0, stream, a);
  } else {
    if (g == 4) hipLaunchKernelGGL((conv_taps<C, false, 4>), gd, bd, 0, stream, a);
    else if (g == 2) hipLaunchKernelGGL((conv_taps<C, false, 2>), gd, bd, 0, stream, a);
    else if (g == 1) hipLaunchKernelGGL((conv_taps<C, false, 1>), gd, bd, 0, stream, a);
    else hipLaunchKernelGGL((conv_taps<C, false, 0>), gd, bd, 0, stream, a);
  }
  return launch_check("st_conv_sharded: conv_taps launch");
}

template <class C>
constexpr Instance inst_taps() {
  return Instance{C::NDIM, C::CIN, C::COUT, C::KS, C::CK, C::KVP, C::NT,
                  1, C::BH, C::BW, 1, C::LDS, &run_taps<C>, 0, 3};
}

// 2D 256->256 k3: 4x96 output tiles x 128 output channels, 16-channel K chunks
using GemmImg256 = GemmCfg<256, 256, 3, 4, 96, 128>;
// 3D 16->16 k5: 4x32 strips, 8 output planes per step, whole shard depth per job
using TapsVol16k5 = TapsCfg<4, 8>;
// 2D 64->64 k3: 64-column strips, 8 rows per step (4 per wave), 32 or 24 rows per job, 4
// waves, two passes over K per step (32 output channels each)
using RowsImg64 = RowsCfg<2, 64, 64, 3, 1, 64, 8, 32, 4, 2>;
using RowsImg64J24 = RowsCfg<2, 64, 64, 3, 1, 64, 8, 24, 4, 2>;
// 3D 32->32 k3: 4x32 strips, 4 planes per step (all per wave), 16 planes per job, 4 waves
using RowsVol32 = RowsCfg<3, 32, 32, 3, 4, 32, 4, 16, 4, 1>;

// The streaming kernel deals its jobs statically (a contiguous eighth per XCD,
// strided over that XCD's workgroups), so the slowest workgroup sets the
// time.  rows_deal_cost replays that deal for a job height and returns the
// most slices any workgroup streams, counting each job's k - 1 prologue
// slices.  The job height does not change any output: each output's
// accumulation order depends only on its taps.
template <class C>
int64_t rows_deal_cost(const st_plan* p, int cus) {
  constexpr int RA = C::NDIM == 3 ? 0 : 1;
  std::vector<int32_t> cost;
  for (const Shard& sd : p->shards) {
    const int64_t rows = sd.ext[RA];
    const int64_t chunks = (rows + C::RC - 1) / C::RC;
    const int64_t strips = (C::NDIM == 3 ? (sd.ext[1] + C::BH - 1) / C::BH : 1) * ((sd.ext[2] + C::BW - 1) / C::BW);
    for (int64_t n = 0; n < p->batch; ++n)
      for (int64_t c = 0; c < chunks; ++c) {
        const int64_t r = std::min<int64_t>(C::RC, rows - c * C::RC);
        const int32_t steps = (int32_t)((r + C::TS - 1) / C::TS);
        for (int64_t t = 0; t < strips; ++t) cost.push_back(steps * C::TS + C::KS - 1);
        if (cost.size() > (1u << 22)) return INT64_MAX;          // too many jobs to replay: no preference
      }
  }
  const int64_t total = (int64_t)cost.size();
  int grid = (int)std::min<int64_t>(total, cus);
  if (grid >= 8) grid &= ~7;
  if (grid < 1) return 0;
  std::vector<int64_t> load(grid, 0);
  if (grid >= 8 && (grid & 7) == 0) {
    const int per = grid >> 3;
    for (int x = 0; x < 8; ++x) {
      const int64_t b = total * x / 8, e = total * (x + 1) / 8;
      for (int64_t j = b; j < e; ++j) load[x + 8 * (int)((j - b) % per)] += cost[j];
    }
  } else {
    for (int64_t j = 0; j < total; ++j) load[j % grid] += cost[j];
  }
  return *std::max_element(load.begin(), load.end());
}

// image 64->64: the job height with the better-balanced deal for this plan
st_status run_rows_img64(ConvArgs& a, const st_plan* in_plan, hipStream_t stream) {
  const int cus = device_cus();
  if (rows_deal_cost<RowsImg64J24>(in_plan, cus) < rows_deal_cost<RowsImg64>(in_plan, cus))
    return run_rows<RowsImg64J24>(a, in_plan, stream);
  return run_rows<RowsImg64>(a, in_plan, stream);
}

template <class C>
constexpr Instance inst_rows_with(st_status (*run)(ConvArgs&, const st_plan*, hipStream_t)) {
  Instance i = inst_rows<C>();
  i.run = run;
  return i;
}

// one matrix-core instance per supported (ndim, cin, cout, k)
const Instance kInstances[] = {
    inst_rows_with<RowsImg64>(&run_rows_img64),
    inst_rows<RowsVol32>(),
    inst_taps<TapsVol16k5>(),
    inst_gemm<GemmImg256>(),
};

const Instance* find_instance(int ndim, int cin, int cout, int ks) {
  for (const Instance& i : kInstances)
    if (i.ndim == ndim && i.cin == cin && i.cout == cout && i.ks == ks) return &i;
  return nullptr;
}

int64_t taps_of(int ndim, int ks) { return ndim == 3 ? (int64_t)ks * ks * ks : (int64_t)ks * ks; }

// Packs raw [Cout][Cin][k^d] weights into the layout of the kernel that runs
// this shape and zeroes clr[0, nclr) in the same launch.
st_status pack_weights(int ndim, int cin, int cout, int ksize, st_dtype dtype, const void* weight, void* packed,
                       uint32_t* clr, int nclr, hipStream_t st, const char* who) {
  const int taps = (int)taps_of(ndim, ksize);
  const std::string what = std::string(who) + ": weight packing launch";
  auto grid = [&](int64_t total) { return dim3((unsigned)((std::max<int64_t>(total, nclr) + 255) / 256)); };
  if (dtype == ST_BF16) {
    const uint16_t* w = static_cast<const uint16_t*>(weight);
    uint16_t* out = static_cast<uint16_t*>(packed);
    if (const Instance* i = find_instance(ndim, cin, cout, ksize)) {
      if (i->kind == 3) {
        const int64_t total = (int64_t)(cin / i->ck) * cout * i->kvp;
        hipLaunchKernelGGL(pack_w_taps, grid(total), dim3(256), 0, st, w, out, total, clr, nclr);
        return launch_check(what.c_str());
      }
      if (i->kind == 1) {
        const int64_t total = (int64_t)cout * taps * cin;
        hipLaunchKernelGGL(pack_w_gemm, grid(total), dim3(256), 0, st, w, out, cin, cout, taps, i->ck, i->bn, total,
                           clr, nclr);
        return launch_check(what.c_str());
      }
      const int64_t total = (int64_t)(cin / i->ck) * cout * i->kvp;
      hipLaunchKernelGGL(pack_w_mfma, grid(total), dim3(256), 0, st, w, out, cin, cout, taps, i->ck, i->kvp, total,
                         clr, nclr);
      return launch_check(what.c_str());
    }
  }
  // every other shape (the matrix-core 'same' conv and the direct kernel):
  // fp32 [taps][Cin][Cout]
  return pack_tab_launch(weight, dtype, static_cast<float*>(packed), cin, cout, taps, false, clr, nclr, st, who);
}

// Host checks shared by the conv entry points; nothing is enqueued.
st_status conv_check(const char* who, const st_plan* in_plan, const void* const* in_bufs, const void* weight,
                     const float* bias, int32_t cout, int32_t ksize, float* const* y_bufs, const uint32_t* ymax,
                     int32_t groups) {
  auto err = [&](st_status s, const char* m) { return fail(s, std::string(who) + ": " + m); };
  if (!in_plan || !in_bufs || !y_bufs || !weight) return err(ST_ERR_INVALID_ARG, "NULL argument");
  if (ksize < 1 || ksize % 2 == 0) return err(ST_ERR_UNSUPPORTED, "kernel size must be odd");
  if (cout < 1) return err(ST_ERR_INVALID_ARG, "cout < 1");
  const int ndim = in_plan->ndim;
  for (int a = kAxes - ndim; a < kAxes; ++a)
    if (in_plan->halo[a] < ksize / 2) return err(ST_ERR_BAD_SHAPE, "input halo narrower than ksize/2");
  if (ymax && (groups < 1 || cout % groups != 0)) return err(ST_ERR_INVALID_ARG, "groups must divide cout");
  if (!aligned16(weight) || (bias && !aligned16(bias)) || (ymax && (reinterpret_cast<uintptr_t>(ymax) & 3)))
    return err(ST_ERR_ALIGNMENT, "misaligned weight/bias/ymax");
  for (size_t s = 0; s < in_plan->shards.size(); ++s) {
    if (!in_bufs[s] || !y_bufs[s]) return err(ST_ERR_INVALID_ARG, "NULL shard buffer");
    if (!aligned16(in_bufs[s]) || !aligned16(y_bufs[s]))
      return err(ST_ERR_ALIGNMENT, "shard buffers must be 16-byte aligned");
    for (int a = 0; a < kAxes; ++a)
      if (in_plan->shards[s].pad[a] > INT32_MAX / 2) return err(ST_ERR_UNSUPPORTED, "extent too large");
  }
  return ST_OK;
}

// Launches the conv of every shard from packed weights (arguments checked).
// y of shard s: unpadded channels-last fp32 [N][ext...][cout].
st_status conv_run(const st_plan* in_plan, const void* const* in_bufs, const void* packed_weight,
                   const float* bias_or_null, int32_t cout, int32_t ksize, float* const* y_bufs,
                   uint32_t* ymax_or_null, int32_t groups, hipStream_t st) {
  const int ndim = in_plan->ndim;
  const int cin = (int)in_plan->channels;
  const Instance* inst = in_plan->dtype == ST_BF16 ? find_instance(ndim, cin, cout, ksize) : nullptr;
  if (inst) {
    ConvArgs a{};
    a.nshards = (int)in_plan->shards.size();
    a.groups = groups;
    a.batch = (int)in_plan->batch;
    for (int ax = 0; ax < kAxes; ++ax) {
      const bool real = ax >= kAxes - ndim;
      a.origin[ax] = real ? in_plan->halo[ax] - ksize / 2 : 0;
    }
    a.w = static_cast<const uint16_t*>(packed_weight);
    a.bias = bias_or_null;
    a.ymax = ymax_or_null;
    for (size_t s = 0; s < in_plan->shards.size(); ++s) {
      const Shard& sd = in_plan->shards[s];
      ConvShardArg& sh = a.sh[s];
      sh.in = static_cast<const uint16_t*>(in_bufs[s]);
      sh.out = y_bufs[s];
      for (int ax = 0; ax < kAxes; ++ax) {
        sh.ext[ax] = (int)sd.ext[ax];
        sh.pad[ax] = (int)sd.pad[ax];
      }
    }
    return inst->run(a, in_plan, st);
  }

  if (in_plan->dtype == ST_BF16 && cout <= 1024 && sx_same_fits(ndim, cin, cout, ksize)) {
    // the matrix-core implicit GEMM of the strided conv at stride 1, then
    // max |y| in a pass of its own
    st_status s = sx_same_conv(in_plan, in_bufs, static_cast<const float*>(packed_weight), bias_or_null, cout, ksize,
                               y_bufs, st);
    if (s != ST_OK || !ymax_or_null) return s;
    YmaxArgs m{};
    m.nshards = (int)in_plan->shards.size();
    m.batch = (int)in_plan->batch;
    m.cout = cout;
    m.groups = groups;
    m.ymax = ymax_or_null;
    int64_t most = 0;
    for (size_t i = 0; i < in_plan->shards.size(); ++i) {
      const Shard& sd = in_plan->shards[i];
      m.y[i] = y_bufs[i];
      m.positions[i] = sd.ext[0] * sd.ext[1] * sd.ext[2];
      most = std::max(most, m.positions[i]);
    }
    const int per_block = 256 / (cout / 4);
    const int64_t gx = std::min<int64_t>((most + per_block - 1) / per_block,
                                         std::max<int64_t>(1, 4 * device_cus() / (m.nshards * m.batch)));
    if (most == 0) return ST_OK;
    if ((int64_t)m.nshards * m.batch > 65535) return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: batch too large");
    hipLaunchKernelGGL(ymax_pass, dim3((unsigned)std::max<int64_t>(1, gx), (unsigned)(m.nshards * m.batch)), dim3(256),
                       0, st, m);
    return launch_check("st_conv_sharded: max |y| launch");
  }

  DirectArgs a{};
  a.nshards = (int)in_plan->shards.size();
  a.cin = cin;
  a.cout = cout;
  a.ks = ksize;
  a.taps = (int)taps_of(ndim, ksize);
  a.groups = ymax_or_null ? groups : 1;
  for (int ax = 0; ax < kAxes; ++ax) {
    const bool real = ax >= kAxes - ndim;
    a.origin[ax] = real ? in_plan->halo[ax] - ksize / 2 : 0;
  }
  a.w = static_cast<const float*>(packed_weight);
  a.bias = bias_or_null;
  a.ymax = ymax_or_null;
  int64_t pos = 0;
  for (size_t s = 0; s < in_plan->shards.size(); ++s) {
    const Shard& sd = in_plan->shards[s];
    DirectShardArg& sh = a.sh[s];
    sh.in = in_bufs[s];
    sh.out = y_bufs[s];
    sh.pos_begin = pos;
    for (int ax = 0; ax < kAxes; ++ax) {
      sh.ext[ax] = (int)sd.ext[ax];
      sh.pad[ax] = (int)sd.pad[ax];
    }
    pos += in_plan->batch * sd.ext[0] * sd.ext[1] * sd.ext[2];
  }
  a.total_pos = pos;
  if (pos == 0) return ST_OK;
  // a thread per (position, 4 output channels) when Cout allows; 16-byte
  // input loads when Cin allows; weights in LDS when they fit
  const int ob = cout % 4 == 0 ? 4 : 1;
  const int64_t blocks = (pos * (cout / ob) + 255) / 256;
  if (blocks > INT32_MAX) return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: volume too large for the direct kernel");
  const size_t wbytes = (size_t)a.taps * cin * cout * 4;
  const bool wl = wbytes + (size_t)cout * 4 <= 64 * 1024;
  const size_t shmem = (wl ? wbytes : 0) + (size_t)cout * 4;
  if (shmem > 64 * 1024) return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: cout too large for the direct kernel");
  const bool bf = in_plan->dtype == ST_BF16;
  const bool vec = bf ? cin % 8 == 0 : cin % 4 == 0;
  const dim3 gd((unsigned)blocks), bd(256);
#define ST_DIRECT(T_, CV_)                                                                              \
  do {                                                                                                  \
    if (ob == 4) {                                                                                      \
      if (wl) hipLaunchKernelGGL((conv_direct<T_, 4, CV_, true>), gd, bd, shmem, st, a);                  \
      else hipLaunchKernelGGL((conv_direct<T_, 4, CV_, false>), gd, bd, shmem, st, a);                    \
    } else {                                                                                            \
      if (wl) hipLaunchKernelGGL((conv_direct<T_, 1, CV_, true>), gd, bd, shmem, st, a);                  \
      else hipLaunchKernelGGL((conv_direct<T_, 1, CV_, false>), gd, bd, shmem, st, a);                    \
    }                                                                                                   \
  } while (0)
  if (bf) {
    if (vec) ST_DIRECT(uint16_t, 8);
    else ST_DIRECT(uint16_t, 1);
  } else {
    if (vec) ST_DIRECT(float, 4);
    else ST_DIRECT(float, 1);
  }
#undef ST_DIRECT
  return launch_check("st_conv_sharded: conv_direct launch");
}

}  // namespace
}  // namespace st

using namespace st;

extern "C" {

size_t st_conv_weight_bytes(int32_t ndim, int32_t cin, int32_t cout, int32_t ksize, st_dtype dtype) {
  if ((ndim != 2 && ndim != 3) || cin < 1 || cout < 1 || ksize < 1 || ksize % 2 == 0) return 0;
  if (dtype != ST_F32 && dtype != ST_BF16) return 0;
  const int64_t taps = taps_of(ndim, ksize);
  if (dtype == ST_BF16)
    if (const Instance* i = find_instance(ndim, cin, cout, ksize)) return (size_t)(cin / i->ck) * cout * i->kvp * 2;
  // every other shape: fp32 [taps][Cin][Cout]
  return (size_t)cout * taps * cin * 4;
}

st_status st_conv_pack_weights(int32_t ndim, int32_t cin, int32_t cout, int32_t ksize,
                               st_dtype dtype, const void* weight, void* packed, void* stream) {
  const size_t bytes = st_conv_weight_bytes(ndim, cin, cout, ksize, dtype);
  if (bytes == 0) return fail(ST_ERR_UNSUPPORTED, "st_conv_pack_weights: unsupported ndim/ksize/dtype");
  if (!weight || !packed) return fail(ST_ERR_INVALID_ARG, "st_conv_pack_weights: NULL pointer");
  if (!aligned16(weight) || !aligned16(packed))
    return fail(ST_ERR_ALIGNMENT, "st_conv_pack_weights: pointers must be 16-byte aligned");
  return pack_weights(ndim, cin, cout, ksize, dtype, weight, packed, nullptr, 0, static_cast<hipStream_t>(stream),
                      "st_conv_pack_weights");
}

st_status st_conv_dgrad_weights(int32_t ndim, int32_t cin, int32_t cout, int32_t ksize, st_dtype dtype,
                                const void* weight, void* out, void* stream) {
  if ((ndim != 2 && ndim != 3) || cin < 1 || cout < 1 || ksize < 1 || ksize % 2 == 0)
    return fail(ST_ERR_UNSUPPORTED, "st_conv_dgrad_weights: unsupported ndim/ksize");
  if (dtype != ST_F32 && dtype != ST_BF16) return fail(ST_ERR_UNSUPPORTED, "st_conv_dgrad_weights: dtype");
  if (!weight || !out) return fail(ST_ERR_INVALID_ARG, "st_conv_dgrad_weights: NULL pointer");
  if (weight == out) return fail(ST_ERR_INVALID_ARG, "st_conv_dgrad_weights: in place is not supported");
  const int taps = (int)taps_of(ndim, ksize);
  const int64_t total = (int64_t)cout * cin * taps;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 gd((unsigned)((total + 255) / 256)), bd(256);
  if (dtype == ST_BF16)
    hipLaunchKernelGGL(dgrad_weights<uint16_t>, gd, bd, 0, st, static_cast<const uint16_t*>(weight),
                       static_cast<uint16_t*>(out), cin, cout, taps, total);
  else
    hipLaunchKernelGGL(dgrad_weights<float>, gd, bd, 0, st, static_cast<const float*>(weight),
                       static_cast<float*>(out), cin, cout, taps, total);
  return launch_check("st_conv_dgrad_weights: launch");
}

size_t st_conv_workspace_bytes(const st_plan* in_plan, int32_t cout, int32_t ksize) {
  if (!in_plan) return 0;
  const size_t w = st_conv_weight_bytes(in_plan->ndim, (int32_t)in_plan->channels, cout, ksize, in_plan->dtype);
  return w == 0 ? 0 : (w + 255) / 256 * 256;
}

st_status st_conv_sharded(const st_plan* in_plan, const void* const* in_bufs, const void* weight,
                          const float* bias_or_null, int32_t cout, int32_t ksize, float* const* y_bufs,
                          uint32_t* ymax_or_null, int32_t groups, void* workspace, size_t workspace_bytes,
                          void* stream) {
  static const char* who = "st_conv_sharded";
  st_status s = conv_check(who, in_plan, in_bufs, weight, bias_or_null, cout, ksize, y_bufs, ymax_or_null, groups);
  if (s != ST_OK) return s;
  const size_t need = st_conv_workspace_bytes(in_plan, cout, ksize);
  if (need == 0) return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: unsupported ndim/ksize/dtype");
  if (!workspace || workspace_bytes < need)
    return fail(ST_ERR_WORKSPACE, "st_conv_sharded: workspace missing or smaller than st_conv_workspace_bytes");
  if (!aligned16(workspace)) return fail(ST_ERR_ALIGNMENT, "st_conv_sharded: workspace not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // one launch packs the weights into the workspace and clears max |y|
  const int nclr = ymax_or_null ? (int)(in_plan->batch * groups) : 0;
  s = pack_weights(in_plan->ndim, (int)in_plan->channels, cout, ksize, in_plan->dtype, weight, workspace,
                   ymax_or_null, nclr, st, who);
  if (s != ST_OK) return s;
  return conv_run(in_plan, in_bufs, workspace, bias_or_null, cout, ksize, y_bufs, ymax_or_null, groups, st);
}

st_status st_conv_sharded_packed(const st_plan* in_plan, const void* const* in_bufs, const void* packed_weight,
                                 const float* bias_or_null, int32_t cout, int32_t ksize, float* const* y_bufs,
                                 uint32_t* ymax_or_null, int32_t groups, void* stream) {
  static const char* who = "st_conv_sharded_packed";
  st_status s = conv_check(who, in_plan, in_bufs, packed_weight, bias_or_null, cout, ksize, y_bufs, ymax_or_null,
                           groups);
  if (s != ST_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (ymax_or_null) {
    const int n = (int)(in_plan->batch * groups);
    hipLaunchKernelGGL(fill_u32, dim3((n + 255) / 256), dim3(256), 0, st, ymax_or_null, 0u, n);
    s = launch_check("st_conv_sharded_packed: ymax clear");
    if (s != ST_OK) return s;
  }
  return conv_run(in_plan, in_bufs, packed_weight, bias_or_null, cout, ksize, y_bufs, ymax_or_null, groups, st);
}

}  // extern "C"
