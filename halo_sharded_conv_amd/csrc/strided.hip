// Shape-changing sharded op: strided convolution (downsampling conv).
//
// "Technical summary: ShardTensor - domain parallelism for scientific machine
// learning", section 2 "Design principles": each local chunk carries its own
// shape, so an op that changes shapes derives the output chunks from the
// input ones.  For a 'same'-padded cross-correlation with odd window k,
// padding p = k/2 and stride s, output j along an axis reads inputs
// [j*s - p, j*s + p]; it belongs to the shard whose interior holds the
// window's centre j*s, so a shard with interior [a, a + e) owns outputs
// [ceil(a / s), min(ceil((a + e) / s), n_out)) and reads at most p cells
// beyond its interior on either side: the conv's usual halo of k/2 suffices.
//
// st_plan_strided derives the output plan; st_conv_strided_sharded runs one
// launch over every shard: on the matrix cores for bf16 shapes with Cin % 16
// == 0 and Cout % 16 == 0 (conv_sx_mfma, further down), else on fp32
// FMA (a thread takes one output position and up to 64 output channels,
// blockIdx.y picks the channel block, reads the window's input cells once and
// the weights as wave-uniform values).  Both accumulate in a fixed order
// (taps lexicographic, input channels ascending), so an output's bits do not
// depend on the shard plan.
//
// Its adjoint, the transposed (upsampling) convolution, is the same section's
// rule run the other way: input cell i scatters onto outputs i*s + t - p, the
// output has s times the input's extent, and a shard with interior [a, a + e)
// owns outputs [a*s, (a + e)*s).  An output j = q*s + r (phase r in [0, s))
// gathers from the taps t = r + p (mod s), i.e. input cells q + (r + p - t)/s,
// all within p cells of q, so the input's halo of k/2 again suffices.
// st_plan_transposed derives the output plan; st_conv_transposed_sharded runs
// the same matrix-core kernel with every phase of a position block in one
// wave, or the fp32 FMA kernel with one phase per blockIdx.z, so the tap set
// is uniform over a block and the weights stay wave-uniform.
#include <algorithm>
#include <cstdio>
#include <string>
#include <type_traits>

#include "internal.h"

namespace st {
namespace {

constexpr int kMaxTransposedStride = 8;


struct StrShard {
  const char* in;                   // padded input shard at (n=0, window 0's first cell)
  float* out;                       // output interior origin
  int64_t is[3], isn;               // input element strides (d, h, w) and batch stride
  int64_t os[3], osn;               // output element strides
  int32_t oext[3];                  // output interior extents (d, h, w)
  int64_t begin;                    // first output position of this shard
};

struct StrArgs {
  int32_t nshards, batch, cin, cout, k, stride, ndim;
  int64_t total;                    // output positions over all shards and samples
  const float* w;                   // [taps][Cin][Cout] fp32
  const float* bias;                // [Cout] or NULL
  StrShard sh[ST_MAX_SHARDS];
};
static_assert(sizeof(StrArgs) <= kMaxKernargBytes, "kernel argument struct too large");

// CV consecutive input channels as fp32 (one 16-byte load when CV > 1)
template <typename T, int CV> __device__ __forceinline__ void ldc(const T* p, float (&x)[CV]);
template <> __device__ __forceinline__ void ldc<float, 1>(const float* p, float (&x)[1]) { x[0] = *p; }
template <> __device__ __forceinline__ void ldc<float, 4>(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <> __device__ __forceinline__ void ldc<uint16_t, 1>(const uint16_t* p, float (&x)[1]) {
  x[0] = __uint_as_float((uint32_t)*p << 16);
}
template <> __device__ __forceinline__ void ldc<uint16_t, 8>(const uint16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// OB output channels per thread (the largest of 64, 32, ... that divides Cout);
// CV input channels per load (16 bytes when Cin allows)
template <typename TI, int OB, int CV>
__global__ __launch_bounds__(256) void conv_strided_kernel(const StrArgs a) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int o0 = blockIdx.y * OB;
  if (item >= a.total) return;
  int s = 0;
  while (s + 1 < a.nshards && a.sh[s + 1].begin <= item) ++s;
  const StrShard& sh = a.sh[s];
  int64_t r = item - sh.begin;
  const int ow = (int)(r % sh.oext[2]);
  r /= sh.oext[2];
  const int oh = (int)(r % sh.oext[1]);
  r /= sh.oext[1];
  const int od = (int)(r % sh.oext[0]);
  const int n = (int)(r / sh.oext[0]);
  const TI* base = reinterpret_cast<const TI*>(sh.in) + n * sh.isn + (int64_t)od * a.stride * sh.is[0] +
                   (int64_t)oh * a.stride * sh.is[1] + (int64_t)ow * a.stride * sh.is[2];
  float acc[OB];
#pragma unroll
  for (int i = 0; i < OB; ++i) acc[i] = a.bias ? a.bias[o0 + i] : 0.f;
  const int kd = a.ndim == 3 ? a.k : 1;
  const float* wt = a.w + o0;
  for (int tz = 0; tz < kd; ++tz)
    for (int ty = 0; ty < a.k; ++ty)
      for (int tx = 0; tx < a.k; ++tx) {
        const TI* px = base + tz * sh.is[0] + ty * sh.is[1] + tx * sh.is[2];
        for (int c = 0; c < a.cin; c += CV) {
          float x[CV];
          ldc<TI, CV>(px + c, x);
#pragma unroll
          for (int v = 0; v < CV; ++v) {
#pragma unroll
            for (int i = 0; i < OB; ++i) acc[i] = fmaf(wt[i], x[v], acc[i]);
            wt += a.cout;
          }
        }
      }
  float* o = sh.out + n * sh.osn + od * sh.os[0] + oh * sh.os[1] + ow * sh.os[2] + o0;
#pragma unroll
  for (int i = 0; i < OB; ++i) o[i] = acc[i];
}

struct TrShard {
  const char* in;                   // padded input shard at the interior origin (n=0)
  float* out;                       // output interior origin
  int64_t is[3], isn;               // input element strides (d, h, w) and batch stride
  int64_t os[3], osn;               // output element strides
  int32_t iext[3];                  // input interior extents (d, h, w)
  int64_t begin;                    // first input position of this shard
};

struct TrArgs {
  int32_t nshards, batch, cin, cout, k, stride, ndim;
  int64_t total;                    // input positions over all shards and samples (per phase)
  const float* w;                   // [taps][Cin][Cout] fp32, Cin = the input's channels
  const float* bias;                // [Cout] or NULL
  TrShard sh[ST_MAX_SHARDS];
};
static_assert(sizeof(TrArgs) <= kMaxKernargBytes, "kernel argument struct too large");

// Gather form of the transposed conv: blockIdx.z is the output phase
// (rd, rh, rw), a thread takes input position q and writes output q*s + r for
// OB output channels (blockIdx.y picks the block).  Taps of the phase in
// lexicographic order, input channels ascending, fp32 FMA.
template <typename TI, int OB, int CV>
__global__ __launch_bounds__(256) void conv_transposed_kernel(const TrArgs a) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int o0 = blockIdx.y * OB;
  if (item >= a.total) return;
  const int s = a.stride, k = a.k, p = k / 2;
  const bool v3 = a.ndim == 3;
  const int sd = v3 ? s : 1, kd = v3 ? k : 1, pd = kd / 2;
  const int ph = blockIdx.z;
  const int rw = ph % s, rh = (ph / s) % s, rd = v3 ? ph / (s * s) : 0;
  // first tap of the phase per axis and the input offset it reads
  const int t0w = (rw + p) % s, t0h = (rh + p) % s, t0d = (rd + pd) % sd;
  const int dw = (rw + p - t0w) / s, dh = (rh + p - t0h) / s, dd = (rd + pd - t0d) / sd;
  int sh_i = 0;
  while (sh_i + 1 < a.nshards && a.sh[sh_i + 1].begin <= item) ++sh_i;
  const TrShard& sh = a.sh[sh_i];
  int64_t r = item - sh.begin;
  const int qw = (int)(r % sh.iext[2]);
  r /= sh.iext[2];
  const int qh = (int)(r % sh.iext[1]);
  r /= sh.iext[1];
  const int qd = (int)(r % sh.iext[0]);
  const int n = (int)(r / sh.iext[0]);
  const TI* base = reinterpret_cast<const TI*>(sh.in) + n * sh.isn + (int64_t)(qd + dd) * sh.is[0] +
                   (int64_t)(qh + dh) * sh.is[1] + (int64_t)(qw + dw) * sh.is[2];
  float acc[OB];
#pragma unroll
  for (int i = 0; i < OB; ++i) acc[i] = a.bias ? a.bias[o0 + i] : 0.f;
  const int64_t tap_stride = (int64_t)a.cin * a.cout;
  for (int tz = t0d, mz = 0; tz < kd; tz += sd, ++mz)
    for (int ty = t0h, my = 0; ty < k; ty += s, ++my)
      for (int tx = t0w, mx = 0; tx < k; tx += s, ++mx) {
        // tap t reads input cell q + (r + p - t)/s: one cell back per step of s
        const TI* px = base - mz * sh.is[0] - my * sh.is[1] - mx * sh.is[2];
        const float* wt = a.w + ((tz * k + ty) * k + tx) * tap_stride + o0;
        for (int c = 0; c < a.cin; c += CV) {
          float x[CV];
          ldc<TI, CV>(px + c, x);
#pragma unroll
          for (int v = 0; v < CV; ++v) {
#pragma unroll
            for (int i = 0; i < OB; ++i) acc[i] = fmaf(wt[i], x[v], acc[i]);
            wt += a.cout;
          }
        }
      }
  float* o = sh.out + n * sh.osn + (int64_t)(qd * sd + rd) * sh.os[0] + (int64_t)(qh * s + rh) * sh.os[1] +
             (int64_t)(qw * s + rw) * sh.os[2] + o0;
  if constexpr (OB % 4 == 0) {
#pragma unroll
    for (int i = 0; i < OB; i += 4)
      *reinterpret_cast<float4*>(o + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < OB; ++i) o[i] = acc[i];
  }
}

// input offsets (relative to q) an output phase of the transposed conv reads
// along one axis, over all phases: [lo, hi]; false when no phase has a tap
bool transposed_reach(int k, int s, int& lo, int& hi) {
  const int p = k / 2;
  bool any = false;
  lo = 0;
  hi = 0;
  for (int r = 0; r < s; ++r)
    for (int t = (r + p) % s; t < k; t += s) {
      const int off = (r + p - t) / s;
      if (!any) { lo = hi = off; any = true; }
      lo = std::min(lo, off);
      hi = std::max(hi, off);
    }
  return any;
}

// --------------------------------------------------------------------------
// matrix-core path (bf16 operands): implicit GEMM per output phase
// --------------------------------------------------------------------------
//
// M = output channels (A = weights, staged once per workgroup in LDS in
// fragment order), N = 32 output positions per block (B = input cells, one
// 16-byte load of 8 channels per lane straight from the padded shard),
// K = taps x input channels, v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  A wave owns NB x 32 consecutive positions of one shard and
// MB x 32 output channels; every output sums its K steps in the same order
// (bias first, taps lexicographic, channels ascending in blocks of 16), so its
// bits do not depend on the shard plan.  The transposed conv runs every
// output phase of a position block in turn in the same wave (the phases read
// overlapping input cells, which then stay in L1/L2).

typedef __bf16 sx_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sx_f32x16 __attribute__((ext_vector_type(16)));
typedef float sx_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSxTile = 64;                     // positions per wave tile
constexpr bool kSxPrefer16 = true;              // 16x16x32 fragments where Cin % 32 == 0
constexpr int kSxWaves = 4;
constexpr int kSxDepth = 3;                     // K steps of input fragments held per wave

struct SxShard {
  const uint16_t* in;               // strided: first window's first cell; transposed: interior origin
  float* out;                       // output interior origin
  int64_t is[3], isn;               // input element strides
  int64_t os[3], osn;               // output element strides
  int32_t ext[3];                   // position extents (strided: outputs; transposed: inputs)
  int64_t positions;                // batch x ext product
  int64_t tile_begin;               // first wave tile of this shard
};

struct SxArgs {
  int32_t nshards, cin, cout, k, stride, ndim, taps, iters;
  int64_t tiles;                    // wave tiles over all shards
  const float* w;                   // [taps][Cin][Cout] fp32 (bf16 values)
  const float* bias;                // [Cout] or NULL
  SxShard sh[ST_MAX_SHARDS];
};
static_assert(sizeof(SxArgs) <= kMaxKernargBytes, "kernel argument struct too large");

__device__ __forceinline__ uint16_t sx_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// FR = 32: v_mfma_f32_32x32x16_bf16 (lane holds 8 of 16 K for position
// lane % 32); FR = 16: v_mfma_f32_16x16x32_bf16 (8 of 32 K for position
// lane % 16), whose B loads cover 16 cells x 64 bytes instead of 32 cells x
// 32 bytes per instruction.  A wave owns 64 positions and MB x FR channels.
// HALF (FR 32, MB 1, Cout 16): the tile's rows 16-31 are zeros, so LDS holds
// only the 32 lane slots of rows 0-15 per fragment (half the bytes, which
// lets a 3D k5 16-channel layer's weights fit two workgroups per CU) and
// lanes of rows 16-31 take zero operands instead of reading them.
template <int FR, int MB, int KG, bool TR, int CAP, bool HALF = false>
__global__ __launch_bounds__(256, CAP <= 80 * 1024 ? 2 : 1) void conv_sx_mfma(const SxArgs a) {
  using acc_t = typename std::conditional<FR == 32, sx_f32x16, sx_f32x4>::type;
  constexpr int KS = FR == 32 ? 16 : 32;          // channels per K step
  constexpr int NBK = 64 / FR;                    // position blocks per wave
  constexpr int NACC = FR == 32 ? 16 : 4;         // accumulators per block and lane
  static_assert(!HALF || (FR == 32 && MB == 1), "half tiles are single 32-row blocks");
  constexpr int SLOTS = HALF ? 32 : 64;           // stored lane slots per fragment
  constexpr int ROWS = HALF ? 16 : FR;            // stored rows per block
  __shared__ __attribute__((aligned(16))) uint16_t wl[CAP / 2];   // [taps][Cin/KS][MB][SLOTS lanes][8]
  const int KC = a.cin / KS;
  const int ob = blockIdx.y * MB * FR;
  {
    // weights of this channel block, read in global order 4 output channels
    // (16 bytes) at a time, rounded to bf16, written to their fragment slots
    // (4 consecutive output channels are 4 consecutive lanes' slots)
    const int per_tap4 = a.cin * MB * ROWS / 4;
    const int total4 = a.taps * per_tap4;
#pragma unroll 4
    for (int f = threadIdx.x; f < total4; f += blockDim.x) {
      const int t = f / per_tap4;
      const int rem = f - t * per_tap4;
      const int c = rem / (MB * ROWS / 4);
      const int o = (rem - c * (MB * ROWS / 4)) * 4;
      // rows past Cout (a 16-channel layer in a 32-row tile) hold zeros
      const float4 v = ob + o < a.cout ? *reinterpret_cast<const float4*>(a.w + ((int64_t)t * a.cin + c) * a.cout + ob + o)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
      const int l = ((c % KS) >> 3) * ROWS + (o % FR);
      uint16_t* d = wl + ((((t * KC + c / KS) * MB + o / FR) * SLOTS + l) << 3) + (c & 7);
      d[0] = sx_rne(v.x);
      d[8] = sx_rne(v.y);
      d[16] = sx_rne(v.z);
      d[24] = sx_rne(v.w);
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lp = lane % FR, grp = lane / FR;      // position in the block, K group of 8
  const int s = a.stride, k = a.k, p = k / 2;
  const bool v3 = a.ndim == 3;
  const int sd = v3 ? s : 1, kd = v3 ? k : 1, pd = kd / 2;
  const int phases = TR ? s * s * sd : 1;
  // XCD-aware order: consecutive logical workgroups share one XCD's L2
  int g = blockIdx.x;
  if ((gridDim.x & 7) == 0) g = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  // the workgroup's tile groups in the order 0, h, 1, h + 1, ... (h = half):
  // a block two rows tall takes its two rows' matching column segments back
  // to back, so the input rows they share are still in L2
  const int half = (a.iters + 1) >> 1;
  for (int it = 0; it < a.iters; ++it) {
    const int itp = (it & 1) ? half + (it >> 1) : (it >> 1);
    const int64_t tile = ((int64_t)g * a.iters + itp) * kSxWaves + wave;
    if (tile >= a.tiles) continue;
    int si = 0;
    while (si + 1 < a.nshards && a.sh[si + 1].tile_begin <= tile) ++si;
    const SxShard& sh = a.sh[si];
    const int64_t p0 = (tile - sh.tile_begin) * 64;
    int pz[NBK], py[NBK], px[NBK], pn[NBK];
    bool ok[NBK];
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) {
      const int64_t q = p0 + nb * FR + lp;
      ok[nb] = q < sh.positions;
      int64_t r = ok[nb] ? q : 0;
      px[nb] = (int)(r % sh.ext[2]);
      r /= sh.ext[2];
      py[nb] = (int)(r % sh.ext[1]);
      r /= sh.ext[1];
      pz[nb] = (int)(r % sh.ext[0]);
      pn[nb] = (int)(r / sh.ext[0]);
    }
    for (int ph = 0; ph < phases; ++ph) {
      // taps of this phase: per axis from t0 in steps of s (all taps for the strided conv)
      const int rw = TR ? ph % s : 0, rh = TR ? (ph / s) % s : 0, rd = TR && v3 ? ph / (s * s) : 0;
      const int t0w = TR ? (rw + p) % s : 0, t0h = TR ? (rh + p) % s : 0, t0d = TR ? (rd + pd) % sd : 0;
      const int tstep = TR ? s : 1, tstepd = TR ? sd : 1;
      const int dw = TR ? (rw + p - t0w) / s : 0, dh = TR ? (rh + p - t0h) / s : 0, dd = TR ? (rd + pd - t0d) / sd : 0;
      const uint16_t* bp[NBK];
      float* op[NBK];
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) {
        if (TR) {
          bp[nb] = sh.in + pn[nb] * sh.isn + (int64_t)(pz[nb] + dd) * sh.is[0] + (int64_t)(py[nb] + dh) * sh.is[1] +
                   (int64_t)(px[nb] + dw) * sh.is[2] + grp * 8;
          op[nb] = sh.out + pn[nb] * sh.osn + (int64_t)(pz[nb] * sd + rd) * sh.os[0] +
                   (int64_t)(py[nb] * s + rh) * sh.os[1] + (int64_t)(px[nb] * s + rw) * sh.os[2];
        } else {
          bp[nb] = sh.in + pn[nb] * sh.isn + (int64_t)pz[nb] * s * sh.is[0] + (int64_t)py[nb] * s * sh.is[1] +
                   (int64_t)px[nb] * s * sh.is[2] + grp * 8;
          op[nb] = sh.out + pn[nb] * sh.osn + (int64_t)pz[nb] * sh.os[0] + (int64_t)py[nb] * sh.os[1] +
                   (int64_t)px[nb] * sh.os[2];
        }
      }
      // accumulator e of a lane is row 8(e/4) + 4 grp + e%4 (FR 32) or
      // 4 grp + e (FR 16) of the block, column lp
      acc_t acc[MB][NBK];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < NACC; ++e) {
          const int row = ob + mb * FR + 8 * (e >> 2) + 4 * grp + (e & 3);
          const float b = a.bias && row < a.cout ? a.bias[row] : 0.f;
#pragma unroll
          for (int nb = 0; nb < NBK; ++nb) acc[mb][nb][e] = b;
        }
      // K steps: (tap of the phase, block of KG x KS channels), taps lexicographic;
      // the next step's input fragments are loaded before this step's MFMAs
      const int nz = (kd - t0d + tstepd - 1) / tstepd, ny = (k - t0h + tstep - 1) / tstep,
                nx = (k - t0w + tstep - 1) / tstep;
      const int cg = KC / KG;
      const int nsteps = nz * ny * nx * cg;
      auto step_at = [&](int st, int64_t& off, int& wbase) __attribute__((always_inline)) {
        const int m = st / cg, c0 = (st - m * cg) * KG;
        const int mx = m % nx, my = (m / nx) % ny, mz = m / (nx * ny);
        const int tz = t0d + mz * tstepd, ty = t0h + my * tstep, tx = t0w + mx * tstep;
        // strided: cell j*s + t - p (base at the window's first cell);
        // transposed: cell q + (r + p - t)/s, one back per step of s
        off = (TR ? -(mz * sh.is[0] + my * sh.is[1] + mx * sh.is[2]) : tz * sh.is[0] + ty * sh.is[1] + tx * sh.is[2]) +
              c0 * KS;
        wbase = (((tz * k + ty) * k + tx) * KC + c0) * MB * SLOTS * 8;
      };
      auto load_b = [&](int64_t off, sx_bf16x8 (&bv)[KG][NBK]) __attribute__((always_inline)) {
#pragma unroll
        for (int kc = 0; kc < KG; ++kc)
#pragma unroll
          for (int nb = 0; nb < NBK; ++nb)
            bv[kc][nb] = *reinterpret_cast<const sx_bf16x8*>(bp[nb] + off + kc * KS);
      };
      // HALF: lane (row lp, K group grp) reads slot grp * 16 + lp for rows < 16
      const int slot = HALF ? grp * 16 + (lp & 15) : lane;
      const bool zero_row = HALF && lp >= 16;
      auto mma = [&](int wbase, const sx_bf16x8 (&bv)[KG][NBK]) __attribute__((always_inline)) {
        const uint16_t* wt = wl + wbase + slot * 8;
#pragma unroll
        for (int kc = 0; kc < KG; ++kc)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            sx_bf16x8 av = *reinterpret_cast<const sx_bf16x8*>(wt + (kc * MB + mb) * SLOTS * 8);
            if (HALF && zero_row) av = sx_bf16x8{};
#pragma unroll
            for (int nb = 0; nb < NBK; ++nb) {
              if constexpr (FR == 32)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[kc][nb], acc[mb][nb], 0, 0, 0);
              else
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[kc][nb], acc[mb][nb], 0, 0, 0);
            }
          }
      };
      // ring of kSxDepth fragment sets: kSxDepth - 1 steps in flight ahead of the MFMAs
      {
        sx_bf16x8 bf[kSxDepth][KG][NBK];
        int wb[kSxDepth];
#pragma unroll
        for (int i = 0; i < kSxDepth - 1; ++i)
          if (i < nsteps) {
            int64_t off;
            step_at(i, off, wb[i]);
            load_b(off, bf[i]);
          }
        for (int st = 0; st < nsteps; st += kSxDepth) {
#pragma unroll
          for (int b = 0; b < kSxDepth; ++b) {
            if (st + b < nsteps) {
              const int nx_ = st + b + kSxDepth - 1;
              if (nx_ < nsteps) {
                int64_t off;
                step_at(nx_, off, wb[(b + kSxDepth - 1) % kSxDepth]);
                load_b(off, bf[(b + kSxDepth - 1) % kSxDepth]);
              }
              mma(wb[b], bf[b]);
            }
          }
        }
      }
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) {
        if (!ok[nb]) continue;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < NACC / 4; ++j)
            if (ob + mb * FR + 8 * j + 4 * grp < a.cout) {
              typedef float nf4 __attribute__((ext_vector_type(4)));
              __builtin_nontemporal_store(
                  nf4{acc[mb][nb][4 * j], acc[mb][nb][4 * j + 1], acc[mb][nb][4 * j + 2], acc[mb][nb][4 * j + 3]},
                  reinterpret_cast<nf4*>(op[nb] + ob + mb * FR + 8 * j + 4 * grp));
            }
      }
    }
  }
}

constexpr int kSxCapSmall = 80 * 1024;          // two workgroups per CU
constexpr int kSxCapLarge = 160 * 1024;         // one workgroup per CU

// Launches the matrix-core path when the layer fits it; false leaves the call
// to the fp32 FMA kernels.  `in` of every shard as the FMA kernel's (strided:
// first window's first cell; transposed: interior origin), ext = position
// extents.
template <bool TR>
bool launch_sx_mfma(const SxShard* shards, int nshards, int batch, int cin, int cout, int k, int stride, int ndim,
                    const float* w, const float* bias, hipStream_t st) {
  // Cout a multiple of 16: a 16-channel layer fills half of one 32-row tile
  if (cin % 16 != 0 || cout % 16 != 0 || (reinterpret_cast<uintptr_t>(w) & 15)) return false;
  const int taps = ndim == 3 ? k * k * k : k * k;
  // 16x16x32 fragments when Cin % 32 == 0 (wider B loads), else 32x32x16
  const int fr = kSxPrefer16 && cin % 32 == 0 ? 16 : 32;
  int mb = fr == 16 ? (cout % 64 == 0 ? 4 : cout % 32 == 0 ? 2 : 1) : (cout % 64 == 0 ? 2 : 1);
  // a 16-channel layer stores only its 16 real rows of the 32-row tile
  const bool half = fr == 32 && cout == 16;
  int64_t need = (int64_t)taps * cin * mb * (half ? 16 : fr) * 2;
  while (need > kSxCapLarge && mb > 1) {
    mb /= 2;
    need /= 2;
  }
  if (need > kSxCapLarge) return false;
  SxArgs a{};
  a.nshards = nshards;
  a.cin = cin;
  a.cout = cout;
  a.k = k;
  a.stride = stride;
  a.ndim = ndim;
  a.taps = taps;
  a.w = w;
  a.bias = bias;
  int64_t tiles = 0;
  for (int i = 0; i < nshards; ++i) {
    a.sh[i] = shards[i];
    a.sh[i].positions = batch * (int64_t)shards[i].ext[0] * shards[i].ext[1] * shards[i].ext[2];
    a.sh[i].tile_begin = tiles;
    tiles += (a.sh[i].positions + kSxTile - 1) / kSxTile;
  }
  a.tiles = tiles;
  if (tiles == 0) return true;
  const int64_t groups = (tiles + kSxWaves - 1) / kSxWaves;
  // persistent: as many workgroups as fit at once (two per CU with <= 80 KiB
  // of weights, else one), each staging the weights once
  const bool small = need <= kSxCapSmall;
  int64_t grid = std::min<int64_t>(groups, small ? 512 : 256);
  grid = (grid + 7) / 8 * 8;
  a.iters = (int)((groups + grid - 1) / grid);
  // K steps loaded together: 64 channels when Cin allows
  const int ks = fr == 16 ? 32 : 16;
  const int kg = cin % 64 == 0 ? 64 / ks : cin % 32 == 0 ? 32 / ks : 1;
  const dim3 g3((unsigned)grid, (unsigned)((cout + mb * fr - 1) / (mb * fr))), block(kSxWaves * 64);
#define ST_SX(FR_, MB_, KG_, CAP_) hipLaunchKernelGGL((conv_sx_mfma<FR_, MB_, KG_, TR, CAP_>), g3, block, 0, st, a)
#define ST_SX_CAP(FR_, MB_, KG_)                  \
  do {                                            \
    if (small) ST_SX(FR_, MB_, KG_, kSxCapSmall); \
    else ST_SX(FR_, MB_, KG_, kSxCapLarge);       \
  } while (0)
#define ST_SX_KG(FR_, MB_)                   \
  do {                                       \
    if (kg == 4) ST_SX_CAP(FR_, MB_, 4);     \
    else if (kg == 2) ST_SX_CAP(FR_, MB_, 2); \
    else ST_SX_CAP(FR_, MB_, 1);             \
  } while (0)
  if (fr == 16) {
    // kg is 1 or 2 here
    if (mb == 4) {
      if (kg == 2) ST_SX_CAP(16, 4, 2);
      else ST_SX_CAP(16, 4, 1);
    } else if (mb == 2) {
      if (kg == 2) ST_SX_CAP(16, 2, 2);
      else ST_SX_CAP(16, 2, 1);
    } else {
      if (kg == 2) ST_SX_CAP(16, 1, 2);
      else ST_SX_CAP(16, 1, 1);
    }
  } else if (mb == 2) {
    ST_SX_KG(32, 2);
  } else if (half) {
    // Cin % 16 == 0 and cout 16: kg is 1, 2 or 4
#define ST_SX_H(KG_)                                                                                               \
  do {                                                                                                             \
    if (small) hipLaunchKernelGGL((conv_sx_mfma<32, 1, KG_, TR, kSxCapSmall, true>), g3, block, 0, st, a);       \
    else hipLaunchKernelGGL((conv_sx_mfma<32, 1, KG_, TR, kSxCapLarge, true>), g3, block, 0, st, a);             \
  } while (0)
    if (kg == 4) ST_SX_H(4);
    else if (kg == 2) ST_SX_H(2);
    else ST_SX_H(1);
#undef ST_SX_H
  } else {
    ST_SX_KG(32, 1);
  }
#undef ST_SX_KG
#undef ST_SX_CAP
#undef ST_SX
  return true;
}

// output sizes along one internal axis: output j owns the window centred at j*s
bool strided_sizes(const std::vector<int64_t>& in, int64_t k, int64_t s, std::vector<int64_t>& out,
                   std::vector<int64_t>& first) {
  int64_t n = 0;
  for (int64_t v : in) n += v;
  const int64_t p = k / 2;
  if (n + 2 * p < k) return false;
  const int64_t n_out = (n + 2 * p - k) / s + 1;
  out.clear();
  first.clear();
  int64_t a = 0;
  for (int64_t e : in) {
    const int64_t f = (a + s - 1) / s;
    out.push_back(std::min((a + e + s - 1) / s, n_out) - f);
    first.push_back(f);
    a += e;
  }
  return true;
}


// Raw weights -> the fp32 [taps][A][B] layout both kernels read (A = the
// op's input channels, B = its output channels), widening bf16 exactly.
// Strided conv: raw [B][A][taps] ([Cout][Cin], PyTorch's conv order);
// transposed conv: raw [A][B][taps] ([in][out], PyTorch's conv_transpose
// order).
template <typename T>
__global__ void pack_w_tab(const T* __restrict__ w, float* __restrict__ out, int a_ch, int b_ch, int taps,
                           int a_major, int64_t total, uint32_t* clr, int nclr) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nclr) clr[i] = 0u;                        // e.g. the max |y| of the conv that follows
  if (i >= total) return;
  const int j = (int)(i % b_ch);
  const int64_t r = i / b_ch;
  const int ia = (int)(r % a_ch);
  const int t = (int)(r / a_ch);
  const int64_t src = a_major ? ((int64_t)ia * b_ch + j) * taps + t : ((int64_t)j * a_ch + ia) * taps + t;
  if constexpr (std::is_same<T, uint16_t>::value) out[i] = __uint_as_float((uint32_t)w[src] << 16);
  else out[i] = w[src];
}

size_t tab_workspace_bytes(const st_plan* in_plan, int32_t cout, int32_t ksize) {
  if (!in_plan || cout < 1 || ksize < 1 || ksize % 2 == 0) return 0;
  int64_t taps = 1;
  for (int a = 0; a < in_plan->ndim; ++a) taps *= ksize;
  const size_t b = (size_t)taps * (size_t)in_plan->channels * (size_t)cout * 4;
  return (b + 255) / 256 * 256;
}

// Checks the workspace and enqueues the packing of the raw weights into it.
st_status pack_tab(const st_plan* in_plan, int32_t cout, int32_t ksize, const void* weight, bool a_major,
                   void* workspace, size_t workspace_bytes, hipStream_t st, const char* who) {
  const size_t need = tab_workspace_bytes(in_plan, cout, ksize);
  if (!workspace || workspace_bytes < need)
    return fail(ST_ERR_WORKSPACE, std::string(who) + ": workspace missing or too small");
  if (!aligned16(workspace) || !aligned16(weight))
    return fail(ST_ERR_ALIGNMENT, std::string(who) + ": weight and workspace must be 16-byte aligned");
  int taps = 1;
  for (int a = 0; a < in_plan->ndim; ++a) taps *= ksize;
  const int a_ch = (int)in_plan->channels;
  const int64_t total = (int64_t)taps * a_ch * cout;
  return pack_tab_launch(weight, in_plan->dtype, static_cast<float*>(workspace), a_ch, (int)cout, taps, a_major,
                         nullptr, 0, st, who);
}

}  // namespace

st_status pack_tab_launch(const void* weight, st_dtype dtype, float* out, int a_ch, int b_ch, int taps, bool a_major,
                          uint32_t* clr, int nclr, hipStream_t st, const char* who) {
  const int64_t total = (int64_t)taps * a_ch * b_ch;
  const dim3 gd((unsigned)((std::max<int64_t>(total, nclr) + 255) / 256)), bd(256);
  if (dtype == ST_BF16)
    hipLaunchKernelGGL(pack_w_tab<uint16_t>, gd, bd, 0, st, static_cast<const uint16_t*>(weight), out, a_ch, b_ch,
                       taps, a_major ? 1 : 0, total, clr, nclr);
  else
    hipLaunchKernelGGL(pack_w_tab<float>, gd, bd, 0, st, static_cast<const float*>(weight), out, a_ch, b_ch, taps,
                       a_major ? 1 : 0, total, clr, nclr);
  return launch_check((std::string(who) + ": weight packing launch").c_str());
}

bool sx_same_fits(int ndim, int cin, int cout, int ksize) {
  if (cin % 16 != 0 || cout % 16 != 0 || ksize < 1 || ksize % 2 == 0) return false;
  const int taps = ndim == 3 ? ksize * ksize * ksize : ksize * ksize;
  const int fr = kSxPrefer16 && cin % 32 == 0 ? 16 : 32;
  return (int64_t)taps * cin * fr * 2 <= kSxCapLarge;     // one FR-channel block of weights in LDS
}

st_status sx_same_conv(const st_plan* in_plan, const void* const* in_bufs, const float* w_tco, const float* bias,
                       int cout, int ksize, float* const* y_bufs, hipStream_t st) {
  const int p = ksize / 2;
  const int cin = (int)in_plan->channels;
  SxShard sx[ST_MAX_SHARDS];
  for (size_t i = 0; i < in_plan->shards.size(); ++i) {
    const Shard& si = in_plan->shards[i];
    SxShard& q = sx[i];
    q = SxShard{};
    q.is[2] = cin;
    q.is[1] = si.pad[2] * cin;
    q.is[0] = si.pad[1] * q.is[1];
    q.isn = si.pad[0] * q.is[0];
    q.os[2] = cout;
    q.os[1] = si.ext[2] * cout;
    q.os[0] = si.ext[1] * q.os[1];
    q.osn = si.ext[0] * q.os[0];
    int64_t in_off = 0;
    for (int ax = 0; ax < kAxes; ++ax) {
      const bool sp = ax >= kAxes - in_plan->ndim;
      in_off += (sp ? in_plan->halo[ax] - p : 0) * q.is[ax];
      q.ext[ax] = (int32_t)si.ext[ax];
    }
    q.in = static_cast<const uint16_t*>(in_bufs[i]) + in_off;
    q.out = y_bufs[i];
  }
  if (!launch_sx_mfma<false>(sx, (int)in_plan->shards.size(), (int)in_plan->batch, cin, cout, ksize, 1,
                             in_plan->ndim, w_tco, bias, st))
    return fail(ST_ERR_UNSUPPORTED, "st_conv_sharded: shape does not fit the matrix-core 'same' conv");
  return launch_check("st_conv_sharded: conv_sx_mfma launch");
}

}  // namespace st

using namespace st;

extern "C" {

st_status st_plan_strided(const st_plan* in_plan, int32_t ksize, int32_t stride, int32_t cout,
                          const int32_t* out_halo_or_null, st_plan** out) {
  auto err = [](st_status s, const std::string& m) { return fail(s, "st_plan_strided: " + m); };
  if (!in_plan || !out) return err(ST_ERR_INVALID_ARG, "NULL argument");
  *out = nullptr;
  if (ksize < 1 || ksize % 2 == 0) return err(ST_ERR_UNSUPPORTED, "odd kernel sizes only");
  if (stride < 1 || cout < 1) return err(ST_ERR_INVALID_ARG, "stride and cout must be >= 1");
  const int nd = in_plan->ndim;
  int64_t spatial[ST_MAX_NDIM];
  int32_t counts[ST_MAX_NDIM], halo[ST_MAX_NDIM];
  std::vector<int64_t> concat;
  for (int a = 0; a < nd; ++a) {
    std::vector<int64_t> sz, first;
    if (!strided_sizes(in_plan->sizes[axis_of(in_plan, a)], ksize, stride, sz, first))
      return err(ST_ERR_BAD_SHAPE, "window larger than the padded volume");
    int64_t tot = 0;
    for (size_t i = 0; i < sz.size(); ++i) {
      if (sz[i] < 1) {
        char buf[160];
        std::snprintf(buf, sizeof buf, "axis %d shard %zu holds no window centre", a, i);
        return err(ST_ERR_SHARD_TOO_SMALL, buf);
      }
      tot += sz[i];
      concat.push_back(sz[i]);
    }
    spatial[a] = tot;
    counts[a] = (int32_t)sz.size();
    halo[a] = out_halo_or_null ? out_halo_or_null[a] : 0;
  }
  return st_plan_shards(nd, in_plan->batch, cout, spatial, counts, concat.data(), halo, ST_F32, out);
}

size_t st_conv_strided_workspace_bytes(const st_plan* in_plan, int32_t cout, int32_t ksize) {
  return tab_workspace_bytes(in_plan, cout, ksize);
}

st_status st_conv_strided_sharded(const st_plan* in_plan, const void* const* in_bufs, const void* weight,
                                  const float* bias_or_null, int32_t ksize, int32_t stride,
                                  const st_plan* out_plan, float* const* out_bufs, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  auto err = [](st_status s, const std::string& m) { return fail(s, "st_conv_strided_sharded: " + m); };
  if (!in_plan || !out_plan || !in_bufs || !out_bufs || !weight)
    return err(ST_ERR_INVALID_ARG, "NULL argument");
  const float* weight_tco = static_cast<const float*>(workspace);
  if (ksize < 1 || ksize % 2 == 0) return err(ST_ERR_UNSUPPORTED, "odd kernel sizes only");
  if (stride < 1) return err(ST_ERR_INVALID_ARG, "stride must be >= 1");
  if (out_plan->dtype != ST_F32) return err(ST_ERR_BAD_SHAPE, "outputs are fp32");
  if (out_plan->ndim != in_plan->ndim || out_plan->batch != in_plan->batch ||
      out_plan->shards.size() != in_plan->shards.size())
    return err(ST_ERR_BAD_SHAPE, "output plan does not match the input plan");
  if (bias_or_null && (reinterpret_cast<uintptr_t>(bias_or_null) & 3)) return err(ST_ERR_ALIGNMENT, "misaligned bias");
  if (!workspace || workspace_bytes < tab_workspace_bytes(in_plan, (int32_t)out_plan->channels, ksize))
    return err(ST_ERR_WORKSPACE, "workspace missing or smaller than st_conv_strided_workspace_bytes");
  if (!aligned16(workspace) || !aligned16(weight)) return err(ST_ERR_ALIGNMENT, "misaligned weight or workspace");
  StrArgs a{};
  a.nshards = (int)in_plan->shards.size();
  a.batch = (int)in_plan->batch;
  a.cin = (int)in_plan->channels;
  a.cout = (int)out_plan->channels;
  a.k = ksize;
  a.stride = stride;
  a.ndim = in_plan->ndim;
  a.w = weight_tco;
  a.bias = bias_or_null;
  const int p = ksize / 2;
  std::vector<int64_t> first[kAxes];
  for (int ax = 0; ax < kAxes; ++ax) {
    if (ax < kAxes - in_plan->ndim) {
      first[ax].assign(in_plan->nshards[ax], 0);
      continue;
    }
    std::vector<int64_t> sz;
    if (!strided_sizes(in_plan->sizes[ax], ksize, stride, sz, first[ax]))
      return err(ST_ERR_BAD_SHAPE, "window larger than the padded volume");
    if (sz != out_plan->sizes[ax]) return err(ST_ERR_BAD_SHAPE, "output plan is not the strided plan of the input");
  }
  const int ie = in_plan->esize;
  int64_t total = 0;
  for (size_t i = 0; i < in_plan->shards.size(); ++i) {
    if (!in_bufs[i] || !out_bufs[i]) return err(ST_ERR_INVALID_ARG, "NULL shard buffer");
    if (!aligned16(in_bufs[i]) || !aligned16(out_bufs[i])) return err(ST_ERR_ALIGNMENT, "shard buffers must be 16-byte aligned");
    const Shard& si = in_plan->shards[i];
    const Shard& so = out_plan->shards[i];
    StrShard& q = a.sh[i];
    q.is[2] = a.cin;
    q.is[1] = si.pad[2] * a.cin;
    q.is[0] = si.pad[1] * q.is[1];
    q.isn = si.pad[0] * q.is[0];
    q.os[2] = a.cout;
    q.os[1] = so.pad[2] * a.cout;
    q.os[0] = so.pad[1] * q.os[1];
    q.osn = so.pad[0] * q.os[0];
    int64_t in_off = 0, out_off = 0;
    for (int ax = 0; ax < kAxes; ++ax) {
      const bool sp = ax >= kAxes - in_plan->ndim;
      // first owned window's first cell (centre f*s, minus p) in padded coordinates
      const int64_t lo = sp ? first[ax][si.grid[ax]] * stride - p - si.off[ax] + in_plan->halo[ax] : 0;
      const int64_t hi = sp ? lo + (so.ext[ax] - 1) * stride + ksize : 1;
      if (lo < 0 || hi > si.pad[ax]) return err(ST_ERR_BAD_SHAPE, "input halo smaller than ksize/2");
      in_off += lo * q.is[ax];
      out_off += out_plan->halo[ax] * q.os[ax];
      q.oext[ax] = (int32_t)so.ext[ax];
    }
    q.in = static_cast<const char*>(in_bufs[i]) + in_off * ie;
    q.out = out_bufs[i] + out_off;
    q.begin = total;
    total += a.batch * (int64_t)so.ext[0] * so.ext[1] * so.ext[2];
  }
  a.total = total;
  if (total == 0) return ST_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  st_status ps = pack_tab(in_plan, a.cout, ksize, weight, false, workspace, workspace_bytes, st,
                          "st_conv_strided_sharded");
  if (ps != ST_OK) return ps;
  const bool bf = in_plan->dtype == ST_BF16;
  if (bf) {
    SxShard sx[ST_MAX_SHARDS];
    for (int i = 0; i < a.nshards; ++i) {
      sx[i] = SxShard{};
      sx[i].in = reinterpret_cast<const uint16_t*>(a.sh[i].in);
      sx[i].out = a.sh[i].out;
      for (int ax = 0; ax < 3; ++ax) {
        sx[i].is[ax] = a.sh[i].is[ax];
        sx[i].os[ax] = a.sh[i].os[ax];
        sx[i].ext[ax] = a.sh[i].oext[ax];
      }
      sx[i].isn = a.sh[i].isn;
      sx[i].osn = a.sh[i].osn;
    }
    if (launch_sx_mfma<false>(sx, a.nshards, a.batch, a.cin, a.cout, a.k, a.stride, a.ndim, a.w, a.bias, st))
      return launch_check("st_conv_strided_sharded: launch");
  }
  int ob = 1;
  for (int c : {64, 32, 16, 8, 4, 2, 1})
    if (a.cout % c == 0) { ob = c; break; }
  const dim3 grid((unsigned)((total + 255) / 256), (unsigned)(a.cout / ob)), block(256);
  const bool vec = bf ? a.cin % 8 == 0 : a.cin % 4 == 0;
#define ST_STR_LAUNCH(OB)                                                                            \
  do {                                                                                               \
    if (bf && vec) hipLaunchKernelGGL((conv_strided_kernel<uint16_t, OB, 8>), grid, block, 0, st, a); \
    else if (bf) hipLaunchKernelGGL((conv_strided_kernel<uint16_t, OB, 1>), grid, block, 0, st, a);  \
    else if (vec) hipLaunchKernelGGL((conv_strided_kernel<float, OB, 4>), grid, block, 0, st, a);    \
    else hipLaunchKernelGGL((conv_strided_kernel<float, OB, 1>), grid, block, 0, st, a);             \
  } while (0)
  switch (ob) {
    case 64: ST_STR_LAUNCH(64); break;
    case 32: ST_STR_LAUNCH(32); break;
    case 16: ST_STR_LAUNCH(16); break;
    case 8: ST_STR_LAUNCH(8); break;
    case 4: ST_STR_LAUNCH(4); break;
    case 2: ST_STR_LAUNCH(2); break;
    default: ST_STR_LAUNCH(1); break;
  }
#undef ST_STR_LAUNCH
  return launch_check("st_conv_strided_sharded: launch");
}

st_status st_plan_transposed(const st_plan* in_plan, int32_t ksize, int32_t stride, int32_t cout,
                             const int32_t* out_halo_or_null, st_plan** out) {
  auto err = [](st_status s, const std::string& m) { return fail(s, "st_plan_transposed: " + m); };
  if (!in_plan || !out) return err(ST_ERR_INVALID_ARG, "NULL argument");
  *out = nullptr;
  if (ksize < 1 || ksize % 2 == 0) return err(ST_ERR_UNSUPPORTED, "odd kernel sizes only");
  if (stride < 1 || stride > kMaxTransposedStride || cout < 1)
    return err(ST_ERR_INVALID_ARG, "stride must be in [1, 8] and cout >= 1");
  const int nd = in_plan->ndim;
  int64_t spatial[ST_MAX_NDIM];
  int32_t counts[ST_MAX_NDIM], halo[ST_MAX_NDIM];
  std::vector<int64_t> concat;
  for (int a = 0; a < nd; ++a) {
    int64_t tot = 0;
    const auto& sz = in_plan->sizes[axis_of(in_plan, a)];
    for (int64_t e : sz) {
      tot += e * stride;
      concat.push_back(e * stride);
    }
    spatial[a] = tot;
    counts[a] = (int32_t)sz.size();
    halo[a] = out_halo_or_null ? out_halo_or_null[a] : 0;
  }
  return st_plan_shards(nd, in_plan->batch, cout, spatial, counts, concat.data(), halo, ST_F32, out);
}

size_t st_conv_transposed_workspace_bytes(const st_plan* in_plan, int32_t cout, int32_t ksize) {
  return tab_workspace_bytes(in_plan, cout, ksize);
}

st_status st_conv_transposed_sharded(const st_plan* in_plan, const void* const* in_bufs, const void* weight,
                                     const float* bias_or_null, int32_t ksize, int32_t stride,
                                     const st_plan* out_plan, float* const* out_bufs, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  auto err = [](st_status s, const std::string& m) { return fail(s, "st_conv_transposed_sharded: " + m); };
  if (!in_plan || !out_plan || !in_bufs || !out_bufs || !weight)
    return err(ST_ERR_INVALID_ARG, "NULL argument");
  const float* weight_tio = static_cast<const float*>(workspace);
  if (ksize < 1 || ksize % 2 == 0) return err(ST_ERR_UNSUPPORTED, "odd kernel sizes only");
  if (stride < 1 || stride > kMaxTransposedStride) return err(ST_ERR_INVALID_ARG, "stride must be in [1, 8]");
  if (out_plan->dtype != ST_F32) return err(ST_ERR_BAD_SHAPE, "outputs are fp32");
  if (out_plan->ndim != in_plan->ndim || out_plan->batch != in_plan->batch ||
      out_plan->shards.size() != in_plan->shards.size())
    return err(ST_ERR_BAD_SHAPE, "output plan does not match the input plan");
  if (bias_or_null && (reinterpret_cast<uintptr_t>(bias_or_null) & 3)) return err(ST_ERR_ALIGNMENT, "misaligned bias");
  if (!workspace || workspace_bytes < tab_workspace_bytes(in_plan, (int32_t)out_plan->channels, ksize))
    return err(ST_ERR_WORKSPACE, "workspace missing or smaller than st_conv_transposed_workspace_bytes");
  if (!aligned16(workspace) || !aligned16(weight)) return err(ST_ERR_ALIGNMENT, "misaligned weight or workspace");
  TrArgs a{};
  a.nshards = (int)in_plan->shards.size();
  a.batch = (int)in_plan->batch;
  a.cin = (int)in_plan->channels;
  a.cout = (int)out_plan->channels;
  a.k = ksize;
  a.stride = stride;
  a.ndim = in_plan->ndim;
  a.w = weight_tio;
  a.bias = bias_or_null;
  for (int ax = kAxes - in_plan->ndim; ax < kAxes; ++ax) {
    const auto& si = in_plan->sizes[ax];
    const auto& so = out_plan->sizes[ax];
    bool same = si.size() == so.size();
    for (size_t i = 0; same && i < si.size(); ++i) same = so[i] == si[i] * stride;
    if (!same) return err(ST_ERR_BAD_SHAPE, "output plan is not the transposed plan of the input");
  }
  int lo = 0, hi = 0;
  const bool any_tap = transposed_reach(ksize, stride, lo, hi);
  const int ie = in_plan->esize;
  int64_t total = 0;
  for (size_t i = 0; i < in_plan->shards.size(); ++i) {
    if (!in_bufs[i] || !out_bufs[i]) return err(ST_ERR_INVALID_ARG, "NULL shard buffer");
    if (!aligned16(in_bufs[i]) || !aligned16(out_bufs[i])) return err(ST_ERR_ALIGNMENT, "shard buffers must be 16-byte aligned");
    const Shard& si = in_plan->shards[i];
    const Shard& so = out_plan->shards[i];
    TrShard& q = a.sh[i];
    q.is[2] = a.cin;
    q.is[1] = si.pad[2] * a.cin;
    q.is[0] = si.pad[1] * q.is[1];
    q.isn = si.pad[0] * q.is[0];
    q.os[2] = a.cout;
    q.os[1] = so.pad[2] * a.cout;
    q.os[0] = so.pad[1] * q.os[1];
    q.osn = so.pad[0] * q.os[0];
    int64_t in_off = 0, out_off = 0;
    for (int ax = 0; ax < kAxes; ++ax) {
      const bool sp = ax >= kAxes - in_plan->ndim;
      const int64_t h = in_plan->halo[ax];
      // every read cell lies in [q + lo, q + hi] for q in the interior
      if (sp && any_tap && si.ext[ax] > 0 && (h + lo < 0 || h + si.ext[ax] - 1 + hi >= si.pad[ax]))
        return err(ST_ERR_BAD_SHAPE, "input halo smaller than ksize/2");
      in_off += h * q.is[ax];
      out_off += out_plan->halo[ax] * q.os[ax];
      q.iext[ax] = (int32_t)si.ext[ax];
    }
    q.in = static_cast<const char*>(in_bufs[i]) + in_off * ie;
    q.out = out_bufs[i] + out_off;
    q.begin = total;
    total += a.batch * (int64_t)si.ext[0] * si.ext[1] * si.ext[2];
  }
  a.total = total;
  if (total == 0) return ST_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  st_status ps = pack_tab(in_plan, a.cout, ksize, weight, true, workspace, workspace_bytes, st,
                          "st_conv_transposed_sharded");
  if (ps != ST_OK) return ps;
  const bool bf = in_plan->dtype == ST_BF16;
  if (bf) {
    SxShard sx[ST_MAX_SHARDS];
    for (int i = 0; i < a.nshards; ++i) {
      sx[i] = SxShard{};
      sx[i].in = reinterpret_cast<const uint16_t*>(a.sh[i].in);
      sx[i].out = a.sh[i].out;
      for (int ax = 0; ax < 3; ++ax) {
        sx[i].is[ax] = a.sh[i].is[ax];
        sx[i].os[ax] = a.sh[i].os[ax];
        sx[i].ext[ax] = a.sh[i].iext[ax];
      }
      sx[i].isn = a.sh[i].isn;
      sx[i].osn = a.sh[i].osn;
    }
    if (launch_sx_mfma<true>(sx, a.nshards, a.batch, a.cin, a.cout, a.k, a.stride, a.ndim, a.w, a.bias, st))
      return launch_check("st_conv_transposed_sharded: launch");
  }
  int ob = 1;
  for (int c : {64, 32, 16, 8, 4, 2, 1})
    if (a.cout % c == 0) { ob = c; break; }
  int phases = stride * stride * (a.ndim == 3 ? stride : 1);
  const dim3 grid((unsigned)((total + 255) / 256), (unsigned)(a.cout / ob), (unsigned)phases), block(256);
  const bool vec = bf ? a.cin % 8 == 0 : a.cin % 4 == 0;
#define ST_TR_LAUNCH(OB)                                                                                \
  do {                                                                                                  \
    if (bf && vec) hipLaunchKernelGGL((conv_transposed_kernel<uint16_t, OB, 8>), grid, block, 0, st, a); \
    else if (bf) hipLaunchKernelGGL((conv_transposed_kernel<uint16_t, OB, 1>), grid, block, 0, st, a);  \
    else if (vec) hipLaunchKernelGGL((conv_transposed_kernel<float, OB, 4>), grid, block, 0, st, a);    \
    else hipLaunchKernelGGL((conv_transposed_kernel<float, OB, 1>), grid, block, 0, st, a);             \
  } while (0)
  switch (ob) {
    case 64: ST_TR_LAUNCH(64); break;
    case 32: ST_TR_LAUNCH(32); break;
    case 16: ST_TR_LAUNCH(16); break;
    case 8: ST_TR_LAUNCH(8); break;
    case 4: ST_TR_LAUNCH(4); break;
    case 2: ST_TR_LAUNCH(2); break;
    default: ST_TR_LAUNCH(1); break;
  }
#undef ST_TR_LAUNCH
  return launch_check("st_conv_transposed_sharded: launch");
}

}  // extern "C"
