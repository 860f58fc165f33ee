// Shape-changing sharded op: 'valid' pooling (downsampling).
//
// "Technical summary: ShardTensor - domain parallelism for scientific machine
// learning", section 2 "Design principles": every local chunk carries its own
// shape ("sharding shapes"), which lets an op change the shapes.  For a
// window k and stride s, output j along an axis covers inputs [j*s, j*s + k).
// Output j belongs to the shard whose interior holds j*s, the first cell of
// its window, so a shard with interior [a, a + e) owns outputs
// [ceil(a / s), min(ceil((a + e) / s), n_out)) and reads at most k - 1 cells
// past its interior: a halo of k - 1 suffices.  Every output is computed from
// the same cells in the same order whatever the plan, so sharded and
// unsharded outputs agree bit for bit.
//
// st_plan_pooled derives the output plan; st_pool_sharded runs one launch
// over every shard: each thread takes one 16-byte vector of channels of one
// output position, sums (or takes the max of) its k^d window in fp32 in
// lexicographic tap order, and writes it in the output type.
#include <algorithm>
#include <cstdio>

#include "internal.h"

namespace st {
namespace {

struct PoolShard {
  const char* in;          // input element (n=0, window 0's first cell) of this shard
  char* out;               // output interior origin
  int64_t is[3];           // input element strides (d, h, w); batch stride isn
  int64_t isn;
  int64_t os[3];           // output element strides (d, h, w); batch stride osn
  int64_t osn;
  int32_t oext[3];         // output interior extents (d, h, w)
  int64_t begin;           // first work item of this shard
};

// n / d for 0 <= n < 2^31 as (n * m) >> p with p = 31 + ceil(log2 d) and
// m = ceil(2^p / d) < 2^32 (the round-up multiplier method: the error term
// stays below 1 / d, so the floor is exact)
struct PoolDiv {
  uint32_t m;
  int32_t p;
};
PoolDiv pool_div(uint32_t d) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  return PoolDiv{(uint32_t)(((1ull << (31 + l)) + d - 1) / d), 31 + l};
}
__device__ __forceinline__ uint32_t pdiv(uint32_t n, PoolDiv f) { return (uint32_t)(((uint64_t)n * f.m) >> f.p); }

struct PoolArgs {
  int32_t nshards, batch, channels, vec, k, stride, ndim, mode;
  float inv_count;
  int64_t total;
  PoolDiv dcv;                     // dividers by C / vec and by the output extents (w, h, d)
  PoolDiv dext[ST_MAX_SHARDS][3];
  PoolShard sh[ST_MAX_SHARDS];
};
static_assert(sizeof(PoolArgs) <= kMaxKernargBytes, "kernel argument struct too large");

// VEC consecutive channels as fp32 (one 16-byte load for VEC > 1)
template <typename T, int VEC> __device__ __forceinline__ void ldv(const T* p, float (&x)[VEC]);
template <> __device__ __forceinline__ void ldv<float, 1>(const float* p, float (&x)[1]) { x[0] = *p; }
template <> __device__ __forceinline__ void ldv<float, 4>(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <> __device__ __forceinline__ void ldv<uint16_t, 1>(const uint16_t* p, float (&x)[1]) {
  x[0] = __uint_as_float((uint32_t)*p << 16);
}
template <> __device__ __forceinline__ void ldv<uint16_t, 8>(const uint16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <typename T, int VEC> __device__ __forceinline__ void ldv_nt(const T* p, float (&x)[VEC]);
template <> __device__ __forceinline__ void ldv_nt<float, 1>(const float* p, float (&x)[1]) {
  x[0] = __builtin_nontemporal_load(p);
}
template <> __device__ __forceinline__ void ldv_nt<float, 4>(const float* p, float (&x)[4]) {
  typedef float nf4 __attribute__((ext_vector_type(4)));
  const nf4 v = __builtin_nontemporal_load(reinterpret_cast<const nf4*>(p));
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <> __device__ __forceinline__ void ldv_nt<uint16_t, 1>(const uint16_t* p, float (&x)[1]) {
  x[0] = __uint_as_float((uint32_t)__builtin_nontemporal_load(p) << 16);
}
template <> __device__ __forceinline__ void ldv_nt<uint16_t, 8>(const uint16_t* p, float (&x)[8]) {
  typedef unsigned int nu4 __attribute__((ext_vector_type(4)));
  const nu4 v = __builtin_nontemporal_load(reinterpret_cast<const nu4*>(p));
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint32_t bf16_bits(float v) {    // nearest even (finite values)
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// non-temporal stores of the pooled output (read back only by a later pass)
template <typename T, int VEC> __device__ __forceinline__ void stv_nt(T* p, const float (&x)[VEC]);
template <> __device__ __forceinline__ void stv_nt<float, 1>(float* p, const float (&x)[1]) {
  __builtin_nontemporal_store(x[0], p);
}
template <> __device__ __forceinline__ void stv_nt<float, 4>(float* p, const float (&x)[4]) {
  typedef float nf4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(nf4{x[0], x[1], x[2], x[3]}, reinterpret_cast<nf4*>(p));
}
template <> __device__ __forceinline__ void stv_nt<float, 8>(float* p, const float (&x)[8]) {
  typedef float nf4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(nf4{x[0], x[1], x[2], x[3]}, reinterpret_cast<nf4*>(p));
  __builtin_nontemporal_store(nf4{x[4], x[5], x[6], x[7]}, reinterpret_cast<nf4*>(p) + 1);
}
template <> __device__ __forceinline__ void stv_nt<uint16_t, 1>(uint16_t* p, const float (&x)[1]) {
  __builtin_nontemporal_store((uint16_t)bf16_bits(x[0]), p);
}
template <> __device__ __forceinline__ void stv_nt<uint16_t, 8>(uint16_t* p, const float (&x)[8]) {
  typedef unsigned int nu4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(nu4{bf16_bits(x[0]) | (bf16_bits(x[1]) << 16), bf16_bits(x[2]) | (bf16_bits(x[3]) << 16),
                                  bf16_bits(x[4]) | (bf16_bits(x[5]) << 16), bf16_bits(x[6]) | (bf16_bits(x[7]) << 16)},
                              reinterpret_cast<nu4*>(p));
}

template <typename T, int VEC> __device__ __forceinline__ void stv(T* p, const float (&x)[VEC]);
template <> __device__ __forceinline__ void stv<float, 1>(float* p, const float (&x)[1]) { *p = x[0]; }
template <> __device__ __forceinline__ void stv<float, 4>(float* p, const float (&x)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
template <> __device__ __forceinline__ void stv<float, 8>(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}
template <> __device__ __forceinline__ void stv<uint16_t, 1>(uint16_t* p, const float (&x)[1]) {
  *p = (uint16_t)bf16_bits(x[0]);
}
template <> __device__ __forceinline__ void stv<uint16_t, 8>(uint16_t* p, const float (&x)[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(bf16_bits(x[0]) | (bf16_bits(x[1]) << 16), bf16_bits(x[2]) | (bf16_bits(x[3]) << 16),
                                            bf16_bits(x[4]) | (bf16_bits(x[5]) << 16), bf16_bits(x[6]) | (bf16_bits(x[7]) << 16));
}

// one thread: VEC channels of one output position
template <typename TI, typename TO, int VEC, bool MAX>
__global__ __launch_bounds__(256) void pool_kernel(const PoolArgs a) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= a.total) return;
  int s = 0;
  while (s + 1 < a.nshards && a.sh[s + 1].begin <= item) ++s;
  const PoolShard& sh = a.sh[s];
  const int cv = a.channels / VEC;
  int64_t r = item - sh.begin;
  const int c = (int)(r % cv) * VEC;
  r /= cv;
  const int ow = (int)(r % sh.oext[2]);
  r /= sh.oext[2];
  const int oh = (int)(r % sh.oext[1]);
  r /= sh.oext[1];
  const int od = (int)(r % sh.oext[0]);
  const int n = (int)(r / sh.oext[0]);
  const TI* base = reinterpret_cast<const TI*>(sh.in) + n * sh.isn + (int64_t)od * a.stride * sh.is[0] +
                   (int64_t)oh * a.stride * sh.is[1] + (int64_t)ow * a.stride * sh.is[2] + c;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = MAX ? -INFINITY : 0.f;
  const int kd = a.ndim == 3 ? a.k : 1;
  for (int tz = 0; tz < kd; ++tz)
    for (int ty = 0; ty < a.k; ++ty)
      for (int tx = 0; tx < a.k; ++tx) {
        float x[VEC];
        ldv<TI, VEC>(base + tz * sh.is[0] + ty * sh.is[1] + tx * sh.is[2], x);
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = MAX ? fmaxf(acc[v], x[v]) : acc[v] + x[v];
      }
  if (!MAX) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] *= a.inv_count;
  }
  stv<TO, VEC>(reinterpret_cast<TO*>(sh.out) + n * sh.osn + od * sh.os[0] + oh * sh.os[1] + ow * sh.os[2] + c, acc);
}

// output sizes of one internal axis for the given input sizes
// The common windows (k = 2 or 3, 2D or 3D): all K^ND taps' loads in flight
// at once, and the work item split into channel vector, column, row, plane
// and batch item by multiply-shift division (every shard's item count is
// below 2^31 on this path).  2D loads are non-temporal: 2x2 pooling of the
// 2048^2 image and of the 256-channel grid 0.138 -> 0.108 and 0.238 -> 0.189
// ms against the general kernel (plain loads: 0.116, 0.202); on the 3D
// volumes non-temporal loads were 4% slower and plain ones 0-5% faster.
template <typename TI, typename TO, int VEC, bool MAX, int K, int ND>
__global__ __launch_bounds__(256) void pool_fixed(const PoolArgs a) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= a.total) return;
  int s = 0;
  while (s + 1 < a.nshards && a.sh[s + 1].begin <= item) ++s;
  const PoolShard& sh = a.sh[s];
  const uint32_t r0 = (uint32_t)(item - sh.begin);
  const uint32_t r1 = pdiv(r0, a.dcv);
  const int c = (int)(r0 - r1 * (uint32_t)(a.channels / VEC)) * VEC;
  const uint32_t r2 = pdiv(r1, a.dext[s][0]);
  const int ow = (int)(r1 - r2 * (uint32_t)sh.oext[2]);
  const uint32_t r3 = pdiv(r2, a.dext[s][1]);
  const int oh = (int)(r2 - r3 * (uint32_t)sh.oext[1]);
  const uint32_t r4 = pdiv(r3, a.dext[s][2]);
  const int od = (int)(r3 - r4 * (uint32_t)sh.oext[0]);
  const int n = (int)r4;
  const TI* base = reinterpret_cast<const TI*>(sh.in) + n * sh.isn + (int64_t)od * a.stride * sh.is[0] +
                   (int64_t)oh * a.stride * sh.is[1] + (int64_t)ow * a.stride * sh.is[2] + c;
  constexpr int KD = ND == 3 ? K : 1;
  float x[KD * K * K][VEC];
#pragma unroll
  for (int tz = 0; tz < KD; ++tz)
#pragma unroll
    for (int ty = 0; ty < K; ++ty)
#pragma unroll
      for (int tx = 0; tx < K; ++tx)
        if constexpr (ND == 2) ldv_nt<TI, VEC>(base + ty * sh.is[1] + tx * sh.is[2], x[ty * K + tx]);
        else ldv<TI, VEC>(base + tz * sh.is[0] + ty * sh.is[1] + tx * sh.is[2], x[(tz * K + ty) * K + tx]);
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = MAX ? -INFINITY : 0.f;
#pragma unroll
  for (int t = 0; t < KD * K * K; ++t)     // taps in the general kernel's order
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = MAX ? fmaxf(acc[v], x[t][v]) : acc[v] + x[t][v];
  if (!MAX) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] *= a.inv_count;
  }
  stv_nt<TO, VEC>(reinterpret_cast<TO*>(sh.out) + n * sh.osn + od * sh.os[0] + oh * sh.os[1] + ow * sh.os[2] + c, acc);
}

bool pooled_sizes(const std::vector<int64_t>& in, int64_t k, int64_t s, std::vector<int64_t>& out,
                  std::vector<int64_t>& first) {
  int64_t n = 0;
  for (int64_t v : in) n += v;
  if (n < k) return false;
  const int64_t n_out = (n - k) / s + 1;
  out.clear();
  first.clear();
  int64_t a = 0;
  for (int64_t e : in) {
    const int64_t f = (a + s - 1) / s;
    const int64_t end = std::min((a + e + s - 1) / s, n_out);
    out.push_back(end - f);
    first.push_back(f);
    a += e;
  }
  return true;
}

}  // namespace
}  // namespace st

using namespace st;

extern "C" {

st_status st_plan_pooled(const st_plan* in_plan, int32_t ksize, int32_t stride, const int32_t* out_halo_or_null,
                         st_dtype out_dtype, st_plan** out) {
  auto err = [](st_status s, const std::string& m) { return fail(s, "st_plan_pooled: " + m); };
  if (!in_plan || !out) return err(ST_ERR_INVALID_ARG, "NULL argument");
  *out = nullptr;
  if (ksize < 1 || stride < 1) return err(ST_ERR_INVALID_ARG, "ksize and stride must be >= 1");
  const int nd = in_plan->ndim;
  int64_t spatial[ST_MAX_NDIM];
  int32_t counts[ST_MAX_NDIM], halo[ST_MAX_NDIM];
  std::vector<int64_t> concat;
  for (int a = 0; a < nd; ++a) {
    const int ia = axis_of(in_plan, a);
    std::vector<int64_t> sz, first;
    if (!pooled_sizes(in_plan->sizes[ia], ksize, stride, sz, first))
      return err(ST_ERR_BAD_SHAPE, "window larger than the volume");
    int64_t tot = 0;
    for (size_t i = 0; i < sz.size(); ++i) {
      if (sz[i] < 1) {
        char buf[160];
        std::snprintf(buf, sizeof buf, "axis %d shard %zu holds no window start", a, i);
        return err(ST_ERR_SHARD_TOO_SMALL, buf);
      }
      tot += sz[i];
      concat.push_back(sz[i]);
    }
    spatial[a] = tot;
    counts[a] = (int32_t)sz.size();
    halo[a] = out_halo_or_null ? out_halo_or_null[a] : 0;
  }
  return st_plan_shards(nd, in_plan->batch, in_plan->channels, spatial, counts, concat.data(), halo, out_dtype, out);
}

st_status st_pool_sharded(const st_plan* in_plan, const void* const* in_bufs, int32_t ksize, int32_t stride,
                          int32_t mode, const st_plan* out_plan, void* const* out_bufs, void* stream) {
  auto err = [](st_status s, const std::string& m) { return fail(s, "st_pool_sharded: " + m); };
  if (!in_plan || !out_plan || !in_bufs || !out_bufs) return err(ST_ERR_INVALID_ARG, "NULL argument");
  if (ksize < 1 || stride < 1) return err(ST_ERR_INVALID_ARG, "ksize and stride must be >= 1");
  if (mode != 0 && mode != 1) return err(ST_ERR_INVALID_ARG, "mode must be 0 (average) or 1 (max)");
  if (out_plan->ndim != in_plan->ndim || out_plan->batch != in_plan->batch ||
      out_plan->channels != in_plan->channels || out_plan->shards.size() != in_plan->shards.size())
    return err(ST_ERR_BAD_SHAPE, "output plan does not match the input plan");
  if (out_plan->dtype != in_plan->dtype && out_plan->dtype != ST_F32)
    return err(ST_ERR_UNSUPPORTED, "output dtype must be the input's or fp32");
  PoolArgs a{};
  a.nshards = (int)in_plan->shards.size();
  a.batch = (int)in_plan->batch;
  a.channels = (int)in_plan->channels;
  a.k = ksize;
  a.stride = stride;
  a.ndim = in_plan->ndim;
  a.mode = mode;
  int64_t count = 1;
  for (int i = 0; i < in_plan->ndim; ++i) count *= ksize;
  a.inv_count = 1.0f / (float)count;
  const int ie = in_plan->esize, oe = out_plan->esize;
  a.vec = a.channels % (16 / ie) == 0 ? 16 / ie : 1;      // one 16-byte load per tap
  // per-axis pooled sizes and first owned outputs; the output plan must be the derived one
  std::vector<int64_t> first[kAxes];
  for (int ax = 0; ax < kAxes; ++ax) {
    if (ax < kAxes - in_plan->ndim) {
      first[ax].assign(in_plan->nshards[ax], 0);
      continue;
    }
    std::vector<int64_t> sz;
    if (!pooled_sizes(in_plan->sizes[ax], ksize, stride, sz, first[ax]))
      return err(ST_ERR_BAD_SHAPE, "window larger than the volume");
    if (sz != out_plan->sizes[ax]) return err(ST_ERR_BAD_SHAPE, "output plan is not the pooled plan of the input");
  }
  int64_t total = 0;
  bool small = true;
  for (size_t i = 0; i < in_plan->shards.size(); ++i) {
    if (!in_bufs[i] || !out_bufs[i]) return err(ST_ERR_INVALID_ARG, "NULL shard buffer");
    if (!aligned16(in_bufs[i]) || !aligned16(out_bufs[i])) return err(ST_ERR_ALIGNMENT, "shard buffers must be 16-byte aligned");
    const Shard& si = in_plan->shards[i];
    const Shard& so = out_plan->shards[i];
    PoolShard& p = a.sh[i];
    const int64_t C = a.channels;
    p.is[2] = C;
    p.is[1] = si.pad[2] * C;
    p.is[0] = si.pad[1] * p.is[1];
    p.isn = si.pad[0] * p.is[0];
    p.os[2] = C;
    p.os[1] = so.pad[2] * C;
    p.os[0] = so.pad[1] * p.os[1];
    p.osn = so.pad[0] * p.os[0];
    int64_t in_off = 0, out_off = 0;
    for (int ax = 0; ax < kAxes; ++ax) {
      const bool sp = ax >= kAxes - in_plan->ndim;
      const int64_t f = sp ? first[ax][si.grid[ax]] : 0;
      // first window's first cell in the shard's padded coordinates
      const int64_t lo = sp ? f * stride - si.off[ax] + in_plan->halo[ax] : 0;
      // last window's end must stay inside the padded buffer
      const int64_t hi = sp ? lo + (so.ext[ax] - 1) * stride + ksize : 1;
      if (lo < 0 || hi > si.pad[ax]) return err(ST_ERR_BAD_SHAPE, "input halo smaller than the window needs (ksize - 1)");
      in_off += lo * p.is[ax];
      out_off += out_plan->halo[ax] * p.os[ax];
      p.oext[ax] = (int32_t)so.ext[ax];
    }
    p.in = static_cast<const char*>(in_bufs[i]) + in_off * ie;
    p.out = static_cast<char*>(out_bufs[i]) + out_off * oe;
    p.begin = total;
    const int64_t items = a.batch * (int64_t)so.ext[0] * so.ext[1] * so.ext[2] * (a.channels / a.vec);
    total += items;
    small = small && items < ((int64_t)1 << 31);
    for (int e = 0; e < 3; ++e) a.dext[i][e] = pool_div((uint32_t)std::max<int64_t>(1, so.ext[2 - e]));
  }
  a.total = total;
  if (total == 0) return ST_OK;
  a.dcv = pool_div((uint32_t)(a.channels / a.vec));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  const bool mx = mode == 1;
  const bool bi = in_plan->dtype == ST_BF16, bo = out_plan->dtype == ST_BF16;
  // k = 2 or 3 with every shard's items below 2^31: pool_fixed
  const int fixed = small && (ksize == 2 || ksize == 3) ? ksize * 10 + in_plan->ndim : 0;
#define ST_POOL_FIXED(TI, TO, V, MX)                                                                       \
  do {                                                                                                     \
    if (fixed == 22) hipLaunchKernelGGL((pool_fixed<TI, TO, V, MX, 2, 2>), grid, block, 0, st, a);         \
    else if (fixed == 23) hipLaunchKernelGGL((pool_fixed<TI, TO, V, MX, 2, 3>), grid, block, 0, st, a);    \
    else if (fixed == 32) hipLaunchKernelGGL((pool_fixed<TI, TO, V, MX, 3, 2>), grid, block, 0, st, a);    \
    else hipLaunchKernelGGL((pool_fixed<TI, TO, V, MX, 3, 3>), grid, block, 0, st, a);                     \
  } while (0)
#define ST_POOL_LAUNCH(TI, TO, V)                                                                     \
  do {                                                                                                \
    if (fixed && mx) ST_POOL_FIXED(TI, TO, V, true);                                                  \
    else if (fixed) ST_POOL_FIXED(TI, TO, V, false);                                                  \
    else if (mx) hipLaunchKernelGGL((pool_kernel<TI, TO, V, true>), grid, block, 0, st, a);           \
    else hipLaunchKernelGGL((pool_kernel<TI, TO, V, false>), grid, block, 0, st, a);                  \
  } while (0)
  if (bi && bo) {
    if (a.vec == 8) ST_POOL_LAUNCH(uint16_t, uint16_t, 8); else ST_POOL_LAUNCH(uint16_t, uint16_t, 1);
  } else if (bi) {
    if (a.vec == 8) ST_POOL_LAUNCH(uint16_t, float, 8); else ST_POOL_LAUNCH(uint16_t, float, 1);
  } else {
    if (a.vec == 4) ST_POOL_LAUNCH(float, float, 4); else ST_POOL_LAUNCH(float, float, 1);
  }
#undef ST_POOL_LAUNCH
#undef ST_POOL_FIXED
  return launch_check("st_pool_sharded: launch");
}

}  // extern "C"
