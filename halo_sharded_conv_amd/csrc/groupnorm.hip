// Split-statistics GroupNorm over all shards.
//
// "Technical summary: ShardTensor - domain parallelism for scientific machine
// learning", section 2, "Implementation details", "Communication":
// normalisation stays consistent with the unsharded model because per-chunk
// statistics are combined with a collective (all-reduce).  On one GPU the
// all-reduce is the combine kernel below, summing the per-shard partials in
// HBM.  GroupNorm itself (contiguous channel groups, biased variance, eps
// inside the square root, per-channel affine) is the standard definition;
// the pages only say "normalisation".
//
// Exact statistics.  For a group with element count M (over all shards) and
// m = max |y|, let L be the bit length of M and e the exponent with
// 2^(e-1) <= m < 2^e.  Each element contributes
//     q1 = rint(y   * 2^(52 - L - e))       |q1| <= 2^(52-L)
//     q2 = rint(y^2 * 2^(52 - L - 2e))      |q2| <= 2^(52-L)
// so every partial sum of at most M terms is an integer of magnitude below
// 2^52.  fp64 adds such integers exactly, in any order and grouping, so the
// per-shard partials, their combine and the final (mean, rstd) are the same
// bits for every shard plan.  y^2 of an fp32 value is exact in fp64.
//
// Kernels (all HBM-streaming over y, float4 per lane):
//   gn_fill    zero the partial sums (and the max scratch)
//   gn_max     max |y| per (n, group)   (only when the conv did not fuse it)
//   gn_stats   per-shard sum q1, sum q2 per (n, group)
//   gn_combine sum over shards; mean, var, rstd in fp64 -> fp32
//   gn_apply_stream  z = (y - mean_g) * (rstd_g * gamma_c) + beta_c, one
//              workgroup per chunk of the output in chunk order
//   gn_apply   the same as persistent workgroups, optionally with the
//              combine in its prologue (one launch fewer: small outputs)
#include <algorithm>
#include <mutex>
#include <type_traits>
#include <string>

#include "internal.h"

namespace st {
namespace {

constexpr int kNT = 256;        // threads per block
constexpr int kIter = 32;       // vectors per thread per item (a multiple of kPart)
constexpr int kPart = 8;        // vectors per thread per apply work unit
// threads (and vectors) per chunk of the chunked apply kernels: 64 where the
// batch item's coefficient row (C x 16 bytes) is at most a chunk, else 256
constexpr int kStreamSmall = 64, kStreamLarge = 256;
constexpr int stream_tpb(int C) { return C <= kStreamSmall ? kStreamSmall : kStreamLarge; }
static_assert(kNT * kIter % kStreamLarge == 0 && kStreamLarge % kStreamSmall == 0, "whole chunks per item");

struct GnShard {
  const float* y;
  float* z;                     // backward: dy
  const float* dz;              // backward only: the gradient arriving at z
  int64_t vecs_per_n;           // vectors in one batch item of this shard
  int32_t item_begin;           // first item of this shard
  int32_t items_per_n;
};

struct GnArgs {
  int32_t nshards, batch, channels, groups;
  int32_t total_items;
  int32_t lbits;                // bit length of the per-group element count M
  double m_count;               // M (exact in fp64)
  double eps;
  double* partials;             // [S][N][G][2]
  float* stats;                 // [N][G][2]
  int32_t* scales;              // [N][G][2]
  uint32_t* ymax;               // [N][G]
  float4* chan;                 // [N][C] (mean, scale, beta, 0)
  const float* gamma;
  const float* beta;
  GnShard sh[ST_MAX_SHARDS];
};
static_assert(sizeof(GnArgs) <= kMaxKernargBytes, "kernel argument struct too large");

template <int VW> struct Vec;
template <> struct Vec<4> {
  using T = float4;
  static __device__ __forceinline__ float get(const T& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
  }
};
template <> struct Vec<1> {
  using T = float;
  static __device__ __forceinline__ float get(const T& v, int) { return v; }
};

// streaming load (y is read once per pass): the non-temporal hint keeps
// it from displacing lines that other blocks still need
template <int VW>
__device__ __forceinline__ typename Vec<VW>::T load_nt(const typename Vec<VW>::T* p, int64_t i) {
  if constexpr (VW == 4) {
    typedef float nf4 __attribute__((ext_vector_type(4)));
    const nf4 t = __builtin_nontemporal_load(reinterpret_cast<const nf4*>(p) + i);
    return make_float4(t.x, t.y, t.z, t.w);
  } else {
    return __builtin_nontemporal_load(p + i);
  }
}

__device__ __forceinline__ void decode_item(const GnArgs& a, int item, int& s, int& n, int& k) {
  s = 0;
  while (s + 1 < a.nshards && a.sh[s + 1].item_begin <= item) ++s;
  const int r = item - a.sh[s].item_begin;
  n = r / a.sh[s].items_per_n;
  k = r - n * a.sh[s].items_per_n;
}

// rint(d * f) for a power of two f and |d * f| <= 2^51 (d * f is exact): the
// fused multiply-add fl(d * f + 1.5 * 2^52) rounds once, to the integer
// nearest d * f with ties to even (1.5 * 2^52 is even and its ulp is 1), and
// its bit pattern exceeds that of 1.5 * 2^52 by exactly that integer, also
// across the exponent step at 2^53.  Lanes add the patterns as 64-bit
// integers (one instruction) and subtract count * bits(1.5 * 2^52) once, so
// each term costs one FMA and one integer add instead of a multiply, a
// rounding and an fp64 add, with the same exact sum.
constexpr double kRoundMagic = 6755399441055744.0;            // 1.5 * 2^52
constexpr uint64_t kRoundMagicBits = 0x4338000000000000ull;
__device__ __forceinline__ uint64_t rint_bits(double d, double f) {
  return (uint64_t)__double_as_longlong(fma(d, f, kRoundMagic));
}
// the exact sum of `count` terms accumulated by rint_bits (|sum| < 2^53)
__device__ __forceinline__ double rint_sum(uint64_t acc, uint64_t count) {
  return (double)(int64_t)(acc - count * kRoundMagicBits);
}

// exponents (e1, e2) of a group from its max |y| (bits)
__device__ __forceinline__ void group_scales(uint32_t mbits, int lbits, int& e1, int& e2) {
  const float m = __uint_as_float(mbits);
  if (!(m > 0.f)) { e1 = 0; e2 = 0; return; }
  int e;
  (void)frexpf(m, &e);            // m = f * 2^e, f in [0.5, 1)
  e1 = 52 - lbits - e;
  e2 = 52 - lbits - 2 * e;
}

__global__ void gn_fill(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int VW, bool FIXED>
__global__ __launch_bounds__(kNT) void gn_max(const GnArgs a) {
  using V = Vec<VW>;
  extern __shared__ uint32_t smax[];   // C entries
  const int tid = threadIdx.x;
  const int C = a.channels;
  for (int i = tid; i < C; i += kNT) smax[i] = 0u;
  float mx[VW];
#pragma unroll
  for (int j = 0; j < VW; ++j) mx[j] = 0.f;
  int cur = -1, cur_n = 0;
  auto flush = [&](int n) {
    __syncthreads();
    if (FIXED) {
      const int c0 = (tid * VW) % C;
#pragma unroll
      for (int j = 0; j < VW; ++j) atomicMax(&smax[c0 + j], __float_as_uint(mx[j]));
    }
    __syncthreads();
    const int gs = C / a.groups;
    for (int g = tid; g < a.groups; g += kNT) {
      uint32_t m = 0;
      for (int c = g * gs; c < (g + 1) * gs; ++c) m = max(m, smax[c]);
      atomicMax(&a.ymax[n * a.groups + g], m);
    }
    __syncthreads();
    for (int i = tid; i < C; i += kNT) smax[i] = 0u;
#pragma unroll
    for (int j = 0; j < VW; ++j) mx[j] = 0.f;
  };
  for (int item = blockIdx.x; item < a.total_items; item += gridDim.x) {
    int s, n, k;
    decode_item(a, item, s, n, k);
    const int key = s * a.batch + n;
    if (key != cur) {
      if (cur >= 0) flush(cur_n);
      cur = key;
      cur_n = n;
    }
    const GnShard& sh = a.sh[s];
    const typename V::T* y = reinterpret_cast<const typename V::T*>(sh.y) + n * sh.vecs_per_n;
    const int64_t v0 = (int64_t)k * kNT * kIter + tid;
    // as in gn_stats: every load issues before the first is used, non-temporal,
    // and only an item that ends past the shard clamps and masks
    auto body = [&](auto tail_tag) {
      constexpr bool kTail = decltype(tail_tag)::value;
      typename V::T val[kIter];
#pragma unroll
      for (int i = 0; i < kIter; ++i) {
        const int64_t v = v0 + i * kNT;
        if (kTail) {
          const typename V::T t = load_nt<VW>(y, v < sh.vecs_per_n ? v : sh.vecs_per_n - 1);
          val[i] = v < sh.vecs_per_n ? t : typename V::T{};
        } else {
          val[i] = load_nt<VW>(y, v);
        }
      }
#pragma unroll
      for (int i = 0; i < kIter; ++i) {
        const int64_t v = v0 + i * kNT;
#pragma unroll
        for (int j = 0; j < VW; ++j) {
          const float f = fabsf(V::get(val[i], j));
          if (FIXED) mx[j] = fmaxf(mx[j], f);
          else if (!kTail || v < sh.vecs_per_n) atomicMax(&smax[(int)((v * VW + j) % C)], __float_as_uint(f));
        }
      }
    };
    if ((int64_t)(k + 1) * kNT * kIter <= sh.vecs_per_n) body(std::false_type{});
    else body(std::true_type{});
  }
  if (cur >= 0) flush(cur_n);
}

template <int VW, bool FIXED>
__global__ __launch_bounds__(kNT) void gn_stats(const GnArgs a) {
  using V = Vec<VW>;
  extern __shared__ double gn_lds[];   // 4*C: sums, sums of squares, 2^e1, 2^e2 per channel
  const int tid = threadIdx.x;
  const int C = a.channels;
  double* s1 = gn_lds;
  double* s2 = gn_lds + C;
  double* sc1 = gn_lds + 2 * C;
  double* sc2 = gn_lds + 3 * C;
  const int gs = C / a.groups;
  if (blockIdx.x == 0) {
    for (int i = tid; i < a.batch * a.groups; i += kNT) {
      int e1, e2;
      group_scales(a.ymax[i], a.lbits, e1, e2);
      a.scales[2 * i + 0] = e1;
      a.scales[2 * i + 1] = e2;
    }
  }
  for (int i = tid; i < C; i += kNT) { s1[i] = 0.0; s2[i] = 0.0; }
  uint64_t acc1[VW], acc2[VW], cnt = 0;   // FIXED: rint_bits sums over cnt terms per channel
#pragma unroll
  for (int j = 0; j < VW; ++j) { acc1[j] = 0; acc2[j] = 0; }
  int cur = -1, cur_s = 0, cur_n = 0;
  double f1[VW], f2[VW];
  auto flush = [&](int s, int n) {
    __syncthreads();
    if (FIXED) {
      const int c0 = (tid * VW) % C;
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        atomicAdd(&s1[c0 + j], rint_sum(acc1[j], cnt));
        atomicAdd(&s2[c0 + j], rint_sum(acc2[j], cnt));
      }
    }
    __syncthreads();
    for (int g = tid; g < a.groups; g += kNT) {
      double t1 = 0.0, t2 = 0.0;
      for (int c = g * gs; c < (g + 1) * gs; ++c) { t1 += s1[c]; t2 += s2[c]; }
      double* p = a.partials + (((size_t)s * a.batch + n) * a.groups + g) * 2;
      atomicAdd(p + 0, t1);
      atomicAdd(p + 1, t2);
    }
    __syncthreads();
    for (int i = tid; i < C; i += kNT) { s1[i] = 0.0; s2[i] = 0.0; }
#pragma unroll
    for (int j = 0; j < VW; ++j) { acc1[j] = 0; acc2[j] = 0; }
    cnt = 0;
  };
  for (int item = blockIdx.x; item < a.total_items; item += gridDim.x) {
    int s, n, k;
    decode_item(a, item, s, n, k);
    const int key = s * a.batch + n;
    if (key != cur) {
      if (cur >= 0) flush(cur_s, cur_n);
      __syncthreads();
      for (int c = tid; c < C; c += kNT) {
        int e1, e2;
        group_scales(a.ymax[n * a.groups + c / gs], a.lbits, e1, e2);
        sc1[c] = ldexp(1.0, e1);
        sc2[c] = ldexp(1.0, e2);
      }
      __syncthreads();
      if (FIXED) {
        const int c0 = (tid * VW) % C;
#pragma unroll
        for (int j = 0; j < VW; ++j) { f1[j] = sc1[c0 + j]; f2[j] = sc2[c0 + j]; }
      }
      cur = key;
      cur_s = s;
      cur_n = n;
    }
    const GnShard& sh = a.sh[s];
    const typename V::T* y = reinterpret_cast<const typename V::T*>(sh.y) + n * sh.vecs_per_n;
    const int64_t v0 = (int64_t)k * kNT * kIter + tid;
    // an item that ends inside the shard needs no clamps or masks
    auto body = [&](auto tail_tag) {
      constexpr bool kTail = decltype(tail_tag)::value;
      typename V::T val[kIter];
#pragma unroll
      for (int i = 0; i < kIter; ++i) {
        const int64_t v = v0 + i * kNT;
        // every load issues (clamped index; the tail is masked afterwards), so
        // all of them are in flight before the first is used
        if (kTail) {
          const typename V::T t = load_nt<VW>(y, v < sh.vecs_per_n ? v : sh.vecs_per_n - 1);
          val[i] = v < sh.vecs_per_n ? t : typename V::T{};   // zeros contribute 0
        } else {
          val[i] = load_nt<VW>(y, v);
        }
      }
#pragma unroll
      for (int i = 0; i < kIter; ++i) {
        const int64_t v = v0 + i * kNT;
#pragma unroll
        for (int j = 0; j < VW; ++j) {
          const double d = (double)V::get(val[i], j);
          if (FIXED) {
            acc1[j] += rint_bits(d, f1[j]);
            acc2[j] += rint_bits(d, d * f2[j]);   // d * (d * 2^e2) = d^2 * 2^e2 exactly
          } else if (!kTail || v < sh.vecs_per_n) {
            const int c = (int)((v * VW + j) % C);
            atomicAdd(&s1[c], rint(d * sc1[c]));
            atomicAdd(&s2[c], rint((d * d) * sc2[c]));
          }
        }
      }
    };
    if ((int64_t)(k + 1) * kNT * kIter <= sh.vecs_per_n) body(std::false_type{});
    else body(std::true_type{});
    cnt += kIter;
  }
  if (cur >= 0) flush(cur_s, cur_n);
}

// (mean, rstd) of group i = n * G + g from the per-shard partials, in fp64;
// the shard sums are exact integers, so their order does not matter
__device__ __forceinline__ void group_moments(const GnArgs& a, int i, double& mean, double& rstd) {
  const int n = i / a.groups, g = i - n * a.groups;
  double t1 = 0.0, t2 = 0.0;
  for (int s = 0; s < a.nshards; ++s) {
    const double* p = a.partials + (((size_t)s * a.batch + n) * a.groups + g) * 2;
    t1 += p[0];
    t2 += p[1];
  }
  const int e1 = a.scales[2 * i + 0], e2 = a.scales[2 * i + 1];
  mean = ldexp(t1, -e1) / a.m_count;
  const double ey2 = ldexp(t2, -e2) / a.m_count;
  double var = ey2 - mean * mean;
  if (var < 0.0) var = 0.0;
  rstd = 1.0 / sqrt(var + a.eps);
}

__global__ void gn_combine(const GnArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.batch * a.groups) return;
  const int n = i / a.groups, g = i - n * a.groups;
  double mean, rstd;
  group_moments(a, i, mean, rstd);
  a.stats[2 * i + 0] = (float)mean;
  a.stats[2 * i + 1] = (float)rstd;
  const int gs = a.channels / a.groups;
  for (int c = g * gs; c < (g + 1) * gs; ++c) {
    const double gam = a.gamma ? (double)a.gamma[c] : 1.0;
    const float bet = a.beta ? a.beta[c] : 0.f;
    a.chan[(size_t)n * a.channels + c] = make_float4((float)mean, (float)(rstd * gam), bet, 0.f);
  }
}

// COMBINE (with FIXED): the combine runs in the prologue of every workgroup
// (one thread per (n, group) into LDS, workgroup 0 also writes the
// statistics), so the three-kernel chain is two launches; each lane then
// forms its channels' coefficients exactly as gn_combine does.
template <int VW, bool FIXED, bool COMBINE>
__global__ __launch_bounds__(kNT) void gn_apply(const GnArgs a) {
  using V = Vec<VW>;
  static_assert(!COMBINE || FIXED, "the fused combine serves the per-lane coefficient path");
  extern __shared__ double2 smom[];                   // COMBINE: [N * G] (mean, rstd)
  const int tid = threadIdx.x;
  const int C = a.channels;
  if constexpr (COMBINE) {
    for (int i = tid; i < a.batch * a.groups; i += kNT) {
      double mean, rstd;
      group_moments(a, i, mean, rstd);
      smom[i] = make_double2(mean, rstd);
      if (blockIdx.x == 0) {
        a.stats[2 * i + 0] = (float)mean;
        a.stats[2 * i + 1] = (float)rstd;
      }
    }
    __syncthreads();
  }
  int cur = -1;
  float4 p[VW];
  // work units of kPart vectors per thread (a part of an item: more waves
  // in flight), visited last unit first so the pass begins on the part of y
  // the statistics pass read last
  constexpr int kParts = kIter / kPart;
  static_assert(kIter % kPart == 0, "whole parts per item");
  for (int h = blockIdx.x; h < kParts * a.total_items; h += gridDim.x) {
    const int hr = kParts * a.total_items - 1 - h;
    int s, n, k;
    decode_item(a, hr / kParts, s, n, k);
    const int key = s * a.batch + n;
    if (FIXED && key != cur) {
      const int c0 = (tid * VW) % C;
      const int gs = C / a.groups;
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        if constexpr (COMBINE) {
          const int c = c0 + j;
          const double2 m = smom[n * a.groups + c / gs];
          const double gam = a.gamma ? (double)a.gamma[c] : 1.0;
          p[j] = make_float4((float)m.x, (float)(m.y * gam), a.beta ? a.beta[c] : 0.f, 0.f);
        } else {
          p[j] = a.chan[(size_t)n * C + c0 + j];
        }
      }
      cur = key;
    }
    const GnShard& sh = a.sh[s];
    const typename V::T* y = reinterpret_cast<const typename V::T*>(sh.y) + n * sh.vecs_per_n;
    typename V::T* z = reinterpret_cast<typename V::T*>(sh.z) + n * sh.vecs_per_n;
    const int64_t v0 = (int64_t)k * kNT * kIter + (hr % kParts) * kNT * kPart + tid;
    typename V::T val[kPart];
#pragma unroll
    for (int i = 0; i < kPart; ++i) {
      const int64_t v = v0 + i * kNT;
      val[i] = load_nt<VW>(y, v < sh.vecs_per_n ? v : sh.vecs_per_n - 1);   // tail: stored by no lane
    }
#pragma unroll
    for (int i = 0; i < kPart; ++i) {
      const int64_t v = v0 + i * kNT;
      if (v >= sh.vecs_per_n) break;
      float out[VW];
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        float4 q;
        if (FIXED) q = p[j];
        else q = a.chan[(size_t)n * C + (int)((v * VW + j) % C)];
        out[j] = fmaf(V::get(val[i], j) - q.x, q.y, q.z);
      }
      if constexpr (VW == 4) {
        typedef float nf4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(nf4{out[0], out[1], out[2], out[3]}, reinterpret_cast<nf4*>(&z[v]));
      }
      else __builtin_nontemporal_store(out[0], &z[v]);
    }
  }
}

// The same apply with one vector per lane and one workgroup per chunk of kNT
// vectors, in chunk order and without a grid-stride loop: the workgroups in
// flight then cover one compact, advancing window of y and z, which streams
// faster than persistent workgroups spread over the volume (a plain
// read-and-write pass moves ~6.5-6.8 TB/s this way against ~5.3 TB/s with
// 32 persistent workgroups per CU and 8 vectors per lane).  The coefficients
// of the chunk's batch item go through LDS, loaded after y's load is issued.
template <int VW, bool FIXED, int TPB>
__global__ __launch_bounds__(TPB) void gn_apply_stream(const GnArgs a) {
  using V = Vec<VW>;
  extern __shared__ float4 srow[];                    // [C] (mean, scale, beta, 0) of batch item n
  const int tid = threadIdx.x;
  const int C = a.channels;
  const int chunk = blockIdx.x;
  int s, n, k;
  constexpr int kChunks = kNT * kIter / TPB;          // chunks per item
  decode_item(a, chunk / kChunks, s, n, k);
  const GnShard& sh = a.sh[s];
  const int64_t first = ((int64_t)k * kChunks + chunk % kChunks) * TPB;
  if (first >= sh.vecs_per_n) return;                 // past the item's last vector: the whole workgroup
  const int64_t v = first + tid;
  const bool in = v < sh.vecs_per_n;
  const typename V::T* y = reinterpret_cast<const typename V::T*>(sh.y) + n * sh.vecs_per_n;
  typename V::T* z = reinterpret_cast<typename V::T*>(sh.z) + n * sh.vecs_per_n;
  const typename V::T val = load_nt<VW>(y, in ? v : first);
  for (int i = tid; i < C; i += TPB) srow[i] = a.chan[(size_t)n * C + i];
  __syncthreads();
  if (!in) return;
  float out[VW];
#pragma unroll
  for (int j = 0; j < VW; ++j) {
    const float4 q = srow[FIXED ? (tid * VW + j) % C : (int)((v * VW + j) % C)];
    out[j] = fmaf(V::get(val, j) - q.x, q.y, q.z);
  }
  if constexpr (VW == 4) {
    typedef float nf4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(nf4{out[0], out[1], out[2], out[3]}, reinterpret_cast<nf4*>(&z[v]));
  }
  else __builtin_nontemporal_store(out[0], &z[v]);
}

// ---------------------------------------------------------------- backward
//
// Gradients of z = GroupNorm(y) for an upstream gradient dz.  Per (n, g) with
// r = rstd, yhat = (y - mean) * r and g_c = gamma_c * dz:
//     dy = r * (g - mean_g(g) - yhat * mean_g(g * yhat))
//     dgamma_c = sum_{n, positions} dz * yhat,   dbeta_c = sum_{n, positions} dz
// Both group means come from two per-(n, channel) sums, S1 = sum dz and
// S2 = sum dz * yhat:  mean_g(g) = sum_c gamma_c S1 / M and
// mean_g(g * yhat) = sum_c gamma_c S2 / M.  The per-channel sums are exact in
// the same way as the forward statistics: with m = max |dz| of the group
// (2^(ed-1) <= m < 2^ed) and B >= max |yhat| (2^(eh-1) <= B < 2^eh), every
// element contributes
//     q1 = rint(dz        * 2^(52 - L - ed))         |q1| <= 2^(52-L)
//     q2 = rint(dz * yhat * 2^(52 - L - ed - eh))    |q2| <= 2^(52-L)
// (dz * yhat of two fp32 values is exact in fp64).  B comes from the forward
// pass: |yhat| <= (max |y| + |mean|) * rstd, widened by 2^-20 for the two fp32
// roundings of yhat.  So the sums, dgamma, dbeta and dy are the same bits for
// every shard plan.
//
// Kernels: gn_fill (partials), gn_max on dz (unless the caller supplies
// max |dz|), gnb_stats (per-shard S1, S2 per (n, c)), gnb_combine (sums over
// shards; per-channel coefficients; dgamma, dbeta), gnb_apply_stream (or the
// persistent gnb_apply for batch items of 2^31 vectors or more)
//     dy = a_c * dz + k_g * (y - mean_g) + b_g
// with a_c = r gamma_c, k_g = -r^2 mean_g(g yhat), b_g = -r mean_g(g).

// dy written into another shard layout (a padded plan, fp32 or bf16):
// element (n, d, h, w, c) of a shard at p + n*sn + d*sd + h*sh + w*C + c
// n / d for 0 <= n < 2^31 as (n * m) >> p, with p = 31 + ceil(log2 d) and
// m = ceil(2^p / d) < 2^32: the error n (m - 2^p / d) / 2^p stays below 1 / d,
// so the floor is exact (the round-up multiplier method)
struct FastDiv {
  uint32_t m;
  int32_t p;
};
FastDiv fast_div(uint32_t d) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  const int p = 31 + l;
  return FastDiv{(uint32_t)(((1ull << p) + d - 1) / d), p};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (uint32_t)(((uint64_t)n * f.m) >> f.p); }

struct GnbOut {
  void* p;                      // the shard's interior origin
  int64_t sn, sd, sh;           // element strides
  int32_t H, W;                 // interior extents of the two inner spatial axes
  FastDiv fH, fW;               // dividers by H and W
};

enum GnbMode { kDyLikeY = 0, kDyPaddedF32 = 1, kDyPaddedBf16 = 2 };

struct GnbArgs {
  GnArgs g;                     // y = forward input of GroupNorm, z = dy (kDyLikeY), dz
  const float* fstats;          // [N][G][2] (mean, rstd) of the forward pass
  const uint32_t* dzmax;        // [N][G] bits of max |dz|
  double* bpart;                // [S][N][C][2] exact (sum q1, sum q2)
  int32_t* bscales;             // [N][G][2] exponents of q1, q2
  float4* bchan;                // [N][C] (mean, a, k, b)
  float* dgamma;                // [C] or NULL
  float* dbeta;                 // [C] or NULL
  FastDiv fCv;                  // divider by C / VW (vectors per position)
  GnbOut out[ST_MAX_SHARDS];    // kDyPadded*: where dy goes
};
static_assert(sizeof(GnbArgs) <= kMaxKernargBytes, "kernel argument struct too large");

// fp32 -> bf16, round to nearest, ties to even (finite values)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void bwd_scales(uint32_t dzbits, uint32_t ybits, float mean, float rstd, int lbits,
                                           int& e1, int& e2) {
  const float m = __uint_as_float(dzbits);
  if (!(m > 0.f)) { e1 = 0; e2 = 0; return; }
  int ed;
  (void)frexpf(m, &ed);
  e1 = 52 - lbits - ed;
  const double bound = ((double)__uint_as_float(ybits) + fabs((double)mean)) * (double)rstd * (1.0 + 0x1p-20);
  int eh = 0;
  if (bound > 0.0 && bound < 0x1p1000) (void)frexp(bound, &eh);
  e2 = 52 - lbits - ed - eh;
}

template <int VW, bool FIXED>
__global__ __launch_bounds__(kNT) void gnb_stats(const GnbArgs b) {
  using V = Vec<VW>;
  const GnArgs& a = b.g;
  constexpr int kHalf = kIter / 2;      // vectors of y and of dz in flight per thread
  extern __shared__ double gnb_lds[];   // per channel: s1, s2, 2^e1, 2^e2, (mean, rstd)
  const int tid = threadIdx.x;
  const int C = a.channels;
  double* s1 = gnb_lds;
  double* s2 = gnb_lds + C;
  double* sc1 = gnb_lds + 2 * C;
  double* sc2 = gnb_lds + 3 * C;
  float2* mr = reinterpret_cast<float2*>(gnb_lds + 4 * C);
  const int gs = C / a.groups;
  if (blockIdx.x == 0) {
    for (int i = tid; i < a.batch * a.groups; i += kNT) {
      int e1, e2;
      bwd_scales(b.dzmax[i], a.ymax[i], b.fstats[2 * i], b.fstats[2 * i + 1], a.lbits, e1, e2);
      b.bscales[2 * i + 0] = e1;
      b.bscales[2 * i + 1] = e2;
    }
  }
  for (int i = tid; i < C; i += kNT) { s1[i] = 0.0; s2[i] = 0.0; }
  uint64_t acc1[VW], acc2[VW], cnt = 0;   // FIXED: rint_bits sums over cnt terms per channel
  double f1[VW], f2[VW];
  float mu[VW], rs[VW];
#pragma unroll
  for (int j = 0; j < VW; ++j) { acc1[j] = 0; acc2[j] = 0; }
  int cur = -1, cur_s = 0, cur_n = 0;
  auto flush = [&](int s, int n) {
    __syncthreads();
    if (FIXED) {
      const int c0 = (tid * VW) % C;
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        atomicAdd(&s1[c0 + j], rint_sum(acc1[j], cnt));
        atomicAdd(&s2[c0 + j], rint_sum(acc2[j], cnt));
      }
    }
    __syncthreads();
    for (int c = tid; c < C; c += kNT) {
      double* p = b.bpart + (((size_t)s * a.batch + n) * C + c) * 2;
      atomicAdd(p + 0, s1[c]);
      atomicAdd(p + 1, s2[c]);
    }
    __syncthreads();
    for (int i = tid; i < C; i += kNT) { s1[i] = 0.0; s2[i] = 0.0; }
#pragma unroll
    for (int j = 0; j < VW; ++j) { acc1[j] = 0; acc2[j] = 0; }
    cnt = 0;
  };
  for (int item = blockIdx.x; item < a.total_items; item += gridDim.x) {
    int s, n, k;
    decode_item(a, item, s, n, k);
    const int key = s * a.batch + n;
    if (key != cur) {
      if (cur >= 0) flush(cur_s, cur_n);
      __syncthreads();
      for (int c = tid; c < C; c += kNT) {
        const int i = n * a.groups + c / gs;
        int e1, e2;
        bwd_scales(b.dzmax[i], a.ymax[i], b.fstats[2 * i], b.fstats[2 * i + 1], a.lbits, e1, e2);
        sc1[c] = ldexp(1.0, e1);
        sc2[c] = ldexp(1.0, e2);
        mr[c] = make_float2(b.fstats[2 * i], b.fstats[2 * i + 1]);
      }
      __syncthreads();
      if (FIXED) {
        const int c0 = (tid * VW) % C;
#pragma unroll
        for (int j = 0; j < VW; ++j) {
          f1[j] = sc1[c0 + j];
          f2[j] = sc2[c0 + j];
          mu[j] = mr[c0 + j].x;
          rs[j] = mr[c0 + j].y;
        }
      }
      cur = key;
      cur_s = s;
      cur_n = n;
    }
    const GnShard& sh = a.sh[s];
    const typename V::T* y = reinterpret_cast<const typename V::T*>(sh.y) + n * sh.vecs_per_n;
    const typename V::T* dz = reinterpret_cast<const typename V::T*>(sh.dz) + n * sh.vecs_per_n;
#pragma unroll
    for (int hb = 0; hb < kIter; hb += kHalf) {
      const int64_t v0 = (int64_t)k * kNT * kIter + hb * kNT + tid;
      typename V::T vy[kHalf], vd[kHalf];
#pragma unroll
      for (int i = 0; i < kHalf; ++i) {
        const int64_t v = v0 + i * kNT;
        const int64_t vc = v < sh.vecs_per_n ? v : sh.vecs_per_n - 1;
        vy[i] = load_nt<VW>(y, vc);
        vd[i] = load_nt<VW>(dz, vc);
      }
#pragma unroll
      for (int i = 0; i < kHalf; ++i) {
        const int64_t v = v0 + i * kNT;
        const bool in = v < sh.vecs_per_n;
#pragma unroll
        for (int j = 0; j < VW; ++j) {
          if (FIXED) {
            const float yh = (V::get(vy[i], j) - mu[j]) * rs[j];
            const double d = in ? (double)V::get(vd[i], j) : 0.0;   // the tail contributes 0
            acc1[j] += rint_bits(d, f1[j]);
            acc2[j] += rint_bits(d, (double)yh * f2[j]);   // d * (yh * 2^e2) exactly
          } else if (in) {
            const int c = (int)((v * VW + j) % C);
            const float yh = (V::get(vy[i], j) - mr[c].x) * mr[c].y;
            const double d = (double)V::get(vd[i], j);
            atomicAdd(&s1[c], rint(d * sc1[c]));
            atomicAdd(&s2[c], rint((d * (double)yh) * sc2[c]));
          }
        }
      }
    }
    cnt += kIter;
  }
  if (cur >= 0) flush(cur_s, cur_n);
}

__global__ void gnb_combine(const GnbArgs b) {
  const GnArgs& a = b.g;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int C = a.channels, G = a.groups, N = a.batch, gs = C / G;
  auto chan_sum = [&](int n, int c, int q) {   // exact per-(n, c) sum, scaled back
    double t = 0.0;
    for (int s = 0; s < a.nshards; ++s) t += b.bpart[(((size_t)s * N + n) * C + c) * 2 + q];
    return ldexp(t, -b.bscales[2 * (n * G + c / gs) + q]);
  };
  if (i < N * G) {
    const int n = i / G, g = i - n * G;
    const double r = (double)b.fstats[2 * i + 1];
    double t1 = 0.0, t2 = 0.0;
    for (int c = g * gs; c < (g + 1) * gs; ++c) {
      const double gam = a.gamma ? (double)a.gamma[c] : 1.0;
      t1 += gam * chan_sum(n, c, 0);
      t2 += gam * chan_sum(n, c, 1);
    }
    const double m1 = t1 / a.m_count, m2 = t2 / a.m_count;
    const float kk = (float)(-r * r * m2), bb = (float)(-r * m1);
    for (int c = g * gs; c < (g + 1) * gs; ++c) {
      const double gam = a.gamma ? (double)a.gamma[c] : 1.0;
      b.bchan[(size_t)n * C + c] = make_float4(b.fstats[2 * i], (float)(r * gam), kk, bb);
    }
  }
  if (i < C) {
    double db = 0.0, dg = 0.0;
    for (int n = 0; n < N; ++n) {
      db += chan_sum(n, i, 0);
      dg += chan_sum(n, i, 1);
    }
    if (b.dbeta) b.dbeta[i] = (float)db;
    if (b.dgamma) b.dgamma[i] = (float)dg;
  }
}

template <int VW, bool FIXED, int MODE>
__global__ __launch_bounds__(kNT) void gnb_apply(const GnbArgs b) {
  using V = Vec<VW>;
  const GnArgs& a = b.g;
  const int tid = threadIdx.x;
  const int C = a.channels;
  int cur = -1;
  float4 p[VW];
  constexpr int kParts = kIter / kPart;
  for (int h = blockIdx.x; h < kParts * a.total_items; h += gridDim.x) {
    const int hr = kParts * a.total_items - 1 - h;
    int s, n, k;
    decode_item(a, hr / kParts, s, n, k);
    const int key = s * a.batch + n;
    if (FIXED && key != cur) {
      const int c0 = (tid * VW) % C;
#pragma unroll
      for (int j = 0; j < VW; ++j) p[j] = b.bchan[(size_t)n * C + c0 + j];
      cur = key;
    }
    const GnShard& sh = a.sh[s];
    const typename V::T* y = reinterpret_cast<const typename V::T*>(sh.y) + n * sh.vecs_per_n;
    const typename V::T* dz = reinterpret_cast<const typename V::T*>(sh.dz) + n * sh.vecs_per_n;
    typename V::T* dy = reinterpret_cast<typename V::T*>(sh.z) + n * sh.vecs_per_n;
    const int64_t v0 = (int64_t)k * kNT * kIter + (hr % kParts) * kNT * kPart + tid;
    typename V::T vy[kPart], vd[kPart];
#pragma unroll
    for (int i = 0; i < kPart; ++i) {
      const int64_t v = v0 + i * kNT;
      const int64_t vc = v < sh.vecs_per_n ? v : sh.vecs_per_n - 1;   // tail: stored by no lane
      vy[i] = load_nt<VW>(y, vc);
      vd[i] = load_nt<VW>(dz, vc);
    }
#pragma unroll
    for (int i = 0; i < kPart; ++i) {
      const int64_t v = v0 + i * kNT;
      if (v >= sh.vecs_per_n) break;
      float out[VW];
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        float4 q;
        if (FIXED) q = p[j];
        else q = b.bchan[(size_t)n * C + (int)((v * VW + j) % C)];
        out[j] = fmaf(q.y, V::get(vd[i], j), fmaf(q.z, V::get(vy[i], j) - q.x, q.w));
      }
      if constexpr (MODE == kDyLikeY) {
        if constexpr (VW == 4) {
          typedef float nf4 __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(nf4{out[0], out[1], out[2], out[3]}, reinterpret_cast<nf4*>(&dy[v]));
        }
        else __builtin_nontemporal_store(out[0], &dy[v]);
      } else {
        // the VW channels of this vector sit at one position (C % VW == 0)
        const GnbOut& o = b.out[s];
        const int64_t e0 = v * VW;
        const int64_t pos = e0 / C;
        const int c = (int)(e0 - pos * C);
        const int64_t t = pos / o.W;
        const int w = (int)(pos - t * o.W);
        const int64_t d = t / o.H;
        const int hh = (int)(t - d * o.H);
        const int64_t off = n * o.sn + d * o.sd + hh * o.sh + (int64_t)w * C + c;
        if constexpr (MODE == kDyPaddedF32) {
          if constexpr (VW == 4) {
            typedef float nf4 __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(nf4{out[0], out[1], out[2], out[3]}, reinterpret_cast<nf4*>(static_cast<float*>(o.p) + off));
          }
          else __builtin_nontemporal_store(out[0], static_cast<float*>(o.p) + off);
        } else {
          if constexpr (VW == 4) {
            typedef unsigned int nu2 __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(nu2{bf16_rne(out[0]) | (bf16_rne(out[1]) << 16), bf16_rne(out[2]) | (bf16_rne(out[3]) << 16)},
                                        reinterpret_cast<nu2*>(static_cast<uint16_t*>(o.p) + off));
          }
          else __builtin_nontemporal_store((uint16_t)bf16_rne(out[0]), static_cast<uint16_t*>(o.p) + off);
        }
      }
    }
  }
}

// The backward apply as one vector per lane and one workgroup per chunk of
// kNT vectors in chunk order (the streaming layout of gn_apply_stream).  The
// batch item's coefficients go through LDS.  A padded dy takes its position,
// row and plane by multiply-shift division (every vector index of a batch
// item is below 2^31 on this path).
template <int VW, int MODE, int TPB>
__global__ __launch_bounds__(TPB) void gnb_apply_stream(const GnbArgs b) {
  using V = Vec<VW>;
  const GnArgs& a = b.g;
  extern __shared__ float4 srow[];                    // [C] (mean, a, k, b) of batch item n
  const int tid = threadIdx.x;
  const int C = a.channels;
  const int chunk = blockIdx.x;
  int s, n, k;
  constexpr int kChunks = kNT * kIter / TPB;          // chunks per item
  decode_item(a, chunk / kChunks, s, n, k);
  const GnShard& sh = a.sh[s];
  const int64_t first = ((int64_t)k * kChunks + chunk % kChunks) * TPB;
  if (first >= sh.vecs_per_n) return;                 // past the item's last vector: the whole workgroup
  const int64_t v = first + tid;
  const bool in = v < sh.vecs_per_n;
  const typename V::T* y = reinterpret_cast<const typename V::T*>(sh.y) + n * sh.vecs_per_n;
  const typename V::T* dz = reinterpret_cast<const typename V::T*>(sh.dz) + n * sh.vecs_per_n;
  const typename V::T vy = load_nt<VW>(y, in ? v : first);
  const typename V::T vd = load_nt<VW>(dz, in ? v : first);
  for (int i = tid; i < C; i += TPB) srow[i] = b.bchan[(size_t)n * C + i];
  __syncthreads();
  if (!in) return;
  // the VW channels of a vector sit at one position (VW == 4 only when C % 4 == 0)
  int c0;
  uint32_t pu = 0;
  if constexpr (MODE == kDyLikeY) {
    c0 = (int)((v * VW) % C);
  } else {
    const uint32_t vv = (uint32_t)v;
    pu = fdiv(vv, b.fCv);
    c0 = (int)(vv - pu * (uint32_t)(C / VW)) * VW;
  }
  float out[VW];
#pragma unroll
  for (int j = 0; j < VW; ++j) {
    const float4 q = srow[c0 + j];
    out[j] = fmaf(q.y, V::get(vd, j), fmaf(q.z, V::get(vy, j) - q.x, q.w));
  }
  if constexpr (MODE == kDyLikeY) {
    typename V::T* dy = reinterpret_cast<typename V::T*>(sh.z) + n * sh.vecs_per_n;
    if constexpr (VW == 4) {
      typedef float nf4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(nf4{out[0], out[1], out[2], out[3]}, reinterpret_cast<nf4*>(&dy[v]));
    }
    else __builtin_nontemporal_store(out[0], &dy[v]);
  } else {
    const GnbOut& o = b.out[s];
    const uint32_t tu = fdiv(pu, o.fW), du = fdiv(tu, o.fH);
    const int w = (int)(pu - tu * (uint32_t)o.W);
    const int hh = (int)(tu - du * (uint32_t)o.H);
    const int64_t off = n * o.sn + (int64_t)du * o.sd + hh * o.sh + (int64_t)w * C + c0;
    // non-temporal stores, as for z: dy is read back only by the next pass
    if constexpr (MODE == kDyPaddedF32) {
      if constexpr (VW == 4) {
        typedef float nf4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(nf4{out[0], out[1], out[2], out[3]}, reinterpret_cast<nf4*>(static_cast<float*>(o.p) + off));
      }
      else __builtin_nontemporal_store(out[0], static_cast<float*>(o.p) + off);
    } else {
      if constexpr (VW == 4) {
        typedef unsigned int nu2 __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(nu2{bf16_rne(out[0]) | (bf16_rne(out[1]) << 16), bf16_rne(out[2]) | (bf16_rne(out[3]) << 16)},
                                    reinterpret_cast<nu2*>(static_cast<uint16_t*>(o.p) + off));
      }
      else __builtin_nontemporal_store((uint16_t)bf16_rne(out[0]), static_cast<uint16_t*>(o.p) + off);
    }
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

st_gn_layout layout_of(const st_plan* p, int groups) {
  st_gn_layout l{};
  const size_t S = p->shards.size(), N = (size_t)p->batch, G = (size_t)groups, C = (size_t)p->channels;
  size_t off = 0;
  l.partials_offset = off; off = align256(off + S * N * G * 2 * sizeof(double));
  l.ymax_offset = off;     off = align256(off + N * G * sizeof(uint32_t));
  l.stats_offset = off;    off = align256(off + N * G * 2 * sizeof(float));
  l.scales_offset = off;   off = align256(off + N * G * 2 * sizeof(int32_t));
  l.chan_offset = off;     off = align256(off + N * C * sizeof(float4));
  l.total_bytes = off;
  return l;
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    hipDeviceProp_t prop;
    cus[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess ? prop.multiProcessorCount : 256;
  }
  return cus[dev];
}

// Validates the arguments shared by the three stages and fills GnArgs.
st_status prepare(const st_plan* y_plan, const float* const* y_bufs, float* const* z_bufs,
                  const uint32_t* ymax, int32_t groups, float eps, const float* gamma,
                  const float* beta, void* workspace, size_t workspace_bytes, const char* who,
                  GnArgs& a, int& vw, bool& fixed) {
  auto err = [&](st_status s, const char* m) { return fail(s, std::string(who) + ": " + m); };
  if (!y_plan) return err(ST_ERR_INVALID_ARG, "NULL plan");
  if (y_plan->dtype != ST_F32) return err(ST_ERR_BAD_SHAPE, "y must be fp32");
  for (int ax = 0; ax < kAxes; ++ax)
    if (y_plan->halo[ax] != 0) return err(ST_ERR_BAD_SHAPE, "y plan must have halo 0");
  const int C = (int)y_plan->channels;
  if (groups < 1 || C % groups) return err(ST_ERR_INVALID_ARG, "groups must divide C");
  if (C > 1024) return err(ST_ERR_UNSUPPORTED, "more than 1024 channels");
  if (!(eps >= 0.f)) return err(ST_ERR_INVALID_ARG, "eps must be >= 0");
  const st_gn_layout l = layout_of(y_plan, groups);
  if (!workspace || workspace_bytes < l.total_bytes) return err(ST_ERR_WORKSPACE, "workspace missing or too small");
  if (!aligned16(workspace)) return err(ST_ERR_ALIGNMENT, "workspace not 16-byte aligned");
  for (size_t s = 0; s < y_plan->shards.size(); ++s) {
    if (y_bufs) {
      if (!y_bufs[s]) return err(ST_ERR_INVALID_ARG, "NULL y buffer");
      if (!aligned16(y_bufs[s])) return err(ST_ERR_ALIGNMENT, "y buffers must be 16-byte aligned");
    }
    if (z_bufs) {
      if (!z_bufs[s]) return err(ST_ERR_INVALID_ARG, "NULL z buffer");
      if (!aligned16(z_bufs[s])) return err(ST_ERR_ALIGNMENT, "z buffers must be 16-byte aligned");
    }
  }
  if ((gamma && (reinterpret_cast<uintptr_t>(gamma) & 3)) || (beta && (reinterpret_cast<uintptr_t>(beta) & 3)) ||
      (ymax && (reinterpret_cast<uintptr_t>(ymax) & 3)))
    return err(ST_ERR_ALIGNMENT, "misaligned gamma/beta/ymax");

  char* ws = static_cast<char*>(workspace);
  a = GnArgs{};
  a.nshards = (int)y_plan->shards.size();
  a.batch = (int)y_plan->batch;
  a.channels = C;
  a.groups = groups;
  int64_t positions = 1;
  for (int ax = 0; ax < kAxes; ++ax) positions *= y_plan->spatial[ax];
  const uint64_t M = (uint64_t)(C / groups) * (uint64_t)positions;
  int lbits = 0;
  while (lbits < 64 && (M >> lbits) != 0) ++lbits;
  if (lbits > 50) return err(ST_ERR_UNSUPPORTED, "group too large for exact sums");
  a.lbits = lbits;
  a.m_count = (double)M;
  a.eps = (double)eps;
  a.partials = reinterpret_cast<double*>(ws + l.partials_offset);
  a.stats = reinterpret_cast<float*>(ws + l.stats_offset);
  a.scales = reinterpret_cast<int32_t*>(ws + l.scales_offset);
  a.ymax = ymax ? const_cast<uint32_t*>(ymax) : reinterpret_cast<uint32_t*>(ws + l.ymax_offset);
  a.chan = reinterpret_cast<float4*>(ws + l.chan_offset);
  a.gamma = gamma;
  a.beta = beta;
  vw = C % 4 == 0 ? 4 : 1;
  fixed = (vw * kNT) % C == 0;
  const int64_t item_vecs = (int64_t)kNT * kIter;
  int64_t items = 0;
  for (size_t s = 0; s < y_plan->shards.size(); ++s) {
    const Shard& sd = y_plan->shards[s];
    GnShard& g = a.sh[s];
    g.y = y_bufs ? y_bufs[s] : nullptr;
    g.z = z_bufs ? z_bufs[s] : nullptr;
    g.vecs_per_n = sd.ext[0] * sd.ext[1] * sd.ext[2] * C / vw;
    g.items_per_n = (int32_t)((g.vecs_per_n + item_vecs - 1) / item_vecs);
    g.item_begin = (int32_t)items;
    items += (int64_t)g.items_per_n * a.batch;
    if (items > INT32_MAX / (kIter / kPart)) return err(ST_ERR_UNSUPPORTED, "volume too large");
  }
  a.total_items = (int)items;
  return ST_OK;
}

// 2 blocks of 32 in-flight 16-byte loads per thread per CU (4 blocks: the
// statistics 4-8% slower on every workload, the backward's max and sums 0-4%;
// 1 block: 6-17% slower)
int grid_of(const GnArgs& a) { return std::max(1, std::min(a.total_items, device_cus() * 2)); }

template <int VW, bool FIXED>
st_status launch_partials(GnArgs& a, bool need_max, hipStream_t st) {
  const int grid = grid_of(a);
  if (need_max) {
    hipLaunchKernelGGL((gn_max<VW, FIXED>), dim3(grid), dim3(kNT), (size_t)a.channels * 4, st, a);
    st_status s = launch_check("st_groupnorm_partials: max launch");
    if (s != ST_OK) return s;
  }
  hipLaunchKernelGGL((gn_stats<VW, FIXED>), dim3(grid), dim3(kNT), (size_t)a.channels * 32, st, a);
  return launch_check("st_groupnorm_partials: stats launch");
}

// the chunked apply keeps one batch item's C coefficients in LDS and
// launches one workgroup per chunk
constexpr int kMaxStreamChannels = 4096;   // 64 KiB
bool stream_fits(const GnArgs& a) {
  return a.channels <= kMaxStreamChannels && (int64_t)a.total_items * (kNT * kIter / kStreamSmall) <= INT32_MAX;
}

template <int VW, int TPB>
st_status launch_apply_stream(GnArgs& a, hipStream_t st) {
  const dim3 grid(a.total_items * (kNT * kIter / TPB));
  const size_t shmem = (size_t)a.channels * sizeof(float4);
  // a lane's channels stay fixed when a chunk holds whole positions
  if ((VW * TPB) % a.channels == 0) hipLaunchKernelGGL((gn_apply_stream<VW, true, TPB>), grid, dim3(TPB), shmem, st, a);
  else hipLaunchKernelGGL((gn_apply_stream<VW, false, TPB>), grid, dim3(TPB), shmem, st, a);
  return launch_check("st_groupnorm_apply: launch");
}

template <int VW, bool FIXED, bool COMBINE = false>
st_status launch_apply(GnArgs& a, hipStream_t st) {
  // 32 workgroups per CU: 1-2% faster than 8 or 16 on the 512^3, 256^3 and
  // 2048^2 outputs (8-vector parts; 4 and 16 were slower)
  const int grid = std::max(1, std::min((kIter / kPart) * a.total_items, device_cus() * 32));
  const size_t shmem = COMBINE ? (size_t)a.batch * a.groups * sizeof(double2) : 0;
  hipLaunchKernelGGL((gn_apply<VW, FIXED, COMBINE>), dim3(grid), dim3(kNT), shmem, st, a);
  return launch_check("st_groupnorm_apply: launch");
}
// the fused combine keeps N * G moments (16 bytes each) in LDS
constexpr int kMaxFusedGroups = 256;   // 4 KiB: 32 workgroups per CU still fit
// below this many items (8192 vectors each) the fused combine's saved launch
// outweighs the chunked apply's faster streaming
constexpr int kMaxFusedItems = 64;


// backward workspace: [S][N][C][2] double partials, [N][G] max |dz|,
// [N][G][2] exponents, [N][C] float4 coefficients
struct GnbLayout {
  size_t part, dzmax, scales, chan, total;
};
GnbLayout bwd_layout_of(const st_plan* p, int groups) {
  GnbLayout l{};
  const size_t S = p->shards.size(), N = (size_t)p->batch, G = (size_t)groups, C = (size_t)p->channels;
  size_t off = 0;
  l.part = off;   off = align256(off + S * N * C * 2 * sizeof(double));
  l.dzmax = off;  off = align256(off + N * G * sizeof(uint32_t));
  l.scales = off; off = align256(off + N * G * 2 * sizeof(int32_t));
  l.chan = off;   off = align256(off + N * C * sizeof(float4));
  l.total = off;
  return l;
}

template <int VW, bool FIXED>
st_status launch_backward(GnbArgs& b, bool need_max, int mode, hipStream_t st) {
  GnArgs& a = b.g;
  const int grid = grid_of(a);
  if (need_max) {
    GnArgs m = a;                         // max |dz| with the forward's max kernel
    for (int s = 0; s < m.nshards; ++s) m.sh[s].y = m.sh[s].dz;
    m.ymax = const_cast<uint32_t*>(b.dzmax);
    hipLaunchKernelGGL((gn_max<VW, FIXED>), dim3(grid), dim3(kNT), (size_t)a.channels * 4, st, m);
    st_status s = launch_check("st_groupnorm_backward: max launch");
    if (s != ST_OK) return s;
  }
  hipLaunchKernelGGL((gnb_stats<VW, FIXED>), dim3(grid), dim3(kNT), (size_t)a.channels * 40, st, b);
  st_status s = launch_check("st_groupnorm_backward: stats launch");
  if (s != ST_OK) return s;
  const int nthreads = std::max(a.batch * a.groups, a.channels);
  hipLaunchKernelGGL(gnb_combine, dim3((nthreads + 63) / 64), dim3(64), 0, st, b);
  s = launch_check("st_groupnorm_backward: combine launch");
  if (s != ST_OK) return s;
  // the chunked apply: coefficients within LDS, chunks within a grid, and
  // for a padded dy every vector index of a batch item below 2^31
  bool stream = stream_fits(a);
  if (mode != kDyLikeY)
    for (int i = 0; i < a.nshards; ++i) stream = stream && a.sh[i].vecs_per_n < ((int64_t)1 << 31);
  if (stream) {
    const size_t shmem = (size_t)a.channels * sizeof(float4);
    if (stream_tpb(a.channels) == kStreamSmall) {
      constexpr int T = kStreamSmall;
      const dim3 grid(a.total_items * (kNT * kIter / T));
      if (mode == kDyPaddedBf16) hipLaunchKernelGGL((gnb_apply_stream<VW, kDyPaddedBf16, T>), grid, dim3(T), shmem, st, b);
      else if (mode == kDyPaddedF32) hipLaunchKernelGGL((gnb_apply_stream<VW, kDyPaddedF32, T>), grid, dim3(T), shmem, st, b);
      else hipLaunchKernelGGL((gnb_apply_stream<VW, kDyLikeY, T>), grid, dim3(T), shmem, st, b);
    } else {
      constexpr int T = kStreamLarge;
      const dim3 grid(a.total_items * (kNT * kIter / T));
      if (mode == kDyPaddedBf16) hipLaunchKernelGGL((gnb_apply_stream<VW, kDyPaddedBf16, T>), grid, dim3(T), shmem, st, b);
      else if (mode == kDyPaddedF32) hipLaunchKernelGGL((gnb_apply_stream<VW, kDyPaddedF32, T>), grid, dim3(T), shmem, st, b);
      else hipLaunchKernelGGL((gnb_apply_stream<VW, kDyLikeY, T>), grid, dim3(T), shmem, st, b);
    }
    return launch_check("st_groupnorm_backward: apply launch");
  }
  const int agrid = std::max(1, std::min((kIter / kPart) * a.total_items, device_cus() * 16));
  if (mode == kDyPaddedBf16) hipLaunchKernelGGL((gnb_apply<VW, FIXED, kDyPaddedBf16>), dim3(agrid), dim3(kNT), 0, st, b);
  else if (mode == kDyPaddedF32) hipLaunchKernelGGL((gnb_apply<VW, FIXED, kDyPaddedF32>), dim3(agrid), dim3(kNT), 0, st, b);
  else hipLaunchKernelGGL((gnb_apply<VW, FIXED, kDyLikeY>), dim3(agrid), dim3(kNT), 0, st, b);
  return launch_check("st_groupnorm_backward: apply launch");
}
}  // namespace

// Scratch of st_groupnorm_sharded_noalloc: the whole GroupNorm workspace
// (per-shard partials, max |y|, statistics, exponents, per-channel
// coefficients) in a static device array, so that entry point allocates
// nothing.  Every GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = ST_GN_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes % 256 == 0, "whole 256-byte blocks");
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};   // device address of `scratch` per device index

st_status scratch_address(void** out) {
  int dev = -1;
  st_status s = hip_check(hipGetDevice(&dev), "st_groupnorm_sharded_noalloc: hipGetDevice");
  if (s != ST_OK) return s;
  if (dev < 0 || dev >= 64) return fail(ST_ERR_UNSUPPORTED, "st_groupnorm_sharded_noalloc: device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    s = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                  "st_groupnorm_sharded_noalloc: hipGetSymbolAddress(scratch)");
    if (s != ST_OK) return s;
    if (!p) return fail(ST_ERR_HIP, "st_groupnorm_sharded_noalloc: no device address for the scratch array");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return ST_OK;
}
}  // namespace
}  // namespace st

using namespace st;

extern "C" {

size_t st_groupnorm_workspace_bytes(const st_plan* y_plan, int32_t groups) {
  if (!y_plan || groups < 1) return 0;
  return layout_of(y_plan, groups).total_bytes;
}

st_status st_groupnorm_workspace_layout(const st_plan* y_plan, int32_t groups, st_gn_layout* out) {
  if (!y_plan || !out) return fail(ST_ERR_INVALID_ARG, "st_groupnorm_workspace_layout: NULL argument");
  if (groups < 1 || y_plan->channels % groups)
    return fail(ST_ERR_INVALID_ARG, "st_groupnorm_workspace_layout: groups must divide C");
  *out = layout_of(y_plan, groups);
  return ST_OK;
}

st_status st_groupnorm_partials(const st_plan* y_plan, const float* const* y_bufs,
                                const uint32_t* ymax_or_null, int32_t groups, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!y_bufs) return fail(ST_ERR_INVALID_ARG, "st_groupnorm_partials: NULL y array");
  GnArgs a;
  int vw;
  bool fixed;
  st_status s = prepare(y_plan, y_bufs, nullptr, ymax_or_null, groups, 0.f, nullptr, nullptr, workspace,
                        workspace_bytes, "st_groupnorm_partials", a, vw, fixed);
  if (s != ST_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // clear the partial sums (and the max scratch when this call computes it)
  const st_gn_layout l = layout_of(y_plan, groups);
  const int64_t words = (int64_t)(l.ymax_offset + (ymax_or_null ? 0 : (size_t)a.batch * groups * 4)) / 4;
  hipLaunchKernelGGL(gn_fill, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(workspace), words);
  s = launch_check("st_groupnorm_partials: clear launch");
  if (s != ST_OK) return s;
  const bool need_max = ymax_or_null == nullptr;
  if (vw == 4) return fixed ? launch_partials<4, true>(a, need_max, st) : launch_partials<4, false>(a, need_max, st);
  return fixed ? launch_partials<1, true>(a, need_max, st) : launch_partials<1, false>(a, need_max, st);
}

st_status st_groupnorm_combine(const st_plan* y_plan, int32_t groups, float eps, const float* gamma_or_null,
                               const float* beta_or_null, void* workspace, size_t workspace_bytes,
                               void* stream) {
  GnArgs a;
  int vw;
  bool fixed;
  st_status s = prepare(y_plan, nullptr, nullptr, nullptr, groups, eps, gamma_or_null, beta_or_null, workspace,
                        workspace_bytes, "st_groupnorm_combine", a, vw, fixed);
  if (s != ST_OK) return s;
  const int ng = a.batch * a.groups;
  hipLaunchKernelGGL(gn_combine, dim3((ng + 63) / 64), dim3(64), 0, static_cast<hipStream_t>(stream), a);
  return launch_check("st_groupnorm_combine: launch");
}

st_status st_groupnorm_apply(const st_plan* y_plan, const float* const* y_bufs, int32_t groups,
                             float* const* z_bufs, void* workspace, size_t workspace_bytes, void* stream) {
  if (!y_bufs || !z_bufs) return fail(ST_ERR_INVALID_ARG, "st_groupnorm_apply: NULL buffer array");
  GnArgs a;
  int vw;
  bool fixed;
  st_status s = prepare(y_plan, y_bufs, z_bufs, nullptr, groups, 0.f, nullptr, nullptr, workspace,
                        workspace_bytes, "st_groupnorm_apply", a, vw, fixed);
  if (s != ST_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (stream_fits(a)) {
    const bool small = stream_tpb(a.channels) == kStreamSmall;
    if (vw == 4) return small ? launch_apply_stream<4, kStreamSmall>(a, st) : launch_apply_stream<4, kStreamLarge>(a, st);
    return small ? launch_apply_stream<1, kStreamSmall>(a, st) : launch_apply_stream<1, kStreamLarge>(a, st);
  }
  if (vw == 4) return fixed ? launch_apply<4, true>(a, st) : launch_apply<4, false>(a, st);
  return fixed ? launch_apply<1, true>(a, st) : launch_apply<1, false>(a, st);
}

st_status st_groupnorm_combine_apply(const st_plan* y_plan, const float* const* y_bufs, int32_t groups,
                                     float eps, const float* gamma_or_null, const float* beta_or_null,
                                     float* const* z_bufs, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (!y_bufs || !z_bufs) return fail(ST_ERR_INVALID_ARG, "st_groupnorm_combine_apply: NULL buffer array");
  GnArgs a;
  int vw;
  bool fixed;
  st_status s = prepare(y_plan, y_bufs, z_bufs, nullptr, groups, eps, gamma_or_null, beta_or_null, workspace,
                        workspace_bytes, "st_groupnorm_combine_apply", a, vw, fixed);
  if (s != ST_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fixed && (int64_t)a.batch * a.groups <= kMaxFusedGroups && (a.total_items <= kMaxFusedItems || !stream_fits(a)))
    return vw == 4 ? launch_apply<4, true, true>(a, st) : launch_apply<1, true, true>(a, st);
  s = st_groupnorm_combine(y_plan, groups, eps, gamma_or_null, beta_or_null, workspace, workspace_bytes, stream);
  if (s != ST_OK) return s;
  return st_groupnorm_apply(y_plan, y_bufs, groups, z_bufs, workspace, workspace_bytes, stream);
}

st_status st_groupnorm_sharded(const st_plan* y_plan, const float* const* y_bufs,
                               const uint32_t* ymax_or_null, int32_t groups, float eps,
                               const float* gamma_or_null, const float* beta_or_null,
                               float* const* z_bufs, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!y_bufs || !z_bufs) return fail(ST_ERR_INVALID_ARG, "st_groupnorm_sharded: NULL buffer array");
  GnArgs a;
  int vw;
  bool fixed;
  // validate everything up front so a failure enqueues nothing
  st_status s = prepare(y_plan, y_bufs, z_bufs, ymax_or_null, groups, eps, gamma_or_null, beta_or_null,
                        workspace, workspace_bytes, "st_groupnorm_sharded", a, vw, fixed);
  if (s != ST_OK) return s;
  s = st_groupnorm_partials(y_plan, y_bufs, ymax_or_null, groups, workspace, workspace_bytes, stream);
  if (s != ST_OK) return s;
  return st_groupnorm_combine_apply(y_plan, y_bufs, groups, eps, gamma_or_null, beta_or_null, z_bufs, workspace,
                                    workspace_bytes, stream);
}

st_status st_groupnorm_sharded_noalloc(const st_plan* y_plan, const float* const* y_bufs,
                                       const uint32_t* ymax_or_null, int32_t groups, float eps,
                                       const float* gamma_or_null, const float* beta_or_null,
                                       float* const* z_bufs, void* stream) {
  if (!y_plan) return fail(ST_ERR_INVALID_ARG, "st_groupnorm_sharded_noalloc: NULL plan");
  if (groups < 1 || y_plan->channels % groups)
    return fail(ST_ERR_INVALID_ARG, "st_groupnorm_sharded_noalloc: groups must divide C");
  // size check first: an oversized request makes no GPU call at all
  const size_t need = layout_of(y_plan, groups).total_bytes;
  if (need > kNoAllocScratchBytes)
    return fail(ST_ERR_WORKSPACE, "st_groupnorm_sharded_noalloc: needs " + std::to_string(need) +
                                      " bytes of scratch, the static scratch holds " +
                                      std::to_string(kNoAllocScratchBytes));
  void* ws = nullptr;
  st_status s = scratch_address(&ws);
  if (s != ST_OK) return s;
  return st_groupnorm_sharded(y_plan, y_bufs, ymax_or_null, groups, eps, gamma_or_null, beta_or_null, z_bufs, ws,
                              kNoAllocScratchBytes, stream);
}

size_t st_groupnorm_backward_workspace_bytes(const st_plan* y_plan, int32_t groups) {
  if (!y_plan || groups < 1) return 0;
  return bwd_layout_of(y_plan, groups).total;
}

st_status st_groupnorm_backward(const st_plan* y_plan, const float* const* y_bufs, const float* const* dz_bufs,
                                const uint32_t* ymax_or_null, const uint32_t* dzmax_or_null, int32_t groups,
                                const float* gamma_or_null, const void* fwd_workspace,
                                size_t fwd_workspace_bytes, const st_plan* dy_plan_or_null, void* const* dy_bufs,
                                float* dgamma_or_null, float* dbeta_or_null, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const char* who = "st_groupnorm_backward";
  auto err = [&](st_status st, const char* m) { return fail(st, std::string(who) + ": " + m); };
  if (!y_bufs || !dz_bufs || !dy_bufs) return err(ST_ERR_INVALID_ARG, "NULL buffer array");
  GnbArgs b{};
  int vw;
  bool fixed;
  // validates the plan, y, gamma, ymax and the forward workspace (and dy when it has y's layout)
  st_status s = prepare(y_plan, y_bufs, dy_plan_or_null ? nullptr : reinterpret_cast<float* const*>(dy_bufs),
                        ymax_or_null, groups, 0.f, gamma_or_null, nullptr, const_cast<void*>(fwd_workspace),
                        fwd_workspace_bytes, who, b.g, vw, fixed);
  if (s != ST_OK) return s;
  int mode = kDyLikeY;
  if (dy_plan_or_null) {
    const st_plan* q = dy_plan_or_null;
    if (q->ndim != y_plan->ndim || q->batch != y_plan->batch || q->channels != y_plan->channels ||
        q->shards.size() != y_plan->shards.size())
      return err(ST_ERR_BAD_SHAPE, "dy plan differs from the y plan in ndim, batch, channels or shards");
    for (size_t i = 0; i < q->shards.size(); ++i)
      for (int ax = 0; ax < kAxes; ++ax)
        if (q->shards[i].ext[ax] != y_plan->shards[i].ext[ax] || q->shards[i].off[ax] != y_plan->shards[i].off[ax])
          return err(ST_ERR_BAD_SHAPE, "dy plan differs from the y plan in shard sizes");
    if (vw != 4 && q->dtype == ST_BF16) return err(ST_ERR_UNSUPPORTED, "bf16 dy needs C divisible by 4");
    mode = q->dtype == ST_BF16 ? kDyPaddedBf16 : kDyPaddedF32;
    const int64_t C = q->channels;
    b.fCv = fast_div((uint32_t)(C / vw));
    for (size_t i = 0; i < q->shards.size(); ++i) {
      if (!dy_bufs[i]) return err(ST_ERR_INVALID_ARG, "NULL dy buffer");
      if (!aligned16(dy_bufs[i])) return err(ST_ERR_ALIGNMENT, "dy buffers must be 16-byte aligned");
      const Shard& sd = q->shards[i];
      GnbOut& o = b.out[i];
      o.sh = sd.pad[2] * C;
      o.sd = sd.pad[1] * o.sh;
      o.sn = sd.pad[0] * o.sd;
      o.H = (int32_t)sd.ext[1];
      o.W = (int32_t)sd.ext[2];
      o.fH = fast_div((uint32_t)o.H);
      o.fW = fast_div((uint32_t)o.W);
      const int64_t origin = q->halo[0] * o.sd + q->halo[1] * o.sh + q->halo[2] * C;
      o.p = static_cast<char*>(dy_bufs[i]) + origin * q->esize;
      if (dy_bufs[i] == static_cast<const void*>(y_bufs[i]) || dy_bufs[i] == static_cast<const void*>(dz_bufs[i]))
        return err(ST_ERR_INVALID_ARG, "dy in another layout must not alias y or dz");
    }
  }
  for (size_t i = 0; i < y_plan->shards.size(); ++i) {
    if (!dz_bufs[i]) return fail(ST_ERR_INVALID_ARG, std::string(who) + ": NULL dz buffer");
    if (!aligned16(dz_bufs[i])) return fail(ST_ERR_ALIGNMENT, std::string(who) + ": dz buffers must be 16-byte aligned");
    b.g.sh[i].dz = dz_bufs[i];
  }
  if ((dzmax_or_null && (reinterpret_cast<uintptr_t>(dzmax_or_null) & 3)) ||
      (dgamma_or_null && (reinterpret_cast<uintptr_t>(dgamma_or_null) & 3)) ||
      (dbeta_or_null && (reinterpret_cast<uintptr_t>(dbeta_or_null) & 3)))
    return fail(ST_ERR_ALIGNMENT, std::string(who) + ": misaligned dzmax/dgamma/dbeta");
  const GnbLayout l = bwd_layout_of(y_plan, groups);
  if (!workspace || workspace_bytes < l.total)
    return fail(ST_ERR_WORKSPACE, std::string(who) + ": workspace missing or too small");
  if (!aligned16(workspace)) return fail(ST_ERR_ALIGNMENT, std::string(who) + ": workspace not 16-byte aligned");
  if (workspace == fwd_workspace) return fail(ST_ERR_INVALID_ARG, std::string(who) + ": workspace must not be the forward workspace");
  const st_gn_layout fl = layout_of(y_plan, groups);
  char* ws = static_cast<char*>(workspace);
  b.fstats = reinterpret_cast<const float*>(static_cast<const char*>(fwd_workspace) + fl.stats_offset);
  b.dzmax = dzmax_or_null ? dzmax_or_null : reinterpret_cast<const uint32_t*>(ws + l.dzmax);
  b.bpart = reinterpret_cast<double*>(ws + l.part);
  b.bscales = reinterpret_cast<int32_t*>(ws + l.scales);
  b.bchan = reinterpret_cast<float4*>(ws + l.chan);
  b.dgamma = dgamma_or_null;
  b.dbeta = dbeta_or_null;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // clear the partials (and the max scratch when this call computes it)
  const int64_t words = (int64_t)(l.dzmax + (dzmax_or_null ? 0 : (size_t)b.g.batch * groups * 4)) / 4;
  hipLaunchKernelGGL(gn_fill, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(workspace), words);
  s = launch_check("st_groupnorm_backward: clear launch");
  if (s != ST_OK) return s;
  const bool need_max = dzmax_or_null == nullptr;
  if (vw == 4)
    return fixed ? launch_backward<4, true>(b, need_max, mode, st) : launch_backward<4, false>(b, need_max, mode, st);
  return fixed ? launch_backward<1, true>(b, need_max, mode, st) : launch_backward<1, false>(b, need_max, mode, st);
}

}  // extern "C"
