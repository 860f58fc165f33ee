// Halo pack / unpack: the on-device form of the halo exchange.
//
// "Technical summary: ShardTensor - domain parallelism for scientific machine
// learning", section 2, "Implementation details", "Communication": the cells
// next to a chunk boundary are fetched from the adjacent chunk so that a
// convolution over the chunk sees the same neighbourhood as the unsharded
// one.  With every shard in HBM the exchange is two bit-exact copies:
// interior boxes -> contiguous message (pack), message -> neighbour margins
// (unpack, plus zeros on the global faces).  When sender and receiver share
// one device the two fuse into one copy, interior -> neighbour margin, with
// no message in between (exchange): half the bytes.  Boxes read only
// interiors and write only margins, each margin cell by exactly one box, so
// the boxes of one launch never touch each other's data.
//
// One launch covers every box.  Each box is a set of rows of contiguous
// words (a W-run of cells times C channels); a block copies 512 consecutive
// words of one box, so loads and stores are unit-stride across the wave, and
// reads its box from a per-block table that the plan uploads with the
// descriptors (two dependent loads instead of a binary search).  Short blocks
// in block order keep the bytes in flight within a compact window: 2 words
// per lane copy the 512^3 k5 volume's halo 7-9% faster than 4.  The kernels
// are HBM-bound: every payload byte is read once and written once.
#include "internal.h"

namespace st {
namespace {

struct ShardPtrs {
  char* p[ST_MAX_SHARDS];
};
static_assert(sizeof(ShardPtrs) <= kMaxKernargBytes, "kernel argument struct too large");

template <int VEC> struct Word;
template <> struct Word<16> { typedef unsigned int T __attribute__((ext_vector_type(4))); };
template <> struct Word<8> { typedef unsigned int T __attribute__((ext_vector_type(2))); };
template <> struct Word<4> { using T = uint32_t; };
template <> struct Word<2> { using T = uint16_t; };

__device__ __forceinline__ uint32_t mdiv(uint32_t n, uint32_t m, int32_t p) {
  return (uint32_t)(((uint64_t)n * m) >> p);
}

enum CopyMode { kPack, kUnpack, kExchange };

// plain loads, non-temporal stores (the copies' outputs are read back only by
// a later pass): 512^3 k5 pack 82 -> 70 us, unpack 131 -> 94 us; non-temporal
// loads as well were slower (77 / 102 us)
#define HALO_LOAD(p) (*(p))
#define HALO_STORE(p, v) __builtin_nontemporal_store((v), (p))

// kPack: message <- sender interior.  kUnpack: receiver margin <- message (or
// 0).  kExchange: receiver margin <- sender interior (or 0).
template <int VEC, int MODE>
__global__ __launch_bounds__(kHaloThreads) void halo_copy(const HaloDesc* __restrict__ descs,
                                                           const int32_t* __restrict__ box_of, ShardPtrs bufs,
                                                           char* __restrict__ msg) {
  using W = typename Word<VEC>::T;
  const int64_t block = blockIdx.x;
  const HaloDesc d = descs[box_of[block]];
  const int64_t first = (block - d.block_begin) * kHaloWordsPerBlock;
#pragma unroll
  for (int i = 0; i < kHaloWordsPerThread; ++i) {
    const int64_t u = first + i * kHaloThreads + threadIdx.x;
    if (u >= d.units) break;
    const uint32_t uu = (uint32_t)u;                  // units < 2^31 (the plan checks)
    const uint32_t row = mdiv(uu, d.m_upr, d.p_upr);
    const uint32_t col = uu - row * (uint32_t)d.upr;
    const uint32_t n = mdiv(row, d.m_rdh, d.p_rdh);
    const uint32_t r = row - n * (uint32_t)d.rows_dh;
    const uint32_t dd = mdiv(r, d.m_rh, d.p_rh);
    const uint32_t hh = r - dd * (uint32_t)d.rows_h;
    if (MODE == kPack) {
      const W* src = reinterpret_cast<const W*>(bufs.p[d.src]);
      const int64_t s = d.src_base + n * d.src_sn + dd * d.src_sd + hh * d.src_sh + col;
      HALO_STORE(reinterpret_cast<W*>(msg) + d.msg_base + u, HALO_LOAD(src + s));
    } else {
      W* dst = reinterpret_cast<W*>(bufs.p[d.dst]);
      const int64_t t = d.dst_base + n * d.dst_sn + dd * d.dst_sd + hh * d.dst_sh + col;
      W v = W{};
      if (d.src >= 0) {
        if (MODE == kUnpack) {
          v = HALO_LOAD(reinterpret_cast<const W*>(msg) + d.msg_base + u);
        } else {
          const W* src = reinterpret_cast<const W*>(bufs.p[d.src]);
          v = HALO_LOAD(src + d.src_base + n * d.src_sn + dd * d.src_sd + hh * d.src_sh + col);
        }
      }
      HALO_STORE(dst + t, v);
    }
  }
}

template <int MODE>
void launch(const st_plan* plan, int64_t blocks, const ShardPtrs& bufs, char* msg, hipStream_t stream) {
  const dim3 grid((unsigned)blocks), block(kHaloThreads);
  const HaloDesc* descs = plan->d_descs;
  const int32_t* box_of = reinterpret_cast<const int32_t*>(plan->d_descs + plan->descs.size());
  switch (plan->vec) {
    case 16: hipLaunchKernelGGL((halo_copy<16, MODE>), grid, block, 0, stream, descs, box_of, bufs, msg); break;
    case 8: hipLaunchKernelGGL((halo_copy<8, MODE>), grid, block, 0, stream, descs, box_of, bufs, msg); break;
    case 4: hipLaunchKernelGGL((halo_copy<4, MODE>), grid, block, 0, stream, descs, box_of, bufs, msg); break;
    default: hipLaunchKernelGGL((halo_copy<2, MODE>), grid, block, 0, stream, descs, box_of, bufs, msg); break;
  }
}

st_status check_bufs(const st_plan* plan, const void* const* bufs, ShardPtrs& out, const char* who) {
  if (!bufs) return fail(ST_ERR_INVALID_ARG, std::string(who) + ": shard buffer array is NULL");
  for (size_t i = 0; i < plan->shards.size(); ++i) {
    if (!bufs[i]) return fail(ST_ERR_INVALID_ARG, std::string(who) + ": shard buffer is NULL");
    if (!aligned16(bufs[i])) return fail(ST_ERR_ALIGNMENT, std::string(who) + ": shard buffer not 16-byte aligned");
    out.p[i] = const_cast<char*>(static_cast<const char*>(bufs[i]));
  }
  return ST_OK;
}

}  // namespace
}  // namespace st

using namespace st;

extern "C" {

st_status st_halo_pack(st_plan* plan, const void* const* shard_bufs, void* msg, void* stream) {
  if (!plan) return fail(ST_ERR_INVALID_ARG, "st_halo_pack: NULL plan");
  ShardPtrs bufs{};
  st_status s = check_bufs(plan, shard_bufs, bufs, "st_halo_pack");
  if (s != ST_OK) return s;
  if (plan->n_real == 0) return ST_OK;
  if (!msg) return fail(ST_ERR_INVALID_ARG, "st_halo_pack: message buffer is NULL");
  if (!aligned16(msg)) return fail(ST_ERR_ALIGNMENT, "st_halo_pack: message not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = plan_device_table(plan, st);
  if (s != ST_OK) return s;
  launch<kPack>(plan, plan->blocks_real, bufs, static_cast<char*>(msg), st);
  return launch_check("st_halo_pack: launch");
}

st_status st_halo_unpack(st_plan* plan, const void* msg, void* const* shard_bufs,
                         int32_t zero_global_margins, void* stream) {
  if (!plan) return fail(ST_ERR_INVALID_ARG, "st_halo_unpack: NULL plan");
  ShardPtrs bufs{};
  st_status s = check_bufs(plan, reinterpret_cast<const void* const*>(shard_bufs), bufs, "st_halo_unpack");
  if (s != ST_OK) return s;
  const int64_t nbox = zero_global_margins ? plan->n_real + plan->n_zero : plan->n_real;
  const int64_t blocks = zero_global_margins ? plan->blocks_all : plan->blocks_real;
  if (nbox == 0) return ST_OK;
  if (plan->n_real > 0) {
    if (!msg) return fail(ST_ERR_INVALID_ARG, "st_halo_unpack: message buffer is NULL");
    if (!aligned16(msg)) return fail(ST_ERR_ALIGNMENT, "st_halo_unpack: message not 16-byte aligned");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = plan_device_table(plan, st);
  if (s != ST_OK) return s;
  launch<kUnpack>(plan, blocks, bufs, const_cast<char*>(static_cast<const char*>(msg)), st);
  return launch_check("st_halo_unpack: launch");
}

st_status st_halo_exchange(st_plan* plan, void* const* shard_bufs, int32_t zero_global_margins, void* stream) {
  if (!plan) return fail(ST_ERR_INVALID_ARG, "st_halo_exchange: NULL plan");
  ShardPtrs bufs{};
  st_status s = check_bufs(plan, reinterpret_cast<const void* const*>(shard_bufs), bufs, "st_halo_exchange");
  if (s != ST_OK) return s;
  // one launch reads some shards while writing others: their bytes must not
  // overlap
  const int64_t esz = plan->dtype == ST_F32 ? 4 : 2;
  for (size_t i = 0; i < plan->shards.size(); ++i)
    for (size_t j = i + 1; j < plan->shards.size(); ++j) {
      const char *a = bufs.p[i], *b = bufs.p[j];
      const int64_t na = plan->shards[i].elems * esz, nb = plan->shards[j].elems * esz;
      if (a < b + nb && b < a + na)
        return fail(ST_ERR_INVALID_ARG, "st_halo_exchange: shard buffers overlap");
    }
  const int64_t nbox = zero_global_margins ? plan->n_real + plan->n_zero : plan->n_real;
  const int64_t blocks = zero_global_margins ? plan->blocks_all : plan->blocks_real;
  if (nbox == 0) return ST_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = plan_device_table(plan, st);
  if (s != ST_OK) return s;
  launch<kExchange>(plan, blocks, bufs, nullptr, st);
  return launch_check("st_halo_exchange: launch");
}

}  // extern "C"
