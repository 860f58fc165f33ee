// Halo pack / unpack: the on-device form of the halo exchange.
//
// "Technical summary: ShardTensor - domain parallelism for scientific machine
// learning", section 2, "Implementation details", "Communication": the cells
// next to a chunk boundary are fetched from the adjacent chunk so that a
// convolution over the chunk sees the same neighbourhood as the unsharded
// one.  With every shard in HBM the exchange is two bit-exact copies:
// interior boxes -> contiguous message (pack), message -> neighbour margins
// (unpack, plus zeros on the global faces).
//
// One launch covers every box.  Each box is a set of rows of contiguous
// words (a W-run of cells times C channels); a block copies 1024 consecutive
// words of one box, so loads and stores are unit-stride across the wave.
// The kernels are HBM-bound: every payload byte is read once and written
// once.
#include "internal.h"

namespace st {
namespace {

struct ShardPtrs {
  char* p[ST_MAX_SHARDS];
};

template <int VEC> struct Word;
template <> struct Word<16> { using T = uint4; };
template <> struct Word<8> { using T = uint2; };
template <> struct Word<4> { using T = uint32_t; };
template <> struct Word<2> { using T = uint16_t; };

__device__ __forceinline__ int find_box(const HaloDesc* d, int n, int64_t block) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (d[mid].block_begin <= block) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// PACK: message <- sender interior.  !PACK: receiver margin <- message (or 0).
template <int VEC, bool PACK>
__global__ __launch_bounds__(kHaloThreads) void halo_copy(const HaloDesc* __restrict__ descs,
                                                           int ndesc, ShardPtrs bufs,
                                                           char* __restrict__ msg) {
  using W = typename Word<VEC>::T;
  const int64_t block = blockIdx.x;
  const int bi = find_box(descs, ndesc, block);
  const HaloDesc d = descs[bi];
  const int64_t first = (block - d.block_begin) * kHaloWordsPerBlock;
#pragma unroll
  for (int i = 0; i < kHaloWordsPerThread; ++i) {
    const int64_t u = first + i * kHaloThreads + threadIdx.x;
    if (u >= d.units) break;
    const uint32_t uu = (uint32_t)u;
    const uint32_t row = uu / (uint32_t)d.upr;
    const uint32_t col = uu - row * (uint32_t)d.upr;
    const uint32_t n = row / (uint32_t)d.rows_dh;
    const uint32_t r = row - n * (uint32_t)d.rows_dh;
    const uint32_t dd = r / (uint32_t)d.rows_h;
    const uint32_t hh = r - dd * (uint32_t)d.rows_h;
    if (PACK) {
      const W* src = reinterpret_cast<const W*>(bufs.p[d.src]);
      const int64_t s = d.src_base + n * d.src_sn + dd * d.src_sd + hh * d.src_sh + col;
      reinterpret_cast<W*>(msg)[d.msg_base + u] = src[s];
    } else {
      W* dst = reinterpret_cast<W*>(bufs.p[d.dst]);
      const int64_t t = d.dst_base + n * d.dst_sn + dd * d.dst_sd + hh * d.dst_sh + col;
      W v;
      if (d.src >= 0) v = reinterpret_cast<const W*>(msg)[d.msg_base + u];
      else v = W{};
      dst[t] = v;
    }
  }
}

template <bool PACK>
void launch(int vec, int64_t blocks, const HaloDesc* descs, int ndesc, const ShardPtrs& bufs,
            char* msg, hipStream_t stream) {
  const dim3 grid((unsigned)blocks), block(kHaloThreads);
  switch (vec) {
    case 16: hipLaunchKernelGGL((halo_copy<16, PACK>), grid, block, 0, stream, descs, ndesc, bufs, msg); break;
    case 8: hipLaunchKernelGGL((halo_copy<8, PACK>), grid, block, 0, stream, descs, ndesc, bufs, msg); break;
    case 4: hipLaunchKernelGGL((halo_copy<4, PACK>), grid, block, 0, stream, descs, ndesc, bufs, msg); break;
    default: hipLaunchKernelGGL((halo_copy<2, PACK>), grid, block, 0, stream, descs, ndesc, bufs, msg); break;
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
  launch<true>(plan->vec, plan->blocks_real, plan->d_descs, (int)plan->n_real, bufs,
               static_cast<char*>(msg), st);
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
  launch<false>(plan->vec, blocks, plan->d_descs, (int)nbox, bufs,
                const_cast<char*>(static_cast<const char*>(msg)), st);
  return launch_check("st_halo_unpack: launch");
}

}  // extern "C"
