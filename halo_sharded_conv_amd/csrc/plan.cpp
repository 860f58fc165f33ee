// Shard planner: sharding shapes, padded extents and the halo box table.
//
// "Technical summary: ShardTensor - domain parallelism for scientific machine
// learning", section 2 "Design principles" (uneven per-chunk "sharding
// shapes" along each split spatial axis) and section 2 "Implementation
// details", "Communication" (halo exchange of the cells next to a chunk
// boundary).  Host only: no GPU call happens here except the lazy upload of
// the descriptor table and its release.
#include <algorithm>
#include <cstdio>
#include <array>
#include <cstring>
#include <new>

#include "internal.h"

namespace st {

static thread_local std::string g_last_error;

st_status fail(st_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}
st_status ok() { return ST_OK; }

st_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return ST_OK;
  return fail(ST_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

st_status launch_check(const char* what) { return hip_check(hipGetLastError(), what); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int32_t pick_vec(int64_t row_bytes) {
  for (int32_t v : {16, 8, 4, 2})
    if (row_bytes % v == 0) return v;
  return 1;
}

// Directions {-1,0,1}^ndim \ {0} over the plan's real axes, lexicographic,
// expanded to internal axes (a leading 2D dummy axis gets 0).
static std::vector<std::array<int, kAxes>> directions(int ndim) {
  std::vector<std::array<int, kAxes>> out;
  int count = 1;
  for (int a = 0; a < ndim; ++a) count *= 3;
  for (int code = 0; code < count; ++code) {
    std::array<int, kAxes> d{0, 0, 0};
    int c = code;
    bool any = false;
    for (int a = ndim - 1; a >= 0; --a) {   // last axis varies fastest
      d[a + (kAxes - ndim)] = (c % 3) - 1;
      c /= 3;
    }
    for (int a = 0; a < kAxes; ++a) any |= d[a] != 0;
    if (any) out.push_back(d);
  }
  return out;
}

static int shard_index(const st_plan* p, const int g[kAxes]) {
  return (g[0] * p->nshards[1] + g[1]) * p->nshards[2] + g[2];
}

}  // namespace st

using namespace st;

extern "C" {

const char* st_version(void) { return "shardconv 0.1 (gfx950)"; }
const char* st_last_error(void) { return st::g_last_error.c_str(); }

const char* st_status_string(st_status s) {
  switch (s) {
    case ST_OK: return "ok";
    case ST_ERR_INVALID_ARG: return "invalid argument";
    case ST_ERR_BAD_SHAPE: return "bad shape";
    case ST_ERR_SHARD_TOO_SMALL: return "shard thinner than the halo";
    case ST_ERR_UNSUPPORTED: return "unsupported";
    case ST_ERR_WORKSPACE: return "workspace too small";
    case ST_ERR_HIP: return "HIP error";
    case ST_ERR_ALIGNMENT: return "misaligned pointer";
  }
  return "unknown status";
}

st_status st_plan_shards(int32_t ndim, int64_t batch, int64_t channels, const int64_t* spatial,
                         const int32_t* nshards_per_axis, const int64_t* sizes_concat,
                         const int32_t* halo_per_axis, st_dtype dtype, st_plan** out) {
  if (!out) return fail(ST_ERR_INVALID_ARG, "st_plan_shards: out is NULL");
  *out = nullptr;
  if (ndim != 2 && ndim != 3)
    return fail(ST_ERR_UNSUPPORTED, "st_plan_shards: ndim must be 2 or 3");
  if (!spatial || !nshards_per_axis || !sizes_concat || !halo_per_axis)
    return fail(ST_ERR_INVALID_ARG, "st_plan_shards: NULL array argument");
  if (dtype != ST_F32 && dtype != ST_BF16)
    return fail(ST_ERR_INVALID_ARG, "st_plan_shards: unknown dtype");
  if (batch < 1 || channels < 1)
    return fail(ST_ERR_INVALID_ARG, "st_plan_shards: batch and channels must be >= 1");

  st_plan* p = new (std::nothrow) st_plan();
  if (!p) return fail(ST_ERR_INVALID_ARG, "st_plan_shards: out of host memory");
  p->ndim = ndim;
  p->batch = batch;
  p->channels = channels;
  p->dtype = dtype;
  p->esize = dtype == ST_F32 ? 4 : 2;
  p->sizes.assign(kAxes, {});
  for (int a = 0; a < kAxes; ++a) {
    p->spatial[a] = 1;
    p->nshards[a] = 1;
    p->halo[a] = 0;
    p->sizes[a] = {1};
  }
  int64_t total_shards = 1;
  int64_t cursor = 0;
  for (int a = 0; a < ndim; ++a) {
    const int ia = a + (kAxes - ndim);
    if (spatial[a] < 1) { delete p; return fail(ST_ERR_INVALID_ARG, "st_plan_shards: spatial extent < 1"); }
    if (nshards_per_axis[a] < 1) { delete p; return fail(ST_ERR_INVALID_ARG, "st_plan_shards: shard count < 1"); }
    if (halo_per_axis[a] < 0) { delete p; return fail(ST_ERR_INVALID_ARG, "st_plan_shards: negative halo"); }
    total_shards *= nshards_per_axis[a];
    if (total_shards > ST_MAX_SHARDS) {
      delete p;
      return fail(ST_ERR_UNSUPPORTED, "st_plan_shards: more than ST_MAX_SHARDS shards");
    }
    p->spatial[ia] = spatial[a];
    p->nshards[ia] = nshards_per_axis[a];
    p->halo[ia] = halo_per_axis[a];
    p->sizes[ia].clear();
    int64_t sum = 0;
    for (int i = 0; i < nshards_per_axis[a]; ++i) {
      const int64_t s = sizes_concat[cursor++];
      if (s < 1) { delete p; return fail(ST_ERR_BAD_SHAPE, "st_plan_shards: shard size < 1"); }
      if (nshards_per_axis[a] > 1 && s < halo_per_axis[a]) {
        delete p;
        char buf[160];
        std::snprintf(buf, sizeof buf, "st_plan_shards: axis %d shard %d has size %lld < halo %d",
                      a, i, (long long)s, halo_per_axis[a]);
        return fail(ST_ERR_SHARD_TOO_SMALL, buf);
      }
      sum += s;
      p->sizes[ia].push_back(s);
    }
    if (sum != spatial[a]) {
      delete p;
      char buf[160];
      std::snprintf(buf, sizeof buf, "st_plan_shards: axis %d sizes sum to %lld, extent is %lld", a,
                    (long long)sum, (long long)spatial[a]);
      return fail(ST_ERR_BAD_SHAPE, buf);
    }
  }

  // shards, row-major over the grid
  int g[kAxes];
  for (g[0] = 0; g[0] < p->nshards[0]; ++g[0])
    for (g[1] = 0; g[1] < p->nshards[1]; ++g[1])
      for (g[2] = 0; g[2] < p->nshards[2]; ++g[2]) {
        Shard s{};
        int64_t elems = batch * channels;
        for (int a = 0; a < kAxes; ++a) {
          s.grid[a] = g[a];
          int64_t off = 0;
          for (int i = 0; i < g[a]; ++i) off += p->sizes[a][i];
          s.off[a] = off;
          s.ext[a] = p->sizes[a][g[a]];
          s.pad[a] = s.ext[a] + 2 * p->halo[a];
          elems *= s.pad[a];
        }
        s.elems = elems;
        p->shards.push_back(s);
      }

  // halo boxes: for every shard and direction, either the neighbour sends
  // (real box, message order = sending shard, then direction) or the margin
  // lies on the global face (zero box).
  const auto dirs = directions(ndim);
  std::vector<PublicBox> zero_boxes;
  const int64_t C = channels;
  const int64_t row_unit_bytes = C * p->esize;
  p->vec = pick_vec(row_unit_bytes);
  for (size_t si = 0; si < p->shards.size(); ++si) {
    const Shard& s = p->shards[si];
    for (const auto& d : dirs) {
      bool empty = false;
      for (int a = 0; a < kAxes; ++a) empty |= (d[a] != 0 && p->halo[a] == 0);
      if (empty) continue;
      // (a) the box this shard sends in direction d, if the neighbour exists
      int nb[kAxes];
      bool exists = true;
      for (int a = 0; a < kAxes; ++a) {
        nb[a] = s.grid[a] + d[a];
        exists &= nb[a] >= 0 && nb[a] < p->nshards[a];
      }
      if (exists) {
        const Shard& r = p->shards[shard_index(p, nb)];
        PublicBox b{};
        b.src = (int32_t)si;
        b.dst = shard_index(p, nb);
        for (int a = 0; a < kAxes; ++a) {
          const int64_t h = p->halo[a];
          b.dir[a] = d[a];
          if (d[a] == 1) {        // my last h cells -> neighbour's low margin
            b.src_lo[a] = s.ext[a];
            b.dst_lo[a] = 0;
            b.ext[a] = h;
          } else if (d[a] == -1) { // my first h cells -> neighbour's high margin
            b.src_lo[a] = h;
            b.dst_lo[a] = h + r.ext[a];
            b.ext[a] = h;
          } else {
            b.src_lo[a] = h;
            b.dst_lo[a] = h;
            b.ext[a] = s.ext[a];
          }
        }
        p->boxes.push_back(b);
      }
      // (b) this shard's own margin in direction d on a global face
      bool face = false;
      for (int a = 0; a < kAxes; ++a) face |= (s.grid[a] + d[a] < 0 || s.grid[a] + d[a] >= p->nshards[a]);
      if (face) {
        PublicBox z{};
        z.src = -1;
        z.dst = (int32_t)si;
        for (int a = 0; a < kAxes; ++a) {
          const int64_t h = p->halo[a];
          z.dir[a] = d[a];
          z.src_lo[a] = 0;
          if (d[a] == -1) { z.dst_lo[a] = 0; z.ext[a] = h; }
          else if (d[a] == 1) { z.dst_lo[a] = h + s.ext[a]; z.ext[a] = h; }
          else { z.dst_lo[a] = h; z.ext[a] = s.ext[a]; }
        }
        z.msg_offset = -1;
        zero_boxes.push_back(z);
      }
    }
  }
  p->n_real = (int64_t)p->boxes.size();
  p->n_zero = (int64_t)zero_boxes.size();

  // message offsets (16-byte aligned boxes) and word descriptors
  int64_t msg = 0;
  const int64_t vec = p->vec;
  for (auto& b : p->boxes) {
    msg = (msg + 15) / 16 * 16;
    b.msg_offset = msg;
    msg += batch * b.ext[0] * b.ext[1] * b.ext[2] * C * p->esize;
  }
  p->msg_bytes = msg;
  p->boxes.insert(p->boxes.end(), zero_boxes.begin(), zero_boxes.end());

  int64_t blocks = 0;
  for (size_t i = 0; i < p->boxes.size(); ++i) {
    const PublicBox& b = p->boxes[i];
    HaloDesc h{};
    const Shard& dst = p->shards[b.dst];
    const int64_t upr = b.ext[2] * C * p->esize / vec;
    const int64_t rows_dh = b.ext[0] * b.ext[1];
    h.src = b.src;
    h.dst = b.dst;
    h.rows_h = (int32_t)b.ext[1];
    h.rows_dh = (int32_t)rows_dh;
    h.upr = (int32_t)upr;
    h.units = batch * rows_dh * upr;
    if (upr > INT32_MAX || rows_dh > INT32_MAX || h.units > (int64_t)INT32_MAX) {
      delete p;
      return fail(ST_ERR_UNSUPPORTED, "st_plan_shards: halo box too large");
    }
    const int64_t wpc = C * p->esize / vec;   // words per cell (may be fractional -> vec divides row only)
    auto strides = [&](const Shard& s, int64_t& sn, int64_t& sd, int64_t& sh) {
      const int64_t row_words = s.pad[2] * C * p->esize / vec;
      sh = row_words;
      sd = row_words * s.pad[1];
      sn = sd * s.pad[0];
    };
    (void)wpc;
    strides(dst, h.dst_sn, h.dst_sd, h.dst_sh);
    h.dst_base = b.dst_lo[0] * h.dst_sd + b.dst_lo[1] * h.dst_sh + b.dst_lo[2] * C * p->esize / vec;
    if (b.src >= 0) {
      const Shard& src = p->shards[b.src];
      strides(src, h.src_sn, h.src_sd, h.src_sh);
      h.src_base = b.src_lo[0] * h.src_sd + b.src_lo[1] * h.src_sh + b.src_lo[2] * C * p->esize / vec;
      h.msg_base = b.msg_offset / vec;
    } else {
      h.src_base = h.src_sn = h.src_sd = h.src_sh = 0;
      h.msg_base = -1;
    }
    auto magic = [](int64_t d, uint32_t& m, int32_t& sh) {
      int l = 0;
      while ((1ll << l) < d) ++l;
      sh = 31 + l;
      m = (uint32_t)(((1ull << sh) + (uint64_t)d - 1) / (uint64_t)d);
    };
    magic(h.upr, h.m_upr, h.p_upr);
    magic(h.rows_dh, h.m_rdh, h.p_rdh);
    magic(h.rows_h, h.m_rh, h.p_rh);
    h.block_begin = blocks;
    blocks += (h.units + kHaloWordsPerBlock - 1) / kHaloWordsPerBlock;
    if ((int64_t)i + 1 == p->n_real) p->blocks_real = blocks;
    p->descs.push_back(h);
  }
  if (p->n_real == 0) p->blocks_real = 0;
  p->blocks_all = blocks;
  *out = p;
  return ST_OK;
}

st_status st_plan_destroy(st_plan* plan) {
  if (!plan) return fail(ST_ERR_INVALID_ARG, "st_plan_destroy: NULL plan");
  st_status s = ST_OK;
  if (plan->d_descs) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != plan->dev_id) (void)hipSetDevice(plan->dev_id);
    s = hip_check(hipFree(plan->d_descs), "st_plan_destroy: hipFree");
    if (cur >= 0 && cur != plan->dev_id) (void)hipSetDevice(cur);
  }
  delete plan;
  return s;
}

st_status st_plan_upload(st_plan* plan, void* stream) {
  if (!plan) return fail(ST_ERR_INVALID_ARG, "st_plan_upload: NULL plan");
  st_status s = plan_device_table(plan, static_cast<hipStream_t>(stream));
  if (s != ST_OK) return s;
  return hip_check(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "st_plan_upload: hipStreamSynchronize");
}

int64_t st_plan_num_shards(const st_plan* p) { return p ? (int64_t)p->shards.size() : -1; }
int64_t st_plan_msg_bytes(const st_plan* p) { return p ? p->msg_bytes : -1; }
int64_t st_plan_num_halo_boxes(const st_plan* p) { return p ? p->n_real : -1; }
int64_t st_plan_num_zero_boxes(const st_plan* p) { return p ? p->n_zero : -1; }

st_status st_plan_shard_info(const st_plan* p, int32_t shard, st_shard_info* out) {
  if (!p || !out) return fail(ST_ERR_INVALID_ARG, "st_plan_shard_info: NULL argument");
  if (shard < 0 || shard >= (int32_t)p->shards.size())
    return fail(ST_ERR_INVALID_ARG, "st_plan_shard_info: shard index out of range");
  const Shard& s = p->shards[shard];
  std::memset(out, 0, sizeof *out);
  out->index = shard;
  for (int a = 0; a < kAxes; ++a) {
    out->grid[a] = 0;
    out->offset[a] = 0;
    out->extent[a] = 1;
    out->padded[a] = 1;
  }
  for (int a = 0; a < p->ndim; ++a) {
    const int ia = axis_of(p, a);
    out->grid[a] = s.grid[ia];
    out->offset[a] = s.off[ia];
    out->extent[a] = s.ext[ia];
    out->padded[a] = s.pad[ia];
  }
  out->elems = s.elems;
  out->bytes = s.elems * p->esize;
  return ST_OK;
}

st_status st_plan_halo_box(const st_plan* p, int32_t i, st_halo_box* out) {
  if (!p || !out) return fail(ST_ERR_INVALID_ARG, "st_plan_halo_box: NULL argument");
  if (i < 0 || i >= (int32_t)p->boxes.size())
    return fail(ST_ERR_INVALID_ARG, "st_plan_halo_box: index out of range");
  const PublicBox& b = p->boxes[i];
  std::memset(out, 0, sizeof *out);
  out->src_shard = b.src;
  out->dst_shard = b.dst;
  out->msg_offset = b.msg_offset;
  for (int a = 0; a < kAxes; ++a) out->ext[a] = 1;
  for (int a = 0; a < p->ndim; ++a) {
    const int ia = axis_of(p, a);
    out->dir[a] = b.dir[ia];
    out->dst_lo[a] = b.dst_lo[ia];
    out->src_lo[a] = b.src_lo[ia];
    out->ext[a] = b.ext[ia];
  }
  return ST_OK;
}

}  // extern "C"

namespace st {

st_status plan_device_table(st_plan* p, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(p->dev_mu);
  int dev = -1;
  st_status s = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (s != ST_OK) return s;
  if (p->d_descs) {
    if (dev != p->dev_id)
      return fail(ST_ERR_INVALID_ARG, "plan's descriptor table lives on another device");
    return ST_OK;
  }
  if (p->descs.empty()) { p->dev_id = dev; return ST_OK; }
  // the first upload allocates: refuse it inside a graph capture rather than
  // record an allocation and a pageable copy into the graph
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  s = hip_check(hipStreamIsCapturing(stream, &cap), "hipStreamIsCapturing");
  if (s != ST_OK) return s;
  if (cap != hipStreamCaptureStatusNone)
    return fail(ST_ERR_UNSUPPORTED,
                "the plan's descriptor table is not on the device yet: call st_plan_upload before capturing");
  // one allocation: the descriptors, then the box of every block of a launch
  // over all boxes (a block reads its box index instead of searching)
  std::vector<char> host(p->descs.size() * sizeof(HaloDesc) + (size_t)p->blocks_all * sizeof(int32_t));
  std::memcpy(host.data(), p->descs.data(), p->descs.size() * sizeof(HaloDesc));
  int32_t* box_of = reinterpret_cast<int32_t*>(host.data() + p->descs.size() * sizeof(HaloDesc));
  for (size_t i = 0; i < p->descs.size(); ++i) {
    const int64_t end = i + 1 < p->descs.size() ? p->descs[i + 1].block_begin : p->blocks_all;
    for (int64_t b = p->descs[i].block_begin; b < end; ++b) box_of[b] = (int32_t)i;
  }
  s = hip_check(hipMalloc(&p->d_descs, host.size()), "plan descriptor table: hipMalloc");
  if (s != ST_OK) { p->d_descs = nullptr; return s; }
  s = hip_check(hipMemcpy(p->d_descs, host.data(), host.size(), hipMemcpyHostToDevice),
                "plan descriptor table: hipMemcpy");
  if (s != ST_OK) { (void)hipFree(p->d_descs); p->d_descs = nullptr; return s; }
  p->dev_id = dev;
  return ST_OK;
}

}  // namespace st
