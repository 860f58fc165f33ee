// Weight gradient of the sharded convolution.
//
// Training at native resolution needs the backward pass ("Technical summary:
// ShardTensor - domain parallelism for scientific machine learning", section 1
// "Problem statement"; section 4 "Results and benchmarks", the ViT and
// StormScope training runs).  For y[n, i, o] = sum_t sum_c w[o, c, t] *
// x[n, i + t - p, c] the weight gradient is
//     dw[o, c, t] = sum_n sum_i dy[n, i, o] * x[n, i + t - p, c],
// a contraction over every position of every shard.  Each shard reads only its
// own halo-padded x (the margins already hold the neighbours' cells and the
// zero padding), so the shards contribute independent partial sums; the
// partials are then reduced in a fixed order (the all-reduce a multi-device
// run would do, section 2 "Implementation details", "Communication").
//
// Matrix-core kernel (bf16 operands, fp32 accumulation).  Work is cut into
// output rows (n, d, h) of a shard and, along W, into chunks of 64 columns
// u = i + tx (the x column a tap reads, shifted to start at 0):
//   A[(tx, o)][u] = dy[i = u - tx][o]      (zero where i is outside the row)
//   B[(r, c)][u]  = x[row r of the taps][u - p][c]
// where r enumerates the taps off the W axis ((tz, ty) in 3D, ty in 2D).
// Then C[(tx, o)][(r, c)] = sum_u A B^T = dw[o, c, (r, tx)]: every product of
// the definition appears exactly once, and the contraction index u runs along
// memory-contiguous positions.  The operands stay in LDS in their memory
// layout (positions, then channels), filled by LDS-DMA, and the fragments,
// which need 8 consecutive positions of one channel per lane, come from
// transposing LDS reads; wgrad_tr works row by row, wgrad_grp over groups of
// rows and channel tiles (below).
//
// A workgroup owns a tile of output blocks (32 x 32, or 16 x 16 for the
// row-group kernel's 16 x 16 x 32 form) and a fixed contiguous band
// of the rows (partition p of GP), accumulating over all of them in
// registers, then stores its partial dw.  The reduction sums the GP partials
// in partition order in fp64: the result does not depend on the device, the
// launch or timing, only on the shard plan (for another plan the rows fall
// into other partitions and rounding differs within the fp32 accumulation).
//
// Other shapes and the fp32 path use a direct kernel: one thread per
// (dw element, partition), fp32 FMA in row order.
#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace st {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWgMaxShards = ST_MAX_SHARDS;

struct WgShard {
  const void* x;        // padded x shard
  const void* dy;       // dy shard (own halo)
  int64_t xs[3];        // element strides of x: d, h, w (c contiguous); batch stride xn
  int64_t xn;
  int64_t ds[3];        // element strides of dy
  int64_t dn;
  int32_t ext[3];       // interior extents (d, h, w); 2D: d = 1
  int32_t xo[3];        // x buffer coordinate of tap 0 for output 0: halo_x - p per axis
  int32_t dyo[3];       // dy buffer coordinate of output 0: halo_dy per axis
  int32_t row_begin;    // first global row index of this shard
  int32_t rows_per_n;   // ext[0] * ext[1]
};

struct WgArgs {
  int32_t nshards, batch, total_rows, parts;
  float* partial;       // [parts][Cout][Cin][taps]
  WgShard sh[kWgMaxShards];
};
static_assert(sizeof(WgArgs) <= kMaxKernargBytes, "kernel argument struct too large");

// raw buffer descriptor over [base, base + bytes) (clamped to 2^31 - 1); an
// offset at or past kWtOob reads zeros
constexpr uint32_t kWtOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wt_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ void decode_row(const WgArgs& a, int row, int& s, int& n, int& d, int& h) {
  s = 0;
  while (s + 1 < a.nshards && a.sh[s + 1].row_begin <= row) ++s;
  const int r = row - a.sh[s].row_begin;
  n = r / a.sh[s].rows_per_n;
  const int q = r - n * a.sh[s].rows_per_n;
  d = q / a.sh[s].ext[1];
  h = q - d * a.sh[s].ext[1];
}

// Partition p owns the contiguous band of rows [p * R / P, (p + 1) * R / P):
// neighbouring output rows share x rows, which a band then reads from the
// same L2.
__device__ __forceinline__ int band_begin(const WgArgs& a, int p) {
  return (int)(((int64_t)p * a.total_rows) / a.parts);
}

// --------------------------------------------------------------------------
// matrix-core kernel with natural-layout LDS tiles and transposing reads
// --------------------------------------------------------------------------
//
// The same contraction C[(tx, o)][(r, c)] = sum_u A B^T, chunk by chunk along
// W, with the operands kept in LDS as they lie in memory: the dy run of a
// chunk ([u][o], the k - 1 positions before it included, so every tap shift
// tx is an address offset) and one x run per tap row of the tile ([u][c]).
// Both are filled by LDS-DMA straight from the shard buffers (no registers,
// no ALU work; out-of-row positions read zeros through the buffer range),
// and the MFMA fragments, which need 8 consecutive positions of one channel
// per lane, come from two ds_read_b64_tr_b16 each: within a group of 16
// lanes, source lane s reads 4 consecutive channels of position k0 + s/4,
// and output lane i receives channel i of positions k0 .. k0 + 3.  A chunk is
// 64 columns of a row (a row's tail of up to 16 more joins its last chunk);
// a partition sums its rows in order, chunk by chunk and K step by K step.

template <int NDIM_, int K_, int CIN_, int COUT_, int WGM_, int WGN_, int WM_, int WN_, int TILES_N_, int LW_ = 0>
struct WtCfg {
  static constexpr int NDIM = NDIM_, K = K_, CIN = CIN_, COUT = COUT_;
  static constexpr int WGM = WGM_, WGN = WGN_, WM = WM_, WN = WN_;
  static constexpr int P = K / 2;
  static constexpr int TAPS = NDIM == 3 ? K * K * K : K * K;
  static constexpr int R = NDIM == 3 ? K * K : K;        // tap rows off the W axis
  static constexpr int MR = K * COUT, NR = R * CIN;       // rows of A and of B
  static constexpr int MB = (MR + 31) / 32, NB = (NR + 31) / 32;
  static constexpr int TM = WGM * WM, TN = WGN * WN;     // blocks per tile
  static constexpr int TILES_M = 1, TILES_N = TILES_N_;
  static constexpr int NWC = WGM * WGN;                  // waves with MFMA work
  static constexpr int NW = NWC + LW_, NT = 64 * NW;    // plus LW_ waves that only issue transfers
  static constexpr int COLS = 64;                        // chunk width along W ...
  static constexpr int CMAX = COLS + 16;                 // ... or up to 16 more: a row's last chunk takes its tail
  static constexpr int DQ = CMAX + K - 1;                // dy positions of a chunk
  static constexpr int DPITCH = COUT * 2, XPITCH = CIN * 2;
  static constexpr int RT = TN * 32 / CIN;               // tap rows of a tile
  static constexpr int D_BYTES = (DQ * DPITCH + 1023) / 1024 * 1024;
  static constexpr int XR_BYTES = CMAX * XPITCH;         // one tap row's run
  static constexpr int NJ = (D_BYTES + RT * XR_BYTES + 1023) / 1024;   // 1 KiB LDS-DMA transfers per stage
  static constexpr int JPW = (NJ + NW - 1) / NW;         // per wave; every wave issues exactly JPW
  static constexpr int STAGE = JPW * NW * 1024;          // (the padding transfers fill the stage's tail)
  static constexpr int NSTAGE = 3;                       // chunks c (read), c + 1 (landed), c + 2 (in flight)
  static constexpr int LDS = NSTAGE * STAGE;
  static_assert(TM * 32 >= MR, "one tile spans every (tx, o) row");
  static_assert(TILES_N * TN >= NB, "tiles cover the blocks");
  static_assert(COUT % 16 == 0 && CIN % 16 == 0, "16 rows of a lane group share one tap shift / tap row");
  static_assert((TN * 32) % CIN == 0, "tiles hold whole tap rows");
  static_assert(XR_BYTES % 512 == 0, "tap-row runs in whole 16-byte slots of 32 rows");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <class C>
__global__ __launch_bounds__(C::NT) void wgrad_tr(const WgArgs a) {
  __shared__ __attribute__((aligned(1024))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage2[C::STAGE];
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g2 = lane >> 5;
  const int tile = blockIdx.x % C::TILES_N;
  const int part = blockIdx.x / C::TILES_N;
  const int n0 = tile * C::TN * 32;                   // first B row of the tile
  const int r0 = n0 / C::CIN;                         // its first tap row
  const int wm = (wave % C::NWC) / C::WGN, wn = (wave % C::NWC) % C::WGN;
  const bool mma = wave < C::NWC;

  f32x16 acc[C::WM][C::WN];
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) acc[i][j] = f32x16{};

  // fragment read offsets within a stage for K step 0 (a step adds 16
  // positions): lane s of 16-lane group g reads position 8 (g >> 1) + s / 4
  // (+ 4 for the second read) at the 4 channels 16 (g & 1) + 4 (s & 3) of
  // its 32-row block
  const int g16 = lane >> 4, s16 = lane & 15;
  const int kq = 8 * (g16 >> 1) + (s16 >> 2);
  const int rq = 16 * (g16 & 1) + 4 * (s16 & 3);
  int aoff[C::WM], boff[C::WN];
#pragma unroll
  for (int i = 0; i < C::WM; ++i) {
    int mrow = (wm * C::WM + i) * 32 + rq;
    mrow = mrow < C::MR ? mrow : 0;                   // padding rows read anything: their sums are not stored
    const int tx = mrow / C::COUT, o = mrow % C::COUT;
    aoff[i] = (kq + (C::K - 1) - tx) * C::DPITCH + o * 2;
  }
#pragma unroll
  for (int j = 0; j < C::WN; ++j) {
    const int nrow = (wn * C::WN + j) * 32 + rq;       // within the tile (tap rows r0 ..)
    const int rl = nrow / C::CIN, c = nrow % C::CIN;
    boff[j] = C::D_BYTES + rl * C::XR_BYTES + kq * C::XPITCH + c * 2;
  }
  auto frags = [&](const char* st, int ks, bf16x8 (&av)[C::WM], bf16x8 (&bv)[C::WN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::WM; ++i) {
      const char* p = st + aoff[i] + ks * 16 * C::DPITCH;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)p);
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 4 * C::DPITCH));
      av[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      const char* p = st + boff[j] + ks * 16 * C::XPITCH;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)p);
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 4 * C::XPITCH));
      bv[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mfmas = [&](const bf16x8 (&av)[C::WM], const bf16x8 (&bv)[C::WN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::WM; ++i)
#pragma unroll
      for (int j = 0; j < C::WN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
  };

  // Rows advance incrementally (h, then d, n and shard) from one decode at
  // the band's start, and each row's pointers are formed by multiplication:
  // no divisions per row.
  struct TrChunk {
    int valid, row, s, n, d, h, j0, W;
    int32_t xs0, xs1;
    const char* dyrow;       // dy at (n, d, h), output column 0
    const char* xrow;        // x at tap (0, 0) of output row (n, d, h), column 0
    int64_t dy_left, x_left; // bytes from there to the end of the shard buffer
  };
  auto set_row = [&](TrChunk& c) __attribute__((always_inline)) {
    const WgShard& sh = a.sh[c.s];
    const int64_t dyo = (int64_t)c.n * sh.dn + (int64_t)(c.d + sh.dyo[0]) * sh.ds[0] +
                        (int64_t)(c.h + sh.dyo[1]) * sh.ds[1] + (int64_t)sh.dyo[2] * sh.ds[2];
    const int64_t xo = (int64_t)c.n * sh.xn + (int64_t)(c.d + sh.xo[0]) * sh.xs[0] + (int64_t)(c.h + sh.xo[1]) * sh.xs[1] +
                       (int64_t)sh.xo[2] * sh.xs[2];
    c.dyrow = static_cast<const char*>(sh.dy) + dyo * 2;
    c.xrow = static_cast<const char*>(sh.x) + xo * 2;
    c.dy_left = ((int64_t)a.batch * sh.dn - dyo) * 2;
    c.x_left = ((int64_t)a.batch * sh.xn - xo) * 2;
    c.xs0 = (int32_t)sh.xs[0];
    c.xs1 = (int32_t)sh.xs[1];
    c.W = sh.ext[2];
  };
  const int row_end = band_begin(a, part + 1);
  auto first_tr = [&]() __attribute__((always_inline)) -> TrChunk {
    TrChunk c{};
    c.row = band_begin(a, part);
    c.valid = c.row < row_end;
    if (c.valid) decode_row(a, c.row, c.s, c.n, c.d, c.h);
    c.j0 = 0;
    set_row(c);
    return c;
  };
  // a chunk is COLS columns of its row, or the rest of the row when at most
  // 16 more would remain (so no chunk holds only a row's last few columns)
  auto chunk_len = [&](const TrChunk& ch) __attribute__((always_inline)) -> int {
    const int rem = ch.W + 2 * C::P - ch.j0;
    return rem <= C::CMAX ? rem : C::COLS;
  };
  auto next_of = [&](const TrChunk& ch) __attribute__((always_inline)) -> TrChunk {
    if (!ch.valid) return ch;
    TrChunk c = ch;
    const int len = chunk_len(ch);
    if (ch.j0 + len < ch.W + 2 * C::P) {
      c.j0 += len;
      return c;
    }
    c.j0 = 0;
    c.row = ch.row + 1;
    c.valid = c.row < row_end;
    if (!c.valid) return c;
    if (++c.h == a.sh[c.s].ext[1]) {
      c.h = 0;
      if (++c.d == a.sh[c.s].ext[0]) {
        c.d = 0;
        if (++c.n == a.batch) {
          c.n = 0;
          ++c.s;
        }
      }
    }
    set_row(c);
    return c;
  };
  // One chunk into a stage by LDS-DMA.  Transfer j moves 1 KiB: lane l's 16
  // bytes are slot 64 j + l of the stage.  dy slots: position q = slot /
  // (DPITCH / 16) of the run that starts k - 1 before the chunk (its byte
  // offset in the dy row is (j0 - k + 1) DPITCH + 16 slot); x slots: tap row,
  // then position, then 8-channel octet (offset 16 rem + tap-row offset +
  // j0 XPITCH).  Out-of-row positions, tap rows past the kernel and the
  // stage's padding slots get an out-of-range offset and land as zeros.  Every
  // wave issues exactly JPW transfers (an invalid chunk's too: its
  // descriptors have no range), so a wave's count of outstanding transfers
  // per chunk is the constant JPW.  The per-lane parts are fixed per kernel.
  int tpos[C::JPW];          // dy: position in the run; x: column in the chunk (-1: padding slot)
  int tcon[C::JPW];          // dy: 16 slot; x: 16 rem
  int ttz[C::JPW], tty[C::JPW];
  {
    constexpr int DS = C::DPITCH / 16, XS = C::XPITCH / 16;
    constexpr int D_SLOTS = C::D_BYTES / 16, XR_SLOTS = C::XR_BYTES / 16;
#pragma unroll
    for (int q = 0; q < C::JPW; ++q) {
      const int j = wave + q * C::NW;
      const int slot = 64 * j + lane;
      if (slot < D_SLOTS) {
        const int pos = slot / DS;
        tpos[q] = pos < C::DQ ? pos : -1;
        tcon[q] = 16 * slot;
        ttz[q] = tty[q] = 0;
      } else {
        const int xs = slot - D_SLOTS;
        const int rl = xs / XR_SLOTS, rem = xs - rl * XR_SLOTS;
        const int r = r0 + rl;
        tpos[q] = rl < C::RT && r < C::R ? rem / XS : -1;
        tcon[q] = 16 * rem;
        ttz[q] = C::NDIM == 3 ? r / C::K : 0;
        tty[q] = C::NDIM == 3 ? r % C::K : r;
      }
    }
  }
  auto fetch = [&](char* dst, const TrChunk& ch) __attribute__((always_inline)) {
    constexpr int D_SLOTS = C::D_BYTES / 16;
    const __amdgpu_buffer_rsrc_t rd = wt_rsrc(ch.dyrow, ch.valid ? ch.dy_left : 0);
    const __amdgpu_buffer_rsrc_t rx = wt_rsrc(ch.xrow, ch.valid ? ch.x_left : 0);
    const int i0 = ch.j0 - (C::K - 1);
    const int uend = ch.W + 2 * C::P - ch.j0;       // columns of the chunk with an x cell
    const uint32_t dbase = (uint32_t)(i0 * C::DPITCH), xbase = (uint32_t)(ch.j0 * C::XPITCH);
#pragma unroll
    for (int q = 0; q < C::JPW; ++q) {
      const int j = wave + q * C::NW;
      if (j * 64 < D_SLOTS) {                         // wave-uniform: a transfer is all dy or all x
        const int i = i0 + tpos[q];
        const bool ok = tpos[q] >= 0 && i >= 0 && i < ch.W;
        const uint32_t off = ok ? dbase + (uint32_t)tcon[q] : kWtOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_ptr)(dst + j * 1024), 16, off, 0, 0, 0);
      } else {
        const bool ok = tpos[q] >= 0 && tpos[q] < uend;
        const uint32_t off =
            ok ? xbase + (uint32_t)tcon[q] + (uint32_t)((ttz[q] * ch.xs0 + tty[q] * ch.xs1) * 2) : kWtOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr)(dst + j * 1024), 16, off, 0, 0, 0);
      }
    }
  };
  constexpr int VM_NEXT = 0x0F70 | (C::JPW & 15) | ((C::JPW >> 4) << 14);   // vmcnt(JPW): the newest chunk may fly

  TrChunk c0 = first_tr();
  TrChunk c1 = next_of(c0);
  fetch(stage0, c0);
  fetch(stage1, c1);
  __builtin_amdgcn_s_waitcnt(VM_NEXT);                // chunk 0 is in LDS
  __syncthreads();
  // one chunk per phase, three phases per loop turn so that the stages
  // rotate at compile time: chunk c + 2's transfers go into the stage chunk
  // c - 1 used while chunk c computes; at the phase's end chunk c + 1 has
  // landed (vmcnt(JPW) leaves chunk c + 2 in flight) and a barrier makes it
  // visible and frees chunk c's stage
  auto phase = [&](auto PP) __attribute__((always_inline)) {
    constexpr int par = decltype(PP)::value;
    const char* const cur = par == 0 ? stage0 : par == 1 ? stage1 : stage2;
    char* const far = par == 0 ? stage2 : par == 1 ? stage0 : stage1;
    const TrChunk c2 = next_of(c1);
    fetch(far, c2);
    if (mma) {
      const int nks = (chunk_len(c0) + 15) / 16;
      bf16x8 av0[C::WM], bv0[C::WN], av1[C::WM], bv1[C::WN];
      frags(cur, 0, av0, bv0);
      frags(cur, 1, av1, bv1);                        // a chunk has at least 2 K steps unless its row is short
      mfmas(av0, bv0);
      if (nks > 2) frags(cur, 2, av0, bv0);
      if (nks > 1) mfmas(av1, bv1);
      if (nks > 2) {
        if (nks > 3) frags(cur, 3, av1, bv1);
        mfmas(av0, bv0);
        if (nks > 3) {
          if (nks > 4) frags(cur, 4, av0, bv0);
          mfmas(av1, bv1);
          if (nks > 4) mfmas(av0, bv0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(VM_NEXT);
    __syncthreads();
    c0 = c1;
    c1 = c2;
  };
  while (c0.valid) {
    phase(std::integral_constant<int, 0>{});
    if (!c0.valid) break;
    phase(std::integral_constant<int, 1>{});
    if (!c0.valid) break;
    phase(std::integral_constant<int, 2>{});
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0): no transfer outlives the kernel's LDS

  // partial dw of this partition: C[(tx, o)][(r, c)] -> [o][c][r * K + tx]
  if (!mma) return;
  float* out = a.partial + (size_t)part * C::COUT * C::CIN * C::TAPS;
#pragma unroll
  for (int i = 0; i < C::WM; ++i) {
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      const int nn = n0 + (wn * C::WN + j) * 32 + l32;
      if (nn >= C::NR) continue;
      const int r = nn / C::CIN, c = nn % C::CIN;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = (wm * C::WM + i) * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
        if (m >= C::MR) continue;
        const int tx = m / C::COUT, o = m % C::COUT;
        out[((size_t)o * C::CIN + c) * C::TAPS + r * C::K + tx] = acc[i][j][e];
      }
    }
  }
}

// --------------------------------------------------------------------------
// matrix-core kernel over row groups and channel tiles
// --------------------------------------------------------------------------
//
// wgrad_tr's operand handling (memory-layout runs in LDS by LDS-DMA,
// fragments by transposing reads), with two changes.  (1) A chunk step covers
// G consecutive output rows h0 .. h0 + G - 1 of one (shard, n, d): output row
// g reads x rows (d + tz, h0 + g + ty), so the step loads the K (G + K - 1)
// x runs (tz, h0 + t), t < G + K - 1, once for all G rows instead of K^2
// runs per row.  (2) A workgroup's tile is OT output channels x every tap
// shift (M) by CT input channels x RT tap rows (N), so layers with more
// channels than one tile holds split into channel ranges, each tile reading
// only its channels.  A partition's sums run group by group, chunk by chunk,
// row by row and K step by K step: a fixed order for a given shard plan.

// F16: v_mfma_f32_16x16x32_bf16 blocks of 16 rows and K steps of 32
// positions instead of 32 x 32 x 16 (a 16-channel k5 layer's 80 x 400 tile
// then needs no padding rows: 5 x 25 blocks, against 3 x 13 of 32 rows with
// 35% of their products on padding); chunks then take no extra tail columns.
// NSTG: LDS stages (3: the transfers of step c + 2 fly while step c computes).
template <int NDIM_, int K_, int CIN_, int COUT_, int OT_, int CT_, int G_, int COLS_, int WGM_, int WGN_, int WM_,
          int WN_, int LW_ = 0, bool F16_ = false, int NSTG_ = 2>
struct WrCfg {
  static constexpr int NDIM = NDIM_, K = K_, CIN = CIN_, COUT = COUT_;
  static constexpr int OT = OT_, CT = CT_, G = G_;
  static constexpr int WGM = WGM_, WGN = WGN_, WM = WM_, WN = WN_;
  static constexpr bool F16 = F16_;
  static constexpr int NSTG = NSTG_;
  static constexpr int BM = F16 ? 16 : 32;               // rows per MFMA block
  static constexpr int KSTEP = F16 ? 32 : 16;            // positions per K step
  static constexpr int P = K / 2;
  static constexpr int TAPS = NDIM == 3 ? K * K * K : K * K;
  static constexpr int R = NDIM == 3 ? K * K : K;        // tap rows (tz, ty)
  static constexpr int KZ = NDIM == 3 ? K : 1;           // tz values
  static constexpr int MRT = K * OT, NRT = R * CT;       // tile rows of A (tx, o) and of B (r, c)
  static constexpr int TM = WGM * WM, TN = WGN * WN;     // blocks per tile
  static constexpr int TILES_O = COUT / OT, TILES_C = CIN / CT, NTILE = TILES_O * TILES_C;
  static constexpr int NWC = WGM * WGN, NW = NWC + LW_, NT = 64 * NW;
  // 32 x 32 x 16: a row's last chunk takes up to 16 more columns
  static constexpr int COLS = COLS_, CMAX = COLS + (F16 ? 0 : 16);
  static constexpr int NKS = CMAX / KSTEP;               // K steps of the widest chunk
  static constexpr int DQ = CMAX + K - 1;                // dy positions of a chunk
  static constexpr int DPT = OT * 2, XPT = CT * 2;       // bytes per position in LDS
  static constexpr int HR = G + K - 1;                   // x rows per tz of a group
  static constexpr int D_RUN = DQ * DPT;                 // one output row's dy run
  static constexpr int X_RUN = CMAX * XPT;               // one x run
  static constexpr int D_BYTES = (G * D_RUN + 1023) / 1024 * 1024;
  static constexpr int NJ = (D_BYTES + KZ * HR * X_RUN + 1023) / 1024;
  static constexpr int JPW = (NJ + NW - 1) / NW;         // transfers per wave, every wave the same
  static constexpr int STAGE = JPW * NW * 1024;
  static constexpr int LDS = NSTG * STAGE;
  static_assert(NSTG == 2 || NSTG == 3, "two or three stages");
  static_assert(CMAX % KSTEP == 0, "whole K steps per chunk");
  static_assert(OT % 16 == 0 && CT % 16 == 0, "a 16-row block never straddles a tap shift or tap row");
  static_assert(TM * BM >= MRT && TN * BM >= NRT, "one tile of blocks spans the tile's rows");
  static_assert(COUT % OT == 0 && CIN % CT == 0 && OT % 16 == 0 && CT % 16 == 0,
                "channel tiles in whole 16-channel groups (one lane group reads one tap shift / tap row)");
  static_assert(DPT % 16 == 0 && XPT % 16 == 0 && D_RUN % 16 == 0, "16-byte slots");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <class C>
__global__ __launch_bounds__(C::NT) void wgrad_grp(const WgArgs a) {
  __shared__ __attribute__((aligned(1024))) char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[C::STAGE];
  __shared__ __attribute__((aligned(16))) char stage2[C::NSTG == 3 ? C::STAGE : 16];
  using acc_t = typename std::conditional<C::F16, f32x4, f32x16>::type;
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g2 = lane >> 5;
  const int tile = blockIdx.x % C::NTILE;
  const int part = blockIdx.x / C::NTILE;
  const int o0 = (tile / C::TILES_C) * C::OT;         // the tile's output channels
  const int c0 = (tile % C::TILES_C) * C::CT;         // and input channels
  const int wm = (wave % C::NWC) / C::WGN, wn = (wave % C::NWC) % C::WGN;
  const bool mma = wave < C::NWC;

  acc_t acc[C::WM][C::WN];
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) acc[i][j] = acc_t{};

  // fragment offsets for output row 0 of a group and K step 0 (a row adds
  // D_RUN / X_RUN, a K step KSTEP positions): lane s of 16-lane group q reads
  // position 8 (q >> 1) + s / 4 (+ 4 for its second read) at the 4 channels
  // 16 (q & 1) + 4 (s & 3) of its 32-row block; with 16-row blocks (F16)
  // position 8 q + s / 4 at the channels 4 (s & 3), the 16 lanes of a group
  // holding one K group of 8 positions of the block's 16 rows
  const int g16 = lane >> 4, s16 = lane & 15;
  const int kq = C::F16 ? 8 * g16 + (s16 >> 2) : 8 * (g16 >> 1) + (s16 >> 2);
  const int rq = C::F16 ? 4 * (s16 & 3) : 16 * (g16 & 1) + 4 * (s16 & 3);
  int aoff[C::WM], boff[C::WN];
#pragma unroll
  for (int i = 0; i < C::WM; ++i) {
    int mrow = (wm * C::WM + i) * C::BM + rq;
    mrow = mrow < C::MRT ? mrow : 0;                  // padding rows read anything: their sums are not stored
    const int tx = mrow / C::OT, oi = mrow % C::OT;
    aoff[i] = (kq + (C::K - 1) - tx) * C::DPT + oi * 2;
  }
#pragma unroll
  for (int j = 0; j < C::WN; ++j) {
    int nrow = (wn * C::WN + j) * C::BM + rq;
    nrow = nrow < C::NRT ? nrow : 0;
    const int r = nrow / C::CT, ci = nrow % C::CT;
    const int tz = C::NDIM == 3 ? r / C::K : 0, ty = C::NDIM == 3 ? r % C::K : r;
    boff[j] = C::D_BYTES + (tz * C::HR + ty) * C::X_RUN + kq * C::XPT + ci * 2;
  }
  auto frags = [&](const char* st, int g, int ks, bf16x8 (&av)[C::WM], bf16x8 (&bv)[C::WN])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::WM; ++i) {
      const char* p = st + aoff[i] + g * C::D_RUN + ks * C::KSTEP * C::DPT;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)p);
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 4 * C::DPT));
      av[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      const char* p = st + boff[j] + g * C::X_RUN + ks * C::KSTEP * C::XPT;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)p);
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p + 4 * C::XPT));
      bv[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mfmas = [&](const bf16x8 (&av)[C::WM], const bf16x8 (&bv)[C::WN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::WM; ++i)
#pragma unroll
      for (int j = 0; j < C::WN; ++j) {
        if constexpr (C::F16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
  };

  // A step: rows h0 .. h0 + ng - 1 (ng <= G) of one (shard, n, d) in the band,
  // columns [j0, j0 + len) of them.  Rows advance incrementally from one
  // decode at the band's start.
  struct Step {
    int valid, row, ng, s, n, d, h, j0, W;
    int32_t xs0, xs1;
    const char* dyrow;       // dy at (n, d, h), output column 0
    const char* xrow;        // x at tap (0, 0) of output row (n, d, h), column 0
    int64_t dy_left, x_left; // bytes from there to the end of the shard buffer
  };
  const int row_end = band_begin(a, part + 1);
  auto set_rows = [&](Step& c) __attribute__((always_inline)) {
    const WgShard& sh = a.sh[c.s];
    c.ng = min(min(C::G, sh.ext[1] - c.h), row_end - c.row);
    const int64_t dyo = (int64_t)c.n * sh.dn + (int64_t)(c.d + sh.dyo[0]) * sh.ds[0] +
                        (int64_t)(c.h + sh.dyo[1]) * sh.ds[1] + (int64_t)sh.dyo[2] * sh.ds[2];
    const int64_t xo = (int64_t)c.n * sh.xn + (int64_t)(c.d + sh.xo[0]) * sh.xs[0] + (int64_t)(c.h + sh.xo[1]) * sh.xs[1] +
                       (int64_t)sh.xo[2] * sh.xs[2];
    c.dyrow = static_cast<const char*>(sh.dy) + dyo * 2;
    c.xrow = static_cast<const char*>(sh.x) + xo * 2;
    c.dy_left = ((int64_t)a.batch * sh.dn - dyo) * 2;
    c.x_left = ((int64_t)a.batch * sh.xn - xo) * 2;
    c.xs0 = (int32_t)sh.xs[0];
    c.xs1 = (int32_t)sh.xs[1];
    c.W = sh.ext[2];
  };
  auto first_step = [&]() __attribute__((always_inline)) -> Step {
    Step c{};
    c.row = band_begin(a, part);
    c.valid = c.row < row_end;
    if (c.valid) decode_row(a, c.row, c.s, c.n, c.d, c.h);
    c.j0 = 0;
    set_rows(c);
    return c;
  };
  auto chunk_len = [&](const Step& c) __attribute__((always_inline)) -> int {
    const int rem = c.W + 2 * C::P - c.j0;
    return rem <= C::CMAX ? rem : C::COLS;
  };
  auto next_of = [&](const Step& c) __attribute__((always_inline)) -> Step {
    if (!c.valid) return c;
    Step n = c;
    const int len = chunk_len(c);
    if (c.j0 + len < c.W + 2 * C::P) {
      n.j0 += len;
      return n;
    }
    n.j0 = 0;
    n.row = c.row + c.ng;
    n.valid = n.row < row_end;
    if (!n.valid) return n;
    n.h += c.ng;
    if (n.h == a.sh[n.s].ext[1]) {
      n.h = 0;
      if (++n.d == a.sh[n.s].ext[0]) {
        n.d = 0;
        if (++n.n == a.batch) {
          n.n = 0;
          ++n.s;
        }
      }
    }
    set_rows(n);
    return n;
  };

  // One step into a stage by LDS-DMA: the ng dy runs ([position][OT
  // channels], positions j0 - k + 1 ..), then the x runs (tz, t) for t < HR
  // ([position][CT channels], positions j0 ..).  Transfer j moves 1 KiB:
  // lane l's 16 bytes are slot 64 j + l.  Positions outside a row, rows past
  // the group or the shard and the stage's padding slots get an out-of-range
  // offset and land as zeros; every wave issues exactly JPW transfers (an
  // invalid step's too), so its count of outstanding transfers per step is
  // the constant JPW.  The per-lane parts are fixed per kernel.
  int tq[C::JPW];            // dy: output row g; x: tz * HR + t (-1: padding slot)
  int tp[C::JPW];            // position within the run
  int tc[C::JPW];            // byte offset of the slot's 8 channels within its position
  {
    constexpr int DSL = C::DPT / 16, XSL = C::XPT / 16;
    constexpr int D_SLOTS = C::D_BYTES / 16, RUN_D = C::D_RUN / 16, RUN_X = C::X_RUN / 16;
#pragma unroll
    for (int q = 0; q < C::JPW; ++q) {
      const int slot = 64 * (wave + q * C::NW) + lane;
      if (slot < D_SLOTS) {
        const int g = slot / RUN_D, rem = slot - g * RUN_D;
        tq[q] = g < C::G ? g : -1;
        tp[q] = rem / DSL;
        tc[q] = (o0 + 8 * (rem % DSL)) * 2;
      } else {
        const int xs = slot - D_SLOTS;
        const int run = xs / RUN_X, rem = xs - run * RUN_X;
        tq[q] = run < C::KZ * C::HR ? run : -1;
        tp[q] = rem / XSL;
        tc[q] = (c0 + 8 * (rem % XSL)) * 2;
      }
    }
  }
  auto fetch = [&](char* dst, const Step& c) __attribute__((always_inline)) {
    constexpr int D_SLOTS = C::D_BYTES / 16;
    const __amdgpu_buffer_rsrc_t rd = wt_rsrc(c.dyrow, c.valid ? c.dy_left : 0);
    const __amdgpu_buffer_rsrc_t rx = wt_rsrc(c.xrow, c.valid ? c.x_left : 0);
    const int i0 = c.j0 - (C::K - 1);
    const int uend = c.W + 2 * C::P - c.j0;          // chunk columns with an x cell
    // x rows: tz planes down, t rows along H; a row exists up to the padded extent
    const WgShard& sh = a.sh[c.s];
    const int hrows = (int)(sh.xs[0] / sh.xs[1]) - (c.h + sh.xo[1]);   // padded rows from tap row 0
#pragma unroll
    for (int q = 0; q < C::JPW; ++q) {
      const int j = wave + q * C::NW;
      if (j * 64 < D_SLOTS) {                         // wave-uniform: a transfer is all dy or all x
        const int i = i0 + tp[q];
        const bool ok = tq[q] >= 0 && tq[q] < c.ng && tp[q] < C::DQ && i >= 0 && i < c.W;
        const uint32_t off =
            ok ? (uint32_t)(tq[q] * (int)(sh.ds[1] * 2) + i * (C::COUT * 2) + tc[q]) : kWtOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_ptr)(dst + j * 1024), 16, off, 0, 0, 0);
      } else {
        const int tz = tq[q] / C::HR, t = tq[q] - tz * C::HR;
        const bool ok = tq[q] >= 0 && t < c.ng + C::K - 1 && t < hrows && tp[q] < uend;
        const uint32_t off =
            ok ? (uint32_t)((tz * c.xs0 + t * c.xs1 + (c.j0 + tp[q]) * C::CIN) * 2 + tc[q]) : kWtOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr)(dst + j * 1024), 16, off, 0, 0, 0);
      }
    }
  };

  // two stages: step c + 1 flies while step c computes, and a phase ends with
  // vmcnt(0); three: steps c + 1 and c + 2 fly, and vmcnt(JPW) asks only for
  // the older step's transfers at the phase's end.  The workgroup fence of
  // __syncthreads() then makes the compiler wait for every transfer in flight
  // (vmcnt(0)) all the same; a raw s_barrier behind the counted wait gave
  // the same times (within 0.5% on the three layers that use this kernel)
  constexpr int VM_END = C::NSTG == 3 ? 0x0F70 | (C::JPW & 15) | ((C::JPW >> 4) << 14) : 0x0F70;
  Step c0s = first_step();
  Step c1s = c0s;
  fetch(stage0, c0s);
  if constexpr (C::NSTG == 3) {
    c1s = next_of(c0s);
    fetch(stage1, c1s);
    __builtin_amdgcn_s_waitcnt(VM_END);               // step 0 is in LDS
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0)
  }
  __syncthreads();
  // one step per phase, NSTG phases per loop turn so that the stages rotate
  // at compile time; inside a step the (row, K step) pairs are pipelined:
  // the fragments of the next pair are read while the current pair's MFMAs run
  auto phase = [&](auto PP) __attribute__((always_inline)) {
    constexpr int par = decltype(PP)::value;
    const char* const cur = par == 0 ? stage0 : par == 1 ? stage1 : stage2;
    // the stage that receives the step NSTG - 1 ahead: the one step c - 1 used
    char* const nxt = C::NSTG == 2 ? (par ? stage0 : stage1) : (par == 0 ? stage2 : par == 1 ? stage0 : stage1);
    Step cn;
    if constexpr (C::NSTG == 3) cn = next_of(c1s);
    else cn = next_of(c0s);
    fetch(nxt, cn);
    if (mma) {
      const int nks = (chunk_len(c0s) + C::KSTEP - 1) / C::KSTEP;
      const int ng = c0s.ng;
      constexpr int NP = C::G * C::NKS;
      bf16x8 av[2][C::WM], bv[2][C::WN];
      frags(cur, 0, 0, av[0], bv[0]);
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        const int g = t / C::NKS, ks = t % C::NKS;
        const int g1 = (t + 1) / C::NKS, ks1 = (t + 1) % C::NKS;
        if (t + 1 < NP && g1 < ng && ks1 < nks) frags(cur, g1, ks1, av[(t + 1) & 1], bv[(t + 1) & 1]);
        if (g < ng && ks < nks) mfmas(av[t & 1], bv[t & 1]);
      }
    }
    __builtin_amdgcn_s_waitcnt(VM_END);               // this wave's transfers of the next step are in LDS
    __syncthreads();
    if constexpr (C::NSTG == 3) {
      c0s = c1s;
      c1s = cn;
    } else {
      c0s = cn;
    }
  };
  while (c0s.valid) {
    phase(std::integral_constant<int, 0>{});
    if (!c0s.valid) break;
    phase(std::integral_constant<int, 1>{});
    if constexpr (C::NSTG == 3) {
      if (!c0s.valid) break;
      phase(std::integral_constant<int, 2>{});
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // partial dw of this partition: C[(tx, o)][(r, c)] -> [o][c][r * K + tx]
  if (!mma) return;
  float* out = a.partial + (size_t)part * C::COUT * C::CIN * C::TAPS;
#pragma unroll
  for (int i = 0; i < C::WM; ++i) {
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      // accumulator e of a lane: column lane % BM, row 8 (e / 4) + 4 (lane / 32)
      // + e % 4 of a 32-row block, or 4 (lane / 16) + e of a 16-row one
      const int nn = (wn * C::WN + j) * C::BM + (C::F16 ? s16 : l32);
      if (nn >= C::NRT) continue;
      const int r = nn / C::CT, c = c0 + nn % C::CT;
#pragma unroll
      for (int e = 0; e < (C::F16 ? 4 : 16); ++e) {
        const int m = (wm * C::WM + i) * C::BM + (C::F16 ? 4 * g16 + e : 8 * (e >> 2) + 4 * g2 + (e & 3));
        if (m >= C::MRT) continue;
        const int tx = m / C::OT, o = o0 + m % C::OT;
        out[((size_t)o * C::CIN + c) * C::TAPS + r * C::K + tx] = acc[i][j][e];
      }
    }
  }
}

// --------------------------------------------------------------------------
// direct kernel (fp32, and bf16 shapes without a matrix-core instance)
// --------------------------------------------------------------------------

template <typename T> __device__ __forceinline__ float ld(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

template <typename T>
__global__ __launch_bounds__(256) void wgrad_direct(const WgArgs a, int ndim, int k, int cin, int cout) {
  const int64_t taps = ndim == 3 ? (int64_t)k * k * k : (int64_t)k * k;
  const int64_t elems = (int64_t)cout * cin * taps;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int part = blockIdx.y;
  if (e >= elems) return;
  const int t = (int)(e % taps);
  const int c = (int)((e / taps) % cin);
  const int o = (int)(e / (taps * cin));
  const int tx = t % k, ty = (t / k) % k, tz = ndim == 3 ? t / (k * k) : 0;
  float acc = 0.f;
  for (int row = part; row < a.total_rows; row += a.parts) {
    int s, n, d, h;
    decode_row(a, row, s, n, d, h);
    const WgShard& sh = a.sh[s];
    const T* dyr = static_cast<const T*>(sh.dy) + (int64_t)n * sh.dn + (int64_t)(d + sh.dyo[0]) * sh.ds[0] +
                   (int64_t)(h + sh.dyo[1]) * sh.ds[1] + (int64_t)sh.dyo[2] * sh.ds[2] + o;
    const T* xr = static_cast<const T*>(sh.x) + (int64_t)n * sh.xn + (int64_t)(d + tz + sh.xo[0]) * sh.xs[0] +
                  (int64_t)(h + ty + sh.xo[1]) * sh.xs[1] + (int64_t)(tx + sh.xo[2]) * sh.xs[2] + c;
    for (int i = 0; i < sh.ext[2]; ++i) acc = fmaf(ld(dyr, (int64_t)i * sh.ds[2]), ld(xr, (int64_t)i * sh.xs[2]), acc);
  }
  a.partial[(size_t)part * elems + e] = acc;
}

__global__ void wgrad_reduce(const float* __restrict__ partial, int parts, int64_t elems, float* __restrict__ dw) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= elems) return;
  // 8 independent loads in flight, then added in partition order
  double t = 0.0;
  for (int g0 = 0; g0 < parts; g0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = g0 + k < parts ? partial[(size_t)(g0 + k) * elems + e] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (g0 + k < parts) t += (double)v[k];
  }
  dw[e] = (float)t;
}

// --------------------------------------------------------------------------
// instances and launch
// --------------------------------------------------------------------------

// Instances.  The image 64->64 layer runs the row-by-row kernel (wgrad_tr:
// 64 to 80 column chunks, three stages); the others run row groups
// (wgrad_grp) on 16 x 16 x 32 blocks with three stages: the 16-channel k5
// layer's 80 x 400 tile needs no padding rows then (5 x 25 blocks of 16
// against 3 x 13 of 32, 35% of whose products were padding), and the 256^3
// and 256-channel layers gain from the third stage.  Same-box A/B against
// the previous instances (wgrad_tr for the 256^3 layer, 32 x 32 x 16 row
// groups with two stages for the other two): 256^3 1.75 -> 1.67 ms, 512^3 k5
// 14.4 -> 10.7 ms, 256-channel grid 3.89 -> 2.88 ms; the image layer on
// 16 x 16 x 32 row groups took 0.63 ms against wgrad_tr's 0.53.
using WtImg64 = WtCfg<2, 3, 64, 64, 2, 2, 3, 3, 1>;                     // 6 x 6 blocks, 2 x 2 waves of 3 x 3
using WrVol32F = WrCfg<3, 3, 32, 32, 32, 32, 4, 32, 2, 2, 3, 9, 0, true, 3>;       // 6 x 18 blocks of 16, 2 x 2 waves of 3 x 9
using WrVol16k5F = WrCfg<3, 5, 16, 16, 16, 16, 4, 32, 1, 4, 5, 7, 0, true, 3>;     // 5 x 25 blocks of 16, 1 x 4 waves
using WrImg256F = WrCfg<2, 3, 256, 256, 64, 64, 4, 32, 2, 2, 6, 6, 0, true, 3>;    // 4 x 4 tiles of 12 x 12 blocks

constexpr int kPartitions = 256;   // partial sums (workgroups per tile set): one per CU

struct WgInstance {
  int ndim, cin, cout, k;
  int parts;                       // partitions
  int ntile;
  int lds;
  int nt;
  void (*kernel)(WgArgs);
};


template <class C>
WgInstance make_instance_grp() {
  return WgInstance{C::NDIM, C::CIN, C::COUT, C::K, std::max(1, kPartitions / C::NTILE), C::NTILE, C::LDS, C::NT,
                    wgrad_grp<C>};
}

template <class C>
WgInstance make_instance_tr() {
  return WgInstance{C::NDIM, C::CIN, C::COUT, C::K, std::max(1, kPartitions / C::TILES_N), C::TILES_N, C::LDS, C::NT,
                    wgrad_tr<C>};
}

const WgInstance* find_instance(int ndim, int cin, int cout, int k) {
  static const WgInstance table[] = {make_instance_tr<WtImg64>(), make_instance_grp<WrVol32F>(),
                                     make_instance_grp<WrVol16k5F>(), make_instance_grp<WrImg256F>()};
  for (const WgInstance& w : table)
    if (w.ndim == ndim && w.cin == cin && w.cout == cout && w.k == k) return &w;
  return nullptr;
}

constexpr int kDirectParts = 64;

int parts_of(const st_plan* x_plan, int cout, int k) {
  const WgInstance* w = x_plan->dtype == ST_BF16
                            ? find_instance(x_plan->ndim, (int)x_plan->channels, cout, k) : nullptr;
  return w ? w->parts : kDirectParts;
}

int64_t wgrad_elems(const st_plan* x_plan, int cout, int k) {
  int64_t taps = 1;
  for (int i = 0; i < x_plan->ndim; ++i) taps *= k;
  return (int64_t)cout * x_plan->channels * taps;
}

}  // namespace
}  // namespace st

using namespace st;

extern "C" {

size_t st_conv_wgrad_workspace_bytes(const st_plan* x_plan, int32_t cout, int32_t ksize) {
  if (!x_plan || cout < 1 || ksize < 1 || ksize % 2 == 0) return 0;
  return (size_t)parts_of(x_plan, cout, ksize) * (size_t)wgrad_elems(x_plan, cout, ksize) * sizeof(float);
}

st_status st_conv_wgrad(const st_plan* x_plan, const void* const* x_bufs, const st_plan* dy_plan,
                        const void* const* dy_bufs, int32_t ksize, float* dweight, void* workspace,
                        size_t workspace_bytes, void* stream) {
  auto err = [](st_status s, const char* m) { return fail(s, std::string("st_conv_wgrad: ") + m); };
  if (!x_plan || !dy_plan || !x_bufs || !dy_bufs || !dweight) return err(ST_ERR_INVALID_ARG, "NULL argument");
  if (ksize < 1 || ksize % 2 == 0) return err(ST_ERR_UNSUPPORTED, "odd kernel sizes only");
  const int p = ksize / 2;
  if (dy_plan->ndim != x_plan->ndim || dy_plan->batch != x_plan->batch || dy_plan->dtype != x_plan->dtype)
    return err(ST_ERR_BAD_SHAPE, "x and dy plans differ in ndim, batch or dtype");
  if (dy_plan->shards.size() != x_plan->shards.size()) return err(ST_ERR_BAD_SHAPE, "x and dy plans differ in shards");
  for (size_t s = 0; s < x_plan->shards.size(); ++s)
    for (int ax = 0; ax < kAxes; ++ax)
      if (x_plan->shards[s].ext[ax] != dy_plan->shards[s].ext[ax] || x_plan->shards[s].off[ax] != dy_plan->shards[s].off[ax])
        return err(ST_ERR_BAD_SHAPE, "x and dy plans differ in shard sizes");
  for (int a = 0; a < x_plan->ndim; ++a)
    if (x_plan->halo[axis_of(x_plan, a)] < p) return err(ST_ERR_BAD_SHAPE, "x halo smaller than ksize/2");
  const int cin = (int)x_plan->channels, cout = (int)dy_plan->channels;
  const int64_t elems = wgrad_elems(x_plan, cout, ksize);
  if (elems > INT32_MAX) return err(ST_ERR_UNSUPPORTED, "weight too large");
  const WgInstance* inst = x_plan->dtype == ST_BF16 ? find_instance(x_plan->ndim, cin, cout, ksize) : nullptr;
  const int parts = inst ? inst->parts : kDirectParts;
  const size_t need = (size_t)parts * (size_t)elems * sizeof(float);
  if (!workspace || workspace_bytes < need) return err(ST_ERR_WORKSPACE, "workspace missing or too small");
  if (!aligned16(workspace) || !aligned16(dweight)) return err(ST_ERR_ALIGNMENT, "workspace and dweight must be 16-byte aligned");
  WgArgs a{};
  a.nshards = (int)x_plan->shards.size();
  a.batch = (int)x_plan->batch;
  a.parts = parts;
  a.partial = static_cast<float*>(workspace);
  int64_t rows = 0;
  for (size_t s = 0; s < x_plan->shards.size(); ++s) {
    if (!x_bufs[s] || !dy_bufs[s]) return err(ST_ERR_INVALID_ARG, "NULL shard buffer");
    if (!aligned16(x_bufs[s]) || !aligned16(dy_bufs[s])) return err(ST_ERR_ALIGNMENT, "shard buffers must be 16-byte aligned");
    const Shard& xs = x_plan->shards[s];
    const Shard& ds = dy_plan->shards[s];
    WgShard& w = a.sh[s];
    w.x = x_bufs[s];
    w.dy = dy_bufs[s];
    w.xs[2] = cin;
    w.xs[1] = xs.pad[2] * cin;
    w.xs[0] = xs.pad[1] * w.xs[1];
    w.xn = xs.pad[0] * w.xs[0];
    w.ds[2] = cout;
    w.ds[1] = ds.pad[2] * cout;
    w.ds[0] = ds.pad[1] * w.ds[1];
    w.dn = ds.pad[0] * w.ds[0];
    for (int ax = 0; ax < kAxes; ++ax) {
      w.ext[ax] = (int32_t)xs.ext[ax];
      // a 2D plan's leading axis has extent 1 and halo 0: its tap offset is 0
      const bool spatial_ax = ax >= kAxes - x_plan->ndim;
      w.xo[ax] = spatial_ax ? x_plan->halo[ax] - p : 0;
      w.dyo[ax] = dy_plan->halo[ax];
    }
    w.rows_per_n = (int32_t)(xs.ext[0] * xs.ext[1]);
    w.row_begin = (int32_t)rows;
    rows += (int64_t)a.batch * w.rows_per_n;
    if (rows > INT32_MAX) return err(ST_ERR_UNSUPPORTED, "volume too large");
  }
  a.total_rows = (int)rows;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (inst) {
    const int grid = inst->ntile * parts;
    hipLaunchKernelGGL(inst->kernel, dim3(grid), dim3(inst->nt), 0, st, a);
  } else if (x_plan->dtype == ST_F32) {
    hipLaunchKernelGGL(wgrad_direct<float>, dim3((unsigned)((elems + 255) / 256), parts), dim3(256), 0, st, a,
                       x_plan->ndim, ksize, cin, cout);
  } else {
    hipLaunchKernelGGL(wgrad_direct<uint16_t>, dim3((unsigned)((elems + 255) / 256), parts), dim3(256), 0, st, a,
                       x_plan->ndim, ksize, cin, cout);
  }
  st_status s = launch_check("st_conv_wgrad: launch");
  if (s != ST_OK) return s;
  hipLaunchKernelGGL(wgrad_reduce, dim3((unsigned)((elems + 63) / 64)), dim3(64), 0, st,
                     static_cast<const float*>(workspace), parts, elems, dweight);
  return launch_check("st_conv_wgrad: reduce launch");
}

}  // extern "C"
