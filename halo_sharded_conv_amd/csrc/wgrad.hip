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
// memory-contiguous positions.  Two kernels take the operands to LDS:
// wgrad_mfma (the 256-channel layer, tiled over M and N) stages them through
// registers and writes them transposed (positions contiguous, one row per
// (tx, o) or (r, c)) so that a lane's 8 consecutive K values are one 16-byte
// read, A holding dy once per tx shift; wgrad_tr (the other layers) keeps
// them in their memory layout, filled by LDS-DMA, and forms the fragments
// with transposing LDS reads (below).
//
// A workgroup owns a tile of 32x32 output blocks and a fixed contiguous band
// of the rows (partition p of GP), accumulating over all of them in
// registers, then stores its partial dw.  The reduction sums the GP partials
// in partition order in fp64: the result does not depend on the device, the
// launch or timing, only on the shard plan (for another plan the rows fall
// into other partitions and rounding differs within the fp32 accumulation).
//
// Other shapes and the fp32 path use a direct kernel: one thread per
// (dw element, partition), fp32 FMA in row order.
#include <algorithm>

#include "internal.h"

namespace st {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
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

// --------------------------------------------------------------------------
// matrix-core kernel
// --------------------------------------------------------------------------

template <int NDIM_, int K_, int CIN_, int COUT_, int WGM_, int WGN_, int WM_, int WN_, int TILES_M_, int TILES_N_,
          int LW_ = 0>
struct WgCfg {
  static constexpr int NDIM = NDIM_, K = K_, CIN = CIN_, COUT = COUT_;
  static constexpr int WGM = WGM_, WGN = WGN_, WM = WM_, WN = WN_;
  static constexpr int P = K / 2;
  static constexpr int TAPS = NDIM == 3 ? K * K * K : K * K;
  static constexpr int R = NDIM == 3 ? K * K : K;        // tap rows off the W axis
  static constexpr int MR = K * COUT, NR = R * CIN;       // rows of A and of B
  static constexpr int MB = (MR + 31) / 32, NB = (NR + 31) / 32;
  static constexpr int TM = WGM * WM, TN = WGN * WN;     // blocks per tile
  static constexpr int TILES_M = TILES_M_, TILES_N = TILES_N_;
  static constexpr int NWC = WGM * WGN;                  // waves with MFMA work
  static constexpr int NW = NWC + LW_, NT = 64 * NW;    // plus LW_ waves that only load
  static constexpr int COLS = 64;                        // chunk width along W
  static constexpr int RS = COLS * 2;                    // LDS row stride (bytes), 16-byte slots permuted
  static_assert(RS == 128, "8 slots of 16 bytes per row");
  static constexpr int LA_ROWS = (TM < MB ? TM : MB) * 32;
  static constexpr int LB_ROWS = (TN < NB ? TN : NB) * 32;
  static constexpr int LDS = (LA_ROWS + LB_ROWS) * RS;
  // loader: one wave instruction moves OG channel octets of 64 / OG columns
  static constexpr int OCT_A = LA_ROWS / 8, OCT_B = LB_ROWS / 8;
  // an octet group stays inside one tap shift (A) or one tap row (B)
  static constexpr int OG_A = COUT / 8 < 8 ? COUT / 8 : 8;
  static constexpr int OG_B = CIN / 8 < 8 ? CIN / 8 : 8;
  static constexpr int G_A = OCT_A / OG_A, G_B = OCT_B / OG_B;   // octet groups
  static constexpr int JG_A = 64 / OG_A, JG_B = 64 / OG_B;       // columns per loader instruction
  static constexpr int A_PER = OCT_A / NW, B_PER = OCT_B / NW;
  static_assert(COUT % 8 == 0 && CIN % 8 == 0, "channel octets");
  static_assert(OCT_A % NW == 0 && OCT_B % NW == 0, "loader instructions divide the waves");
  static_assert(OCT_A % OG_A == 0 && OCT_B % OG_B == 0, "octet groups");
  static_assert(COUT % (8 * OG_A) == 0 && CIN % (8 * OG_B) == 0 && (TM * 32) % (8 * OG_A) == 0 &&
                (TN * 32) % (8 * OG_B) == 0, "octet groups do not straddle taps");
  static_assert(TILES_M * TM >= MB && TILES_N * TN >= NB, "tiles cover the blocks");
};

// 16-byte slot permutation of LDS row r (8 slots of a 128-byte row)
__device__ __forceinline__ int wg_key(int r) { return ((r >> 1) ^ (r >> 3)) & 7; }

struct WgChunk {
  int row, j0;
  bool valid;
  // per row (uniform): dy at (n, d, h, column 0), x at (n, d, h) for tap
  // (0, 0) and column u = 0, the shard's x strides and row length
  const uint16_t* dyrow;
  const uint16_t* xrow;
  int32_t xs0, xs1, W;
  int64_t dy_left, x_left;   // bytes from dyrow / xrow to the end of the shard buffer
};

// Partition p owns the contiguous band of rows [p * R / P, (p + 1) * R / P):
// neighbouring output rows share x rows, which a band then reads from the
// same L2.
__device__ __forceinline__ int band_begin(const WgArgs& a, int p) {
  return (int)(((int64_t)p * a.total_rows) / a.parts);
}

__device__ __forceinline__ WgChunk first_chunk(const WgArgs& a, int row, int row_end) {
  WgChunk c{};
  c.row = row;
  c.j0 = 0;
  c.valid = row < row_end;
  int s = 0, n = 0, d = 0, h = 0;
  if (c.valid) decode_row(a, row, s, n, d, h);
  const WgShard& sh = a.sh[s];
  c.dyrow = static_cast<const uint16_t*>(sh.dy) + (int64_t)n * sh.dn + (int64_t)(d + sh.dyo[0]) * sh.ds[0] +
            (int64_t)(h + sh.dyo[1]) * sh.ds[1] + (int64_t)sh.dyo[2] * sh.ds[2];
  c.xrow = static_cast<const uint16_t*>(sh.x) + (int64_t)n * sh.xn + (int64_t)(d + sh.xo[0]) * sh.xs[0] +
           (int64_t)(h + sh.xo[1]) * sh.xs[1] + (int64_t)sh.xo[2] * sh.xs[2];
  c.xs0 = (int32_t)sh.xs[0];
  c.xs1 = (int32_t)sh.xs[1];
  c.W = sh.ext[2];
  c.dy_left = ((int64_t)a.batch * sh.dn - (c.dyrow - static_cast<const uint16_t*>(sh.dy))) * 2;
  c.x_left = ((int64_t)a.batch * sh.xn - (c.xrow - static_cast<const uint16_t*>(sh.x))) * 2;
  return c;
}

// the chunk after c: 64 columns further along the row, else the band's next row
template <int K>
__device__ __forceinline__ WgChunk next_chunk(const WgArgs& a, WgChunk c, int cols, int row_end) {
  if (!c.valid) return c;
  if (c.j0 + cols < c.W + 2 * (K / 2)) {
    c.j0 += cols;
    return c;
  }
  return first_chunk(a, c.row + 1, row_end);
}

template <class C>
__global__ __launch_bounds__(C::NT) void wgrad_mfma(const WgArgs a) {
  // two LDS stages: the MFMAs read one while the other is written (1 KiB
  // aligned: the slot permutation XORs address bits 4-6)
  __shared__ __attribute__((aligned(1024))) char stage0[C::LDS];
  __shared__ __attribute__((aligned(1024))) char stage1[C::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g2 = lane >> 5;
  const int ntile = C::TILES_M * C::TILES_N;
  const int tile = blockIdx.x % ntile;
  const int part = blockIdx.x / ntile;
  const int m0 = (tile / C::TILES_N) * C::TM * 32;        // first A row of the tile
  const int n0 = (tile % C::TILES_N) * C::TN * 32;        // first B row of the tile
  const int wm = (wave % C::NWC) / C::WGN, wn = (wave % C::NWC) % C::WGN;
  const bool mma = wave < C::NWC;                       // a loader-only wave skips the MFMAs

  f32x16 acc[C::WM][C::WN];
#pragma unroll
  for (int i = 0; i < C::WM; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) acc[i][j] = f32x16{};

  uint4 ra0[C::A_PER], rb0[C::B_PER];
  // Loader instruction k (k = wave + q * NW) of a chunk covers octet group
  // g = k % G (OG octet rows, all in one tap shift or tap row) at column group
  // jg = k / G (64 / OG columns); lane l takes octet l % OG of column l / OG,
  // so OG lanes read one contiguous run of channels.  Everything but the lane
  // terms is wave-uniform.
  auto fetch = [&](const WgChunk& ch, uint4 (&qa)[C::A_PER], uint4 (&qb)[C::B_PER]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < C::A_PER; ++q) {
      const int k = wave + q * C::NW;
      const int mb = m0 + (k % C::G_A) * (8 * C::OG_A);          // first A row of the group
      const int tx = mb / C::COUT;
      const int i = ch.j0 + (k / C::G_A) * C::JG_A - tx + lane / C::OG_A;
      const bool ok = ch.valid && mb < C::MR && (unsigned)i < (unsigned)ch.W;
      const int off = ok ? i * C::COUT + (mb % C::COUT) + 8 * (lane % C::OG_A) : 0;
      const uint4 v = *reinterpret_cast<const uint4*>(ch.dyrow + off);
      qa[q] = ok ? v : make_uint4(0, 0, 0, 0);
    }
    const int uend = ch.W + 2 * C::P;                       // columns u with an x cell
#pragma unroll
    for (int q = 0; q < C::B_PER; ++q) {
      const int k = wave + q * C::NW;
      const int nb = n0 + (k % C::G_B) * (8 * C::OG_B);          // first B row of the group
      const int r = nb / C::CIN;
      const int tz = C::NDIM == 3 ? r / C::K : 0;
      const int ty = C::NDIM == 3 ? r % C::K : r;
      const int u = ch.j0 + (k / C::G_B) * C::JG_B + lane / C::OG_B;
      const bool ok = ch.valid && nb < C::NR && u < uend;
      const int off = ok ? tz * ch.xs0 + ty * ch.xs1 + u * C::CIN + (nb % C::CIN) + 8 * (lane % C::OG_B) : 0;
      const uint4 v = *reinterpret_cast<const uint4*>(ch.xrow + off);
      qb[q] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  };
  // registers -> LDS, transposed: the 8 channels of a column go to 8 rows.
  // Row r keeps its 16-byte column slots permuted by key(r) = ((r >> 1) ^
  // (r >> 3)) & 7, so that both the 8-row column writes and the 32-row
  // fragment reads spread over the banks.  For r = 8 ro + e the key is
  // (4 ro ^ ro ^ (e >> 1)) & 7, so one base address per item serves all 8 rows.
  auto put = [&](char* base, int ro, int j, const uint4& v) __attribute__((always_inline)) {
    const int slot = ((j >> 3) ^ ro ^ (ro << 2)) & 7;
    char* p = base + ro * 8 * C::RS + (slot << 4) + (j & 7) * 2;
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      char* pe = reinterpret_cast<char*>(reinterpret_cast<uintptr_t>(p) ^ (uintptr_t)((e >> 1) << 4)) + e * C::RS;
      *reinterpret_cast<uint16_t*>(pe) = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
    }
  };
  auto store = [&](char* st, const uint4 (&qa)[C::A_PER], const uint4 (&qb)[C::B_PER]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < C::A_PER; ++q) {
      const int k = wave + q * C::NW;
      put(st, (k % C::G_A) * C::OG_A + lane % C::OG_A, (k / C::G_A) * C::JG_A + lane / C::OG_A, qa[q]);
    }
#pragma unroll
    for (int q = 0; q < C::B_PER; ++q) {
      const int k = wave + q * C::NW;
      put(st + C::LA_ROWS * C::RS, (k % C::G_B) * C::OG_B + lane % C::OG_B, (k / C::G_B) * C::JG_B + lane / C::OG_B,
          qb[q]);
    }
  };
  // fragments of K step ks (8 consecutive columns per lane: one 16-byte slot)
  auto frags = [&](const char* st, int ks, bf16x8 (&av)[C::WM], bf16x8 (&bv)[C::WN]) __attribute__((always_inline)) {
    const char* la = st;
    const char* lb = st + C::LA_ROWS * C::RS;
    const int slot = ks * 2 + g2;
#pragma unroll
    for (int i = 0; i < C::WM; ++i) {
      const int row = (wm * C::WM + i) * 32 + l32;
      av[i] = *reinterpret_cast<const bf16x8*>(la + row * C::RS + ((slot ^ wg_key(row)) << 4));
    }
#pragma unroll
    for (int j = 0; j < C::WN; ++j) {
      const int row = (wn * C::WN + j) * 32 + l32;
      bv[j] = *reinterpret_cast<const bf16x8*>(lb + row * C::RS + ((slot ^ wg_key(row)) << 4));
    }
  };
  auto mfmas = [&](const bf16x8 (&av)[C::WM], const bf16x8 (&bv)[C::WN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::WM; ++i)
#pragma unroll
      for (int j = 0; j < C::WN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
  };

  const int row_end = band_begin(a, part + 1);
  // chunks of this partition: c0 in stage0, c1 staged in registers
  WgChunk c0 = first_chunk(a, band_begin(a, part), row_end);
  WgChunk c1 = next_chunk<C::K>(a, c0, C::COLS, row_end);
  fetch(c0, ra0, rb0);
  store(stage0, ra0, rb0);
  fetch(c1, ra0, rb0);
  __syncthreads();
  // one chunk per phase; the loop body handles two so that the LDS stages
  // alternate at compile time.  In a phase: K step 0's fragments, the next
  // chunk's registers into the other stage, the chunk after that into the
  // registers, and each K step's MFMAs with the next step's fragments in
  // flight.
  auto phase = [&](auto P) __attribute__((always_inline)) {
    constexpr int par = decltype(P)::value;
    char* const cur = par ? stage1 : stage0;
    char* const nxt = par ? stage0 : stage1;
    const WgChunk c2 = next_chunk<C::K>(a, c1, C::COLS, row_end);
    const int nks = (min(C::COLS, c0.W + 2 * C::P - c0.j0) + 15) / 16;
    bf16x8 av0[C::WM], bv0[C::WN], av1[C::WM], bv1[C::WN];
    if (mma) frags(cur, 0, av0, bv0);
    if (c1.valid) store(nxt, ra0, rb0);                    // the next chunk, while this one computes
    fetch(c2, ra0, rb0);                                    // and the one after it
    if (mma) {
      if (nks > 1) frags(cur, 1, av1, bv1);
      mfmas(av0, bv0);
      if (nks > 1) {
        if (nks > 2) frags(cur, 2, av0, bv0);
        mfmas(av1, bv1);
        if (nks > 2) {
          if (nks > 3) frags(cur, 3, av1, bv1);
          mfmas(av0, bv0);
          if (nks > 3) mfmas(av1, bv1);
        }
      }
    }
    __syncthreads();
    c0 = c1;
    c1 = c2;
  };
  while (c0.valid) {
    phase(std::integral_constant<int, 0>{});
    if (!c0.valid) break;
    phase(std::integral_constant<int, 1>{});
  }

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
        const int m = m0 + (wm * C::WM + i) * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
        if (m >= C::MR) continue;
        const int tx = m / C::COUT, o = m % C::COUT;
        out[((size_t)o * C::CIN + c) * C::TAPS + r * C::K + tx] = acc[i][j][e];
      }
    }
  }
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
// and output lane i receives channel i of positions k0 .. k0 + 3.  Chunks,
// K steps and partitions are those of wgrad_mfma, so each MFMA sees the
// same operands in the same positions.

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

// image 64->64 k3: 6x6 blocks, 2x2 waves of 3x3
using WgImg64 = WgCfg<2, 3, 64, 64, 2, 2, 3, 3, 1, 1>;
// 3D 32->32 k3: 3x9 blocks, 1x3 waves of 3x3, and a fourth wave that only loads
using WgVol32 = WgCfg<3, 3, 32, 32, 1, 3, 3, 3, 1, 1, 1>;
// 3D 16->16 k5: 3x13 blocks in two tiles of 3x8, 1x4 waves of 3x2
using WgVol16k5 = WgCfg<3, 5, 16, 16, 1, 4, 3, 2, 1, 2>;
// image 256->256 k3: 24x24 blocks in 4x4 tiles of 6x6, 2x2 waves of 3x3
using WgImg256 = WgCfg<2, 3, 256, 256, 2, 2, 3, 3, 4, 4>;
// transposing-read kernel: the same tilings (one tile along M)
using WtImg64 = WtCfg<2, 3, 64, 64, 2, 2, 3, 3, 1>;
using WtVol32 = WtCfg<3, 3, 32, 32, 1, 3, 3, 3, 1, 1>;
using WtVol16k5 = WtCfg<3, 5, 16, 16, 1, 4, 3, 2, 2>;

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
WgInstance make_instance() {
  const int ntile = C::TILES_M * C::TILES_N;
  return WgInstance{C::NDIM, C::CIN, C::COUT, C::K, std::max(1, kPartitions / ntile), ntile, C::LDS, C::NT,
                    wgrad_mfma<C>};
}

template <class C>
WgInstance make_instance_tr() {
  return WgInstance{C::NDIM, C::CIN, C::COUT, C::K, std::max(1, kPartitions / C::TILES_N), C::TILES_N, C::LDS, C::NT,
                    wgrad_tr<C>};
}

const WgInstance* find_instance(int ndim, int cin, int cout, int k) {
  static const WgInstance table[] = {make_instance_tr<WtImg64>(), make_instance_tr<WtVol32>(),
                                     make_instance_tr<WtVol16k5>(), make_instance<WgImg256>()};
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
