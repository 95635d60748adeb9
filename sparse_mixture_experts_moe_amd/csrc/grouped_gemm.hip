// Grouped SwiGLU experts: for every group g (an expert) and every row r of
// that group,  hid = SiLU(a_r W_gate[g]^T) * (a_r W_up[g]^T),  y_r = hid W_down[g]^T.
//
// Source: "Zen-Max: Maximum Capability via Mixture-of-Experts Architecture",
// section "Fine-Grained Expert Architecture", expert equation
// (SiLU(x W_gate) * x W_up) W_down, weights stored transposed so that every
// operand is contiguous along its reduction axis.
//
// bf16 path (gfx950 MFMA, fp32 accumulation):
//   GEMM 1 (gate || up, fused SiLU*mul): one B tile holds 128 gate rows and
//     the 128 up rows of the same hidden columns, so each wave owns matching
//     gate and up accumulators and the epilogue writes hid directly (bf16).
//   GEMM 2 (down): y = hid W_down^T.
//   Output tiles are 256 columns wide and 256 rows high, except that the last
//   m-tile of each group runs as a 64-, 128- or 256-row tile according to the
//   rows left, so a short remainder costs a quarter or a half of a full tile.
//   Four waves form a 2 x 2 (256 rows) or 1 x 4 (64 and 128 rows) grid of
//   v_mfma_f32_32x32x16_bf16 tiles.  K advances in slices of 64 (one
//   128-byte line per row) that direct-to-LDS copies stream through a
//   two-stage A ring and a three-stage B ring (160 KB); the copies are spread
//   over the whole slice, since a compute unit accepts one about every 16
//   cycles.  Fragment reads are double-buffered in registers and interleaved
//   one-for-one with the MFMAs (see gemm_tile).
//   Tiles are ordered group-major, then in bands of four m-tiles (band,
//   n-tile, m-tile fastest).  Both GEMMs run persistent, one workgroup per
//   compute unit: the order is cut into one contiguous run per XCD, of equal
//   estimated cost, so that tiles sharing a weight or activation panel run
//   together on one XCD's L2 and every XCD stays busy to the end.
// fp32 path: a plain LDS-tiled FMA kernel, one workgroup per tile, in
// contiguous runs per XCD.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kTileMBundle = 256;  // m-tile height of the bundled order

// ---------------------------------------------------------------------------
// Bundled order of the gate/up tiles.  A group of rows = 256 m + r rows has m
// full 256-row m-tiles (a remainder r > 128 runs as one more) and, when
// 0 < r <= 128, a short last m-tile of r rows.  Short tiles would finish in a
// quarter (r <= 64) or half (r <= 128) of the time of a full one and throw the
// tiles that share an activation panel out of step, so that the panel is
// fetched again; instead the group's n-tiles go in blocks of B = 4 (or 2):
// the m x B full tiles of a block (m fastest), then one unit that runs the
// block's B short tiles one after the other, about one full tile's time.
// ---------------------------------------------------------------------------
// Estimated time of one tile of bm rows (any n-tile): 6 for 256 rows, 4 for
// 128, 3 for 64.  A short tile still copies the whole weight panel, so its
// time falls by less than its rows.  Only the balance of the XCD runs (see
// tile_table_kernel) depends on these numbers.
__host__ __device__ constexpr int tile_cost(int bm) { return bm / 64 + 2; }

struct GroupUnits {
  int mfull, bsz, units;  // full m-tiles, short tiles per bundle (0: none), work units
  int cost;               // estimated time of all of the group's units
};

__device__ __forceinline__ GroupUnits group_units(int rows, int ntn) {
  int mfull = rows / kTileMBundle, r = rows % kTileMBundle;
  if (r > kTileMBundle / 2) {
    ++mfull;
    r = 0;
  }
  // a group without full tiles has nothing to keep in step: one short tile
  // per unit, all of them in parallel
  const int bsz = r == 0 ? 0 : (mfull == 0 ? 1 : (r <= kTileMBundle / 4 ? 4 : 2));
  const int cost = mfull * ntn * tile_cost(kTileMBundle) +
                   (bsz ? ntn * tile_cost(r <= kTileMBundle / 4 ? 64 : 128) : 0);
  return GroupUnits{mfull, bsz, mfull * ntn + (bsz ? (ntn + bsz - 1) / bsz : 0), cost};
}

// Estimated time of a group's tiles in the plain order (every m-tile is 256
// rows high but the last, which runs as 64, 128 or 256 rows).
__device__ __forceinline__ int group_tile_cost(int rows, int ntn) {
  if (rows <= 0) return 0;
  const int mt = (rows + kTileMBundle - 1) / kTileMBundle;
  const int last = rows - (mt - 1) * kTileMBundle;
  const int bm = last <= 64 ? 64 : (last <= 128 ? 128 : 256);
  return ((mt - 1) * tile_cost(kTileMBundle) + tile_cost(bm)) * ntn;
}

// ---------------------------------------------------------------------------
// Split-K of the last tiles.  With a long K (the down projection) one tile
// runs long enough that a final partial round of tiles leaves most compute
// units idle.  The last n_sk = total mod ncu tiles (in tile order) are cut
// along K into S parts (2 <= S <= kSkMaxSplit, n_sk S <= kSkUnits, at least
// kSkMinSlices slices per part), which run after the whole tiles; part p of
// split tile i writes the fp32 partial sums of its 256 x 256 tile to
// workspace unit i S + p, and sk_reduce_kernel adds the parts in part order
// (a fixed order: results are deterministic) and writes the output.
// ---------------------------------------------------------------------------
constexpr int kSkUnits = 256;        // partial tiles the workspace holds
constexpr int kSkMaxSplit = 4;
constexpr int kSkMinSlices = 16;     // 64-wide K slices per part, at least

struct SkPlan {
  int n_dp, n_sk, S;  // whole tiles, split tiles, parts per split tile
};

__device__ __forceinline__ SkPlan sk_plan(int total, int ncu, int nk, bool enabled) {
  SkPlan p{total, 0, 1};
  const int rem = ncu > 0 ? total % ncu : 0;
  if (!enabled || rem == 0) return p;
  const int S = min(kSkMaxSplit, min(kSkUnits / rem, nk / kSkMinSlices));
  if (S < 2) return p;
  p.n_dp = total - rem;
  p.n_sk = rem;
  p.S = S;
  return p;
}

// ---------------------------------------------------------------------------
// Persistent launches.  The bf16 GEMMs run one workgroup per compute unit;
// workgroup b runs on XCD b mod 8 (checked with the hardware id register).
// The whole tiles (or work units) are cut into kXcds contiguous runs of about
// equal estimated cost, and the workgroups of XCD x take the units of run x
// in order from a counter: the units that an XCD runs together are
// consecutive in the order, so they share activation and weight panels in its
// L2, and hot and cold experts (costly full tiles, cheap short ones) no
// longer leave some XCDs idle while others still work.  When split-K is on
// (long tiles), the runs are equal counts of whole rounds instead; the split
// parts follow from one counter shared by all XCDs.
// Workspace (int32): mstart [G + 1] | cstart [G + 1] | runs [kXcds + 1] |
// counters [kXcds + 1], each array from a 64-entry boundary.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

__host__ __device__ constexpr int tt_pad(int n) { return (n + 63) / 64 * 64; }
__host__ __device__ constexpr int tt_cstart(int G) { return tt_pad(G + 1); }
__host__ __device__ constexpr int tt_runs(int G) { return 2 * tt_pad(G + 1); }
__host__ __device__ constexpr int tt_counters(int G) { return 2 * tt_pad(G + 1) + 64; }
__host__ __device__ constexpr int tt_entries(int G) { return 2 * tt_pad(G + 1) + 128; }

// ---------------------------------------------------------------------------
// Tile table (one workgroup): mstart[g] = sum over g' < g of ceil(rows_g' /
// BM), g = 0..G, or with `units` of the work units of the bundled order.
// With `tt` (the workspace of the persistent launches, mstart at its start):
// also the cost prefixes cstart, the XCD runs of the whole tiles (ntn n-tiles
// per m-tile; the split plan of ncu compute units and nk K slices decides
// which tiles are whole) and zeroed counters.  A cut falls inside the group
// whose cost range holds it, placed by linear interpolation of its cost.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ off, int G,
                                                          int BM, int ntn, bool units,
                                                          int32_t* __restrict__ mstart,
                                                          int32_t* __restrict__ tt, int ncu,
                                                          int nk, bool split) {
  __shared__ long long wsum[16];
  __shared__ long long carry;
  __shared__ int s_ndp, s_cdp;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int32_t* cstart = tt ? tt + tt_cstart(G) : nullptr;
  if (tid == 0) carry = 0;
  __syncthreads();
  // prefix sums of the unit counts (low 32 bits) and costs (high 32 bits)
  for (int base = 0; base < G; base += 1024) {
    const int g = base + tid;
    const int rows = g < G ? off[g + 1] - off[g] : 0;
    int v, c;
    if (units) {
      const GroupUnits gu = group_units(rows, ntn);
      v = gu.units;
      c = gu.cost;
    } else {
      v = (rows + BM - 1) / BM;
      c = tt ? group_tile_cost(rows, ntn) : 0;
    }
    const long long vc = (static_cast<long long>(c) << 32) | static_cast<unsigned>(v);
    long long incl = vc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const long long n = __shfl_up(incl, o);
      if (lane >= o) incl += n;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    long long pre = carry;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    pre += incl - vc;  // this group's exclusive prefix
    if (g < G) {
      mstart[g] = static_cast<int>(pre & 0xffffffffLL);
      if (cstart) cstart[g] = static_cast<int>(pre >> 32);
    }
    __syncthreads();
    if (tid == 1023) carry = pre + vc;
    __syncthreads();
  }
  const int total_v = static_cast<int>(carry & 0xffffffffLL);
  const int total_c = static_cast<int>(carry >> 32);
  if (tid == 0) {
    mstart[G] = total_v;
    if (cstart) cstart[G] = total_c;
  }
  if (!tt) return;
  __syncthreads();  // the prefixes above are visible to the whole workgroup
  const int per = units ? 1 : ntn;  // work items per entry of mstart
  // index of work item L -> its group, by binary search over mstart
  auto group_of = [&](int L) {
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (mstart[mid] * per <= L) lo = mid; else hi = mid;
    }
    return lo;
  };
  if (tid == 0) {
    const int n_all = total_v * per;
    const int n_dp = units ? n_all : sk_plan(n_all, ncu, nk, split).n_dp;
    int c_dp = total_c;
    if (n_dp < n_all) {  // estimated cost of the whole tiles before item n_dp
      const int g = group_of(n_dp);
      const int u0 = mstart[g] * per, nu = (mstart[g + 1] - mstart[g]) * per;
      const int cg = cstart[g + 1] - cstart[g];
      c_dp = cstart[g] + static_cast<int>(static_cast<long long>(n_dp - u0) * cg / nu);
    }
    s_ndp = n_dp;
    s_cdp = c_dp;
  }
  __syncthreads();
  int32_t* runs = tt + tt_runs(G);
  int32_t* counters = tt + tt_counters(G);
  const int n_dp = s_ndp;
  if (tid > 0 && tid < kXcds) {
    const long long target = static_cast<long long>(s_cdp) * tid / kXcds;
    int cut = n_dp;
    if (n_dp < total_v * per) {
      // split-K is on: tiles are long and n_dp is a multiple of the compute
      // units, so equal counts give every XCD the same whole rounds (a cut
      // by estimated cost could leave one XCD a round more)
      cut = static_cast<int>(static_cast<long long>(n_dp) * tid / kXcds);
    } else if (target < s_cdp) {
      // the last group whose cost range starts at or before the target
      int lo = 0, hi = G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cstart[mid] <= target) lo = mid; else hi = mid;
      }
      const int cg = cstart[lo + 1] - cstart[lo];
      const int u0 = mstart[lo] * per, nu = (mstart[lo + 1] - mstart[lo]) * per;
      cut = u0 + (cg > 0 ? static_cast<int>((target - cstart[lo]) * nu / cg) : 0);
      cut = min(cut, n_dp);
    }
    runs[tid] = cut;
  }
  if (tid == 0) {
    runs[0] = 0;
    runs[kXcds] = n_dp;
  }
  if (tid <= kXcds) counters[tid] = 0;
}

struct Tile {
  int g, m0, row_end, n0;
};

// Workgroup b of a run of n8 (a multiple of 8) runs on XCD b mod 8; this
// gives each XCD a contiguous run of logical indices.
__device__ __forceinline__ int xcd_run(int b, int n8) { return (b & 7) * (n8 >> 3) + (b >> 3); }

// A group's m-tiles go in bands of kBand: band, then n-tile, then m-tile
// fastest within the band.  The 32 tiles that one XCD runs together (a run of
// consecutive indices) then cover kBand m-tiles by 32 / kBand n-tiles of a
// tall group, so every activation and weight slice they copy has several
// readers in that XCD's L2 (with the m-tiles of a tall group fastest, each
// activation slice had one reader and came from memory every time).  The last
// band takes 1 .. kBand m-tiles.
constexpr int kBand = 4;

__device__ __forceinline__ int band_lead(int mtiles) {
  return mtiles > kBand ? ((mtiles - 1) / kBand) * kBand : 0;
}

// Logical tile L: group-major, then the banded order above.
__device__ __forceinline__ Tile tile_at(int L, const int32_t* __restrict__ off,
                                        const int32_t* __restrict__ mstart, int G, int ntn,
                                        int BM, int ncol) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mstart[mid] * ntn <= L) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int mtg = mstart[g + 1] - mstart[g];
  int local = L - mstart[g] * ntn;
  const int lead = band_lead(mtg);
  int nt, mt;
  if (local < lead * ntn) {
    const int band = local / (kBand * ntn), i = local - band * (kBand * ntn);
    nt = i / kBand;
    mt = band * kBand + (i - nt * kBand);
  } else {
    local -= lead * ntn;
    const int mtail = mtg - lead;
    nt = local / mtail;
    mt = lead + (local - nt * mtail);
  }
  Tile tile;
  tile.g = g;
  tile.m0 = off[g] + mt * BM;
  tile.row_end = off[g + 1];
  tile.n0 = nt * ncol;
  return tile;
}

// Work unit L of the bundled order: a full tile (count = 0) or a bundle of
// `count` short tiles of n-tiles nt0 .. nt0 + count - 1.
struct Unit {
  int g, m0, row_end, nt0, count;
};

__device__ __forceinline__ Unit unit_at(int L, const int32_t* __restrict__ off,
                                        const int32_t* __restrict__ ustart, int G, int ntn) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ustart[mid] <= L) lo = mid; else hi = mid;
  }
  const int g = lo;
  int local = L - ustart[g];
  const GroupUnits gu = group_units(off[g + 1] - off[g], ntn);
  Unit u;
  u.g = g;
  u.row_end = off[g + 1];
  u.count = 0;
  // leading bands of full m-tiles (banded order, as in tile_at)
  const int lead = band_lead(gu.mfull);
  if (local < lead * ntn) {
    const int band = local / (kBand * ntn), i = local - band * (kBand * ntn);
    const int nt = i / kBand;
    u.m0 = off[g] + (band * kBand + (i - nt * kBand)) * kTileMBundle;
    u.nt0 = nt;
    return u;
  }
  // last band: its full m-tiles and the short tile, n-tiles in blocks of bsz
  local -= lead * ntn;
  const int mfull = gu.mfull - lead;
  const int m_base = off[g] + lead * kTileMBundle;
  if (gu.bsz == 0) {
    const int nt = local / mfull;
    u.m0 = m_base + (local - nt * mfull) * kTileMBundle;
    u.nt0 = nt;
    return u;
  }
  const int per = mfull * gu.bsz + 1;  // units of a whole block
  const int blk = local / per, i = local - blk * per;
  const int nb = min(gu.bsz, ntn - blk * gu.bsz);
  if (i < mfull * nb) {
    const int nt = i / mfull;
    u.m0 = m_base + (i - nt * mfull) * kTileMBundle;
    u.nt0 = blk * gu.bsz + nt;
  } else {
    u.m0 = m_base + mfull * kTileMBundle;
    u.nt0 = blk * gu.bsz;
    u.count = nb;
  }
  return u;
}

// Logical tile of this workgroup, or false if it has none.
__device__ __forceinline__ bool decode_tile(const int32_t* __restrict__ off,
                                            const int32_t* __restrict__ mstart, int G, int ntn,
                                            int BM, int ncol, Tile& tile) {
  const int total = mstart[G] * ntn;
  const int nw8 = (total + 7) & ~7;
  const int bid = blockIdx.x;
  if (bid >= nw8) return false;
  const int L = xcd_run(bid, nw8);
  if (L >= total) return false;
  tile = tile_at(L, off, mstart, G, ntn, BM, ncol);
  return true;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  kFused: B rows [0, BN/2) are W_gate rows n0.., rows
// [BN/2, BN) are W_up rows n0..; output columns n0 .. n0 + BN/2 of hid.
// Otherwise B rows are W rows n0 .. n0 + BN and the output is A W^T.
//
// K advances in slices of 64 (one 128-byte line per row); direct-to-LDS
// copies stream the A slices through a two-stage LDS ring and the B slices
// through a three-stage ring, one barrier per slice (see gemm_tile for the
// copy placement, the LDS swizzle and the wait counts).
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// bf16 tiles are 256 rows high except the last m-tile of each group, which
// runs as a 64-, 128- or 256-row tile according to the rows it holds (so a
// short remainder costs a quarter or a half of a full tile).  It stays in the
// group-major order, next to the tiles that share its weight panel.
// ---------------------------------------------------------------------------
constexpr int kTileM = 256;
// LDS ring depths (stages of 32 KB: 64 bf16 of 256 rows): two for A, three
// for B, 160 KB in all.  The third B stage lets the weight copies of a slice
// go out before the barrier that retires the previous one.
constexpr int kRingA = 2;
constexpr int kRingB = 3;

struct Tile2 {
  int g, m0, row_end, n0, cls;  // cls 0: 256 rows, 1: 128 rows, 2: 64 rows
};

__device__ __forceinline__ Tile2 classify(const Tile& t) {
  Tile2 tile;
  tile.g = t.g;
  tile.m0 = t.m0;
  tile.row_end = t.row_end;
  tile.n0 = t.n0;
  const int rem = t.row_end - t.m0;
  tile.cls = rem <= 64 ? 2 : (rem <= 128 ? 1 : 0);
  return tile;
}

// s_waitcnt with only the vector-memory counter constrained to <= n (n < 64)
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00);
}

// The direct-to-LDS copy of 16 bytes per lane written as an instruction the
// compiler does not model: it then adds no waits of its own around the copies
// and does not keep LDS reads ordered after them, which leaves both to the
// kernel (every wait on a copy is the explicit vmcnt wait before a barrier).
// M0 holds the wave's LDS destination; one wait state separates its write
// from the copy.
__device__ __forceinline__ void dma_lds16(const uint16_t* g, const uint16_t* l) {
  const uint32_t m0 = static_cast<uint32_t>(
      reinterpret_cast<size_t>((const __attribute__((address_space(3))) uint16_t*)l));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0)
               : "m0");
}

// The same copy from a workgroup-uniform base `sbase` plus a 32-bit per-lane
// byte offset.
__device__ __forceinline__ void dma_lds16_s(const uint16_t* sbase, uint32_t voff,
                                            const uint16_t* l) {
  const uint32_t m0 = static_cast<uint32_t>(
      reinterpret_cast<size_t>((const __attribute__((address_space(3))) uint16_t*)l));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(sbase), "s"(m0)
               : "m0");
}

// K slice per stage: 64 bf16, one 128-byte line of every row.  A compute
// unit's L2-to-LDS rate is bounded by its requests, one per row segment, so
// full-line rows move twice the bytes of half-line rows per request.
constexpr int kBK = 64;

// Element offset of 16-byte chunk `chunk` (0..7) of row `row` in a stage of
// 64-element rows.  The XOR with (row >> 1) & 7 puts the same chunk of 16
// consecutive rows on 16 distinct 16-byte bank groups, so that the 16 lanes
// served together by a 128-bit LDS read never collide.
__device__ __forceinline__ int swz64(int row, int chunk) {
  return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// Operand storage of the bf16 tiles.
//   kOpRows:  rows of the operand (tile rows for A, weight rows for B) are
//             contiguous along K (the forward's layout; A rows may be gathered).
//   kOpSlabT: B only; the expert's weight slab is stored K-major, [K][N] with
//             rows of N elements (the input-gradient GEMMs read the forward's
//             weights this way).
//   kOpSlabI: B only; K-major like kOpSlabT, with the even K rows 2i from row
//             i of B0's slab and the odd rows 2i + 1 from row i of B1's (the
//             gate and up weights against the interleaved (du, dv) columns).
//   kOpRowsT: K-major data rows: K runs over the rows r0 .. rend - 1 of a
//             row-major buffer whose columns are the tile's M (A, row length
//             lda) or N (B, row length ldb); K rows past rend read the zero
//             row (the weight gradients contract over an expert's rows).
// A K-major stage is read with ds_read_b64_tr_b16: within each 16-lane group
// lane s passes the address of 4 consecutive columns x0 + 4 (s mod 4) of row
// k0 + s / 4 and receives column x0 + s of rows k0 .. k0 + 3, which is the
// MFMA operand layout (a lane holds one column and consecutive k).
constexpr int kOpRows = 0;
constexpr int kOpSlabT = 1;
constexpr int kOpRowsT = 2;
constexpr int kOpSlabI = 3;

struct OpArgs {
  int r0, rend;          // kOpRowsT: row range of the K axis
  int lda, ldb;          // kOpRowsT: row lengths of A and B
  int a_cols;            // kOpRowsT: columns of A (the GEMM's M)
  const uint16_t* zero;  // kOpRowsT: a row of zeros, at least as long as any row read
};

// Chunk swizzle of a K-major stage with rows of X columns: the half-wave of a
// transposed read covers 4 rows x 64 bytes, which land on distinct bank
// groups (rows of 256 and 512 bytes: XOR of bits 2-3 of the chunk with k mod
// 4; rows of 128 bytes: bit 2 with bit 1 of k).
__device__ __forceinline__ int swz_kmajor(int k, int X) {
  return X >= 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
}

// LDS element offset of this lane's first transposed read of the 32-column
// fragment at column xb (k step 0); the second read is 4 rows further.
__device__ __forceinline__ int kmajor_frag(int xb, int X, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  const int x = xb + 16 * (g & 1) + 4 * (sl & 3);
  const int k = 8 * (g >> 1) + (sl >> 2);
  return k * X + (((x >> 3) ^ swz_kmajor(k, X)) << 3) + (x & 7);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Fragment of 8 consecutive k (rows p, p + 1, ... of a K-major stage) for this
// lane's column: two transposed reads of 4 rows each.
__device__ __forceinline__ bf16x8 read_kmajor(const uint16_t* p, int X) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  lds_i16x4* q0 = (lds_i16x4*)((__attribute__((address_space(3))) uint16_t*)(p));
  lds_i16x4* q1 = (lds_i16x4*)((__attribute__((address_space(3))) uint16_t*)(p + 4 * X));
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Epilogue modes of the bf16 tiles.
//   kEpiNone:    C = A B^T (fused: C = SiLU(gate) * up).
//   kEpiSaveUV:  fused only; also keeps the two pre-activations of every
//                output, uv[r, 2c] = gate sum and uv[r, 2c + 1] = up sum
//                (bf16), for the backward pass.
//   kEpiSiluBwd: unfused, N = h, the accumulator is dhid = dout W_down; with
//                u, v read back from uv:
//                  du = dhid v SiLU'(u),  dv = dhid SiLU(u)
//                written to dab[r, 2c] = du, dab[r, 2c + 1] = dv (bf16).  C
//                is not written.
//   kEpiRowPairs: unfused fp32; even output rows 2m go to C row m, odd rows
//                2m + 1 to row m of c_odd (the gate and up weight gradients of
//                one GEMM over the interleaved (du, dv) columns).
constexpr int kEpiNone = 0;
constexpr int kEpiSaveUV = 1;
constexpr int kEpiSiluBwd = 2;
constexpr int kEpiRowPairs = 3;

struct EpiArgs {
  uint16_t* uv;   // [rows, 2N]
  uint16_t* dab;  // [rows, 2N]
  float* c_odd;   // kEpiRowPairs
};

// bf16 outputs leave the tile in 16-byte stores of eight columns.  For the
// MFMA layout, lane l holds columns 8q + 4 (l / 32) + 0..3 of a 32-column
// block (four bf16, `lo` for q, `hi` for q + 1, packed in pairs); exchanging
// lane i's columns of q + 1 with lane i + 32's columns of q
// (v_permlane32_swap: lanes 32..63 of the first operand trade places with
// lanes 0..31 of the second) leaves lane i with columns 8q + 0..7 and lane
// i + 32 with 8q + 8..15.  In this layout a compute unit retires stores at
// about one lane per cycle, 8 or 16 bytes alike, so 16 bytes per lane halve
// the store phase of a bf16 tile against 8.
__device__ __forceinline__ u32x4 pair_cols(u32x2 lo, u32x2 hi) {
  const auto a = __builtin_amdgcn_permlane32_swap(lo[0], hi[0], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(lo[1], hi[1], false, false);
  return u32x4{a[0], b[0], a[1], b[1]};
}

// fp32 weight-gradient tiles leave through LDS.  In the MFMA layout one store
// of a wave covers 32 rows x 32 bytes, and a compute unit retires such stores
// at about one lane per cycle: a 256 x 256 fp32 tile takes about 7 us even
// when few compute units store at once.  Stores that each cover one whole
// 1 KB row retire about 3.5 times as fast.  (When every compute unit stores
// at once, as in lock-step weight-gradient tiles, the chip's write rate of
// about 5.5 TB/s bounds both forms; the whole rows gain where the units
// drift apart.)  After the K loop the rings are
// free, so the tile is written into a row-major LDS image (rounds of at most
// 128 rows of 1 KB; 16-byte chunk c of image row r at chunk c ^ (r & 15), so
// that the 16 rows of one write pass fall on distinct bank groups and the
// chunks of a row, read by consecutive lanes, on all 64 banks) and copied out
// one whole row per wave store.
constexpr int kImgRows = 128;

__device__ __forceinline__ int img_off(int r, int b) {  // image rows of 1 KB
  return r * 1024 + ((((b >> 4) ^ (r & 15)) << 4) | (b & 15));
}

// acc[i][j] element 4q + e of lane l is C[row, col] with row = m-block i row
// (l & 31) and col = n-block j column 8q + 4 (l >> 5) + e.  kEpiRowPairs:
// even rows 2m go to row m of C, odd rows to row m of ep.c_odd.  Rows past
// row_end and columns past N are not written.  The caller has passed a
// barrier after the K loop (every wave has read its last slice and every copy
// has landed).
template <int BM, int WM, int WN, int BN, int kEpi, int MT, int NT>
__device__ __forceinline__ void rows_out_f32(const f32x16 (&acc)[MT][NT], uint16_t* smem, int tid,
                                             int lane, int wm, int wn, const Tile2& tile, int N,
                                             float* C, const EpiArgs& ep) {
  static_assert(BN * 4 == 1024, "image rows of 1 KB");
  constexpr int RR = BM < kImgRows ? BM : kImgRows;  // image rows per round
  constexpr int R = BM / RR;                          // rounds
  constexpr int IPR = MT / R;                         // m-blocks of a wave per round
  constexpr int RW = RR / WM;                         // image rows of a wave per round
  static_assert(R * RR == BM && IPR * R == MT && RW == IPR * 32, "rounds of whole m-blocks");
  static_assert(RR * 1024 <= (kRingA * kTileM + kRingB * 256) * kBK * 2, "image fits the rings");
  char* img = reinterpret_cast<char*>(smem);
  const int cq = 4 * (lane >> 5);
#pragma unroll
  for (int rho = 0; rho < R; ++rho) {
    if (rho > 0) __syncthreads();  // the previous round's image has been read
#pragma unroll
    for (int ii = 0; ii < IPR; ++ii) {
      const int i = rho * IPR + ii;
      const int lr = wm * RW + ii * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lc = wn * (BN / WN) + j * 32 + cq + 8 * q;
          *reinterpret_cast<f32x4*>(img + img_off(lr, 4 * lc)) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                    acc[i][j][4 * q + 3]};
        }
    }
    __syncthreads();
#pragma unroll 8
    for (int it = 0; it < RR * 64 / kThreads; ++it) {
      const int g = it * kThreads + tid;
      const int lr = g >> 6, b = (g & 63) * 16;
      const int row = tile.m0 + (lr / RW) * (BM / WM) + rho * RW + lr % RW;
      const int col = tile.n0 + b / 4;
      if (row >= tile.row_end || col >= N) continue;
      float* dst = kEpi == kEpiRowPairs
                       ? (row & 1 ? ep.c_odd : C) + static_cast<int64_t>(row >> 1) * N + col
                       : C + static_cast<int64_t>(row) * N + col;
      *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(img + img_off(lr, b));
    }
  }
}

// One output tile of BM rows (BM = 256, 128 or 64) and BN columns; the four
// waves form a WM x WN grid, each wave a (BM/WM) x (BN/WN) block of MFMA
// tiles.  The LDS rings are laid out for kTileM rows of A whatever BM is.
template <int BM, int WM, int WN, int BN, int SA, int SB, bool kFused, typename OutT, int kEpi,
          int kAM = kOpRows, int kBM = kOpRows>
__device__ __forceinline__ void gemm_tile(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows, int a_div,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, int64_t b_stride, int K,
    int N, const Tile2& tile, int ks0, int nk, uint16_t* smem, OutT* __restrict__ C,
    float* __restrict__ part_out, const EpiArgs& ep, const OpArgs& oa = OpArgs{}) {
  static_assert(WM * WN == 4, "four waves");
  static_assert(kEpi == kEpiNone || (kEpi == kEpiSaveUV) == kFused, "epilogue mode");
  constexpr int MT = BM / WM / 32;            // 32-row MFMA tiles per wave
  constexpr int NT = BN / WN / 32;            // 32-col MFMA tiles per wave
  constexpr int AP = BM / 32;                 // copies per wave per stage (A): 8 rows each
  constexpr int BP = BN / 32;                 // (B)
  constexpr int P = AP + BP;
  static_assert(!kFused || NT % 2 == 0, "fused tile needs matching gate/up halves");

  uint16_t* As = smem;                         // [SA][kTileM * kBK]
  uint16_t* Bs = smem + SA * kTileM * kBK;     // [SB][BN * kBK]

  // the thread index is made opaque here so that nothing derived from it is
  // hoisted out of the persistent loop around this tile (such values would
  // stay live through the epilogue and push accumulators out to scratch)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid % kWave, wave = tid / kWave;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = WM == 1 ? 0 : (wave & 1), wn = WM == 1 ? wave : (wave >> 1);
  // Copy j of a wave covers the 8 tile rows 8 (4 j + wave) + 0..7: lane l
  // lands in row l / 8, chunk slot l % 8 of that 1 KB block and fetches the
  // global chunk that the swizzle stores there.  ((row >> 1) & 7 of those
  // rows depends only on the wave's parity and l / 16.)
  const int lrow = lane >> 3;
  const int gchunk = (lane & 7) ^ (((wave & 1) << 2) | (lrow >> 1));

  // K-major operands (kAM / kBM != kOpRows): a stage holds 64 K rows of the
  // tile's X = BM (A) or BN (B) columns, row-major, 16-byte chunk c of row k
  // at slot c ^ swz_kmajor(k, X); copy j of a wave fills 1 KB = 512 / X rows.
  // Each lane copies the same global chunk column in every copy (the swizzle
  // depends on k mod 4 only, and each copy advances k by a multiple of 4).
  constexpr int AXR = 512 / BM, BXR = 512 / BN;  // K rows per 1 KB copy
  const int a_kr0 = wave * AXR + lane / (BM / 8);
  const int b_kr0 = wave * BXR + lane / (BN / 8);
  const int a_kcol = tile.m0 + 8 * ((lane % (BM / 8)) ^ swz_kmajor(a_kr0, BM));
  const int b_kcol = tile.n0 + 8 * ((lane % (BN / 8)) ^ swz_kmajor(b_kr0, BN));

  int src[AP];
  const uint16_t* ap[AP];
  if constexpr (kAM == kOpRows) {
#pragma unroll
    for (int j = 0; j < AP; ++j) {
      const int r = tile.m0 + 8 * (4 * j + wave) + lrow;
      src[j] = r < tile.row_end ? r : tile.row_end - 1;  // rows past the group: valid row, unused
    }
    if (a_rows) {  // gather: all index loads first, then the divisions
#pragma unroll
      for (int j = 0; j < AP; ++j) src[j] = a_rows[src[j]];
#pragma unroll
      for (int j = 0; j < AP; ++j) src[j] /= a_div;
    }
#pragma unroll
    for (int j = 0; j < AP; ++j) ap[j] = A + static_cast<int64_t>(src[j]) * K + gchunk * 8;
  }
  // B copies: the expert's weight slab (gate rows for j < BP/2 of a fused
  // tile, up rows after) is uniform, the row offset within it per lane
  uint32_t boff[BP];
  if constexpr (kBM == kOpRows) {
#pragma unroll
    for (int j = 0; j < BP; ++j) {
      const int r = 8 * (4 * j + wave) + lrow;
      int n = tile.n0 + ((kFused && r >= BN / 2) ? r - BN / 2 : r);
      n = n < N ? n : N - 1;
      boff[j] = static_cast<uint32_t>(n) * static_cast<uint32_t>(K * 2) + gchunk * 16;
    }
  } else if constexpr (kBM == kOpSlabT) {
    // K-major weight slab: lane offset of copy j in bytes (columns past N
    // read a valid column, unused)
    const int col = b_kcol < N ? b_kcol : N - 8;
#pragma unroll
    for (int j = 0; j < BP; ++j)
      boff[j] = (static_cast<uint32_t>(b_kr0 + 4 * j * BXR) * static_cast<uint32_t>(N) +
                 static_cast<uint32_t>(col)) * 2u;
  }
  const uint16_t* bslab0 = B0 + tile.g * b_stride;
  const uint16_t* bslab1 = (kFused ? B1 : B0) + tile.g * b_stride;
  // interleaved slabs: each lane's K rows have one parity in every copy (the
  // copies advance k by a multiple of 4), so it always reads one slab
  const uint16_t* bi_lane = nullptr;
  if constexpr (kBM == kOpSlabI) {
    const int col = b_kcol < N ? b_kcol : N - 8;
    bi_lane = ((b_kr0 & 1) ? B1 : B0) + tile.g * b_stride + static_cast<int64_t>(b_kr0 >> 1) * N +
              col;
  }
  static_assert(!kFused || sizeof(OutT) == 2, "split-K partials are for the unfused GEMM");
  static_assert(!kFused || (kAM == kOpRows && kBM == kOpRows), "fused tiles read row-major operands");

  // this tile covers K slices ks0 .. ks0 + nk - 1 (all of K unless split)
  if constexpr (kAM == kOpRows) {
#pragma unroll
    for (int j = 0; j < AP; ++j) ap[j] += ks0 * kBK;
  }
  if constexpr (kBM == kOpRows) {
    bslab0 += ks0 * kBK;
    bslab1 += ks0 * kBK;
  }
  // K-major data rows (kOpRowsT): global row of K slice ks, copy j; rows past
  // the range read the zero row
  const int a_col = a_kcol < oa.a_cols ? a_kcol : oa.a_cols - 8;
  const int b_col = b_kcol < N ? b_kcol : N - 8;
  // Copy j's pointer at slice 0 and how far (in K rows) it may advance before
  // its row passes rend, computed once per tile: a slice then costs one
  // uniform 64-bit step and a compare per copy instead of a 64-bit multiply.
  const uint16_t* at0[kAM == kOpRowsT ? AP : 1];
  int alim[kAM == kOpRowsT ? AP : 1];
  if constexpr (kAM == kOpRowsT) {
#pragma unroll
    for (int j = 0; j < AP; ++j) {
      const int row = oa.r0 + ks0 * kBK + a_kr0 + 4 * j * AXR;
      at0[j] = A + static_cast<int64_t>(row) * oa.lda + a_col;
      alim[j] = oa.rend - row;
    }
  }
  const uint16_t* bt0[kBM == kOpRowsT ? BP : 1];
  int blim[kBM == kOpRowsT ? BP : 1];
  if constexpr (kBM == kOpRowsT) {
#pragma unroll
    for (int j = 0; j < BP; ++j) {
      const int row = oa.r0 + ks0 * kBK + b_kr0 + 4 * j * BXR;
      bt0[j] = B0 + static_cast<int64_t>(row) * oa.ldb + b_col;
      blim[j] = oa.rend - row;
    }
  }
  auto rows_t_ptr = [&](const uint16_t* p0, int lim, int ld, int col, int ks) {
    return ks * kBK < lim ? p0 + static_cast<int64_t>(ks * kBK) * ld : oa.zero + col;
  };
  auto slab_t_base = [&](int ks) { return bslab0 + static_cast<int64_t>(ks0 + ks) * kBK * N; };
  // copy K slice `ks` (clamped into range: surplus copies reload the last slice
  // into a stage nobody reads again, which keeps the loop branch-free)
#define MOE_COPY_A(j, stage, ks)                                                     \
  do {                                                                               \
    const int ksc_ = (ks) < nk ? (ks) : nk - 1;                                      \
    uint16_t* dst_ = As + (stage) * kTileM * kBK + 8 * (4 * (j) + wave_u) * kBK;     \
    if constexpr (kAM == kOpRows)                                                    \
      dma_lds16(ap[(j)] + ksc_ * kBK, dst_);                                         \
    else                                                                             \
      dma_lds16(rows_t_ptr(at0[(j)], alim[(j)], oa.lda, a_col, ksc_), dst_);         \
  } while (0)
#define MOE_COPY_B(j, stage, ks)                                                     \
  do {                                                                               \
    const int ksc_ = (ks) < nk ? (ks) : nk - 1;                                      \
    uint16_t* dst_ = Bs + (stage) * BN * kBK + 8 * (4 * (j) + wave_u) * kBK;         \
    if constexpr (kBM == kOpRows)                                                    \
      dma_lds16_s(((kFused && (j) >= BP / 2) ? bslab1 : bslab0) + ksc_ * kBK, boff[(j)], \
                  dst_);                                                             \
    else if constexpr (kBM == kOpSlabT)                                              \
      dma_lds16_s(slab_t_base(ksc_), boff[(j)], dst_);                               \
    else if constexpr (kBM == kOpSlabI)                                              \
      dma_lds16(bi_lane + (static_cast<int64_t>(ks0 + ksc_) * (kBK / 2) + 2 * (j) * BXR) * N, \
                dst_);                                                               \
    else                                                                             \
      dma_lds16(rows_t_ptr(bt0[(j)], blim[(j)], oa.ldb, b_col, ksc_), dst_);         \
  } while (0)

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

  // LDS element offsets of this lane's fragments for k step 0; step s is the
  // same offset XOR (s << 4), as the swizzle flips only chunk bits
  // (K-major stages: the offset of the first transposed read of step 0;
  // step s adds 16 s rows, the second read 4 rows)
  int aoff[MT], boffl[NT];
  const int khalf = lane >> 5;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int x = wm * (BM / WM) + i * 32;
    aoff[i] = kAM == kOpRows ? swz64(x + (lane & 31), khalf) : kmajor_frag(x, BM, lane);
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int row;
    if (kFused) {
      row = (j < NT / 2) ? wn * (BN / (2 * WN)) + j * 32
                         : BN / 2 + wn * (BN / (2 * WN)) + (j - NT / 2) * 32;
    } else {
      row = wn * (BN / WN) + j * 32;
    }
    boffl[j] = kBM == kOpRows ? swz64(row + (lane & 31), khalf) : kmajor_frag(row, BN, lane);
  }

  // read r < MT is A fragment r, else B fragment r - MT, of k step `step`
#define MOE_READ1(F, sa, sb, step, r)                                                \
  do {                                                                               \
    if ((r) < MT) {                                                                  \
      const int i_ = (r) < MT ? (r) : 0;                                             \
      const uint16_t* base_ = As + (sa) * kTileM * kBK;                              \
      if constexpr (kAM == kOpRows)                                                  \
        F##a[i_] = *reinterpret_cast<const bf16x8*>(base_ + (aoff[i_] ^ ((step) << 4))); \
      else                                                                           \
        F##a[i_] = read_kmajor(base_ + aoff[i_] + (step) * 16 * BM, BM);             \
    } else {                                                                         \
      const int j_ = (r) >= MT ? (r) - MT : 0;                                       \
      const uint16_t* base_ = Bs + (sb) * BN * kBK;                                  \
      if constexpr (kBM == kOpRows)                                                  \
        F##b[j_] = *reinterpret_cast<const bf16x8*>(base_ + (boffl[j_] ^ ((step) << 4))); \
      else                                                                           \
        F##b[j_] = read_kmajor(base_ + boffl[j_] + (step) * 16 * BN, BN);            \
    }                                                                                \
  } while (0)
// acc[i][j] accumulates the transposed product of m-block i and n-block j
// (the weight fragment is the MFMA's first operand), so that a lane ends up
// holding one row of C and runs of four consecutive columns
#define MOE_MFMA1(F, t)                                                              \
  acc[(t) / NT][(t) % NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                 \
      F##b[(t) % NT], F##a[(t) / NT], acc[(t) / NT][(t) % NT], 0, 0, 0)

  bf16x8 f0a[MT], f0b[NT], f1a[MT], f1b[NT];
  constexpr int kSlots = MT * NT;                 // MFMAs per k step
  constexpr int kReads = MT + NT;                 // LDS reads per k step
  static_assert(kReads <= kSlots, "one read per MFMA slot at most");
  static_assert(SA == 2 && SB == 3, "copy placement below assumes rings of 2 (A) and 3 (B)");
  // A compute unit takes a copy instruction about every 16 cycles, so the
  // copies are spread over the whole slice: B slice kt+2 during the three k
  // steps before the barrier of iteration kt (into the stage of slice kt-1,
  // retired by the previous barrier), A slice kt+2 during the step after it
  // (into the stage of slice kt).  Slot t of a k step issues MFMA t, then
  // read t (t < kReads) of the next step's fragments, then its copies.
#define MOE_STEP(FU, FL, sa_, sb_, step_, MODE, PART, stage_, ks_)                     \
  _Pragma("unroll") for (int t = 0; t < kSlots; ++t) {                               \
    MOE_MFMA1(FU, t);                                                                \
    if (t < kReads) MOE_READ1(FL, sa_, sb_, step_, t);                               \
    if (MODE == 1) {                                                                 \
      _Pragma("unroll") for (int c = 0; c < BP; ++c)                                 \
        if (c * 3 * kSlots / BP == (PART) * kSlots + t) MOE_COPY_B(c, stage_, ks_);  \
    } else if (MODE == 2) {                                                          \
      _Pragma("unroll") for (int c = 0; c < AP; ++c)                                 \
        if (c * kSlots / AP == t) MOE_COPY_A(c, stage_, ks_);                        \
    }                                                                                \
    __builtin_amdgcn_sched_barrier(0);                                               \
  }

  // Virtual iteration v issues B slice v+2 and then A slice v+2; the prologue
  // runs v = -2, -1.  Loads of a wave complete in issue order: when A slice
  // kt+1 (issued in iteration kt-1) has landed, only B slice kt+2 (issued
  // before the barrier of iteration kt) may still be in flight, and B slice
  // kt+1 (issued before A slice kt+1) has landed.
#pragma unroll
  for (int v = -2; v < 0; ++v) {
#pragma unroll
    for (int j = 0; j < BP; ++j) MOE_COPY_B(j, v + 2, v + 2);
#pragma unroll
    for (int j = 0; j < AP; ++j) MOE_COPY_A(j, v + 2, v + 2);
  }
  wait_vm<P>();
  __syncthreads();
  int sa = 0, sb = 0;  // stages of slice kt
  int sbn = 2;         // B stage of slice kt+2
#pragma unroll
  for (int r = 0; r < kReads; ++r) MOE_READ1(f0, 0, 0, 0, r);
  for (int kt = 0; kt < nk; ++kt) {
    const int sa1 = sa + 1 == SA ? 0 : sa + 1, sb1 = sb + 1 == SB ? 0 : sb + 1;
    __builtin_amdgcn_sched_barrier(0);
    MOE_STEP(f0, f1, sa, sb, 1, 1, 0, sbn, kt + 2)
    MOE_STEP(f1, f0, sa, sb, 2, 1, 1, sbn, kt + 2)
    MOE_STEP(f0, f1, sa, sb, 3, 1, 2, sbn, kt + 2)
    // every wave has read slice kt (the compiler's LDS wait precedes the
    // barrier); slice kt+1 has landed once this wave's A copies of it have
    wait_vm<BP>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    MOE_STEP(f1, f0, sa1, sb1, 0, 2, 0, sa, kt + 2)
    sbn = sb;
    sa = sa1;
    sb = sb1;
  }
  wait_vm<0>();
#undef MOE_COPY_A
#undef MOE_COPY_B
#undef MOE_READ1
#undef MOE_MFMA1
#undef MOE_STEP
  if constexpr (kAM == kOpRowsT) {  // weight gradients: fp32 tiles through the LDS image
    static_assert(sizeof(OutT) == 4 && !kFused, "fp32 weight-gradient tiles");
    __syncthreads();
    rows_out_f32<BM, WM, WN, BN, kEpi>(acc, smem, tid, lane, wm, wn, tile, N,
                                       reinterpret_cast<float*>(C), ep);
    return;
  }
  // epilogue: acc[i][j] element 4q + e of lane l is C[row, col] with row =
  // m-block i row (l & 31) and col = n-block j column 8q + 4 (l >> 5) + e, so
  // every lane holds runs of four columns (bf16 outputs pair two runs into
  // eight, pair_cols; N % 64 == 0 keeps a run whole)
  const int row0 = tile.m0 + wm * (BM / WM) + (lane & 31);
  const int cq = 4 * (lane >> 5);
  if constexpr (kEpi == kEpiSiluBwd) {
    // dab[r] = (du, dv) pairs from the accumulator (dhid) and the kept (u, v)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = row0 + i * 32;
      if (row >= tile.row_end) continue;
      const uint16_t* urow = ep.uv + static_cast<int64_t>(row) * (2 * N);
      uint16_t* drow = ep.dab + static_cast<int64_t>(row) * (2 * N);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int cb = tile.n0 + wn * (BN / WN) + j * 32 + cq;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = cb + 8 * q;
          if (col >= N) continue;
          const u32x4 uv = *reinterpret_cast<const u32x4*>(urow + 2 * col);
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float u = __uint_as_float(uv[e] << 16);
            const float v = __uint_as_float(uv[e] & 0xFFFF0000u);
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-u));  // 0 once exp overflows
            // dv = dh u sg, du = dh v sg (1 + u (1 - sg)), sharing dh sg
            const float a = acc[i][j][4 * q + e] * sg;
            o[e] = pack_bf16x2((a * v) * __builtin_fmaf(u, 1.0f - sg, 1.0f), a * u);
          }
          *reinterpret_cast<u32x4*>(drow + 2 * col) = u32x4{o[0], o[1], o[2], o[3]};
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = row0 + i * 32;
    if (row >= tile.row_end) continue;
    OutT* crow = C + static_cast<int64_t>(row) * N;
    if constexpr (kEpi == kEpiRowPairs)
      crow = reinterpret_cast<OutT*>(row & 1 ? ep.c_odd : reinterpret_cast<float*>(C)) +
             static_cast<int64_t>(row >> 1) * N;
    if constexpr (kFused) {
#pragma unroll
      for (int j = 0; j < NT / 2; ++j) {
        const int cb = tile.n0 + wn * (BN / (2 * WN)) + j * 32;  // the n-block's first column
        u32x2 pk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = silu_f32(acc[i][j][4 * q + e]) * acc[i][j + NT / 2][4 * q + e];
          pk[q] = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          if constexpr (kEpi == kEpiSaveUV) {
            // (u, v) pairs of the four columns: one 16-byte store
            const int col = cb + cq + 8 * q;
            const f32x16& ga = acc[i][j];
            const f32x16& ua = acc[i][j + NT / 2];
            if (col < N)
              *reinterpret_cast<u32x4*>(ep.uv + static_cast<int64_t>(row) * (2 * N) + 2 * col) =
                  u32x4{pack_bf16x2(ga[4 * q], ua[4 * q]), pack_bf16x2(ga[4 * q + 1], ua[4 * q + 1]),
                        pack_bf16x2(ga[4 * q + 2], ua[4 * q + 2]),
                        pack_bf16x2(ga[4 * q + 3], ua[4 * q + 3])};
          }
        }
#pragma unroll
        for (int qp = 0; qp < 4; qp += 2) {
          const u32x4 o = pair_cols(pk[qp], pk[qp + 1]);
          const int col = cb + 8 * qp + 2 * cq;
          if (col < N) *reinterpret_cast<u32x4*>(crow + col) = o;
        }
      }
    } else if (part_out) {  // fp32 partial sums, [256][256] relative to (m0, n0)
      float* prow = part_out + (row - tile.m0) * BN;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int cb = wn * (BN / WN) + j * 32 + cq;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = cb + 8 * q;
          if (tile.n0 + c >= N) continue;
          f32x4 o = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                     acc[i][j][4 * q + 3]};
          *reinterpret_cast<f32x4*>(prow + c) = o;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int cb = tile.n0 + wn * (BN / WN) + j * 32;  // the n-block's first column
        if constexpr (sizeof(OutT) == 2) {
          u32x2 pk[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            pk[q] = u32x2{pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                          pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
#pragma unroll
          for (int qp = 0; qp < 4; qp += 2) {
            const u32x4 o = pair_cols(pk[qp], pk[qp + 1]);
            const int col = cb + 8 * qp + 2 * cq;
            if (col < N) *reinterpret_cast<u32x4*>(crow + col) = o;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = cb + cq + 8 * q;
            if (col >= N) continue;
            f32x4 o = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                       acc[i][j][4 * q + 3]};
            *reinterpret_cast<f32x4*>(crow + col) = o;
          }
        }
      }
    }
  }
}

// Next work item of a persistent workgroup on XCD x: a whole tile (or work
// unit) of run x; once run x is empty, one of the other XCDs' runs, taken in
// turn (x + 1, x + 2, ... mod 8) from the same counters, so that an XCD that
// finishes early helps with the units another XCD has not started (the
// estimated costs that cut the runs are only estimates); after all runs,
// (n_parts > 0) a split-K part from the shared counter.  Returns the item
// (>= 0), -2 - p for split part p, or -1 when none is left.  `victim`
// (thread 0's, kept by the caller across calls) is the offset of the run
// being taken from.
// Thread 0 takes it from the counters and hands it to the four waves through
// the first word of the third B stage: between two items no copy and no real
// fragment read touches that word (it lies in row 0, which only wave 0's
// copies write, and wave 0 waited for all of its copies at the end of the
// previous item; the next item first writes the third stage after its
// prologue barrier, which every wave reaches only after reading the word).
__device__ __forceinline__ int next_work(const int32_t* __restrict__ runs, int32_t* counters, int x,
                                         int n_parts, uint16_t* smem, int& victim) {
  volatile int32_t* word =
      reinterpret_cast<volatile int32_t*>(smem + (kRingA * kTileM + 2 * 256) * kBK);
  if (threadIdx.x == 0) {
    int code = -1;
    for (; victim < kXcds; ++victim) {
      const int v = (x + victim) & (kXcds - 1);
      const int c = runs[v] + atomicAdd(&counters[v], 1);
      if (c < runs[v + 1]) {
        code = c;
        break;
      }
    }
    if (code < 0 && n_parts > 0) {
      const int p = atomicAdd(&counters[kXcds], 1);
      if (p < n_parts) code = -2 - p;
    }
    *word = code;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*word);
}

// Persistent: one workgroup per compute unit (see tile_table_kernel for the
// runs).  tt: the tile-table workspace (mstart first); skw: split-K
// workspace (kSkUnits fp32 256 x 256 tiles) or NULL (no split); ncu: compute
// units of the device, as given to tile_table_kernel.
template <bool kFused, typename OutT, int kEpi, int kBM = kOpRows>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows, int a_div,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, int64_t b_stride, int K,
    int N, const int32_t* __restrict__ off, int32_t* __restrict__ tt, int G, int ntn,
    OutT* __restrict__ C, float* __restrict__ skw, int ncu, EpiArgs ep, OpArgs oa) {
  constexpr int BN = 256;
  extern __shared__ __align__(16) uint16_t smem[];
  const int32_t* mstart = tt;
  const int32_t* runs = tt + tt_runs(G);
  int32_t* counters = tt + tt_counters(G);
  const int x = blockIdx.x % kXcds;
  int victim = 0;
  if constexpr (kFused) {  // bundled order, no split
    for (;;) {
      const int L = next_work(runs, counters, x, 0, smem, victim);
      if (L < 0) return;
      const Unit u = unit_at(L, off, mstart, G, ntn);
      Tile t{u.g, u.m0, u.row_end, 0};
      if (u.count == 0) {
        t.n0 = u.nt0 * (BN / 2);
        const Tile2 tile = classify(t);
        gemm_tile<256, 2, 2, BN, kRingA, kRingB, kFused, OutT, kEpi, kOpRows, kBM>(A, a_rows, a_div, B0, B1,
                                                              b_stride, K, N, tile, 0, K / kBK,
                                                              smem, C, nullptr, ep, oa);
        continue;
      }
      for (int s = 0; s < u.count; ++s) {
        if (s > 0) __syncthreads();  // the previous tile's last LDS reads are done
        t.n0 = (u.nt0 + s) * (BN / 2);
        const Tile2 tile = classify(t);
        if (tile.cls == 1)
          gemm_tile<128, 1, 4, BN, kRingA, kRingB, kFused, OutT, kEpi, kOpRows, kBM>(A, a_rows, a_div, B0, B1,
                                                                b_stride, K, N, tile, 0, K / kBK,
                                                                smem, C, nullptr, ep, oa);
        else
          gemm_tile<64, 1, 4, BN, kRingA, kRingB, kFused, OutT, kEpi, kOpRows, kBM>(A, a_rows, a_div, B0, B1,
                                                               b_stride, K, N, tile, 0, K / kBK,
                                                               smem, C, nullptr, ep, oa);
      }
    }
  } else {
    const int nk_all = K / kBK;
    const SkPlan plan = sk_plan(mstart[G] * ntn, ncu, nk_all, skw != nullptr);
    const int n_parts = plan.n_sk * plan.S;
    for (;;) {
      const int code = next_work(runs, counters, x, n_parts, smem, victim);
      if (code == -1) return;
      int L = code, ks0 = 0, nk = nk_all;
      float* part_out = nullptr;
      if (code < 0) {
        const int u = -2 - code;
        const int slot = u / plan.S, part = u - slot * plan.S;
        L = plan.n_dp + slot;
        ks0 = part * nk_all / plan.S;
        nk = (part + 1) * nk_all / plan.S - ks0;
        part_out = skw + static_cast<size_t>(u) * (kTileM * BN);
      }
      const Tile2 tile = classify(tile_at(L, off, mstart, G, ntn, kTileM, BN));
      if (tile.cls == 0) {
        gemm_tile<256, 2, 2, BN, kRingA, kRingB, kFused, OutT, kEpi, kOpRows, kBM>(A, a_rows, a_div, B0, B1,
                                                              b_stride, K, N, tile, ks0, nk,
                                                              smem, C, part_out, ep, oa);
      } else if (tile.cls == 1) {
        gemm_tile<128, 1, 4, BN, kRingA, kRingB, kFused, OutT, kEpi, kOpRows, kBM>(A, a_rows, a_div, B0, B1,
                                                              b_stride, K, N, tile, ks0, nk,
                                                              smem, C, part_out, ep, oa);
      } else {
        gemm_tile<64, 1, 4, BN, kRingA, kRingB, kFused, OutT, kEpi, kOpRows, kBM>(A, a_rows, a_div, B0, B1,
                                                             b_stride, K, N, tile, ks0, nk,
                                                             smem, C, part_out, ep, oa);
      }
    }
  }
}

// Adds the S parts of every split tile in part order and writes the rows and
// columns of the tile that exist; 32 workgroups per split tile, each thread 8
// columns of one row.
template <typename OutT>
__global__ __launch_bounds__(256) void sk_reduce_kernel(const float* __restrict__ skw,
                                                        const int32_t* __restrict__ off,
                                                        const int32_t* __restrict__ mstart, int G,
                                                        int ntn, int K, int N, int ncu,
                                                        OutT* __restrict__ C) {
  constexpr int BN = 256;
  const int total = mstart[G] * ntn;
  const SkPlan plan = sk_plan(total, ncu, K / kBK, true);
  const int slot = blockIdx.x / 32;
  if (slot >= plan.n_sk) return;
  const Tile t = tile_at(plan.n_dp + slot, off, mstart, G, ntn, kTileM, BN);
  const int lr = (blockIdx.x % 32) * 8 + threadIdx.x / 32;
  const int lc = (threadIdx.x % 32) * 8;
  const int row = t.m0 + lr, col = t.n0 + lc;
  if (row >= t.row_end || col >= N) return;
  f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f}, b = a;
  for (int part = 0; part < plan.S; ++part) {
    const float* src = skw + static_cast<size_t>(slot * plan.S + part) * (kTileM * BN) + lr * BN + lc;
    a += *reinterpret_cast<const f32x4*>(src);
    b += *reinterpret_cast<const f32x4*>(src + 4);
  }
  OutT* dst = C + static_cast<int64_t>(row) * N + col;
  if constexpr (sizeof(OutT) == 2) {
    u32x4 pk = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                pack_bf16x2(b[2], b[3])};
    *reinterpret_cast<u32x4*>(dst) = pk;
  } else {
    *reinterpret_cast<f32x4*>(dst) = a;
    *reinterpret_cast<f32x4*>(dst + 4) = b;
  }
}

// ---------------------------------------------------------------------------
// Skinny bf16 kernel for groups of a few rows (decode-shaped batches): the
// weights are streamed once from HBM and dominate the bytes, so one wave per
// workgroup walks one or a few consecutive 64-row slabs of one group's weight
// matrix (fused: 32 gate rows and the matching 32 up rows) along K, with the weight rows as the 16-row A
// operand of v_mfma_f32_16x16x32_bf16 and up to TBN blocks of 16 token rows as
// the B operand.  No LDS: per 64-wide K chunk each lane loads two 16-byte
// pieces of a weight row, at k = 64c + 8 (lane/16) and 32 later, so that every
// load instruction covers 64 contiguous bytes of each of its 16 rows (the two
// instructions together the full 128-byte line), and the matching pieces of
// its token row.  The K order inside a chunk is permuted identically for both
// operands, which leaves the contraction unchanged: MFMA step i of chunk c
// uses k = 64c + 32i + 8 (lane/16) + 0..7.  Groups with more than 16*TBN rows
// loop over row blocks.
// When the slabs alone are too few waves to keep the memory system busy (a
// shared expert: one group), K is split into nsplit parts (blockIdx.y): part
// p covers chunks [p nchunk / nsplit, (p + 1) nchunk / nsplit) and writes its
// fp32 sums (fused: gate columns [0, N), up columns [N, 2N)) to
// part[(p * part_rows + row) * cols + col]; skinny_reduce_kernel adds the
// parts in part order (and applies SiLU * up) afterwards.
// ---------------------------------------------------------------------------
constexpr int kSkinnyBatch = 4;   // 64-wide K chunks loaded per step
constexpr int kSkinnyWaves = 768;  // fewer waves cost latency, more cost partial-sum traffic (measured)
// Past about 12 waves per compute unit more waves gain nothing, and a longer
// wave amortizes its start and the last partial round of waves: a launch of
// more slabs gives each wave slabs / kSkinnyWavesMax consecutive slabs
// (measured on the decode shapes: 4 per wave for the down projection's 12288
// slabs, 2 for gate/up's 8192, 10% and 3% faster than one).
constexpr int kSkinnyWavesMax = 3072;

template <bool kFused, int TBN, typename OutT>
__global__ __launch_bounds__(64) void skinny_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows, int a_div,
    const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1, int64_t w_stride, int K,
    int N, const int32_t* __restrict__ off, int nslices, OutT* __restrict__ C,
    float* __restrict__ part, int part_rows, int spw) {
  constexpr int NBW = 4;                            // 16-row weight blocks per wave
  constexpr int NOUT = kFused ? 32 : 64;            // output columns per wave
  const int nsg = (nslices + spw - 1) / spw;  // wave = spw consecutive slabs of one group
  const int g = blockIdx.x / nsg;
  const int sg = blockIdx.x - g * nsg;
  const int r0 = off[g], r1 = off[g + 1];
  if (r0 >= r1) return;
  const int lane = threadIdx.x;
  const int l16 = lane & 15, kq = (lane >> 4) * 8;
  for (int slice = sg * spw; slice < nslices && slice < (sg + 1) * spw; ++slice) {
  const int n0 = slice * NOUT;

  const uint16_t* wrow[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const uint16_t* base = W0;
    int n = n0 + 16 * b + l16;
    if (kFused && b >= NBW / 2) {
      base = W1;
      n = n0 + 16 * (b - NBW / 2) + l16;
    }
    n = n < N ? n : N - 1;
    wrow[b] = base + static_cast<int64_t>(g) * w_stride + static_cast<int64_t>(n) * K + kq;
  }

  for (int rb = r0; rb < r1; rb += 16 * TBN) {
    const uint16_t* xrow[TBN];
#pragma unroll
    for (int tb = 0; tb < TBN; ++tb) {
      int r = rb + 16 * tb + l16;
      r = r < r1 ? r : r1 - 1;  // rows past the group: valid row, result unused
      const int64_t src = a_rows ? static_cast<int64_t>(a_rows[r] / a_div) : r;
      xrow[tb] = A + src * K + kq;
    }
    f32x4 acc[NBW][TBN];
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
      for (int tb = 0; tb < TBN; ++tb) acc[b][tb] = f32x4{};

    const int nchunk_all = K / 64;
    const int c_begin = static_cast<int>(blockIdx.y) * nchunk_all / static_cast<int>(gridDim.y);
    const int nchunk = (static_cast<int>(blockIdx.y) + 1) * nchunk_all / static_cast<int>(gridDim.y);
    int c = c_begin;
    // kSkinnyBatch chunks per step: all loads first, then the MFMAs
    for (; c + kSkinnyBatch <= nchunk; c += kSkinnyBatch) {
      bf16x8 wf[kSkinnyBatch][NBW][2], xf[kSkinnyBatch][TBN][2];
#pragma unroll
      for (int u = 0; u < kSkinnyBatch; ++u) {
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
          const bf16x8* p = reinterpret_cast<const bf16x8*>(wrow[b] + (c + u) * 64);
          wf[u][b][0] = p[0];
          wf[u][b][1] = p[4];
        }
#pragma unroll
        for (int tb = 0; tb < TBN; ++tb) {
          const bf16x8* p = reinterpret_cast<const bf16x8*>(xrow[tb] + (c + u) * 64);
          xf[u][tb][0] = p[0];
          xf[u][tb][1] = p[4];
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the whole batch of loads in flight
#pragma unroll
      for (int u = 0; u < kSkinnyBatch; ++u)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int tb = 0; tb < TBN; ++tb)
              acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u][b][i], xf[u][tb][i],
                                                                  acc[b][tb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (; c < nchunk; ++c) {
      bf16x8 wf[NBW][2], xf[TBN][2];
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        const bf16x8* p = reinterpret_cast<const bf16x8*>(wrow[b] + c * 64);
        wf[b][0] = p[0];
        wf[b][1] = p[4];
      }
#pragma unroll
      for (int tb = 0; tb < TBN; ++tb) {
        const bf16x8* p = reinterpret_cast<const bf16x8*>(xrow[tb] + c * 64);
        xf[tb][0] = p[0];
        xf[tb][1] = p[4];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
          for (int tb = 0; tb < TBN; ++tb)
            acc[b][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[b][i], xf[tb][i], acc[b][tb],
                                                                0, 0, 0);
    }

    // D[weight row][token]: lane holds token column l16 and weight rows 4*(lane/16)+j
    if (part) {  // fp32 partial sums of this K part, four consecutive columns per store
      const int cols = kFused ? 2 * N : N;
#pragma unroll
      for (int tb = 0; tb < TBN; ++tb) {
        const int row = rb + 16 * tb + l16;
        if (row >= r1) continue;
        float* prow = part + (static_cast<int64_t>(blockIdx.y) * part_rows + row) * cols;
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
          const int n = n0 + 16 * (kFused && b >= NBW / 2 ? b - NBW / 2 : b) + (lane >> 4) * 4;
          if (n >= N) continue;  // N % 4 == 0: a run of four is whole
          *reinterpret_cast<f32x4*>(prow + (kFused && b >= NBW / 2 ? N : 0) + n) = acc[b][tb];
        }
      }
      continue;
    }
#pragma unroll
    for (int tb = 0; tb < TBN; ++tb) {
      const int row = rb + 16 * tb + l16;
      if (row >= r1) continue;
      OutT* crow = C + static_cast<int64_t>(row) * N;
#pragma unroll
      for (int b = 0; b < (kFused ? NBW / 2 : NBW); ++b) {
        // four consecutive columns per lane, one store (N % 4 == 0 keeps the
        // run whole; the stores issue about one lane per cycle, whatever
        // their width)
        const int n = n0 + 16 * b + (lane >> 4) * 4;
        if (n >= N) continue;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = acc[b][tb][j];
          if constexpr (kFused) v[j] = silu_f32(v[j]) * acc[b + NBW / 2][tb][j];
        }
        if constexpr (sizeof(OutT) == 2)
          *reinterpret_cast<u32x2*>(crow + n) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        else
          *reinterpret_cast<f32x4*>(crow + n) = f32x4{v[0], v[1], v[2], v[3]};
      }
    }
  }
}  // slabs of this wave
}

// Adds the nsplit K parts of the skinny kernel in part order for rows below
// off[G]; each thread four consecutive columns of one row.  Fused: SiLU of the
// gate sum times the up sum.
template <bool kFused, typename OutT>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ part,
                                                            int nsplit, int part_rows,
                                                            const int32_t* __restrict__ off,
                                                            int G, int N,
                                                            OutT* __restrict__ C) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int q = N / 4;
  const int64_t row = i / q;
  const int col = static_cast<int>(i - row * q) * 4;
  if (row >= off[G]) return;
  const int cols = kFused ? 2 * N : N;
  f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f}, u = a;
  for (int p = 0; p < nsplit; ++p) {
    const float* src = part + (static_cast<int64_t>(p) * part_rows + row) * cols + col;
    a += *reinterpret_cast<const f32x4*>(src);
    if constexpr (kFused) u += *reinterpret_cast<const f32x4*>(src + N);
  }
  f32x4 v = a;
  if constexpr (kFused) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = silu_f32(a[e]) * u[e];
  }
  OutT* dst = C + row * N + col;
  if constexpr (sizeof(OutT) == 2) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else {
    *reinterpret_cast<f32x4*>(dst) = v;
  }
}

// ---------------------------------------------------------------------------
// fp32 FMA kernel: 64 x 64 output tile, K step 16, 4 x 4 outputs per thread.
// kFused computes gate and up accumulators for the same 64 hidden columns.
// ---------------------------------------------------------------------------
constexpr int kF32Tile = 64;
constexpr int kF32K = 16;

template <bool kFused>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ a_rows, int a_div,
    const float* __restrict__ B0, const float* __restrict__ B1, int64_t b_stride, int K, int N,
    const int32_t* __restrict__ off, const int32_t* __restrict__ mstart, int G, int ntn,
    void* __restrict__ Cv, bool out_bf16, float* __restrict__ uv) {
  Tile tile;
  if (!decode_tile(off, mstart, G, ntn, kF32Tile, kF32Tile, tile)) return;
  __shared__ float As[kF32K][kF32Tile + 1];
  __shared__ float Bg[kF32K][kF32Tile + 1];
  __shared__ float Bu[kFused ? kF32K : 1][kF32Tile + 1];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  float cg[4][4] = {}, cu[4][4] = {};
  const float* Bg0 = B0 + tile.g * b_stride;
  const float* Bu0 = kFused ? B1 + tile.g * b_stride : nullptr;
  for (int k0 = 0; k0 < K; k0 += kF32K) {
    for (int i = tid; i < kF32K * kF32Tile; i += kThreads) {
      const int r = i / kF32K, kk = i % kF32K;
      const int kg = k0 + kk;
      int row = tile.m0 + r;
      row = row < tile.row_end ? row : tile.row_end - 1;
      const int64_t src = a_rows ? static_cast<int64_t>(a_rows[row] / a_div) : row;
      As[kk][r] = kg < K ? A[src * K + kg] : 0.0f;
      int n = tile.n0 + r;
      n = n < N ? n : N - 1;
      Bg[kk][r] = kg < K ? Bg0[static_cast<int64_t>(n) * K + kg] : 0.0f;
      if constexpr (kFused) Bu[kk][r] = kg < K ? Bu0[static_cast<int64_t>(n) * K + kg] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32K; ++kk) {
      float a[4], bg[4], bu[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bg[j] = Bg[kk][tx * 4 + j];
        if constexpr (kFused) bu[j] = Bu[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cg[i][j] = fmaf(a[i], bg[j], cg[i][j]);
          if constexpr (kFused) cu[i][j] = fmaf(a[i], bu[j], cu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tile.m0 + ty * 4 + i;
    if (row >= tile.row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tile.n0 + tx * 4 + j;
      if (col >= N) continue;
      const float v = kFused ? silu_f32(cg[i][j]) * cu[i][j] : cg[i][j];
      const int64_t o = static_cast<int64_t>(row) * N + col;
      if (kFused && uv) {  // pre-activations for the backward pass, (u, v) pairs
        uv[2 * o] = cg[i][j];
        uv[2 * o + 1] = cu[i][j];
      }
      if (out_bf16) static_cast<uint16_t*>(Cv)[o] = f32_to_bf16_bits(v);
      else static_cast<float*>(Cv)[o] = v;
    }
  }
}

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

constexpr size_t kGemmLds = sizeof(uint16_t) * (kRingA * kTileM + kRingB * 256) * kBK;

// one workgroup per compute unit, kXcds at least (every run needs one)
unsigned persistent_grid(int ncu) {
  return static_cast<unsigned>(ncu >= kXcds ? ncu / kXcds * kXcds : kXcds);
}

// The grid of a persistent launch limited to max_cus workgroups (<= 0: no
// limit), so that a launch on another stream keeps the other compute units.
// Only the grid shrinks: the tile table, the XCD runs and the split-K plan
// still follow the device's compute-unit count, so every output tile is
// computed exactly as by the unlimited launch (the persistent workgroups take
// the same units in another interleaving).
unsigned limited_grid(int ncu, int max_cus) {
  return persistent_grid(max_cus > 0 && max_cus < ncu ? max_cus : ncu);
}

hipError_t gate_up_bf16(const SwigluArgs& s, hipStream_t stream) {
  const int ntn = (s.h + 127) / 128;
  const int ncu = compute_units();
  tile_table_kernel<<<1, 1024, 0, stream>>>(s.group_offset, s.G, kTileM, ntn, true, s.mstart,
                                            s.mstart, ncu, s.d / kBK, false);
  EpiArgs ep{};
  ep.uv = static_cast<uint16_t*>(s.uv);
  auto kern = s.uv ? gemm_bf16_kernel<true, uint16_t, kEpiSaveUV>
                   : gemm_bf16_kernel<true, uint16_t, kEpiNone>;
  ensure_dynamic_lds(reinterpret_cast<const void*>(kern), static_cast<int>(kGemmLds));
  kern<<<limited_grid(ncu, s.max_cus), kThreads, kGemmLds, stream>>>(
      static_cast<const uint16_t*>(s.a), s.a_rows, s.a_div, static_cast<const uint16_t*>(s.w_gate),
      static_cast<const uint16_t*>(s.w_up), static_cast<int64_t>(s.h) * s.d, s.d, s.h,
      s.group_offset, s.mstart, s.G, ntn, static_cast<uint16_t*>(s.hid), nullptr, ncu, ep,
      OpArgs{});
  return hipGetLastError();
}

template <typename OutT>
hipError_t down_bf16(const SwigluArgs& s, hipStream_t stream) {
  const int ntn = (s.d + 255) / 256;
  const int ncu = compute_units();
  tile_table_kernel<<<1, 1024, 0, stream>>>(s.group_offset, s.G, kTileM, ntn, false, s.mstart,
                                            s.mstart, ncu, s.h / kBK, s.sk_ws != nullptr);
  auto kern = gemm_bf16_kernel<false, OutT, kEpiNone>;
  ensure_dynamic_lds(reinterpret_cast<const void*>(kern), static_cast<int>(kGemmLds));
  kern<<<limited_grid(ncu, s.max_cus), kThreads, kGemmLds, stream>>>(
      static_cast<const uint16_t*>(s.hid), nullptr, 1, static_cast<const uint16_t*>(s.w_down),
      nullptr, static_cast<int64_t>(s.d) * s.h, s.h, s.d, s.group_offset, s.mstart, s.G, ntn,
      static_cast<OutT*>(s.y), s.sk_ws, ncu, EpiArgs{}, OpArgs{});
  if (s.sk_ws)
    sk_reduce_kernel<OutT><<<kSkUnits * 32, 256, 0, stream>>>(
        s.sk_ws, s.group_offset, s.mstart, s.G, ntn, s.h, s.d, ncu, static_cast<OutT*>(s.y));
  return hipGetLastError();
}

hipError_t gate_up_f32(const SwigluArgs& s, hipStream_t stream) {
  const int64_t mt_ub = (s.max_rows + kF32Tile - 1) / kF32Tile + s.G;
  const int ntn = static_cast<int>((s.h + kF32Tile - 1) / kF32Tile);
  tile_table_kernel<<<1, 1024, 0, stream>>>(s.group_offset, s.G, kF32Tile, 0, false, s.mstart,
                                            nullptr, 0, 0, false);
  gemm_f32_kernel<true><<<static_cast<unsigned>(round_up(mt_ub * ntn, 8)), kThreads, 0, stream>>>(
      static_cast<const float*>(s.a), s.a_rows, s.a_div, static_cast<const float*>(s.w_gate),
      static_cast<const float*>(s.w_up), static_cast<int64_t>(s.h) * s.d, s.d, s.h, s.group_offset,
      s.mstart, s.G, ntn, s.hid, false, static_cast<float*>(s.uv));
  return hipGetLastError();
}

hipError_t down_f32(const SwigluArgs& s, hipStream_t stream) {
  const int64_t mt_ub = (s.max_rows + kF32Tile - 1) / kF32Tile + s.G;
  const int ntn = static_cast<int>((s.d + kF32Tile - 1) / kF32Tile);
  tile_table_kernel<<<1, 1024, 0, stream>>>(s.group_offset, s.G, kF32Tile, 0, false, s.mstart,
                                            nullptr, 0, 0, false);
  gemm_f32_kernel<false><<<static_cast<unsigned>(round_up(mt_ub * ntn, 8)), kThreads, 0, stream>>>(
      static_cast<const float*>(s.hid), nullptr, 1, static_cast<const float*>(s.w_down), nullptr,
      static_cast<int64_t>(s.d) * s.h, s.h, s.d, s.group_offset, s.mstart, s.G, ntn, s.y,
      s.y_bf16, nullptr);
  return hipGetLastError();
}

template <bool kFused, typename OutT>
hipError_t skinny_bf16(const SwigluArgs& s, int K, int N, const void* a, const int32_t* a_rows,
                       int a_div, const void* w0, const void* w1, void* out, hipStream_t stream) {
  const int per_wave = kFused ? 32 : 64;
  const int nslices = (N + per_wave - 1) / per_wave;
  const int64_t waves = static_cast<int64_t>(s.G) * nslices;
  const int64_t mean = (s.max_rows + s.G - 1) / s.G;
  const int64_t wstride = static_cast<int64_t>(N) * K;
  // split K when the slabs are too few waves (at least kSkinnyBatch chunks
  // per part, partial sums within the split-K workspace)
  int nsplit = 1;
  if (s.sk_ws && waves < kSkinnyWaves) {
    const int64_t cols = kFused ? 2 * N : N;
    const int64_t cap = static_cast<int64_t>(split_k_workspace_bytes() / sizeof(float)) /
                        (s.max_rows * cols);
    int64_t want = (kSkinnyWaves + waves - 1) / waves;
    want = std::min<int64_t>(want, (K / 64) / kSkinnyBatch);
    want = std::min<int64_t>(want, cap);
    nsplit = static_cast<int>(std::max<int64_t>(want, 1));
  }
  float* part = nsplit > 1 ? s.sk_ws : nullptr;
  const int spw = nsplit > 1 ? 1 : static_cast<int>(std::max<int64_t>(1, waves / kSkinnyWavesMax));
  const dim3 grid(static_cast<unsigned>(s.G * ((nslices + spw - 1) / spw)),
                  static_cast<unsigned>(nsplit));
  const int part_rows = static_cast<int>(s.max_rows);
#define MOE_SKINNY(TBN)                                                                    \
  skinny_kernel<kFused, TBN, OutT><<<grid, 64, 0, stream>>>(                               \
      static_cast<const uint16_t*>(a), a_rows, a_div, static_cast<const uint16_t*>(w0),    \
      static_cast<const uint16_t*>(w1), wstride, K, N, s.group_offset, nslices,            \
      static_cast<OutT*>(out), part, part_rows, spw)
  if (mean <= 16) MOE_SKINNY(1);
  else if (mean <= 32) MOE_SKINNY(2);
  else MOE_SKINNY(4);
#undef MOE_SKINNY
  if (part) {
    const int64_t threads = s.max_rows * (N / 4);
    skinny_reduce_kernel<kFused, OutT><<<static_cast<unsigned>((threads + 255) / 256), 256, 0,
                                         stream>>>(part, nsplit, part_rows, s.group_offset, s.G,
                                                   N, static_cast<OutT*>(out));
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 backward GEMMs: 64 x 64 tiles of plain FMAs through LDS, K steps of 16.
//   f32_dgrad_kernel: for the rows of each group, C[r, n] = sum_k A[r, k] B(k, n)
//     with B read K-major, B(k, n) = B0[g][k][n] or, kInter, the rows
//     alternating between B0[g][k / 2] (even k) and B1[g][k / 2] (odd k);
//     kSilu: the SiLU-backward epilogue on the interleaved (u, v) -> (du, dv).
//   f32_wgrad_kernel: for each group g, C_g[m, n] = sum over its rows r of
//     A[r][m] B[row(r)][n], row(r) = b_rows[r] / b_div (or r); kPairs sends
//     the even rows of C_g to C and the odd rows to C_odd.
// ---------------------------------------------------------------------------
template <bool kInter, bool kSilu>
__global__ __launch_bounds__(kThreads) void f32_dgrad_kernel(
    const float* __restrict__ A, int K, const float* __restrict__ B0, const float* __restrict__ B1,
    int64_t b_stride, int N, const int32_t* __restrict__ off, const int32_t* __restrict__ mstart,
    int G, int ntn, float* __restrict__ C, const float* __restrict__ uv, float* __restrict__ dab) {
  Tile tile;
  if (!decode_tile(off, mstart, G, ntn, kF32Tile, kF32Tile, tile)) return;
  __shared__ float As[kF32K][kF32Tile + 1];
  __shared__ float Bs[kF32K][kF32Tile + 1];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  const float* b0 = B0 + tile.g * b_stride;
  const float* b1 = kInter ? B1 + tile.g * b_stride : b0;
  for (int k0 = 0; k0 < K; k0 += kF32K) {
    for (int i = tid; i < kF32K * kF32Tile; i += kThreads) {
      const int r = i / kF32K, kk = i % kF32K;
      const int kg = k0 + kk;
      int row = tile.m0 + r;
      row = row < tile.row_end ? row : tile.row_end - 1;
      As[kk][r] = kg < K ? A[static_cast<int64_t>(row) * K + kg] : 0.0f;
      const int kb = i / kF32Tile, c = i % kF32Tile;  // B: consecutive threads along n
      const int kgb = k0 + kb;
      int n = tile.n0 + c;
      n = n < N ? n : N - 1;
      float bv = 0.0f;
      if (kgb < K) {
        if constexpr (kInter) bv = ((kgb & 1) ? b1 : b0)[static_cast<int64_t>(kgb >> 1) * N + n];
        else bv = b0[static_cast<int64_t>(kgb) * N + n];
      }
      Bs[kb][c] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32K; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tile.m0 + ty * 4 + i;
    if (row >= tile.row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tile.n0 + tx * 4 + j;
      if (col >= N) continue;
      const int64_t o = static_cast<int64_t>(row) * N + col;
      if constexpr (kSilu) {
        const float u = uv[2 * o], v = uv[2 * o + 1];
        const float sg = 1.0f / (1.0f + expf(-u));
        dab[2 * o] = acc[i][j] * v * (sg * (1.0f + u * (1.0f - sg)));
        dab[2 * o + 1] = acc[i][j] * (u * sg);
      } else {
        C[o] = acc[i][j];
      }
    }
  }
}

template <bool kPairs>
__global__ __launch_bounds__(kThreads) void f32_wgrad_kernel(
    const float* __restrict__ A, int lda, const float* __restrict__ B, int ldb,
    const int32_t* __restrict__ b_rows, int b_div, int M, int N,
    const int32_t* __restrict__ off, int mtn, int ntn, float* __restrict__ C,
    float* __restrict__ C_odd) {
  const int per = mtn * ntn;
  const int g = blockIdx.x / per;
  const int local = blockIdx.x - g * per;
  const int m0 = (local / ntn) * kF32Tile, n0 = (local % ntn) * kF32Tile;
  const int r0 = off[g], r1 = off[g + 1];
  __shared__ float As[kF32K][kF32Tile + 1];
  __shared__ float Bs[kF32K][kF32Tile + 1];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = r0; k0 < r1; k0 += kF32K) {
    for (int i = tid; i < kF32K * kF32Tile; i += kThreads) {
      const int kk = i / kF32Tile, c = i % kF32Tile;
      const int r = k0 + kk;
      const bool in = r < r1;
      const int64_t br = in ? (b_rows ? b_rows[r] / b_div : r) : 0;
      As[kk][c] = (in && m0 + c < M) ? A[static_cast<int64_t>(r) * lda + m0 + c] : 0.0f;
      Bs[kk][c] = (in && n0 + c < N) ? B[br * ldb + n0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32K; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int64_t gsz = static_cast<int64_t>(kPairs ? M / 2 : M) * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    float* crow = kPairs ? (m & 1 ? C_odd : C) + g * gsz + static_cast<int64_t>(m >> 1) * N
                         : C + g * gsz + static_cast<int64_t>(m) * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) crow[n] = acc[i][j];
    }
  }
}

// Groups averaging at most 64 rows stream weights through the skinny kernel;
// the others run the tiled MFMA kernel.
bool skinny(const SwigluArgs& s) { return s.max_rows <= static_cast<int64_t>(s.G) * 64; }

// ---------------------------------------------------------------------------
// Backward pass of the experts (bf16).  With dout_r the upstream gradient of
// row r's expert output (the gate already applied), per group g:
//   dhid = dout W_down[g]                           (dgrad 1, K = d, N = h)
//   du = dhid v SiLU'(u),  dv = dhid SiLU(u)        (its epilogue)
//   da = du W_gate[g] + dv W_up[g]                  (dgrad 2, K = 2h, N = d)
//   dW_down[g] = sum_r dout_r^T hid_r               (weight gradients, K = rows)
//   dW_gate[g] = sum_r du_r^T a_r,  dW_up[g] = sum_r dv_r^T a_r
// The input-gradient GEMMs contract over the weights' leading axis: they read
// the forward's weights K-major (kOpSlabT, W_gate's slab for the first h/64
// slices of dgrad 2 and W_up's after).  The weight gradients contract over a
// group's rows: both operands are read K-major from the row-major buffers
// (kOpRowsT), so no operand is ever transposed in memory.
// ---------------------------------------------------------------------------

// xs[r] = a[a_rows[r] / a_div] for r < off[G]: 16-byte copies, one row per
// workgroup pass.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ a,
                                                          const int32_t* __restrict__ a_rows,
                                                          int a_div,
                                                          const int32_t* __restrict__ off, int G,
                                                          int d, uint16_t* __restrict__ xs) {
  const int rows = off[G];
  const int per = d / 8;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
       i < static_cast<int64_t>(rows) * per; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / per;
    const int c = static_cast<int>(i - r * per) * 8;
    const int64_t sr = a_rows[r] / a_div;
    *reinterpret_cast<u32x4*>(xs + r * d + c) = *reinterpret_cast<const u32x4*>(a + sr * d + c);
  }
}

// Weight gradients: for every group g, C_g[M, N] = sum over the group's rows r
// of A[r, :M]^T B[r, :N] (fp32, at C + g M N), A and B row-major with rows of
// lda and ldb elements; with kPairs the even rows of C_g go to C and the odd
// rows to C_odd (M / 2 rows each, at g M N / 2).  One workgroup per output tile (tiles of a group in
// the banded order, groups in order, contiguous runs per XCD); a group
// without rows gets zeros.
template <bool kPairs>
__global__ __launch_bounds__(kThreads) void wgrad_bf16_kernel(
    const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ B, int ldb, int M,
    int N, const int32_t* __restrict__ off, int G, int mtn, int ntn,
    const uint16_t* __restrict__ zero, float* __restrict__ C, float* __restrict__ C_odd) {
  extern __shared__ __align__(16) uint16_t smem[];
  const int per = mtn * ntn, total = G * per, nw8 = (total + 7) & ~7;
  const int L = xcd_run(blockIdx.x, nw8);
  if (L >= total) return;
  const int g = L / per;
  int local = L - g * per;
  const int lead = band_lead(mtn);
  int nt, mt;
  if (local < lead * ntn) {
    const int band = local / (kBand * ntn), i = local - band * (kBand * ntn);
    nt = i / kBand;
    mt = band * kBand + (i - nt * kBand);
  } else {
    local -= lead * ntn;
    const int mtail = mtn - lead;
    nt = local / mtail;
    mt = lead + (local - nt * mtail);
  }
  const Tile2 tile = classify(Tile{0, mt * kTileM, M, nt * 256});
  // this group's output (row pairs: M / 2 rows in each of C and C_odd)
  const int64_t gsz = static_cast<int64_t>(kPairs ? M / 2 : M) * N;
  float* Cg = C + g * gsz;
  EpiArgs ep{};
  ep.c_odd = kPairs ? C_odd + g * gsz : nullptr;
  const int r0 = off[g], r1 = off[g + 1];
  const int nk = (r1 - r0 + kBK - 1) / kBK;
  if (nk == 0) {
    const int rows = min(kTileM, M - tile.m0);
    for (int i = threadIdx.x; i < rows * 64; i += kThreads) {
      const int r = tile.m0 + i / 64, c = tile.n0 + (i % 64) * 4;
      if (c >= N) continue;
      float* dst = kPairs ? (r & 1 ? ep.c_odd : Cg) + static_cast<int64_t>(r >> 1) * N
                          : Cg + static_cast<int64_t>(r) * N;
      *reinterpret_cast<f32x4*>(dst + c) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    return;
  }
  OpArgs oa{};
  oa.r0 = r0;
  oa.rend = r1;
  oa.lda = lda;
  oa.ldb = ldb;
  oa.a_cols = M;
  oa.zero = zero;
  if (tile.cls == 0)
    gemm_tile<256, 2, 2, 256, kRingA, kRingB, false, float, kPairs ? kEpiRowPairs : kEpiNone, kOpRowsT,
              kOpRowsT>(
        A, nullptr, 1, B, nullptr, 0, 0, N, tile, 0, nk, smem, Cg, nullptr, ep, oa);
  else if (tile.cls == 1)
    gemm_tile<128, 1, 4, 256, kRingA, kRingB, false, float, kPairs ? kEpiRowPairs : kEpiNone, kOpRowsT,
              kOpRowsT>(
        A, nullptr, 1, B, nullptr, 0, 0, N, tile, 0, nk, smem, Cg, nullptr, ep, oa);
  else
    gemm_tile<64, 1, 4, 256, kRingA, kRingB, false, float, kPairs ? kEpiRowPairs : kEpiNone, kOpRowsT,
              kOpRowsT>(
        A, nullptr, 1, B, nullptr, 0, 0, N, tile, 0, nk, smem, Cg, nullptr, ep, oa);
}

hipError_t wgrad_bf16(const uint16_t* A, int lda, const uint16_t* B, int ldb, int M, int N,
                      const int32_t* off, int G, const uint16_t* zero, float* C, float* C_odd,
                      hipStream_t stream) {
  const int mtn = (M + kTileM - 1) / kTileM, ntn = (N + 255) / 256;
  const int64_t total = static_cast<int64_t>(G) * mtn * ntn;
  auto kern = C_odd ? wgrad_bf16_kernel<true> : wgrad_bf16_kernel<false>;
  ensure_dynamic_lds(reinterpret_cast<const void*>(kern), static_cast<int>(kGemmLds));
  kern<<<static_cast<unsigned>((total + 7) & ~7), kThreads, kGemmLds, stream>>>(
      A, lda, B, ldb, M, N, off, G, mtn, ntn, zero, C, C_odd);
  return hipGetLastError();
}

// Input-gradient GEMM: C[r] = A[r] . W[g] for the rows of each group, W read
// K-major (kBM = kOpSlabT: one slab [K][N] per group; kOpSlabI: the K rows
// alternate between B0's and B1's slabs), persistent like the forward's down
// projection (split-K of the last round when skw is given).
template <int kEpi, int kBM, typename OutT>
hipError_t dgrad_bf16(const uint16_t* A, int K, int N, const uint16_t* B0, const uint16_t* B1,
                      int64_t b_stride, const int32_t* off, int G, int32_t* tt, OutT* C,
                      float* skw, const EpiArgs& ep, hipStream_t stream) {
  const int ntn = (N + 255) / 256;
  const int ncu = compute_units();
  tile_table_kernel<<<1, 1024, 0, stream>>>(off, G, kTileM, ntn, false, tt, tt, ncu, K / kBK,
                                            skw != nullptr);
  auto kern = gemm_bf16_kernel<false, OutT, kEpi, kBM>;
  ensure_dynamic_lds(reinterpret_cast<const void*>(kern), static_cast<int>(kGemmLds));
  kern<<<persistent_grid(ncu), kThreads, kGemmLds, stream>>>(A, nullptr, 1, B0, B1, b_stride, K,
                                                              N, off, tt, G, ntn, C, skw, ncu, ep,
                                                              OpArgs{});
  if (skw)
    sk_reduce_kernel<OutT><<<kSkUnits * 32, 256, 0, stream>>>(skw, off, tt, G, ntn, K, N, ncu, C);
  return hipGetLastError();
}

}  // namespace

size_t tile_table_bytes(int G) { return sizeof(int32_t) * static_cast<size_t>(tt_entries(G)); }

size_t split_k_workspace_bytes() {
  return sizeof(float) * static_cast<size_t>(kSkUnits) * kTileM * 256;
}

hipError_t launch_gate_up(const SwigluArgs& s, hipStream_t stream) {
  if (!s.bf16) return gate_up_f32(s, stream);
  if (skinny(s) && !s.uv)
    return skinny_bf16<true, uint16_t>(s, s.d, s.h, s.a, s.a_rows, s.a_div, s.w_gate, s.w_up,
                                       s.hid, stream);
  return gate_up_bf16(s, stream);
}

hipError_t launch_down(const SwigluArgs& s, hipStream_t stream) {
  if (!s.bf16) return down_f32(s, stream);
  if (skinny(s)) {
    if (s.y_bf16)
      return skinny_bf16<false, uint16_t>(s, s.h, s.d, s.hid, nullptr, 1, s.w_down, nullptr, s.y,
                                          stream);
    return skinny_bf16<false, float>(s, s.h, s.d, s.hid, nullptr, 1, s.w_down, nullptr, s.y,
                                     stream);
  }
  return s.y_bf16 ? down_bf16<uint16_t>(s, stream) : down_bf16<float>(s, stream);
}

hipError_t launch_expert_backward_f32(const SwigluBwdArgs& b, hipStream_t stream) {
  const int d = b.d, h = b.h, G = b.G;
  const auto* a = static_cast<const float*>(b.a);
  const auto* dout = static_cast<const float*>(b.dout);
  const auto* hid = static_cast<const float*>(b.hid);
  const auto* uv = static_cast<const float*>(b.uv);
  const auto* wg = static_cast<const float*>(b.w_gate);
  const auto* wu = static_cast<const float*>(b.w_up);
  const auto* wd = static_cast<const float*>(b.w_down);
  float* dab = reinterpret_cast<float*>(b.dab);
  if (b.max_rows > 0) {
    const int64_t mt_ub = (b.max_rows + kF32Tile - 1) / kF32Tile + G;
    tile_table_kernel<<<1, 1024, 0, stream>>>(b.group_offset, G, kF32Tile, 0, false, b.mstart,
                                              nullptr, 0, 0, false);
    // dgrad 1 (W_down read K-major) with the SiLU backward epilogue
    const int ntn1 = (h + kF32Tile - 1) / kF32Tile;
    f32_dgrad_kernel<false, true>
        <<<static_cast<unsigned>(round_up(mt_ub * ntn1, 8)), kThreads, 0, stream>>>(
            dout, d, wd, wd, static_cast<int64_t>(d) * h, h, b.group_offset, b.mstart, G, ntn1,
            nullptr, uv, dab);
    // dgrad 2 over the interleaved (du, dv) and the alternating gate/up rows
    const int ntn2 = (d + kF32Tile - 1) / kF32Tile;
    f32_dgrad_kernel<true, false>
        <<<static_cast<unsigned>(round_up(mt_ub * ntn2, 8)), kThreads, 0, stream>>>(
            dab, 2 * h, wg, wu, static_cast<int64_t>(h) * d, d, b.group_offset, b.mstart, G, ntn2,
            b.da, nullptr, nullptr);
  }
  // weight gradients over each group's rows
  {
    const int mtn = (d + kF32Tile - 1) / kF32Tile, ntn = (h + kF32Tile - 1) / kF32Tile;
    f32_wgrad_kernel<false><<<static_cast<unsigned>(G * mtn * ntn), kThreads, 0, stream>>>(
        dout, d, hid, h, nullptr, 1, d, h, b.group_offset, mtn, ntn, b.dw_down, nullptr);
  }
  {
    const int mtn = (2 * h + kF32Tile - 1) / kF32Tile, ntn = (d + kF32Tile - 1) / kF32Tile;
    f32_wgrad_kernel<true><<<static_cast<unsigned>(G * mtn * ntn), kThreads, 0, stream>>>(
        dab, 2 * h, a, d, b.a_rows, b.a_div, 2 * h, d, b.group_offset, mtn, ntn, b.dw_gate,
        b.dw_up);
  }
  return hipGetLastError();
}

hipError_t launch_expert_backward(const SwigluBwdArgs& b, hipStream_t stream) {
  if (!b.bf16) return launch_expert_backward_f32(b, stream);
  const int d = b.d, h = b.h, G = b.G;
  const auto* a = static_cast<const uint16_t*>(b.a);
  const auto* dout = static_cast<const uint16_t*>(b.dout);
  const auto* hid = static_cast<const uint16_t*>(b.hid);
  const auto* wg = static_cast<const uint16_t*>(b.w_gate);
  const auto* wu = static_cast<const uint16_t*>(b.w_up);
  const auto* wd = static_cast<const uint16_t*>(b.w_down);
  // a row of zeros (max(d, 2h) bf16) for the K tails of the weight gradients
  hipError_t e = launch_fill_i32(reinterpret_cast<int32_t*>(b.zero), std::max(d, 2 * h) / 2, 0,
                                 stream);
  if (e != hipSuccess) return e;
  const uint16_t* xs = a;
  if (b.a_rows && b.max_rows > 0) {
    const int64_t n = b.max_rows * (d / 8);
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 16384));
    gather_rows_kernel<<<grid, 256, 0, stream>>>(a, b.a_rows, b.a_div, b.group_offset, G, d,
                                                 b.xs);
    xs = b.xs;
  }
  if (b.max_rows > 0) {
    // dgrad 1 (dhid = dout W_down, K-major W_down) with the SiLU backward epilogue
    EpiArgs ep{};
    ep.uv = const_cast<uint16_t*>(static_cast<const uint16_t*>(b.uv));
    ep.dab = static_cast<uint16_t*>(b.dab);
    e = dgrad_bf16<kEpiSiluBwd, kOpSlabT, uint16_t>(dout, d, h, wd, wd,
                                                    static_cast<int64_t>(d) * h, b.group_offset,
                                                    G, b.mstart, nullptr, nullptr, ep, stream);
    if (e != hipSuccess) return e;
    // dgrad 2: da = du W_gate + dv W_up, K = 2h over the interleaved (du, dv)
    // columns and the two K-major slabs
    e = dgrad_bf16<kEpiNone, kOpSlabI, float>(static_cast<const uint16_t*>(b.dab), 2 * h, d, wg, wu,
                                              static_cast<int64_t>(h) * d, b.group_offset, G,
                                              b.mstart, b.da, b.sk_ws, EpiArgs{}, stream);
    if (e != hipSuccess) return e;
  }
  // weight gradients: dW_down, then dW_gate and dW_up as one GEMM over the
  // interleaved (du, dv) columns (even output rows to dW_gate, odd to dW_up)
  e = wgrad_bf16(dout, d, hid, h, d, h, b.group_offset, G, b.zero, b.dw_down, nullptr, stream);
  if (e == hipSuccess)
    e = wgrad_bf16(static_cast<const uint16_t*>(b.dab), 2 * h, xs, d, 2 * h, d, b.group_offset, G, b.zero, b.dw_gate, b.dw_up,
                   stream);
  return e;
}

}  // namespace moe
