// Grouped SwiGLU experts: for every group g (an expert) and every row r of
// that group,  hid = SiLU(a_r W_gate[g]^T) * (a_r W_up[g]^T),  y_r = hid W_down[g]^T.
//
// Source: "Zen-Max: Maximum Capability via Mixture-of-Experts Architecture",
// section "Fine-Grained Expert Architecture", expert equation
// (SiLU(x W_gate) * x W_up) W_down, weights stored transposed so that every
// operand is contiguous along its reduction axis.
//
// bf16 path (gfx950 MFMA, fp32 accumulation):
//   GEMM 1 (gate || up, fused SiLU*mul): one B tile holds BN/2 gate rows and
//     the BN/2 up rows of the same hidden columns, so each wave owns matching
//     gate and up accumulators and the epilogue writes hid directly (bf16).
//   GEMM 2 (down): y = hid W_down^T.
//   Block tile BM x BN x 64, 4 waves in a 2 x 2 grid, each wave a
//   (BM/2) x (BN/2) grid of v_mfma_f32_32x32x16_bf16 tiles.  A and B tiles are
//   staged through LDS, double-buffered, with the next K slice prefetched into
//   registers while the current one feeds the matrix cores.  LDS rows are 128
//   bytes (8 chunks of 16 bytes); chunk c of row r is stored at c ^ (r & 7), so
//   both the 16-byte stores and the 16-byte fragment reads are conflict-free.
//   Tiles are ordered group-major, n-tile next, m-tile fastest, and spread in
//   contiguous runs over the 8 XCDs so that tiles that share a weight panel
//   or an activation panel run together on one XCD's L2.
// fp32 path: a plain LDS-tiled FMA kernel with the same tile order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kBK = 64;
constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Tile table: mstart[g] = sum over g' < g of ceil(rows_g' / BM), g = 0..G.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ off, int G,
                                                          int BM, int32_t* __restrict__ mstart) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < G; base += 1024) {
    const int g = base + tid;
    const int rows = g < G ? off[g + 1] - off[g] : 0;
    const int v = (rows + BM - 1) / BM;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int n = __shfl_up(incl, o);
      if (lane >= o) incl += n;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int pre = carry;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    if (g < G) mstart[g] = pre + incl - v;
    __syncthreads();
    if (tid == 1023) carry = pre + incl;
    __syncthreads();
  }
  if (tid == 0) mstart[G] = carry;
}

struct Tile {
  int g, m0, row_end, n0;
};

// Logical tile of this workgroup, or false if it has none.
__device__ __forceinline__ bool decode_tile(const int32_t* __restrict__ off,
                                            const int32_t* __restrict__ mstart, int G, int ntn,
                                            int BM, int ncol, Tile& tile) {
  const int total = mstart[G] * ntn;
  const int nw8 = (total + 7) & ~7;
  const int bid = blockIdx.x;
  if (bid >= nw8) return false;
  const int L = (bid & 7) * (nw8 >> 3) + (bid >> 3);  // contiguous runs per XCD
  if (L >= total) return false;
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mstart[mid] * ntn <= L) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int mtg = mstart[g + 1] - mstart[g];
  const int local = L - mstart[g] * ntn;
  const int nt = local / mtg, mt = local - nt * mtg;
  tile.g = g;
  tile.m0 = off[g] + mt * BM;
  tile.row_end = off[g + 1];
  tile.n0 = nt * ncol;
  return true;
}

__device__ __forceinline__ int swz(int row, int chunk) {  // element offset in a 64-wide LDS row
  return row * kBK + ((chunk ^ (row & 7)) << 3);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  kFused: B rows [0, BN/2) are W_gate rows n0.., rows
// [BN/2, BN) are W_up rows n0..; output columns n0 .. n0 + BN/2 of hid.
// Otherwise B rows are W rows n0 .. n0 + BN and the output is A W^T.
// ---------------------------------------------------------------------------
template <int BM, int BN, bool kFused, typename OutT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows, int a_div,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, int64_t b_stride, int K,
    int N, const int32_t* __restrict__ off, const int32_t* __restrict__ mstart, int G, int ntn,
    OutT* __restrict__ C) {
  constexpr int NCOL = kFused ? BN / 2 : BN;  // output columns per tile
  constexpr int MT = BM / 64;                 // 32-row MFMA tiles per wave
  constexpr int NT = BN / 64;                 // 32-col MFMA tiles per wave
  constexpr int AP = BM / 32;                 // A rows loaded per thread per K slice
  constexpr int BP = BN / 32;
  static_assert(!kFused || NT % 2 == 0, "fused tile needs matching gate/up halves");

  Tile tile;
  if (!decode_tile(off, mstart, G, ntn, BM, NCOL, tile)) return;

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;                     // [2][BM * 64]
  uint16_t* Bs = smem + 2 * BM * kBK;      // [2][BN * 64]

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  const int lrow = tid >> 3, lchunk = tid & 7;

  // per-thread source rows of the A and B tiles
  const uint16_t* ap[AP];
#pragma unroll
  for (int j = 0; j < AP; ++j) {
    int r = tile.m0 + lrow + 32 * j;
    r = r < tile.row_end ? r : tile.row_end - 1;  // rows past the group: valid row, result unused
    const int64_t src = a_rows ? static_cast<int64_t>(a_rows[r] / a_div) : r;
    ap[j] = A + src * K + lchunk * 8;
  }
  const uint16_t* bp[BP];
#pragma unroll
  for (int j = 0; j < BP; ++j) {
    const int r = lrow + 32 * j;
    const uint16_t* base = B0;
    int n = tile.n0 + r;
    if (kFused && r >= BN / 2) {
      base = B1;
      n = tile.n0 + r - BN / 2;
    }
    n = n < N ? n : N - 1;
    bp[j] = base + tile.g * b_stride + static_cast<int64_t>(n) * K + lchunk * 8;
  }

  u32x4 ra[AP], rb[BP];
#define MOE_LOAD_GLOBAL(k0)                                                          \
  do {                                                                               \
    _Pragma("unroll") for (int j = 0; j < AP; ++j)                                   \
        ra[j] = *reinterpret_cast<const u32x4*>(ap[j] + (k0));                       \
    _Pragma("unroll") for (int j = 0; j < BP; ++j)                                   \
        rb[j] = *reinterpret_cast<const u32x4*>(bp[j] + (k0));                       \
  } while (0)
#define MOE_STORE_LDS(buf)                                                           \
  do {                                                                               \
    uint16_t* as_ = As + (buf) * BM * kBK;                                           \
    uint16_t* bs_ = Bs + (buf) * BN * kBK;                                           \
    _Pragma("unroll") for (int j = 0; j < AP; ++j)                                   \
        *reinterpret_cast<u32x4*>(as_ + swz(lrow + 32 * j, lchunk)) = ra[j];         \
    _Pragma("unroll") for (int j = 0; j < BP; ++j)                                   \
        *reinterpret_cast<u32x4*>(bs_ + swz(lrow + 32 * j, lchunk)) = rb[j];         \
  } while (0)

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

  // rows of this wave's fragments inside the tiles
  int arow[MT], brow[NT];
#pragma unroll
  for (int i = 0; i < MT; ++i) arow[i] = wm * (BM / 2) + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (kFused) {
      brow[j] = (j < NT / 2) ? wn * (BN / 4) + j * 32 : BN / 2 + wn * (BN / 4) + (j - NT / 2) * 32;
    } else {
      brow[j] = wn * (BN / 2) + j * 32;
    }
    brow[j] += lane & 31;
  }
  const int khalf = lane >> 5;

  const int nk = K / kBK;
  MOE_LOAD_GLOBAL(0);
  MOE_STORE_LDS(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) MOE_LOAD_GLOBAL((kt + 1) * kBK);
    const uint16_t* as = As + cur * BM * kBK;
    const uint16_t* bs = Bs + cur * BN * kBK;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + khalf;
      bf16x8 af[MT], bfr[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i) af[i] = *reinterpret_cast<const bf16x8*>(as + swz(arow[i], c));
#pragma unroll
      for (int j = 0; j < NT; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(bs + swz(brow[j], c));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) MOE_STORE_LDS(cur ^ 1);
    __syncthreads();
  }
#undef MOE_LOAD_GLOBAL
#undef MOE_STORE_LDS

  // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
  const int rbase = tile.m0 + wm * (BM / 2) + (lane >> 5) * 4;
  if constexpr (kFused) {
#pragma unroll
    for (int j = 0; j < NT / 2; ++j) {
      const int col = tile.n0 + wn * (BN / 4) + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + i * 32 + (r >> 2) * 8 + (r & 3);
          if (row < tile.row_end) {
            const float v = silu_f32(acc[i][j][r]) * acc[i][j + NT / 2][r];
            C[static_cast<int64_t>(row) * N + col] = static_cast<OutT>(f32_to_bf16_bits(v));
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int col = tile.n0 + wn * (BN / 2) + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + i * 32 + (r >> 2) * 8 + (r & 3);
          if (row < tile.row_end) {
            const float v = acc[i][j][r];
            if constexpr (sizeof(OutT) == 2) {
              C[static_cast<int64_t>(row) * N + col] = f32_to_bf16_bits(v);
            } else {
              C[static_cast<int64_t>(row) * N + col] = v;
            }
          }
        }
    }
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
    void* __restrict__ Cv, bool out_bf16) {
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
      if (out_bf16) static_cast<uint16_t*>(Cv)[o] = f32_to_bf16_bits(v);
      else static_cast<float*>(Cv)[o] = v;
    }
  }
}

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

template <int BM, int BN>
hipError_t gate_up_bf16(const SwigluArgs& s, hipStream_t stream) {
  const int64_t mt_ub = (s.max_rows + BM - 1) / BM + s.G;
  const int ntn = static_cast<int>((s.h + BN / 2 - 1) / (BN / 2));
  const size_t lds = sizeof(uint16_t) * 2 * (BM + BN) * kBK;
  tile_table_kernel<<<1, 1024, 0, stream>>>(s.group_offset, s.G, BM, s.mstart);
  auto kern = gemm_bf16_kernel<BM, BN, true, uint16_t>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  kern<<<static_cast<unsigned>(round_up(mt_ub * ntn, 8)), kThreads, lds, stream>>>(
      static_cast<const uint16_t*>(s.a), s.a_rows, s.a_div, static_cast<const uint16_t*>(s.w_gate),
      static_cast<const uint16_t*>(s.w_up), static_cast<int64_t>(s.h) * s.d, s.d, s.h,
      s.group_offset, s.mstart, s.G, ntn, static_cast<uint16_t*>(s.hid));
  return hipGetLastError();
}

template <int BM, int BN, typename OutT>
hipError_t down_bf16(const SwigluArgs& s, hipStream_t stream) {
  const int64_t mt_ub = (s.max_rows + BM - 1) / BM + s.G;
  const int ntn = static_cast<int>((s.d + BN - 1) / BN);
  const size_t lds = sizeof(uint16_t) * 2 * (BM + BN) * kBK;
  tile_table_kernel<<<1, 1024, 0, stream>>>(s.group_offset, s.G, BM, s.mstart);
  auto kern = gemm_bf16_kernel<BM, BN, false, OutT>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  kern<<<static_cast<unsigned>(round_up(mt_ub * ntn, 8)), kThreads, lds, stream>>>(
      static_cast<const uint16_t*>(s.hid), nullptr, 1, static_cast<const uint16_t*>(s.w_down),
      nullptr, static_cast<int64_t>(s.d) * s.h, s.h, s.d, s.group_offset, s.mstart, s.G, ntn,
      static_cast<OutT*>(s.y));
  return hipGetLastError();
}

hipError_t gate_up_f32(const SwigluArgs& s, hipStream_t stream) {
  const int64_t mt_ub = (s.max_rows + kF32Tile - 1) / kF32Tile + s.G;
  const int ntn = static_cast<int>((s.h + kF32Tile - 1) / kF32Tile);
  tile_table_kernel<<<1, 1024, 0, stream>>>(s.group_offset, s.G, kF32Tile, s.mstart);
  gemm_f32_kernel<true><<<static_cast<unsigned>(round_up(mt_ub * ntn, 8)), kThreads, 0, stream>>>(
      static_cast<const float*>(s.a), s.a_rows, s.a_div, static_cast<const float*>(s.w_gate),
      static_cast<const float*>(s.w_up), static_cast<int64_t>(s.h) * s.d, s.d, s.h, s.group_offset,
      s.mstart, s.G, ntn, s.hid, false);
  return hipGetLastError();
}

hipError_t down_f32(const SwigluArgs& s, hipStream_t stream) {
  const int64_t mt_ub = (s.max_rows + kF32Tile - 1) / kF32Tile + s.G;
  const int ntn = static_cast<int>((s.d + kF32Tile - 1) / kF32Tile);
  tile_table_kernel<<<1, 1024, 0, stream>>>(s.group_offset, s.G, kF32Tile, s.mstart);
  gemm_f32_kernel<false><<<static_cast<unsigned>(round_up(mt_ub * ntn, 8)), kThreads, 0, stream>>>(
      static_cast<const float*>(s.hid), nullptr, 1, static_cast<const float*>(s.w_down), nullptr,
      static_cast<int64_t>(s.d) * s.h, s.h, s.d, s.group_offset, s.mstart, s.G, ntn, s.y,
      s.y_bf16);
  return hipGetLastError();
}

// Large tiles once groups average at least 384 rows; otherwise 128 x 128.
bool big_tiles(const SwigluArgs& s) { return s.max_rows >= static_cast<int64_t>(s.G) * 384; }

}  // namespace

hipError_t launch_gate_up(const SwigluArgs& s, hipStream_t stream) {
  if (!s.bf16) return gate_up_f32(s, stream);
  return big_tiles(s) ? gate_up_bf16<256, 256>(s, stream) : gate_up_bf16<128, 128>(s, stream);
}

hipError_t launch_down(const SwigluArgs& s, hipStream_t stream) {
  if (!s.bf16) return down_f32(s, stream);
  if (s.y_bf16)
    return big_tiles(s) ? down_bf16<256, 256, uint16_t>(s, stream)
                        : down_bf16<128, 128, uint16_t>(s, stream);
  return big_tiles(s) ? down_bf16<256, 256, float>(s, stream)
                      : down_bf16<128, 128, float>(s, stream);
}

}  // namespace moe
