// Dispatch: group routed pairs by expert in token order, apply the capacity
// drop, build the permutation and gather token rows into expert order.
//
// Sources: "Every parameter, every token", sections "A budget" (pairs past an
// expert's budget are dropped) and "What you still pay for" (each token
// travels to the expert it was assigned).  Reading: an expert keeps its first
// `capacity` pairs in token order.
//
// Integer-only and deterministic without atomics deciding any order:
//   1. rank:    each 1024-pair chunk (4 waves x 256 pairs) computes, for every
//               pair, its rank among earlier pairs of the same expert inside the
//               chunk (wave-level match via ballots, then a wave prefix), and
//               the chunk's per-expert histogram;
//   2. scan:    one workgroup turns the histograms into per-chunk exclusive
//               bases (column scan), counts, kept = min(count, C) and offsets;
//   3. scatter: pair_row / row_pair from base + local rank;
//   4. gather:  x rows into x_perm, one wave per row, 16-byte accesses.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kChunk = 1024;          // pairs per rank/scatter workgroup
constexpr int kRankThreads = 256;     // 4 waves x 256 pairs, 4 sub-steps of 64
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kRankThreads) void rank_kernel(const int32_t* __restrict__ idx,
                                                            int64_t R, int E,
                                                            int32_t* __restrict__ local_rank,
                                                            int32_t* __restrict__ hist) {
  __shared__ int cnt[4][kMaxExperts];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  for (int i = tid; i < 4 * kMaxExperts; i += kRankThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();

  const int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk + wave * 256;
  int my_e[4], my_r[4];
  const uint64_t lt = lanemask_lt();
  const int ebits = E > 1 ? 32 - __builtin_clz(static_cast<unsigned>(E - 1)) : 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t p = base + s * 64 + lane;
    // a slot whose expert lies outside [0, E) (an empty slot of ReLU routing)
    // is not routed
    const int e_raw = p < R ? idx[p] : -1;
    const bool valid = static_cast<unsigned>(e_raw) < static_cast<unsigned>(E);
    const int e = valid ? e_raw : -1;
    // lanes holding the same expert: the lanes that agree with this one on
    // every bit of the expert id (one ballot per bit, constant time)
    uint64_t mine = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      mine &= bit ? m : ~m;
    }
    int r = 0;
    if (valid) {
      const int before = __popcll(mine & lt);
      r = cnt[wave][e] + before;
      // the last lane of each match group advances the counter; lanes of
      // other groups touch other addresses, and this wave's reads above are
      // ordered before its writes
      if (before == __popcll(mine) - 1) cnt[wave][e] = r + 1;
    }
    my_e[s] = e;
    my_r[s] = r;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t p = base + s * 64 + lane;
    if (p < R && my_e[s] >= 0) {
      int add = 0;
      for (int w = 0; w < wave; ++w) add += cnt[w][my_e[s]];
      local_rank[p] = my_r[s] + add;
    }
  }
  for (int e = tid; e < E; e += kRankThreads)
    hist[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[0][e] + cnt[1][e] + cnt[2][e] + cnt[3][e];
}

// One workgroup.  hist[nchunk][E] -> exclusive column prefix (in place);
// count[e]; offset[0..E] = exclusive scan of min(count, cap).
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* __restrict__ hist, int nchunk,
                                                            int E, int64_t cap,
                                                            const int32_t* __restrict__ cap_e,
                                                            int32_t* __restrict__ count,
                                                            int32_t* __restrict__ offset) {
  __shared__ int part[kScanThreads];
  __shared__ int kept[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int segs = kScanThreads / E;  // segments per column (E <= 256 -> >= 4)
  const int col = tid % E, seg = tid / E;
  const bool worker = seg < segs;
  const int rows_per = (nchunk + segs - 1) / segs;
  const int r0 = seg * rows_per;
  const int r1 = min(nchunk, r0 + rows_per);
  int sum = 0;
  if (worker)
    for (int r = r0; r < r1; ++r) sum += hist[static_cast<int64_t>(r) * E + col];
  part[tid] = sum;
  __syncthreads();
  if (worker) {
    int pre = 0;
    for (int s = 0; s < seg; ++s) pre += part[s * E + col];
    for (int r = r0; r < r1; ++r) {
      const int64_t i = static_cast<int64_t>(r) * E + col;
      const int v = hist[i];
      hist[i] = pre;
      pre += v;
    }
    if (seg == segs - 1) {
      count[col] = pre;
      const int64_t c = cap_e ? static_cast<int64_t>(cap_e[col]) : cap;  // per-expert budget
      kept[col] = (c >= 0 && pre > c) ? static_cast<int>(c) : pre;
    }
  }
  __syncthreads();
  // exclusive scan of kept[0..E) by one wave: each lane owns up to 4 entries
  if (tid < kWave) {
    int v[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      v[i] = e < E ? kept[e] : 0;
      local += v[i];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int n = __shfl_up(incl, o);
      if (tid >= o) incl += n;
    }
    int run = incl - local;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < E) offset[e] = run;
      run += v[i];
    }
    if (tid == kWave - 1) offset[E] = incl;
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ idx, int64_t R,
                                                      int E, int64_t cap,
                                                      const int32_t* __restrict__ cap_e,
                                                      const int32_t* __restrict__ local_rank,
                                                      const int32_t* __restrict__ hist,
                                                      const int32_t* __restrict__ offset,
                                                      int32_t* __restrict__ pair_row,
                                                      int32_t* __restrict__ row_pair) {
  const int64_t chunk = blockIdx.x;
  const int total = offset[E];
  for (int i = threadIdx.x; i < kChunk; i += 256) {
    const int64_t p = chunk * kChunk + i;
    if (p >= R) break;
    const int e = idx[p];
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) {  // not routed
      pair_row[p] = -1;
      if (p >= total) row_pair[p] = -1;
      continue;
    }
    const int r = hist[chunk * E + e] + local_rank[p];
    const int64_t c = cap_e ? static_cast<int64_t>(cap_e[e]) : cap;
    const bool kept = c < 0 || r < c;
    const int row = offset[e] + r;
    pair_row[p] = kept ? row : -1;
    if (kept) row_pair[row] = static_cast<int32_t>(p);
    if (p >= total) row_pair[p] = -1;  // rows past the kept total are empty
  }
}

// One wave per destination row; rows_bytes = d * element size.
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ x,
                                                     int64_t row_bytes, int k,
                                                     const int32_t* __restrict__ row_pair,
                                                     const int32_t* __restrict__ offset, int E,
                                                     int64_t R, uint8_t* __restrict__ x_perm) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= R || row >= offset[E]) return;
  const int64_t t = row_pair[row] / k;
  const uint8_t* src = x + t * row_bytes;
  uint8_t* dst = x_perm + row * row_bytes;
  if ((row_bytes & 15) == 0) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    for (int64_t i = lane; i < row_bytes / 16; i += kWave) d4[i] = s4[i];
  } else {
    const uint16_t* s2 = reinterpret_cast<const uint16_t*>(src);
    uint16_t* d2 = reinterpret_cast<uint16_t*>(dst);
    for (int64_t i = lane; i < row_bytes / 2; i += kWave) d2[i] = s2[i];
  }
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

int64_t permute_chunks(int64_t R) { return (R + kChunk - 1) / kChunk; }

// A kernel rather than hipMemsetAsync so that callers may capture it in a graph.
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int E, int64_t cap,
                          const int32_t* cap_e, const void* x, int elem_bytes, int d,
                          int32_t* count, int32_t* offset,
                          int32_t* pair_row, int32_t* row_pair, void* x_perm,
                          int32_t* local_rank, int32_t* hist, hipStream_t stream) {
  const int64_t R = T * k;
  const int64_t nchunk = permute_chunks(R);
  rank_kernel<<<static_cast<unsigned>(nchunk), kRankThreads, 0, stream>>>(idx, R, E, local_rank,
                                                                          hist);
  scan_kernel<<<1, kScanThreads, 0, stream>>>(hist, static_cast<int>(nchunk), E, cap, cap_e,
                                              count, offset);
  scatter_kernel<<<static_cast<unsigned>(nchunk), 256, 0, stream>>>(idx, R, E, cap, cap_e,
                                                                   local_rank, hist, offset,
                                                                   pair_row, row_pair);
  if (x != nullptr) {
    const int64_t row_bytes = static_cast<int64_t>(d) * elem_bytes;
    gather_kernel<<<static_cast<unsigned>((R + 3) / 4), 256, 0, stream>>>(
        static_cast<const uint8_t*>(x), row_bytes, k, row_pair, offset, E, R,
        static_cast<uint8_t*>(x_perm));
  }
  return hipGetLastError();
}

}  // namespace moe
