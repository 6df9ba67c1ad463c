// Expert-sorted permutation of the T*k assignments (gfx950).
//
// Page legend:
//   [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
//
// [Qwen3-MoE page] §2.2 reorders the tokens by their assigned expert so each
// expert works on a contiguous block, and scatters the results back
// afterwards.  Here, with f = t*k + j the flat assignment index:
//   counts[e]  = #{f : ids[f] == e}
//   offsets    = exclusive prefix sum of counts (E+1 entries)
//   perm[r]    = f of row r, rows in (expert, f) order (stable)
//   inv[f]     = r with perm[r] == f
// Three passes, all deterministic and free of order-deciding atomics:
//   1. per-chunk expert histograms (LDS integer counters),
//   2. one workgroup per expert scans its chunk counts into chunk-local row
//      bases and the expert's count,
//   3. each chunk derives the expert offsets from the counts, ranks its
//      elements in order (wave match + LDS prefix) and writes perm / inv.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int CH = kPermChunk;

__global__ __launch_bounds__(256) void perm_hist_kernel(PermuteArgs a) {
  __shared__ int hist[kMaxE];
  const int tid = threadIdx.x;
  hist[tid] = 0;
  __syncthreads();
  const int64_t f0 = static_cast<int64_t>(blockIdx.x) * CH;
  const int64_t f1 = (f0 + CH < a.M) ? f0 + CH : a.M;
  for (int64_t f = f0 + tid; f < f1; f += 256) {
    const unsigned e = static_cast<unsigned>(a.ids[f]);
    if (e < static_cast<unsigned>(a.E)) atomicAdd(&hist[e], 1);   // out-of-range ids are dropped
  }
  __syncthreads();
  if (tid < a.E) a.block_hist[static_cast<int64_t>(blockIdx.x) * a.E + tid] = hist[tid];
}

// Exclusive scan of a 256-entry workgroup vector in LDS; returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int add = tid >= d ? buf[tid - d] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid], total = buf[255];
  __syncthreads();
  buf[tid] = incl - v;
  return total;
}

// One workgroup per expert: the expert's chunk counts become chunk-local row
// bases (exclusive prefix over chunks, in chunk order); counts[e] = total.
__global__ __launch_bounds__(256) void perm_scan_kernel(PermuteArgs a, int nblocks) {
  __shared__ int buf[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  int carry = 0;
  for (int b0 = 0; b0 < nblocks; b0 += 256) {
    const int b = b0 + tid;
    int* p = a.block_hist + static_cast<int64_t>(b) * a.E + e;
    const int v = b < nblocks ? *p : 0;
    const int total = block_exclusive_scan(v, buf);
    if (b < nblocks) *p = carry + buf[tid];
    carry += total;
    __syncthreads();
  }
  if (tid == 0) a.counts[e] = carry;
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(PermuteArgs a) {
  __shared__ int base[kMaxE];
  __shared__ int wc[4][kMaxE];
  __shared__ int buf[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  // expert offsets = exclusive prefix of the counts (every workgroup derives
  // them; the first one also writes them out)
  const int cnt = tid < E ? a.counts[tid] : 0;
  const int all = block_exclusive_scan(cnt, buf);
  if (blockIdx.x == 0) {
    if (tid < E) a.offsets[tid] = buf[tid];
    if (tid == 0) a.offsets[E] = all;
  }
  if (tid < E) base[tid] = buf[tid] + a.block_hist[static_cast<int64_t>(blockIdx.x) * E + tid];
  for (int i = tid; i < 4 * kMaxE; i += 256) (&wc[0][0])[i] = 0;
  __syncthreads();

  const int64_t f0 = static_cast<int64_t>(blockIdx.x) * CH;
  const int64_t f1 = (f0 + CH < a.M) ? f0 + CH : a.M;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int64_t fr = f0; fr < f1; fr += 256) {
    const int64_t f = fr + tid;
    int e = (f < f1) ? a.ids[f] : -1;
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    if (!valid) e = 0;
    // lanes of this wave holding the same expert
    unsigned long long same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool b = (e >> bit) & 1;
      const unsigned long long m = __ballot(valid && b);
      same &= b ? m : ~m;
    }
    const int rank = __popcll(same & lt);
    if (valid && rank == 0) wc[wave][e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int pre = base[e];
      for (int w = 0; w < wave; ++w) pre += wc[w][e];
      const int r = pre + rank;
      a.perm[r] = static_cast<int32_t>(f);
      a.inv[f] = r;
    }
    __syncthreads();
    if (tid < E) {
      base[tid] += wc[0][tid] + wc[1][tid] + wc[2][tid] + wc[3][tid];
      wc[0][tid] = 0; wc[1][tid] = 0; wc[2][tid] = 0; wc[3][tid] = 0;
    }
    __syncthreads();
  }
}

// x_perm[r] = x[perm[r] / k], 16-byte chunks.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          int64_t M, int64_t T, int chunks,
                                                          int k, uint4* __restrict__ xp) {
  const int64_t total = M * chunks;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / chunks;
    const int c = static_cast<int>(i - r * chunks);
    int64_t src = perm[r] / k;
    src = src < 0 ? 0 : (src >= T ? T - 1 : src);   // malformed perm stays in bounds
    xp[i] = x[src * chunks + c];
  }
}

__global__ void dense_offsets_kernel(int32_t* offsets, int64_t M) {
  if (threadIdx.x == 0) {
    offsets[0] = 0;
    offsets[1] = static_cast<int32_t>(M);
  }
}

__global__ __launch_bounds__(256) void tile_schedule_kernel(const int32_t* offsets, int E, int bm,
                                                            int64_t M, int32_t* prefix) {
  __shared__ int mt[kMaxE];
  const int e = threadIdx.x;
  if (e < E) {
    // rows of expert e, clamped to [0, M] so malformed offsets stay in bounds
    int64_t c = static_cast<int64_t>(offsets[e + 1]) - offsets[e];
    c = c < 0 ? 0 : (c > M ? M : c);
    mt[e] = static_cast<int>((c + bm - 1) / bm);
  }
  __syncthreads();
  if (e == 0) {
    int s = 0;
    for (int i = 0; i < E; ++i) { prefix[i] = s; s += mt[i]; }
    prefix[E] = s;
  }
}

}  // namespace

size_t permute_scratch_bytes(int64_t M, int E) {
  const int64_t nb = (M + CH - 1) / CH;
  return align_up(static_cast<size_t>(nb > 0 ? nb : 1) * E * 4, 256);
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const int nb = static_cast<int>((a.M + CH - 1) / CH);
  hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(256), 0, s, a);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(a.E), dim3(256), 0, s, a, nb);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* perm, int64_t M, int H, int k,
                              int elem_bytes, void* x_perm, hipStream_t s) {
  const int chunks = H * elem_bytes / 16;
  const int64_t total = M * chunks;
  int64_t grid = (total + 255) / 256;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 16;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                     static_cast<const uint4*>(x), perm, M, M / k, chunks, k,
                     static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_dense_offsets(int32_t* offsets, int64_t M, hipStream_t s) {
  hipLaunchKernelGGL(dense_offsets_kernel, dim3(1), dim3(64), 0, s, offsets, M);
  return hipGetLastError();
}

hipError_t launch_tile_schedule(const int32_t* offsets, int E, int bm, int64_t M, int32_t* prefix,
                                hipStream_t s) {
  hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(256), 0, s, offsets, E, bm, M, prefix);
  return hipGetLastError();
}

}  // namespace moe
