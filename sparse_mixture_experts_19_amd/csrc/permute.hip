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
// Deterministic passes, free of order-deciding atomics:
//   1. per-chunk expert histograms (LDS integer counters);
//   2. each chunk sums the histograms of the chunks before it (its row base
//      inside each expert) and of all chunks (the expert counts), derives
//      the expert offsets, ranks its elements in order (wave match + LDS
//      prefix) and writes perm / inv; the first chunk also writes counts,
//      offsets and, when asked, the grouped GEMM's tile prefix.
// A problem of one chunk (at most 1024 assignments) counts its histogram in
// pass 2 itself: one launch.
// When the histogram table is large (chunks x experts above 32768 entries)
// those sums would cost each chunk too many loads: a separate pass with one
// workgroup per expert then turns the table into chunk bases and counts
// first, and pass 2 reads them from there.
#include "moe_internal.h"

#include <mutex>

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

// INLINE_SCAN: block_hist holds the raw chunk histograms (chunk-major) and
// this kernel sums them; otherwise perm_scan_kernel has already turned them
// into chunk bases and written the counts.
template <bool INLINE_SCAN>
__global__ __launch_bounds__(256) void perm_scatter_kernel(PermuteArgs a, int nb) {
  __shared__ int base[kMaxE];
  __shared__ int wc[4][kMaxE];
  __shared__ int buf[256];
  __shared__ int red[2][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  const int bx = blockIdx.x;
  int cnt = 0, before = 0;   // expert tid: rows in all chunks / in chunks before this one
  if (INLINE_SCAN && nb == 1) {
    // the whole problem is one chunk: its histogram is counted here and no
    // separate histogram pass runs (out-of-range ids are dropped, as there)
    red[0][tid] = 0;
    __syncthreads();
    for (int64_t f = tid; f < a.M; f += 256) {
      const unsigned e = static_cast<unsigned>(a.ids[f]);
      if (e < static_cast<unsigned>(E)) atomicAdd(&red[0][e], 1);
    }
    __syncthreads();
    if (tid < E) cnt = red[0][tid];
    if (tid < E) a.counts[tid] = cnt;
    __syncthreads();                 // red is reused below
  } else if constexpr (INLINE_SCAN) {
    // thread (g, e) sums chunks g, g + G, ... of column e; eight loads in
    // flight per thread
    const int G = 256 / E;
    int tot = 0, bef = 0;
    if (tid < G * E) {
      const int g = tid / E, e = tid - g * E;
      const int32_t* h = a.block_hist + e;
      int b = g;
      for (; b + 7 * G < nb; b += 8 * G) {
        int v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = h[static_cast<int64_t>(b + q * G) * E];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          tot += v[q];
          if (b + q * G < bx) bef += v[q];
        }
      }
      for (; b < nb; b += G) {
        const int v = h[static_cast<int64_t>(b) * E];
        tot += v;
        if (b < bx) bef += v;
      }
    }
    red[0][tid] = tot;
    red[1][tid] = bef;
    __syncthreads();
    if (tid < E)
      for (int g = 0; g < G; ++g) {
        cnt += red[0][g * E + tid];
        before += red[1][g * E + tid];
      }
    if (bx == 0 && tid < E) a.counts[tid] = cnt;
  } else {
    if (tid < E) {
      cnt = a.counts[tid];
      before = a.block_hist[static_cast<int64_t>(bx) * E + tid];
    }
  }
  // expert offsets = exclusive prefix of the counts (every workgroup derives
  // them; the first one also writes them out, and the tile prefix)
  const int all = block_exclusive_scan(cnt, buf);
  if (bx == 0) {
    if (tid < E) a.offsets[tid] = buf[tid];
    if (tid == 0) a.offsets[E] = all;
  }
  if (tid < E) base[tid] = buf[tid] + before;
  for (int i = tid; i < 4 * kMaxE; i += 256) (&wc[0][0])[i] = 0;
  if (bx == 0 && a.tile_prefix) {
    // m-tiles of tile_bm rows per expert, exclusive prefix over experts
    const int mt = tid < E ? (cnt + a.tile_bm - 1) / a.tile_bm : 0;
    const int tiles = block_exclusive_scan(mt, red[0]);
    if (tid < E) a.tile_prefix[tid] = red[0][tid];
    if (tid == 0) a.tile_prefix[E] = tiles;
  }
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

// x_perm[inv[t*k + j]] = x[t] for j < k: one workgroup per token.  Each
// thread loads up to four of the row's 16-byte chunks (i, i + 256, ...) into
// registers and stores each of them k times, so x is read once in all (the
// loads are nontemporal: nothing here reads a row twice) and every row of
// x_perm is written once, by whole 4 KB lines per store instruction.  A
// destination outside [0, M) (a malformed inv) is skipped.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ inv,
                                                          int64_t M, int chunks, int k,
                                                          uint4* __restrict__ xp) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int64_t t = blockIdx.x;
  const u32x4* in = reinterpret_cast<const u32x4*>(x) + t * chunks;
  u32x4* out = reinterpret_cast<u32x4*>(xp);
  const int32_t* dst = inv + t * k;
  for (int c0 = 0; c0 < chunks; c0 += 4 * 256) {
    const int c = c0 + static_cast<int>(threadIdx.x);
    u32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (c + q * 256 < chunks) v[q] = __builtin_nontemporal_load(in + c + q * 256);
    for (int j = 0; j < k; ++j) {
      const int64_t r = dst[j];
      if (static_cast<uint64_t>(r) >= static_cast<uint64_t>(M)) continue;
      u32x4* o = out + r * chunks;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (c + q * 256 < chunks) __builtin_nontemporal_store(v[q], o + c + q * 256);
    }
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

// ------------------------------------------- allocation-free permutation
// The per-chunk expert histograms of moe_permute_static live in this
// file-scope device array (each GPU holds its own copy until the process
// ends).  Host code never passes the array's name to a kernel: the name is
// a host-side stand-in, and the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) int32_t scratch[kPermStaticScratchInts];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t permute_static_scratch(int device, int32_t** ptr) {
  if (device < 0 || device >= kMaxDevices || !ptr) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = static_cast<int32_t*>(p);
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

size_t permute_scratch_bytes(int64_t M, int E) {
  const int64_t nb = (M + CH - 1) / CH;
  return align_up(static_cast<size_t>(nb > 0 ? nb : 1) * E * 4, 256);
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.tile_prefix && a.tile_bm < 1) return hipErrorInvalidValue;
  const int nb = static_cast<int>((a.M + CH - 1) / CH);
  // one chunk: the scatter pass counts its histogram itself
  if (nb > 1) hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(256), 0, s, a);
  if (static_cast<int64_t>(nb) * a.E <= kPermInlineScan) {
    hipLaunchKernelGGL(perm_scatter_kernel<true>, dim3(nb), dim3(256), 0, s, a, nb);
  } else {
    hipLaunchKernelGGL(perm_scan_kernel, dim3(a.E), dim3(256), 0, s, a, nb);
    hipLaunchKernelGGL(perm_scatter_kernel<false>, dim3(nb), dim3(256), 0, s, a, nb);
  }
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* inv, int64_t T, int H, int k,
                              int elem_bytes, void* x_perm, hipStream_t s) {
  if (T > 0x7fffffff || k < 1) return hipErrorInvalidValue;
  const int chunks = H * elem_bytes / 16;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(T)), dim3(256), 0, s,
                     static_cast<const uint4*>(x), inv, T * k, chunks, k, static_cast<uint4*>(x_perm));
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
