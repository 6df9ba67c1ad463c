// Routing-weighted combine back to token order (gfx950).
//
// Page legend:
//   [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
//
// out[t] = sum_{j<k} w[t,j] * y[inv[t*k+j]]: the weighted sum of expert
// outputs of [Qwen3-MoE page] §1 (phase 4) and the scatter back to token
// order of §2.2.  Each thread owns one 16-byte chunk of one output row, so the
// k rows are gathered with 128-bit loads, summed in fp32 in slot order and
// rounded once -- no atomics, bitwise deterministic.  The fused forward has
// its down GEMM write y already in token order (row t*k+j), passes no inv,
// and the k rows of a token are then read contiguously.  With a shared expert
// (moe_forward_shared) its output row is added last, with weight 1.
#include "moe_internal.h"

namespace moe {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int64_t T,
                                                      int chunks, int k, uint4* __restrict__ out,
                                                      const uint4* __restrict__ ys) {
  constexpr int V = BF16 ? 8 : 4;
  const int64_t total = T * chunks;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = i / chunks;
    const int c = static_cast<int>(i - t * chunks);
    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
    for (int j = 0; j < k; ++j) {
      int64_t r = t * k + j;
      if (inv) {
        r = inv[r];
        r = r < 0 ? 0 : (r >= T * k ? T * k - 1 : r);   // malformed inv_perm stays in bounds
      }
      const float wj = w[t * k + j];
      const uint4 q = y[r * chunks + c];
      if constexpr (BF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(&q);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = fmaf(wj, bf16_to_f32(p[v]), acc[v]);
      } else {
        const float* p = reinterpret_cast<const float*>(&q);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = fmaf(wj, p[v], acc[v]);
      }
    }
    if (ys) {                       // shared expert output, weight 1, after the k slots
      const uint4 q = ys[i];
      if constexpr (BF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(&q);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += bf16_to_f32(p[v]);
      } else {
        const float* p = reinterpret_cast<const float*>(&q);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += p[v];
      }
    }
    uint4 o;
    if constexpr (BF16) {
      uint16_t* p = reinterpret_cast<uint16_t*>(&o);
#pragma unroll
      for (int v = 0; v < V; ++v) p[v] = f32_to_bf16(acc[v]);
    } else {
      float* p = reinterpret_cast<float*>(&o);
#pragma unroll
      for (int v = 0; v < V; ++v) p[v] = acc[v];
    }
    out[i] = o;
  }
}

}  // namespace

hipError_t launch_combine(const void* y, const int32_t* inv, const float* w, int64_t T, int H,
                          int k, bool bf16, void* out, hipStream_t s, const void* ys) {
  const int chunks = H * (bf16 ? 2 : 4) / 16;
  const int64_t total = T * chunks;
  int64_t grid = (total + 255) / 256;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 16;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                       static_cast<const uint4*>(y), inv, w, T, chunks, k, static_cast<uint4*>(out),
                       static_cast<const uint4*>(ys));
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                       static_cast<const uint4*>(y), inv, w, T, chunks, k, static_cast<uint4*>(out),
                       static_cast<const uint4*>(ys));
  return hipGetLastError();
}

}  // namespace moe
