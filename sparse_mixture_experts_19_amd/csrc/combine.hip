// Routing-weighted combine back to token order (gfx950).
//
// Page legend:
//   [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
//
// out[t] = sum_{j<k} w[t,j] * y[inv[t*k+j]]: the weighted sum of expert
// outputs of [Qwen3-MoE page] §1 (phase 4) and the scatter back to token
// order of §2.2.  A workgroup owns one output row; its k slot rows are
// gathered with 128-bit loads, summed in fp32 in slot order and rounded once
// -- no atomics, bitwise deterministic.  The fused forward has
// its down GEMM write y already in token order (row t*k+j), passes no inv,
// and the k rows of a token are then read contiguously.  With a shared expert
// (moe_forward_shared) its output row is added last, with weight 1.
#include "moe_internal.h"

namespace moe {
namespace {
// 16-byte vector type the nontemporal builtins take
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));

// One workgroup per token: thread i owns the 16-byte chunks i, i + 256, ...
// of the token's output row.  For each chunk all k slot rows are requested
// before any is summed (k <= 8 loads of 16 bytes in flight per thread); the
// slot rows and weights are the same for the whole workgroup, so their
// indices come through scalar loads and no thread divides.  y is read once
// and out written once: both go through the nontemporal path, which took the
// kernel from 4.7-5.1 to 5.5-5.8 TB/s on the four bf16 workloads (stores
// alone: 4.8-5.4).
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int64_t T,
                                                      int chunks, int k, uint4* __restrict__ out,
                                                      const uint4* __restrict__ ys) {
  constexpr int V = BF16 ? 8 : 4;
  const int64_t t = blockIdx.x;
  const int64_t M = T * k;
  int64_t row[kMaxK];
  float wt[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      int64_t r = t * k + j;
      if (inv) {
        r = inv[r];
        r = r < 0 ? 0 : (r >= M ? M - 1 : r);   // malformed inv_perm stays in bounds
      }
      row[j] = r * chunks;
      wt[j] = w[t * k + j];
    } else {
      row[j] = 0;
      wt[j] = 0.f;
    }
  }
  for (int c = threadIdx.x; c < chunks; c += 256) {
    uint4 q[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) q[j] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(y + row[j] + c)));
    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        if constexpr (BF16) {
          const uint16_t* p = reinterpret_cast<const uint16_t*>(&q[j]);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[v] = fmaf(wt[j], bf16_to_f32(p[v]), acc[v]);
        } else {
          const float* p = reinterpret_cast<const float*>(&q[j]);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[v] = fmaf(wt[j], p[v], acc[v]);
        }
      }
    }
    if (ys) {                       // shared expert output, weight 1, after the k slots
      const uint4 qs = ys[t * chunks + c];
      if constexpr (BF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(&qs);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += bf16_to_f32(p[v]);
      } else {
        const float* p = reinterpret_cast<const float*>(&qs);
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
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, o), reinterpret_cast<u32x4_nt*>(out + t * chunks + c));
  }
}

}  // namespace

hipError_t launch_combine(const void* y, const int32_t* inv, const float* w, int64_t T, int H,
                          int k, bool bf16, void* out, hipStream_t s, const void* ys) {
  if (k < 1 || k > kMaxK || T > 0x7fffffff) return hipErrorInvalidValue;
  const int chunks = H * (bf16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>(T));
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, static_cast<const uint4*>(y), inv, w,
                       T, chunks, k, static_cast<uint4*>(out), static_cast<const uint4*>(ys));
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, static_cast<const uint4*>(y), inv, w,
                       T, chunks, k, static_cast<uint4*>(out), static_cast<const uint4*>(ys));
  return hipGetLastError();
}

}  // namespace moe
