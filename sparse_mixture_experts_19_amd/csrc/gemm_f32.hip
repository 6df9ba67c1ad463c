// Ragged grouped GEMMs of the expert SwiGLU MLPs in true fp32 (gfx950).
//
// Page legend:
//   [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
//
// Same two operations and tile schedule as the bf16 kernels (all experts in
// one launch, [Qwen3-MoE page] §2.1), for fp32 workloads: fp32 fused
// multiply-adds on the vector ALUs, summed in K order, so no reduced-precision
// matrix path touches the data.  64x64 output tiles, 16-wide K stages through
// LDS, 4x4 outputs per thread (the swiglu kernel keeps 4x4 gate and 4x4 up
// sums and applies silu(g)*u before storing).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = kF32BM, BN = kF32BN, BK = kF32BK;

template <bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BR = SWIGLU ? 2 * BN : BN;   // weight rows per tile
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BR + 4];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_pre[kMaxE + 1];

  const int tid = threadIdx.x;
  const int E = a.E;
  for (int i = tid; i <= E; i += 256) { s_off[i] = a.offsets[i]; s_pre[i] = a.prefix[i]; }
  __syncthreads();

  const int N = a.N, K = a.K;
  const int NT = (N + BN - 1) / BN;
  const int total = s_pre[E] * NT;
  const float* Ab = static_cast<const float*>(a.A);
  const float* Bb = static_cast<const float*>(a.B);
  float* Cb = static_cast<float*>(a.C);
  const int ty = tid >> 4, tx = tid & 15;
  const int lr = tid >> 2, lk = (tid & 3) * 4;

  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const int q = L / NT, nt = L - q * NT;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] <= q) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int r0 = s_off[e] + (q - s_pre[e]) * BM;
    int rows = (s_off[e + 1] - r0 < BM) ? s_off[e + 1] - r0 : BM;
    if (r0 < 0 || r0 >= a.M) continue;             // malformed offsets: skip, never fault
    if (rows > a.M - r0) rows = static_cast<int>(a.M - r0);
    if (rows <= 0) continue;
    const int n0 = nt * BN;

    const int rr = r0 + (lr < rows ? lr : rows - 1);
    int64_t src = rr;
    if constexpr (GATHER) {
      src = a.gather[rr] / a.gather_div;
      src = src < 0 ? 0 : (src >= a.a_rows ? a.a_rows - 1 : src);
    }
    const float* ap = Ab + src * K + lk;
    const float* bp[BR / 64];
#pragma unroll
    for (int h = 0; h < BR / 64; ++h) {
      int64_t wr;
      if constexpr (SWIGLU) {
        const int n = n0 + lr;
        wr = (n < a.I ? n : a.I - 1) + (h == 1 ? a.I : 0);
      } else {
        const int n = n0 + lr;
        wr = n < N ? n : N - 1;
      }
      bp[h] = Bb + static_cast<int64_t>(e) * a.b_stride + wr * K + lk;
    }

    float acc[4][4], accu[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) { acc[i][j] = 0.f; accu[i][j] = 0.f; }

    for (int k0 = 0; k0 < K; k0 += BK) {
      __syncthreads();
      const float4 av = *reinterpret_cast<const float4*>(ap + k0);
      As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
#pragma unroll
      for (int h = 0; h < BR / 64; ++h) {
        const float4 bv = *reinterpret_cast<const float4*>(bp[h] + k0);
        const int c = h * 64 + lr;
        Bs[lk + 0][c] = bv.x; Bs[lk + 1][c] = bv.y; Bs[lk + 2][c] = bv.z; Bs[lk + 3][c] = bv.w;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float av4[4], bv4[4], uv4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av4[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv4[j] = Bs[kk][tx * 4 + j];
        if constexpr (SWIGLU) {
#pragma unroll
          for (int j = 0; j < 4; ++j) uv4[j] = Bs[kk][BN + tx * 4 + j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = fmaf(av4[i], bv4[j], acc[i][j]);
            if constexpr (SWIGLU) accu[i][j] = fmaf(av4[i], uv4[j], accu[i][j]);
          }
      }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = ty * 4 + i;
      if (m >= rows) continue;
      float* crow = Cb + static_cast<int64_t>(a.scatter ? a.scatter[r0 + m] : r0 + m) * N;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx * 4 + j;
        if (n >= N) continue;
        float v = acc[i][j];
        if constexpr (SWIGLU) v = (v / (1.f + __expf(-v))) * accu[i][j];
        crow[n] = v;
      }
    }
  }
}

template <bool SWIGLU, bool GATHER>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_f32_kernel<SWIGLU, GATHER>), dim3(a.grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32_swiglu(const GemmArgs& a, hipStream_t s) {
  return a.gather ? launch<true, true>(a, s) : launch<true, false>(a, s);
}

hipError_t launch_gemm_f32_down(const GemmArgs& a, hipStream_t s) {
  return launch<false, false>(a, s);
}

}  // namespace moe
