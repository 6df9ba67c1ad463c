// Ragged grouped GEMMs of the expert SwiGLU MLPs in true fp32 (gfx950).
//
// Page legend:
//   [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
//
// Same two operations and tile schedule as the bf16 kernels (all experts in
// one launch, [Qwen3-MoE page] §2.1), for fp32 workloads: fp32 fused
// multiply-adds on the vector ALUs, summed in K order, so no reduced-precision
// matrix path touches the data.  64x32 output tiles for gate/up (4x2
// outputs per thread; 4x2 gate and 4x2 up sums, silu(g)*u applied before
// storing) and 64x16 for down (4x1), so that the small fp32 problems still
// give most CUs a tile; 16-wide K stages through two LDS buffers fed from
// registers that run two stages ahead, one barrier per stage.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = kF32BM, BK = kF32BK;

// BN output columns per tile: kF32BN for the gate/up GEMM (N = I, two
// weight rows per column), kF32BN / 2 for the down GEMM (N = H), so that
// both give about as many tiles for the small fp32 problems.
template <bool SWIGLU, bool GATHER, int BN>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BR = SWIGLU ? 2 * BN : BN;   // weight rows per tile
  constexpr int TN = BN / 16;                // output columns per thread
  static_assert(BM == 64 && BR <= 64 && BN % 16 == 0, "one 64-row load group per operand");
  __shared__ float As[2][BK][BM + 4];
  __shared__ float Bs[2][BK][BR + 4];
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
    // weight row of tile column lr (swiglu: gate rows, then up rows); lanes
    // past BR load a clamped row and store nothing
    const bool bl = lr < BR;
    const float* bp;
    {
      int64_t wr;
      if constexpr (SWIGLU) {
        const int c = lr < BN ? lr : lr - BN;
        const int n = n0 + c;
        wr = (n < a.I ? n : a.I - 1) + (lr < BN ? 0 : a.I);
      } else {
        const int n = n0 + (bl ? lr : 0);
        wr = n < N ? n : N - 1;
      }
      bp = Bb + static_cast<int64_t>(e) * a.b_stride + wr * K + lk;
    }

    float acc[4][TN], accu[4][TN];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) { acc[i][j] = 0.f; accu[i][j] = 0.f; }

    // stage loads go to registers first: while stage s is multiplied, stage
    // s + 1 waits in registers (av1, bv1) and stage s + 2 is being loaded
    auto load = [&](int k0, float4& av, float4& bv) {
      av = *reinterpret_cast<const float4*>(ap + k0);
      bv = *reinterpret_cast<const float4*>(bp + k0);
    };
    auto store = [&](int buf, const float4& av, const float4& bv) {
      As[buf][lk + 0][lr] = av.x; As[buf][lk + 1][lr] = av.y; As[buf][lk + 2][lr] = av.z;
      As[buf][lk + 3][lr] = av.w;
      if (bl) {
        Bs[buf][lk + 0][lr] = bv.x; Bs[buf][lk + 1][lr] = bv.y; Bs[buf][lk + 2][lr] = bv.z;
        Bs[buf][lk + 3][lr] = bv.w;
      }
    };
    __syncthreads();                 // the previous tile's reads of both buffers are done
    float4 av1, bv1;
    load(0, av1, bv1);
    store(0, av1, bv1);
    if (BK < K) load(BK, av1, bv1);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < K; k0 += BK) {
      const bool more = k0 + BK < K;          // stage s + 1 exists (in av1, bv1)
      float4 av2 = av1, bv2 = bv1;
      if (k0 + 2 * BK < K) load(k0 + 2 * BK, av2, bv2);
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float av4[4], bv4[TN], uv4[TN];
#pragma unroll
        for (int i = 0; i < 4; ++i) av4[i] = As[buf][kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < TN; ++j) bv4[j] = Bs[buf][kk][tx * TN + j];
        if constexpr (SWIGLU) {
#pragma unroll
          for (int j = 0; j < TN; ++j) uv4[j] = Bs[buf][kk][BN + tx * TN + j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            acc[i][j] = fmaf(av4[i], bv4[j], acc[i][j]);
            if constexpr (SWIGLU) accu[i][j] = fmaf(av4[i], uv4[j], accu[i][j]);
          }
      }
      // the other buffer was last read before the previous barrier
      if (more) store(buf ^ 1, av1, bv1);
      __syncthreads();
      av1 = av2;
      bv1 = bv2;
      buf ^= 1;
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = ty * 4 + i;
      if (m >= rows) continue;
      float* crow = Cb + static_cast<int64_t>(a.scatter ? a.scatter[r0 + m] : r0 + m) * N;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + tx * TN + j;
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
  constexpr int BN = SWIGLU ? kF32BN : kF32BN / 2;
  hipLaunchKernelGGL((gemm_f32_kernel<SWIGLU, GATHER, BN>), dim3(a.grid), dim3(256), 0, s, a);
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
