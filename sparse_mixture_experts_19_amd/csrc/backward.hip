// Backward of the MoE block (gfx950): everything around the grouped GEMMs.
//
// Page legend:
//   [SonicMoE page] "SonicMoE与传统MoE架构对比：Token舍入技术如何实现训练效率跃升"
//   [Hunyuan page]  "混合专家架构大模型Hunyuan-Large：原理剖析与实现机制"
//
// [SonicMoE page] 核心差异 §1 keeps only the gate outputs and the final
// expert outputs of the forward and recomputes the rest: here the forward's
// routing (ids, weights, permutation) and its expert outputs y are reused,
// g and u are recomputed by the grouped GEMM and h from them.  [Hunyuan
// page] §二.2: only the experts a token activated receive gradients.  With
// L = sum(dout * out) and the top-k choice held fixed:
//   dw[t,j]  = <dout_t, y_tj>                          (bwd_dw_kernel)
//   dl[t,e]  = p_e (dp_e - sum_e' dp_e' p_e')          (bwd_router_kernel)
//              with dp the scatter of dw through the renormalisation
//   dx      += dl W_r,  dW_r = dl^T x,  db = sum_t dl  (bwd_dxr / bwd_dwr / bwd_dbias)
//   dh       = (w_r dout) W2_e  (grouped GEMM, then scaled here)
//   dg = dh u silu'(g),  du = dh silu(g),  h = silu(g) u   (bwd_swiglu_kernel)
//   dx_slot  = [dg du] W13_e,  dW2_e = dy^T h,  dW13_e = [dg du]^T x
// The weight-gradient GEMMs reduce over each expert's rows: their operands
// are transposed here into [features, padded rows], each expert's rows
// padded to a multiple of 64 (and to at least 64, so an expert without
// tokens contributes one stage of zeros and its gradients come out zero).
// Every reduction runs in a fixed order: no atomics, deterministic.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v[2 * u] = __uint_as_float(w[u] << 16);
    v[2 * u + 1] = __uint_as_float(w[u] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  uint4 q;
  q.x = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
  q.y = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
  q.z = f32_to_bf16(v[4]) | (static_cast<uint32_t>(f32_to_bf16(v[5])) << 16);
  q.w = f32_to_bf16(v[6]) | (static_cast<uint32_t>(f32_to_bf16(v[7])) << 16);
  *reinterpret_cast<uint4*>(p) = q;
}

// dw[t*k+j] = <dout_t, y[t*k+j]>: one wave per token, dout read once.
__global__ __launch_bounds__(256) void bwd_dw_kernel(const uint16_t* __restrict__ dout,
                                                     const uint16_t* __restrict__ y, int64_t T,
                                                     int H, int k, float* __restrict__ dw) {
  const int lane = threadIdx.x & 63;
  const int64_t t = blockIdx.x * 4LL + (threadIdx.x >> 6);
  if (t >= T) return;
  float acc[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) acc[j] = 0.f;
  for (int c = lane * 8; c < H; c += 512) {
    float d[8];
    load8(dout + t * H + c, d);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        float v[8];
        load8(y + (t * k + j) * H + c, v);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[j] += d[u] * v[u];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      const float s = wave_sum(acc[j]);
      if (lane == 0) dw[t * k + j] = s;
    }
  }
}

// dl[t,e] from the token's logits (softmax max and sum from the router), its
// routing and dw.  One wave per token, lanes over experts.
__global__ __launch_bounds__(256) void bwd_router_kernel(const float* __restrict__ logits,
                                                         const float* __restrict__ meta,
                                                         const int32_t* __restrict__ ids,
                                                         const float* __restrict__ dw, int64_t T,
                                                         int E, int k, int renorm,
                                                         float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = blockIdx.x * 4LL + (threadIdx.x >> 6);
  if (t >= T) return;
  const float mx = meta[t * 4], inv_sum = 1.f / meta[t * 4 + 1];
  // selected probabilities, the gradient through the renormalisation, and
  // c = sum_j dps_j p_j (every lane computes the same k values)
  float ps[kMaxK], dps[kMaxK];
  int sel[kMaxK];
  float S = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    sel[j] = -1;
    ps[j] = dps[j] = 0.f;
    if (j < k) {
      sel[j] = ids[t * k + j];
      ps[j] = __expf(logits[t * E + sel[j]] - mx) * inv_sum;
      dps[j] = dw[t * k + j];
      S += ps[j];
    }
  }
  if (renorm) {
    float mean = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) mean += dps[j] * ps[j];
    mean /= S;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) dps[j] = (dps[j] - mean) / S;
  }
  float c = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) c += dps[j] * ps[j];
  for (int e = lane; e < E; e += 64) {
    const float p = __expf(logits[t * E + e] - mx) * inv_sum;
    float dp = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (sel[j] == e) dp = dps[j];
    dl[t * E + e] = p * (dp - c);
  }
}

// dxr[t,h] = sum_e dl[t,e] W_r[e,h] (bf16 out): 16 tokens x 256 columns per
// block, dl of the 16 tokens in LDS, one column per thread.
constexpr int kDxrTok = 16;
__global__ __launch_bounds__(256) void bwd_dxr_kernel(const float* __restrict__ dl,
                                                      const uint16_t* __restrict__ wr, int64_t T,
                                                      int H, int E, uint16_t* __restrict__ dxr) {
  __shared__ float sdl[kDxrTok * kMaxE];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kDxrTok;
  const int h = blockIdx.y * 256 + threadIdx.x;
  for (int i = threadIdx.x; i < kDxrTok * E; i += 256) {
    const int64_t t = t0 + i / E;
    sdl[i] = t < T ? dl[t0 * E + i] : 0.f;
  }
  __syncthreads();
  if (h >= H) return;
  float acc[kDxrTok];
#pragma unroll
  for (int i = 0; i < kDxrTok; ++i) acc[i] = 0.f;
  for (int e = 0; e < E; ++e) {
    const float w = bf16_to_f32(wr[static_cast<int64_t>(e) * H + h]);
#pragma unroll
    for (int i = 0; i < kDxrTok; ++i) acc[i] += sdl[i * E + e] * w;
  }
#pragma unroll
  for (int i = 0; i < kDxrTok; ++i)
    if (t0 + i < T) dxr[(t0 + i) * H + h] = f32_to_bf16(acc[i]);
}

// dW_r partial sums over token slices: part[s,e,h] = sum_{t in slice s}
// dl[t,e] x[t,h], tokens in order; NE experts x 1024 columns per block, a
// thread owning 4 consecutive columns (one 8-byte load of x per token, the
// loads of 16 tokens issued before their sums).  The block's dl values come
// through LDS, 256 tokens at a time (one cooperative load instead of a
// round trip per token).
constexpr int kDwrExp = 16;      // experts per block (8 when E <= 8)
constexpr int kDwrCols = 4;
constexpr int kDwrChunk = 256;
constexpr int kDwrBatch = 16;    // tokens whose x loads are in flight together
template <int NE>
__global__ __launch_bounds__(256) void bwd_dwr_partial_kernel(const float* __restrict__ dl,
                                                              const uint16_t* __restrict__ x,
                                                              int64_t T, int H, int E, int64_t slice,
                                                              float* __restrict__ part) {
  __shared__ float sdl[kDwrChunk * NE];
  const int tid = threadIdx.x;
  const int h = (blockIdx.y * 256 + tid) * kDwrCols;
  const bool live = h < H;
  const int e0 = blockIdx.x * NE;
  const int s = blockIdx.z;
  const int64_t ta = s * slice, tb = ta + slice < T ? ta + slice : T;
  float acc[NE][kDwrCols];
#pragma unroll
  for (int i = 0; i < NE; ++i)
#pragma unroll
    for (int c = 0; c < kDwrCols; ++c) acc[i][c] = 0.f;
  const uint16_t* xc = x + (live ? h : 0);
  auto add = [&](const float* d, uint2 xr) {
    const float xv[kDwrCols] = {bf16_to_f32(static_cast<uint16_t>(xr.x)), bf16_to_f32(static_cast<uint16_t>(xr.x >> 16)),
                                bf16_to_f32(static_cast<uint16_t>(xr.y)), bf16_to_f32(static_cast<uint16_t>(xr.y >> 16))};
#pragma unroll
    for (int i = 0; i < NE; ++i)
#pragma unroll
      for (int c = 0; c < kDwrCols; ++c) acc[i][c] += d[i] * xv[c];
  };
  for (int64_t c0 = ta; c0 < tb; c0 += kDwrChunk) {
    const int n = static_cast<int>(tb - c0 < kDwrChunk ? tb - c0 : kDwrChunk);
    __syncthreads();                       // the previous chunk's dl is no longer read
    for (int idx = tid; idx < n * NE; idx += 256) {
      const int tt = idx / NE, i = idx % NE;
      sdl[idx] = e0 + i < E ? dl[(c0 + tt) * E + e0 + i] : 0.f;
    }
    __syncthreads();
    if (live) {
      int u0 = 0;
      for (; u0 + kDwrBatch <= n; u0 += kDwrBatch) {
        uint2 xr[kDwrBatch];
#pragma unroll
        for (int u = 0; u < kDwrBatch; ++u) xr[u] = *reinterpret_cast<const uint2*>(xc + (c0 + u0 + u) * H);
#pragma unroll
        for (int u = 0; u < kDwrBatch; ++u) add(sdl + (u0 + u) * NE, xr[u]);
      }
      for (; u0 < n; ++u0) add(sdl + u0 * NE, *reinterpret_cast<const uint2*>(xc + (c0 + u0) * H));
    }
  }
  if (!live) return;
#pragma unroll
  for (int i = 0; i < NE; ++i)
    if (e0 + i < E) {
      float4 v;
      v.x = acc[i][0]; v.y = acc[i][1]; v.z = acc[i][2]; v.w = acc[i][3];
      *reinterpret_cast<float4*>(part + (static_cast<int64_t>(s) * E + e0 + i) * H + h) = v;
    }
}

// dW_r = sum over slices in slice order
__global__ __launch_bounds__(256) void bwd_dwr_reduce_kernel(const float* __restrict__ part, int S,
                                                             int64_t n, float* __restrict__ dwr) {
  const int64_t i = blockIdx.x * 256LL + threadIdx.x;
  if (i >= n) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[s * n + i];
  dwr[i] = v;
}

// db[e] = sum_t dl[t,e]: one block per expert, strided sums then a fixed tree
__global__ __launch_bounds__(256) void bwd_dbias_kernel(const float* __restrict__ dl, int64_t T,
                                                        int E, float* __restrict__ db) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float v = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += 256) v += dl[t * E + e];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) db[e] = red[0];
}

// Padded expert segments of the weight-gradient operands and the tables of
// the two weight-gradient GEMMs (one block, thread 0 walks the experts).
__global__ void bwd_tables_kernel(const int32_t* __restrict__ counts, int E, int H, int I,
                                  int32_t* __restrict__ poff, int32_t* __restrict__ goff_h,
                                  int32_t* __restrict__ pre_h, int32_t* __restrict__ goff_i,
                                  int32_t* __restrict__ pre_i) {
  if (threadIdx.x != 0) return;
  int acc = 0;
  const int th = (H + kGemmBM - 1) / kGemmBM, ti = (2 * I + kGemmBM - 1) / kGemmBM;
  for (int e = 0; e <= E; ++e) {
    poff[e] = acc;
    goff_h[e] = e * H;
    pre_h[e] = e * th;
    goff_i[e] = e * 2 * I;
    pre_i[e] = e * ti;
    if (e < E) {
      const int c = counts[e];
      const int padded = (c + 63) / 64 * 64;
      acc += padded > 64 ? padded : 64;
    }
  }
}

// dst[j][c] (pitch ld) for the padded column c of expert e (c in
// [poff[e], poff[e+1])): the value of feature j of permuted row
// r = offsets[e] + c - poff[e] if that row exists, else 0.  Row r of the
// source is src row perm[r] / k (gather != 0: x or dout, [T, C]) or src row r
// ([M, C]); scale != null multiplies it by scale[perm[r]] (the routing
// weight).  64 columns x 64 features per block through LDS.
__global__ __launch_bounds__(256) void gather_transpose_kernel(
    const uint16_t* __restrict__ src, int C, const int32_t* __restrict__ perm, int gather, int k,
    const float* __restrict__ scale, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ poff, int E, int64_t ld,
    uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][66];
  __shared__ int s_e;
  const int c0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  if (threadIdx.x == 0) {
    int lo = 0, hi = E;                    // largest e with poff[e] <= c0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (poff[mid] <= c0) lo = mid; else hi = mid;
    }
    s_e = c0 < poff[E] ? lo : -1;
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int q0 = c0 - poff[e];
  const int cnt = counts[e];
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int i = ty + 32 * p;              // column c0 + i of the destination
    float v[8];
    if (q0 + i < cnt) {
      const int64_t r = offsets[e] + q0 + i;
      const int64_t srow = gather ? perm[r] / k : r;
      load8(src + srow * C + j0 + tx * 8, v);
      if (scale) {
        const float s = scale[perm[r]];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] *= s;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) tile[i][tx * 8 + u] = f32_to_bf16(v[u]);
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int j = ty + 32 * p;
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[u] = tile[tx * 8 + 2 * u][j] | (static_cast<uint32_t>(tile[tx * 8 + 2 * u + 1][j]) << 16);
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(j0 + j) * ld + c0 + tx * 8) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// dg, du (into dgdu [M, 2I]) and h (into h [M, I]) from dh [M, I] (before
// the routing weight), g and u (gu [M, 2I]) and the routing weight of each
// row; 8 columns per thread.
__global__ __launch_bounds__(256) void bwd_swiglu_kernel(const uint16_t* __restrict__ dh,
                                                         const uint16_t* __restrict__ gu,
                                                         const float* __restrict__ wts,
                                                         const int32_t* __restrict__ perm, int64_t M,
                                                         int I, uint16_t* __restrict__ dgdu,
                                                         uint16_t* __restrict__ h) {
  const int64_t idx = blockIdx.x * 256LL + threadIdx.x;
  const int per_row = I / 8;
  if (idx >= M * per_row) return;
  const int64_t r = idx / per_row;
  const int c = static_cast<int>(idx % per_row) * 8;
  const float w = wts[perm[r]];
  float d[8], g[8], u[8], dg[8], du[8], hv[8];
  load8(dh + r * I + c, d);
  load8(gu + r * 2 * I + c, g);
  load8(gu + r * 2 * I + I + c, u);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float s = 1.f / (1.f + __expf(-g[q]));      // sigma(g)
    const float silu = g[q] * s;
    const float dhw = w * d[q];
    dg[q] = dhw * u[q] * (s * (1.f + g[q] * (1.f - s)));
    du[q] = dhw * silu;
    hv[q] = silu * u[q];
  }
  store8(dgdu + r * 2 * I + c, dg);
  store8(dgdu + r * 2 * I + I + c, du);
  store8(h + r * I + c, hv);
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = blockIdx.x * 256LL + threadIdx.x;
  if (i < n) p[i] = v;
}

inline uint32_t blocks(int64_t n, int per) { return static_cast<uint32_t>((n + per - 1) / per); }

}  // namespace

hipError_t launch_bwd_dw(const void* dout, const void* y, int64_t T, int H, int k, float* dw,
                         hipStream_t s) {
  hipLaunchKernelGGL(bwd_dw_kernel, dim3(blocks(T, 4)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(y), T, H, k, dw);
  return hipGetLastError();
}

hipError_t launch_bwd_router(const float* logits, const float* meta, const int32_t* ids,
                             const float* dw, int64_t T, int E, int k, int renorm, float* dl,
                             hipStream_t s) {
  hipLaunchKernelGGL(bwd_router_kernel, dim3(blocks(T, 4)), dim3(256), 0, s, logits, meta, ids, dw,
                     T, E, k, renorm, dl);
  return hipGetLastError();
}

int bwd_dwr_slices(int64_t T) {
  const int64_t s = T / 128;
  return static_cast<int>(s < 1 ? 1 : s > 64 ? 64 : s);
}

hipError_t launch_bwd_router_grads(const float* dl, const void* x, const void* w_router, int64_t T,
                                   int H, int E, void* dxr, float* dwr, float* db, float* part,
                                   hipStream_t s) {
  hipLaunchKernelGGL(bwd_dxr_kernel, dim3(blocks(T, kDxrTok), blocks(H, 256)), dim3(256), 0, s, dl,
                     static_cast<const uint16_t*>(w_router), T, H, E, static_cast<uint16_t*>(dxr));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int S = bwd_dwr_slices(T);
  const int64_t slice = (T + S - 1) / S;
  if (E <= 8)
    hipLaunchKernelGGL(bwd_dwr_partial_kernel<8>, dim3(1, blocks(H / kDwrCols, 256), S), dim3(256), 0, s,
                       dl, static_cast<const uint16_t*>(x), T, H, E, slice, part);
  else
    hipLaunchKernelGGL(bwd_dwr_partial_kernel<kDwrExp>, dim3(blocks(E, kDwrExp), blocks(H / kDwrCols, 256), S),
                       dim3(256), 0, s, dl, static_cast<const uint16_t*>(x), T, H, E, slice, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(E) * H;
  hipLaunchKernelGGL(bwd_dwr_reduce_kernel, dim3(blocks(n, 256)), dim3(256), 0, s, part, S, n, dwr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (db) hipLaunchKernelGGL(bwd_dbias_kernel, dim3(E), dim3(256), 0, s, dl, T, E, db);
  return hipGetLastError();
}

hipError_t launch_bwd_tables(const int32_t* counts, int E, int H, int I, int32_t* poff,
                             int32_t* goff_h, int32_t* pre_h, int32_t* goff_i, int32_t* pre_i,
                             hipStream_t s) {
  hipLaunchKernelGGL(bwd_tables_kernel, dim3(1), dim3(64), 0, s, counts, E, H, I, poff, goff_h, pre_h,
                     goff_i, pre_i);
  return hipGetLastError();
}

hipError_t launch_gather_transpose(const void* src, int C, const int32_t* perm, bool gather, int k,
                                   const float* scale, const int32_t* offsets, const int32_t* counts,
                                   const int32_t* poff, int E, int64_t ld, void* dst, hipStream_t s) {
  if (C % 64 || ld % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_transpose_kernel, dim3(static_cast<uint32_t>(ld / 64), C / 64), dim3(256),
                     0, s, static_cast<const uint16_t*>(src), C, perm, gather ? 1 : 0, k, scale,
                     offsets, counts, poff, E, ld, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_bwd_swiglu(const void* dh, const void* gu, const float* wts, const int32_t* perm,
                             int64_t M, int I, void* dgdu, void* h, hipStream_t s) {
  if (I % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_swiglu_kernel, dim3(blocks(M * (I / 8), 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(dh), static_cast<const uint16_t*>(gu), wts, perm, M,
                     I, static_cast<uint16_t*>(dgdu), static_cast<uint16_t*>(h));
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(blocks(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace moe
