// Router: logits, softmax over all experts, per-token top-k (gfx950).
//
// Page legend:
//   [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
//   [Hunyuan page]   "混合专家架构大模型Hunyuan-Large：原理剖析与实现机制"
//
// The gate is the linear layer W_g x + b_g followed by a softmax over all
// experts ([Hunyuan page] §二.1 gating formula); the k largest are kept
// ([Qwen3-MoE page] §1 forward listing).  Ties go to the lowest expert id and
// slot j holds the (j+1)-th largest logit.
//
// Exact selection.  The fp32 logits differ from the exact ones by at most
//   delta_t = D * 2^-23 * (1 + D*2^-23) * S_t,
//   S_t = ||x_t||_2 * max_e ||W_e||_2 + max_e |b_e|   (bounds sum_h |x_th W_eh| + |b_e|),
// where D is the longest chain of roundings any product passes through in the
// summation structure below (each MFMA is treated as a chain of 16 rounded
// additions, each rounding worth at most 2^-23 relative, i.e. even a
// truncating adder is covered).  A token is flagged when its fp32 top-k is not
// provably the exact one: some expert outside the top-k is within 2*delta of
// the k-th logit, or two adjacent top-k logits are within 2*delta.  Flagged
// tokens are re-ranked by route_refine with float64 dot products (exact
// products, float64 sums) over the candidate set {e : L_k - L_e <= 2*delta},
// which provably contains the exact top-k.
#include "moe_internal.h"
#include "cdna4.h"

#include <math.h>

namespace moe {
namespace {

constexpr int RT = kRouteTok;   // tokens per workgroup
constexpr float kUlp2 = 1.1920928955078125e-07f;   // 2^-23
constexpr float kSafety = 1.0009765625f;            // 1 + 2^-10

__device__ __forceinline__ float xor_sum8(float v) {   // sum over an 8-lane group
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  return v;
}

// delta from the squared norms (see file comment).
__device__ __forceinline__ float route_delta(float xsq, float wsq_max, float bmax, int depth) {
  float S = sqrtf(xsq) * sqrtf(wsq_max) * kSafety * kSafety + bmax;
  float d = static_cast<float>(depth) * kUlp2;
  return d * (1.f + d) * S * kSafety;
}

// Softmax + top-k + near-tie flag for the RT tokens of a workgroup whose fp32
// logits (without bias) sit in lg[RT][EP+1].  8 threads per token.
template <int EP>
__device__ void route_select(const RouteArgs& a, int64_t t0, float (*lg)[EP + 1],
                             const float* delta) {
  constexpr int PER = EP / 8;
  const int tid = threadIdx.x;
  const int tok = tid >> 3, sub = tid & 7;
  const int64_t t = t0 + tok;
  const int E = a.E, k = a.k;

  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int e = sub + 8 * i;
    v[i] = (e < E) ? lg[tok][e] + (a.bias ? a.bias[e] : 0.f) : -INFINITY;
  }

  // k rounds of (max value, lowest id) selection over the 8-lane group.
  uint32_t taken = 0;
  float sel_v[kMaxK];
  int sel_e[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int e = sub + 8 * i;
        bool free_ = !((taken >> i) & 1u) && e < E;
        if (free_ && (v[i] > bv || (v[i] == bv && e < be))) { bv = v[i]; be = e; }
      }
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) {
        float ov = __shfl_xor(bv, off);
        int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      sel_v[j] = bv;
      sel_e[j] = be;
      if ((be & 7) == sub) taken |= 1u << (be >> 3);
    }
  }

  const float mx = sel_v[0];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (sub + 8 * i < E) s += __expf(v[i] - mx);
  s = xor_sum8(s);

  const float band = 2.f * delta[tok] * kSafety;
  const float vk = sel_v[k - 1];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (sub + 8 * i < E && (vk - v[i]) <= band) ++cnt;
  cnt += __shfl_xor(cnt, 1);
  cnt += __shfl_xor(cnt, 2);
  cnt += __shfl_xor(cnt, 4);
  bool flag = cnt > k;
#pragma unroll
  for (int j = 0; j + 1 < kMaxK; ++j)
    if (j + 1 < k && (sel_v[j] - sel_v[j + 1]) <= band) flag = true;

  if (t >= a.T) return;
  float p[kMaxK];
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) { p[j] = __expf(sel_v[j] - mx) / s; ps += p[j]; }
  if (sub < k) {
    float pj = 0.f;
    int ej = 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j == sub) { pj = p[j]; ej = sel_e[j]; }
    a.ids[t * k + sub] = ej;
    a.weights[t * k + sub] = a.renorm ? pj / ps : pj;
  }
  if (sub == 0) a.flag[t] = flag ? 1 : 0;
  if (flag) {
    if (sub == 0) {
      a.meta[t * 4 + 0] = mx;
      a.meta[t * 4 + 1] = s;
      a.meta[t * 4 + 2] = band;
      a.meta[t * 4 + 3] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int e = sub + 8 * i;
      if (e < E) a.logits[t * E + e] = v[i];
    }
  }
}

// ---------------------------------------------------------------- bf16 path
// Logits: a workgroup owns 128 tokens x 64 experts; wave w multiplies tokens
// 32w..32w+31 by both 32-expert halves (MFMA 32x32x16, router rows as A,
// tokens as B).  K moves in 64-wide stages through four LDS buffers, loaded
// by direct-to-LDS DMA three stages ahead.  Each stage's four MFMAs start
// from zero and are then added to the running sum (the summation structure
// the error bound counts).  Squared norms of the token rows and router rows
// are summed from the very operand fragments the MFMAs consume.
constexpr int LT = 128;               // tokens per workgroup
constexpr int LE = 64;                // experts per workgroup
constexpr int LBK = 64;               // K per stage
constexpr int LSTAGE = (LT + LE) * 8; // uint4 per stage buffer

__device__ __forceinline__ float sumsq8(const bf16x8_t& v) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float f = static_cast<float>(v[i]);
    s = fmaf(f, f, s);
  }
  return s;
}

__global__ __launch_bounds__(256) void route_logits_bf16_kernel(RouteArgs a) {
  __shared__ uint4 R0[LSTAGE];
  __shared__ uint4 R1[LSTAGE];
  __shared__ uint4 R2[LSTAGE];
  __shared__ uint4 R3[LSTAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * LT;
  const int e0 = blockIdx.y * LE;
  const int H = a.H, E = a.E;
  const int nk = H / LBK;
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);

  // DMA rows of this lane (clamped in bounds; clamped rows are never stored)
  const int lchunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow = 8 * wave + (lane >> 3);
  const uint16_t* xp[4];
  const uint16_t* wp[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t t = t0 + lrow + 32 * j;
    t = t < a.T ? t : a.T - 1;
    xp[j] = X + t * H + lchunk * 8;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int e = e0 + lrow + 32 * j;
    e = e < E ? e : E - 1;
    wp[j] = W + static_cast<int64_t>(e) * H + lchunk * 8;
  }
  const uint32_t wofs = static_cast<uint32_t>(wave) * 64 * 16;
  const uint32_t rb0 = __builtin_amdgcn_readfirstlane(lds_addr(R0) + wofs);
  const uint32_t rb1 = __builtin_amdgcn_readfirstlane(lds_addr(R1) + wofs);
  const uint32_t rb2 = __builtin_amdgcn_readfirstlane(lds_addr(R2) + wofs);
  const uint32_t rb3 = __builtin_amdgcn_readfirstlane(lds_addr(R3) + wofs);
  auto issue = [&](int kc, uint32_t rb) {
    const int ko = kc * LBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(xp[j] + ko, rb + j * 4 * 64 * 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(wp[j] + ko, rb + LT * 8 * 16 + j * 4 * 64 * 16);
  };

  f32x16_t acc[2];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  float xsq = 0.f, wsq[2] = {0.f, 0.f};

  auto step = [&](int kc, const uint4* Rs, uint32_t rbn) {
    const int after = nk - 1 - kc;          // stages issued after kc (at most 2)
    if (after >= 2) wait_vmcnt12();
    else if (after == 1) wait_vmcnt6();
    else wait_vmcnt0();
    lds_barrier();
    if (kc + 3 < nk) issue(kc + 3, rbn);
    f32x16_t part[2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[n][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 2 * s + (lane >> 5);
      const bf16x8_t bx = *reinterpret_cast<const bf16x8_t*>(&Rs[swz128(wave * 32 + (lane & 31), c)]);
      xsq += sumsq8(bx);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const bf16x8_t aw =
            *reinterpret_cast<const bf16x8_t*>(&Rs[LT * 8 + swz128(n * 32 + (lane & 31), c)]);
        wsq[n] += sumsq8(aw);
        part[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, bx, part[n], 0, 0, 0);
      }
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[n] += part[n];
  };

  issue(0, rb0);
  if (1 < nk) issue(1, rb1);
  if (2 < nk) issue(2, rb2);
  int kc = 0;
  for (; kc + 4 <= nk; kc += 4) {
    step(kc, R0, rb3);
    step(kc + 1, R1, rb0);
    step(kc + 2, R2, rb1);
    step(kc + 3, R3, rb2);
  }
  if (kc < nk) step(kc, R0, rb3);       // H is a multiple of 64: 0..3 stages remain
  if (kc + 1 < nk) step(kc + 1, R1, rb0);
  if (kc + 2 < nk) step(kc + 2, R2, rb1);

  // norms: lanes l and l+32 hold the two K halves of the same row
  xsq += __shfl_xor(xsq, 32);
#pragma unroll
  for (int n = 0; n < 2; ++n) wsq[n] += __shfl_xor(wsq[n], 32);
  const int64_t t = t0 + wave * 32 + (lane & 31);
  if (blockIdx.y == 0 && lane < 32 && t < a.T) a.xnorm2[t] = xsq;
  if (blockIdx.x == 0 && wave == 0 && lane < 32) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int e = e0 + n * 32 + lane;
      if (e < E) a.wnorm2[e] = wsq[n];
    }
  }
  // logits: lane holds token t and experts 8(r/4) + 4(lane/32) + (r%4) of each half
  if (t < a.T) {
    float* row = a.logits + t * E;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = e0 + n * 32 + 8 * g + 4 * (lane >> 5);
        if ((E & 3) == 0) {
          if (e < E)
            *reinterpret_cast<float4*>(row + e) =
                make_float4(acc[n][4 * g], acc[n][4 * g + 1], acc[n][4 * g + 2], acc[n][4 * g + 3]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (e + q < E) row[e + q] = acc[n][4 * g + q];
        }
      }
  }
}

// Softmax + top-k + near-tie flag for 32 tokens per workgroup from the fp32
// logits, with delta from the squared norms (see the file comment).
template <int EP>
__global__ __launch_bounds__(256) void route_select_bf16_kernel(RouteArgs a) {
  __shared__ float lg[RT][EP + 1];
  __shared__ float delta_s[RT];
  __shared__ unsigned wmax_bits, bmax_bits;
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;
  const int E = a.E;
  if (tid == 0) { wmax_bits = 0u; bmax_bits = 0u; }
  __syncthreads();
  if (tid < E) {
    atomicMax(&wmax_bits, __float_as_uint(a.wnorm2[tid]));
    if (a.bias) atomicMax(&bmax_bits, __float_as_uint(fabsf(a.bias[tid])));
  }
  for (int i = tid; i < RT * E; i += 256) {
    const int tk = i / E, e = i - tk * E;
    const int64_t t = t0 + tk;
    lg[tk][e] = (t < a.T) ? a.logits[t * E + e] : 0.f;
  }
  __syncthreads();
  if (tid < RT) {
    const int64_t t = t0 + tid;
    const int nch = a.H / LBK;
    const int depth = 64 + nch + 2;       // 4 MFMAs per stage, stage sums, bias
    delta_s[tid] = route_delta(t < a.T ? a.xnorm2[t] : 0.f, __uint_as_float(wmax_bits),
                               __uint_as_float(bmax_bits), depth);
  }
  __syncthreads();
  route_select<EP>(a, t0, lg, delta_s);
}

// ----------------------------------------------------------------- f32 path
// Plain fp32 FMA chains (no reduced-precision matrix path).  Thread = one
// token (tid % 32) x experts tid/32 + 8 i.  K is summed in chunks of 64 from
// zero and the chunk sums are added in order.
template <int EP>
__global__ __launch_bounds__(256) void route_f32_kernel(RouteArgs a) {
  constexpr int PER = EP / 8;
  constexpr int KF = 64;
  __shared__ float xs[RT][KF + 1];
  __shared__ float lg[RT][EP + 1];
  __shared__ float xsq_s[RT];
  __shared__ float delta_s[RT];
  __shared__ unsigned wmax_bits, bmax_bits;

  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;
  const int H = a.H, E = a.E;
  const float* X = static_cast<const float*>(a.x);
  const float* W = static_cast<const float*>(a.w);
  if (tid == 0) { wmax_bits = 0u; bmax_bits = 0u; }

  const int tok = tid & 31, eg = tid >> 5;
  const int lrow = tid >> 3, lc = tid & 7;
  const int64_t tl = t0 + lrow;
  float acc[PER], wsq[PER], xsq = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) { acc[i] = 0.f; wsq[i] = 0.f; }

  const int nch = H / KF;
  for (int ch = 0; ch < nch; ++ch) {
    __syncthreads();
    const int64_t ko = static_cast<int64_t>(ch) * KF + lc * 8;
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (tl < a.T) {
      x0 = *reinterpret_cast<const float4*>(X + tl * H + ko);
      x1 = *reinterpret_cast<const float4*>(X + tl * H + ko + 4);
    }
    xsq = fmaf(x0.x, x0.x, xsq); xsq = fmaf(x0.y, x0.y, xsq);
    xsq = fmaf(x0.z, x0.z, xsq); xsq = fmaf(x0.w, x0.w, xsq);
    xsq = fmaf(x1.x, x1.x, xsq); xsq = fmaf(x1.y, x1.y, xsq);
    xsq = fmaf(x1.z, x1.z, xsq); xsq = fmaf(x1.w, x1.w, xsq);
    float* xd = &xs[lrow][lc * 8];
    xd[0] = x0.x; xd[1] = x0.y; xd[2] = x0.z; xd[3] = x0.w;
    xd[4] = x1.x; xd[5] = x1.y; xd[6] = x1.z; xd[7] = x1.w;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = eg + 8 * i;
      if (e >= E) continue;
      const float* wrow = W + static_cast<int64_t>(e) * H + static_cast<int64_t>(ch) * KF;
      float part = 0.f, sq = 0.f;
      for (int kk = 0; kk < KF; ++kk) {
        float wv = wrow[kk];
        part = fmaf(xs[tok][kk], wv, part);
        sq = fmaf(wv, wv, sq);
      }
      acc[i] += part;
      wsq[i] += sq;
    }
  }
  xsq = xor_sum8(xsq);
  if (lc == 0) xsq_s[lrow] = xsq;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = eg + 8 * i;
    if (e < E) {
      lg[tok][e] = acc[i];
      if (tok == 0) atomicMax(&wmax_bits, __float_as_uint(wsq[i]));
    }
  }
  if (a.bias && tid < E) atomicMax(&bmax_bits, __float_as_uint(fabsf(a.bias[tid])));
  __syncthreads();
  if (tid < RT) {
    const int depth = KF + nch + 1;
    delta_s[tid] = route_delta(xsq_s[tid], __uint_as_float(wmax_bits), __uint_as_float(bmax_bits), depth);
  }
  __syncthreads();
  route_select<EP>(a, t0, lg, delta_s);
}

// ------------------------------------------------------------------ refine
// One wave per flagged token: float64 logits of the candidate set, exact
// re-ranking by (logit desc, id asc); weights from the stored fp32 softmax.
template <typename ELEM>
__global__ __launch_bounds__(256) void route_refine_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  if (a.flag[t] == 0) return;
  const int E = a.E, k = a.k, H = a.H;
  constexpr int VEC = 16 / sizeof(ELEM);
  const float mx = a.meta[t * 4 + 0], s = a.meta[t * 4 + 1], band = a.meta[t * 4 + 2];

  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    v[q] = (e < E) ? a.logits[t * E + e] : -INFINITY;
  }
  // fp32 k-th largest (same rule as the first pass)
  uint32_t taken = 0;
  float vk = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (e < E && !((taken >> q) & 1u) && (v[q] > bv || (v[q] == bv && e < be))) { bv = v[q]; be = e; }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      float ov = __shfl_xor(bv, off);
      int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    vk = bv;
  }

  const ELEM* xrow = static_cast<const ELEM*>(a.x) + t * H;
  double d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    const bool cand = e < E && (vk - v[q]) <= band;
    d[q] = -INFINITY;
    unsigned long long m = __ballot(cand);
    while (m) {
      const int ln = __ffsll(static_cast<long long>(m)) - 1;
      m &= m - 1;
      const int ec = ln + 64 * q;
      const ELEM* wrow = static_cast<const ELEM*>(a.w) + static_cast<int64_t>(ec) * H;
      double accd = 0.0;
      for (int c = lane; c * VEC < H; c += 64) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xrow + c * VEC);
        const uint4 wv = *reinterpret_cast<const uint4*>(wrow + c * VEC);
        const ELEM* xe = reinterpret_cast<const ELEM*>(&xv);
        const ELEM* wq = reinterpret_cast<const ELEM*>(&wv);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          double xf, wf;
          if constexpr (sizeof(ELEM) == 2) {
            xf = static_cast<double>(bf16_to_f32(xe[i]));
            wf = static_cast<double>(bf16_to_f32(wq[i]));
          } else {
            xf = static_cast<double>(xe[i]);
            wf = static_cast<double>(wq[i]);
          }
          accd = fma(xf, wf, accd);
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) accd += __shfl_xor(accd, off);
      if (a.bias) accd += static_cast<double>(a.bias[ec]);
      if (lane == ln) d[q] = accd;
    }
  }

  // exact top-k over the candidates
  taken = 0;
  float p[kMaxK];
  int ids[kMaxK];
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      double bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        if (e < E && !((taken >> q) & 1u) && d[q] != -INFINITY && (d[q] > bv || (d[q] == bv && e < be))) {
          bv = d[q];
          be = e;
        }
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        double ov = __shfl_xor(bv, off);
        int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      // fp32 logit of the chosen expert from its owner lane
      const int q = be >> 6;
      float lv = (q == 0) ? v[0] : (q == 1) ? v[1] : (q == 2) ? v[2] : v[3];
      lv = __shfl(lv, be & 63);
      ids[j] = be;
      p[j] = __expf(lv - mx) / s;
      ps += p[j];
    }
  }
  if (lane < k) {
    float pj = 0.f;
    int ej = 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j == lane) { pj = p[j]; ej = ids[j]; }
    a.ids[t * k + lane] = ej;
    a.weights[t * k + lane] = a.renorm ? pj / ps : pj;
  }
}

template <int EP>
hipError_t launch_select_bf16(const RouteArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.T + RT - 1) / RT);
  hipLaunchKernelGGL((route_select_bf16_kernel<EP>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int EP>
hipError_t launch_f32(const RouteArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.T + RT - 1) / RT);
  hipLaunchKernelGGL((route_f32_kernel<EP>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t route_scratch_bytes(int64_t T, int E) {
  return align_up(static_cast<size_t>(T) * 4, 256) + align_up(static_cast<size_t>(T) * 16, 256) +
         align_up(static_cast<size_t>(T) * E * 4, 256) + align_up(static_cast<size_t>(T) * 4, 256) +
         align_up(static_cast<size_t>(E) * 4, 256);
}

hipError_t launch_route(const RouteArgs& a, bool bf16, hipStream_t s) {
  // every scratch region must have been carved before anything is launched
  if (!a.x || !a.w || !a.ids || !a.weights || !a.flag || !a.meta || !a.logits ||
      (bf16 && (!a.xnorm2 || !a.wnorm2)))
    return hipErrorInvalidValue;
  hipError_t err;
  if (bf16) {
    const dim3 grid(static_cast<unsigned>((a.T + LT - 1) / LT), static_cast<unsigned>((a.E + LE - 1) / LE));
    hipLaunchKernelGGL(route_logits_bf16_kernel, grid, dim3(256), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.E <= 32) err = launch_select_bf16<32>(a, s);
    else if (a.E <= 64) err = launch_select_bf16<64>(a, s);
    else if (a.E <= 128) err = launch_select_bf16<128>(a, s);
    else err = launch_select_bf16<256>(a, s);
  } else {
    if (a.E <= 32) err = launch_f32<32>(a, s);
    else if (a.E <= 64) err = launch_f32<64>(a, s);
    else if (a.E <= 128) err = launch_f32<128>(a, s);
    else err = launch_f32<256>(a, s);
  }
  if (err != hipSuccess) return err;
  const unsigned grid = static_cast<unsigned>((a.T + 3) / 4);
  if (bf16) hipLaunchKernelGGL((route_refine_kernel<uint16_t>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((route_refine_kernel<float>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
