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
#include <type_traits>

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

// Softmax + top-k + near-tie flag for the 256 / LPT tokens of a workgroup
// whose fp32 logits (without bias) sit in lg[256 / LPT][EP + 1].  LPT lanes
// per token, each holding EP / LPT logits (experts sub + LPT i).
template <int EP, int LPT>
__device__ void route_select(const RouteArgs& a, int64_t t0, float (*lg)[EP + 1],
                             const float* delta) {
  constexpr int PER = EP / LPT;
  const int tid = threadIdx.x;
  const int tok = tid / LPT, sub = tid % LPT;
  const int64_t t = t0 + tok;
  const int E = a.E, k = a.k;
  auto group_sum = [](float v) {
#pragma unroll
    for (int off = 1; off < LPT; off <<= 1) v += __shfl_xor(v, off);
    return v;
  };

  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int e = sub + LPT * i;
    v[i] = (e < E) ? lg[tok][e] + (a.bias ? a.bias[e] : 0.f) : -INFINITY;
  }

  // k rounds of (max value, lowest id) selection over the LPT-lane group.
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
        int e = sub + LPT * i;
        bool free_ = !((taken >> i) & 1u) && e < E;
        if (free_ && (v[i] > bv || (v[i] == bv && e < be))) { bv = v[i]; be = e; }
      }
#pragma unroll
      for (int off = 1; off < LPT; off <<= 1) {
        float ov = __shfl_xor(bv, off);
        int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      sel_v[j] = bv;
      sel_e[j] = be;
      if ((be % LPT) == sub) taken |= 1u << (be / LPT);
    }
  }

  const float mx = sel_v[0];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (sub + LPT * i < E) s += __expf(v[i] - mx);
  s = group_sum(s);

  const float band = 2.f * delta[tok] * kSafety;
  const float vk = sel_v[k - 1];
  float cnt = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (sub + LPT * i < E && (vk - v[i]) <= band) cnt += 1.f;
  cnt = group_sum(cnt);
  bool flag = cnt > static_cast<float>(k);
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
  if (flag || a.keep_all) {
    if (sub == 0) {
      a.meta[t * 4 + 0] = mx;
      a.meta[t * 4 + 1] = s;
      a.meta[t * 4 + 2] = band;
      a.meta[t * 4 + 3] = vk;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int e = sub + LPT * i;
      if (e < E) a.logits[t * E + e] = v[i];
    }
  }
}

// ---------------------------------------------------------------- bf16 path
// Logits: a workgroup owns 128 tokens x 64 (E > 64: 128) experts; wave w
// multiplies tokens 32w..32w+31 by every 32-expert part (MFMA 32x32x16,
// router rows as A, tokens as B).  K moves in 64-wide stages through four LDS buffers, loaded
// by direct-to-LDS DMA three stages ahead.  Each stage's four MFMAs start
// from zero and are then added to the running sum (the summation structure
// the error bound counts).  Squared norms of the token rows and router rows
// are summed from the very operand fragments the MFMAs consume.
constexpr int LT = 128;               // tokens per workgroup
constexpr int LBK = 64;               // K per stage
// experts per workgroup: 64 (two 32-expert MFMA halves per wave) or, for
// E > 64, 128 (four), which halves the re-reads of x across expert blocks
__host__ __device__ constexpr int route_ne(int E) { return E > 64 ? 4 : 2; }

// s_waitcnt immediate for vmcnt(n), n < 64 (expcnt / lgkmcnt at their maxima)
constexpr int vmcnt_code(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// sum of squares of 8 bf16 by packed dot products (v_dot2c_f32_bf16); every
// term is non-negative, and a square the instruction might flush (below
// 2^-126) is covered by the slack the norm gets before use
__device__ __forceinline__ float sumsq8_dot(const bf16x8_t& v, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2_t p = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}

__device__ __forceinline__ float sumsq8(const bf16x8_t& v) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float f = static_cast<float>(v[i]);
    s = fmaf(f, f, s);
  }
  return s;
}

template <int NE>
__global__ __launch_bounds__(256) void route_logits_bf16_kernel(RouteArgs a) {
  constexpr int LE = 32 * NE;
  constexpr int LSTAGE = (LT + LE) * 8;   // uint4 per stage buffer
  constexpr int ND = 4 + NE;              // DMAs per lane per stage
  __shared__ uint4 R[4][LSTAGE];       // ring of 4 stage buffers
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * LT;
  const int e0 = blockIdx.y * LE;
  const int H = a.H, E = a.E;
  // K range z of ksplit: stages [kb, kb + nk) of the H / 64
  const int z = blockIdx.z, nch = H / LBK;
  const int kb = z * nch / a.ksplit;
  const int nk = (z + 1) * nch / a.ksplit - kb;
  const uint16_t* X = static_cast<const uint16_t*>(a.x) + kb * LBK;
  const uint16_t* W = static_cast<const uint16_t*>(a.w) + kb * LBK;

  // DMA rows of this lane (clamped in bounds; clamped rows are never
  // stored): scalar tile bases plus 32-bit lane offsets, no per-DMA ALU work
  const int lchunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow = 8 * wave + (lane >> 3);
  const char* xbase = reinterpret_cast<const char*>(X + t0 * H);
  const char* wbase = reinterpret_cast<const char*>(W + static_cast<int64_t>(e0) * H);
  uint32_t xo[4], wo[NE];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t t = t0 + lrow + 32 * j;
    t = t < a.T ? t : a.T - 1;
    xo[j] = static_cast<uint32_t>((t - t0) * H * 2 + lchunk * 16);
  }
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    int e = e0 + lrow + 32 * j;
    e = e < E ? e : E - 1;
    wo[j] = static_cast<uint32_t>((e - e0) * H * 2 + lchunk * 16);
  }
  const uint32_t wofs = static_cast<uint32_t>(wave) * 64 * 16;
  const uint32_t rb = __builtin_amdgcn_readfirstlane(lds_addr(&R[0][0]) + wofs);
  auto issue = [&](int kc) {
    const int ko = kc * LBK * 2;
    const uint32_t dst = rb + (kc & 3) * LSTAGE * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16s(xbase + ko, xo[j], dst + j * 4 * 64 * 16);
#pragma unroll
    for (int j = 0; j < NE; ++j) dma16s(wbase + ko, wo[j], dst + LT * 8 * 16 + j * 4 * 64 * 16);
  };

  f32x16_t acc[NE];
#pragma unroll
  for (int n = 0; n < NE; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  float xsq = 0.f, wsq[NE];
#pragma unroll
  for (int n = 0; n < NE; ++n) wsq[n] = 0.f;

  // router-row norms: only wave 0 of the first token block stores them (a
  // wave-uniform choice, taken once per stage outside the MFMA sequence)
  const bool wnorms = blockIdx.x == 0 && __builtin_amdgcn_readfirstlane(wave) == 0;
  auto multiply = [&](const uint4* Rs, f32x16_t* part, auto with_w) {
    // all fragments of the stage first, so their LDS latencies overlap
    bf16x8_t bx[4], aw[4][NE];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 2 * s + (lane >> 5);
      bx[s] = *reinterpret_cast<const bf16x8_t*>(&Rs[swz128(wave * 32 + (lane & 31), c)]);
#pragma unroll
      for (int n = 0; n < NE; ++n)
        aw[s][n] = *reinterpret_cast<const bf16x8_t*>(&Rs[LT * 8 + swz128(n * 32 + (lane & 31), c)]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      xsq = sumsq8_dot(bx[s], xsq);
#pragma unroll
      for (int n = 0; n < NE; ++n) {
        if constexpr (decltype(with_w)::value) wsq[n] += sumsq8(aw[s][n]);
        part[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[s][n], bx[s], part[n], 0, 0, 0);
      }
    }
  };
  issue(0);
  if (1 < nk) issue(1);
  if (2 < nk) issue(2);
  for (int kc = 0; kc < nk; ++kc) {
    const int after = nk - 1 - kc;          // stages issued after kc (at most 2)
    // loads of a wave complete in order: keep the newer stages' ND DMAs each
    if (after >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_code(2 * ND));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_code(ND));
    else wait_vmcnt0();
    lds_barrier();
    if (kc + 3 < nk) issue(kc + 3);
    const uint4* Rs = R[kc & 3];
    f32x16_t part[NE];
#pragma unroll
    for (int n = 0; n < NE; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[n][r] = 0.f;
    if (wnorms) multiply(Rs, part, std::true_type{});
    else multiply(Rs, part, std::false_type{});
#pragma unroll
    for (int n = 0; n < NE; ++n) acc[n] += part[n];
  }

  // norms: lanes l and l+32 hold the two K halves of the same row
  xsq += __shfl_xor(xsq, 32);
#pragma unroll
  for (int n = 0; n < NE; ++n) wsq[n] += __shfl_xor(wsq[n], 32);
  const int64_t t = t0 + wave * 32 + (lane & 31);
  if (blockIdx.y == 0 && lane < 32 && t < a.T) a.xnorm2[z * a.T + t] = xsq;
  if (wnorms && lane < 32) {
#pragma unroll
    for (int n = 0; n < NE; ++n) {
      const int e = e0 + n * 32 + lane;
      if (e < E) a.wnorm2[z * E + e] = wsq[n];
    }
  }
  // logits: lane holds token t and experts 8(r/4) + 4(lane/32) + (r%4) of each half
  if (t < a.T) {
    float* row = a.logits + (z * a.T + t) * E;
#pragma unroll
    for (int n = 0; n < NE; ++n)
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

// Softmax + top-k + near-tie flag from the fp32 logits, with delta from the
// squared norms (see the file comment).  max(8, EP / 8) lanes per token, so
// every lane holds at most 8 logits.
template <int EP>
__global__ __launch_bounds__(256) void route_select_bf16_kernel(RouteArgs a) {
  constexpr int LPT = EP / 8 > 8 ? EP / 8 : 8;
  constexpr int NT = 256 / LPT;           // tokens per workgroup
  __shared__ float lg[NT][EP + 1];
  __shared__ float delta_s[NT];
  __shared__ unsigned wmax_bits, bmax_bits;
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * NT;
  const int E = a.E;
  const int ks = a.ksplit;
  if (tid == 0) { wmax_bits = 0u; bmax_bits = 0u; }
  __syncthreads();
  if (tid < E) {
    float w2 = 0.f;
    for (int z = 0; z < ks; ++z) w2 += a.wnorm2[z * E + tid];
    atomicMax(&wmax_bits, __float_as_uint(w2));
    if (a.bias) atomicMax(&bmax_bits, __float_as_uint(fabsf(a.bias[tid])));
  }
  // logits = the K ranges' partial sums added in range order
  for (int i = tid; i < NT * E; i += 256) {
    const int tk = i / E, e = i - tk * E;
    const int64_t t = t0 + tk;
    float v = 0.f;
    if (t < a.T)
      for (int z = 0; z < ks; ++z) v += a.logits[(z * a.T + t) * E + e];
    lg[tk][e] = v;
  }
  __syncthreads();
  if (tid < NT) {
    const int64_t t = t0 + tid;
    float x2 = 0.f;
    if (t < a.T)
      for (int z = 0; z < ks; ++z) x2 += a.xnorm2[z * a.T + t];
    x2 += static_cast<float>(a.H) * 1.1754943508222875e-38f;   // H * 2^-126: flushed squares
    const int nch = a.H / LBK;
    // 4 chained MFMAs per stage, stage sums within a range, range sums, bias
    const int depth = 64 + (nch + ks - 1) / ks + ks + 2;
    delta_s[tid] = route_delta(x2, __uint_as_float(wmax_bits), __uint_as_float(bmax_bits), depth);
  }
  __syncthreads();
  route_select<EP, LPT>(a, t0, lg, delta_s);
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
  route_select<EP, 8>(a, t0, lg, delta_s);
}

// ------------------------------------------------------------------ refine
// Position of the i-th set bit (from 0) of m, i < popcount(m).
__device__ __forceinline__ int nth_set_bit(unsigned long long m, int i) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __popcll(m & ((1ull << w) - 1ull));
    if (i >= c) { i -= c; m >>= w; pos += w; }
  }
  return pos;
}

// One wave per flagged token.  The candidates C = {e : L_k - L_e <= band}
// hold the exact top-k.  Within C only the ambiguous ones -- those whose
// fp32 logit lies within band of another candidate's -- need their exact
// (float64: exact products, float64 sums) logit: for an unambiguous e and any
// other candidate e', |v_e - v_e'| > band >= 2 delta, so v_e against either
// v_e' or the exact L_e' orders them as L_e against L_e'.  The exact top-k
// by (logit desc, id asc) is then taken over C with exact logits for the
// ambiguous candidates and fp32 ones for the rest.  Weights come from the
// stored fp32 softmax.
template <typename ELEM>
__global__ __launch_bounds__(256) void route_refine_kernel(RouteArgs a) {
  __shared__ float cv[4][kMaxE];     // candidate fp32 logits, in candidate order
  __shared__ int ce[4][kMaxE];       // candidate expert ids
  __shared__ double cd[4][kMaxE];    // candidate logits used for the final ranking
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);
  if (t >= a.T) return;
  if (a.flag[t] == 0) return;
  const int E = a.E, k = a.k, H = a.H;
  constexpr int VEC = 16 / sizeof(ELEM);
  const float mx = a.meta[t * 4 + 0], s = a.meta[t * 4 + 1], band = a.meta[t * 4 + 2];
  const float vk = a.meta[t * 4 + 3];
  const unsigned long long below = (1ull << lane) - 1ull;

  // candidate list (expert order), fp32 logits
  float v[4];
  int nc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    v[q] = (e < E) ? a.logits[t * E + e] : -INFINITY;
    const bool cand = e < E && (vk - v[q]) <= band;
    const unsigned long long m = __ballot(cand);
    if (cand) {
      const int i = nc + __popcll(m & below);
      cv[wave][i] = v[q];
      ce[wave][i] = e;
    }
    nc += __popcll(m);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();

  // ambiguity and default (fp32) ranking logits; amb[q] of candidate lane + 64 q
  unsigned long long am[4];
  int na = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    bool amb = false;
    if (i < nc) {
      const float vi = cv[wave][i];
      for (int j = 0; j < nc; ++j)
        if (j != i && fabsf(vi - cv[wave][j]) <= band) amb = true;
      cd[wave][i] = static_cast<double>(vi);
    }
    am[q] = __ballot(amb);
    na += __popcll(am[q]);
  }
  auto amb_index = [&](int r) -> int {    // candidate index of the r-th ambiguous one
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = __popcll(am[q]);
      if (r < c) return 64 * q + nth_set_bit(am[q], r);
      r -= c;
    }
    return 0;
  };

  const ELEM* xrow = static_cast<const ELEM*>(a.x) + t * H;
  // P ambiguous candidates at a time (a power of two >= na, at most 8), G =
  // 64 / P lanes each; a lane sums chunks sub, sub + G, ... with 4 loads of x
  // and of W in flight
  const int P = na <= 1 ? 1 : na <= 2 ? 2 : na <= 4 ? 4 : 8;
  const int G = 64 / P;
  const int slot = lane / G, sub = lane % G;
  const int nchunk = H / VEC;
  auto dot_chunk = [&](const uint4& xv, const uint4& wv, double acc) {
    const ELEM* xe = reinterpret_cast<const ELEM*>(&xv);
    const ELEM* wq = reinterpret_cast<const ELEM*>(&wv);
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
      double xf, wf;
      if constexpr (sizeof(ELEM) == 2) {
        xf = static_cast<double>(bf16_to_f32(xe[u]));
        wf = static_cast<double>(bf16_to_f32(wq[u]));
      } else {
        xf = static_cast<double>(xe[u]);
        wf = static_cast<double>(wq[u]);
      }
      acc = fma(xf, wf, acc);
    }
    return acc;
  };
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  for (int r0 = 0; r0 < na; r0 += P) {
    const int r = r0 + slot;
    const bool live = r < na;
    const int ci = live ? amb_index(r) : 0;
    const int ec = live ? ce[wave][ci] : 0;
    const ELEM* wrow = static_cast<const ELEM*>(a.w) + static_cast<int64_t>(ec) * H;
    double accd = 0.0;
    int c = sub;
    for (; c + 3 * G < nchunk; c += 4 * G) {
      uint4 xv[4], wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xv[u] = *reinterpret_cast<const uint4*>(xrow + (c + u * G) * VEC);
        wv[u] = *reinterpret_cast<const uint4*>(wrow + (c + u * G) * VEC);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) accd = dot_chunk(xv[u], wv[u], accd);
    }
    for (; c < nchunk; c += G) {
      const uint4 xv = *reinterpret_cast<const uint4*>(xrow + c * VEC);
      const uint4 wv = *reinterpret_cast<const uint4*>(wrow + c * VEC);
      accd = dot_chunk(xv, wv, accd);
    }
    for (int off = 1; off < G; off <<= 1) accd += __shfl_xor(accd, off);
    if (a.bias) accd += static_cast<double>(a.bias[ec]);
    if (live && sub == 0) cd[wave][ci] = accd;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();

  // exact top-k over the candidates, lane owns candidates lane + 64 q
  double d[4];
  int de[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    d[q] = i < nc ? cd[wave][i] : -INFINITY;
    de[q] = i < nc ? ce[wave][i] : 0x7fffffff;
  }
  uint32_t taken = 0;
  float p[kMaxK];
  int ids[kMaxK];
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      double bv = -INFINITY;
      int be = 0x7fffffff, bq = -1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (lane + 64 * q < nc && !((taken >> q) & 1u) && (d[q] > bv || (d[q] == bv && de[q] < be))) {
          bv = d[q];
          be = de[q];
          bq = q;
        }
      }
      int bl = bq >= 0 ? lane + 64 * bq : 0x7fffffff;   // candidate index of the best
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        const int ol = __shfl_xor(bl, off);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; bl = ol; }
      }
      if ((bl & 63) == lane) taken |= 1u << (bl >> 6);
      // fp32 logit of the chosen expert from the lane that loaded it
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
  constexpr int NT = 256 / (EP / 8 > 8 ? EP / 8 : 8);
  const unsigned grid = static_cast<unsigned>((a.T + NT - 1) / NT);
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

int route_ksplit(int64_t T, int H, int E, bool bf16) {
  if (!bf16) return 1;
  // about 256 workgroups: split H when tokens x expert blocks are fewer
  const int le = 32 * route_ne(E);
  const int64_t wg = ((T + LT - 1) / LT) * ((E + le - 1) / le);
  int64_t ks = wg > 0 ? 256 / wg : 1;
  const int nch = H / LBK;
  if (ks > nch) ks = nch;
  if (ks > 16) ks = 16;
  return ks < 1 ? 1 : static_cast<int>(ks);
}

size_t route_scratch_bytes(int64_t T, int H, int E, bool bf16) {
  const size_t ks = static_cast<size_t>(route_ksplit(T, H, E, bf16));
  return align_up(static_cast<size_t>(T) * 4, 256) + align_up(static_cast<size_t>(T) * 16, 256) +
         align_up(ks * static_cast<size_t>(T) * E * 4, 256) + align_up(ks * static_cast<size_t>(T) * 4, 256) +
         align_up(ks * static_cast<size_t>(E) * 4, 256);
}

hipError_t launch_route(const RouteArgs& a, bool bf16, hipStream_t s) {
  // every scratch region must have been carved before anything is launched
  if (!a.x || !a.w || !a.ids || !a.weights || !a.flag || !a.meta || !a.logits ||
      (bf16 && (!a.xnorm2 || !a.wnorm2)))
    return hipErrorInvalidValue;
  hipError_t err;
  if (bf16) {
    if (a.ksplit < 1 || a.ksplit > a.H / LBK) return hipErrorInvalidValue;
    const int le = 32 * route_ne(a.E);
    const dim3 grid(static_cast<unsigned>((a.T + LT - 1) / LT), static_cast<unsigned>((a.E + le - 1) / le),
                    static_cast<unsigned>(a.ksplit));
    if (route_ne(a.E) == 4) hipLaunchKernelGGL(route_logits_bf16_kernel<4>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(route_logits_bf16_kernel<2>, grid, dim3(256), 0, s, a);
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
