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
// summation structure of the kernel (an MFMA that starts from zero is
// counted as a chain of as many rounded additions as it has products, each
// rounding worth at most 2^-23 relative, so even a truncating adder is
// covered).  A token is flagged when its fp32 top-k is not provably the exact
// one: some expert outside the top-k is within 2*delta of the k-th logit, or
// two adjacent top-k logits are within 2*delta.  Flagged tokens are re-ranked
// with float64 dot products (exact products, float64 sums) over the
// candidate set {e : L_k - L_e <= 2*delta}, which provably contains the exact
// top-k, in the same workgroup that selected them.
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

// Top-k scan keys.  logit_key orders as the logits do (larger value,
// larger key; -0 and +0, which compare equal, share a key), so a lane's best
// element is one signed integer compare per element and the scan compiles
// to selects rather than branches; a NaN logit, which no comparison selects,
// gets kNoKey, the key of elements out of range or already taken.
constexpr int kNoKey = -2147483647 - 1;
__device__ __forceinline__ int logit_key(float v) {
  const int b = __float_as_int(v + 0.f);
  return v != v ? kNoKey : (b ^ ((b >> 31) & 0x7fffffff));
}
__device__ __forceinline__ float key_logit(int key) {   // inverse, for keys other than kNoKey
  return __int_as_float(key ^ ((key >> 31) & 0x7fffffff));
}

// One round of the per-lane scan: the lane's largest remaining logit and
// its expert (elements e = sub + LPT i, ties to the lowest e, i.e. the first
// in scan order); -inf and 0x7fffffff when none is left.
template <int PER, int LPT>
__device__ __forceinline__ void lane_best(const int (&key)[PER], int sub, float& bv, int& be) {
  int bk = kNoKey;
  be = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool better = key[i] > bk;
    bk = better ? key[i] : bk;
    be = better ? sub + LPT * i : be;
  }
  bv = bk == kNoKey ? -INFINITY : key_logit(bk);
}

// The round's winner (group-wide) leaves the scan: its owner lane drops it.
template <int PER, int LPT>
__device__ __forceinline__ void drop_taken(int (&key)[PER], int sub, int be) {
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = be == sub + LPT * i ? kNoKey : key[i];
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
__device__ __forceinline__ void route_select(const RouteArgs& a, int64_t t0, float (*lg)[EP + 1],
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
  int key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = sub + LPT * i < E ? logit_key(v[i]) : kNoKey;
  float sel_v[kMaxK];
  int sel_e[kMaxK];
  float vk = 0.f;        // the k-th largest logit (kept without a runtime index)
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      float bv;
      int be;
      lane_best<PER, LPT>(key, sub, bv, be);
#pragma unroll
      for (int off = 1; off < LPT; off <<= 1) {
        float ov = __shfl_xor(bv, off);
        int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      sel_v[j] = bv;
      sel_e[j] = be;
      if (j == k - 1) vk = bv;
      drop_taken<PER, LPT>(key, sub, be);
    }
  }

  const float mx = sel_v[0];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (sub + LPT * i < E) s += __expf(v[i] - mx);
  s = group_sum(s);

  const float band = 2.f * delta[tok] * kSafety;
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

template <typename ELEM>
__device__ __forceinline__ void rerank_token(const RouteArgs& a, int64_t t, const float* row,
                                             const float* meta, float* cv, int* ce, double* cd);

// ----------------------------------------------------------------- f32 path
// Plain fp32 FMA chains (no reduced-precision matrix path).  Thread = one
// token (tid % 32) x experts tid/32 + 8 i.  K is summed in chunks of 64 from
// zero and the chunk sums are added in order.  The workgroup then re-ranks
// its own flagged tokens (one wave per token) from the logits and softmax
// statistics the selection wrote for them.
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
  __syncthreads();                 // this workgroup's flags, logits and statistics are written

  __shared__ float cv[4][kMaxE];     // re-rank: candidate fp32 logits (per wave)
  __shared__ int ce[4][kMaxE];       //          candidate expert ids
  __shared__ double cd[4][kMaxE];    //          logits used for the final ranking
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int tok = wave; tok < RT; tok += 4) {
    const int64_t t = t0 + tok;
    if (t >= a.T) break;
    if (__builtin_amdgcn_readfirstlane(a.flag[t]) == 0) continue;
    rerank_token<float>(a, t, a.logits + t * a.E, a.meta + t * 4, cv[wave], ce[wave], cd[wave]);
  }
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
// The wave's token t: fp32 logits (bias included) at row[0..E), softmax max,
// sum, band and k-th logit at meta[0..3]; cv / ce / cd are the wave's own
// kMaxE-entry scratch arrays.  Writes the token's ids and weights.
template <typename ELEM>
__device__ __forceinline__ void rerank_token(const RouteArgs& a, int64_t t, const float* row, const float* meta,
                             float* cv, int* ce, double* cd) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k, H = a.H;
  constexpr int VEC = 16 / sizeof(ELEM);
  const float mx = meta[0], s = meta[1], band = meta[2];
  const float vk = meta[3];
  const unsigned long long below = (1ull << lane) - 1ull;

  // candidate list (expert order), fp32 logits
  float v[4];
  int nc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    v[q] = (e < E) ? row[e] : -INFINITY;
    const bool cand = e < E && (vk - v[q]) <= band;
    const unsigned long long m = __ballot(cand);
    if (cand) {
      const int i = nc + __popcll(m & below);
      cv[i] = v[q];
      ce[i] = e;
    }
    nc += __popcll(m);
  }
  __builtin_amdgcn_s_waitcnt(0);   // the wave's scratch writes (LDS or flat) are done
  __builtin_amdgcn_wave_barrier();

  // ambiguity and default (fp32) ranking logits; amb[q] of candidate lane + 64 q
  unsigned long long am[4];
  int na = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    bool amb = false;
    if (i < nc) {
      const float vi = cv[i];
      for (int j = 0; j < nc; ++j)
        if (j != i && fabsf(vi - cv[j]) <= band) amb = true;
      cd[i] = static_cast<double>(vi);
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
  // 64 / P lanes each; a lane sums chunks sub, sub + G, ...
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
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  for (int r0 = 0; r0 < na; r0 += P) {
    const int r = r0 + slot;
    const bool live = r < na;
    const int ci = live ? amb_index(r) : 0;
    const int ec = live ? ce[ci] : 0;
    const ELEM* wrow = static_cast<const ELEM*>(a.w) + static_cast<int64_t>(ec) * H;
    // batches of NB chunks per lane, all their loads issued before any is
    // used (one memory round trip per batch; H = 4096 with two candidates at
    // a time is one batch)
    constexpr int NB = 16;
    double accd = 0.0;
    for (int c0 = sub; c0 < nchunk; c0 += NB * G) {
      uint4 xv[NB], wv[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int c = c0 + u * G;
        const int cc = c < nchunk ? c : sub;          // in-range address; its data is not used
        xv[u] = *reinterpret_cast<const uint4*>(xrow + cc * VEC);
        wv[u] = *reinterpret_cast<const uint4*>(wrow + cc * VEC);
      }
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (c0 + u * G < nchunk) accd = dot_chunk(xv[u], wv[u], accd);
    }
    for (int off = 1; off < G; off <<= 1) accd += __shfl_xor(accd, off);
    if (a.bias) accd += static_cast<double>(a.bias[ec]);
    if (live && sub == 0) cd[ci] = accd;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();

  // exact top-k over the candidates by rank: candidate i (lane + 64 q) is
  // beaten by every candidate with a larger logit, or an equal logit and a
  // lower id; those of rank < k take slot rank (no cross-lane reductions)
  int rank[4], myid[4];
  float myp[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    rank[q] = kMaxE;
    myid[q] = 0;
    myp[q] = 0.f;
    if (i < nc) {
      const double di = cd[i];
      const int ei = ce[i];
      int r = 0;
      for (int j = 0; j < nc; ++j) {
        const double dj = cd[j];
        r += (dj > di || (dj == di && ce[j] < ei)) ? 1 : 0;
      }
      rank[q] = r;
      myid[q] = ei;
      myp[q] = __expf(cv[i] - mx) / s;   // weights from the stored fp32 softmax
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (rank[q] < k) { ce[rank[q]] = myid[q]; cv[rank[q]] = myp[q]; }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  if (lane < k) {
    float ps = 0.f;
    for (int j = 0; j < k; ++j) ps += cv[j];   // slot order, as the unflagged path sums
    const float pj = cv[lane];
    a.ids[t * k + lane] = ce[lane];
    a.weights[t * k + lane] = a.renorm ? pj / ps : pj;
  }
}


// ---------------------------------------------------------- fused bf16 path
// One workgroup owns BT tokens and every expert over the whole of H, and
// does the whole router for them in one pass: logits (MFMA 16x16x32, rows
// of x as A, router rows as B), bias, softmax, top-k, the exactness check,
// and the float64 re-rank of the few tokens that fail it.  Nothing but ids
// and weights leaves the workgroup (plus the logits and softmax statistics
// when the caller keeps them).
//
// Waves: WE expert groups x WK K ranges (WE * WK = 4, or WE = 8 with one K
// range when a workgroup streams a large router matrix).  Wave w owns experts
// [eg*EPW, (eg+1)*EPW), eg = w % WE, and the K32 steps
// [kq*S/WK, (kq+1)*S/WK), kq = w / WE, S = H / 32.  Router rows are loaded
// straight into registers, PF steps ahead, four lanes per 64-byte row
// segment, and moved into the MFMA operand layout (lane l: row l % 16, K
// values 8*(l/16) .. 8*(l/16)+7 of the step) by a lane permutation.  Rows
// of x take the same path when the waves split K; when they split only the
// experts, the waves share x through LDS, one barrier per PF steps.
//
// Summation (the structure the error bound counts): every MFMA starts from
// zero (a chain of at most 32 roundings), the results of PF consecutive steps
// form a group sum (the first assigned, the others added), group sums are
// added into the wave's sum, the WK wave sums in K order, then the bias:
//   D = 32 + PF + ceil(n / PF) + WK + 1,  n = K32 steps per wave.
// The squared norms of the router rows, which the bound needs, come from one
// more MFMA per step on the matrix cores (the row block times itself,
// accumulated over the steps; the diagonal holds them), so the vector ALU
// only adds the MFMA results.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// rounding depth D of a logit summed over n K32 steps per wave, groups of
// g steps, wk wave sums
__host__ __device__ constexpr int fused_depth(int n, int g, int wk) {
  return 32 + g + (n + g - 1) / g + wk + 1;
}

// sum of squares of 8 bf16 by packed dot products (v_dot2_f32_bf16); every
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

// v of the lane whose index differs from this one's in bit OFF (OFF < 32):
// quad permutes by DPP, wider distances by ds_swizzle (xor mode within 32
// lanes); neither needs an address register or LDS storage
template <int OFF>
__device__ __forceinline__ int xor_lane(int v) {
  if constexpr (OFF == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  else if constexpr (OFF == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  else return __builtin_amdgcn_ds_swizzle(v, (OFF << 10) | 0x1F);
}
template <int OFF>
__device__ __forceinline__ float xor_lane(float v) {
  return __int_as_float(xor_lane<OFF>(__float_as_int(v)));
}

// (value, id) maximum over the LPT-lane group, ties to the lower id
template <int LPT, int OFF = 1>
__device__ __forceinline__ void group_argmax(float& bv, int& be) {
  if constexpr (OFF < LPT) {
    const float ov = xor_lane<OFF>(bv);
    const int oe = xor_lane<OFF>(be);
    if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    group_argmax<LPT, OFF * 2>(bv, be);
  }
}
template <int LPT, int OFF = 1>
__device__ __forceinline__ float group_add(float v) {
  if constexpr (OFF < LPT) return group_add<LPT, OFF * 2>(v + xor_lane<OFF>(v));
  else return v;
}

// delta of the fused kernel.  The norms are fp32 sums of exact squares
// (token norms by v_dot2, router-row norms by MFMA accumulation), at most H
// non-negative terms added in some order, each addition within 2^-23 of its
// result even if the adder truncates: a computed norm is at least
// (1 - H * 2^-23) >= (1 - 2^-9) of the exact one (H <= 16384).  The product of
// the two square roots is then at least (1 - 2^-8 - 2^-20) of the exact
// product, which kNormSafety (with the roundings of the products) covers.
constexpr float kNormSafety = 1.0078125f;   // 1 + 2^-7
__device__ __forceinline__ float fused_delta(float xsq, float wsq_max, float bmax, int depth) {
  const float S = sqrtf(xsq) * sqrtf(wsq_max) * kNormSafety + bmax;
  const float d = static_cast<float>(depth) * kUlp2;
  return d * (1.f + d) * S * kSafety;
}

template <int BT, int EPW, int WE, int WK, int PF>
__global__ __launch_bounds__(64 * WE * WK) void route_fused_bf16_kernel(RouteArgs a) {
  // NW waves: 4, or 8 when they split the experts (more loads in flight per
  // CU for a workgroup that streams a large router matrix)
  constexpr int NW = WE * WK, NTH = 64 * NW;
  static_assert((NW == 4 || (NW == 8 && WK == 1)) && BT % 16 == 0 && EPW % 16 == 0 && 256 % BT == 0,
                "shape");
  constexpr int NT = BT / 16, NJ = EPW / 16, EP = EPW * WE;
  constexpr int LPT = 256 / BT;                 // select: lanes per token
  constexpr int PER = EP / LPT;                 // select: logits per lane
  static_assert(PER >= 1 && PER <= 32, "select layout");
  __shared__ float lg[WK][BT][EP + 1];          // wave sums; lg[0] then holds the totals
  __shared__ float xsq_s[WK][BT];
  __shared__ float wsq_s[WK][EP];
  __shared__ float fmeta[BT][4];                // flagged tokens: max, sum, band, k-th logit
  __shared__ int flagged[BT];
  __shared__ int nflag;
  __shared__ unsigned wmax_bits, bmax_bits;
  __shared__ float cv[NW][kMaxE];               // re-rank: candidate fp32 logits (per wave)
  __shared__ int ce[NW][kMaxE];                 //          candidate expert ids
  __shared__ double cd[NW][kMaxE];              //          logits used for the final ranking

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int eg = wave % WE, kq = wave / WE;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * BT;
  const int H = a.H, E = a.E, k = a.k;
  const int64_t T = a.T;
  const int S = H / 32;
  const int sb = kq * S / WK, n = (kq + 1) * S / WK - sb;
  const int r16 = lane & 15, g4 = lane >> 4;
  if (tid == 0) { nflag = 0; wmax_bits = 0u; bmax_bits = 0u; }

  // ---- logits
  // Loads are coalesced (four or sixteen lanes per row segment); the MFMA
  // wants row l % 16 and the 16-byte chunk l / 16 of the step in lane l.
  const int lrow = lane >> 2, lchk = lane & 3;
  const char* wp[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int e = eg * EPW + 16 * j + lrow;
    e = e < E ? e : E - 1;
    wp[j] = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.w) + static_cast<int64_t>(e) * H +
                                          sb * 32 + 8 * lchk);
  }
  // lane permutation into the MFMA layout: lane l takes the 16 bytes of the
  // lane that loaded (row l % 16, chunk l / 16)
  const int src_lane4 = 4 * (4 * r16 + g4);
  auto to_mfma = [&](const bf16x8_t& v) {
    const i32x4_t q = __builtin_bit_cast(i32x4_t, v);
    i32x4_t o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = __builtin_amdgcn_ds_bpermute(src_lane4, q[d]);
    return __builtin_bit_cast(bf16x8_t, o);
  };
  // every load is unconditional (steps past the wave's range reload its last
  // step, whose data is then not used), so that the loop body is straight-line
  // code and the compiler's waits count exactly the loads in flight
  const int slast = n > 0 ? n - 1 : 0;
  auto clamp_step = [&](int s) { return s < slast ? s : slast; };
  bf16x8_t wb[PF][NJ];
  auto wload = [&](int s, bf16x8_t* wr) {
    s = clamp_step(s);
#pragma unroll
    for (int j = 0; j < NJ; ++j) wr[j] = *reinterpret_cast<const bf16x8_t*>(wp[j] + s * 64);
  };

  f32x4_t acc[NT][NJ], grp[NT][NJ];
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) { acc[i][j] = zero4; grp[i][j] = zero4; }
  // router-row norms: W times itself on the matrix cores, accumulated over
  // all steps; the diagonal holds the squared norms
  f32x4_t wsqm[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) wsqm[j] = zero4;
  // a group's first step assigns its MFMA results, later steps add them
  auto close_group = [&]() {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] += grp[i][j];
  };
  auto mfmas = [&](const bf16x8_t* xf, const bf16x8_t* wr, bool first) {
    bf16x8_t wf[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) wf[j] = to_mfma(wr[j]);
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[i], wf[j], zero4, 0, 0, 0);
        grp[i][j] = first ? p : grp[i][j] + p;
      }
#pragma unroll
    for (int j = 0; j < NJ; ++j) wsqm[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], wf[j], wsqm[j], 0, 0, 0);
  };

  if constexpr (WK == 1) {
    // The waves share x through LDS.  An iteration covers PF steps (64·PF
    // bytes of each row): every wave loads BT / NW rows of the next iteration
    // (4·PF lanes per row), writes them to one of two LDS buffers (16-byte
    // chunk c of row r in slot c ^ (r % 16): conflict-free both for the
    // row-wise writes and for the MFMA reads of 16 rows at one chunk), and the
    // waves meet at one barrier per iteration.
    constexpr int CPR = 4 * PF;                   // 16-byte chunks of a row per iteration
    constexpr int RPI = 64 / CPR;                 // rows per 64-lane load
    static_assert((PF == 4 || PF == 8) && BT % (RPI * NW) == 0, "whole rows per wave");
    constexpr int XR = BT / (RPI * NW);           // 64-lane loads per wave per iteration
    __shared__ uint4 xs[2][BT * CPR];
    const int xchk = lane % CPR;
    const char* xq[XR];
    int xrow[XR];
    float xsq[XR];
#pragma unroll
    for (int q = 0; q < XR; ++q) {
      xrow[q] = RPI * (wave * XR + q) + lane / CPR;
      int64_t t = t0 + xrow[q];
      t = t < T ? t : T - 1;
      xq[q] = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.x) + t * H) + (xchk & 3) * 16;
      xsq[q] = 0.f;
    }
    uint4 xr[XR];
    auto xload = [&](int it) {
      const int s = clamp_step(PF * it + (xchk >> 2));
#pragma unroll
      for (int q = 0; q < XR; ++q) xr[q] = *reinterpret_cast<const uint4*>(xq[q] + s * 64);
    };
    auto xstore = [&](int buf) {
#pragma unroll
      for (int q = 0; q < XR; ++q) {
        xs[buf][xrow[q] * CPR + (xchk ^ (xrow[q] & 15))] = xr[q];
        // token norms, one wave per row; a last partial iteration re-reads
        // its last step, which only enlarges the norm (the bound stays valid)
        xsq[q] = sumsq8_dot(__builtin_bit_cast(bf16x8_t, xr[q]), xsq[q]);
      }
    };
    auto xfrags = [&](int buf, int u, bf16x8_t* xf) {
#pragma unroll
      for (int i = 0; i < NT; ++i)
        xf[i] = __builtin_bit_cast(bf16x8_t, xs[buf][(16 * i + r16) * CPR + ((4 * u + g4) ^ r16)]);
    };
    // prologue: x of iteration 0 in LDS, x of iteration 1 and W of iteration 0 in flight
    xload(0);
    xstore(0);
    __builtin_amdgcn_sched_barrier(0);
    xload(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      wload(u, wb[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
    const int nfull = n / PF;
    for (int it = 0; it < nfull; ++it) {
      const int buf = it & 1;
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        bf16x8_t xf[NT];
        xfrags(buf, u, xf);
        mfmas(xf, wb[u], u == 0);
        wload((it + 1) * PF + u, wb[u]);
        if (u == 0) {
          xstore(buf ^ 1);                        // x of iteration it + 1
          xload(it + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      close_group();
      lds_barrier();
    }
    const int rem = n - nfull * PF;
    if (rem > 0) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        if (u < rem) {
          bf16x8_t xf[NT];
          xfrags(nfull & 1, u, xf);
          mfmas(xf, wb[u], u == 0);
        }
      }
      close_group();
    }
    // norms of the rows this wave loaded: the 16 lanes of a row hold its chunks
#pragma unroll
    for (int q = 0; q < XR; ++q) {
      float v = xsq[q] + xor_lane<1>(xsq[q]);
      v += xor_lane<2>(v);
      v += xor_lane<4>(v);
      v += xor_lane<8>(v);
      if (xchk == 0) xsq_s[0][xrow[q]] = v;
    }
  } else {
    // WK K ranges: every wave has its own x columns, loaded to registers
    const char* xp[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      int64_t t = t0 + 16 * i + lrow;
      t = t < T ? t : T - 1;          // clamped rows are computed, never stored
      xp[i] = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.x) + t * H + sb * 32 + 8 * lchk);
    }
    bf16x8_t xb[PF][NT];
    float xsq[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) xsq[i] = 0.f;
    auto load = [&](int s, int u) {
      const int sc = clamp_step(s);
#pragma unroll
      for (int i = 0; i < NT; ++i) xb[u][i] = *reinterpret_cast<const bf16x8_t*>(xp[i] + sc * 64);
      wload(s, wb[u]);
    };
    auto step = [&](int u) {
      bf16x8_t xf[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) xf[i] = to_mfma(xb[u][i]);
      mfmas(xf, wb[u], u == 0);
#pragma unroll
      for (int i = 0; i < NT; ++i) xsq[i] = sumsq8_dot(xb[u][i], xsq[i]);
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      load(u, u);
      // issue order = step order here as in the loop, so that the count of
      // newer loads is the same at every use (entry and back edge alike)
      __builtin_amdgcn_sched_barrier(0);
    }
    // PF steps per iteration, each iteration's sum closed into the wave's
    // sum; the loop body is branch-free, the last n % PF steps run after it
    const int nfull = n / PF;
    for (int it = 0; it < nfull; ++it) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        step(u);
        load((it + 1) * PF + u, u);
        // keep this order: the loads of step s + PF go out right after step
        // s, so each step's data has PF - 1 steps of work to arrive in
        __builtin_amdgcn_sched_barrier(0);
      }
      close_group();
    }
    const int rem = n - nfull * PF;
    if (rem > 0) {
#pragma unroll
      for (int u = 0; u < PF; ++u)
        if (u < rem) step(u);
      close_group();
    }
    // norms: the four lanes 4r .. 4r+3 of a quad hold the four chunks of row r
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      float v = xsq[i] + xor_lane<1>(xsq[i]);
      v += xor_lane<2>(v);
      if (lchk == 0) xsq_s[kq][16 * i + lrow] = v;
    }
  }

  // wave sums to LDS: lane holds tokens 16 i + 4 g4 + v of expert column 16 j + r16
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) lg[kq][16 * i + 4 * g4 + v][eg * EPW + 16 * j + r16] = acc[i][j][v];
  if ((r16 >> 2) == g4) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) wsq_s[kq][eg * EPW + 16 * j + r16] = wsqm[j][r16 & 3];
  }
  __syncthreads();

  // ---- totals (wave sums in K order), norm maxima
  if constexpr (WK > 1) {
    for (int c = tid; c < BT * EP; c += NTH) {
      const int tk = c / EP, e = c - tk * EP;
      float v = lg[0][tk][e];
#pragma unroll
      for (int q = 1; q < WK; ++q) v += lg[q][tk][e];
      lg[0][tk][e] = v;
    }
  }
  {
    // largest squared router-row norm and |bias|: the values are
    // non-negative, so their bit patterns order as they do; a maximum over
    // the wave first, then one LDS atomic per wave (one per expert cost
    // 3-5 us per call with 64-256 experts)
    float w2 = 0.f, bm = 0.f;
    if (tid < E) {
#pragma unroll
      for (int q = 0; q < WK; ++q) w2 += wsq_s[q][tid];
      if (a.bias) bm = fabsf(a.bias[tid]);
    }
    unsigned wb = __float_as_uint(w2), bb = __float_as_uint(bm);
    wb = max(wb, static_cast<unsigned>(xor_lane<1>(static_cast<int>(wb))));
    bb = max(bb, static_cast<unsigned>(xor_lane<1>(static_cast<int>(bb))));
    wb = max(wb, static_cast<unsigned>(xor_lane<2>(static_cast<int>(wb))));
    bb = max(bb, static_cast<unsigned>(xor_lane<2>(static_cast<int>(bb))));
    wb = max(wb, static_cast<unsigned>(xor_lane<4>(static_cast<int>(wb))));
    bb = max(bb, static_cast<unsigned>(xor_lane<4>(static_cast<int>(bb))));
    wb = max(wb, static_cast<unsigned>(xor_lane<8>(static_cast<int>(wb))));
    bb = max(bb, static_cast<unsigned>(xor_lane<8>(static_cast<int>(bb))));
    wb = max(wb, static_cast<unsigned>(xor_lane<16>(static_cast<int>(wb))));
    bb = max(bb, static_cast<unsigned>(xor_lane<16>(static_cast<int>(bb))));
    wb = max(wb, static_cast<unsigned>(__shfl_xor(static_cast<int>(wb), 32)));
    bb = max(bb, static_cast<unsigned>(__shfl_xor(static_cast<int>(bb), 32)));
    if (lane == 0 && wave * 64 < E) {
      atomicMax(&wmax_bits, wb);
      if (a.bias) atomicMax(&bmax_bits, bb);
    }
  }
  __syncthreads();

  // ---- softmax, top-k, exactness check: LPT lanes per token (the first
  // 256 threads; whole waves)
  if (tid < 256) {
    const int tok = tid / LPT, sub = tid % LPT;
    const int64_t t = t0 + tok;
    float x2 = 0.f;
#pragma unroll
    for (int q = 0; q < WK; ++q) x2 += xsq_s[q][tok];
    x2 += static_cast<float>(H) * 1.1754943508222875e-38f;   // H * 2^-126: flushed squares
    const int nmax = (S + WK - 1) / WK;
    const float delta = fused_delta(x2, __uint_as_float(wmax_bits), __uint_as_float(bmax_bits),
                                    fused_depth(nmax, PF, WK));
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = sub + LPT * i;
      v[i] = (e < E) ? lg[0][tok][e] + (a.bias ? a.bias[e] : 0.f) : -INFINITY;
    }
    int key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = sub + LPT * i < E ? logit_key(v[i]) : kNoKey;
    float sel_v[kMaxK];
    int sel_e[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        float bv;
        int be;
        lane_best<PER, LPT>(key, sub, bv, be);
        group_argmax<LPT>(bv, be);
        sel_v[j] = bv;
        sel_e[j] = be;
        drop_taken<PER, LPT>(key, sub, be);
      }
    }
    const float mx = sel_v[0];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (sub + LPT * i < E) sum += __expf(v[i] - mx);
    sum = group_add<LPT>(sum);
    const float band = 2.f * delta * kSafety;
    const float vk = sel_v[k - 1];
    float cnt = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (sub + LPT * i < E && (vk - v[i]) <= band) cnt += 1.f;
    cnt = group_add<LPT>(cnt);
    bool flag = cnt > static_cast<float>(k);
#pragma unroll
    for (int j = 0; j + 1 < kMaxK; ++j)
      if (j + 1 < k && (sel_v[j] - sel_v[j + 1]) <= band) flag = true;

    if (t < T) {
      if (flag) {
        if (sub == 0) {
          const int slot = atomicAdd(&nflag, 1);
          flagged[slot] = tok;
          fmeta[tok][0] = mx; fmeta[tok][1] = sum; fmeta[tok][2] = band; fmeta[tok][3] = vk;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int e = sub + LPT * i;
          if (e < E) lg[0][tok][e] = v[i];          // the re-rank reads logits with bias
        }
      } else {
        float p[kMaxK];
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
          if (j < k) { p[j] = __expf(sel_v[j] - mx) / sum; ps += p[j]; }
        // slot j is written by lane j % LPT of the token's group (LPT may be < k)
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
          if (j < k && j % LPT == sub) {
            a.ids[t * k + j] = sel_e[j];
            a.weights[t * k + j] = a.renorm ? p[j] / ps : p[j];
          }
        }
      }
      if (a.keep_all) {
        if (sub == 0) {
          a.meta[t * 4 + 0] = mx;
          a.meta[t * 4 + 1] = sum;
          a.meta[t * 4 + 2] = band;
          a.meta[t * 4 + 3] = vk;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int e = sub + LPT * i;
          if (e < E) a.logits[t * E + e] = v[i];
        }
      }
    }
  }
  __syncthreads();

  // ---- float64 re-rank of the flagged tokens, one wave per token
  const int nf = nflag;
  for (int f = wave; f < nf; f += NW) {
    const int tok = flagged[f];
    rerank_token<uint16_t>(a, t0 + tok, &lg[0][tok][0], fmeta[tok], cv[wave], ce[wave], cd[wave]);
  }
}

template <int BT, int EPW, int WE, int WK>
hipError_t launch_fused(const RouteArgs& a, hipStream_t s) {
  // shared x: iterations of 8 steps where the x buffers leave room (half the
  // barriers of 4-step iterations: fine 62 -> 57.5 us, very fine 95 -> 86 us;
  // with 16 experts per wave the larger x buffers halve the workgroups per CU
  // and 8 steps were slower, 52 -> 80 us on the skewed workload, and 128
  // tokens do not fit); K ranges: about 24 16-byte loads per lane in flight
  // (96 registers)
  constexpr int L = BT / 16 + EPW / 16;
  constexpr int PF = WK == 1 ? (EPW >= 32 && BT <= 64 ? 8 : 4) : (24 / L > 8 ? 8 : (24 / L < 3 ? 3 : 24 / L));
  const unsigned grid = static_cast<unsigned>((a.T + BT - 1) / BT);
  hipLaunchKernelGGL((route_fused_bf16_kernel<BT, EPW, WE, WK, PF>), dim3(grid), dim3(64 * WE * WK), 0, s, a);
  return hipGetLastError();
}

template <int EP>
hipError_t launch_f32(const RouteArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.T + RT - 1) / RT);
  hipLaunchKernelGGL((route_f32_kernel<EP>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t route_scratch_bytes(int64_t T, int H, int E, bool bf16) {
  (void)H;
  (void)bf16;
  return align_up(static_cast<size_t>(T) * 4, 256) + align_up(static_cast<size_t>(T) * 16, 256) +
         align_up(static_cast<size_t>(T) * E * 4, 256);
}

hipError_t launch_route(const RouteArgs& a, bool bf16, hipStream_t s) {
  // every scratch region must have been carved before anything is launched
  if (!a.x || !a.w || !a.ids || !a.weights || !a.flag || !a.meta || !a.logits)
    return hipErrorInvalidValue;
  if (a.H % 64 || a.E < 1 || a.E > kMaxE || a.k < 1 || a.k > kMaxK || a.k > a.E) return hipErrorInvalidValue;
  if (bf16) {
    const int64_t T = a.T;
    // token blocks: about 512 workgroups (two per CU) up to 128 experts,
    // 256 beyond (every workgroup reads all of W_r; measured on the
    // fine, very fine and skewed workloads)
    if (a.E <= 16) return launch_fused<16, 16, 1, 4>(a, s);
    if (a.E <= 64) {
      if (T >= 512 * 128) return launch_fused<128, 16, 4, 1>(a, s);
      if (T >= 512 * 64) return launch_fused<64, 16, 4, 1>(a, s);
      return launch_fused<32, 16, 4, 1>(a, s);
    }
    if (a.E <= 128) {
      if (T >= 512 * 64) return launch_fused<64, 32, 4, 1>(a, s);
      return launch_fused<32, 32, 4, 1>(a, s);
    }
    // beyond 128 experts the workgroup streams 2 MB of router rows per 32
    // tokens: eight waves (32 experts each) keep twice the loads in flight
    // (measured on the very fine workload: 0.134 -> 0.118-0.121 ms; with 128
    // experts the eight-wave form was slower, 0.071 -> 0.094 ms)
    if (T >= 256 * 32) return launch_fused<32, 32, 8, 1>(a, s);
    return launch_fused<16, 64, 4, 1>(a, s);
  }
  hipError_t err;
  if (a.E <= 32) err = launch_f32<32>(a, s);
  else if (a.E <= 64) err = launch_f32<64>(a, s);
  else if (a.E <= 128) err = launch_f32<128>(a, s);
  else err = launch_f32<256>(a, s);
  return err;
}

}  // namespace moe
