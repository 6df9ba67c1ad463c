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

#include <math.h>

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int RT = kRouteTok;   // tokens per workgroup
constexpr int KC = 64;          // K elements per LDS stage (bf16 path)
constexpr float kUlp2 = 1.1920928955078125e-07f;   // 2^-23
constexpr float kSafety = 1.0009765625f;            // 1 + 2^-10

// 16-byte chunk c (0..7) of row r in an LDS tile of 8-chunk rows, XOR-swizzled
// so that 8 consecutive rows reading the same chunk hit distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ (r & 7)); }

__device__ __forceinline__ float sumsq8_bf16(const uint4& v) {
  const uint16_t* p = reinterpret_cast<const uint16_t*>(&v);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float f = bf16_to_f32(p[i]);
    s = fmaf(f, f, s);
  }
  return s;
}

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
// Workgroup: RT tokens x all experts.  MFMA 32x32x16 bf16 with the router
// weight rows as the A operand (32 experts) and the tokens as B (32 tokens).
// Waves split experts (WE groups of NTW 32-expert tiles) and the 4 K16 steps
// of each 64-wide K stage (WK groups).
template <int NTW, int WK>
__global__ __launch_bounds__(256) void route_bf16_kernel(RouteArgs a) {
  constexpr int WE = 4 / WK;
  constexpr int EP = 32 * NTW * WE;
  constexpr int WR = EP / 32;          // W rows loaded per thread per stage
  constexpr int SPW = 4 / WK;          // K16 steps per wave per stage
  __shared__ uint4 xs[2][RT * 8];
  __shared__ uint4 ws[2][EP * 8];
  __shared__ float lg[RT][EP + 1];
  __shared__ float xsq_s[RT];
  __shared__ float delta_s[RT];
  __shared__ unsigned wmax_bits, bmax_bits;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int we = wave % WE, wk = wave / WE;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;
  const int H = a.H, E = a.E;
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);

  if (tid == 0) { wmax_bits = 0u; bmax_bits = 0u; }

  const int lrow = tid >> 3, lc = tid & 7;
  const int64_t tl = t0 + lrow;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  uint4 xr, wr[WR];
  float xsq = 0.f, wsq[WR];
#pragma unroll
  for (int i = 0; i < WR; ++i) wsq[i] = 0.f;

  auto gload = [&](int ch) {
    const int64_t ko = static_cast<int64_t>(ch) * KC + lc * 8;
    xr = (tl < a.T) ? *reinterpret_cast<const uint4*>(X + tl * H + ko) : zero;
#pragma unroll
    for (int i = 0; i < WR; ++i) {
      int er = lrow + 32 * i;
      wr[i] = (er < E) ? *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(er) * H + ko) : zero;
    }
  };
  auto stash = [&](int buf) {
    xsq += sumsq8_bf16(xr);
    xs[buf][swz(lrow, lc)] = xr;
#pragma unroll
    for (int i = 0; i < WR; ++i) {
      wsq[i] += sumsq8_bf16(wr[i]);
      ws[buf][swz(lrow + 32 * i, lc)] = wr[i];
    }
  };

  const int nch = H / KC;
  gload(0);
  stash(0);
  __syncthreads();

  f32x16_t acc[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;

  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nch) gload(ch + 1);
    f32x16_t part[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[n][r] = 0.f;
#pragma unroll
    for (int ss = 0; ss < SPW; ++ss) {
      const int s = wk * SPW + ss;
      const int c = 2 * s + (lane >> 5);
      const bf16x8_t bx = *reinterpret_cast<const bf16x8_t*>(&xs[buf][swz(lane & 31, c)]);
#pragma unroll
      for (int n = 0; n < NTW; ++n) {
        const int er = (we * NTW + n) * 32 + (lane & 31);
        const bf16x8_t aw = *reinterpret_cast<const bf16x8_t*>(&ws[buf][swz(er, c)]);
        part[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, bx, part[n], 0, 0, 0);
      }
    }
#pragma unroll
    for (int n = 0; n < NTW; ++n) acc[n] += part[n];
    if (ch + 1 < nch) stash(buf ^ 1);
    __syncthreads();
  }

  // norms
  xsq = xor_sum8(xsq);
  if (lc == 0) xsq_s[lrow] = xsq;
#pragma unroll
  for (int i = 0; i < WR; ++i) {
    float w2 = xor_sum8(wsq[i]);
    if (lc == 0 && lrow + 32 * i < E) atomicMax(&wmax_bits, __float_as_uint(w2));
  }
  if (a.bias && tid < E) atomicMax(&bmax_bits, __float_as_uint(fabsf(a.bias[tid])));

  // partial logits -> LDS, K-split waves added in a fixed order
#pragma unroll
  for (int p = 0; p < WK; ++p) {
    if (wk == p) {
#pragma unroll
      for (int n = 0; n < NTW; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = (we * NTW + n) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int tk = lane & 31;
          if (p == 0) lg[tk][e] = acc[n][r];
          else lg[tk][e] += acc[n][r];
        }
    }
    __syncthreads();
  }

  if (tid < RT) {
    const int depth = 16 * SPW + nch + WK + 1;
    delta_s[tid] = route_delta(xsq_s[tid], __uint_as_float(wmax_bits), __uint_as_float(bmax_bits), depth);
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

template <int NTW, int WK>
hipError_t launch_bf16(const RouteArgs& a, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((a.T + RT - 1) / RT);
  hipLaunchKernelGGL((route_bf16_kernel<NTW, WK>), dim3(grid), dim3(256), 0, s, a);
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
         align_up(static_cast<size_t>(T) * E * 4, 256);
}

hipError_t launch_route(const RouteArgs& a, bool bf16, hipStream_t s) {
  hipError_t err;
  if (bf16) {
    if (a.E <= 32) err = launch_bf16<1, 4>(a, s);
    else if (a.E <= 64) err = launch_bf16<1, 2>(a, s);
    else if (a.E <= 128) err = launch_bf16<1, 1>(a, s);
    else err = launch_bf16<2, 1>(a, s);
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
