// Ragged grouped GEMMs of the expert SwiGLU MLPs on bf16 MFMA (gfx950).
//
// Page legend:
//   [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
//   [SonicMoE page]  "SonicMoE与传统MoE架构对比：Token舍入技术如何实现训练效率跃升"
//
// [Qwen3-MoE page] §2.1 computes all experts in one batched launch over the
// stacked expert weights, scheduled over the compute units; the rows of each
// expert are the contiguous block offsets[e]..offsets[e+1]-1 of the
// permutation (§2.2).  Two kernels:
//   swiglu: h[r, n]  = silu(sum_k A[r,k] Wg[e,n,k]) * (sum_k A[r,k] Wu[e,n,k])
//   down:   y[r, n]  = sum_k h[r,k] W2[e,n,k]
// Row r of A is either row r of a grouped buffer or, for the fused forward,
// row gather[r] / k of x (the permutation is applied while loading).
//
// Design (CDNA4): one persistent workgroup per CU walks a list of 256x256
// output tiles.  Tiles are numbered expert by expert; inside an expert, up to
// 8 m-tiles form a group that is walked n-tile-major, so the ~32 tiles an
// XCD runs at once share their weight panels and their rows.  The tile list is
// cut into 8 contiguous ranges, one per XCD (workgroup b runs on XCD b % 8),
// so each range is served by one L2.  Tail m-tiles are masked: no padded rows
// exist in memory ([SonicMoE page] §核心差异 3 counts the padding such tails
// cost; it is reported, never materialised).  Empty experts own no tiles and
// their weights are never read.
//
// Per tile: 4 waves in 2x2, each 128x128 outputs = 4x4 MFMA 32x32x16 tiles
// with fp32 accumulators.  K advances in 64-wide stages through two LDS
// stage buffers; stage k+1 is fetched straight from L2/HBM into LDS
// (global_load_lds_dwordx4, no staging registers, whole 128-byte lines per
// row) while stage k is multiplied, each DMA issued between two MFMAs; the
// first stage of a workgroup's next tile is issued before the current tile's
// epilogue, so loads overlap the stores.  Operand fragments are
// double-buffered across the four K16 steps of a stage.  LDS rows are 128
// bytes whose 16-byte chunks are XOR-swizzled by row pairs, which keeps the
// MFMA operand reads free of bank conflicts.  The MFMA
// takes the weight rows as its A operand and the token rows as B, so each
// lane ends with 4 consecutive output columns of one row: the epilogue
// applies silu(g)*u in registers and stores 8-byte bf16 quads.
#include "moe_internal.h"
#include "cdna4.h"

namespace moe {
namespace {

constexpr int BM = kGemmBM;   // 256 rows
constexpr int BN = kGemmBN;   // 256 weight rows (swiglu: 128 gate + 128 up)
constexpr int BK = kGemmBK;   // 64
constexpr int kGroupM = 8;    // m-tiles walked together inside an expert

__device__ __forceinline__ int swz(int r, int c) { return swz128(r, c); }

__device__ __forceinline__ float silu_f(float g) { return g / (1.f + __expf(-g)); }

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  uint2 o;
  o.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
  o.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
  return o;
}

struct Tile {
  int e, r0, rows, n0;
};

template <bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs a) {
  // two stage buffers as distinct arrays (each holds the A rows then the B
  // rows of one 64-wide K stage)
  __shared__ uint4 S0[(BM + BN) * 8];
  __shared__ uint4 S1[(BM + BN) * 8];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_pre[kMaxE + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int E = a.E;
  for (int i = tid; i <= E; i += 256) { s_off[i] = a.offsets[i]; s_pre[i] = a.prefix[i]; }
  __syncthreads();

  constexpr int NOUT = SWIGLU ? BN / 2 : BN;   // output columns per tile
  const int N = a.N, K = a.K;
  const int NT = (N + NOUT - 1) / NOUT;
  const int total = s_pre[E] * NT;
  const int nk = K / BK;

  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int begin = xcd * chunk;
  const int end = (begin + chunk < total) ? begin + chunk : total;

  const uint16_t* Ab = static_cast<const uint16_t*>(a.A);
  const uint16_t* Bb = static_cast<const uint16_t*>(a.B);
  uint16_t* Cb = static_cast<uint16_t*>(a.C);

  // tile L -> (expert, first row, rows, first output column); false for
  // tiles that malformed offsets would place outside [0, M)
  auto decode = [&](int L, Tile& t) -> bool {
    const int q = L / NT;
    int lo = 0, hi = E;            // largest e with s_pre[e] <= q
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] <= q) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int local = L - s_pre[e] * NT;
    const int mte = s_pre[e + 1] - s_pre[e];
    // up to kGroupM m-tiles of the expert walked n-tile-major: the ~32 tiles
    // an XCD runs at once cover every m-tile of a weight panel, so a panel
    // streams from HBM once per group instead of once per m-tile
    const int G = mte < kGroupM ? mte : kGroupM;
    const int g = local / (G * NT);
    const int rem = local - g * G * NT;
    const int gsz = (mte - g * G < G) ? mte - g * G : G;
    const int nt = rem / gsz;
    const int mt = g * G + rem % gsz;
    t.e = e;
    t.r0 = s_off[e] + mt * BM;
    t.rows = (s_off[e + 1] - t.r0 < BM) ? s_off[e + 1] - t.r0 : BM;
    t.n0 = nt * NOUT;
    if (t.r0 < 0 || t.r0 >= a.M) return false;
    if (t.rows > a.M - t.r0) t.rows = static_cast<int>(a.M - t.r0);
    return t.rows > 0;
  };

  // Per-lane source rows.  Wave w's j-th DMA of a stage fills LDS rows
  // 32 j + 8 w .. +7 (8 rows x 8 slots = 64 lanes x 16 bytes); the lane
  // writes slot lane & 7 of row 32 j + 8 w + lane / 8 and so fetches chunk
  // (lane & 7) ^ ((row >> 1) & 7) == (lane & 7) ^ ((4 w + lane / 16) & 7).
  const int lchunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow = 8 * wave + (lane >> 3);
  const uint16_t* ap[8];
  const uint16_t* bp[8];
  auto set_rows = [&](const Tile& t) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ri = lrow + 32 * j;
      const int rr = t.r0 + (ri < t.rows ? ri : t.rows - 1);
      int64_t src = rr;
      if constexpr (GATHER) {
        src = a.gather[rr] / a.gather_div;
        src = src < 0 ? 0 : (src >= a.a_rows ? a.a_rows - 1 : src);
      }
      ap[j] = Ab + src * K + lchunk * 8;
      int64_t wr;
      if constexpr (SWIGLU) {
        const int n = t.n0 + (ri & 127);
        wr = (n < a.I ? n : a.I - 1) + (j >= 4 ? a.I : 0);
      } else {
        const int n = t.n0 + ri;
        wr = n < N ? n : N - 1;
      }
      bp[j] = Bb + static_cast<int64_t>(t.e) * a.b_stride + wr * K + lchunk * 8;
    }
  };

  // LDS byte address of stage buffer b for this wave's first DMA
  const uint32_t wofs = static_cast<uint32_t>(wave) * 64 * 16;
  const uint32_t sb0 = __builtin_amdgcn_readfirstlane(lds_addr(S0) + wofs);
  const uint32_t sb1 = __builtin_amdgcn_readfirstlane(lds_addr(S1) + wofs);
  auto dma1 = [&](int kc, uint32_t sb, int t) {   // t < 8: A rows 32t.., else B rows 32(t-8)..
    const int ko = kc * BK;
    if (t < 8) dma16(ap[t] + ko, sb + t * 4 * 64 * 16);
    else dma16(bp[t - 8] + ko, sb + BM * 8 * 16 + (t - 8) * 4 * 64 * 16);
  };

  f32x16_t acc[4][4];
  struct Frag {
    bf16x8_t x[4], w[4];
  };
  auto mfma1 = [&](const Frag& F, int t) {
    const int i = t >> 2, j = t & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.w[j], F.x[i], acc[i][j], 0, 0, 0);
  };
  // fragment t (< 4: x[t], else w[t-4]) of K16 step s (0..3) of the stage in Ss
  auto frag1 = [&](const uint4* Ss, int s, Frag& F, int t) {
    const int c = 2 * s + (lane >> 5);
    if (t < 4) {
      F.x[t] = *reinterpret_cast<const bf16x8_t*>(&Ss[swz(wm * 128 + t * 32 + (lane & 31), c)]);
    } else {
      const int j = t - 4;
      int wrow;
      if constexpr (SWIGLU) wrow = (j < 2) ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32;
      else wrow = wn * 128 + j * 32;
      F.w[j] = *reinterpret_cast<const bf16x8_t*>(&Ss[BM * 8 + swz(wrow + (lane & 31), c)]);
    }
  };

  // Stage kc sits in buffer kc & 1.  Iteration kc: this lane's DMA of stage
  // kc has landed, the barrier makes it visible everywhere and retires every
  // read of stage kc-1, whose buffer then receives stage kc+1.  The fragments
  // of K16 step s+1 are read while step s is multiplied, and every LDS read
  // and DMA is issued between two MFMAs, so with one wave per SIMD the matrix
  // pipe idles only at the barrier and the first fragment read of a stage.
  Frag Fa, Fb;
  auto stage = [&](int kc, const uint4* Ss, uint32_t sbn) {
    wait_vmcnt0();
    lds_barrier();
    const bool dma = kc + 1 < nk;
#pragma unroll
    for (int t = 0; t < 8; ++t) frag1(Ss, 0, Fa, t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 16; ++t) {     // step 0; read step 1, DMA half of stage kc+1
      mfma1(Fa, t);
      if (t < 8) frag1(Ss, 1, Fb, t);
      else if (dma) dma1(kc + 1, sbn, t - 8);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {     // step 1; read step 2, DMA the other half
      mfma1(Fb, t);
      if (t < 8) frag1(Ss, 2, Fa, t);
      else if (dma) dma1(kc + 1, sbn, t);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {     // step 2; read step 3
      mfma1(Fa, t);
      if (t < 8) frag1(Ss, 3, Fb, t);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {     // step 3
      mfma1(Fb, t);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  Tile cur;
  int L = begin + slot;
  bool have = false;
  for (; L < end; L += nslot)
    if (decode(L, cur)) { have = true; break; }
  if (!have) return;
  set_rows(cur);
#pragma unroll
  for (int t = 0; t < 16; ++t) dma1(0, sb0, t);

  while (true) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    int kc = 0;
    for (; kc + 2 <= nk; kc += 2) {
      stage(kc, S0, sb1);
      stage(kc + 1, S1, sb0);
    }
    if (kc < nk) stage(kc, S0, sb1);   // odd number of stages: the last one is in S0

    // next tile of this workgroup; its first stages load during the epilogue
    Tile nxt;
    bool more = false;
    for (L += nslot; L < end; L += nslot)
      if (decode(L, nxt)) { more = true; break; }
    lds_barrier();          // every wave is done reading this tile's stage buffers
    if (more) {
      set_rows(nxt);
#pragma unroll
      for (int t = 0; t < 16; ++t) dma1(0, sb0, t);
    }

    // ---- epilogue: lane holds row m, columns 8*grp + 4*(lane>>5) + 0..3 of each 32x32 tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 128 + i * 32 + (lane & 31);
      if (m >= cur.rows) continue;
      uint16_t* crow = Cb + static_cast<int64_t>(cur.r0 + m) * N;
      if constexpr (SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int n = cur.n0 + wn * 64 + j * 32 + 8 * grp + 4 * (lane >> 5);
            if (n >= N) continue;
            const f32x16_t& gg = acc[i][j];
            const f32x16_t& uu = acc[i][j + 2];
            const int b = grp * 4;
            *reinterpret_cast<uint2*>(crow + n) =
                pack4_bf16(silu_f(gg[b]) * uu[b], silu_f(gg[b + 1]) * uu[b + 1],
                           silu_f(gg[b + 2]) * uu[b + 2], silu_f(gg[b + 3]) * uu[b + 3]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int n = cur.n0 + wn * 128 + j * 32 + 8 * grp + 4 * (lane >> 5);
            if (n >= N) continue;
            const f32x16_t& cc = acc[i][j];
            const int b = grp * 4;
            *reinterpret_cast<uint2*>(crow + n) = pack4_bf16(cc[b], cc[b + 1], cc[b + 2], cc[b + 3]);
          }
      }
    }
    if (!more) break;
    cur = nxt;
  }
}

template <bool SWIGLU, bool GATHER>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_bf16_kernel<SWIGLU, GATHER>), dim3(a.grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_swiglu(const GemmArgs& a, hipStream_t s) {
  return a.gather ? launch<true, true>(a, s) : launch<true, false>(a, s);
}

hipError_t launch_gemm_bf16_down(const GemmArgs& a, hipStream_t s) {
  return launch<false, false>(a, s);
}

}  // namespace moe
