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
// with fp32 accumulators; K advances in 64-wide stages through two LDS
// buffers.  Stage s+1 is fetched straight from HBM into LDS
// (global_load_lds_dwordx4, no staging registers) while stage s is
// multiplied.  LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by
// row pairs so that MFMA operand reads are free of bank conflicts.  The MFMA
// takes the weight rows as its A operand and the token rows as B, so each
// lane ends with 4 consecutive output columns of one row: the epilogue
// applies silu(g)*u in registers and stores 8-byte bf16 quads.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = kGemmBM;   // 256 rows
constexpr int BN = kGemmBN;   // 256 weight rows (swiglu: 128 gate + 128 up)
constexpr int BK = kGemmBK;   // 64
constexpr int kGroupM = 8;    // m-tiles walked together inside an expert

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// 16-byte chunk c (0..7) of row r of a 128-byte-row LDS tile sits in slot
// c ^ ((r >> 1) & 7): the 16 lanes an LDS cycle serves (16 consecutive rows,
// same chunk) then cover all 64 banks exactly once.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// s_waitcnt vmcnt(0): wait for this lane's outstanding vector-memory loads,
// including the direct-to-LDS ones (expcnt / lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float silu_f(float g) { return g / (1.f + __expf(-g)); }

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  uint2 o;
  o.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
  o.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
  return o;
}

template <bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs a) {
  // two LDS stages per operand as four distinct arrays: the compiler's
  // memory-model tracking can then see that a DMA into one stage never
  // aliases reads of the other and adds no wait of its own
  __shared__ uint4 As0[BM * 8];
  __shared__ uint4 As1[BM * 8];
  __shared__ uint4 Bs0[BN * 8];
  __shared__ uint4 Bs1[BN * 8];
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

  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int begin = xcd * chunk;
  const int end = (begin + chunk < total) ? begin + chunk : total;

  const uint16_t* Ab = static_cast<const uint16_t*>(a.A);
  const uint16_t* Bb = static_cast<const uint16_t*>(a.B);
  uint16_t* Cb = static_cast<uint16_t*>(a.C);
  const int lrow = tid >> 3, lc = tid & 7;
  const int nk = K / BK;

  for (int L = begin + slot; L < end; L += nslot) {
    // ---- decode tile L -> (expert, m-tile, n-tile)
    const int q = L / NT;
    int lo = 0, hi = E;            // largest e with s_pre[e] <= q
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] <= q) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int local = L - s_pre[e] * NT;
    const int mte = s_pre[e + 1] - s_pre[e];
    // group up to kGroupM m-tiles of the expert: the ~32 tiles an XCD runs at
    // once then cover every m-tile of a weight panel, so each panel streams
    // from HBM once per group instead of once per m-tile
    const int G = mte < kGroupM ? mte : kGroupM;
    const int g = local / (G * NT);
    const int rem = local - g * G * NT;
    const int gsz = (mte - g * G < G) ? mte - g * G : G;
    const int nt = rem / gsz;
    const int mt = g * G + rem % gsz;
    const int r0 = s_off[e] + mt * BM;
    int rows = (s_off[e + 1] - r0 < BM) ? s_off[e + 1] - r0 : BM;
    if (r0 < 0 || r0 >= a.M) continue;             // malformed offsets: skip, never fault
    if (rows > a.M - r0) rows = static_cast<int>(a.M - r0);
    if (rows <= 0) continue;
    const int n0 = nt * NOUT;

    // ---- per-thread source rows (8 of A, 8 of B), clamped in bounds.  Each
    // lane fetches the 16-byte chunk that lands, through the swizzle, at its
    // own slot of the direct-to-LDS write (slot lane & 7 of row
    // r = 32 j + 8 wave + lane / 8), i.e. chunk (lane & 7) ^ ((r >> 1) & 7),
    // and (r >> 1) & 7 == (4 wave + lane / 16) & 7 for every j.
    const int lchunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
    const uint16_t* ap[8];
    const uint16_t* bp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ri = lrow + 32 * j;
      const int rr = r0 + (ri < rows ? ri : rows - 1);
      int64_t src = rr;
      if constexpr (GATHER) {
        src = a.gather[rr] / a.gather_div;
        src = src < 0 ? 0 : (src >= a.a_rows ? a.a_rows - 1 : src);
      }
      ap[j] = Ab + src * K + lchunk * 8;
      int64_t wr;
      if constexpr (SWIGLU) {
        const int n = n0 + lrow + 32 * (j & 3);
        wr = (n < a.I ? n : a.I - 1) + (j >= 4 ? a.I : 0);
      } else {
        const int n = n0 + lrow + 32 * j;
        wr = n < N ? n : N - 1;
      }
      bp[j] = Bb + static_cast<int64_t>(e) * a.b_stride + wr * K + lchunk * 8;
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // K stage kc -> LDS stage (Ad, Bd): global_load_lds_dwordx4, 8 per operand
    // per lane; wave w's j-th load fills rows 32j + 8w .. 32j + 8w + 7.
    auto issue = [&](int kc, uint4* Ad, uint4* Bd) {
      const int ko = kc * BK;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        __builtin_amdgcn_global_load_lds((glb_void*)(ap[j] + ko), (lds_void*)&Ad[(j * 4 + wave) * 64],
                                         16, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        __builtin_amdgcn_global_load_lds((glb_void*)(bp[j] + ko), (lds_void*)&Bd[(j * 4 + wave) * 64],
                                         16, 0, 0);
    };
    auto compute = [&](const uint4* Asrc, const uint4* Bsrc) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 2 * s + (lane >> 5);
        bf16x8_t xf[4], wf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xf[i] = *reinterpret_cast<const bf16x8_t*>(&Asrc[swz(wm * 128 + i * 32 + (lane & 31), c)]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int wrow;
          if constexpr (SWIGLU) wrow = (j < 2) ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32;
          else wrow = wn * 128 + j * 32;
          wf[j] = *reinterpret_cast<const bf16x8_t*>(&Bsrc[swz(wrow + (lane & 31), c)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
      }
    };

    // stage kc lives in stage buffer kc & 1; one barrier per stage both
    // publishes stage kc and frees the buffer stage kc+1 is loaded into
    issue(0, As0, Bs0);
    int kc = 0;
    for (; kc + 1 < nk; kc += 2) {
      wait_vmem();
      __syncthreads();
      issue(kc + 1, As1, Bs1);
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the MFMAs
      compute(As0, Bs0);
      wait_vmem();
      __syncthreads();
      if (kc + 2 < nk) issue(kc + 2, As0, Bs0);
      __builtin_amdgcn_sched_barrier(0);
      compute(As1, Bs1);
    }
    if (kc < nk) {          // odd number of stages: the last one sits in stage buffer 0
      wait_vmem();
      __syncthreads();
      compute(As0, Bs0);
    }
    __syncthreads();        // all reads of this tile's buffers done before the next tile's loads

    // ---- epilogue: lane holds row m, columns 8*grp + 4*(lane>>5) + 0..3 of each 32x32 tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 128 + i * 32 + (lane & 31);
      if (m >= rows) continue;
      uint16_t* crow = Cb + static_cast<int64_t>(r0 + m) * N;
      if constexpr (SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int n = n0 + wn * 64 + j * 32 + 8 * grp + 4 * (lane >> 5);
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
            const int n = n0 + wn * 128 + j * 32 + 8 * grp + 4 * (lane >> 5);
            if (n >= N) continue;
            const f32x16_t& cc = acc[i][j];
            const int b = grp * 4;
            *reinterpret_cast<uint2*>(crow + n) = pack4_bf16(cc[b], cc[b + 1], cc[b + 2], cc[b + 3]);
          }
      }
    }
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
