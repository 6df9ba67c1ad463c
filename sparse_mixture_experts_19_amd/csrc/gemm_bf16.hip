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

// silu(g) = g / (1 + e^-g), with the hardware reciprocal (1 ulp) in place of
// an IEEE divide
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// four floats -> four bf16 (round to nearest even, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  const f32x2_t lo = {a, b}, hi = {c, d};
  uint2 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t));
  o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t));
  return o;
}

// Read one accumulator element out of its AGPR at this point of the
// program.  Plain element accesses let the compiler copy all 256
// accumulators to VGPRs right after the K loop, which overflows the VGPR
// file; reading them one tile at a time keeps the epilogue small.
__device__ __forceinline__ float acc_rd(float v) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
  return r;
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
    // wave-uniform: keep the tile in scalar registers
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.r0 = __builtin_amdgcn_readfirstlane(t.r0);
    t.rows = __builtin_amdgcn_readfirstlane(t.rows);
    t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
    return t.rows > 0;
  };

  // Per-lane source rows.  Wave w's j-th DMA of a stage fills LDS rows
  // 32 j + 8 w .. +7 (8 rows x 8 slots = 64 lanes x 16 bytes); the lane
  // writes slot lane & 7 of row 32 j + 8 w + lane / 8 and so fetches chunk
  // (lane & 7) ^ ((row >> 1) & 7) == (lane & 7) ^ ((4 w + lane / 16) & 7).
  const int lchunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow = 8 * wave + (lane >> 3);
  // Row of A for DMA j of the current tile: gathered rows are looked up once
  // per tile (32-bit indices); all other rows follow from the tile scalars.
  Tile dt;                       // tile whose rows the DMAs currently fetch
  uint32_t arow[GATHER ? 8 : 1];
  auto set_rows = [&](const Tile& t) {
    dt = t;
    if constexpr (GATHER) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ri = lrow + 32 * j;
        const int rr = t.r0 + (ri < t.rows ? ri : t.rows - 1);
        int64_t src = a.gather[rr] / a.gather_div;
        src = src < 0 ? 0 : (src >= a.a_rows ? a.a_rows - 1 : src);
        arow[j] = static_cast<uint32_t>(src);
      }
    }
  };
  // The per-DMA row arithmetic is recomputed at each use (a few VALU ops
  // between MFMAs) rather than kept live across the K loop: lrow is made
  // opaque to the optimiser so that it cannot hoist 16 64-bit addresses.
  auto opaque_lrow = [&]() {
    int v = lrow;
    asm volatile("" : "+v"(v));
    return v;
  };
  auto a_row = [&](int j) -> uint64_t {
    if constexpr (GATHER) {
      uint32_t v = arow[j];
      asm volatile("" : "+v"(v));
      return v;
    } else {
      const int ri = opaque_lrow() + 32 * j;
      return static_cast<uint64_t>(dt.r0 + (ri < dt.rows ? ri : dt.rows - 1));
    }
  };
  auto b_row = [&](int j) -> uint64_t {     // row of the stacked weights [E * rows_per_expert, K]
    const int ri = opaque_lrow() + 32 * j;
    if constexpr (SWIGLU) {
      const int n = dt.n0 + (ri & 127);
      return static_cast<uint64_t>(dt.e) * (2 * a.I) + (n < a.I ? n : a.I - 1) + (j >= 4 ? a.I : 0);
    } else {
      const int n = dt.n0 + ri;
      return static_cast<uint64_t>(dt.e) * N + (n < N ? n : N - 1);
    }
  };
  const uint64_t rowbytes = static_cast<uint64_t>(K) * 2;
  const char* Abytes = reinterpret_cast<const char*>(Ab) + lchunk * 16;
  const char* Bbytes = reinterpret_cast<const char*>(Bb) + lchunk * 16;

  // LDS byte address of stage buffer b for this wave's first DMA
  const uint32_t wofs = static_cast<uint32_t>(wave) * 64 * 16;
  const uint32_t sb0 = __builtin_amdgcn_readfirstlane(lds_addr(S0) + wofs);
  const uint32_t sb1 = __builtin_amdgcn_readfirstlane(lds_addr(S1) + wofs);
  auto dma1 = [&](int kc, uint32_t sb, int t) {   // t < 8: A rows 32t.., else B rows 32(t-8)..
    const uint64_t ko = static_cast<uint64_t>(kc) * BK * 2;
    if (t < 8) dma16(Abytes + a_row(t) * rowbytes + ko, sb + t * 4 * 64 * 16);
    else dma16(Bbytes + b_row(t - 8) * rowbytes + ko, sb + BM * 8 * 16 + (t - 8) * 4 * 64 * 16);
  };

  f32x16_t acc[4][4];
  struct Frag {
    bf16x8_t x[4], w[4];
  };
  auto mfma1 = [&](const Frag& F, int t) {
    const int i = t >> 2, j = t & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.w[j], F.x[i], acc[i][j], 0, 0, 0);
  };
  // Fragment rows are (multiple of 32) + lane % 32, so their swizzle term
  // ((row >> 1) & 7) is the same lane constant sl for every fragment: one
  // byte offset per K16 step and operand, with the row differences as
  // immediates.  xo[s] / wo[s]: offsets of the first x / w fragment row.
  const int sl = ((lane & 31) >> 1) & 7;
  uint32_t xo[4], wo[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int slotv = (2 * st + (lane >> 5)) ^ sl;
    xo[st] = static_cast<uint32_t>(((wm * 128 + (lane & 31)) * 8 + slotv) * 16);
    wo[st] = static_cast<uint32_t>((BM * 8 + ((SWIGLU ? wn * 64 : wn * 128) + (lane & 31)) * 8 + slotv) * 16);
  }
  // fragment t (< 4: x[t], else w[t-4]) of K16 step s (0..3) of the stage in Ss
  auto frag1 = [&](const uint4* Ss, int s, Frag& F, int t) {
    const char* base = reinterpret_cast<const char*>(Ss);
    if (t < 4) {
      F.x[t] = *reinterpret_cast<const bf16x8_t*>(base + xo[s] + t * 32 * 128);
    } else {
      const int j = t - 4;
      const int rowoff = SWIGLU ? ((j < 2) ? j * 32 : 128 + (j - 2) * 32) : j * 32;
      F.w[j] = *reinterpret_cast<const bf16x8_t*>(base + wo[s] + rowoff * 128);
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

    // ---- epilogue.  The MFMA result leaves each lane with 4 consecutive
    // columns of one row per 32x32 tile (row i*32 + lane%32, columns
    // 8 g + 4 (lane/32) + 0..3).  Each wave stages its outputs as bf16 in its
    // own 16 KB of stage buffer S1 (free here: the next tile's first stage
    // goes to S0, and S1 is written again only after the next barrier) and
    // writes them back row-contiguously, 16 bytes per lane, so every store
    // instruction covers whole 128-byte lines.
    {
      uint8_t* stg = reinterpret_cast<uint8_t*>(S1) + wave * 16384;
      if constexpr (SWIGLU) {
        // 128 rows x 64 h-columns, 128-byte rows, chunk c of row r in slot c ^ ((r>>1)&7)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
              const int r = i * 32 + (lane & 31);
              const int c4 = j * 8 + 2 * grp + (lane >> 5);      // 4-column group 0..15
              const f32x16_t& gg = acc[i][j];
              const f32x16_t& uu = acc[i][j + 2];
              const int b = grp * 4;
              float v[4];
#pragma unroll
              for (int u = 0; u < 4; ++u) v[u] = silu_f(acc_rd(gg[b + u])) * acc_rd(uu[b + u]);
              *reinterpret_cast<uint2*>(stg + r * 128 + (((c4 >> 1) ^ ((r >> 1) & 7)) << 4) + (c4 & 1) * 8) =
                  pack4_bf16(v[0], v[1], v[2], v[3]);
              __builtin_amdgcn_sched_barrier(0);   // bounds the registers in flight
            }
        const int ncol = cur.n0 + wn * 64;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int idx = q * 64 + lane;
          const int r = idx >> 3, c = idx & 7;
          const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
          const int m = wm * 128 + r;
          if (m < cur.rows && ncol < N)
            *reinterpret_cast<uint4*>(Cb + static_cast<int64_t>(cur.r0 + m) * N + ncol + c * 8) = v;
        }
      } else {
        // two passes of 64 rows x 128 columns, 256-byte rows, chunk c of row r in slot c ^ (r&15)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int grp = 0; grp < 4; ++grp) {
                const int r = ii * 32 + (lane & 31);
                const int c4 = j * 8 + 2 * grp + (lane >> 5);    // 4-column group 0..31
                const f32x16_t& cc = acc[2 * p + ii][j];
                const int b = grp * 4;
                *reinterpret_cast<uint2*>(stg + r * 256 + (((c4 >> 1) ^ (r & 15)) << 4) + (c4 & 1) * 8) =
                    pack4_bf16(acc_rd(cc[b]), acc_rd(cc[b + 1]), acc_rd(cc[b + 2]), acc_rd(cc[b + 3]));
                __builtin_amdgcn_sched_barrier(0);
              }
          const int ncol = cur.n0 + wn * 128;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int idx = q * 64 + lane;
            const int r = idx >> 4, c = idx & 15;
            const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 256 + ((c ^ (r & 15)) << 4));
            const int m = wm * 128 + p * 64 + r;
            if (m < cur.rows && ncol + c * 8 < N)
              *reinterpret_cast<uint4*>(Cb + static_cast<int64_t>(cur.r0 + m) * N + ncol + c * 8) = v;
          }
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
