// Ragged grouped GEMMs of the expert SwiGLU MLPs on the MFMA units (gfx950),
// with bf16 operands or MXFP8 operands (e4m3 elements, one E8M0 scale per 32
// values along K).
//
// Page legend:
//   [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
//   [SonicMoE page]  "SonicMoE与传统MoE架构对比：Token舍入技术如何实现训练效率跃升"
//   [Hunyuan page]   "混合专家架构大模型Hunyuan-Large：原理剖析与实现机制"
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
// with fp32 accumulators.  K advances in 64-wide stages (whole 128-byte
// lines per row) through two 64 KB LDS buffers, fetched straight from
// L2/HBM into LDS (global_load_lds_dwordx4, no staging registers).  The
// stages of all of a workgroup's tiles form one sequence: one barrier per
// stage both publishes stage g+1 and frees stage g's buffer, stage g+2 is
// fetched while the last K16 step of stage g and the first of stage g+1 are
// multiplied, half in each, so a DMA has at least two K16 steps of MFMAs to
// land in, also across tile boundaries and under the epilogue.  DMAs take a scalar base plus a per-lane 32-bit offset set
// once per tile, so issuing one costs no vector ALU work.  Operand fragments
// are double-buffered across the four K16 steps, and the first fragments of
// a stage are read during the previous one.  LDS rows are 128 bytes whose
// 16-byte chunks are XOR-swizzled by row pairs, which keeps the MFMA operand
// reads free of bank conflicts.  The MFMA takes the weight rows as its A
// operand and the token rows as B, so each lane ends with 4 consecutive
// output columns of one row: the epilogue applies silu(g)*u in registers,
// stages bf16 rows in LDS and writes whole 128-byte lines.
//
// The data gradients of the backward multiply by W2 and W13 the other way
// round, K running along the stored weight rows' index: the weight operand
// is then N-major ([E, K, N] as stored).  In that form (BT) a stage's weight
// part holds 64 K rows of the tile's 256 columns, fetched by the same DMAs,
// and its fragments are read with the transposing LDS read, so no transposed
// copy of a weight is ever written.
//
// MXFP8 ([Hunyuan page] §七.1 runs the experts in FP8; the format is OCP
// MXFP8): the same tiles, stages and DMA plan over e4m3 bytes, so a 128-byte
// stage row holds 128 K values, multiplied in two K64 steps of the
// block-scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4.  That instruction takes
// 32 bytes per lane -- row lane % 32, bytes 0..15 holding K 16 (lane / 32) +
// 0..15 of the step and bytes 16..31 holding K 32 + 16 (lane / 32) + 0..15,
// exactly the 16-byte chunks of two bf16 K16 steps -- and per operand one
// E8M0 scale per lane, for row lane % 32 and the K values 32 (lane / 32) ..
// +31 of the step, taken from a byte of a 32-bit register that an immediate
// selects.  The four scale bytes a stage covers of a row form one 32-bit
// word, stored stage-major (the words of one stage of consecutive rows are
// contiguous: a row-major [rows, K/32] array would make each 4-byte DMA touch
// 64 cache lines, which stalled the fetch of the data behind it); the words
// of the stage's 256 token rows and 256 weight rows are
// fetched into LDS by two 4-byte DMAs per wave next to the data, and each
// lane shifts the words it reads by 8 (lane / 32) bits, so that K64 step s
// takes byte 2 s.  The SwiGLU epilogue quantizes h along its columns (the K
// of the down GEMM): the 32 columns of a block of one token row sit in lanes
// l and l + 32 of one 32x32 result tile, which agree on the block's largest
// magnitude through one lane exchange.
#include <type_traits>

#include "moe_internal.h"
#include "cdna4.h"

namespace moe {
namespace {

constexpr int BM = kGemmBM;   // 256 rows
constexpr int BN = kGemmBN;   // 256 weight rows (swiglu: 128 gate + 128 up)
constexpr int BK = kGemmBK;   // 64
constexpr int kStageBytes = 128;  // bytes of a row per K stage (both formats)
constexpr int kGroupM = 8;    // m-tiles walked together inside an expert

// K values per stage: 64 bf16 or 128 e4m3
template <bool MX>
constexpr int stage_k() { return MX ? 2 * BK : BK; }

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int swz(int r, int c) { return swz128(r, c); }

// silu(g) = g / (1 + e^-g), with the hardware reciprocal (1 ulp) in place of
// an IEEE divide
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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

// Tile L of a grouped GEMM with NT output-column tiles of nout columns ->
// (expert, first row, rows, first output column).  pre/off: tile prefix and
// row offsets per expert.  Inside an expert up to kGroupM m-tiles are walked
// n-tile-major: the ~32 tiles an XCD runs at once cover every m-tile of a
// weight panel, so a panel streams from HBM once per group instead of once
// per m-tile.  False for tiles that malformed offsets would place outside
// [0, M).  L is wave-uniform, and so is the tile: it is kept, with every
// decision taken on it, in scalar registers.
__device__ __forceinline__ bool decode_tile(int L, int NT, int nout, int E, const int* pre,
                                            const int* off, int64_t M, Tile& t) {
  const int q = L / NT;
  int lo = 0, hi = E;            // largest e with pre[e] <= q
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= q) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int local = L - pre[e] * NT;
  const int mte = pre[e + 1] - pre[e];
  const int G = mte < kGroupM ? mte : kGroupM;
  const int g = local / (G * NT);
  const int rem = local - g * G * NT;
  const int gsz = (mte - g * G < G) ? mte - g * G : G;
  const int nt = rem / gsz;
  const int mt = g * G + rem % gsz;
  t.e = __builtin_amdgcn_readfirstlane(e);
  t.r0 = __builtin_amdgcn_readfirstlane(off[e] + mt * BM);
  const int e_end = __builtin_amdgcn_readfirstlane(off[e + 1]);
  t.rows = (e_end - t.r0 < BM) ? e_end - t.r0 : BM;
  t.n0 = nt * nout;
  if (t.r0 < 0 || t.r0 >= M) return false;
  if (t.rows > M - t.r0) t.rows = static_cast<int>(M - t.r0);
  return t.rows > 0;
}

// Work split of a grouped GEMM over G persistent workgroups.  The first
// `full` tiles (a multiple of G) are computed whole, full / G per workgroup.
// The remaining rem < G tiles would leave most workgroups idle for a whole
// tile; when G allows, each is cut along K into `ways` pieces of at least
// kMinPiece stages (shorter pieces cost more in partial sums than they save)
// that run on different workgroups and leave fp32 partial sums, which the
// fixup kernel adds in piece order (deterministic) and finishes with the
// epilogue.
constexpr int kMinPiece = 16;
struct Split {
  int full, rem, ways;
};
__device__ __forceinline__ Split split_work(int total, int G, int nk, int max_pieces) {
  Split sp;
  sp.full = total / G * G;
  sp.rem = total - sp.full;
  sp.ways = 1;
  if (sp.rem > 0) {
    int w = G / sp.rem;
    w = w < nk / kMinPiece ? w : nk / kMinPiece;
    w = w < max_pieces / sp.rem ? w : max_pieces / sp.rem;
    if (w >= 2) sp.ways = w;
  }
  return sp;
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// BT: B is N-major (element (k, n) of expert e at B + ((e K + k) N + n) * 2,
// as the expert weights are stored for the transposed products of the
// backward).  A stage's B part then holds 64 K rows of 512 bytes (the tile's
// 256 columns), 16-byte chunk c of K row k in slot c ^ (4 (k & 3)); the B
// fragments are read with ds_read_b64_tr_b16, which, within each group of 16
// lanes, hands lane i element i of the four 16-value rows that lanes 4j..4j+3
// supply: lanes reading 4 K rows x 16 consecutive columns thus receive, per
// column, 4 consecutive K values, the MFMA operand layout (two reads give the
// 8 values of a K16 step).
template <bool MX, bool SWIGLU, bool GATHER, bool WG = false, bool SAVE = false, bool BT = false>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs a) {
  // two stage buffers as distinct arrays (each holds the A rows then the B
  // rows of one 128-byte K stage)
  __shared__ uint4 S0[(BM + BN) * 8];
  __shared__ uint4 S1[(BM + BN) * 8];
  __shared__ uint4 STG[4 * 256];        // epilogue staging, 4 KB per wave
  __shared__ int32_t SROW[2 * 256];     // scattered output rows, by tile parity
  // MX: scale words of the two stages, each 256 token rows then 256 weight rows
  __shared__ uint32_t SSC[MX ? 2 * 512 : 1];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_pre[kMaxE + 1];
  __shared__ int s_koff[WG ? kMaxE + 1 : 1];   // WG: K range of each group, in stages

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int E = a.E;
  for (int i = tid; i <= E; i += 256) {
    s_off[i] = a.offsets[i];
    s_pre[i] = a.prefix[i];
    if constexpr (WG) s_koff[i] = a.koff[i] / BK;
  }
  __syncthreads();

  constexpr int NOUT = SWIGLU ? BN / 2 : BN;   // output columns per tile
  const int N = a.N, K = a.K;
  const int NT = (N + NOUT - 1) / NOUT;
  const int total = s_pre[E] * NT;
  const int nk = K / stage_k<MX>();

  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  const Split sp = split_work(total, gridDim.x, nk, a.max_pieces);
  const int nf = sp.full / gridDim.x;          // whole tiles of this workgroup
  const int xbegin = xcd * (sp.full >> 3);     // its XCD's range of whole tiles

  const uint16_t* Bb = static_cast<const uint16_t*>(a.B);
  uint16_t* Cb = static_cast<uint16_t*>(a.C);

  // Work item i of this workgroup: its whole tiles (XCD-aware walk), then
  // one remainder tile or one K piece of one.  Returns 0 past the end, 2 for
  // an item that malformed offsets make empty (skipped), else 1.
  struct Item {
    Tile t;
    int k0, k1, pslot;      // K stages [k0, k1); partial-sum slot or -1
  };
  auto item = [&](int i, Item& it) -> int {
    int L;
    it.k0 = 0;
    it.k1 = nk;
    it.pslot = -1;
    if (i < nf) {
      L = xbegin + slot + i * nslot;
    } else if (i == nf) {
      const int b = blockIdx.x;
      if (sp.ways > 1) {
        if (b >= sp.rem * sp.ways) return 0;
        L = sp.full + b / sp.ways;
        const int p = b % sp.ways;
        it.k0 = p * nk / sp.ways;
        it.k1 = (p + 1) * nk / sp.ways;
        it.pslot = b;
      } else {
        if (b >= sp.rem) return 0;
        L = sp.full + b;
      }
    } else {
      return 0;
    }
    if (!decode_tile(L, NT, NOUT, E, s_pre, s_off, a.M, it.t)) return 2;
    if constexpr (WG) {
      it.k0 = s_koff[it.t.e];
      it.k1 = s_koff[it.t.e + 1];
      if (it.k1 <= it.k0) return 2;
    }
    return 1;
  };
  auto next_item = [&](int i, Item& it) -> int {   // index of the first item >= i, or -1
    for (;; ++i) {
      const int r = item(i, it);
      if (r == 1) return i;
      if (r == 0) return -1;
    }
  };

  // DMA addressing.  Wave w's DMA t of a stage fills LDS rows 32 (t & 7) +
  // 8 w .. +7 of the A part (t < 8) or the B part (t >= 8): 8 rows x 8 slots
  // = 64 lanes x 16 bytes; the lane writes slot lane & 7 of row
  // 32 (t & 7) + 8 w + lane / 8 and so fetches chunk
  // (lane & 7) ^ ((row >> 1) & 7) == (lane & 7) ^ ((4 w + lane / 16) & 7).
  // Each DMA is "wave-uniform base (SGPR pair) + 32-bit lane offset": the
  // bases of a tile are set once and move by the stage's K offset; the lane
  // offsets (row within the tile, clamped for tails, times the row pitch,
  // plus the chunk) are computed once per tile, so issuing a DMA costs no
  // vector ALU work.  Gathered A rows are looked up when the DMA cursor
  // enters a tile and converted (permutation entry / k, clamped) at the
  // first issue after the next barrier, when the loads are known to be done.
  //
  // MX: lane l of wave w also fetches the scale words of tile row 64 w + l
  // (clamped): a token row and a weight row (swiglu: waves 0-1 gate rows,
  // waves 2-3 up rows).  The words are stage-major (word s of row r at index
  // s * rows + r), so a wave's 64 words are 256 contiguous bytes; the A-side
  // words follow the GEMM's own rows, also when A itself is gathered (the
  // forward writes them in permuted row order).  The bases move by rows * 4
  // bytes per stage.
  const int lchunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow = 8 * wave + (lane >> 3);
  const uint64_t rowbytes = WG ? static_cast<uint64_t>(a.ld) * 2 : static_cast<uint64_t>(K) * (MX ? 1 : 2);
  const uint32_t rb32 = static_cast<uint32_t>(rowbytes);
  const char* Ach = static_cast<const char*>(a.A);
  const char* Bch = reinterpret_cast<const char*>(Bb);
  uint32_t voff[16];
  const char* dA;                 // A base of the DMA tile (stage 0)
  const char* dB0;                // B base (swiglu: gate rows)
  const char* dB1;                // swiglu: up rows
  int32_t graw[GATHER ? 8 : 1];   // raw permutation entries of the gathered rows
  bool gpend = false;
  const int srow = 64 * wave + lane;                     // MX: tile row of this lane's scale words
  uint32_t sxoff = 0, swoff = 0;  // MX: lane offsets of the token / weight scale DMAs
  const uint8_t* dSx = nullptr;   // MX: scale bases of the DMA tile (stage 0)
  const uint8_t* dSw = nullptr;
  auto set_rows = [&](const Tile& t) {
    if constexpr (MX) {
      const int sr = srow < t.rows ? srow : t.rows - 1;
      sxoff = static_cast<uint32_t>(sr) * 4u;
      dSx = a.a_scale + static_cast<uint64_t>(t.r0) * 4;
      if constexpr (SWIGLU) {
        const int nb = a.I - t.n0;
        const int rr = srow & 127;
        swoff = static_cast<uint32_t>(rr < nb ? rr : nb - 1) * 4u;
        dSw = a.b_scale + (static_cast<uint64_t>(t.e) * (2 * a.I) + t.n0 + (wave >= 2 ? a.I : 0)) * 4;
      } else {
        const int nb = N - t.n0;
        swoff = static_cast<uint32_t>(srow < nb ? srow : nb - 1) * 4u;
        dSw = a.b_scale + (static_cast<uint64_t>(t.e) * N + t.n0) * 4;
      }
    }
    if constexpr (GATHER) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ri = lrow + 32 * j;
        graw[j] = a.gather[t.r0 + (ri < t.rows ? ri : t.rows - 1)];
      }
      gpend = true;
      dA = Ach;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ri = lrow + 32 * j;
        voff[j] = static_cast<uint32_t>(ri < t.rows ? ri : t.rows - 1) * rb32 + lchunk * 16;
      }
      // WG: the rows of group e are rows 0.. of A (its K range selects the expert)
      dA = Ach + static_cast<uint64_t>(WG ? t.r0 - t.e * a.group_rows : t.r0) * rowbytes;
    }
    if constexpr (SWIGLU) {
      const int nb = a.I - t.n0;          // rows of each half left from n0
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rr = (lrow + 32 * j) & 127;
        voff[8 + j] = static_cast<uint32_t>(rr < nb ? rr : nb - 1) * rb32 + lchunk * 16;
      }
      dB0 = Bch + (static_cast<uint64_t>(t.e) * (2 * a.I) + t.n0) * rowbytes;
      dB1 = dB0 + static_cast<uint64_t>(a.I) * rowbytes;
    } else if constexpr (BT) {
      // DMA 8 + j of wave w fills K rows 8 j + 2 w and + 1 of the B part (the
      // lane: row + lane / 32, slot lane % 32, i.e. column chunk
      // (lane % 32) ^ (4 ((2 w + lane / 32) & 3)), clamped to the last chunk
      // of the matrix for a tail tile)
      const int nb = N - t.n0;
      const int half = lane >> 5;
      const int cs = (lane & 31) ^ (4 * ((2 * wave + half) & 3));
      const int cc = cs * 8 < nb ? cs : nb / 8 - 1;
      const uint32_t rowb = static_cast<uint32_t>(N) * 2u;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        voff[8 + j] = static_cast<uint32_t>(8 * j + 2 * wave + half) * rowb + static_cast<uint32_t>(cc) * 16u;
      dB0 = Bch + (static_cast<uint64_t>(t.e) * K * N + t.n0) * 2;
      dB1 = dB0;
    } else {
      const int nb = N - t.n0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rr = lrow + 32 * j;
        voff[8 + j] = static_cast<uint32_t>(rr < nb ? rr : nb - 1) * rb32 + lchunk * 16;
      }
      dB0 = Bch + (static_cast<uint64_t>(WG ? 0 : t.e) * N + t.n0) * rowbytes;
      dB1 = dB0;
    }
  };
  // gathered row = entry / k by multiply-high (exact for entries < 2^31),
  // clamped into A; A spans fewer than 2^32 bytes (checked at launch)
  auto grow = [&](int32_t raw) -> uint32_t {
    const uint32_t v = static_cast<uint32_t>(raw < 0 ? 0 : raw);
    const uint32_t q = a.gather_magic ? (__umulhi(v, a.gather_magic) >> a.gather_shift) : (v >> a.gather_shift);
    return q < static_cast<uint32_t>(a.a_rows) ? q : static_cast<uint32_t>(a.a_rows - 1);
  };
  auto gconv = [&]() {
    if constexpr (GATHER) {
      if (gpend) {
#pragma unroll
        for (int j = 0; j < 8; ++j) voff[j] = grow(graw[j]) * rb32 + lchunk * 16;
        gpend = false;
      }
    }
  };

  // LDS byte address of stage buffer b for this wave's first DMA
  const uint32_t wofs = static_cast<uint32_t>(wave) * 64 * 16;
  const uint32_t sb0 = __builtin_amdgcn_readfirstlane(lds_addr(S0) + wofs);
  const uint32_t sb1 = __builtin_amdgcn_readfirstlane(lds_addr(S1) + wofs);
  // MX: LDS byte address of this wave's token scale words in stage buffer 0
  // (buffer b: + 2048 b; weight scale words: + 1024)
  const uint32_t scb = MX ? __builtin_amdgcn_readfirstlane(lds_addr(SSC) + wave * 256) : 0;
  // bytes a stage moves the B base: 64 K values of a row, or (BT) 64 rows
  const uint64_t bstage = BT ? static_cast<uint64_t>(BK) * N * 2 : static_cast<uint64_t>(kStageBytes);
  auto dma1 = [&](int kc, uint32_t sb, int t) {   // t < 8: A rows 32t.., else B rows 32(t-8)..
    const uint64_t ko = static_cast<uint64_t>(kc) * (t < 8 ? static_cast<uint64_t>(kStageBytes) : bstage);
    const char* base = t < 8 ? dA : ((SWIGLU && t >= 12) ? dB1 : dB0);
    dma16s(base + ko, voff[t], sb + (t < 8 ? t * 4 * 64 * 16 : BM * 8 * 16 + (t - 8) * 4 * 64 * 16));
  };
  auto dma_sc1 = [&](int kc, int buf) {           // MX: the scale words of stage kc
    if constexpr (MX) {
      dma4s(dSx + static_cast<uint64_t>(kc) * a.a_srows * 4, sxoff, scb + buf * 2048);
      dma4s(dSw + static_cast<uint64_t>(kc) * a.b_srows * 4, swoff, scb + buf * 2048 + 1024);
    }
  };
  // The global bases of stage kc, pinned to scalar registers once, so that
  // each DMA of the stage is one M0 write and the load.
  struct StageBase {
    const char *a, *b0, *b1;
    const uint8_t *sx, *sw;
  };
  auto stage_base = [&](int kc) -> StageBase {
    const uint64_t ko = static_cast<uint64_t>(kc) * kStageBytes;
    auto pin = [](const auto* p) {
      const uint64_t v = reinterpret_cast<uintptr_t>(p);
      const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
      const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
      return reinterpret_cast<decltype(p)>(static_cast<uintptr_t>((hi << 32) | lo));
    };
    const uint64_t kob = static_cast<uint64_t>(kc) * bstage;
    StageBase g{pin(dA + ko), pin(dB0 + kob), pin(SWIGLU ? dB1 + kob : dB0 + kob), nullptr, nullptr};
    if constexpr (MX) {
      g.sx = pin(dSx + static_cast<uint64_t>(kc) * a.a_srows * 4);
      g.sw = pin(dSw + static_cast<uint64_t>(kc) * a.b_srows * 4);
    }
    return g;
  };
  auto dma_pre = [&](const StageBase& g, uint32_t sb, int t) {
    const char* base = t < 8 ? g.a : ((SWIGLU && t >= 12) ? g.b1 : g.b0);
    dma16p(base, voff[t], sb + (t < 8 ? t * 4 * 64 * 16 : BM * 8 * 16 + (t - 8) * 4 * 64 * 16));
  };
  auto dma_sc_pre = [&](const StageBase& g, int buf) {
    if constexpr (MX) {
      dma4p(g.sx, sxoff, scb + buf * 2048);
      dma4p(g.sw, swoff, scb + buf * 2048 + 1024);
    }
  };

  f32x16_t acc[4][4];
  struct FragB {
    bf16x8_t x[4], w[4];
  };
  struct FragM {                  // MX: one K64 step
    i32x8_t x[4], w[4];
  };
  using Frag = typename std::conditional<MX, FragM, FragB>::type;
  auto mfma1 = [&](const Frag& F, int t) {
    if constexpr (!MX) {
      const int i = t >> 2, j = t & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.w[j], F.x[i], acc[i][j], 0, 0, 0);
    }
  };
  // MX: an empty asm that reads and rewrites every accumulator in place.  It
  // keeps the MFMAs of a K64 step ahead of the barrier or loop edge that
  // follows: the code generator would otherwise sink the MFMAs, whose results
  // only feed the next iteration, past the stage's LDS reads and DMAs, which
  // then no longer overlap the matrix work.
  auto pin_acc = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
  };
  // MX: K64 step `second` of a stage, with the stage's scale words (shifted
  // by 8 (lane / 32) bits: byte 2 second is this lane's block)
  auto mfma_mx = [&](const Frag& F, int t, bool second, const uint32_t* sx, const uint32_t* sw) {
    if constexpr (MX) {
      const int i = t >> 2, j = t & 3;
      if (second)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            F.w[j], F.x[i], acc[i][j], 0, 0, 2, static_cast<int>(sw[j]), 2, static_cast<int>(sx[i]));
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            F.w[j], F.x[i], acc[i][j], 0, 0, 0, static_cast<int>(sw[j]), 0, static_cast<int>(sx[i]));
    }
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
  // BT: byte offset of this lane's first transposing read of w fragment j:
  // lane 16 g + 4 jr + m reads K row 8 (g / 2) + jr (+ 16 s, + 4 for the
  // second read) at columns 32 j + 16 (g & 1) + 4 m .. + 3 of the wave's 128
  uint32_t btr[4];
  {
    const int g16 = lane >> 4, jr = (lane >> 2) & 3, mm = lane & 3;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      btr[j] = static_cast<uint32_t>(BM * 128 + (8 * (g16 >> 1) + jr) * 512 + (mm & 1) * 8 +
                                     (16 * wn + 4 * (j ^ jr) + 2 * (g16 & 1) + (mm >> 1)) * 16);
  }
  // fragment t (< 4: x[t], else w[t-4]) of K16 step s (0..3) of the stage in
  // Ss; MX: of K64 step s (0..1), the chunks of K16 steps 2 s and 2 s + 1
  auto frag1 = [&](const uint4* Ss, int s, Frag& F, int t) {
    const char* base = reinterpret_cast<const char*>(Ss);
    if constexpr (MX) {
      if (t < 4) {
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(base + xo[2 * s] + t * 32 * 128);
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(base + xo[2 * s + 1] + t * 32 * 128);
        F.x[t] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        const int j = t - 4;
        const int rowoff = SWIGLU ? ((j < 2) ? j * 32 : 128 + (j - 2) * 32) : j * 32;
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(base + wo[2 * s] + rowoff * 128);
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(base + wo[2 * s + 1] + rowoff * 128);
        F.w[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    } else {
      if (t < 4) {
        F.x[t] = *reinterpret_cast<const bf16x8_t*>(base + xo[s] + t * 32 * 128);
      } else if constexpr (BT) {
        const int j = t - 4;
        typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + btr[j] + s * 16 * 512));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + btr[j] + s * 16 * 512 + 4 * 512));
        F.w[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        const int j = t - 4;
        const int rowoff = SWIGLU ? ((j < 2) ? j * 32 : 128 + (j - 2) * 32) : j * 32;
        F.w[j] = *reinterpret_cast<const bf16x8_t*>(base + wo[s] + rowoff * 128);
      }
    }
  };
  // MX: scale words of the fragments of the stage in buffer buf (token rows
  // of x[i], weight rows of w[j]), shifted by 8 (lane / 32) bits
  const int lsh = 8 * (lane >> 5);
  auto read_sc = [&](int buf, uint32_t* sx, uint32_t* sw) {
    if constexpr (MX) {
      const uint32_t* S = SSC + buf * 512;
#pragma unroll
      for (int i = 0; i < 4; ++i) sx[i] = S[wm * 128 + i * 32 + (lane & 31)] >> lsh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int wr = SWIGLU ? (j < 2 ? wn * 64 + 32 * j : 128 + wn * 64 + 32 * (j - 2)) : wn * 128 + 32 * j;
        sw[j] = S[256 + wr + (lane & 31)] >> lsh;
      }
    }
  };

  // ---- pipeline.  The stages of all tiles of this workgroup form one
  // sequence g = 0, 1, ...; stage g sits in buffer g & 1.  Per stage: K16
  // steps 0..2 are multiplied while the fragments of steps 1..3 are read;
  // then one barrier, reached after this lane's DMAs of stage g+1 landed and
  // its reads of stage g completed, both publishes stage g+1 and frees
  // buffer g & 1.  Step 3 is multiplied while the step-0 fragments of stage
  // g+1 are read and the first half of stage g+2 is fetched into that
  // buffer; the second half is fetched during step 0 of stage g+1.  Spread
  // over two K16 steps, 8 DMAs per wave in each, the fetch no longer stalls
  // the MFMA issue the way 16 DMAs in one step did, and every DMA still has
  // at least two K16 steps of MFMAs to land in (one step, as a three-step
  // spread leaves, is too short).  No stage starts with an LDS wait.  The
  // DMA cursor (dkc and the bases above) runs up to two stages ahead of the
  // MFMAs, across tile boundaries and under the epilogue, and decodes tiles
  // on its own; gathered rows of a new tile are loaded one barrier before
  // their first use.  MX stages are two K64 steps, and the whole fetch of
  // stage g+2 already spans the second one.
  Item ci;                                   // item whose outputs the MFMAs compute
  int cidx = next_item(0, ci);
  if (cidx < 0) return;
  // Scattered C rows (down GEMM of the fused forward): the tile's 256
  // scatter entries are fetched into LDS by one 4-byte DMA per wave when the
  // tile starts (row 64 w + lane, clamped into the tile), in the buffer of the
  // tile's parity; the first stage's wait and barrier retire them long before
  // the epilogue reads them.
  const bool scat = !SWIGLU && a.scatter != nullptr;
  int spar = 0;                       // SROW buffer of the tile being multiplied
  auto load_srows = [&](const Tile& t) {
    if constexpr (!SWIGLU) {
      if (scat) {
        const int m = 64 * wave + lane;
        const uint32_t off = static_cast<uint32_t>(m < t.rows ? m : t.rows - 1) * 4u;
        dma4s(a.scatter + t.r0, off, __builtin_amdgcn_readfirstlane(lds_addr(SROW) + spar * 1024 + wave * 256));
      }
    }
  };
  load_srows(ci.t);
  Item di = ci;                              // item the DMAs fetch
  int didx = cidx, dkc = ci.k0;
  bool dlive = true;
  set_rows(ci.t);
  auto dma_advance = [&]() {
    if (++dkc == di.k1) {
      didx = next_item(didx + 1, di);
      if (didx >= 0) {
        dkc = di.k0;
        set_rows(di.t);
      } else {
        dlive = false;
      }
    }
  };

  int ckc = ci.k0;  // K stage being multiplied
  StageBase gq{};   // bf16: bases of the stage whose fetch is under way
  gconv();
#pragma unroll
  for (int t = 0; t < 16; ++t) dma1(dkc, sb0, t);
  dma_sc1(dkc, 0);
  dma_advance();
  if constexpr (MX) {
    if (dlive) {
      gconv();
#pragma unroll
      for (int t = 0; t < 16; ++t) dma1(dkc, sb1, t);
      dma_sc1(dkc, 1);
      dma_advance();
    }
  } else {
    // the first half of stage 1; the first stage fetches the rest
    if (dlive) gconv();
    gq = stage_base(dlive ? dkc : 0);
#pragma unroll
    for (int t = 0; t < 8; ++t) dma_pre(gq, sb1, t);
  }
  wait_vmcnt0();
  lds_barrier();

  Frag Fa, Fb;
  uint32_t csx[4], csw[4];         // MX: scale words of the stage being multiplied
#pragma unroll
  for (int t = 0; t < 8; ++t) frag1(S0, 0, Fa, t);
  read_sc(0, csx, csw);
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  zero_acc();

  // Multiply the stage in buffer par (the other buffer holds the next stage).
  // Returns whether it was the last stage of its tile.
  auto stage = [&](int par) -> bool {
    const uint4* Sc = par ? S1 : S0;
    const uint4* Sn = par ? S0 : S1;
    const uint32_t sbc = par ? sb1 : sb0;
    const uint32_t sbn = par ? sb0 : sb1;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MX) {
      // two K64 steps: step 0 reads the fragments of step 1; after the
      // barrier step 1 reads the fragments and scale words of stage g+1 and
      // fetches stage g+2 (data and scales) into the freed buffer
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        mfma_mx(Fa, t, false, csx, csw);
        if (t < 8) frag1(Sc, 1, Fb, t);
        __builtin_amdgcn_sched_barrier(0);
      }
      pin_acc();
      wait_vmcnt0();
      lds_barrier();
      const bool last = ckc == ci.k1 - 1;
      if (dlive) gconv();
      const StageBase gb = stage_base(dlive ? dkc : 0);
      uint32_t nsx[4], nsw[4];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        mfma_mx(Fb, t, true, csx, csw);
        if (t < 8) frag1(Sn, 0, Fa, t);
        if (t == 8) read_sc(par ^ 1, nsx, nsw);
        dma_pre(gb, sbc, t);
        if (t == 15) dma_sc_pre(gb, par);
        __builtin_amdgcn_sched_barrier(0);
      }
      pin_acc();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        csx[i] = nsx[i];
        csw[i] = nsw[i];
      }
      if (dlive) dma_advance();
      if (!last) ++ckc;
      return last;
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) {     // step 0; read step 1, fetch the rest of g+1
        mfma1(Fa, t);
        if (t < 8) frag1(Sc, 1, Fb, t);
        if ((t & 1) == 0) dma_pre(gq, sbn, 8 + (t >> 1));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (dlive) dma_advance();
#pragma unroll
      for (int t = 0; t < 16; ++t) {     // step 1; read step 2
        mfma1(Fb, t);
        if (t < 8) frag1(Sc, 2, Fa, t);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {     // step 2; read step 3
        mfma1(Fa, t);
        if (t < 8) frag1(Sc, 3, Fb, t);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_vmcnt0();                     // stage g+1 (the only DMAs in flight) landed
      lds_barrier();                     // ... everywhere, and stage g is no longer read
      const bool last = ckc == ci.k1 - 1;
      if (dlive) gconv();
      // Branch-free fetches.  With nothing left to fetch the DMAs re-read
      // stage 0 of the last tile into the buffer just freed (valid memory,
      // never read again); the kernel waits for them before it ends.
      gq = stage_base(dlive ? dkc : 0);
#pragma unroll
      for (int t = 0; t < 16; ++t) {     // step 3; read step 0 of g+1, fetch half of g+2
        mfma1(Fb, t);
        if (t < 8) frag1(Sn, 0, Fa, t);  // stale but harmless when g+1 does not exist
        if ((t & 1) == 0) dma_pre(gq, sbc, t >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!last) ++ckc;
      return last;
    }
  };

  int par = 0;      // buffer of the stage being multiplied
  while (true) {
    bool fin;
    do {
      fin = stage(par);
      par ^= 1;
    } while (!fin);
    // MFMA results are read by VALU instructions below: leave the wait
    // states the last MFMA needs before its accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    if (ci.pslot >= 0) {
      // ---- K piece: raw fp32 sums into its partial slot, [256 token rows]
      // x [256 weight rows of the tile] (swiglu: 128 gate rows, then 128 up)
      float* P = a.partials + static_cast<int64_t>(ci.pslot) * (BM * BN);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int row = wm * 128 + i * 32 + (lane & 31);
            const int wrow = (SWIGLU ? (j < 2 ? wn * 64 + 32 * j : 128 + wn * 64 + 32 * (j - 2))
                                     : wn * 128 + 32 * j) +
                             8 * grp + 4 * (lane >> 5);
            float4 v;
            v.x = acc_rd(acc[i][j][4 * grp]);
            v.y = acc_rd(acc[i][j][4 * grp + 1]);
            v.z = acc_rd(acc[i][j][4 * grp + 2]);
            v.w = acc_rd(acc[i][j][4 * grp + 3]);
            *reinterpret_cast<float4*>(P + row * BN + wrow) = v;
            __builtin_amdgcn_sched_barrier(0);
          }
    } else if constexpr (WG) {
      // ---- weight gradient: fp32 sums to Cf (row-major, N columns).  Each
      // 32x32 result tile is staged in the wave's 4 KB of LDS (128-byte rows,
      // 16-byte chunk c of row r in slot c ^ (r & 7)) and stored as whole
      // 128-byte row segments.
      float* stg = reinterpret_cast<float*>(STG) + wave * 1024;
      const int r = lane & 31;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int c = 2 * grp + (lane >> 5);          // 16-byte chunk of the row
            float4 v;
            v.x = acc_rd(acc[i][j][4 * grp]);
            v.y = acc_rd(acc[i][j][4 * grp + 1]);
            v.z = acc_rd(acc[i][j][4 * grp + 2]);
            v.w = acc_rd(acc[i][j][4 * grp + 3]);
            *reinterpret_cast<float4*>(stg + r * 32 + ((c ^ (r & 7)) << 2)) = v;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int rr = q * 8 + (lane >> 3), c = lane & 7;
            const float4 v = *reinterpret_cast<const float4*>(stg + rr * 32 + ((c ^ (rr & 7)) << 2));
            const int row = wm * 128 + i * 32 + rr;
            const int col = ci.t.n0 + wn * 128 + 32 * j + 4 * c;
            // streaming stores: the fp32 sums are written once and not read
            // back here, and kept out of the way of the operand panels in L2
            if (row < ci.t.rows && col < N)
              __builtin_nontemporal_store(__builtin_bit_cast(f32x4_t, v),
                                          reinterpret_cast<f32x4_t*>(a.Cf + static_cast<int64_t>(ci.t.r0 + row) * N + col));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (MX && SWIGLU) {
      // ---- MXFP8 epilogue: h = silu(g) * u quantized along its columns.
      // Per 32x32 result tile a lane holds 16 of the 32 columns of one token
      // row (columns 8 g + 4 (lane / 32) + 0..3); lanes l and l ^ 32 share
      // the row and exchange their largest magnitudes.  The e4m3 codes of 32
      // rows x the wave's 64 columns are staged in LDS (64-byte rows, 16-byte
      // chunk c of row r in slot c ^ ((r >> 2) & 3)) and stored as whole
      // 64-byte row segments; the two scale bytes of a row go out as one
      // 16-bit store.
      uint8_t* stg = reinterpret_cast<uint8_t*>(STG) + wave * 4096;
      uint8_t* Cq = static_cast<uint8_t*>(a.C);
      const int r = lane & 31;
      const int col0 = ci.t.n0 + wn * 64;             // first h column of the wave
      const int csw_r = ((r >> 2) & 3) << 2;           // staging swizzle of row r, in words
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t sc2 = 0;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const f32x16_t& gg = acc[i][jj];
          const f32x16_t& uu = acc[i][jj + 2];
          float v[16];
          float m = 0.f;
#pragma unroll
          for (int b = 0; b < 16; ++b) {
            v[b] = silu_f(acc_rd(gg[b])) * acc_rd(uu[b]);
            m = __builtin_fmaxf(m, __builtin_fabsf(v[b]));
          }
          m = __builtin_fmaxf(m, __shfl_xor(m, 32));
          const int ex = mx_block_exp(m);
          const float sc = mx_inv_scale(ex);
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int c4 = jj * 8 + 2 * grp + (lane >> 5);   // 4-column group 0..15
            *reinterpret_cast<uint32_t*>(stg + r * 64 + ((c4 ^ csw_r) << 2)) =
                mx_encode4(v[4 * grp], v[4 * grp + 1], v[4 * grp + 2], v[4 * grp + 3], sc);
          }
          sc2 |= static_cast<uint32_t>(ex + 127) << (8 * jj);
          __builtin_amdgcn_sched_barrier(0);
        }
        const int row0 = wm * 128 + i * 32;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int rr = q * 16 + (lane >> 2), c = lane & 3;
          const uint4 v = *reinterpret_cast<const uint4*>(stg + rr * 64 + ((c ^ ((rr >> 2) & 3)) << 4));
          const int m = row0 + rr;
          if (m < ci.t.rows && col0 < N)
            *reinterpret_cast<uint4*>(Cq + static_cast<int64_t>(ci.t.r0 + m) * N + col0 + c * 16) = v;
        }
        const int m = row0 + r;
        if (lane < 32 && m < ci.t.rows && col0 < N)
          *reinterpret_cast<uint16_t*>(a.c_scale + (static_cast<int64_t>(col0 / 128) * a.c_srows + ci.t.r0 + m) * 4 +
                                       (col0 / 32) % 4) = static_cast<uint16_t>(sc2);
      }
    } else
    // ---- epilogue (the next stages are in flight meanwhile).  The MFMA
    // result leaves each lane with 4 consecutive columns of one row per 32x32
    // tile (row i*32 + lane%32, columns 8 g + 4 (lane/32) + 0..3).  A wave
    // writes its 128 x 64 (swiglu) or 128 x 128 (down) outputs in passes of
    // 32 rows x 64 columns: the pass is staged as bf16 in the wave's own 4 KB
    // of LDS (128-byte rows, chunk c of row r in slot c ^ ((r >> 1) & 7)) and
    // read back row-contiguously, so each store instruction writes whole
    // 128-byte lines.
    {
      uint8_t* stg = reinterpret_cast<uint8_t*>(STG) + wave * 4096;
      auto write_back = [&](int row0, int col0) {
        const int r = lane >> 3, c = lane & 7;    // chunk q*64 + lane: row q*8 + r
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = q * 8 + r;
          const uint4 v = *reinterpret_cast<const uint4*>(stg + rr * 128 + ((c ^ ((rr >> 1) & 7)) << 4));
          const int m = row0 + rr;
          int64_t crow = ci.t.r0 + m;
          if constexpr (!SWIGLU) {
            if (scat) crow = SROW[spar * 256 + (m < ci.t.rows ? m : ci.t.rows - 1)];
          }
          if (m < ci.t.rows && col0 < N)
            *reinterpret_cast<uint4*>(Cb + crow * N + col0 + c * 8) = v;
        }
      };
      const int r = lane & 31;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int h = 0; h < (SWIGLU ? 1 : 2); ++h) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
              const int c4 = jj * 8 + 2 * grp + (lane >> 5);     // 4-column group 0..15
              const int b = grp * 4;
              float v[4];
              if constexpr (SWIGLU) {
                const f32x16_t& gg = acc[i][jj];
                const f32x16_t& uu = acc[i][jj + 2];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = silu_f(acc_rd(gg[b + u])) * acc_rd(uu[b + u]);
              } else {
                const f32x16_t& cc = acc[i][2 * h + jj];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = acc_rd(cc[b + u]);
              }
              *reinterpret_cast<uint2*>(stg + r * 128 + (((c4 >> 1) ^ ((r >> 1) & 7)) << 4) + (c4 & 1) * 8) =
                  pack4_bf16(v[0], v[1], v[2], v[3]);
              __builtin_amdgcn_sched_barrier(0);   // bounds the registers in flight
            }
          write_back(wm * 128 + i * 32, ci.t.n0 + (SWIGLU ? wn * 64 : wn * 128 + h * 64));
          if constexpr (SWIGLU && SAVE) {
            // the gate and the up sums too, rounded to bf16, into C2 [M, 2I]
            uint16_t* C2 = static_cast<uint16_t*>(a.C2);
            const int hcol = ci.t.n0 + wn * 64;
#pragma unroll
            for (int part = 0; part < 2; ++part) {
#pragma unroll
              for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                  const int c4 = jj * 8 + 2 * grp + (lane >> 5);
                  const f32x16_t& cc = acc[i][jj + 2 * part];
                  const int b = grp * 4;
                  *reinterpret_cast<uint2*>(stg + r * 128 + (((c4 >> 1) ^ ((r >> 1) & 7)) << 4) + (c4 & 1) * 8) =
                      pack4_bf16(acc_rd(cc[b]), acc_rd(cc[b + 1]), acc_rd(cc[b + 2]), acc_rd(cc[b + 3]));
                  __builtin_amdgcn_sched_barrier(0);
                }
              const int rl = lane >> 3, c = lane & 7;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int rr = q * 8 + rl;
                const uint4 v = *reinterpret_cast<const uint4*>(stg + rr * 128 + ((c ^ ((rr >> 1) & 7)) << 4));
                const int m = wm * 128 + i * 32 + rr;
                if (m < ci.t.rows && hcol < N)
                  *reinterpret_cast<uint4*>(C2 + static_cast<int64_t>(ci.t.r0 + m) * (2 * N) + part * N + hcol + c * 8) = v;
              }
            }
          }
        }
      }
    }

    cidx = next_item(cidx + 1, ci);
    if (cidx < 0) break;
    ckc = ci.k0;
    zero_acc();
    spar ^= 1;
    load_srows(ci.t);
  }
  wait_vmcnt0();                       // the last stages' DMAs landed before the workgroup ends
}

// Finish the K-split remainder tiles: sum each tile's partial slots in piece
// order, apply the epilogue (swiglu: silu(gate) * up) and store bf16 rows.
template <bool MX, bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(GemmArgs a) {
  constexpr int NOUT = SWIGLU ? BN / 2 : BN;
  const int NT = (a.N + NOUT - 1) / NOUT;
  const int total = a.prefix[a.E] * NT;
  const Split sp = split_work(total, a.grid, a.K / stage_k<MX>(), a.max_pieces);
  if (sp.ways < 2) return;
  constexpr int CPR = NOUT / 8;                  // 8-column groups per output row
  const int64_t work = static_cast<int64_t>(sp.rem) * BM * CPR;
  uint16_t* C = static_cast<uint16_t*>(a.C);
  for (int64_t idx = blockIdx.x * 256LL + threadIdx.x; idx < work; idx += gridDim.x * 256LL) {
    const int q = static_cast<int>(idx / (BM * CPR));
    const int row = static_cast<int>(idx / CPR % BM);
    const int c8 = static_cast<int>(idx % CPR);
    Tile t;
    if (!decode_tile(sp.full + q, NT, NOUT, a.E, a.prefix, a.offsets, a.M, t)) continue;
    if (row >= t.rows || t.n0 + c8 * 8 >= a.N) continue;
    float v[8], up[8];             // swiglu: v = gate sums; down: the outputs
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = up[u] = 0.f;
    for (int p = 0; p < sp.ways; ++p) {
      const float* P = a.partials + static_cast<int64_t>(q * sp.ways + p) * (BM * BN) + row * BN;
      const float4 x0 = *reinterpret_cast<const float4*>(P + c8 * 8);
      const float4 x1 = *reinterpret_cast<const float4*>(P + c8 * 8 + 4);
      v[0] += x0.x; v[1] += x0.y; v[2] += x0.z; v[3] += x0.w;
      v[4] += x1.x; v[5] += x1.y; v[6] += x1.z; v[7] += x1.w;
      if constexpr (SWIGLU) {
        const float4 u0 = *reinterpret_cast<const float4*>(P + 128 + c8 * 8);
        const float4 u1 = *reinterpret_cast<const float4*>(P + 128 + c8 * 8 + 4);
        up[0] += u0.x; up[1] += u0.y; up[2] += u0.z; up[3] += u0.w;
        up[4] += u1.x; up[5] += u1.y; up[6] += u1.z; up[7] += u1.w;
      }
    }
    if constexpr (SWIGLU) {
      if (a.C2) {            // the gate and up sums too (bf16), into C2 [M, 2I]
        uint16_t* C2 = static_cast<uint16_t*>(a.C2) + (t.r0 + row) * (2LL * a.N) + t.n0 + c8 * 8;
        uint4 g4, u4;
        uint2 lo = pack4_bf16(v[0], v[1], v[2], v[3]), hi = pack4_bf16(v[4], v[5], v[6], v[7]);
        g4.x = lo.x; g4.y = lo.y; g4.z = hi.x; g4.w = hi.y;
        lo = pack4_bf16(up[0], up[1], up[2], up[3]);
        hi = pack4_bf16(up[4], up[5], up[6], up[7]);
        u4.x = lo.x; u4.y = lo.y; u4.z = hi.x; u4.w = hi.y;
        *reinterpret_cast<uint4*>(C2) = g4;
        *reinterpret_cast<uint4*>(C2 + a.N) = u4;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = silu_f(v[u]) * up[u];
    }
    uint4 o;
    const uint2 lo = pack4_bf16(v[0], v[1], v[2], v[3]);
    const uint2 hi = pack4_bf16(v[4], v[5], v[6], v[7]);
    o.x = lo.x; o.y = lo.y; o.z = hi.x; o.w = hi.y;
    const int64_t crow = a.scatter ? a.scatter[t.r0 + row] : t.r0 + row;
    *reinterpret_cast<uint4*>(C + crow * a.N + t.n0 + c8 * 8) = o;
  }
}

// MX SwiGLU: finish the K-split remainder tiles of the gate/up GEMM.  One
// thread per (tile, row, 32-column block): the gate and up sums of the block
// added in piece order, h = silu(g) * u quantized to MXFP8 as in the main
// kernel's epilogue (32 codes and one scale byte).
__global__ __launch_bounds__(256) void gemm_mx_swiglu_fixup_kernel(GemmArgs a) {
  constexpr int NOUT = BN / 2;
  const int NT = (a.N + NOUT - 1) / NOUT;
  const int total = a.prefix[a.E] * NT;
  const Split sp = split_work(total, a.grid, a.K / stage_k<true>(), a.max_pieces);
  if (sp.ways < 2) return;
  constexpr int BPR = NOUT / 32;                 // 32-column blocks per output row
  const int64_t work = static_cast<int64_t>(sp.rem) * BM * BPR;
  uint8_t* C = static_cast<uint8_t*>(a.C);
  for (int64_t idx = blockIdx.x * 256LL + threadIdx.x; idx < work; idx += gridDim.x * 256LL) {
    const int q = static_cast<int>(idx / (BM * BPR));
    const int row = static_cast<int>(idx / BPR % BM);
    const int blk = static_cast<int>(idx % BPR);
    Tile t;
    if (!decode_tile(sp.full + q, NT, NOUT, a.E, a.prefix, a.offsets, a.M, t)) continue;
    const int col = t.n0 + blk * 32;
    if (row >= t.rows || col >= a.N) continue;
    float g[32], u[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) g[c] = u[c] = 0.f;
    for (int p = 0; p < sp.ways; ++p) {
      const float* P = a.partials + static_cast<int64_t>(q * sp.ways + p) * (BM * BN) + row * BN + blk * 32;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 x = *reinterpret_cast<const float4*>(P + 4 * c);
        const float4 y = *reinterpret_cast<const float4*>(P + 128 + 4 * c);
        g[4 * c] += x.x; g[4 * c + 1] += x.y; g[4 * c + 2] += x.z; g[4 * c + 3] += x.w;
        u[4 * c] += y.x; u[4 * c + 1] += y.y; u[4 * c + 2] += y.z; u[4 * c + 3] += y.w;
      }
    }
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      g[c] = silu_f(g[c]) * u[c];
      m = __builtin_fmaxf(m, __builtin_fabsf(g[c]));
    }
    const int ex = mx_block_exp(m);
    const float sc = mx_inv_scale(ex);
    uint32_t w[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) w[c] = mx_encode4(g[4 * c], g[4 * c + 1], g[4 * c + 2], g[4 * c + 3], sc);
    const int64_t crow = t.r0 + row;
    uint4* dst = reinterpret_cast<uint4*>(C + crow * a.N + col);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    a.c_scale[(static_cast<int64_t>(col / 128) * a.c_srows + crow) * 4 + (col / 32) % 4] =
        static_cast<uint8_t>(ex + 127);
  }
}

template <bool MX, bool SWIGLU, bool GATHER, bool WG = false, bool SAVE = false, bool BT = false>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<MX, SWIGLU, GATHER, WG, SAVE, BT>), dim3(a.grid), dim3(256), 0, s, a);
  if constexpr (WG) return hipGetLastError();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_pieces < 2 || a.K / stage_k<MX>() < 2 * kMinPiece) return e;
  if constexpr (MX && SWIGLU)
    hipLaunchKernelGGL(gemm_mx_swiglu_fixup_kernel, dim3(512), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_fixup_kernel<MX, SWIGLU>), dim3(512), dim3(256), 0, s, a);
  return hipGetLastError();
}

// entry / d for entries in [0, 2^31): d = 2^l is a shift; otherwise, with
// l = ceil(log2 d) and m = floor(2^(31+l) / d) + 1 < 2^32, the quotient is
// floor(entry * m / 2^(31+l)): the excess entry * (m d - 2^(31+l)) / (d 2^(31+l))
// is below 2^-l < 1/d, too small to carry past the next integer.
void set_gather_magic(GemmArgs& a) {
  const uint32_t d = static_cast<uint32_t>(a.gather_div);
  if ((d & (d - 1)) == 0) {
    a.gather_magic = 0;
    a.gather_shift = __builtin_ctz(d);
  } else {
    const int l = 32 - __builtin_clz(d - 1);
    a.gather_magic = static_cast<uint32_t>((uint64_t{1} << (31 + l)) / d + 1);
    a.gather_shift = l - 1;
  }
}

}  // namespace

int gemm_pieces(int64_t M, int H, int I, int E, bool mx) {
  // a K split never makes more pieces than tiles x (K stages / kMinPiece) of
  // either GEMM, and none when a tile cannot be cut in two
  const int64_t mt = (M + BM - 1) / BM + E;           // m-tiles, upper bound
  const int ks = mx ? stage_k<true>() : stage_k<false>();
  auto most = [&](int64_t nt, int nk) -> int64_t {
    const int w = nk / kMinPiece;
    return w >= 2 ? mt * nt * w : 0;
  };
  const int64_t up = most((I + BN / 2 - 1) / (BN / 2), H / ks);
  const int64_t down = most((H + BN - 1) / BN, I / ks);
  const int64_t m = up > down ? up : down;
  return static_cast<int>(m < kGemmPieces ? m : kGemmPieces);
}

bool gemm_gather_fits(int64_t a_rows, int K, int elem_bytes) {
  return static_cast<uint64_t>(a_rows) * static_cast<uint64_t>(K) * elem_bytes <= (uint64_t{1} << 32);
}

hipError_t launch_gemm_bf16_swiglu(const GemmArgs& a0, hipStream_t s) {
  if (!a0.gather)
    return a0.C2 ? launch<false, true, false, false, true>(a0, s) : launch<false, true, false>(a0, s);
  if (a0.gather_div < 1 || !gemm_gather_fits(a0.a_rows, a0.K, 2)) return hipErrorInvalidValue;
  GemmArgs a = a0;
  set_gather_magic(a);
  return a.C2 ? launch<false, true, true, false, true>(a, s) : launch<false, true, true>(a, s);
}

hipError_t launch_gemm_bf16_down(const GemmArgs& a, hipStream_t s) {
  return launch<false, false, false>(a, s);
}

hipError_t launch_gemm_bf16_plain(const GemmArgs& a0, hipStream_t s) {
  if (!a0.gather) return launch<false, false, false>(a0, s);
  if (a0.gather_div < 1 || !gemm_gather_fits(a0.a_rows, a0.K, 2)) return hipErrorInvalidValue;
  GemmArgs a = a0;
  set_gather_magic(a);
  return launch<false, false, true>(a, s);
}

hipError_t launch_gemm_bf16_bt(const GemmArgs& a0, hipStream_t s) {
  if (a0.N % 64 || a0.K % BK) return hipErrorInvalidValue;
  if (!a0.gather) return launch<false, false, false, false, false, true>(a0, s);
  if (a0.gather_div < 1 || !gemm_gather_fits(a0.a_rows, a0.K, 2)) return hipErrorInvalidValue;
  GemmArgs a = a0;
  set_gather_magic(a);
  return launch<false, false, true, false, false, true>(a, s);
}

hipError_t launch_gemm_bf16_wgrad(const GemmArgs& a0, hipStream_t s) {
  if (!a0.koff || !a0.Cf || a0.ld <= 0 || a0.ld % BK || a0.group_rows <= 0 || a0.N % 64 ||
      a0.ld * 2 * BM > (int64_t{1} << 32))
    return hipErrorInvalidValue;
  GemmArgs a = a0;
  a.K = BK;              // the K loop is per group; no tile is cut along K
  a.max_pieces = 0;
  a.gather = nullptr;
  a.scatter = nullptr;
  return launch<false, false, false, true>(a, s);
}

hipError_t launch_gemm_mx_swiglu(const GemmArgs& a0, hipStream_t s) {
  if (!a0.a_scale || !a0.b_scale || !a0.c_scale || a0.K % stage_k<true>() || a0.N % (BN / 2) ||
      a0.a_srows < a0.M || a0.b_srows < static_cast<int64_t>(a0.E) * 2 * a0.I || a0.c_srows < a0.M)
    return hipErrorInvalidValue;
  if (!a0.gather) return launch<true, true, false>(a0, s);
  if (a0.gather_div < 1 || !gemm_gather_fits(a0.a_rows, a0.K, 1)) return hipErrorInvalidValue;
  GemmArgs a = a0;
  set_gather_magic(a);
  return launch<true, true, true>(a, s);
}

hipError_t launch_gemm_mx_down(const GemmArgs& a, hipStream_t s) {
  if (!a.a_scale || !a.b_scale || a.K % stage_k<true>() || a.a_srows < a.M ||
      a.b_srows < static_cast<int64_t>(a.E) * a.N)
    return hipErrorInvalidValue;
  return launch<true, false, false>(a, s);
}

}  // namespace moe
