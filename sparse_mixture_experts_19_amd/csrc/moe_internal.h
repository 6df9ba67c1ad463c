// Internal declarations shared by the HIP translation units of libmoe_mi355x.
// Nothing here is part of the public C ABI (include/moe_mi355x.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace moe {

// ---------------------------------------------------------------- constants
constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kMaxE = 256;             // experts supported
constexpr int kMaxK = 8;               // top-k supported
constexpr int kRouteTok = 32;          // tokens per router workgroup
constexpr int kPermChunk = 1024;       // assignments per permutation workgroup
constexpr int kGemmBM = 256;           // MFMA grouped GEMMs: rows per tile
constexpr int kGemmBN = 256;           // MFMA grouped GEMMs: weight rows per tile
constexpr int kGemmBK = 64;            // bf16 grouped GEMM: K per LDS stage (MXFP8: 128)
constexpr int kGemmPieces = 256;       // MFMA grouped GEMMs: most K-split partial tiles
constexpr int kMxBlock = 32;           // MXFP8: values per E8M0 scale
constexpr int kF32BM = 64;             // fp32 grouped GEMM tile
constexpr int kF32BN = 32;
constexpr int kF32BK = 16;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------ router (route.hip)
struct RouteArgs {
  const void* x;          // [T,H]
  const void* w;          // [E,H]
  const float* bias;      // [E] or null
  int64_t T;
  int H, E, k, renorm;
  int32_t* ids;           // [T,k]
  float* weights;         // [T,k]
  int32_t* flag;          // [T]     fp32 path: 1 = needs the float64 re-rank
  float* meta;            // [T,4]   softmax max and sum, band, k-th logit
  float* logits;          // [T,E]   fp32 logits with bias (fp32 path: of flagged tokens;
                          //         every token's when keep_all)
  int keep_all;           // 1: meta and total logits are written for every token
};
size_t route_scratch_bytes(int64_t T, int H, int E, bool bf16);
hipError_t launch_route(const RouteArgs& a, bool bf16, hipStream_t s);

// ------------------------------------------------- permutation (permute.hip)
struct PermuteArgs {
  const int32_t* ids;     // [M] flat topk ids
  int64_t M;
  int E, k;
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E+1]
  int32_t* perm;          // [M]
  int32_t* inv;           // [M]
  int32_t* block_hist;    // [nblocks, E] scratch
  int32_t* tile_prefix;   // [E+1] or NULL: m-tiles of tile_bm rows per expert, exclusive prefix
  int tile_bm;
};
// chunks x experts up to which each scatter workgroup sums the chunk
// histograms itself (no separate scan pass)
constexpr int64_t kPermInlineScan = 32768;
size_t permute_scratch_bytes(int64_t M, int E);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// Allocation-free permutation: int32 entries of the library's own device
// array for the chunk histograms (4 MiB per GPU), and its address on
// `device`, which must be the current device (looked up once per device).
constexpr size_t kPermStaticScratchInts = size_t(1) << 20;
hipError_t permute_static_scratch(int device, int32_t** ptr);
// x_perm[inv[t*k + j]] = x[t]: T tokens of H elements of elem_bytes each.
hipError_t launch_gather_rows(const void* x, const int32_t* inv, int64_t T, int H, int k,
                              int elem_bytes, void* x_perm, hipStream_t s);

// offsets[0] = 0, offsets[1] = M: one dense group of M rows.
hipError_t launch_dense_offsets(int32_t* offsets, int64_t M, hipStream_t s);

// Tile schedule of the grouped GEMMs: prefix[e] = sum_{e'<e} ceil(count_e'/bm).
hipError_t launch_tile_schedule(const int32_t* offsets, int E, int bm, int64_t M,
                                int32_t* prefix, hipStream_t s);

// --------------------------------------------- grouped GEMMs (gemm_*.hip)
struct GemmArgs {
  const void* A;          // rows: [*,K] (x, x_perm or h; MXFP8: e4m3 codes)
  const int32_t* gather;  // null: row r of A is r; else row r is gather[r] / gather_div
  int gather_div;
  uint32_t gather_magic;  // MFMA kernels: entry / gather_div == umulhi(entry, magic) >> shift
  int gather_shift;       // (magic 0: entry >> shift); set by the launcher
  int64_t a_rows;         // rows of A (gathered row indices are clamped to it)
  int64_t M;              // rows of C (tile rows are clamped to it)
  const void* B;          // stacked weights, expert stride b_stride elements
  int64_t b_stride;
  void* C;                // [M, N]
  int N, K;               // output columns, reduction length
  int I;                  // SwiGLU: rows of the gate block (up rows follow)
  int E;
  const int32_t* offsets; // [E+1]
  const int32_t* prefix;  // [E+1] tile prefix for this kernel's BM
  int grid;               // persistent workgroups launched (bf16: a multiple of 8)
  float* partials;        // bf16: fp32 partial sums of K-split tiles, max_pieces x BM x BN
  int max_pieces;         // capacity of partials in tiles (0: tiles are never split)
  const int32_t* scatter; // null: row r of C is row r; else row r is written to row scatter[r]
  // MXFP8 kernels: E8M0 scales (biased exponents), one byte per 32 values of
  // a row, as stage-major 32-bit words: word s of row r (the scales of K
  // blocks 4s .. 4s+3) at word index s * rows + r, so that the words of one
  // 128-wide K stage of consecutive rows are contiguous
  const uint8_t* a_scale; // rows as the GEMM's own rows (r0 + i; never gathered)
  const uint8_t* b_scale; // rows e * (rows of an expert) + n
  uint8_t* c_scale;       // SwiGLU: scales of h, rows as C (h itself: e4m3 codes in C)
  int64_t a_srows, b_srows, c_srows;   // rows of the three word arrays
  // Weight-gradient form (launch_gemm_bf16_wgrad): group g owns output rows
  // [g*group_rows, (g+1)*group_rows) and reduces over the K range
  // [koff[g], koff[g+1]) (multiples of 64) of A and B, whose rows have pitch ld
  // elements; fp32 results go to Cf [E*group_rows, N].
  // bf16 SwiGLU: also the gate and up sums, rounded to bf16, into C2
  // [M, 2I] (row r: I gate values, then I up values), or null
  void* C2;
  const int32_t* koff;    // [E+1] device
  int64_t ld;
  int64_t group_rows;
  float* Cf;
};
// Partial-sum slots the MFMA GEMMs (mx: MXFP8) of an [M rows, H, I, E]
// expert MLP can use.
int gemm_pieces(int64_t M, int H, int I, int E, bool mx);
// The gathered form (gather != null) needs A to span at most 2^32 bytes.
bool gemm_gather_fits(int64_t a_rows, int K, int elem_bytes);
hipError_t launch_gemm_bf16_swiglu(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_bf16_down(const GemmArgs& a, hipStream_t s);
// The down kernel's plain product C = A B^T with A rows gathered (gather != null).
hipError_t launch_gemm_bf16_plain(const GemmArgs& a, hipStream_t s);
// Plain product C = A B_e per expert e with B N-major ([E, K, N]: B_e is
// [K, N], the expert weights as stored, read for W^T products without a
// transposed copy); gathered A rows when gather is set, scattered C rows when
// scatter is set.  N % 64 == 0 and K % 64 == 0.
hipError_t launch_gemm_bf16_bt(const GemmArgs& a, hipStream_t s);
// Weight gradients: per group g, Cf rows of g = A[rows of g] B^T over K range g.
hipError_t launch_gemm_bf16_wgrad(const GemmArgs& a, hipStream_t s);
// MXFP8 operands: K a multiple of 128; SwiGLU: N (= I) a multiple of 128;
// the down GEMM writes bf16 rows.
hipError_t launch_gemm_mx_swiglu(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_mx_down(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_f32_swiglu(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_f32_down(const GemmArgs& a, hipStream_t s);

// --------------------------------------------------- token rounding (round.hip)
struct RoundArgs {
  int32_t* ids;           // [T,k] in: routed ids; out: rounded ids
  float* weights;         // [T,k] out: weights of tokens whose experts changed
  const float* logits;    // [T,E] fp32 total logits (bias included) of every token
  const float* meta;      // [T,4] softmax max and sum of every token
  const int32_t* counts;  // [E]   of the routed ids
  const int32_t* offsets; // [E+1]
  const int32_t* inv;     // [T*k] inverse of the routed ids' stable permutation
  int64_t T;
  int E, k, B, renorm;
  uint8_t* mask;          // [T] scratch: pooled slots of each token
  uint64_t* packed;       // [T] scratch: the token's ids, one byte per slot
  int32_t* pool_tok;      // [T] scratch: tokens with a pooled slot, in order
  uint64_t* gsid;         // [T] scratch: hand-out state when it does not fit in LDS
  uint8_t* gmask;         // [T]
};
size_t round_scratch_bytes(int64_t T);
// Carves the scratch arrays of `a` from `base` (round_scratch_bytes(T) bytes).
void carve_round(char* base, RoundArgs& a);
hipError_t launch_token_round(const RoundArgs& a, hipStream_t s);

// ------------------------------------------------------ MXFP8 (mxfp8.hip)
// rows x cols values (bf16 or fp32, cols a multiple of 32) -> e4m3 codes
// [rows, cols] and E8M0 scales [rows, cols/32].
hipError_t launch_mx_quantize(const void* src, bool bf16, int64_t rows, int cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);
// Stage-major scale words (see GemmArgs) of R rows from row-major E8M0 scales
// [*, K/32] (K a multiple of 128): dst[s * R + r] = word s of source row r,
// or of source row rows[r] / div when rows is given (a gathered copy).
hipError_t launch_mx_scale_words(const uint8_t* scales, int64_t R, int K, const int32_t* rows, int div,
                                 uint32_t* dst, hipStream_t s);

// ------------------------------------------------------ backward (backward.hip)
hipError_t launch_bwd_dw(const void* dout, const void* y, int64_t T, int H, int k, float* dw,
                         hipStream_t s);
hipError_t launch_bwd_router(const float* logits, const float* meta, const int32_t* ids,
                             const float* dw, int64_t T, int E, int k, int renorm, float* dl,
                             hipStream_t s);
// Token slices of the dW_r reduction (partials: slices x E x H fp32).
int bwd_dwr_slices(int64_t T);
// dxr = dl W_r (bf16), dwr = dl^T x (fp32), db = column sums of dl (null: skipped).
hipError_t launch_bwd_router_grads(const float* dl, const void* x, const void* w_router, int64_t T,
                                   int H, int E, void* dxr, float* dwr, float* db, float* part,
                                   hipStream_t s);
// poff [E+1] padded expert segments; goff/pre [E+1] row offsets and tile
// prefixes of the two weight-gradient GEMMs (H and 2I rows per expert).
hipError_t launch_bwd_tables(const int32_t* counts, int E, int H, int I, int32_t* poff,
                             int32_t* goff_h, int32_t* pre_h, int32_t* goff_i, int32_t* pre_i,
                             hipStream_t s);
hipError_t launch_gather_transpose(const void* src, int C, const int32_t* perm, bool gather, int k,
                                   const float* scale, const int32_t* offsets, const int32_t* counts,
                                   const int32_t* poff, int E, int64_t ld, void* dst, hipStream_t s);
hipError_t launch_bwd_swiglu(const void* dh, const void* gu, const float* wts, const int32_t* perm,
                             int64_t M, int I, void* dgdu, void* h, hipStream_t s);
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s);

// ------------------------------------------------------ combine (combine.hip)
// inv != null: slot (t, j) is row inv[t*k+j] of y; inv == null: row t*k+j.
hipError_t launch_combine(const void* y, const int32_t* inv, const float* w, int64_t T, int H,
                          int k, bool bf16, void* out, hipStream_t s, const void* ys = nullptr);

// ------------------------------------------------------------ device query
int device_cu_count();

}  // namespace moe
