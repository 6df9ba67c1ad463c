// Host side of libmoe_mi355x: argument validation, workspace carving, launch
// sequencing on the caller's stream.  The ABI is declared, with the meaning
// of every argument, in include/moe_mi355x.h.
#include "moe_mi355x.h"
#include "moe_internal.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

// ---------------------------------------------------------------- devices
struct DevInfo {
  int state;   // 0 unknown, 1 gfx950, 2 other
  int cu;
};
constexpr int kMaxDev = 64;
std::mutex g_dev_mu;
DevInfo g_dev[kMaxDev];

int current_device(int* dev_out, int* cu_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev)
    return fail(MOE_ERR_UNSUPPORTED, "no usable HIP device (%s)", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& d = g_dev[dev];
  if (d.state == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    d.state = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    d.cu = p.multiProcessorCount;
  }
  if (d.state != 1) return fail(MOE_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X)", dev);
  if (dev_out) *dev_out = dev;
  if (cu_out) *cu_out = d.cu;
  return MOE_OK;
}

// ------------------------------------------------------------- validation
bool misaligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

int elem_bytes(int dtype) { return dtype == MOE_DTYPE_BF16 ? 2 : 4; }

int check_sizes(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t dtype, bool need_I) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
  if (H <= 0) return fail(MOE_ERR_INVALID_ARG, "H must be > 0 (got %d)", H);
  if (need_I && I <= 0) return fail(MOE_ERR_INVALID_ARG, "I must be > 0 (got %d)", I);
  if (E <= 0) return fail(MOE_ERR_INVALID_ARG, "E must be > 0 (got %d)", E);
  if (k <= 0) return fail(MOE_ERR_INVALID_ARG, "k must be > 0 (got %d)", k);
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "k (%d) must not exceed E (%d)", k, E);
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (E > moe::kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E (%d) > %d", E, moe::kMaxE);
  if (k > moe::kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k (%d) > %d", k, moe::kMaxK);
  if (H % 64) return fail(MOE_ERR_UNSUPPORTED, "H (%d) must be a multiple of 64", H);
  if (H > 16384) return fail(MOE_ERR_UNSUPPORTED, "H (%d) > 16384", H);
  if (need_I && I % 64) return fail(MOE_ERR_UNSUPPORTED, "I (%d) must be a multiple of 64", I);
  if (need_I && I > 65536) return fail(MOE_ERR_UNSUPPORTED, "I (%d) > 65536", I);
  if (T * static_cast<int64_t>(k) > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "T*k (%lld) exceeds 2^31-1", (long long)(T * k));
  if (need_I) {
    // the persistent GEMM numbers its tiles with 32-bit ints
    const int64_t M = T * k;
    const int64_t bm = dtype == MOE_DTYPE_BF16 ? moe::kGemmBM : moe::kF32BM;
    const int64_t nt1 = dtype == MOE_DTYPE_BF16 ? (I + 127) / 128 : (I + 63) / 64;
    const int64_t nt2 = dtype == MOE_DTYPE_BF16 ? (H + 255) / 256 : (H + 63) / 64;
    const int64_t tiles = ((M + bm - 1) / bm + E) * (nt1 > nt2 ? nt1 : nt2);
    if (tiles > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "problem too large for the tile schedule");
  }
  return MOE_OK;
}

#define MOE_CHECK(expr)              \
  do {                               \
    const int _st = (expr);          \
    if (_st != MOE_OK) return _st;   \
  } while (0)

#define MOE_HIP(expr)                                                              \
  do {                                                                             \
    const hipError_t _e = (expr);                                                  \
    if (_e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", #expr, hipGetErrorString(_e)); \
  } while (0)

int need_ptr(const void* p, const char* name, size_t align) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
  if (misaligned(p, align)) return fail(MOE_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return MOE_OK;
}

// ------------------------------------------------------------ workspaces
// Grouped-GEMM scratch: the tile prefix, then (bf16) the fp32 partial sums
// of K-split tiles.
size_t gemm_prefix_bytes(int E) { return moe::align_up(static_cast<size_t>(E + 1) * 4, 256); }
size_t gemm_scratch(int64_t M, int H, int I, int E, int dtype) {
  size_t b = gemm_prefix_bytes(E);
  if (dtype == MOE_DTYPE_BF16)
    b += static_cast<size_t>(moe::gemm_pieces(M, H, I, E, false)) * moe::kGemmBM * moe::kGemmBN * 4;
  return b;
}

struct Carver {
  size_t o = 0;
  size_t take(size_t bytes) {
    const size_t at = o;
    o = moe::align_up(o + bytes, 256);
    return at;
  }
};

moe_forward_layout forward_layout(int64_t T, int H, int I, int E, int k, int dtype) {
  const size_t M = static_cast<size_t>(T) * k;
  const size_t eb = elem_bytes(dtype);
  Carver c;
  moe_forward_layout L;
  L.topk_ids = c.take(M * 4);
  L.topk_weights = c.take(M * 4);
  L.expert_counts = c.take(static_cast<size_t>(E) * 4);
  L.expert_offsets = c.take(static_cast<size_t>(E + 1) * 4);
  L.perm = c.take(M * 4);
  L.inv_perm = c.take(M * 4);
  L.h = c.take(M * I * eb);
  L.y = c.take(M * H * eb);
  const size_t rs = moe::route_scratch_bytes(T, H, E, dtype == MOE_DTYPE_BF16);
  const size_t shared_sz = rs > moe::permute_scratch_bytes(M, E) ? rs : moe::permute_scratch_bytes(M, E);
  L.scratch = c.take(gemm_scratch(static_cast<int64_t>(M), H, I, E, dtype) + shared_sz);
  L.total = c.o;
  return L;
}

// The moe_forward layout, then the shared expert's h [T,Is], output [T,H]
// and its own GEMM scratch: dense offsets {0, T} (256 bytes), then the tile
// prefix and partial sums of a one-group grouped GEMM.
moe_shared_layout shared_layout(int64_t T, int H, int I, int Is, int E, int k, int dtype) {
  moe_shared_layout S;
  S.routed = forward_layout(T, H, I, E, k, dtype);
  const size_t eb = elem_bytes(dtype);
  Carver c;
  c.o = S.routed.total;
  S.h_shared = c.take(static_cast<size_t>(T) * Is * eb);
  S.y_shared = c.take(static_cast<size_t>(T) * H * eb);
  S.scratch = c.take(256 + gemm_scratch(T, H, Is, 1, dtype));
  S.total = c.o;
  return S;
}

// The moe_forward layout with a scratch region that holds the router's,
// the permutation's and the token rounding's scratch side by side: the
// rounding reads the router's logits after the first permutation ran.
moe_forward_layout rounded_layout(int64_t T, int H, int I, int E, int k, int dtype) {
  moe_forward_layout L = forward_layout(T, H, I, E, k, dtype);
  const int64_t M = T * k;
  Carver c;
  c.o = L.scratch;
  c.take(gemm_scratch(M, H, I, E, dtype));
  c.take(moe::route_scratch_bytes(T, H, E, dtype == MOE_DTYPE_BF16));
  c.take(moe::permute_scratch_bytes(M, E));
  c.take(moe::round_scratch_bytes(T));
  L.total = c.o;
  return L;
}

// Router scratch carved from `base`; returns the bytes used.
size_t carve_route(char* base, int64_t T, int E, moe::RouteArgs& a) {
  Carver c;
  a.flag = reinterpret_cast<int32_t*>(base + c.take(static_cast<size_t>(T) * 4));
  a.meta = reinterpret_cast<float*>(base + c.take(static_cast<size_t>(T) * 16));
  a.logits = reinterpret_cast<float*>(base + c.take(static_cast<size_t>(T) * E * 4));
  return c.o;
}

int run_route(const void* x, const void* w_router, const float* bias, int64_t T, int H, int E,
              int k, int dtype, int renorm, int32_t* ids, float* weights, char* scratch,
              hipStream_t s, moe::RouteArgs* out_args = nullptr) {
  moe::RouteArgs a{};
  a.x = x; a.w = w_router; a.bias = bias; a.T = T; a.H = H; a.E = E; a.k = k; a.renorm = renorm;
  a.ids = ids; a.weights = weights; a.keep_all = out_args != nullptr;
  const bool bf16 = dtype == MOE_DTYPE_BF16;
  if (carve_route(scratch, T, E, a) > moe::route_scratch_bytes(T, H, E, bf16))
    return fail(MOE_ERR_WORKSPACE, "internal: router scratch layout exceeds its size");
  MOE_HIP(moe::launch_route(a, bf16, s));
  if (out_args) *out_args = a;
  return MOE_OK;
}

// tile_prefix (optional): also write the grouped GEMM's m-tile prefix for
// tiles of tile_bm rows (the permutation's last pass does it in passing).
int run_permute(const int32_t* ids, int64_t M, int E, int k, int32_t* counts, int32_t* offsets,
                int32_t* perm, int32_t* inv, char* scratch, hipStream_t s,
                int32_t* tile_prefix = nullptr, int tile_bm = 0) {
  moe::PermuteArgs a{};
  a.ids = ids; a.M = M; a.E = E; a.k = k; a.counts = counts; a.offsets = offsets;
  a.perm = perm; a.inv = inv; a.block_hist = reinterpret_cast<int32_t*>(scratch);
  a.tile_prefix = tile_prefix; a.tile_bm = tile_bm;
  MOE_HIP(moe::launch_permute(a, s));
  return MOE_OK;
}

int run_experts(const void* a_ptr, int64_t a_rows, const int32_t* gather, int gather_div,
                const int32_t* offsets, const void* w13, const void* w2, int64_t M, int H, int I,
                int E, int dtype, void* h, void* y, int32_t* prefix, int cu, hipStream_t s) {
  const bool bf16 = dtype == MOE_DTYPE_BF16;
  MOE_HIP(moe::launch_tile_schedule(offsets, E, bf16 ? moe::kGemmBM : moe::kF32BM, M, prefix, s));
  moe::GemmArgs g{};
  g.E = E; g.offsets = offsets; g.prefix = prefix; g.I = I; g.M = M; g.a_rows = a_rows;
  if (bf16) {
    g.partials = reinterpret_cast<float*>(reinterpret_cast<char*>(prefix) + gemm_prefix_bytes(E));
    g.max_pieces = moe::gemm_pieces(M, H, I, E, false);
    g.grid = cu >= 8 ? cu / 8 * 8 : 8;
  } else {
    g.grid = cu * 2;
  }
  // gate/up + SwiGLU
  g.A = a_ptr; g.gather = gather; g.gather_div = gather_div;
  g.B = w13; g.b_stride = static_cast<int64_t>(2) * I * H;
  g.C = h; g.N = I; g.K = H;
  MOE_HIP(bf16 ? moe::launch_gemm_bf16_swiglu(g, s) : moe::launch_gemm_f32_swiglu(g, s));
  // down
  g.A = h; g.gather = nullptr; g.gather_div = 1; g.a_rows = M;
  g.B = w2; g.b_stride = static_cast<int64_t>(H) * I;
  g.C = y; g.N = H; g.K = I;
  MOE_HIP(bf16 ? moe::launch_gemm_bf16_down(g, s) : moe::launch_gemm_f32_down(g, s));
  return MOE_OK;
}

}  // namespace

namespace moe {
int device_cu_count() {
  int cu = 0;
  if (current_device(nullptr, &cu) != MOE_OK || cu <= 0) return 256;
  return cu;
}
}  // namespace moe

extern "C" {

int moe_version(void) { return 106; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err; }

int moe_workspace_size(int32_t entry, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                       int32_t dtype, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  switch (entry) {
    case MOE_ENTRY_ROUTE:
      MOE_CHECK(check_sizes(T, H, 64, E, k, dtype, false));
      *bytes = moe::route_scratch_bytes(T, H, E, dtype == MOE_DTYPE_BF16);
      return ok();
    case MOE_ENTRY_PERMUTE:
      MOE_CHECK(check_sizes(T, H, 64, E, k, dtype, false));
      *bytes = moe::permute_scratch_bytes(T * k, E);
      return ok();
    case MOE_ENTRY_GROUPED_GEMM:
      MOE_CHECK(check_sizes(T, H, I, E, 1, dtype, true));
      *bytes = gemm_scratch(T, H, I, E, dtype);
      return ok();
    case MOE_ENTRY_COMBINE:
      MOE_CHECK(check_sizes(T, H, 64, k, k, dtype, false));
      *bytes = 0;
      return ok();
    case MOE_ENTRY_FORWARD:
      MOE_CHECK(check_sizes(T, H, I, E, k, dtype, true));
      *bytes = forward_layout(T, H, I, E, k, dtype).total;
      return ok();
    default:
      return fail(MOE_ERR_INVALID_ARG, "unknown entry %d", entry);
  }
}

int moe_forward_workspace_layout(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                 int32_t dtype, moe_forward_layout* layout) {
  if (!layout) return fail(MOE_ERR_INVALID_ARG, "layout is NULL");
  MOE_CHECK(check_sizes(T, H, I, E, k, dtype, true));
  *layout = forward_layout(T, H, I, E, k, dtype);
  return ok();
}

int moe_route(const void* x, const void* w_router, const float* router_bias, int64_t T, int32_t H,
              int32_t E, int32_t k, int32_t dtype, int32_t renormalize, int32_t* topk_ids,
              float* topk_weights, void* workspace, size_t workspace_bytes, void* stream) {
  MOE_CHECK(check_sizes(T, H, 64, E, k, dtype, false));
  if (T == 0) return ok();
  MOE_CHECK(need_ptr(x, "x", 16));
  MOE_CHECK(need_ptr(w_router, "w_router", 16));
  if (router_bias) MOE_CHECK(need_ptr(router_bias, "router_bias", 4));
  MOE_CHECK(need_ptr(topk_ids, "topk_ids", 4));
  MOE_CHECK(need_ptr(topk_weights, "topk_weights", 4));
  const size_t need = moe::route_scratch_bytes(T, H, E, dtype == MOE_DTYPE_BF16);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "route needs %zu workspace bytes, got %zu", need, workspace_bytes);
  MOE_CHECK(need_ptr(workspace, "workspace", 16));
  MOE_CHECK(current_device(nullptr, nullptr));
  MOE_CHECK(run_route(x, w_router, router_bias, T, H, E, k, dtype, renormalize, topk_ids,
                      topk_weights, static_cast<char*>(workspace), static_cast<hipStream_t>(stream)));
  return ok();
}

int moe_permute(const int32_t* topk_ids, const void* x, int64_t T, int32_t H, int32_t E, int32_t k,
                int32_t dtype, int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                int32_t* inv_perm, void* x_perm, void* workspace, size_t workspace_bytes,
                void* stream) {
  MOE_CHECK(check_sizes(T, H, 64, E, k, dtype, false));
  if ((x == nullptr) != (x_perm == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "x and x_perm must both be set or both be NULL");
  if (T == 0) return ok();
  MOE_CHECK(need_ptr(topk_ids, "topk_ids", 4));
  MOE_CHECK(need_ptr(expert_counts, "expert_counts", 4));
  MOE_CHECK(need_ptr(expert_offsets, "expert_offsets", 4));
  MOE_CHECK(need_ptr(perm, "perm", 4));
  MOE_CHECK(need_ptr(inv_perm, "inv_perm", 4));
  if (x) {
    MOE_CHECK(need_ptr(x, "x", 16));
    MOE_CHECK(need_ptr(x_perm, "x_perm", 16));
  }
  const int64_t M = T * k;
  const size_t need = moe::permute_scratch_bytes(M, E);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "permute needs %zu workspace bytes, got %zu", need, workspace_bytes);
  MOE_CHECK(need_ptr(workspace, "workspace", 16));
  MOE_CHECK(current_device(nullptr, nullptr));
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_CHECK(run_permute(topk_ids, M, E, k, expert_counts, expert_offsets, perm, inv_perm,
                        static_cast<char*>(workspace), s));
  if (x) MOE_HIP(moe::launch_gather_rows(x, inv_perm, T, H, k, elem_bytes(dtype), x_perm, s));
  return ok();
}

int moe_permute_static(const int32_t* topk_ids, const void* x, int64_t T, int32_t H, int32_t E,
                       int32_t k, int32_t dtype, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* perm, int32_t* inv_perm, void* x_perm, void* stream) {
  MOE_CHECK(check_sizes(T, H, 64, E, k, dtype, false));
  if ((x == nullptr) != (x_perm == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "x and x_perm must both be set or both be NULL");
  if (T == 0) return ok();
  MOE_CHECK(need_ptr(topk_ids, "topk_ids", 4));
  MOE_CHECK(need_ptr(expert_counts, "expert_counts", 4));
  MOE_CHECK(need_ptr(expert_offsets, "expert_offsets", 4));
  MOE_CHECK(need_ptr(perm, "perm", 4));
  MOE_CHECK(need_ptr(inv_perm, "inv_perm", 4));
  if (x) {
    MOE_CHECK(need_ptr(x, "x", 16));
    MOE_CHECK(need_ptr(x_perm, "x_perm", 16));
  }
  const int64_t M = T * k;
  const size_t need = moe::permute_scratch_bytes(M, E);
  if (need > moe::kPermStaticScratchInts * sizeof(int32_t))
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_permute_static: ceil(T*k/%d)*E = %zu histogram entries exceed the library's "
                "static scratch of %zu; use moe_permute with a workspace",
                moe::kPermChunk, need / sizeof(int32_t), moe::kPermStaticScratchInts);
  int dev = -1;
  MOE_CHECK(current_device(&dev, nullptr));
  int32_t* scratch = nullptr;
  MOE_HIP(moe::permute_static_scratch(dev, &scratch));
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_CHECK(run_permute(topk_ids, M, E, k, expert_counts, expert_offsets, perm, inv_perm,
                        reinterpret_cast<char*>(scratch), s));
  if (x) MOE_HIP(moe::launch_gather_rows(x, inv_perm, T, H, k, elem_bytes(dtype), x_perm, s));
  return ok();
}

int moe_grouped_swiglu_gemm(const void* x_perm, const int32_t* expert_offsets, const void* w13,
                            const void* w2, int64_t M, int32_t H, int32_t I, int32_t E,
                            int32_t dtype, void* h, void* y, void* workspace,
                            size_t workspace_bytes, void* stream) {
  MOE_CHECK(check_sizes(M, H, I, E, 1, dtype, true));
  if (M == 0) return ok();
  MOE_CHECK(need_ptr(x_perm, "x_perm", 16));
  MOE_CHECK(need_ptr(expert_offsets, "expert_offsets", 4));
  MOE_CHECK(need_ptr(w13, "w13", 16));
  MOE_CHECK(need_ptr(w2, "w2", 16));
  MOE_CHECK(need_ptr(h, "h", 16));
  MOE_CHECK(need_ptr(y, "y", 16));
  const size_t need = gemm_scratch(M, H, I, E, dtype);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "grouped gemm needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  MOE_CHECK(need_ptr(workspace, "workspace", 16));
  int cu = 0;
  MOE_CHECK(current_device(nullptr, &cu));
  MOE_CHECK(run_experts(x_perm, M, nullptr, 1, expert_offsets, w13, w2, M, H, I, E, dtype, h, y,
                        static_cast<int32_t*>(workspace), cu, static_cast<hipStream_t>(stream)));
  return ok();
}

int moe_combine(const void* y, const int32_t* inv_perm, const float* topk_weights, int64_t T,
                int32_t H, int32_t k, int32_t dtype, void* out, void* stream) {
  MOE_CHECK(check_sizes(T, H, 64, k, k, dtype, false));
  if (T == 0) return ok();
  MOE_CHECK(need_ptr(y, "y", 16));
  MOE_CHECK(need_ptr(inv_perm, "inv_perm", 4));
  MOE_CHECK(need_ptr(topk_weights, "topk_weights", 4));
  MOE_CHECK(need_ptr(out, "out", 16));
  MOE_CHECK(current_device(nullptr, nullptr));
  MOE_HIP(moe::launch_combine(y, inv_perm, topk_weights, T, H, k, dtype == MOE_DTYPE_BF16, out,
                              static_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"

namespace {

// Optional parts of the block: a shared expert (ws13, ws2, Is) or token
// rounding to round_tile rows (0: off).
struct Options {
  const void* ws13 = nullptr;
  const void* ws2 = nullptr;
  int32_t Is = 0;
  int32_t round_tile = 0;
  void* gate_up = nullptr;   // bf16 [T*k, 2I]: the routed gate/up GEMM also writes its sums here
};

int forward_impl(const void* x, const void* w_router, const float* router_bias, const void* w13,
                 const void* w2, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                 int32_t dtype, int32_t renormalize, void* out, void* workspace,
                 size_t workspace_bytes, void* const* events, hipStream_t s,
                 const Options& opt = Options()) {
  const void* ws13 = opt.ws13;
  const void* ws2 = opt.ws2;
  const int32_t Is = opt.Is;
  const bool with_shared = ws13 != nullptr || ws2 != nullptr || Is != 0;
  const bool rounded = opt.round_tile != 0;
  if (rounded && opt.round_tile < 1)
    return fail(MOE_ERR_INVALID_ARG, "tile_rows must be >= 1 (got %d)", opt.round_tile);
  if (rounded && with_shared)
    return fail(MOE_ERR_UNSUPPORTED, "token rounding with a shared expert is not supported");
  MOE_CHECK(check_sizes(T, H, I, E, k, dtype, true));
  if (with_shared) {
    MOE_CHECK(check_sizes(T, H, Is, 1, 1, dtype, true));
    if (T == 0) return ok();
    MOE_CHECK(need_ptr(ws13, "ws13", 16));
    MOE_CHECK(need_ptr(ws2, "ws2", 16));
  }
  if (T == 0) return ok();
  MOE_CHECK(need_ptr(x, "x", 16));
  MOE_CHECK(need_ptr(w_router, "w_router", 16));
  if (router_bias) MOE_CHECK(need_ptr(router_bias, "router_bias", 4));
  MOE_CHECK(need_ptr(w13, "w13", 16));
  MOE_CHECK(need_ptr(w2, "w2", 16));
  MOE_CHECK(need_ptr(out, "out", 16));
  const moe_shared_layout SL = shared_layout(T, H, I, with_shared ? Is : 64, E, k, dtype);
  const moe_forward_layout L = rounded ? rounded_layout(T, H, I, E, k, dtype) : SL.routed;
  const size_t need = with_shared ? SL.total : L.total;
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  MOE_CHECK(need_ptr(workspace, "workspace", 256));
  const int n_events = with_shared ? MOE_PROFILE_EVENTS_SHARED
                       : rounded   ? MOE_PROFILE_EVENTS_ROUNDED
                                   : MOE_PROFILE_EVENTS;
  if (events)
    for (int i = 0; i < n_events; ++i)
      if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "events[%d] is NULL", i);
  int cu = 0;
  MOE_CHECK(current_device(nullptr, &cu));
  char* w = static_cast<char*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(w + L.topk_ids);
  float* wts = reinterpret_cast<float*>(w + L.topk_weights);
  int32_t* counts = reinterpret_cast<int32_t*>(w + L.expert_counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(w + L.expert_offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(w + L.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(w + L.inv_perm);
  int32_t* prefix = reinterpret_cast<int32_t*>(w + L.scratch);
  const int64_t M = T * k;
  char* shared = w + L.scratch + gemm_scratch(M, H, I, E, dtype);
  const bool bf16 = dtype == MOE_DTYPE_BF16;
  const int bm = bf16 ? moe::kGemmBM : moe::kF32BM;
  int next_event = 0;
  auto mark = [&]() -> int {
    if (events) MOE_HIP(hipEventRecord(static_cast<hipEvent_t>(events[next_event]), s));
    ++next_event;
    return MOE_OK;
  };

  MOE_CHECK(mark());
  if (rounded) {
    // router scratch, permutation scratch and rounding scratch side by side
    Carver c;
    char* rs = shared + c.take(moe::route_scratch_bytes(T, H, E, bf16));
    char* ps = shared + c.take(moe::permute_scratch_bytes(M, E));
    char* xs = shared + c.take(moe::round_scratch_bytes(T));
    moe::RouteArgs ra{};
    MOE_CHECK(run_route(x, w_router, router_bias, T, H, E, k, dtype, renormalize, ids, wts, rs, s,
                        &ra));
    MOE_CHECK(mark());
    MOE_CHECK(run_permute(ids, M, E, k, counts, offsets, perm, inv, ps, s));
    moe::RoundArgs r{};
    r.ids = ids; r.weights = wts; r.logits = ra.logits; r.meta = ra.meta;
    r.counts = counts; r.offsets = offsets; r.inv = inv;
    r.T = T; r.E = E; r.k = k; r.B = opt.round_tile; r.renorm = renormalize;
    moe::carve_round(xs, r);
    MOE_HIP(moe::launch_token_round(r, s));
    MOE_CHECK(mark());
    MOE_CHECK(run_permute(ids, M, E, k, counts, offsets, perm, inv, ps, s, prefix, bm));
  } else {
    MOE_CHECK(run_route(x, w_router, router_bias, T, H, E, k, dtype, renormalize, ids, wts, shared,
                        s));
    MOE_CHECK(mark());
    MOE_CHECK(run_permute(ids, M, E, k, counts, offsets, perm, inv, shared, s, prefix, bm));
  }
  // (the permutation's last pass also wrote the GEMMs' tile prefix)
  MOE_CHECK(mark());
  moe::GemmArgs g{};
  g.E = E; g.offsets = offsets; g.prefix = prefix; g.I = I; g.M = M; g.a_rows = T;
  g.grid = bf16 ? (cu >= 8 ? cu / 8 * 8 : 8) : cu * 2;
  if (bf16) {
    g.partials = reinterpret_cast<float*>(w + L.scratch + gemm_prefix_bytes(E));
    g.max_pieces = moe::gemm_pieces(M, H, I, E, false);
  }
  g.A = x; g.gather = perm; g.gather_div = k;
  if (bf16 && !moe::gemm_gather_fits(T, H, 2)) {
    // x spans more than 2^32 bytes: gather its rows into the (not yet used)
    // down-projection output buffer, which has the same [M, H] shape
    MOE_HIP(moe::launch_gather_rows(x, inv, T, H, k, 2, w + L.y, s));
    g.A = w + L.y; g.gather = nullptr; g.gather_div = 1; g.a_rows = M;
  }
  g.B = w13; g.b_stride = static_cast<int64_t>(2) * I * H;
  g.C = w + L.h; g.N = I; g.K = H; g.C2 = opt.gate_up;
  MOE_HIP(bf16 ? moe::launch_gemm_bf16_swiglu(g, s) : moe::launch_gemm_f32_swiglu(g, s));
  MOE_CHECK(mark());
  // y rows go straight to token order (row t*k+j), so the combine streams them
  g.C2 = nullptr;
  g.A = w + L.h; g.gather = nullptr; g.gather_div = 1; g.a_rows = M;
  g.B = w2; g.b_stride = static_cast<int64_t>(H) * I;
  g.C = w + L.y; g.N = H; g.K = I; g.scatter = perm;
  MOE_HIP(bf16 ? moe::launch_gemm_bf16_down(g, s) : moe::launch_gemm_f32_down(g, s));
  MOE_CHECK(mark());
  const void* ys = nullptr;
  if (with_shared) {
    // the shared expert: one dense group of all T rows of x through the same
    // grouped-GEMM kernels
    char* ss = w + SL.scratch;
    int32_t* soff = reinterpret_cast<int32_t*>(ss);
    int32_t* spre = reinterpret_cast<int32_t*>(ss + 256);
    MOE_HIP(moe::launch_dense_offsets(soff, T, s));
    MOE_HIP(moe::launch_tile_schedule(soff, 1, bf16 ? moe::kGemmBM : moe::kF32BM, T, spre, s));
    moe::GemmArgs d{};
    d.E = 1; d.offsets = soff; d.prefix = spre; d.I = Is; d.M = T; d.a_rows = T; d.grid = g.grid;
    if (bf16) {
      d.partials = reinterpret_cast<float*>(ss + 256 + gemm_prefix_bytes(1));
      d.max_pieces = moe::gemm_pieces(T, H, Is, 1, false);
    }
    d.A = x; d.gather = nullptr; d.gather_div = 1;
    d.B = ws13; d.b_stride = static_cast<int64_t>(2) * Is * H;
    d.C = w + SL.h_shared; d.N = Is; d.K = H;
    MOE_HIP(bf16 ? moe::launch_gemm_bf16_swiglu(d, s) : moe::launch_gemm_f32_swiglu(d, s));
    d.A = w + SL.h_shared;
    d.B = ws2; d.b_stride = static_cast<int64_t>(H) * Is;
    d.C = w + SL.y_shared; d.N = H; d.K = Is;
    MOE_HIP(bf16 ? moe::launch_gemm_bf16_down(d, s) : moe::launch_gemm_f32_down(d, s));
    ys = w + SL.y_shared;
    MOE_CHECK(mark());
  }
  MOE_HIP(moe::launch_combine(w + L.y, nullptr, wts, T, H, k, bf16, out, s, ys));
  MOE_CHECK(mark());
  if (next_event != n_events)
    return fail(MOE_ERR_UNSUPPORTED, "internal: %d stage events recorded, %d expected", next_event,
                n_events);
  return ok();
}

}  // namespace

extern "C" {

int moe_forward(const void* x, const void* w_router, const float* router_bias, const void* w13,
                const void* w2, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                int32_t dtype, int32_t renormalize, void* out, void* workspace,
                size_t workspace_bytes, void* stream) {
  return forward_impl(x, w_router, router_bias, w13, w2, T, H, I, E, k, dtype, renormalize, out,
                      workspace, workspace_bytes, nullptr, static_cast<hipStream_t>(stream));
}

int moe_forward_profiled(const void* x, const void* w_router, const float* router_bias,
                         const void* w13, const void* w2, int64_t T, int32_t H, int32_t I,
                         int32_t E, int32_t k, int32_t dtype, int32_t renormalize, void* out,
                         void* workspace, size_t workspace_bytes, void* const* events,
                         int32_t n_events, void* stream) {
  if (!events || n_events != MOE_PROFILE_EVENTS)
    return fail(MOE_ERR_INVALID_ARG, "events must hold MOE_PROFILE_EVENTS (%d) handles",
                MOE_PROFILE_EVENTS);
  return forward_impl(x, w_router, router_bias, w13, w2, T, H, I, E, k, dtype, renormalize, out,
                      workspace, workspace_bytes, events, static_cast<hipStream_t>(stream));
}

int moe_forward_train(const void* x, const void* w_router, const float* router_bias,
                      const void* w13, const void* w2, int64_t T, int32_t H, int32_t I, int32_t E,
                      int32_t k, int32_t dtype, int32_t renormalize, void* out, void* gate_up,
                      void* workspace, size_t workspace_bytes, void* const* events,
                      int32_t n_events, void* stream) {
  if (dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_forward_train needs dtype MOE_DTYPE_BF16");
  if (T > 0) MOE_CHECK(need_ptr(gate_up, "gate_up", 16));
  if (events && n_events != MOE_PROFILE_EVENTS)
    return fail(MOE_ERR_INVALID_ARG, "events must hold MOE_PROFILE_EVENTS (%d) handles",
                MOE_PROFILE_EVENTS);
  Options o;
  o.gate_up = gate_up;
  return forward_impl(x, w_router, router_bias, w13, w2, T, H, I, E, k, dtype, renormalize, out,
                      workspace, workspace_bytes, events, static_cast<hipStream_t>(stream), o);
}

int moe_forward_shared(const void* x, const void* w_router, const float* router_bias,
                       const void* w13, const void* w2, const void* ws13, const void* ws2,
                       int64_t T, int32_t H, int32_t I, int32_t Is, int32_t E, int32_t k,
                       int32_t dtype, int32_t renormalize, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!ws13 || !ws2) return fail(MOE_ERR_INVALID_ARG, "ws13 and ws2 must be set");
  Options o;
  o.ws13 = ws13; o.ws2 = ws2; o.Is = Is;
  return forward_impl(x, w_router, router_bias, w13, w2, T, H, I, E, k, dtype, renormalize, out,
                      workspace, workspace_bytes, nullptr, static_cast<hipStream_t>(stream), o);
}

int moe_forward_shared_profiled(const void* x, const void* w_router, const float* router_bias,
                                const void* w13, const void* w2, const void* ws13,
                                const void* ws2, int64_t T, int32_t H, int32_t I, int32_t Is,
                                int32_t E, int32_t k, int32_t dtype, int32_t renormalize,
                                void* out, void* workspace, size_t workspace_bytes,
                                void* const* events, int32_t n_events, void* stream) {
  if (!ws13 || !ws2) return fail(MOE_ERR_INVALID_ARG, "ws13 and ws2 must be set");
  if (!events || n_events != MOE_PROFILE_EVENTS_SHARED)
    return fail(MOE_ERR_INVALID_ARG, "events must hold MOE_PROFILE_EVENTS_SHARED (%d) handles",
                MOE_PROFILE_EVENTS_SHARED);
  Options o;
  o.ws13 = ws13; o.ws2 = ws2; o.Is = Is;
  return forward_impl(x, w_router, router_bias, w13, w2, T, H, I, E, k, dtype, renormalize, out,
                      workspace, workspace_bytes, events, static_cast<hipStream_t>(stream), o);
}

int moe_forward_shared_layout(int64_t T, int32_t H, int32_t I, int32_t Is, int32_t E, int32_t k,
                              int32_t dtype, moe_shared_layout* layout) {
  if (!layout) return fail(MOE_ERR_INVALID_ARG, "layout is NULL");
  MOE_CHECK(check_sizes(T, H, I, E, k, dtype, true));
  MOE_CHECK(check_sizes(T, H, Is, 1, 1, dtype, true));
  *layout = shared_layout(T, H, I, Is, E, k, dtype);
  return ok();
}

int moe_forward_rounded(const void* x, const void* w_router, const float* router_bias,
                        const void* w13, const void* w2, int64_t T, int32_t H, int32_t I,
                        int32_t E, int32_t k, int32_t dtype, int32_t renormalize,
                        int32_t tile_rows, void* out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (tile_rows < 1) return fail(MOE_ERR_INVALID_ARG, "tile_rows must be >= 1 (got %d)", tile_rows);
  Options o;
  o.round_tile = tile_rows;
  return forward_impl(x, w_router, router_bias, w13, w2, T, H, I, E, k, dtype, renormalize, out,
                      workspace, workspace_bytes, nullptr, static_cast<hipStream_t>(stream), o);
}

int moe_forward_rounded_profiled(const void* x, const void* w_router, const float* router_bias,
                                 const void* w13, const void* w2, int64_t T, int32_t H,
                                 int32_t I, int32_t E, int32_t k, int32_t dtype,
                                 int32_t renormalize, int32_t tile_rows, void* out,
                                 void* workspace, size_t workspace_bytes, void* const* events,
                                 int32_t n_events, void* stream) {
  if (tile_rows < 1) return fail(MOE_ERR_INVALID_ARG, "tile_rows must be >= 1 (got %d)", tile_rows);
  if (!events || n_events != MOE_PROFILE_EVENTS_ROUNDED)
    return fail(MOE_ERR_INVALID_ARG, "events must hold MOE_PROFILE_EVENTS_ROUNDED (%d) handles",
                MOE_PROFILE_EVENTS_ROUNDED);
  Options o;
  o.round_tile = tile_rows;
  return forward_impl(x, w_router, router_bias, w13, w2, T, H, I, E, k, dtype, renormalize, out,
                      workspace, workspace_bytes, events, static_cast<hipStream_t>(stream), o);
}

int moe_forward_rounded_layout(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                               int32_t dtype, moe_forward_layout* layout) {
  if (!layout) return fail(MOE_ERR_INVALID_ARG, "layout is NULL");
  MOE_CHECK(check_sizes(T, H, I, E, k, dtype, true));
  *layout = rounded_layout(T, H, I, E, k, dtype);
  return ok();
}

int moe_mx_quantize(const void* src, int64_t rows, int32_t cols, int32_t dtype, uint8_t* codes,
                    uint8_t* scales, void* stream) {
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
  if (cols <= 0 || cols % moe::kMxBlock)
    return fail(MOE_ERR_INVALID_ARG, "cols must be a positive multiple of 32 (got %d)", cols);
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (rows * static_cast<int64_t>(cols) / 8 / 256 > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "rows*cols (%lld) too large", (long long)(rows * cols));
  if (rows == 0) return ok();
  MOE_CHECK(need_ptr(src, "src", 16));
  MOE_CHECK(need_ptr(codes, "codes", 16));
  MOE_CHECK(need_ptr(scales, "scales", 1));
  MOE_CHECK(current_device(nullptr, nullptr));
  MOE_HIP(moe::launch_mx_quantize(src, dtype == MOE_DTYPE_BF16, rows, cols, codes, scales,
                                  static_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"

namespace {

int check_mxfp8(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t dtype) {
  MOE_CHECK(check_sizes(T, H, I, E, k, dtype, true));
  if (dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "moe_forward_mxfp8 needs dtype MOE_DTYPE_BF16");
  if (H % 128) return fail(MOE_ERR_UNSUPPORTED, "H (%d) must be a multiple of 128", H);
  if (I % 128) return fail(MOE_ERR_UNSUPPORTED, "I (%d) must be a multiple of 128", I);
  if (!moe::gemm_gather_fits(T, H, 1))
    return fail(MOE_ERR_UNSUPPORTED, "T*H (%lld) exceeds 2^32", (long long)(T * H));
  return MOE_OK;
}

moe_mxfp8_layout mxfp8_layout(int64_t T, int H, int I, int E, int k) {
  const size_t M = static_cast<size_t>(T) * k;
  Carver c;
  moe_mxfp8_layout L;
  L.topk_ids = c.take(M * 4);
  L.topk_weights = c.take(M * 4);
  L.expert_counts = c.take(static_cast<size_t>(E) * 4);
  L.expert_offsets = c.take(static_cast<size_t>(E + 1) * 4);
  L.perm = c.take(M * 4);
  L.inv_perm = c.take(M * 4);
  L.x_codes = c.take(static_cast<size_t>(T) * H);
  L.x_scales = c.take(static_cast<size_t>(T) * H / 32);
  L.h_codes = c.take(M * I);
  L.h_scales = c.take(M * I / 32);
  L.y = c.take(M * H * 2);
  L.x_scale_words = c.take(M * H / 32);
  L.w13_scale_words = c.take(static_cast<size_t>(E) * 2 * I * H / 32);
  L.w2_scale_words = c.take(static_cast<size_t>(E) * H * I / 32);
  const size_t rs = moe::route_scratch_bytes(T, H, E, true);
  const size_t ps = moe::permute_scratch_bytes(static_cast<int64_t>(M), E);
  const size_t gs = gemm_prefix_bytes(E) +
                    static_cast<size_t>(moe::gemm_pieces(static_cast<int64_t>(M), H, I, E, true)) *
                        moe::kGemmBM * moe::kGemmBN * 4;
  L.scratch = c.take(gs + (rs > ps ? rs : ps));
  L.total = c.o;
  return L;
}

int forward_mxfp8_impl(const void* x, const void* w_router, const float* router_bias,
                       const uint8_t* w13q, const uint8_t* w13s, const uint8_t* w2q,
                       const uint8_t* w2s, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                       int32_t dtype, int32_t renormalize, void* out, void* workspace,
                       size_t workspace_bytes, void* const* events, hipStream_t s) {
  MOE_CHECK(check_mxfp8(T, H, I, E, k, dtype));
  if (T == 0) return ok();
  MOE_CHECK(need_ptr(x, "x", 16));
  MOE_CHECK(need_ptr(w_router, "w_router", 16));
  if (router_bias) MOE_CHECK(need_ptr(router_bias, "router_bias", 4));
  MOE_CHECK(need_ptr(w13q, "w13q", 16));
  MOE_CHECK(need_ptr(w13s, "w13s", 4));
  MOE_CHECK(need_ptr(w2q, "w2q", 16));
  MOE_CHECK(need_ptr(w2s, "w2s", 4));
  MOE_CHECK(need_ptr(out, "out", 16));
  const moe_mxfp8_layout L = mxfp8_layout(T, H, I, E, k);
  if (!workspace || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", L.total,
                workspace_bytes);
  MOE_CHECK(need_ptr(workspace, "workspace", 256));
  if (events)
    for (int i = 0; i < MOE_PROFILE_EVENTS_MXFP8; ++i)
      if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "events[%d] is NULL", i);
  int cu = 0;
  MOE_CHECK(current_device(nullptr, &cu));
  char* w = static_cast<char*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(w + L.topk_ids);
  float* wts = reinterpret_cast<float*>(w + L.topk_weights);
  int32_t* counts = reinterpret_cast<int32_t*>(w + L.expert_counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(w + L.expert_offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(w + L.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(w + L.inv_perm);
  uint8_t* xq = reinterpret_cast<uint8_t*>(w + L.x_codes);
  uint8_t* xs = reinterpret_cast<uint8_t*>(w + L.x_scales);
  int32_t* prefix = reinterpret_cast<int32_t*>(w + L.scratch);
  const int64_t M = T * k;
  const int pieces = moe::gemm_pieces(M, H, I, E, true);
  char* shared = w + L.scratch + gemm_prefix_bytes(E) +
                 static_cast<size_t>(pieces) * moe::kGemmBM * moe::kGemmBN * 4;
  int next_event = 0;
  auto mark = [&]() -> int {
    if (events) MOE_HIP(hipEventRecord(static_cast<hipEvent_t>(events[next_event]), s));
    ++next_event;
    return MOE_OK;
  };

  MOE_CHECK(mark());
  MOE_CHECK(run_route(x, w_router, router_bias, T, H, E, k, dtype, renormalize, ids, wts, shared, s));
  MOE_CHECK(mark());
  MOE_CHECK(run_permute(ids, M, E, k, counts, offsets, perm, inv, shared, s, prefix,
                        moe::kGemmBM));
  MOE_CHECK(mark());
  MOE_HIP(moe::launch_mx_quantize(x, true, T, H, xq, xs, s));
  // stage-major scale words for the GEMMs: x's in the expert-sorted row order
  // (the GEMM gathers the codes, not the scales), the weights' as given
  uint32_t* xsw = reinterpret_cast<uint32_t*>(w + L.x_scale_words);
  uint32_t* w13sw = reinterpret_cast<uint32_t*>(w + L.w13_scale_words);
  uint32_t* w2sw = reinterpret_cast<uint32_t*>(w + L.w2_scale_words);
  MOE_HIP(moe::launch_mx_scale_words(xs, M, H, perm, k, xsw, s));
  MOE_HIP(moe::launch_mx_scale_words(w13s, static_cast<int64_t>(E) * 2 * I, H, nullptr, 1, w13sw, s));
  MOE_HIP(moe::launch_mx_scale_words(w2s, static_cast<int64_t>(E) * H, I, nullptr, 1, w2sw, s));
  MOE_CHECK(mark());
  moe::GemmArgs g{};
  g.E = E; g.offsets = offsets; g.prefix = prefix; g.I = I; g.M = M;
  g.grid = cu >= 8 ? cu / 8 * 8 : 8;
  g.partials = reinterpret_cast<float*>(w + L.scratch + gemm_prefix_bytes(E));
  g.max_pieces = pieces;
  // gate/up: rows of x gathered through the permutation, h quantized on the way out
  g.A = xq; g.gather = perm; g.gather_div = k; g.a_rows = T;
  g.a_scale = reinterpret_cast<const uint8_t*>(xsw); g.a_srows = M;
  g.B = w13q; g.b_stride = static_cast<int64_t>(2) * I * H;
  g.b_scale = reinterpret_cast<const uint8_t*>(w13sw); g.b_srows = static_cast<int64_t>(E) * 2 * I;
  g.C = w + L.h_codes; g.c_scale = reinterpret_cast<uint8_t*>(w + L.h_scales); g.c_srows = M;
  g.N = I; g.K = H;
  MOE_HIP(moe::launch_gemm_mx_swiglu(g, s));
  MOE_CHECK(mark());
  // down: y rows go straight to token order (row t*k+j), so the combine streams them
  g.A = w + L.h_codes; g.a_scale = reinterpret_cast<uint8_t*>(w + L.h_scales); g.a_srows = M;
  g.gather = nullptr; g.gather_div = 1; g.a_rows = M;
  g.B = w2q; g.b_stride = static_cast<int64_t>(H) * I;
  g.b_scale = reinterpret_cast<const uint8_t*>(w2sw); g.b_srows = static_cast<int64_t>(E) * H;
  g.C = w + L.y; g.c_scale = nullptr; g.c_srows = 0; g.N = H; g.K = I; g.scatter = perm;
  MOE_HIP(moe::launch_gemm_mx_down(g, s));
  MOE_CHECK(mark());
  MOE_HIP(moe::launch_combine(w + L.y, nullptr, wts, T, H, k, true, out, s));
  MOE_CHECK(mark());
  if (next_event != MOE_PROFILE_EVENTS_MXFP8)
    return fail(MOE_ERR_UNSUPPORTED, "internal: %d stage events recorded, %d expected", next_event,
                MOE_PROFILE_EVENTS_MXFP8);
  return ok();
}

}  // namespace

extern "C" {

int moe_forward_mxfp8(const void* x, const void* w_router, const float* router_bias,
                      const uint8_t* w13q, const uint8_t* w13s, const uint8_t* w2q,
                      const uint8_t* w2s, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                      int32_t dtype, int32_t renormalize, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return forward_mxfp8_impl(x, w_router, router_bias, w13q, w13s, w2q, w2s, T, H, I, E, k, dtype,
                            renormalize, out, workspace, workspace_bytes, nullptr,
                            static_cast<hipStream_t>(stream));
}

int moe_forward_mxfp8_profiled(const void* x, const void* w_router, const float* router_bias,
                               const uint8_t* w13q, const uint8_t* w13s, const uint8_t* w2q,
                               const uint8_t* w2s, int64_t T, int32_t H, int32_t I, int32_t E,
                               int32_t k, int32_t dtype, int32_t renormalize, void* out,
                               void* workspace, size_t workspace_bytes, void* const* events,
                               int32_t n_events, void* stream) {
  if (!events || n_events != MOE_PROFILE_EVENTS_MXFP8)
    return fail(MOE_ERR_INVALID_ARG, "events must hold MOE_PROFILE_EVENTS_MXFP8 (%d) handles",
                MOE_PROFILE_EVENTS_MXFP8);
  return forward_mxfp8_impl(x, w_router, router_bias, w13q, w13s, w2q, w2s, T, H, I, E, k, dtype,
                            renormalize, out, workspace, workspace_bytes, events,
                            static_cast<hipStream_t>(stream));
}

int moe_forward_mxfp8_layout(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t dtype,
                             moe_mxfp8_layout* layout) {
  if (!layout) return fail(MOE_ERR_INVALID_ARG, "layout is NULL");
  MOE_CHECK(check_mxfp8(T, H, I, E, k, dtype));
  *layout = mxfp8_layout(T, H, I, E, k);
  return ok();
}

}  // extern "C"

namespace {

int check_backward(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t dtype) {
  MOE_CHECK(check_sizes(T, H, I, E, k, dtype, true));
  if (dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_backward needs dtype MOE_DTYPE_BF16");
  if (!moe::gemm_gather_fits(T, H, 2))
    return fail(MOE_ERR_UNSUPPORTED, "T*H*2 (%lld) exceeds 2^32", (long long)(T * H * 2));
  return MOE_OK;
}

// Padded row count of the weight-gradient operands: every expert's rows
// rounded up to a multiple of 64, and at least 64.
int64_t backward_ld(int64_t M, int E) { return (M + 63) / 64 * 64 + 64 * static_cast<int64_t>(E); }

// Workspace of moe_backward: the public regions, then the scratch (routing
// recompute, dW_r partials, small tables, ones, grouped-GEMM scratch).
struct BwdScratch {
  size_t route, ids, wts, dwr_part, tables, ones, gemm, end;
};
moe_backward_layout backward_layout(int64_t T, int H, int I, int E, int k, BwdScratch* sc = nullptr) {
  const size_t M = static_cast<size_t>(T) * k;
  const int64_t ld = backward_ld(static_cast<int64_t>(M), E);
  Carver c;
  moe_backward_layout L;
  L.dw = c.take(M * 4);
  L.dlogits = c.take(static_cast<size_t>(T) * E * 4);
  L.dx_router = c.take(static_cast<size_t>(T) * H * 2);
  L.gu = c.take(M * 2 * I * 2);
  L.dh = c.take(M * I * 2);
  L.dgdu = c.take(M * 2 * I * 2);
  L.h = c.take(M * I * 2);
  L.dx_slots = c.take(M * H * 2);
  L.padded_offsets = c.take(static_cast<size_t>(E + 1) * 4);
  L.dyT = c.take(static_cast<size_t>(H) * ld * 2);
  L.hT = c.take(static_cast<size_t>(I) * ld * 2);
  L.dgduT = c.take(static_cast<size_t>(2 * I) * ld * 2);
  L.xT = c.take(static_cast<size_t>(H) * ld * 2);
  L.ld = static_cast<size_t>(ld);
  L.scratch = c.o;
  BwdScratch b;
  b.route = c.take(moe::route_scratch_bytes(T, H, E, true));
  b.ids = c.take(M * 4);
  b.wts = c.take(M * 4);
  b.dwr_part = c.take(static_cast<size_t>(moe::bwd_dwr_slices(T)) * E * H * 4);
  b.tables = c.take(static_cast<size_t>(E + 1) * 4 * 4);
  b.ones = c.take(M * 4);
  b.gemm = c.take(gemm_prefix_bytes(E) +
                  static_cast<size_t>(moe::gemm_pieces(static_cast<int64_t>(M), H, 2 * I, E, false)) *
                      moe::kGemmBM * moe::kGemmBN * 4);
  b.end = c.o;
  L.total = c.o;
  if (sc) *sc = b;
  return L;
}

int backward_impl(const void* x, const void* w_router, const float* router_bias, const void* w13,
                  const void* w2, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                  int32_t dtype, int32_t renormalize, const void* fws, size_t fws_bytes,
                  const void* gate_up, const void* dout, void* dx, float* dwr, float* dbias,
                  float* dw13, float* dw2, void* workspace, size_t workspace_bytes,
                  void* const* events, hipStream_t s) {
  MOE_CHECK(check_backward(T, H, I, E, k, dtype));
  if (T == 0) return ok();
  MOE_CHECK(need_ptr(x, "x", 16));
  MOE_CHECK(need_ptr(w_router, "w_router", 16));
  if (router_bias) MOE_CHECK(need_ptr(router_bias, "router_bias", 4));
  MOE_CHECK(need_ptr(w13, "w13", 16));
  MOE_CHECK(need_ptr(w2, "w2", 16));
  MOE_CHECK(need_ptr(dout, "dout", 16));
  if (gate_up) MOE_CHECK(need_ptr(gate_up, "gate_up", 16));
  MOE_CHECK(need_ptr(dx, "dx", 16));
  MOE_CHECK(need_ptr(dwr, "dw_router", 16));
  if (dbias) MOE_CHECK(need_ptr(dbias, "dbias", 4));
  MOE_CHECK(need_ptr(dw13, "dw13", 16));
  MOE_CHECK(need_ptr(dw2, "dw2", 16));
  const moe_forward_layout F = forward_layout(T, H, I, E, k, dtype);
  if (!fws || fws_bytes < F.total)
    return fail(MOE_ERR_WORKSPACE, "forward_workspace must hold %zu bytes (the moe_forward workspace), got %zu",
                F.total, fws_bytes);
  MOE_CHECK(need_ptr(fws, "forward_workspace", 256));
  BwdScratch b;
  const moe_backward_layout L = backward_layout(T, H, I, E, k, &b);
  if (!workspace || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "backward needs %zu workspace bytes, got %zu", L.total,
                workspace_bytes);
  MOE_CHECK(need_ptr(workspace, "workspace", 256));
  if (events)
    for (int i = 0; i < MOE_PROFILE_EVENTS_BACKWARD; ++i)
      if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "events[%d] is NULL", i);
  int cu = 0;
  MOE_CHECK(current_device(nullptr, &cu));
  const char* f = static_cast<const char*>(fws);
  const int32_t* ids = reinterpret_cast<const int32_t*>(f + F.topk_ids);
  const float* wts = reinterpret_cast<const float*>(f + F.topk_weights);
  const int32_t* counts = reinterpret_cast<const int32_t*>(f + F.expert_counts);
  const int32_t* offsets = reinterpret_cast<const int32_t*>(f + F.expert_offsets);
  const int32_t* perm = reinterpret_cast<const int32_t*>(f + F.perm);
  const void* y = f + F.y;
  char* w = static_cast<char*>(workspace);
  float* dw = reinterpret_cast<float*>(w + L.dw);
  float* dl = reinterpret_cast<float*>(w + L.dlogits);
  int32_t* tab = reinterpret_cast<int32_t*>(w + b.tables);
  int32_t* poff = reinterpret_cast<int32_t*>(w + L.padded_offsets);
  int32_t* goff_h = tab;
  int32_t* pre_h = tab + (E + 1);
  int32_t* goff_i = tab + 2 * (E + 1);
  int32_t* pre_i = tab + 3 * (E + 1);
  float* ones = reinterpret_cast<float*>(w + b.ones);
  int32_t* prefix = reinterpret_cast<int32_t*>(w + b.gemm);
  const int64_t M = T * k;
  const int64_t ld = static_cast<int64_t>(L.ld);
  const int pieces = moe::gemm_pieces(M, H, 2 * I, E, false);
  int next_event = 0;
  auto mark = [&]() -> int {
    if (events) MOE_HIP(hipEventRecord(static_cast<hipEvent_t>(events[next_event]), s));
    ++next_event;
    return MOE_OK;
  };

  // 0: router gradients
  MOE_CHECK(mark());
  MOE_HIP(moe::launch_bwd_dw(dout, y, T, H, k, dw, s));
  moe::RouteArgs ra{};
  MOE_CHECK(run_route(x, w_router, router_bias, T, H, E, k, dtype, renormalize,
                      reinterpret_cast<int32_t*>(w + b.ids), reinterpret_cast<float*>(w + b.wts),
                      w + b.route, s, &ra));
  MOE_HIP(moe::launch_bwd_router(ra.logits, ra.meta, ids, dw, T, E, k, renormalize, dl, s));
  MOE_HIP(moe::launch_bwd_router_grads(dl, x, w_router, T, H, E, w + L.dx_router, dwr, dbias,
                                       reinterpret_cast<float*>(w + b.dwr_part), s));
  // 1: g and u again, unless the training forward kept them
  MOE_CHECK(mark());
  MOE_HIP(moe::launch_tile_schedule(offsets, E, moe::kGemmBM, M, prefix, s));
  moe::GemmArgs g{};
  g.E = E; g.offsets = offsets; g.prefix = prefix; g.M = M; g.I = I;
  g.grid = cu >= 8 ? cu / 8 * 8 : 8;
  g.partials = reinterpret_cast<float*>(w + b.gemm + gemm_prefix_bytes(E));
  g.max_pieces = pieces;
  g.A = x; g.gather = perm; g.gather_div = k; g.a_rows = T;
  const void* gu = gate_up ? gate_up : w + L.gu;
  if (!gate_up) {
    g.B = w13; g.C = w + L.gu; g.N = 2 * I; g.K = H;
    MOE_HIP(moe::launch_gemm_bf16_plain(g, s));
  }
  // 2: dh = dout W2_e (W2 read as stored, [E, H, I] = [E, K, N]), then the
  // SwiGLU backward
  MOE_CHECK(mark());
  g.A = dout; g.B = w2; g.C = w + L.dh; g.N = I; g.K = H;
  MOE_HIP(moe::launch_gemm_bf16_bt(g, s));
  MOE_HIP(moe::launch_bwd_swiglu(w + L.dh, gu, wts, perm, M, I, w + L.dgdu, w + L.h, s));
  // 3: dx = sum over a token's slots of [dg du] W13_e (W13 read as stored,
  // [E, 2I, H] = [E, K, N]), plus dl W_r
  MOE_CHECK(mark());
  g.A = w + L.dgdu; g.gather = nullptr; g.gather_div = 1; g.a_rows = M;
  g.B = w13; g.C = w + L.dx_slots; g.N = H; g.K = 2 * I; g.scatter = perm;
  MOE_HIP(moe::launch_gemm_bf16_bt(g, s));
  MOE_HIP(moe::launch_fill(ones, M, 1.f, s));
  MOE_HIP(moe::launch_combine(w + L.dx_slots, nullptr, ones, T, H, k, true, dx, s, w + L.dx_router));
  // 4: transposed, padded operands of the weight-gradient GEMMs
  MOE_CHECK(mark());
  MOE_HIP(moe::launch_bwd_tables(counts, E, H, I, poff, goff_h, pre_h, goff_i, pre_i, s));
  MOE_HIP(moe::launch_gather_transpose(dout, H, perm, true, k, wts, offsets, counts, poff, E, ld,
                                       w + L.dyT, s));
  MOE_HIP(moe::launch_gather_transpose(w + L.h, I, perm, false, k, nullptr, offsets, counts, poff, E,
                                       ld, w + L.hT, s));
  MOE_HIP(moe::launch_gather_transpose(w + L.dgdu, 2 * I, perm, false, k, nullptr, offsets, counts,
                                       poff, E, ld, w + L.dgduT, s));
  MOE_HIP(moe::launch_gather_transpose(x, H, perm, true, k, nullptr, offsets, counts, poff, E, ld,
                                       w + L.xT, s));
  // 5: dW2_e = sum (w dout)^T h over the expert's rows
  MOE_CHECK(mark());
  moe::GemmArgs v{};
  v.E = E; v.koff = poff; v.ld = ld; v.grid = g.grid;
  v.offsets = goff_h; v.prefix = pre_h; v.group_rows = H; v.M = static_cast<int64_t>(E) * H;
  v.A = w + L.dyT; v.B = w + L.hT; v.N = I; v.Cf = dw2; v.a_rows = H;
  MOE_HIP(moe::launch_gemm_bf16_wgrad(v, s));
  // 6: dW13_e = sum [dg du]^T x over the expert's rows
  MOE_CHECK(mark());
  v.offsets = goff_i; v.prefix = pre_i; v.group_rows = 2 * I; v.M = static_cast<int64_t>(E) * 2 * I;
  v.A = w + L.dgduT; v.B = w + L.xT; v.N = H; v.Cf = dw13; v.a_rows = 2 * I;
  MOE_HIP(moe::launch_gemm_bf16_wgrad(v, s));
  MOE_CHECK(mark());
  if (next_event != MOE_PROFILE_EVENTS_BACKWARD)
    return fail(MOE_ERR_UNSUPPORTED, "internal: %d stage events recorded, %d expected", next_event,
                MOE_PROFILE_EVENTS_BACKWARD);
  return ok();
}

}  // namespace

extern "C" {

int moe_backward(const void* x, const void* w_router, const float* router_bias, const void* w13,
                 const void* w2, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                 int32_t dtype, int32_t renormalize, const void* forward_workspace,
                 size_t forward_workspace_bytes, const void* gate_up, const void* dout, void* dx,
                 float* dw_router, float* dbias, float* dw13, float* dw2, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return backward_impl(x, w_router, router_bias, w13, w2, T, H, I, E, k, dtype, renormalize,
                       forward_workspace, forward_workspace_bytes, gate_up, dout, dx, dw_router,
                       dbias, dw13, dw2, workspace, workspace_bytes, nullptr,
                       static_cast<hipStream_t>(stream));
}

int moe_backward_profiled(const void* x, const void* w_router, const float* router_bias,
                          const void* w13, const void* w2, int64_t T, int32_t H, int32_t I,
                          int32_t E, int32_t k, int32_t dtype, int32_t renormalize,
                          const void* forward_workspace, size_t forward_workspace_bytes,
                          const void* gate_up, const void* dout, void* dx, float* dw_router,
                          float* dbias, float* dw13, float* dw2, void* workspace,
                          size_t workspace_bytes, void* const* events, int32_t n_events,
                          void* stream) {
  if (!events || n_events != MOE_PROFILE_EVENTS_BACKWARD)
    return fail(MOE_ERR_INVALID_ARG, "events must hold MOE_PROFILE_EVENTS_BACKWARD (%d) handles",
                MOE_PROFILE_EVENTS_BACKWARD);
  return backward_impl(x, w_router, router_bias, w13, w2, T, H, I, E, k, dtype, renormalize,
                       forward_workspace, forward_workspace_bytes, gate_up, dout, dx, dw_router,
                       dbias, dw13, dw2, workspace, workspace_bytes, events,
                       static_cast<hipStream_t>(stream));
}

int moe_backward_workspace_layout(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                  int32_t dtype, moe_backward_layout* layout) {
  if (!layout) return fail(MOE_ERR_INVALID_ARG, "layout is NULL");
  MOE_CHECK(check_backward(T, H, I, E, k, dtype));
  *layout = backward_layout(T, H, I, E, k);
  return ok();
}

int moe_gemm_tile_rows(int32_t dtype) {
  if (dtype == MOE_DTYPE_BF16) return moe::kGemmBM;
  if (dtype == MOE_DTYPE_F32) return moe::kF32BM;
  fail(MOE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  return 0;
}

}  // extern "C"
