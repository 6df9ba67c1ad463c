// Token rounding (gfx950).
//
// Page legend:
//   [SonicMoE page] "SonicMoE与传统MoE架构对比：Token舍入技术如何实现训练效率跃升"
//
// [SonicMoE page] 核心差异 §3 rounds every expert's assignment count down to a
// multiple of the GEMM row tile and gives the remaining tokens to the
// least-loaded experts, so the grouped GEMM no longer pads its last tile per
// expert.  The rule, made exact (every decision is on integers):
//   1. expert e keeps the first floor(c_e / B) * B of its assignments in flat
//      order f = t*k + j (its segment of the stable permutation); the rest
//      are pooled;
//   2. the pool is handed out in rounds.  A round with P pooled assignments
//      left opens ceil(P / B) tiles of B rows and first picks every tile's
//      owner by water-filling: the expert with the lowest load (kept rows
//      plus B per tile already planned; ties to the lowest id), skipping
//      experts one of whose tiles came out empty.  Then, tile by tile, a tile
//      takes up to B pooled assignments in flat order whose token holds the
//      owner in no other slot, at most one slot per token (per token: the
//      first untaken pooled slot, or only the slot that already holds the
//      owner, if there is one).  What a round leaves goes to the next round;
//   3. a moved slot's weight is the token's softmax probability of its new
//      expert, renormalised over the token's k weights when asked.
//
// Three kernels:
//   mark   - per token: the pooled slots (rank in its expert >= kept rows)
//            and the token's ids packed one byte per slot;
//   tiles  - one 1024-thread workgroup compacts the pool tokens (those with a
//            pooled slot) and loads their state (ids packed one byte per
//            slot, untaken pooled slots) into LDS.  Per round, wave 0 plans
//            the owners (when every load is a multiple of B, water-filling is
//            level by level: at level L every expert with load <= L takes one
//            tile, in id order).  The 16 waves then run tiles w, w + 16, ...:
//            a tile walks the pool tokens 64 at a time from the first block
//            not known to be exhausted, finds each token's candidate slot
//            with a zero-byte test on its packed ids, ranks the candidates
//            with a ballot and takes the first `need`.  Tile i handles block
//            b only after tile i-1 has released it (a progress counter per
//            tile in LDS), so the tiles run as a pipeline one block apart and
//            the result is that of handing them out one after another;
//   finish - per token: writes the new ids of moved slots and recomputes the
//            weights of every token whose experts changed, with the router's
//            own formula (exp(logit - max) / sum, renormalised in slot order).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRoundThreads = 1024;
constexpr int kRoundWaves = kRoundThreads / kWave;
constexpr int kRoundLdsCap = 14336;       // pool tokens whose state fits in LDS
constexpr int kCompactPer = 16;           // tokens per thread in the compaction

}  // namespace
}  // namespace moe

// Device-library wave reduction (DPP row shifts and two lane reads).
extern "C" __device__ unsigned int __ockl_wfred_min_u32(unsigned int);

namespace moe {
namespace {

__global__ __launch_bounds__(256) void round_mark_kernel(RoundArgs a) {
  __shared__ int keep_s[kMaxE];
  __shared__ int off_s[kMaxE];
  const int tid = threadIdx.x;
  if (tid < a.E) {
    const int c = a.counts[tid];
    keep_s[tid] = c / a.B * a.B;
    off_s[tid] = a.offsets[tid];
  }
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + tid;
  if (t >= a.T) return;
  const int k = a.k;
  uint32_t m = 0;
  uint64_t packed = 0;
  for (int j = 0; j < k; ++j) {
    const int64_t f = t * k + j;
    const int e = a.ids[f];
    if (a.inv[f] - off_s[e] >= keep_s[e]) m |= 1u << j;
    packed |= static_cast<uint64_t>(e) << (8 * j);
  }
  a.mask[t] = static_cast<uint8_t>(m);
  a.packed[t] = packed;
}

// Byte j of a packed id word.
__device__ __forceinline__ int id_byte(uint64_t w, int j) {
  return static_cast<int>((w >> (8 * j)) & 0xffu);
}

// The slot of a pool token that a tile of expert o takes: the slot holding o
// if it is an untaken pooled slot, none if a kept or taken slot holds o,
// else the first untaken pooled slot.  -1: none.  ob = o in every byte;
// kbytes = 0x80 in the token's k bytes.  The zero-byte test of w ^ ob flags
// the byte equal to o (ids of a token are distinct, so at most one; a borrow
// can only flag bytes above a true zero byte, never below it).  Written
// with selects only, so a wave runs it without branches.
__device__ __forceinline__ int take_slot(uint32_t m, uint64_t w, uint64_t ob, uint64_t kbytes) {
  const uint64_t x = w ^ ob;
  const uint64_t z = (x - 0x0101010101010101ull) & ~x & kbytes;
  // bit 63 keeps the count defined for z == 0 (that result is not used)
  const int pos = __builtin_ctzll(z | (1ull << 63)) >> 3;
  const int held = ((m >> pos) & 1u) ? pos : -1;
  const int firstp = __builtin_ctz(m | 0x100u);      // 8: no pooled slot
  return z ? held : (firstp < 8 ? firstp : -1);
}

constexpr int kRoundMaxTiles = kMaxE;        // tiles per round: ceil(pooled / B) <= E

// Shared hand-out state of the tiles kernel.
struct RoundShared {
  int owner[kRoundMaxTiles];     // owner expert of each tile of the round
  int prog[kRoundMaxTiles];      // 64-token blocks each tile has finished (INT_MAX: done)
  int got[kRoundMaxTiles];       // rows each tile took
  int got_e[kMaxE];              // rows each expert took in the round
  int empty_e[kMaxE];            // 1: a tile of the expert took nothing
  int n;                         // tiles of the round (0: finished)
  int first;                     // blocks before it are exhausted
  int64_t wtot[2][kRoundWaves];
};

__device__ __forceinline__ int lds_acquire(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_release(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Owners of the n tiles of a round (wave 0): water-filling over load (lane +
// 64 i; ~0u for experts that cannot take), each tile counted as B rows.
// When every load is a multiple of B, water-filling visits levels L = min,
// min + B, ...: at level L every expert with load <= L takes one tile, in id
// order.  Otherwise the lowest (plan, id) is taken tile by tile.  Returns the
// number of tiles with an owner.
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long o = __shfl_xor(v, off);
    v = o < v ? o : v;
  }
  return v;
}

__device__ int round_owners(const uint32_t (&load)[4], int n, int B, int* owner) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  uint32_t m4 = ~0u;
  bool aligned = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m4 = load[i] < m4 ? load[i] : m4;
    if (load[i] != ~0u && load[i] % static_cast<uint32_t>(B) != 0) aligned = false;
  }
  const uint32_t lo = __builtin_amdgcn_readfirstlane(__ockl_wfred_min_u32(m4));
  if (lo == ~0u) return 0;
  if (__ballot(!aligned) == 0) {
    uint64_t lvl = lo;
    int off = 0;
    while (off < n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = load[i] != ~0u && load[i] <= lvl;
        const unsigned long long b = __ballot(in);
        const int pos = off + __popcll(b & below);
        if (in && pos < n) owner[pos] = lane + 64 * i;
        off += __popcll(b);
      }
      lvl += static_cast<uint64_t>(B);
    }
    return n;
  }
  // plan << 8 | id, so the minimum is the lowest (plan, id)
  unsigned long long key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    key[i] = load[i] == ~0u ? ~0ull : (static_cast<unsigned long long>(load[i]) << 8) | (lane + 64 * i);
  for (int t = 0; t < n; ++t) {
    unsigned long long k4 = key[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) k4 = key[i] < k4 ? key[i] : k4;
    const unsigned long long best = wave_min_u64(k4);
    if (best == ~0ull) return t;
    const int o = static_cast<int>(best & 0xffu);
    if (lane == 0) owner[t] = o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i == o) key[i] += static_cast<unsigned long long>(B) << 8;
  }
  return n;
}

// One tile of a round, run by one wave: walks the pool tokens 64 at a time
// from the first block not known to be exhausted and takes up to B candidate
// slots in token order.  Block b is read only after tile i-1 has finished it
// (its progress counter, released after its writes), so the result is the
// one of handing the tiles out one after another.
template <typename SID, typename SMASK>
__device__ void round_tile(SID* sid, SMASK* smask, int Q, int i, RoundShared& sh, int k, int B) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  const uint64_t kbytes = k >= 8 ? 0x8080808080808080ull : (0x8080808080808080ull & ((1ull << (8 * k)) - 1ull));
  const int nblocks = (Q + 63) / 64;
  const int o = sh.owner[i];
  const uint64_t ob = 0x0101010101010101ull * static_cast<uint64_t>(o);
  const int s = lds_acquire(&sh.first);
  lds_release(&sh.prog[i], s);
  int need = B, got = 0;
  bool front = true;
  for (int b = s; b < nblocks && need > 0; ++b) {
    if (i > 0)
      while (lds_acquire(&sh.prog[i - 1]) <= b) __builtin_amdgcn_s_sleep(1);
    const int q = b * 64 + lane;
    const uint32_t m = q < Q ? static_cast<uint32_t>(smask[q]) : 0u;
    const uint64_t w = q < Q ? static_cast<uint64_t>(sid[q]) : 0ull;
    const int j = take_slot(m, w, ob, kbytes);
    const unsigned long long bc = __ballot(j >= 0);
    const bool take = j >= 0 && __popcll(bc & below) < need;
    const uint32_t ma = take ? (m & ~(1u << j)) : m;
    if (take) {
      const int sh8 = 8 * j;
      sid[q] = (w & ~(0xffull << sh8)) | (static_cast<uint64_t>(o) << sh8);
      smask[q] = static_cast<uint8_t>(ma);
    }
    const int c = __popcll(bc);
    const int took = c < need ? c : need;
    need -= took;
    got += took;
    front = front && __ballot(ma != 0) == 0;
    lds_release(&sh.prog[i], b + 1);
    // a hint only (later tiles start there; an older value makes them walk
    // exhausted blocks), so it leaves the hand-over path
    if (front && lane == 0) atomicMax(&sh.first, b + 1);
  }
  if (lane == 0) sh.got[i] = got;
  lds_release(&sh.prog[i], INT_MAX);
}

// The hand-out in rounds: wave 0 plans a round's owners, the waves take its
// tiles w, w + W, ... (each tile one block behind the previous one), wave 0
// folds the rows taken into the loads.  load is kept by wave 0 only.
template <typename SID, typename SMASK>
__device__ void round_hand_out(SID* sid, SMASK* smask, int Q, int64_t P, const RoundArgs& a,
                               uint32_t (&load)[4], RoundShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.B;
  int64_t left = P;
  while (true) {
    if (wave == 0) {
      int n = 0;
      if (left > 0) {
        const int64_t want = (left + B - 1) / B;
        n = round_owners(load, static_cast<int>(want < kRoundMaxTiles ? want : kRoundMaxTiles), B,
                         sh.owner);
      }
      for (int t = lane; t < n; t += kWave) sh.prog[t] = 0;
      for (int e = lane; e < kMaxE; e += kWave) {
        sh.got_e[e] = 0;
        sh.empty_e[e] = 0;
      }
      if (lane == 0) sh.n = n;
    }
    __syncthreads();
    const int n = sh.n;
    if (n == 0) break;
    for (int t = wave; t < n; t += kRoundWaves) round_tile(sid, smask, Q, t, sh, a.k, B);
    __syncthreads();
    if (wave == 0) {
      int taken = 0;
      for (int t = lane; t < n; t += kWave) {
        const int g = sh.got[t], e = sh.owner[t];
        atomicAdd(&sh.got_e[e], g);
        if (g == 0) sh.empty_e[e] = 1;
        taken += g;
      }
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) taken += __shfl_xor(taken, off);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS atomics are done
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < a.E && load[i] != ~0u)
          load[i] = sh.empty_e[e] ? ~0u : load[i] + static_cast<uint32_t>(sh.got_e[e]);
      }
      left -= taken;
    }
  }
}

__global__ __launch_bounds__(kRoundThreads) void round_tiles_kernel(RoundArgs a) {
  __shared__ uint64_t lsid[kRoundLdsCap];
  __shared__ uint8_t lmask[kRoundLdsCap];
  __shared__ RoundShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, B = a.B;

  // expert row counts (kept rows) in every wave; pooled count P
  uint32_t load[4];
  int64_t pooled = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    load[i] = ~0u;
    if (e < E) {
      const int c = a.counts[e];
      const int kept = c / B * B;
      load[i] = static_cast<uint32_t>(kept);
      pooled += c - kept;
    }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) pooled += __shfl_xor(pooled, off);
  if (pooled == 0) return;

  // compaction of the pool tokens, in token order
  int64_t carry = 0;
  int tb = 0;
  for (int64_t base = 0; base < a.T; base += static_cast<int64_t>(kRoundThreads) * kCompactPer) {
    const int64_t t0 = base + static_cast<int64_t>(tid) * kCompactPer;
    uint8_t mk[kCompactPer];
    if (t0 + kCompactPer <= a.T) {
      const uint4 v = *reinterpret_cast<const uint4*>(a.mask + t0);
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < kCompactPer; ++i) mk[i] = static_cast<uint8_t>(wv[i / 4] >> (8 * (i % 4)));
    } else {
#pragma unroll
      for (int i = 0; i < kCompactPer; ++i) mk[i] = t0 + i < a.T ? a.mask[t0 + i] : 0;
    }
    int n = 0;
#pragma unroll
    for (int i = 0; i < kCompactPer; ++i) n += mk[i] != 0;
    // inclusive scan over the wave
    int incl = n;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) sh.wtot[tb][wave] = incl;
    __syncthreads();
    int64_t wbefore = 0, ctotal = 0;
#pragma unroll
    for (int w2 = 0; w2 < kRoundWaves; ++w2) {
      const int64_t v = sh.wtot[tb][w2];
      wbefore += w2 < wave ? v : 0;
      ctotal += v;
    }
    tb ^= 1;
    int64_t q = carry + wbefore + (incl - n);
#pragma unroll
    for (int i = 0; i < kCompactPer; ++i)
      if (mk[i]) a.pool_tok[q++] = static_cast<int32_t>(t0 + i);
    carry += ctotal;
  }
  __syncthreads();
  const int Q = static_cast<int>(carry);
  const bool in_lds = Q <= kRoundLdsCap;

  // state of pool token q
  for (int q = tid; q < Q; q += kRoundThreads) {
    const int64_t t = a.pool_tok[q];
    if (in_lds) {
      lsid[q] = a.packed[t];
      lmask[q] = a.mask[t];
    } else {
      a.gsid[q] = a.packed[t];
      a.gmask[q] = a.mask[t];
    }
  }
  if (tid == 0) sh.first = 0;
  __syncthreads();
  if (in_lds) round_hand_out(lsid, lmask, Q, pooled, a, load, sh);
  else round_hand_out(a.gsid, a.gmask, Q, pooled, a, load, sh);
  __syncthreads();

  // final ids of the pool tokens
  for (int q = tid; q < Q; q += kRoundThreads) {
    const int64_t t = a.pool_tok[q];
    a.packed[t] = in_lds ? lsid[q] : a.gsid[q];
  }
}

__global__ __launch_bounds__(256) void round_finish_kernel(RoundArgs a) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= a.T) return;
  const uint32_t m = a.mask[t];
  if (!m) return;
  const int k = a.k;
  const uint64_t w = a.packed[t];
  int ids[kMaxK];
  bool changed = false;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      ids[j] = a.ids[t * k + j];
      if ((m >> j) & 1u) {
        const int e = id_byte(w, j);
        if (e != ids[j]) {
          ids[j] = e;
          a.ids[t * k + j] = e;
          changed = true;
        }
      }
    }
  }
  if (!changed) return;
  const float mx = a.meta[t * 4 + 0], s = a.meta[t * 4 + 1];
  float p[kMaxK];
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) {
      p[j] = __expf(a.logits[t * a.E + ids[j]] - mx) / s;
      ps += p[j];
    }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) a.weights[t * k + j] = a.renorm ? p[j] / ps : p[j];
}

}  // namespace

size_t round_scratch_bytes(int64_t T) {
  const size_t t = static_cast<size_t>(T);
  return align_up(t + 16, 256) + align_up(t * 8, 256) + align_up(t * 4, 256) +
         align_up(t * 8, 256) + align_up(t, 256);
}

void carve_round(char* base, RoundArgs& a) {
  const size_t t = static_cast<size_t>(a.T);
  size_t o = 0;
  a.mask = reinterpret_cast<uint8_t*>(base + o);
  o += align_up(t + 16, 256);
  a.packed = reinterpret_cast<uint64_t*>(base + o);
  o += align_up(t * 8, 256);
  a.pool_tok = reinterpret_cast<int32_t*>(base + o);
  o += align_up(t * 4, 256);
  a.gsid = reinterpret_cast<uint64_t*>(base + o);
  o += align_up(t * 8, 256);
  a.gmask = reinterpret_cast<uint8_t*>(base + o);
}

hipError_t launch_token_round(const RoundArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.B < 1 || a.E < 1 || a.E > kMaxE || a.k < 1 || a.k > kMaxK || a.k > a.E ||
      a.T > INT32_MAX || !a.ids || !a.weights || !a.logits || !a.meta || !a.counts ||
      !a.offsets || !a.inv || !a.mask || !a.packed || !a.pool_tok || !a.gsid || !a.gmask)
    return hipErrorInvalidValue;
  // A tile larger than every count decides the same as T*k + 1 rows (every
  // count is below it either way), which keeps the hand-out's plans small.
  RoundArgs r = a;
  const int64_t M = a.T * a.k;
  if (static_cast<int64_t>(r.B) > M) r.B = static_cast<int>(M + 1);
  const unsigned grid = static_cast<unsigned>((a.T + 255) / 256);
  hipLaunchKernelGGL(round_mark_kernel, dim3(grid), dim3(256), 0, s, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(round_tiles_kernel, dim3(1), dim3(kRoundThreads), 0, s, r);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(round_finish_kernel, dim3(grid), dim3(256), 0, s, r);
  return hipGetLastError();
}

}  // namespace moe
