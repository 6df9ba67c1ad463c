// MXFP8 quantization of bf16 or fp32 rows (gfx950).
//
// Page legend:
//   [Hunyuan page] "混合专家架构大模型Hunyuan-Large：原理剖析与实现机制"
//
// [Hunyuan page] §七.1 runs the experts in FP8.  The format here is OCP
// MXFP8 (Microscaling Formats v1.0): along each row, every block of 32
// consecutive values shares one E8M0 scale 2^e with e = floor(log2 amax) - 8
// (8 = largest exponent of e4m3), clamped to [-127, 127] (-127 for a block of
// zeros), and each value becomes the e4m3 code nearest to value / 2^e (ties
// to the even code, saturating at +-448).  Codes are stored [rows, cols],
// scales as biased exponents e + 127 in [rows, cols / 32].
//
// The work is HBM-bound (2 or 4 bytes in, 1 + 1/32 bytes out per value): a
// lane converts 8 consecutive values (one 16- or 32-byte load, one 8-byte
// store); the 4 lanes of a DPP quad hold one block and agree on its largest
// magnitude with two quad permutes, and the quad's first lane stores the
// scale byte.
#include "moe_internal.h"
#include "cdna4.h"

namespace moe {
namespace {

__device__ __forceinline__ float quad_max(float v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return v;
}

template <bool BF16>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const void* __restrict__ src, int64_t groups,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const int64_t g = blockIdx.x * 256LL + threadIdx.x;   // group of 8 consecutive values
  float v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = 0.f;
  if (g < groups) {
    if constexpr (BF16) {
      const uint4 q = static_cast<const uint4*>(src)[g];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[2 * u] = __uint_as_float(w[u] << 16);
        v[2 * u + 1] = __uint_as_float(w[u] & 0xFFFF0000u);
      }
    } else {
      const float4 a = static_cast<const float4*>(src)[2 * g];
      const float4 b = static_cast<const float4*>(src)[2 * g + 1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  }
  float m = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) m = __builtin_fmaxf(m, __builtin_fabsf(v[u]));
  // groups is a multiple of 4 and blocks start at multiples of 4 lanes, so a
  // quad is either one whole block or wholly past the end
  m = quad_max(m);
  const int ex = mx_block_exp(m);
  const float sc = mx_inv_scale(ex);
  if (g < groups) {
    uint2 o;
    o.x = mx_encode4(v[0], v[1], v[2], v[3], sc);
    o.y = mx_encode4(v[4], v[5], v[6], v[7], sc);
    reinterpret_cast<uint2*>(codes)[g] = o;
    if ((g & 3) == 0) scales[g >> 2] = static_cast<uint8_t>(ex + 127);
  }
}

// Stage-major scale words: thread r copies the S = K/128 words of its source
// row to word column r of each stage, reading 16 bytes at a time when the
// rows allow it (S % 4 == 0, i.e. K a multiple of 512, and a 16-byte aligned
// source; single words otherwise); the stores of a wave cover 256 contiguous
// bytes.
__global__ __launch_bounds__(256) void mx_scale_words_kernel(const uint32_t* __restrict__ src, int64_t R,
                                                             int S, const int32_t* __restrict__ rows,
                                                             int div, uint32_t* __restrict__ dst) {
  const int64_t r = blockIdx.x * 256LL + threadIdx.x;
  if (r >= R) return;
  const int64_t sr = rows ? rows[r] / div : r;
  const uint32_t* p = src + sr * S;
  if (S % 4 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    for (int st = 0; st < S; st += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(p + st);
      dst[st * R + r] = q.x;
      dst[(st + 1) * R + r] = q.y;
      dst[(st + 2) * R + r] = q.z;
      dst[(st + 3) * R + r] = q.w;
    }
  } else {
    for (int st = 0; st < S; ++st) dst[st * R + r] = p[st];
  }
}

}  // namespace

hipError_t launch_mx_scale_words(const uint8_t* scales, int64_t R, int K, const int32_t* rows, int div,
                                 uint32_t* dst, hipStream_t s) {
  if (R < 0 || K <= 0 || K % (4 * kMxBlock) || div < 1) return hipErrorInvalidValue;
  if (R == 0) return hipSuccess;
  const int64_t blocks = (R + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_scale_words_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(scales), R, K / (4 * kMxBlock), rows, div, dst);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* src, bool bf16, int64_t rows, int cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  if (rows < 0 || cols <= 0 || cols % kMxBlock) return hipErrorInvalidValue;
  const int64_t groups = rows * static_cast<int64_t>(cols) / 8;
  if (groups == 0) return hipSuccess;
  const int64_t blocks = (groups + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(mx_quantize_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                       src, groups, codes, scales);
  else
    hipLaunchKernelGGL(mx_quantize_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                       src, groups, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
