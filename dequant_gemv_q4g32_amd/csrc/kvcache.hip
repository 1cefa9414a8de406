// 8-bit KV-cache group codec, gfx950: quantize on append, dequantize on read.
//
// Method: "二三五六位量化" page section 4.1 (the KV cache quantized to 8 bits with one fp16
// scale per 32 elements, about 1.06 bytes per element, half of fp16). Symmetric int8 codes in
// [-127, 127]; the scale d is the smallest fp16 at or above max|x| / 127, so every element is
// within d/2 of its decoded value; q = rint(x / d) on the exact quotient, halves to even (an
// all-zero group has d = 0 and q = 0); decode is d * q rounded once to fp16 and saturated at
// +-65504 (only d = 516, the scale of a group whose maximum is above 65469, reaches past it).
//
// Both kernels are streaming and HBM-bound: a lane handles 8 consecutive elements of a row
// (one 16-byte fp16 load or store, one 8-byte code load or store), so a wave moves 1 KB of
// fp16 per instruction; the 4 lanes of a 32-element group agree on its max with two DPP
// steps inside their quad.
#include <hip/hip_runtime.h>

#include "../../include/qgemv.h"
#include "device_common.h"
#include "launch.h"

namespace qg {

constexpr int kKvGroup = 32;

// Element offset of lane i's 8 elements in a row-strided fp16 matrix (rows of per_row lanes,
// leading dimension ld): no division when the rows are dense, a 32-bit one when the lane
// count fits, else a 64-bit one.
__device__ __forceinline__ int64_t strided_offset(int64_t i, int64_t per_row, int64_t ld, bool small) {
  if (ld == 8 * per_row) return 8 * i;
  int64_t r, c;
  if (small) {
    const uint32_t r32 = (uint32_t)i / (uint32_t)per_row;
    r = r32;
    c = (uint32_t)i - r32 * (uint32_t)per_row;
  } else {
    r = i / per_row;
    c = i % per_row;
  }
  return r * ld + 8 * c;
}
constexpr int kKvThreads = 256;

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_move<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_move<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
  return v;
}

__global__ __launch_bounds__(kKvThreads) void kv_quant_kernel(const uint16_t *src, int64_t ld, int64_t rows,
                                                             int64_t cols, int8_t *codes, uint16_t *scales) {
  const int64_t per_row = cols / 8;
  const int64_t lanes = rows * per_row;
  const int64_t i = (int64_t)blockIdx.x * kKvThreads + threadIdx.x;
  // lanes is a multiple of 4, so every quad of lanes is one whole group, live or not; codes
  // and scales are dense, so lane i's codes start at 8 i and its group is i / 4
  const bool live = i < lanes;
  u32x4 v = u32x4{0, 0, 0, 0};
  if (live) v = *reinterpret_cast<const u32x4 *>(src + strided_offset(i, per_row, ld, lanes < (int64_t(1) << 32)));
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = half_lo(w[j]);
    f[2 * j + 1] = half_hi(w[j]);
    amax = fmaxf(amax, fmaxf(fabsf(f[2 * j]), fabsf(f[2 * j + 1])));
  }
  amax = quad_max(amax);
  // d = smallest fp16 >= amax / 127 (t is finite and non-negative, at most 65504 / 127). The
  // fp32 quotient cannot cross an fp16 value: amax is fp16, so the exact quotient lies either
  // on an fp16 number or at least 2^-18 of its size away from every one, far beyond fp32's
  // rounding.
  const float t = amax / 127.0f;
  _Float16 h = (_Float16)t;
  if ((float)h < t) h = __builtin_bit_cast(_Float16, (uint16_t)(__builtin_bit_cast(uint16_t, h) + 1));
  const float d = (float)h;
  const float inv = d > 0.f ? 1.0f / d : 0.f;   // one division per group
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // x = a 2^i and d = b 2^k with a, b integers below 2^11 (fp16), so x / d is either a
    // half-integer or at least 1 / (2 b) >= 2^-12 away from every one, which is 1.9e-6 of the
    // largest quotient, 127.5. x * inv (inv = 1 / d rounded once) is within 2^-23 of x / d
    // relative, so q0 = rint(x * inv) is already the nearest integer except at an exact tie,
    // where it may be the odd neighbour. The remainder e = x - q0 d is exact in fp32 (x and d
    // are fp16, |q0| <= 127, and for q0 != 0 |x| >= d / 2, so e is a multiple of half of d's
    // last-place unit below 1.5 d: 13 bits); a tie is 2e = +-d, and then the even code is
    // q0 + sign(e). |x| <= 127 d keeps q within [-127, 127]. (d = 0: inv = 0, q = 0, e = 0.)
    float q = __builtin_rintf(f[j] * inv);
    const float e2 = 2.0f * __builtin_fmaf(-q, d, f[j]);
    const bool fix = __builtin_fabsf(e2) == d && ((int32_t)q & 1) != 0;
    q += fix ? __builtin_copysignf(1.0f, e2) : 0.0f;
    packed[j >> 2] |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * (j & 3));
  }
  if (!live) return;
  *reinterpret_cast<u32x2 *>(codes + 8 * i) = u32x2{packed[0], packed[1]};
  if ((i & 3) == 0) scales[i >> 2] = __builtin_bit_cast(uint16_t, h);
}

__global__ __launch_bounds__(kKvThreads) void kv_dequant_kernel(const int8_t *codes, const uint16_t *scales,
                                                               int64_t rows, int64_t cols, uint16_t *dst,
                                                               int64_t ld) {
  const int64_t per_row = cols / 8;
  const int64_t lanes = rows * per_row;
  const int64_t i = (int64_t)blockIdx.x * kKvThreads + threadIdx.x;
  if (i >= lanes) return;
  const u32x2 q = *reinterpret_cast<const u32x2 *>(codes + 8 * i);
  const float d = half_bits(scales[i >> 2]);
  const uint32_t qw[2] = {q.x, q.y};
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t word = qw[j >> 1] >> (16 * (j & 1));
    // d * q is exact in fp32; only 127 * 516 = 65532 lies past the fp16 maximum, saturated
    const float a = fminf(fmaxf((float)(int8_t)(word & 0xFFu) * d, -65504.f), 65504.f);
    const float b = fminf(fmaxf((float)(int8_t)((word >> 8) & 0xFFu) * d, -65504.f), 65504.f);
    out[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
  }
  *reinterpret_cast<u32x4 *>(dst + strided_offset(i, per_row, ld, lanes < (int64_t(1) << 32))) =
      u32x4{out[0], out[1], out[2], out[3]};
}

namespace {
bool kv_aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
}  // namespace

}  // namespace qg

using namespace qg;

extern "C" {

int qg_kv_quantize(const uint16_t *src, int64_t ld_src, int64_t rows, int64_t cols, int8_t *codes, uint16_t *scales,
                   void *stream) {
  if (rows < 0 || cols < 0 || cols % kKvGroup || (rows > 1 && ld_src < cols)) return QG_ERR_SHAPE;
  if (rows == 0 || cols == 0) return QG_OK;
  if (!src || !codes || !scales) return QG_ERR_NULL;
  if (!kv_aligned(src, 16) || (rows > 1 && ld_src % 8) || !kv_aligned(codes, 8) || !kv_aligned(scales, 2))
    return QG_ERR_ALIGN;
  const int64_t lanes = rows * (cols / 8);
  const int64_t blocks = (lanes + kKvThreads - 1) / kKvThreads;
  if (blocks > 0x7FFFFFFF) return QG_ERR_SHAPE;
  return launch(kv_quant_kernel, dim3((unsigned)blocks), dim3(kKvThreads), 0, static_cast<hipStream_t>(stream), src,
                rows > 1 ? ld_src : cols, rows, cols, codes, scales);
}

int qg_kv_dequantize(const int8_t *codes, const uint16_t *scales, int64_t rows, int64_t cols, uint16_t *dst,
                     int64_t ld_dst, void *stream) {
  if (rows < 0 || cols < 0 || cols % kKvGroup || (rows > 1 && ld_dst < cols)) return QG_ERR_SHAPE;
  if (rows == 0 || cols == 0) return QG_OK;
  if (!dst || !codes || !scales) return QG_ERR_NULL;
  if (!kv_aligned(dst, 16) || (rows > 1 && ld_dst % 8) || !kv_aligned(codes, 8) || !kv_aligned(scales, 2))
    return QG_ERR_ALIGN;
  const int64_t lanes = rows * (cols / 8);
  const int64_t blocks = (lanes + kKvThreads - 1) / kKvThreads;
  if (blocks > 0x7FFFFFFF) return QG_ERR_SHAPE;
  return launch(kv_dequant_kernel, dim3((unsigned)blocks), dim3(kKvThreads), 0, static_cast<hipStream_t>(stream), codes,
                scales, rows, cols, dst, rows > 1 ? ld_dst : cols);
}

}  // extern "C"
