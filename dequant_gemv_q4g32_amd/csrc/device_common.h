// Device helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp16 0x6400 is 1024.0; OR-ing a field n < 1024 into the mantissa gives 1024 + n exactly.
constexpr uint32_t kMagic = 0x64006400u;
// The same trick with the exponent lowered by a code's bit offset gives the code itself with
// unit weight: a code c at mantissa bits 3.. under 128.0 (0x5800) is 128 + c, at bits 4..
// under 64.0 (0x5400) is 64 + c, at bits 6.. under 16.0 (0x4C00) is 16 + c (all exact in fp16),
// so no activation or step has to be divided by the bit position's power of two.
constexpr uint32_t kMagic128 = 0x58005800u;
constexpr uint32_t kMagic64 = 0x54005400u;
constexpr uint32_t kMagic16 = 0x4C004C00u;
constexpr uint32_t kOnes = 0x3C003C00u;   // (1.0, 1.0) in fp16

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
}

// Bit-field constants as opaque register values. GFX9-family VOP3 encodings take no literal
// operand, so with literal masks the compiler would split (v & mask) | t into a v_and and a
// v_or with literals; with the mask in an SGPR and the or-operand in a VGPR, instruction
// selection emits a single v_and_or_b32.
__device__ __forceinline__ uint32_t sreg(uint32_t v) {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}
__device__ __forceinline__ uint32_t vreg(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}
#define QG_SMASK(v) ::qg::sreg(v)
// (v & mask) | t, and (v & mask) | magic (1024.0 by default) in both fp16 halves.
__device__ __forceinline__ uint32_t pick_or(uint32_t v, uint32_t mask, uint32_t t) { return (v & mask) | t; }
template <uint32_t MG = kMagic>
__device__ __forceinline__ uint32_t pick(uint32_t v, uint32_t mask) { return (v & mask) | vreg(MG); }
// Keeps v as computed: stops the compiler from re-associating (a & m) | ((b & m') | c) into
// and, and, or3 (three instructions) instead of two v_and_or_b32.
__device__ __forceinline__ uint32_t keep(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

__device__ __forceinline__ uint32_t rotr(uint32_t v, int s) { return __builtin_amdgcn_alignbit(v, v, s); }

__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ __forceinline__ float half_bits(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }


template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Cross-lane swaps of gfx950 (VOP1 v_permlane32_swap / v_permlane16_swap). permlane32: the
// upper 32 lanes of a trade places with the lower 32 lanes of b, so a = [a_lo, b_lo] and
// b = [a_hi, b_hi]. permlane16: the odd 16-lane rows of a trade places with the even rows of
// b, so a = [a0, b0, a2, b2] and b = [a1, b1, a3, b3]. Written as inline assembly: the
// compiler's builtins for them return one of the two swapped registers twice here. The
// instruction must not read a VGPR within 2 wait states of the VALU write to it (4 after a
// v_cmpx writes exec), which the compiler does not see inside the asm, so the asm waits 4;
// the trailing wait keeps a following DPP read of the results clear of the same rule.
__device__ __forceinline__ void lane_swap32(float &a, float &b) {
  asm volatile("s_nop 3\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lane_swap16(float &a, float &b) {
  asm volatile("s_nop 3\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// Sum over each 16-lane row; every lane of a row ends with the row's sum.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_move<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v += dpp_move<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v += dpp_move<0x141, 0xF>(v);   // row_half_mirror
  v += dpp_move<0x140, 0xF>(v);   // row_mirror
  return v;
}

// Wave sums of T = 1, 2, 4 or 8 values per lane at once. Halving the lanes and the values
// together (permlane32, then permlane16 swaps, each followed by one add per pair) costs
// T/2 + T/4 swaps and adds before the per-row DPP sums, instead of six DPP steps per value.
// Every value is summed in the same order whatever T is, ((v[l] + v[l+32]) + (v[l+16] +
// v[l+48])) and then the 16-lane DPP tree (T = 1 and 2 swap with copies of themselves),
// so a row's result does not depend on how many rows or activation rows share a wave.
// Afterwards lane l holds total wave_sum_value(T, l, j) in v[j]:
//   T = 1: every lane holds value 0 in v[0];
//   T = 2: rows 0 and 1 (lanes 0-31) hold value 0, rows 2 and 3 value 1, in v[0];
//   T >= 4: for j < T/4, every lane of row r = l/16 holds value 4j + {0, 2, 1, 3}[r] in v[j].
template <int T>
__device__ __forceinline__ void wave_sums(float *v) {
  static_assert(T == 1 || T == 2 || T == 4 || T == 8, "values per lane");
  if constexpr (T <= 2) {
    float a = v[0], b = T == 2 ? v[1] : v[0];
    lane_swap32(a, b);
    float c = a + b, d = c;                    // lanes 0-31: value 0, lanes 32-63: value T - 1
    lane_swap16(c, d);
    v[0] = row_sum16(c + d);
  } else {
#pragma unroll
    for (int p = 0; p < T / 2; ++p) {
      lane_swap32(v[2 * p], v[2 * p + 1]);
      v[p] = v[2 * p] + v[2 * p + 1];          // lanes 0-31: value 2p, lanes 32-63: 2p + 1
    }
#pragma unroll
    for (int q = 0; q < T / 4; ++q) {
      lane_swap16(v[2 * q], v[2 * q + 1]);
      v[q] = row_sum16(v[2 * q] + v[2 * q + 1]);
    }
  }
}

// Raw buffer loads: the plane base lives in a buffer resource (scalar registers), the row
// offset in a scalar soffset and only the lane offset in a vector register, so stepping
// from row to row costs scalar instructions only. Loads past num_records return zero.
// Planes whose bytes are each read by exactly one load instruction (codes, and per-unit scale
// words) use the non-temporal hint (nt): they stream through the caches without displacing
// anything. Metadata that several lanes, instructions or consecutive rows share (fp16
// super-scales, 6-bit field windows) uses the default policy so the shared lines stay cached.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;     // dword 3 of a raw buffer descriptor on GFX9 parts
constexpr int kNT = 2;                     // cache-policy operand: nt

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcFlags);
}
__device__ __forceinline__ u32x4 bld4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT));
}
// cached 128-bit load; an offset past the resource's range returns zeros
__device__ __forceinline__ u32x4 bld4c(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 bld2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNT));
}
// the same with the cache policy as a template argument (AUX = kNT streams, 0 caches)
template <int AUX> __device__ __forceinline__ u32x4 bldx4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}
template <int AUX> __device__ __forceinline__ u32x2 bldx2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX));
}
template <int AUX> __device__ __forceinline__ uint32_t bldx1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX);
}
__device__ __forceinline__ uint32_t bld1_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNT);
}
__device__ __forceinline__ uint32_t bld1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t bldh(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

__device__ __forceinline__ u32x4 ld4(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x2 ld2(const uint8_t *p) { return *reinterpret_cast<const u32x2 *>(p); }
__device__ __forceinline__ uint32_t ld1(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }
__device__ __forceinline__ uint16_t ldh(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }

}  // namespace qg
