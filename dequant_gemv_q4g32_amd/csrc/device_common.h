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
// (v & mask) | t, and (v & mask) | 0x6400 in both fp16 halves.
__device__ __forceinline__ uint32_t pick_or(uint32_t v, uint32_t mask, uint32_t t) { return (v & mask) | t; }
__device__ __forceinline__ uint32_t pick(uint32_t v, uint32_t mask) { return (v & mask) | vreg(kMagic); }
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

// Sum over the 64 lanes of a wave; the total lands in lane 63 (other lanes hold partials).
__device__ __forceinline__ float wave_sum_to_63(float v) {
  v += dpp_move<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v += dpp_move<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v += dpp_move<0x141, 0xF>(v);   // row_half_mirror
  v += dpp_move<0x140, 0xF>(v);   // row_mirror: every lane of a row holds the row sum
  v += dpp_move<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
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
