// Per-format decode-and-dot of one 64-weight lane unit (see layout.h for the bit placement).
//
// Terms: a "pair" is two consecutive weights (2t, 2t+1) of the unit, multiplied by one
// activation dword (x[2t], x[2t+1]) with v_dot2_f32_f16. A unit has 32 pairs. With S = 1 a
// lane owns the whole unit; with S = 2 two lanes share it and lane half h owns pairs
// pidx(h, p), p < 16 (the first or second 32 weights for every format but q2sb, whose
// halves interleave; see pidx). M activation rows share every decoded code.
//
// Each code pair is turned into fp16 (1024 + p*c_a, 1024 + p*c_b) by one v_and_or_b32, for
// a power of two p (the "class" of the bit position it sits at). Per class and sub-block
// the products are accumulated in fp32, and the 1024s and the code offsets cancel against
// per-lane constants built from sums of x ("kc"), which the accumulators start from. This
// is the sum-of-x rewrite of "二三五六位量化" section 3.3: s * sum(q x) + m * sum(x).
#pragma once
#include "device_common.h"

namespace qg {

struct Lane {
  rsrc_t rs[4];
  uint32_t prb[4];
  uint32_t off[4];
  uint32_t sh;              // bit offset of this unit's 6-bit fields in its 8-byte window
  uint32_t half16;          // offset of the second halves in a split 16-byte-half plane row
  uint32_t half4;           // same for the split q4g32 scale plane
  uint32_t half8;           // same for the split q4g16 scale plane (8-byte halves)
  int h = 0;                // the lane's half of its unit when two lanes share a unit
  __device__ uint32_t row(int p, int64_t r) const { return (uint32_t)r * prb[p]; }
  __device__ void set_halves(int64_t units) {
    half16 = (uint32_t)(units * 16);
    half4 = (uint32_t)(units * 4);
    half8 = (uint32_t)(units * 8);
  }
};

// 6-bit sub-scale fields (12 bytes per super-block; a unit owns 3 of them, bytes 3q..3q+2 for
// quarter q) are read as an 8-byte window starting at byte 4*max(0, q-1) and shifted right by
// (24q) mod 32 bits: 0, 24, 16, 8 for q = 0..3. The window of q = 3 reaches 4 bytes past the
// super-block, which is in bounds (the next super-block, or the plane that follows, or
// buffer range checking returns zero).
__device__ __forceinline__ uint32_t fields_off(int64_t u) {
  const uint32_t q = (uint32_t)(u & 3);
  return (uint32_t)((u >> 2) * 12) + (q ? 4 * (q - 1) : 0);
}
__device__ __forceinline__ uint32_t fields_sh(int64_t u) { return (uint32_t)((24 * (u & 3)) & 31); }
__device__ __forceinline__ uint32_t fields24(const Lane &L, int p, int64_t r) {
  const uint32_t lo = bld1(L.rs[p], L.off[p], L.row(p, r));
  const uint32_t hi = bld1(L.rs[p], L.off[p] + 4, L.row(p, r));
  return __builtin_amdgcn_alignbit(hi, lo, L.sh);   // low 24 bits are the unit's fields
}

__device__ __forceinline__ uint32_t sel(bool c, uint32_t a, uint32_t b) { return c ? a : b; }

// ---- decode to fp16 weights (for the MFMA path): from a code pair P = (B + c_a, B + c_b)
// (a class magic B: 1024, 128, 64 or 16) to the fp16 pair of w_hat.
// Symmetric formats: w_hat = step * (c - o) = (P - (B + o)) * step. The subtraction is exact
// (small integers); the product is one fp16 rounding of a value whose factor step was itself
// rounded to fp16 once. A step below 2^-14 (an fp16 subnormal) keeps only 2^-25 absolute.
__device__ __forceinline__ uint32_t sym_pair(uint32_t P, _Float16 off, _Float16 mul) {
  const h2_t v = __builtin_bit_cast(h2_t, P);
  const h2_t o = {off, off}, m = {mul, mul};
  return __builtin_bit_cast(uint32_t, (v + o) * m);
}
// Asymmetric formats: w_hat = step * c - off = P * (step / p) + add, add = -(1024 step / p + off),
// in fp32 (so that the cancellation of 1024 * step / p is exact up to fp32 rounding of add),
// then one rounding to fp16.
__device__ __forceinline__ uint32_t asym_pair(uint32_t P, float mul, float add) {
  const h2_t r = {(_Float16)__builtin_fmaf(half_lo(P), mul, add), (_Float16)__builtin_fmaf(half_hi(P), mul, add)};
  return __builtin_bit_cast(uint32_t, r);
}

template <int F> struct Unit;

// Super-scales d, dmin of the super-block formats: fp16 bits, or bf16 bits (the upper half of
// an fp32) in the "_bf16" variants; both widen to fp32 exactly.
template <bool BF> __device__ __forceinline__ float ss_lo(uint32_t v) {
  if constexpr (BF) return __builtin_bit_cast(float, v << 16);
  else return half_lo(v);
}
template <bool BF> __device__ __forceinline__ float ss_hi(uint32_t v) {
  if constexpr (BF) return __builtin_bit_cast(float, v & 0xFFFF0000u);
  else return half_hi(v);
}
template <bool BF> __device__ __forceinline__ float ss_one(uint16_t v) {
  if constexpr (BF) return __builtin_bit_cast(float, (uint32_t)v << 16);
  else return half_bits(v);
}

// ---- INT4 groups of G = 16, 32, 64 or 128 weights, one fp32 scale each. A unit (64
// weights, 8 code dwords; dword i holds weights 8i..8i+7) spans 64 / G groups, or half a
// group of 128. With S = 2 a lane owns half a unit (4 dwords, loaded alone). The lane's
// groups ("lane groups") cover its dwords in runs of G / 8 (at most its 8 / S dwords); their
// scales are loaded into s[0..], in order.
// NKS(S): per-lane constants per activation row, one per lane group.
template <int G> struct UnitQ4 {
  static_assert(G == 16 || G == 32 || G == 64 || G == 128, "INT4 group size");
  static constexpr int NG = G <= 64 ? 64 / G : 1;   // scales a unit touches
  static constexpr int NK = NG;                     // constants per activation row (S = 1)
  __host__ __device__ static constexpr int NKS(int S) { return NG / S > 0 ? NG / S : 1; }
  static constexpr int DPG = G / 8;                 // code dwords per group
  template <int S> static constexpr int dpl() { return DPG < 8 / S ? DPG : 8 / S; }   // dwords per lane group
  struct Raw { u32x4 c0, c1; float s[NG]; };
  __device__ static int pidx(int h, int p, int S) { return S == 1 ? p : 16 * h + p; }
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16);
    off[1] = (uint32_t)(G == 16 ? u * 8 : G == 128 ? (u >> 1) * 4 : u * 4);
  }
  // S = 2: the lane's own half only (half L.h of the unit), into c0 and s[0..NKS(2))
  template <int AUX = kNT, int S = 1> __device__ static void load(Raw &q, const Lane &L, int64_t r, bool half) {
    const uint32_t r0 = L.row(0, r), r1 = L.row(1, r);
    if constexpr (S == 2) {
      // (q4g32) a half unit (k % 64 == 32) has no second group: that lane re-reads the first
      // and meets zero activations
      const bool second = L.h && !half;
      q.c0 = bldx4<AUX>(L.rs[0], L.off[0] + (second ? L.half16 : 0u), r0);
    } else {
      q.c0 = bldx4<AUX>(L.rs[0], L.off[0], r0);
      // (q4g32) a half unit has one group; its second group's activations are zero
      q.c1 = bldx4<AUX>(L.rs[0], L.off[0] + (half ? 0u : L.half16), r0);
    }
    // Scales as separate 32-bit loads or as integer pairs passed through keep(): this
    // toolchain narrows a multi-dword buffer load whose elements are bit-cast to float to its
    // first dword and reuses that dword for the second element.
    if constexpr (G == 32) {
      if constexpr (S == 2) {
        q.s[0] = __builtin_bit_cast(float, bld1(L.rs[1], L.off[1] + (L.h && !half ? L.half4 : 0u), r1));
      } else {
        q.s[0] = __builtin_bit_cast(float, bld1(L.rs[1], L.off[1], r1));
        q.s[1] = __builtin_bit_cast(float, bld1(L.rs[1], L.off[1] + (half ? 0u : L.half4), r1));
      }
    } else if constexpr (G == 16) {
#pragma unroll
      for (int hh = 0; hh < 2 / S; ++hh) {
        const uint32_t o = L.off[1] + (S == 2 ? (L.h ? L.half8 : 0u) : (hh ? L.half8 : 0u));
        const u32x2 v = bldx2<0>(L.rs[1], o, r1);
        q.s[2 * hh] = __builtin_bit_cast(float, keep(v.x));
        q.s[2 * hh + 1] = __builtin_bit_cast(float, keep(v.y));
      }
    } else {
      q.s[0] = __builtin_bit_cast(float, bld1(L.rs[1], L.off[1], r1));
    }
  }
  // xp: the lane's pairs (32 / S; dword i's pairs are 4i..4i+3, classes 1, 16, 1, 16);
  // kc: one constant per lane group
  template <int S> __device__ static void prep(uint32_t *xp, float *kc) {
    constexpr int D = dpl<S>();
#pragma unroll
    for (int g = 0; g < NKS(S); ++g) {
      float x1 = 0.f, x16 = 0.f;
#pragma unroll
      for (int i = D * g; i < D * (g + 1); ++i) {
        x1 = dot2(xp[4 * i + 0], kOnes, x1);
        x1 = dot2(xp[4 * i + 2], kOnes, x1);
        x16 = dot2(xp[4 * i + 1], kOnes, x16);
        x16 = dot2(xp[4 * i + 3], kOnes, x16);
      }
      kc[g] = -(1032.0f * x1 + 72.0f * x16);   // sum (u - 8) x = A1 + A16/16, A1 starting here
    }
  }
  template <int M, int S>
  __device__ static void dot(const Raw &q, int h, const uint32_t (*xp)[32 / S], const float (*kc)[NKS(S)], float *out) {
    constexpr int D = dpl<S>();
    // (S = 2 loaded the lane's own half into c0)
    const uint32_t d[8] = {q.c0.x, q.c0.y, q.c0.z, q.c0.w, S == 1 ? q.c1.x : 0u, S == 1 ? q.c1.y : 0u,
                           S == 1 ? q.c1.z : 0u, S == 1 ? q.c1.w : 0u};
#pragma unroll
    for (int g = 0; g < NKS(S); ++g) {
      float a1[M], a16[M];
#pragma unroll
      for (int m = 0; m < M; ++m) { a1[m] = kc[m][g]; a16[m] = 0.f; }
#pragma unroll
      for (int i = D * g; i < D * (g + 1); ++i) {
        const uint32_t v = d[i], v8 = v >> 8;
        const uint32_t p0 = pick(v, QG_SMASK(0x000F000Fu)), p1 = pick(v, QG_SMASK(0x00F000F0u));
        const uint32_t p2 = pick(v8, QG_SMASK(0x000F000Fu)), p3 = pick(v8, QG_SMASK(0x00F000F0u));
#pragma unroll
        for (int m = 0; m < M; ++m) {
          a1[m] = dot2(p0, xp[m][4 * i + 0], a1[m]);
          a16[m] = dot2(p1, xp[m][4 * i + 1], a16[m]);
          a1[m] = dot2(p2, xp[m][4 * i + 2], a1[m]);
          a16[m] = dot2(p3, xp[m][4 * i + 3], a16[m]);
        }
      }
      const float scale = q.s[g];
#pragma unroll
      for (int m = 0; m < M; ++m) out[m] = __builtin_fmaf(scale, __builtin_fmaf(a16[m], 0.0625f, a1[m]), out[m]);
    }
  }
  // fp16 w_hat of the 16 pairs of half h (dwords 4h..4h+3), in local pair order; S = 2: q
  // holds only that half (loaded by load<AUX, 2>)
  template <int S = 1> __device__ static void wide(const Raw &q, int h, uint32_t *out) {
    const u32x4 c0 = q.c0, c1 = S == 1 ? q.c1 : q.c0;
    const uint32_t dw[4] = {sel(S == 1 && h, c1.x, c0.x), sel(S == 1 && h, c1.y, c0.y), sel(S == 1 && h, c1.z, c0.z),
                            sel(S == 1 && h, c1.w, c0.w)};
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (G == 16) {
        // dwords 0, 1 of the half: group 2h (lane scale 0 when S = 2); dwords 2, 3: 2h + 1
        const int j = i >> 1;
        sc[i] = S == 1 ? __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.s[2 + j]),
                                                       __builtin_bit_cast(uint32_t, q.s[j])))
                       : q.s[j];
      } else if constexpr (G == 32) {
        sc[i] = S == 1 ? __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.s[NG - 1]),
                                                       __builtin_bit_cast(uint32_t, q.s[0])))
                       : q.s[0];
      } else {
        sc[i] = q.s[0];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 m1 = (_Float16)sc[i];
      const uint32_t v = dw[i], v8 = v >> 8;
      out[4 * i + 0] = sym_pair(pick(v, QG_SMASK(0x000F000Fu)), (_Float16)-1032.0f, m1);
      out[4 * i + 1] = sym_pair(pick<kMagic64>(v, QG_SMASK(0x00F000F0u)), (_Float16)-72.0f, m1);
      out[4 * i + 2] = sym_pair(pick(v8, QG_SMASK(0x000F000Fu)), (_Float16)-1032.0f, m1);
      out[4 * i + 3] = sym_pair(pick<kMagic64>(v8, QG_SMASK(0x00F000F0u)), (_Float16)-72.0f, m1);
    }
  }
};
template <> struct Unit<4> : UnitQ4<32> {};
template <> struct Unit<7> : UnitQ4<16> {};
template <> struct Unit<8> : UnitQ4<64> {};
template <> struct Unit<9> : UnitQ4<128> {};

// ---- INT4 groups of 32 with fp16 scales (q4g32h): q4g32's codes and arithmetic; the unit's
// two scales are one dword of fp16 pairs (group order), which both lanes of a shared unit
// read.
template <> struct Unit<kQ4G32H> : UnitQ4<32> {
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16);
    off[1] = (uint32_t)(u * 4);
  }
  template <int AUX = kNT, int S = 1> __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    const uint32_t r0 = L.row(0, r);
    if constexpr (S == 2) {
      q.c0 = bldx4<AUX>(L.rs[0], L.off[0] + (L.h ? L.half16 : 0u), r0);
    } else {
      q.c0 = bldx4<AUX>(L.rs[0], L.off[0], r0);
      q.c1 = bldx4<AUX>(L.rs[0], L.off[0] + L.half16, r0);
    }
    const uint32_t sc = bld1(L.rs[1], L.off[1], L.row(1, r));
    if constexpr (S == 2) {
      q.s[0] = L.h ? half_hi(sc) : half_lo(sc);
    } else {
      q.s[0] = half_lo(sc);
      q.s[1] = half_hi(sc);
    }
  }
};

// ---- INT4 asymmetric, groups of 32 (q4a32): the q4g32 code and scale planes with unsigned
// codes c, and a plane of uint8 zero points z (2 bytes per unit, group order):
// w_hat = s * (c - z), so a group's sum of w_hat * x is s * (sum c x - z * sum x). With S = 2
// a lane owns one group (half h of the unit).
template <> struct Unit<kQ4A32> {
  static constexpr int NK = 4;
  __host__ __device__ static constexpr int NKS(int S) { return NK / S; }
  struct Raw { u32x4 c0, c1; float s[2]; uint32_t z; };
  __device__ static int pidx(int h, int p, int S) { return S == 1 ? p : 16 * h + p; }
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16); off[1] = (uint32_t)(u * 4); off[2] = (uint32_t)(u * 2);
  }
  // S = 2: the lane's own group only, into c0 and s[0]
  template <int AUX = kNT, int S = 1> __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    const uint32_t r0 = L.row(0, r), r1 = L.row(1, r);
    if constexpr (S == 2) {
      q.c0 = bldx4<AUX>(L.rs[0], L.off[0] + (L.h ? L.half16 : 0u), r0);
      q.s[0] = __builtin_bit_cast(float, bld1(L.rs[1], L.off[1] + (L.h ? L.half4 : 0u), r1));
    } else {
      q.c0 = bldx4<AUX>(L.rs[0], L.off[0], r0);
      q.c1 = bldx4<AUX>(L.rs[0], L.off[0] + L.half16, r0);
      q.s[0] = __builtin_bit_cast(float, bld1(L.rs[1], L.off[1], r1));
      q.s[1] = __builtin_bit_cast(float, bld1(L.rs[1], L.off[1] + L.half4, r1));
    }
    q.z = bldh(L.rs[2], L.off[2], L.row(2, r));
  }
  // kc layout (S = 1): [start g0, start g1, sum x g0, sum x g1]; (S = 2): [start, sum x]
  template <int S> __device__ static void prep(uint32_t *xp, float *kc) {
#pragma unroll
    for (int g = 0; g < 2 / S; ++g) {
      float x1 = 0.f, x16 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x1 = dot2(xp[16 * g + 4 * i + 0], kOnes, x1);
        x1 = dot2(xp[16 * g + 4 * i + 2], kOnes, x1);
        x16 = dot2(xp[16 * g + 4 * i + 1], kOnes, x16);
        x16 = dot2(xp[16 * g + 4 * i + 3], kOnes, x16);
      }
      kc[g] = -(1024.0f * x1 + 64.0f * x16);   // A1 + A16 / 16 = sum c x, A1 starting here
      kc[2 / S + g] = x1 + x16;
    }
  }
  template <int M, int S>
  __device__ static void dot(const Raw &q, int h, const uint32_t (*xp)[32 / S], const float (*kc)[NKS(S)], float *out) {
    const uint32_t d[8] = {q.c0.x, q.c0.y, q.c0.z, q.c0.w, S == 1 ? q.c1.x : 0u, S == 1 ? q.c1.y : 0u,
                           S == 1 ? q.c1.z : 0u, S == 1 ? q.c1.w : 0u};
#pragma unroll
    for (int g = 0; g < 2 / S; ++g) {
      float a1[M], a16[M];
#pragma unroll
      for (int m = 0; m < M; ++m) { a1[m] = kc[m][g]; a16[m] = 0.f; }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t v = d[4 * g + i], v8 = v >> 8;
        const uint32_t p0 = pick(v, QG_SMASK(0x000F000Fu)), p1 = pick(v, QG_SMASK(0x00F000F0u));
        const uint32_t p2 = pick(v8, QG_SMASK(0x000F000Fu)), p3 = pick(v8, QG_SMASK(0x00F000F0u));
#pragma unroll
        for (int m = 0; m < M; ++m) {
          a1[m] = dot2(p0, xp[m][16 * g + 4 * i + 0], a1[m]);
          a16[m] = dot2(p1, xp[m][16 * g + 4 * i + 1], a16[m]);
          a1[m] = dot2(p2, xp[m][16 * g + 4 * i + 2], a1[m]);
          a16[m] = dot2(p3, xp[m][16 * g + 4 * i + 3], a16[m]);
        }
      }
      // s * (sum c x - z * sum x), the difference taken before the scale: a code equal to the
      // zero point then contributes exactly 0, as its w_hat does
      const float scale = q.s[g];
      const float zf = (float)((q.z >> (8 * (S == 1 ? g : h))) & 0xFFu);
#pragma unroll
      for (int m = 0; m < M; ++m)
        out[m] = __builtin_fmaf(scale, __builtin_fmaf(-zf, kc[m][2 / S + g], __builtin_fmaf(a16[m], 0.0625f, a1[m])), out[m]);
    }
  }
  // fp16 w_hat of the 16 pairs of half h (group h); S = 2: q holds only that group
  template <int S = 1> __device__ static void wide(const Raw &q, int h, uint32_t *out) {
    const u32x4 c0 = q.c0, c1 = S == 1 ? q.c1 : q.c0;
    const uint32_t dw[4] = {sel(S == 1 && h, c1.x, c0.x), sel(S == 1 && h, c1.y, c0.y), sel(S == 1 && h, c1.z, c0.z),
                            sel(S == 1 && h, c1.w, c0.w)};
    const float sc = S == 1 ? __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.s[1]),
                                                            __builtin_bit_cast(uint32_t, q.s[0])))
                            : q.s[0];
    const float zf = (float)((q.z >> (8 * h)) & 0xFFu);
    // (P - (B + z)) is c - z exactly; times s rounded to fp16
    const _Float16 m1 = (_Float16)sc;
    const _Float16 o1 = (_Float16)(-1024.0f - zf), o16 = (_Float16)(-64.0f - zf);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = dw[i], v8 = v >> 8;
      out[4 * i + 0] = sym_pair(pick(v, QG_SMASK(0x000F000Fu)), o1, m1);
      out[4 * i + 1] = sym_pair(pick<kMagic64>(v, QG_SMASK(0x00F000F0u)), o16, m1);
      out[4 * i + 2] = sym_pair(pick(v8, QG_SMASK(0x000F000Fu)), o1, m1);
      out[4 * i + 3] = sym_pair(pick<kMagic64>(v8, QG_SMASK(0x00F000F0u)), o16, m1);
    }
  }
};

// ---- 2-bit super-block: a unit is a quarter super-block (4 sub-blocks of 16). Sub-block j
// sits at class 4^j in every dword; with S = 2 lane half h owns dwords 2h, 2h+1, i.e. pairs
// r = 4h..4h+3 of every sub-block.
template <bool BF> struct UnitQ2 {
  static constexpr int NK = 4;
  __host__ __device__ static constexpr int NKS(int) { return 4; }  // every half meets all 4 sub-blocks
  struct Raw { u32x4 c; uint32_t sc, dd; };
  __device__ static int pidx(int h, int p, int S) { return S == 1 ? p : 8 * (p >> 2) + 4 * h + (p & 3); }
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16); off[1] = (uint32_t)(u * 4); off[2] = (uint32_t)((u >> 2) * 4);
  }
  // S = 2: only the lane's own code dwords 2h, 2h+1, into c.x, c.y
  template <int AUX = kNT, int S = 1> __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    if constexpr (S == 2) {
      const u32x2 c = bldx2<AUX>(L.rs[0], L.off[0] + 8u * L.h, L.row(0, r));
      q.c.x = c.x;
      q.c.y = c.y;
    } else {
      q.c = bldx4<AUX>(L.rs[0], L.off[0], L.row(0, r));
    }
    q.sc = bldx1<AUX>(L.rs[1], L.off[1], L.row(1, r));
    q.dd = bld1(L.rs[2], L.off[2], L.row(2, r));
  }
  // kc[j]: sum of x over the lane's part of sub-block j (local pairs (8/S) j .. (8/S) j + 8/S - 1)
  template <int S> __device__ static void prep(uint32_t *xp, float *kc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < 8 / S; ++r) s = dot2(xp[(8 / S) * j + r], kOnes, s);
      kc[j] = s;
    }
  }
  // Sub-block j sits at class 4^j: A_j = 1024 sum x + 4^j sum c x, so with sc'_j = sc_j / 4^j
  //   y += d sum_j sc'_j A_j - sum_j (1024 d sc'_j + dmin m_j) sum x_j.
  template <int M, int S>
  __device__ static void dot(const Raw &q, int h, const uint32_t (*xp)[32 / S], const float (*kc)[NKS(S)], float *out) {
    float A[M][4];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) A[m][j] = 0.f;
    const uint32_t d[4] = {q.c.x, q.c.y, q.c.z, q.c.w};
#pragma unroll
    for (int ii = 0; ii < 4 / S; ++ii) {
      const uint32_t v = d[ii];                // (S = 2 loaded the lane's dwords into d[0], d[1])
      const uint32_t v8 = v >> 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t pa = pick(v, QG_SMASK(0x00030003u << (2 * j))), pb = pick(v8, QG_SMASK(0x00030003u << (2 * j)));
#pragma unroll
        for (int m = 0; m < M; ++m) {
          A[m][j] = dot2(pa, xp[m][(8 / S) * j + 2 * ii], A[m][j]);
          A[m][j] = dot2(pb, xp[m][(8 / S) * j + 2 * ii + 1], A[m][j]);
        }
      }
    }
    const uint32_t s = q.sc;
    const float inv4[4] = {1.0f, 0.25f, 0.0625f, 0.015625f};
    const float dv = ss_lo<BF>(q.dd), dm = ss_hi<BF>(q.dd);
    float scj[4], cj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      scj[j] = dv * ((float)((s >> (8 * j)) & 15u) * inv4[j]);
      cj[j] = __builtin_fmaf(1024.0f, scj[j], dm * (float)((s >> (8 * j + 4)) & 15u));
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float acc = out[m];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = __builtin_fmaf(scj[j], A[m][j], acc);
        acc = __builtin_fmaf(-cj[j], kc[m][j], acc);
      }
      out[m] = acc;
    }
  }
  // fp16 w_hat of the 16 pairs of half h (dwords 2h, 2h+1), in local pair order; S = 2: q
  // holds only those dwords, in c.x and c.y
  template <int S = 1> __device__ static void wide(const Raw &q, int h, uint32_t *out) {
    const uint32_t d[4] = {q.c.x, q.c.y, q.c.z, q.c.w};
    const float inv4[4] = {1.0f, 0.25f, 0.0625f, 0.015625f};
    const float dv = ss_lo<BF>(q.dd), dm = ss_hi<BF>(q.dd);
    float mul[4], add[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mul[j] = dv * (float)((q.sc >> (8 * j)) & 15u) * inv4[j];
      add[j] = -__builtin_fmaf(1024.0f, mul[j], dm * (float)((q.sc >> (8 * j + 4)) & 15u));
    }
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const uint32_t v = S == 1 ? sel(h, d[2 + ii], d[ii]) : d[ii], v8 = v >> 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[4 * j + 2 * ii] = asym_pair(pick(v, QG_SMASK(0x00030003u << (2 * j))), mul[j], add[j]);
        out[4 * j + 2 * ii + 1] = asym_pair(pick(v8, QG_SMASK(0x00030003u << (2 * j))), mul[j], add[j]);
      }
    }
  }
};
template <> struct Unit<2> : UnitQ2<false> {};
template <> struct Unit<12> : UnitQ2<true> {};

// ---- 3-bit super-block: a unit is two chunks of 32 codes (sub-blocks a, b each); with S = 2
// lane half h owns chunk h.
template <bool BF> struct UnitQ3 {
  static constexpr int NK = 4;
  __host__ __device__ static constexpr int NKS(int S) { return NK / S; }
  struct Raw { u32x4 a; u32x2 b; uint32_t f; uint16_t d; };
  __device__ static int pidx(int h, int p, int S) { return S == 1 ? p : 16 * h + p; }
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16); off[1] = (uint32_t)(u * 8); off[2] = fields_off(u); off[3] = (uint32_t)((u >> 2) * 2);
  }
  template <int AUX = kNT, int S = 1> __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    q.a = bldx4<AUX>(L.rs[0], L.off[0], L.row(0, r));
    q.b = bldx2<AUX>(L.rs[1], L.off[1], L.row(1, r));
    q.f = fields24(L, 2, r);
    q.d = bldh(L.rs[3], L.off[3], L.row(3, r));
  }
  // The pairs of sub-block a sit at bit classes 1 (pairs 0..5) and 8 (6, 7), those of b at
  // classes 8 (8..11) and 64 (12..15). Each class has its own magic (1024, 128, 16), so every
  // pair decodes to (B + c_a, B + c_b) with unit weight and each sub-block accumulates in one
  // register from the activations as given: sum P x = sum c x + 1024 X1 + 128 X8 (a),
  // sum c x + 128 X8 + 16 X64 (b), with X the sums of x over each class.
  template <int S> __device__ static void prep(uint32_t *xp, float *kc) {
#pragma unroll
    for (int c = 0; c < 2 / S; ++c) {
      uint32_t *x = xp + 16 * c;
      float a1 = 0.f, a8 = 0.f, b8 = 0.f, b64 = 0.f;
#pragma unroll
      for (int r = 0; r < 6; ++r) a1 = dot2(x[r], kOnes, a1);
#pragma unroll
      for (int r = 6; r < 8; ++r) a8 = dot2(x[r], kOnes, a8);
#pragma unroll
      for (int r = 8; r < 12; ++r) b8 = dot2(x[r], kOnes, b8);
#pragma unroll
      for (int r = 12; r < 16; ++r) b64 = dot2(x[r], kOnes, b64);
      kc[2 * c] = -(1028.0f * a1 + 132.0f * a8);       // start of a: sum (c - 4) x
      kc[2 * c + 1] = -(132.0f * b8 + 20.0f * b64);    // start of b: sum (c - 4) x
    }
  }
  // One chunk: three dwords e0..e2 holding 32 codes -> the 16 fp16 pairs of its two
  // sub-blocks (a: P[0..7], classes 1 x6 and 8 x2; b: P[8..15], classes 8 x4 and 64 x4),
  // each (B + c_a, B + c_b) with B = 1024, 128, 16 for classes 1, 8, 64.
  __device__ static void chunk_pairs(uint32_t e0, uint32_t e1, uint32_t e2, uint32_t *P) {
    const uint32_t e09 = e0 >> 9, e19 = e1 >> 9, e29 = e2 >> 9;
    P[0] = pick(e0, QG_SMASK(0x00070007u));
    P[1] = pick(e09, QG_SMASK(0x00070007u));
    P[2] = pick(e1, QG_SMASK(0x00070007u));
    P[3] = pick(e19, QG_SMASK(0x00070007u));
    P[4] = pick(e2, QG_SMASK(0x00070007u));
    P[5] = pick(e29, QG_SMASK(0x00070007u));
    P[6] = pick<kMagic128>(e0, QG_SMASK(0x00380038u));
    P[7] = pick<kMagic128>(e09, QG_SMASK(0x00380038u));
    P[8] = pick<kMagic128>(e1, QG_SMASK(0x00380038u));
    P[9] = pick<kMagic128>(e19, QG_SMASK(0x00380038u));
    P[10] = pick<kMagic128>(e2, QG_SMASK(0x00380038u));
    P[11] = pick<kMagic128>(e29, QG_SMASK(0x00380038u));
    P[12] = pick<kMagic16>(e0, QG_SMASK(0x01C001C0u));
    P[13] = pick<kMagic16>(e1, QG_SMASK(0x01C001C0u));
    P[14] = pick<kMagic16>(e2, QG_SMASK(0x01C001C0u));
    uint32_t t = keep(pick<kMagic16>(e09, QG_SMASK(0x00400040u)));    // bit 15 of e0 -> 6, bit 31 -> 22
    t = keep(pick_or(e1 >> 8, QG_SMASK(0x00800080u), t));    // bit 15 of e1 -> 7
    P[15] = pick_or(e2 >> 7, QG_SMASK(0x01000100u), t);      // bit 15 of e2 -> 8
  }
  // sum (c - 4) x over sub-block a (sa) and over b (sb) for one activation row (x prepared)
  __device__ static void chunk_dot(const uint32_t *P, const uint32_t *x, float ka, float kb, float &sa, float &sb) {
    float a = ka, b = kb;
#pragma unroll
    for (int r = 0; r < 8; ++r) a = dot2(P[r], x[r], a);
#pragma unroll
    for (int r = 8; r < 16; ++r) b = dot2(P[r], x[r], b);
    sa = a;
    sb = b;
  }
  template <int M, int S>
  __device__ static void dot(const Raw &q, int h, const uint32_t (*xp)[32 / S], const float (*kc)[NKS(S)], float *out) {
    const uint32_t f = q.f;
    const float dv = ss_one<BF>(q.d);
    if constexpr (S == 1) {
      uint32_t P0[16], P1[16];
      chunk_pairs(q.a.x, q.a.y, q.a.z, P0);
      chunk_pairs(q.a.w, q.b.x, q.b.y, P1);
      const float s0 = (float)(f & 63u), s1 = (float)((f >> 6) & 63u);
      const float s2 = (float)((f >> 12) & 63u), s3 = (float)((f >> 18) & 63u);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float sa0, sb0, sa1, sb1;
        chunk_dot(P0, xp[m], kc[m][0], kc[m][1], sa0, sb0);
        chunk_dot(P1, xp[m] + 16, kc[m][2], kc[m][3], sa1, sb1);
        float acc = s0 * sa0;
        acc = __builtin_fmaf(s1, sb0, acc);
        acc = __builtin_fmaf(s2, sa1, acc);
        acc = __builtin_fmaf(s3, sb1, acc);
        out[m] = __builtin_fmaf(dv, acc, out[m]);
      }
    } else {
      // chunk h: (a.x, a.y, a.z) or (a.w, b.x, b.y); its sub-blocks are 2h, 2h+1
      uint32_t P[16];
      chunk_pairs(sel(h, q.a.w, q.a.x), sel(h, q.b.x, q.a.y), sel(h, q.b.y, q.a.z), P);
      const uint32_t fh = f >> (12 * h);
      const float s0 = (float)(fh & 63u), s1 = (float)((fh >> 6) & 63u);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float sa, sb;
        chunk_dot(P, xp[m], kc[m][0], kc[m][1], sa, sb);
        out[m] = __builtin_fmaf(dv, __builtin_fmaf(s1, sb, s0 * sa), out[m]);
      }
    }
  }
  // fp16 w_hat of the 16 pairs of chunk h (sub-blocks a = 2h, b = 2h + 1 of the unit)
  template <int S = 1> __device__ static void wide(const Raw &q, int h, uint32_t *out) {
    uint32_t P[16];
    chunk_pairs(sel(h, q.a.w, q.a.x), sel(h, q.b.x, q.a.y), sel(h, q.b.y, q.a.z), P);
    const uint32_t fh = q.f >> (12 * h);
    const float dv = ss_one<BF>(q.d);
    const float sa = dv * (float)(fh & 63u), sb = dv * (float)((fh >> 6) & 63u);
    const _Float16 a1 = (_Float16)sa, b1 = (_Float16)sb;
#pragma unroll
    for (int r = 0; r < 6; ++r) out[r] = sym_pair(P[r], (_Float16)-1028.0f, a1);
    out[6] = sym_pair(P[6], (_Float16)-132.0f, a1);
    out[7] = sym_pair(P[7], (_Float16)-132.0f, a1);
#pragma unroll
    for (int r = 8; r < 12; ++r) out[r] = sym_pair(P[r], (_Float16)-132.0f, b1);
#pragma unroll
    for (int r = 12; r < 16; ++r) out[r] = sym_pair(P[r], (_Float16)-20.0f, b1);
  }
};
template <> struct Unit<3> : UnitQ3<false> {};
template <> struct Unit<13> : UnitQ3<true> {};

// ---- plain group-wise 3-bit codes with an fp32 scale s and min m per group of 32 (q3g32):
// q3sb's code planes (a chunk of 32 codes is one group), scale and min planes of two fp32 per
// unit. w_hat = s c + m, so a group's sum is s * sum(c x) + m * sum(x). With S = 2 lane half
// h owns chunk (group) h.
template <> struct Unit<kQ3G32> : UnitQ3<false> {
  static constexpr int NK = 4;
  __host__ __device__ static constexpr int NKS(int S) { return NK / S; }
  struct Raw { u32x4 a; u32x2 b; float s[2]; float mn[2]; };
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16); off[1] = (uint32_t)(u * 8); off[2] = (uint32_t)(u * 8); off[3] = (uint32_t)(u * 8);
  }
  template <int AUX = kNT, int S = 1> __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    q.a = bldx4<AUX>(L.rs[0], L.off[0], L.row(0, r));
    q.b = bldx2<AUX>(L.rs[1], L.off[1], L.row(1, r));
    // (integer pairs through keep(): see the INT4 scale loads)
    const u32x2 sv = bldx2<0>(L.rs[2], L.off[2], L.row(2, r));
    const u32x2 mv = bldx2<0>(L.rs[3], L.off[3], L.row(3, r));
    q.s[0] = __builtin_bit_cast(float, keep(sv.x));
    q.s[1] = __builtin_bit_cast(float, keep(sv.y));
    q.mn[0] = __builtin_bit_cast(float, keep(mv.x));
    q.mn[1] = __builtin_bit_cast(float, keep(mv.y));
  }
  // Per chunk: the start of its accumulator (sum P x = sum c x + 1024 X1 + 128 X8a + 128 X8b
  // + 16 X64, with q3sb's class magics) and sum x.
  // kc layout (S = 1): [start g0, start g1, sum x g0, sum x g1]; (S = 2): [start, sum x]
  template <int S> __device__ static void prep(uint32_t *xp, float *kc) {
#pragma unroll
    for (int c = 0; c < 2 / S; ++c) {
      uint32_t *x = xp + 16 * c;
      float a1 = 0.f, a8 = 0.f, b8 = 0.f, b64 = 0.f;
#pragma unroll
      for (int r = 0; r < 6; ++r) a1 = dot2(x[r], kOnes, a1);
#pragma unroll
      for (int r = 6; r < 8; ++r) a8 = dot2(x[r], kOnes, a8);
#pragma unroll
      for (int r = 8; r < 12; ++r) b8 = dot2(x[r], kOnes, b8);
#pragma unroll
      for (int r = 12; r < 16; ++r) b64 = dot2(x[r], kOnes, b64);
      kc[c] = -(1024.0f * a1 + 128.0f * (a8 + b8) + 16.0f * b64);
      kc[2 / S + c] = (a1 + a8) + (b8 + b64);
    }
  }
  template <int M, int S>
  __device__ static void dot(const Raw &q, int h, const uint32_t (*xp)[32 / S], const float (*kc)[NKS(S)], float *out) {
    if constexpr (S == 1) {
      uint32_t P0[16], P1[16];
      chunk_pairs(q.a.x, q.a.y, q.a.z, P0);
      chunk_pairs(q.a.w, q.b.x, q.b.y, P1);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a0 = kc[m][0], a1 = kc[m][1];
#pragma unroll
        for (int r = 0; r < 16; ++r) a0 = dot2(P0[r], xp[m][r], a0);
#pragma unroll
        for (int r = 0; r < 16; ++r) a1 = dot2(P1[r], xp[m][16 + r], a1);
        out[m] = __builtin_fmaf(q.s[0], a0, __builtin_fmaf(q.mn[0], kc[m][2], out[m]));
        out[m] = __builtin_fmaf(q.s[1], a1, __builtin_fmaf(q.mn[1], kc[m][3], out[m]));
      }
    } else {
      uint32_t P[16];
      chunk_pairs(sel(h, q.a.w, q.a.x), sel(h, q.b.x, q.a.y), sel(h, q.b.y, q.a.z), P);
      const float sc = __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.s[1]), __builtin_bit_cast(uint32_t, q.s[0])));
      const float mn = __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.mn[1]), __builtin_bit_cast(uint32_t, q.mn[0])));
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a = kc[m][0];
#pragma unroll
        for (int r = 0; r < 16; ++r) a = dot2(P[r], xp[m][r], a);
        out[m] = __builtin_fmaf(sc, a, __builtin_fmaf(mn, kc[m][1], out[m]));
      }
    }
  }
  // fp16 w_hat of the 16 pairs of chunk h: P * s + (m - B s) for class magic B, in fp32, then
  // one rounding
  template <int S = 1> __device__ static void wide(const Raw &q, int h, uint32_t *out) {
    uint32_t P[16];
    chunk_pairs(sel(h, q.a.w, q.a.x), sel(h, q.b.x, q.a.y), sel(h, q.b.y, q.a.z), P);
    const float sc = __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.s[1]), __builtin_bit_cast(uint32_t, q.s[0])));
    const float mn = __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.mn[1]), __builtin_bit_cast(uint32_t, q.mn[0])));
    const float mul1 = sc, add1 = __builtin_fmaf(-1024.0f, sc, mn);
    const float add8 = __builtin_fmaf(-128.0f, sc, mn), add64 = __builtin_fmaf(-16.0f, sc, mn);
#pragma unroll
    for (int r = 0; r < 6; ++r) out[r] = asym_pair(P[r], mul1, add1);
#pragma unroll
    for (int r = 6; r < 12; ++r) out[r] = asym_pair(P[r], mul1, add8);
#pragma unroll
    for (int r = 12; r < 16; ++r) out[r] = asym_pair(P[r], mul1, add64);
  }
};

// ---- nibble plane + high-bit plane (q5sb: 1 high bit, 32-weight sub-blocks;
//      q6sb: 2 high bits, 16-weight sub-blocks). Produces the four pairs of one nibble dword.
// The class-16 pairs take magic M16: 1024 (1024 + 16 c, for the fp32-combined dot) or 64
// (64 + c, for the fp16 decode).
template <int HB, uint32_t M16 = kMagic>
__device__ __forceinline__ void nib_pairs(uint32_t L, uint32_t H, int ip, uint32_t *P) {
  constexpr uint32_t m1 = HB == 1 ? 0x00100010u : 0x00300030u;
  constexpr uint32_t m16 = HB == 1 ? 0x01000100u : 0x03000300u;
  const int ra = HB * ip, rb = 8 + HB * ip;
  const uint32_t ha = ra ? rotr(H, ra) : H, hb = rotr(H, rb);
  const uint32_t L8 = L >> 8;
  P[0] = pick_or(L, QG_SMASK(0x000F000Fu), keep(pick(ha, QG_SMASK(m1))));         // class 1
  P[1] = pick_or(L, QG_SMASK(0x00F000F0u), keep(pick<M16>(ha, QG_SMASK(m16))));   // class 16
  P[2] = pick_or(L8, QG_SMASK(0x000F000Fu), keep(pick(hb, QG_SMASK(m1))));        // class 1
  P[3] = pick_or(L8, QG_SMASK(0x00F000F0u), keep(pick<M16>(hb, QG_SMASK(m16))));  // class 16
}

// ---- 5-bit super-block: a unit is two sub-blocks of 32; with S = 2 lane half h owns one
template <bool BF> struct UnitQ5 {
  static constexpr int NK = 4;
  __host__ __device__ static constexpr int NKS(int S) { return NK / S; }
  struct Raw { u32x4 l0, l1; u32x2 h; uint32_t f, dd; };
  __device__ static int pidx(int h, int p, int S) { return S == 1 ? p : 16 * h + p; }
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16); off[1] = (uint32_t)(u * 8); off[2] = fields_off(u); off[3] = (uint32_t)((u >> 2) * 4);
  }
  // S = 2: only the lane's own sub-block h: its nibble half into l0, its high-bit word into h.x
  template <int AUX = kNT, int S = 1> __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    const uint32_t r0 = L.row(0, r);
    if constexpr (S == 2) {
      q.l0 = bldx4<AUX>(L.rs[0], L.off[0] + (L.h ? L.half16 : 0u), r0);
      q.h.x = bldx1<AUX>(L.rs[1], L.off[1] + 4u * L.h, L.row(1, r));
    } else {
      q.l0 = bldx4<AUX>(L.rs[0], L.off[0], r0);
      q.l1 = bldx4<AUX>(L.rs[0], L.off[0] + L.half16, r0);
      q.h = bldx2<AUX>(L.rs[1], L.off[1], L.row(1, r));
    }
    q.f = fields24(L, 2, r);
    q.dd = bld1(L.rs[3], L.off[3], L.row(3, r));
  }
  // kc layout (S = 1): [start h0, start h1, sum x h0, sum x h1]; (S = 2): [start, sum x]
  template <int S> __device__ static void prep(uint32_t *xp, float *kc) {
#pragma unroll
    for (int hh = 0; hh < 2 / S; ++hh) {
      float x1 = 0.f, x16 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x1 = dot2(xp[16 * hh + 4 * i + 0], kOnes, x1);
        x1 = dot2(xp[16 * hh + 4 * i + 2], kOnes, x1);
        x16 = dot2(xp[16 * hh + 4 * i + 1], kOnes, x16);
        x16 = dot2(xp[16 * hh + 4 * i + 3], kOnes, x16);
      }
      kc[hh] = -(1024.0f * x1 + 64.0f * x16);
      kc[2 / S + hh] = x1 + x16;
    }
  }
  template <int M, int S>
  __device__ static void dot(const Raw &q, int h, const uint32_t (*xp)[32 / S], const float (*kc)[NKS(S)], float *out) {
    // (S = 2 loaded the lane's own nibble half into l0 and its high-bit word into h.x)
    const uint32_t L[8] = {q.l0.x, q.l0.y, q.l0.z, q.l0.w, S == 1 ? q.l1.x : 0u, S == 1 ? q.l1.y : 0u,
                           S == 1 ? q.l1.z : 0u, S == 1 ? q.l1.w : 0u};
    const uint32_t f = q.f;
    const float dv = ss_lo<BF>(q.dd), dm = ss_hi<BF>(q.dd);
#pragma unroll
    for (int hh = 0; hh < 2 / S; ++hh) {
      const int sb = S == 1 ? hh : 0;     // sub-block within what this lane owns
      float a1[M], a16[M];
#pragma unroll
      for (int m = 0; m < M; ++m) { a1[m] = kc[m][sb]; a16[m] = 0.f; }
      const uint32_t H = S == 1 && hh ? q.h.y : q.h.x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t P[4];
        nib_pairs<1>(L[4 * hh + i], H, i, P);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          a1[m] = dot2(P[0], xp[m][16 * sb + 4 * i + 0], a1[m]);
          a16[m] = dot2(P[1], xp[m][16 * sb + 4 * i + 1], a16[m]);
          a1[m] = dot2(P[2], xp[m][16 * sb + 4 * i + 2], a1[m]);
          a16[m] = dot2(P[3], xp[m][16 * sb + 4 * i + 3], a16[m]);
        }
      }
      // sub-block of the super-block: 2q + (S == 1 ? hh : h); fields [sc0, sc1, m0, m1]
      const int which = S == 1 ? hh : h;
      const float scv = (float)((f >> (6 * which)) & 63u), mv = (float)((f >> (12 + 6 * which)) & 63u);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float s = __builtin_fmaf(a16[m], 0.0625f, a1[m]);   // sum c x
        out[m] = __builtin_fmaf(dv * scv, s, __builtin_fmaf(-dm * mv, kc[m][2 / S + sb], out[m]));
      }
    }
  }
  // fp16 w_hat of the 16 pairs of half h (sub-block h of the unit); S = 2: q holds only that
  // sub-block's nibbles (l0) and high bits (h.x)
  template <int S = 1> __device__ static void wide(const Raw &q, int h, uint32_t *out) {
    const uint32_t L[8] = {q.l0.x, q.l0.y, q.l0.z, q.l0.w, S == 1 ? q.l1.x : 0u, S == 1 ? q.l1.y : 0u,
                           S == 1 ? q.l1.z : 0u, S == 1 ? q.l1.w : 0u};
    const uint32_t H = S == 1 ? sel(h, q.h.y, q.h.x) : q.h.x;
    const float dv = ss_lo<BF>(q.dd), dm = ss_hi<BF>(q.dd);
    const float step = dv * (float)((q.f >> (6 * h)) & 63u), off = dm * (float)((q.f >> (12 + 6 * h)) & 63u);
    const float mul1 = step, add1 = -__builtin_fmaf(1024.0f, step, off);
    const float mul16 = step * 0.0625f, add16 = -__builtin_fmaf(64.0f, step, off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t P[4];
      nib_pairs<1>(S == 1 ? sel(h, L[4 + i], L[i]) : L[i], H, i, P);
      out[4 * i + 0] = asym_pair(P[0], mul1, add1);
      out[4 * i + 1] = asym_pair(P[1], mul16, add16);
      out[4 * i + 2] = asym_pair(P[2], mul1, add1);
      out[4 * i + 3] = asym_pair(P[3], mul16, add16);
    }
  }
};
template <> struct Unit<5> : UnitQ5<false> {};
template <> struct Unit<15> : UnitQ5<true> {};

// ---- plain group-wise 5-bit codes with an fp32 scale s and min m per group of 32 (q5g32):
// q5sb's code planes (a sub-block of 32 is one group), scale and min planes of two fp32 per
// unit; w_hat = s c + m. prep is q5sb's (start and sum x per group). With S = 2 lane half h
// owns group h.
template <> struct Unit<kQ5G32> : UnitQ5<false> {
  struct Raw { u32x4 l0, l1; u32x2 h; float s[2]; float mn[2]; };
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16); off[1] = (uint32_t)(u * 8); off[2] = (uint32_t)(u * 8); off[3] = (uint32_t)(u * 8);
  }
  template <int AUX = kNT, int S = 1> __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    const uint32_t r0 = L.row(0, r);
    if constexpr (S == 2) {
      q.l0 = bldx4<AUX>(L.rs[0], L.off[0] + (L.h ? L.half16 : 0u), r0);
      q.h.x = bldx1<AUX>(L.rs[1], L.off[1] + 4u * L.h, L.row(1, r));
    } else {
      q.l0 = bldx4<AUX>(L.rs[0], L.off[0], r0);
      q.l1 = bldx4<AUX>(L.rs[0], L.off[0] + L.half16, r0);
      q.h = bldx2<AUX>(L.rs[1], L.off[1], L.row(1, r));
    }
    const u32x2 sv = bldx2<0>(L.rs[2], L.off[2], L.row(2, r));
    const u32x2 mv = bldx2<0>(L.rs[3], L.off[3], L.row(3, r));
    q.s[0] = __builtin_bit_cast(float, keep(sv.x));
    q.s[1] = __builtin_bit_cast(float, keep(sv.y));
    q.mn[0] = __builtin_bit_cast(float, keep(mv.x));
    q.mn[1] = __builtin_bit_cast(float, keep(mv.y));
  }
  template <int M, int S>
  __device__ static void dot(const Raw &q, int h, const uint32_t (*xp)[32 / S], const float (*kc)[NKS(S)], float *out) {
    const uint32_t L[8] = {q.l0.x, q.l0.y, q.l0.z, q.l0.w, S == 1 ? q.l1.x : 0u, S == 1 ? q.l1.y : 0u,
                           S == 1 ? q.l1.z : 0u, S == 1 ? q.l1.w : 0u};
#pragma unroll
    for (int hh = 0; hh < 2 / S; ++hh) {
      const int sb = S == 1 ? hh : 0;
      float a1[M], a16[M];
#pragma unroll
      for (int m = 0; m < M; ++m) { a1[m] = kc[m][sb]; a16[m] = 0.f; }
      const uint32_t H = S == 1 && hh ? q.h.y : q.h.x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t P[4];
        nib_pairs<1>(L[4 * hh + i], H, i, P);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          a1[m] = dot2(P[0], xp[m][16 * sb + 4 * i + 0], a1[m]);
          a16[m] = dot2(P[1], xp[m][16 * sb + 4 * i + 1], a16[m]);
          a1[m] = dot2(P[2], xp[m][16 * sb + 4 * i + 2], a1[m]);
          a16[m] = dot2(P[3], xp[m][16 * sb + 4 * i + 3], a16[m]);
        }
      }
      const float sc = S == 1 ? q.s[hh]
                              : __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.s[1]), __builtin_bit_cast(uint32_t, q.s[0])));
      const float mn = S == 1 ? q.mn[hh]
                              : __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.mn[1]), __builtin_bit_cast(uint32_t, q.mn[0])));
#pragma unroll
      for (int m = 0; m < M; ++m)
        out[m] = __builtin_fmaf(sc, __builtin_fmaf(a16[m], 0.0625f, a1[m]), __builtin_fmaf(mn, kc[m][2 / S + sb], out[m]));
    }
  }
  // fp16 w_hat of the 16 pairs of half h (group h); S = 2: q holds only that group's codes
  template <int S = 1> __device__ static void wide(const Raw &q, int h, uint32_t *out) {
    const uint32_t L[8] = {q.l0.x, q.l0.y, q.l0.z, q.l0.w, S == 1 ? q.l1.x : 0u, S == 1 ? q.l1.y : 0u,
                           S == 1 ? q.l1.z : 0u, S == 1 ? q.l1.w : 0u};
    const uint32_t H = S == 1 ? sel(h, q.h.y, q.h.x) : q.h.x;
    const float sc = __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.s[1]), __builtin_bit_cast(uint32_t, q.s[0])));
    const float mn = __builtin_bit_cast(float, sel(h, __builtin_bit_cast(uint32_t, q.mn[1]), __builtin_bit_cast(uint32_t, q.mn[0])));
    const float mul1 = sc, add1 = __builtin_fmaf(-1024.0f, sc, mn);
    const float mul16 = sc * 0.0625f, add16 = __builtin_fmaf(-64.0f, sc, mn);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t P[4];
      nib_pairs<1>(S == 1 ? sel(h, L[4 + i], L[i]) : L[i], H, i, P);
      out[4 * i + 0] = asym_pair(P[0], mul1, add1);
      out[4 * i + 1] = asym_pair(P[1], mul16, add16);
      out[4 * i + 2] = asym_pair(P[2], mul1, add1);
      out[4 * i + 3] = asym_pair(P[3], mul16, add16);
    }
  }
};

// ---- 6-bit super-block: a unit is four sub-blocks of 16; with S = 2 lane half h owns
// sub-blocks 2h, 2h+1
template <bool BF> struct UnitQ6 {
  static constexpr int NK = 4;
  __host__ __device__ static constexpr int NKS(int S) { return NK / S; }
  struct Raw { u32x4 l0, l1, h; uint32_t sc; uint16_t d; };
  __device__ static int pidx(int h, int p, int S) { return S == 1 ? p : 16 * h + p; }
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16); off[1] = (uint32_t)(u * 16); off[2] = (uint32_t)(u * 4); off[3] = (uint32_t)((u >> 2) * 2);
  }
  // S = 2: only the lane's own sub-blocks 2h, 2h+1: its nibble half into l0, its two
  // high-field dwords into h.x, h.y
  template <int AUX = kNT, int S = 1> __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    const uint32_t r0 = L.row(0, r);
    if constexpr (S == 2) {
      q.l0 = bldx4<AUX>(L.rs[0], L.off[0] + (L.h ? L.half16 : 0u), r0);
      const u32x2 hh = bldx2<AUX>(L.rs[1], L.off[1] + 8u * L.h, L.row(1, r));
      q.h.x = hh.x;
      q.h.y = hh.y;
    } else {
      q.l0 = bldx4<AUX>(L.rs[0], L.off[0], r0);
      q.l1 = bldx4<AUX>(L.rs[0], L.off[0] + L.half16, r0);
      q.h = bldx4<AUX>(L.rs[1], L.off[1], L.row(1, r));
    }
    q.sc = bldx1<AUX>(L.rs[2], L.off[2], L.row(2, r));
    q.d = bldh(L.rs[3], L.off[3], L.row(3, r));
  }
  template <int S> __device__ static void prep(uint32_t *xp, float *kc) {
#pragma unroll
    for (int j = 0; j < 4 / S; ++j) {
      float x1 = 0.f, x16 = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        x1 = dot2(xp[8 * j + 4 * i + 0], kOnes, x1);
        x1 = dot2(xp[8 * j + 4 * i + 2], kOnes, x1);
        x16 = dot2(xp[8 * j + 4 * i + 1], kOnes, x16);
        x16 = dot2(xp[8 * j + 4 * i + 3], kOnes, x16);
      }
      kc[j] = -(1056.0f * x1 + 96.0f * x16);   // 1024 + 32 offset, 64 + 32 offset
    }
  }
  template <int M, int S>
  __device__ static void dot(const Raw &q, int h, const uint32_t (*xp)[32 / S], const float (*kc)[NKS(S)], float *out) {
    // (S = 2 loaded the lane's own nibble half into l0 and its high-field dwords into h.x, h.y)
    const uint32_t L[8] = {q.l0.x, q.l0.y, q.l0.z, q.l0.w, S == 1 ? q.l1.x : 0u, S == 1 ? q.l1.y : 0u,
                           S == 1 ? q.l1.z : 0u, S == 1 ? q.l1.w : 0u};
    const uint32_t Hd[4] = {q.h.x, q.h.y, S == 1 ? q.h.z : 0u, S == 1 ? q.h.w : 0u};
    const float dv = ss_one<BF>(q.d);
#pragma unroll
    for (int j = 0; j < 4 / S; ++j) {
      float a1[M], a16[M];
#pragma unroll
      for (int m = 0; m < M; ++m) { a1[m] = kc[m][j]; a16[m] = 0.f; }
      const uint32_t H = Hd[j];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        uint32_t P[4];
        nib_pairs<2>(L[2 * j + ii], H, ii, P);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          a1[m] = dot2(P[0], xp[m][8 * j + 4 * ii + 0], a1[m]);
          a16[m] = dot2(P[1], xp[m][8 * j + 4 * ii + 1], a16[m]);
          a1[m] = dot2(P[2], xp[m][8 * j + 4 * ii + 2], a1[m]);
          a16[m] = dot2(P[3], xp[m][8 * j + 4 * ii + 3], a16[m]);
        }
      }
      const int jj = S == 1 ? j : 2 * h + j;
      const float sj = (float)(int8_t)((q.sc >> (8 * jj)) & 0xFFu);
#pragma unroll
      for (int m = 0; m < M; ++m) out[m] = __builtin_fmaf(dv * sj, __builtin_fmaf(a16[m], 0.0625f, a1[m]), out[m]);
    }
  }
  // fp16 w_hat of the 16 pairs of half h (sub-blocks 2h, 2h + 1 of the unit); S = 2: q holds
  // only those sub-blocks' nibbles (l0) and high fields (h.x, h.y)
  template <int S = 1> __device__ static void wide(const Raw &q, int h, uint32_t *out) {
    const uint32_t L[8] = {q.l0.x, q.l0.y, q.l0.z, q.l0.w, S == 1 ? q.l1.x : 0u, S == 1 ? q.l1.y : 0u,
                           S == 1 ? q.l1.z : 0u, S == 1 ? q.l1.w : 0u};
    const uint32_t Hd[4] = {q.h.x, q.h.y, S == 1 ? q.h.z : 0u, S == 1 ? q.h.w : 0u};
    const float dv = ss_one<BF>(q.d);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float step = dv * (float)(int8_t)((q.sc >> (8 * (2 * h + j))) & 0xFFu);
      // The 6-bit codes' step is about max|w| / 31.5, small enough to fall below fp16's normal
      // range on small layers, so it stays fp32: P * step + add is exact in fp32 (step has at
      // most 19 significant bits, 1056 = 33 * 32 and 96 = 3 * 32 keep add exact, and
      // (c - 32) * step fits 24 bits), and the one rounding is to fp16.
      const float add1 = -1056.0f * step, add16 = -96.0f * step;
      const uint32_t H = S == 1 ? sel(h, Hd[2 + j], Hd[j]) : Hd[j];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        uint32_t P[4];
        nib_pairs<2, kMagic64>(S == 1 ? sel(h, L[4 + 2 * j + ii], L[2 * j + ii]) : L[2 * j + ii], H, ii, P);
        out[8 * j + 4 * ii + 0] = asym_pair(P[0], step, add1);
        out[8 * j + 4 * ii + 1] = asym_pair(P[1], step, add16);
        out[8 * j + 4 * ii + 2] = asym_pair(P[2], step, add1);
        out[8 * j + 4 * ii + 3] = asym_pair(P[3], step, add16);
      }
    }
  }
};
template <> struct Unit<6> : UnitQ6<false> {};
template <> struct Unit<16> : UnitQ6<true> {};

}  // namespace qg
