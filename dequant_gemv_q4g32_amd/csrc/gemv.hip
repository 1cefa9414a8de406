// Dequant GEMV (batch 1) and device decode for the five packed formats, gfx950.
//
// Method: "二三五六位量化" page section 3.3 (gemv_q3: y[r] = sum (s*q + m) x, with unpacking
// separated from the multiply-add and the sum-of-x rewrite s*(q.x) + m*sum(x)); DBHOO-CIM
// page section 3.3 (fused dequantization: codes are expanded in registers and meet the
// activations directly; no dequantized weight array is ever written) and section 4.3 (rows
// are split across workers; no write conflicts).
//
// Mapping to CDNA4: a lane owns one 64-weight unit of K for every row its wave visits, keeps
// the activations of that unit in 32 VGPRs as fp16 pairs, and streams the packed planes
// with 128-bit loads (consecutive lanes, consecutive bytes). Codes are turned into fp16
// (1024 + p*c) pairs with one v_and_or_b32 each and multiplied with v_dot2_f32_f16; the
// 1024 and code offsets cancel against per-lane constants computed once from x. Each
// wave reduces its R row partials with DPP; K longer than 4096 weights is split across
// the waves of a workgroup and reduced through LDS.
#include <hip/hip_runtime.h>

#include "../../include/qgemv.h"
#include "device_common.h"
#include "layout.h"

namespace qg {

struct GemvArgs {
  const uint8_t *w;
  int64_t w_bstride;        // bytes between batched matrices
  const uint16_t *x;
  int64_t x_bstride;        // elements
  void *y;
  int64_t y_bstride;        // elements
  int64_t n, k, units;
  int64_t poff[4];
  int64_t prb[4];
  int y_f32;
  int wk;                   // waves per workgroup along K
  int wr;                   // row groups per workgroup
  int nb;                   // row batches per row group (each R rows)
};

// Per-lane view of the planes: one buffer resource per plane (wave-uniform), the plane's row
// stride (uniform) and the lane's byte offset inside a row (per lane).
struct Lane {
  rsrc_t rs[4];
  uint32_t prb[4];
  uint32_t off[4];
  uint32_t sh;              // bit offset of this unit's 6-bit fields in its 8-byte window
  __device__ uint32_t row(int p, int64_t r) const { return (uint32_t)r * prb[p]; }
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

// ------------------------------------------------------------------ per-format units -----
// Each format provides:
//   struct Raw              packed data of one unit of one row (registers)
//   offsets(u, off)         the lane's byte offset in a row of each plane
//   load(Raw&, lane, r)     issue the loads for row r
//   prep(xp, kc)            per-lane constants from the unit's 32 x pairs
//   dot(Raw, xp, kc)        the unit's contribution to y[r]

template <int F> struct Unit;

// ---- INT4 group-32 (two groups per unit)
template <> struct Unit<4> {
  static constexpr int NK = 2;
  struct Raw { u32x4 c0, c1; float s0, s1; };
  __device__ static void offsets(int64_t u, uint32_t *off) { off[0] = (uint32_t)(u * 32); off[1] = (uint32_t)(u * 8); }
  __device__ static void load(Raw &q, const Lane &L, int64_t r, bool half) {
    const uint32_t r0 = L.row(0, r), r1 = L.row(1, r);
    q.c0 = bld4(L.rs[0], L.off[0], r0);
    // a half unit (k % 64 == 32) has one group; its second group's activations are zero
    q.c1 = bld4(L.rs[0], L.off[0] + (half ? 0u : 16u), r0);
    // Two 32-bit loads, not one 64-bit load: this toolchain narrows a multi-dword buffer load
    // whose elements are bit-cast to float to its first dword and reuses that dword for the
    // second element (vectors used in integer arithmetic, like the code words, are unaffected).
    q.s0 = __builtin_bit_cast(float, bld1(L.rs[1], L.off[1], r1));
    q.s1 = __builtin_bit_cast(float, bld1(L.rs[1], L.off[1] + (half ? 0u : 4u), r1));
  }
  __device__ static void prep(const uint32_t *xp, float *kc) {
    for (int g = 0; g < 2; ++g) {
      float x1 = 0.f, x16 = 0.f;
      for (int i = 0; i < 4; ++i) {
        x1 = dot2(xp[16 * g + 4 * i + 0], kOnes, x1);
        x1 = dot2(xp[16 * g + 4 * i + 2], kOnes, x1);
        x16 = dot2(xp[16 * g + 4 * i + 1], kOnes, x16);
        x16 = dot2(xp[16 * g + 4 * i + 3], kOnes, x16);
      }
      kc[g] = -(1032.0f * x1 + 72.0f * x16);   // sum (u - 8) x = A1 + A16/16 with A1 starting here
    }
  }
  __device__ static float group(u32x4 c, const uint32_t *xp, float k0) {
    float a1 = k0, a16 = 0.f;
    uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = d[i], v8 = v >> 8;
      a1 = dot2(pick(v, QG_SMASK(0x000F000Fu)), xp[4 * i + 0], a1);
      a16 = dot2(pick(v, QG_SMASK(0x00F000F0u)), xp[4 * i + 1], a16);
      a1 = dot2(pick(v8, QG_SMASK(0x000F000Fu)), xp[4 * i + 2], a1);
      a16 = dot2(pick(v8, QG_SMASK(0x00F000F0u)), xp[4 * i + 3], a16);
    }
    return __builtin_fmaf(a16, 0.0625f, a1);
  }
  __device__ static float dot(const Raw &q, const uint32_t *xp, const float *kc) {
    float s0 = group(q.c0, xp, kc[0]);
    float s1 = group(q.c1, xp + 16, kc[1]);
    return __builtin_fmaf(q.s1, s1, q.s0 * s0);
  }
};

// ---- 2-bit super-block (a unit is a quarter super-block: 4 sub-blocks of 16)
template <> struct Unit<2> {
  static constexpr int NK = 8;
  struct Raw { u32x4 c; uint32_t sc, dd; };
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16); off[1] = (uint32_t)(u * 4); off[2] = (uint32_t)((u >> 2) * 4);
  }
  __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    q.c = bld4(L.rs[0], L.off[0], L.row(0, r));
    q.sc = bld1_nt(L.rs[1], L.off[1], L.row(1, r));
    q.dd = bld1(L.rs[2], L.off[2], L.row(2, r));
  }
  __device__ static void prep(const uint32_t *xp, float *kc) {
    for (int j = 0; j < 4; ++j) {
      float s = 0.f;
      for (int r = 0; r < 8; ++r) s = dot2(xp[8 * j + r], kOnes, s);
      kc[j] = s;                       // X_j
      kc[4 + j] = -1024.0f * s;        // accumulator start
    }
  }
  __device__ static float dot(const Raw &q, const uint32_t *xp, const float *kc) {
    float A[4] = {kc[4], kc[5], kc[6], kc[7]};
    uint32_t d[4] = {q.c.x, q.c.y, q.c.z, q.c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = d[i], v8 = v >> 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        A[j] = dot2(pick(v, QG_SMASK(0x00030003u << (2 * j))), xp[8 * j + 2 * i], A[j]);
        A[j] = dot2(pick(v8, QG_SMASK(0x00030003u << (2 * j))), xp[8 * j + 2 * i + 1], A[j]);
      }
    }
    const uint32_t s = q.sc;
    float sa = 0.f, sm = 0.f;
    const float inv4[4] = {1.0f, 0.25f, 0.0625f, 0.015625f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float scj = (float)((s >> (8 * j)) & 15u);
      float mj = (float)((s >> (8 * j + 4)) & 15u);
      sa = __builtin_fmaf(scj * inv4[j], A[j], sa);
      sm = __builtin_fmaf(mj, kc[j], sm);
    }
    return __builtin_fmaf(half_lo(q.dd), sa, -half_hi(q.dd) * sm);
  }
};

// ---- 3-bit super-block (quarter super-block = two chunks of 32 codes)
template <> struct Unit<3> {
  static constexpr int NK = 4;
  struct Raw { u32x4 a; u32x2 b; uint32_t f; uint16_t d; };
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 16); off[1] = (uint32_t)(u * 8); off[2] = fields_off(u); off[3] = (uint32_t)((u >> 2) * 2);
  }
  __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    q.a = bld4(L.rs[0], L.off[0], L.row(0, r));
    q.b = bld2(L.rs[1], L.off[1], L.row(1, r));
    q.f = fields24(L, 2, r);
    q.d = bldh(L.rs[3], L.off[3], L.row(3, r));
  }
  __device__ static void prep(const uint32_t *xp, float *kc) {
    for (int c = 0; c < 2; ++c) {
      const uint32_t *x = xp + 16 * c;
      float a1 = 0.f, a8 = 0.f, b8 = 0.f, b64 = 0.f;
      for (int r = 0; r < 6; ++r) a1 = dot2(x[r], kOnes, a1);
      for (int r = 6; r < 8; ++r) a8 = dot2(x[r], kOnes, a8);
      for (int r = 8; r < 12; ++r) b8 = dot2(x[r], kOnes, b8);
      for (int r = 12; r < 16; ++r) b64 = dot2(x[r], kOnes, b64);
      kc[2 * c] = -(1028.0f * a1 + 132.0f * a8);            // start of a's class-1 sum
      kc[2 * c + 1] = -8.0f * (132.0f * b8 + 20.0f * b64);  // start of b's class-8 sum
    }
  }
  __device__ static void chunk(uint32_t e0, uint32_t e1, uint32_t e2, const uint32_t *x, float ka, float kb,
                               float &sa, float &sb) {
    const uint32_t e09 = e0 >> 9, e19 = e1 >> 9, e29 = e2 >> 9;
    float a1 = ka, a8 = 0.f, b8 = kb, b64 = 0.f;
    a1 = dot2(pick(e0, QG_SMASK(0x00070007u)), x[0], a1);
    a1 = dot2(pick(e09, QG_SMASK(0x00070007u)), x[1], a1);
    a1 = dot2(pick(e1, QG_SMASK(0x00070007u)), x[2], a1);
    a1 = dot2(pick(e19, QG_SMASK(0x00070007u)), x[3], a1);
    a1 = dot2(pick(e2, QG_SMASK(0x00070007u)), x[4], a1);
    a1 = dot2(pick(e29, QG_SMASK(0x00070007u)), x[5], a1);
    a8 = dot2(pick(e0, QG_SMASK(0x00380038u)), x[6], a8);
    a8 = dot2(pick(e09, QG_SMASK(0x00380038u)), x[7], a8);
    b8 = dot2(pick(e1, QG_SMASK(0x00380038u)), x[8], b8);
    b8 = dot2(pick(e19, QG_SMASK(0x00380038u)), x[9], b8);
    b8 = dot2(pick(e2, QG_SMASK(0x00380038u)), x[10], b8);
    b8 = dot2(pick(e29, QG_SMASK(0x00380038u)), x[11], b8);
    b64 = dot2(pick(e0, QG_SMASK(0x01C001C0u)), x[12], b64);
    b64 = dot2(pick(e1, QG_SMASK(0x01C001C0u)), x[13], b64);
    b64 = dot2(pick(e2, QG_SMASK(0x01C001C0u)), x[14], b64);
    uint32_t t = keep(pick(e09, QG_SMASK(0x00400040u)));    // bit 15 of e0 -> 6, bit 31 -> 22
    t = keep(pick_or(e1 >> 8, QG_SMASK(0x00800080u), t));    // bit 15 of e1 -> 7
    t = pick_or(e2 >> 7, QG_SMASK(0x01000100u), t);          // bit 15 of e2 -> 8
    b64 = dot2(t, x[15], b64);
    sa = __builtin_fmaf(a8, 0.125f, a1);
    sb = __builtin_fmaf(b64, 0.125f, b8);
  }
  __device__ static float dot(const Raw &q, const uint32_t *xp, const float *kc) {
    float sa0, sb0, sa1, sb1;
    chunk(q.a.x, q.a.y, q.a.z, xp, kc[0], kc[1], sa0, sb0);
    chunk(q.a.w, q.b.x, q.b.y, xp + 16, kc[2], kc[3], sa1, sb1);
    const uint32_t f = q.f;
    float s0 = (float)(f & 63u), s1 = (float)((f >> 6) & 63u) * 0.125f;
    float s2 = (float)((f >> 12) & 63u), s3 = (float)((f >> 18) & 63u) * 0.125f;
    float acc = s0 * sa0;
    acc = __builtin_fmaf(s1, sb0, acc);
    acc = __builtin_fmaf(s2, sa1, acc);
    acc = __builtin_fmaf(s3, sb1, acc);
    return half_bits(q.d) * acc;
  }
};

// ---- nibble plane + high-bit plane (q5sb: 1 high bit, 32-weight sub-blocks;
//      q6sb: 2 high bits, 16-weight sub-blocks)
template <int HB>
__device__ __forceinline__ void nib_dword(uint32_t L, uint32_t H, int ip, const uint32_t *x, float &a1, float &a16) {
  constexpr uint32_t m1 = HB == 1 ? 0x00100010u : 0x00300030u;
  constexpr uint32_t m16 = HB == 1 ? 0x01000100u : 0x03000300u;
  const int ra = HB * ip, rb = 8 + HB * ip;
  const uint32_t ha = ra ? rotr(H, ra) : H, hb = rotr(H, rb);
  const uint32_t L8 = L >> 8;
  a1 = dot2(pick_or(L, QG_SMASK(0x000F000Fu), keep(pick(ha, QG_SMASK(m1)))), x[0], a1);
  a16 = dot2(pick_or(L, QG_SMASK(0x00F000F0u), keep(pick(ha, QG_SMASK(m16)))), x[1], a16);
  a1 = dot2(pick_or(L8, QG_SMASK(0x000F000Fu), keep(pick(hb, QG_SMASK(m1)))), x[2], a1);
  a16 = dot2(pick_or(L8, QG_SMASK(0x00F000F0u), keep(pick(hb, QG_SMASK(m16)))), x[3], a16);
}

template <> struct Unit<5> {
  static constexpr int NK = 4;
  struct Raw { u32x4 l0, l1; u32x2 h; uint32_t f, dd; };
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 32); off[1] = (uint32_t)(u * 8); off[2] = fields_off(u); off[3] = (uint32_t)((u >> 2) * 4);
  }
  __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    const uint32_t r0 = L.row(0, r);
    q.l0 = bld4(L.rs[0], L.off[0], r0);
    q.l1 = bld4(L.rs[0], L.off[0] + 16, r0);
    q.h = bld2(L.rs[1], L.off[1], L.row(1, r));
    q.f = fields24(L, 2, r);
    q.dd = bld1(L.rs[3], L.off[3], L.row(3, r));
  }
  __device__ static void prep(const uint32_t *xp, float *kc) {
    for (int h = 0; h < 2; ++h) {
      float x1 = 0.f, x16 = 0.f;
      for (int i = 0; i < 4; ++i) {
        x1 = dot2(xp[16 * h + 4 * i + 0], kOnes, x1);
        x1 = dot2(xp[16 * h + 4 * i + 2], kOnes, x1);
        x16 = dot2(xp[16 * h + 4 * i + 1], kOnes, x16);
        x16 = dot2(xp[16 * h + 4 * i + 3], kOnes, x16);
      }
      kc[h] = -(1024.0f * x1 + 64.0f * x16);
      kc[2 + h] = x1 + x16;
    }
  }
  __device__ static float dot(const Raw &q, const uint32_t *xp, const float *kc) {
    const uint32_t L[8] = {q.l0.x, q.l0.y, q.l0.z, q.l0.w, q.l1.x, q.l1.y, q.l1.z, q.l1.w};
    const uint32_t H[2] = {q.h.x, q.h.y};
    float S[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float a1 = kc[h], a16 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) nib_dword<1>(L[4 * h + i], H[h], i, xp + 16 * h + 4 * i, a1, a16);
      S[h] = __builtin_fmaf(a16, 0.0625f, a1);
    }
    const uint32_t f = q.f;
    float sc0 = (float)(f & 63u), sc1 = (float)((f >> 6) & 63u);
    float m0 = (float)((f >> 12) & 63u), m1 = (float)((f >> 18) & 63u);
    float sa = __builtin_fmaf(sc1, S[1], sc0 * S[0]);
    float sm = __builtin_fmaf(m1, kc[3], m0 * kc[2]);
    return __builtin_fmaf(half_lo(q.dd), sa, -half_hi(q.dd) * sm);
  }
};

template <> struct Unit<6> {
  static constexpr int NK = 4;
  struct Raw { u32x4 l0, l1, h; uint32_t sc; uint16_t d; };
  __device__ static void offsets(int64_t u, uint32_t *off) {
    off[0] = (uint32_t)(u * 32); off[1] = (uint32_t)(u * 16); off[2] = (uint32_t)(u * 4); off[3] = (uint32_t)((u >> 2) * 2);
  }
  __device__ static void load(Raw &q, const Lane &L, int64_t r, bool) {
    const uint32_t r0 = L.row(0, r);
    q.l0 = bld4(L.rs[0], L.off[0], r0);
    q.l1 = bld4(L.rs[0], L.off[0] + 16, r0);
    q.h = bld4(L.rs[1], L.off[1], L.row(1, r));
    q.sc = bld1_nt(L.rs[2], L.off[2], L.row(2, r));
    q.d = bldh(L.rs[3], L.off[3], L.row(3, r));
  }
  __device__ static void prep(const uint32_t *xp, float *kc) {
    for (int j = 0; j < 4; ++j) {
      float x1 = 0.f, x16 = 0.f;
      for (int i = 0; i < 2; ++i) {
        x1 = dot2(xp[8 * j + 4 * i + 0], kOnes, x1);
        x1 = dot2(xp[8 * j + 4 * i + 2], kOnes, x1);
        x16 = dot2(xp[8 * j + 4 * i + 1], kOnes, x16);
        x16 = dot2(xp[8 * j + 4 * i + 3], kOnes, x16);
      }
      kc[j] = -(1056.0f * x1 + 96.0f * x16);   // 1024 + 32 offset, 64 + 32 offset
    }
  }
  __device__ static float dot(const Raw &q, const uint32_t *xp, const float *kc) {
    const uint32_t L[8] = {q.l0.x, q.l0.y, q.l0.z, q.l0.w, q.l1.x, q.l1.y, q.l1.z, q.l1.w};
    const uint32_t H[4] = {q.h.x, q.h.y, q.h.z, q.h.w};
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a1 = kc[j], a16 = 0.f;
      nib_dword<2>(L[2 * j], H[j], 0, xp + 8 * j, a1, a16);
      nib_dword<2>(L[2 * j + 1], H[j], 1, xp + 8 * j + 4, a1, a16);
      float sj = (float)(int8_t)((q.sc >> (8 * j)) & 0xFFu);
      acc = __builtin_fmaf(sj, __builtin_fmaf(a16, 0.0625f, a1), acc);
    }
    return half_bits(q.d) * acc;
  }
};

// ------------------------------------------------------------------ GEMV kernel ----------

template <int F, int R>
__global__ __launch_bounds__(1024) void gemv_kernel(GemvArgs a) {
  using U = Unit<F>;
  using Raw = typename U::Raw;
  extern __shared__ float red[];               // [wr][R * nb][wk] partial sums when wk > 1
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wk = wave % a.wk;
  const int wr = wave / a.wk;
  const int64_t u_raw = (int64_t)wk * 64 + lane;
  const bool act = u_raw < a.units;
  const int64_t u = act ? u_raw : 0;           // inactive lanes read unit 0 and contribute 0
  const bool half = (F == 4) && act && (u == a.units - 1) && (a.k % 64 != 0);

  const int64_t b = blockIdx.y;
  const uint8_t *w = a.w + b * a.w_bstride;
  const uint16_t *x = a.x + b * a.x_bstride;

  Lane L;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    L.rs[p] = make_rsrc(w + a.poff[p], (uint32_t)(a.prb[p] * a.n));
    L.prb[p] = (uint32_t)a.prb[p];
    L.off[p] = 0;
  }
  U::offsets(u, L.off);
  L.sh = fields_sh(u);

  // this row group's rows: nb consecutive batches of R rows; rows past n re-read row n-1
  const int rows_here = R * a.nb;
  const int64_t row_begin = ((int64_t)blockIdx.x * a.wr + wr) * rows_here;
  auto load_batch = [&](Raw *q, int64_t r0) {
#pragma unroll
    for (int i = 0; i < R; ++i) U::load(q[i], L, r0 + i < a.n ? r0 + i : a.n - 1, half);
  };
  static_assert(R == 1 || R == 2, "rows per batch");
  Raw qa[R], qb[R];
  load_batch(qa, row_begin);                   // weights first: their latency covers the x work

  uint32_t xp[32];
  {
    const uint8_t *px = reinterpret_cast<const uint8_t *>(x) + (uint32_t)(u * 128);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // a half unit (k % 64 == 32) has only 32 activations: re-read the first half, zero it
      u32x4 v = ld4(px + 16 * ((F == 4 && half) ? (i & 3) : i));
      const bool keepx = !(F == 4 && half && i >= 4);
      xp[4 * i + 0] = keepx ? v.x : 0u;
      xp[4 * i + 1] = keepx ? v.y : 0u;
      xp[4 * i + 2] = keepx ? v.z : 0u;
      xp[4 * i + 3] = keepx ? v.w : 0u;
    }
  }
  float kc[U::NK];
  U::prep(xp, kc);

  auto store_y = [&](int64_t r, float v) {
    if (a.y_f32) reinterpret_cast<float *>(a.y)[b * a.y_bstride + r] = v;
    else reinterpret_cast<_Float16 *>(a.y)[b * a.y_bstride + r] = (_Float16)v;
  };
  auto finish_batch = [&](const Raw *q, int j) {
    const int64_t r0 = row_begin + (int64_t)j * R;
    float part[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float v = U::dot(q[i], xp, kc);
      part[i] = wave_sum_to_63(act ? v : 0.f);
    }
    if (lane == 63) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        if (a.wk == 1) {
          if (r0 + i < a.n) store_y(r0 + i, part[i]);
        } else {
          red[(wr * rows_here + j * R + i) * a.wk + wk] = part[i];
        }
      }
    }
  };

  // Software pipeline: the next batch's loads are in flight while this one is computed.
  // Loads inside the steady-state loop are unconditional, so the wait before each compute
  // covers only the older batch (a conditional prefetch would force a wait for everything).
  int j = 0;
  for (; j + 2 < a.nb; j += 2) {
    load_batch(qb, row_begin + (int64_t)(j + 1) * R);
    finish_batch(qa, j);
    load_batch(qa, row_begin + (int64_t)(j + 2) * R);
    finish_batch(qb, j + 1);
  }
  if (j + 1 < a.nb) {
    load_batch(qb, row_begin + (int64_t)(j + 1) * R);
    finish_batch(qa, j);
    finish_batch(qb, j + 1);
  } else {
    finish_batch(qa, j);
  }
  if (a.wk == 1) return;
  // K split over wk waves: one barrier, then the first wave of the row group adds the
  // partial sums of all its rows and writes them (one row per lane)
  __syncthreads();
  if (wk == 0) {
    for (int i = lane; i < rows_here; i += 64) {
      const int64_t r = row_begin + i;
      float sum = 0.f;
      for (int j = 0; j < a.wk; ++j) sum += red[(wr * rows_here + i) * a.wk + j];
      if (r < a.n) store_y(r, sum);
    }
  }
}

__global__ void fill_zero_kernel(void *y, int64_t count, int f32, int64_t bstride, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  int64_t b = i / n, r = i % n;
  if (f32) reinterpret_cast<float *>(y)[b * bstride + r] = 0.f;
  else reinterpret_cast<_Float16 *>(y)[b * bstride + r] = (_Float16)0.f;
}

// ------------------------------------------------------------------ read ceiling ---------
// Streaming read of `bytes` bytes with 128-bit loads and a xor reduction: the achievable
// HBM read bandwidth that a GEMV kernel can be compared with (the DBHOO-CIM page, section
// 5.3, measures the machine's ceiling with STREAM before tuning kernels against it).
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *p, int64_t n16, uint32_t *sink) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 v = i < n16 ? p[i] : u32x4{0, 0, 0, 0};
  uint32_t s = v.x ^ v.y ^ v.z ^ v.w;
  if (s == 0x9E3779B9u) sink[0] = s;          // keeps the loads; practically never taken
}

// ------------------------------------------------------------------ device decode --------

// 24 bits of 6-bit fields for quarter q of a super-block whose 12 field bytes start at sb12.
__device__ __forceinline__ uint32_t load_fields24(const uint8_t *sb12, int q) {
  const uint8_t *p = sb12 + ((q >> 1) << 2);
  uint64_t v = (uint64_t)ld1(p) | ((uint64_t)ld1(p + 4) << 32);
  const int sh = (q == 0) ? 0 : (q == 1) ? 24 : (q == 2) ? 16 : 40;
  return (uint32_t)(v >> sh) & 0xFFFFFFu;
}
// One thread per (row, unit): decodes 64 codes from the device layout by the same bit
// placement the GEMV kernels use and writes logical-order codes and fp32 W_hat.

template <int F>
__device__ void decode_unit(const GemvArgs &a, const uint8_t *w, int64_t r, int64_t u, uint8_t *codes, float *vals,
                            int nvalid) {
  uint8_t c[64];
  float step[4] = {0, 0, 0, 0}, off[4] = {0, 0, 0, 0};
  if (F == 4) {
    const uint8_t *pc = w + a.poff[0] + r * a.prb[0] + u * 32;
    const uint8_t *ps = w + a.poff[1] + r * a.prb[1] + u * 8;
    for (int i = 0; i < 8; ++i) {
      uint32_t v = (i < 4 || nvalid > 32) ? ld1(pc + 4 * i) : 0u;
      for (int e = 0; e < 8; ++e) c[8 * i + e] = (v >> (4 * ((e >> 1) + 4 * (e & 1)))) & 15u;
    }
    float s0 = __builtin_bit_cast(float, ld1(ps));
    float s1 = nvalid > 32 ? __builtin_bit_cast(float, ld1(ps + 4)) : 0.f;
    for (int i = 0; i < nvalid; ++i) {
      codes[i] = c[i];
      vals[i] = (float)((int)c[i] - 8) * (i < 32 ? s0 : s1);
    }
    return;
  }
  if (F == 2) {
    const uint8_t *pc = w + a.poff[0] + r * a.prb[0] + u * 16;
    uint32_t d[4];
    for (int i = 0; i < 4; ++i) d[i] = ld1(pc + 4 * i);
    for (int k = 0; k < 64; ++k) {
      int j = k >> 4, t = k >> 1, h = k & 1, rr = t & 7;
      c[k] = (d[rr >> 1] >> (16 * h + 8 * (rr & 1) + 2 * j)) & 3u;
    }
    uint32_t s = ld1(w + a.poff[1] + r * a.prb[1] + u * 4);
    uint32_t dd = ld1(w + a.poff[2] + r * a.prb[2] + (u >> 2) * 4);
    float dv = half_lo(dd), dm = half_hi(dd);
    for (int j = 0; j < 4; ++j) {
      step[j] = dv * (float)((s >> (8 * j)) & 15u);
      off[j] = dm * (float)((s >> (8 * j + 4)) & 15u);
    }
    for (int k = 0; k < 64; ++k) {
      codes[k] = c[k];
      vals[k] = __builtin_fmaf(step[k >> 4], (float)c[k], -off[k >> 4]);
    }
    return;
  }
  if (F == 3) {
    uint32_t e[6];
    const uint8_t *pa = w + a.poff[0] + r * a.prb[0] + u * 16;
    const uint8_t *pb = w + a.poff[1] + r * a.prb[1] + u * 8;
    for (int i = 0; i < 4; ++i) e[i] = ld1(pa + 4 * i);
    e[4] = ld1(pb);
    e[5] = ld1(pb + 4);
    const int ta[8][2] = {{0, 0}, {0, 3}, {1, 0}, {1, 3}, {2, 0}, {2, 3}, {0, 1}, {0, 4}};
    const int tb[8][2] = {{1, 1}, {1, 4}, {2, 1}, {2, 4}, {0, 2}, {1, 2}, {2, 2}, {-1, -1}};
    for (int k = 0; k < 64; ++k) {
      int ch = k >> 5, cp = k & 31, sub = cp >> 4, rr = (cp & 15) >> 1, h = cp & 1;
      const int *t = sub ? tb[rr] : ta[rr];
      uint32_t v;
      if (t[0] < 0) {
        v = 0;
        for (int bb = 0; bb < 3; ++bb) v |= ((e[3 * ch + bb] >> (15 + 16 * h)) & 1u) << bb;
      } else {
        v = (e[3 * ch + t[0]] >> (16 * h + 3 * t[1])) & 7u;
      }
      c[k] = (uint8_t)v;
    }
    uint32_t f = load_fields24(w + a.poff[2] + r * a.prb[2] + (u >> 2) * 12, (int)(u & 3));
    float dv = half_bits(ldh(w + a.poff[3] + r * a.prb[3] + (u >> 2) * 2));
    for (int k = 0; k < 64; ++k) {
      codes[k] = c[k];
      float st = dv * (float)((f >> (6 * (k >> 4))) & 63u);
      vals[k] = st * (float)((int)c[k] - 4);
    }
    return;
  }
  // q5sb / q6sb
  const uint8_t *pl = w + a.poff[0] + r * a.prb[0] + u * 32;
  uint32_t L[8], H[4];
  for (int i = 0; i < 8; ++i) L[i] = ld1(pl + 4 * i);
  const int hbytes = F == 5 ? 8 : 16;
  const uint8_t *ph = w + a.poff[1] + r * a.prb[1] + u * hbytes;
  for (int i = 0; i < hbytes / 4; ++i) H[i] = ld1(ph + 4 * i);
  const int base[4] = {4, 8, 12, 16};
  for (int k = 0; k < 64; ++k) {
    int i = k >> 3, e = k & 7, pk = e >> 1, h = e & 1;
    uint32_t lo = (L[i] >> (4 * ((e >> 1) + 4 * (e & 1)))) & 15u, hi;
    if (F == 5) hi = (H[i >> 2] >> ((base[pk] + 16 * h + (i & 3)) & 31)) & 1u;
    else hi = (H[i >> 1] >> ((base[pk] + 16 * h + 2 * (i & 1)) & 31)) & 3u;
    c[k] = (uint8_t)(lo | (hi << 4));
  }
  if (F == 5) {
    uint32_t f = load_fields24(w + a.poff[2] + r * a.prb[2] + (u >> 2) * 12, (int)(u & 3));
    uint32_t dd = ld1(w + a.poff[3] + r * a.prb[3] + (u >> 2) * 4);
    float dv = half_lo(dd), dm = half_hi(dd);
    for (int h = 0; h < 2; ++h) {
      step[h] = dv * (float)((f >> (6 * h)) & 63u);
      off[h] = dm * (float)((f >> (12 + 6 * h)) & 63u);
    }
    for (int k = 0; k < 64; ++k) {
      codes[k] = c[k];
      vals[k] = __builtin_fmaf(step[k >> 5], (float)c[k], -off[k >> 5]);
    }
  } else {
    uint32_t s = ld1(w + a.poff[2] + r * a.prb[2] + u * 4);
    float dv = half_bits(ldh(w + a.poff[3] + r * a.prb[3] + (u >> 2) * 2));
    for (int k = 0; k < 64; ++k) {
      codes[k] = c[k];
      float st = dv * (float)(int8_t)((s >> (8 * (k >> 4))) & 0xFFu);
      vals[k] = st * (float)((int)c[k] - 32);
    }
  }
}

template <int F>
__global__ void dequant_kernel(GemvArgs a, float *w_out, uint8_t *codes_out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.n * a.units) return;
  const int64_t r = idx / a.units, u = idx % a.units;
  const int nvalid = (int)((a.k - u * 64) < 64 ? (a.k - u * 64) : 64);
  uint8_t codes[64];
  float vals[64];
  decode_unit<F>(a, a.w, r, u, codes, vals, nvalid);
  for (int i = 0; i < nvalid; ++i) {
    if (codes_out) codes_out[r * a.k + u * 64 + i] = codes[i];
    if (w_out) w_out[r * a.k + u * 64 + i] = vals[i];
  }
}

// ------------------------------------------------------------------ host launchers -------

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

thread_local hipError_t g_last_hip_error = hipSuccess;

// hipLaunchKernel returns the launch status itself, so a stale error left in the runtime's
// last-error slot by an unrelated earlier call cannot be mistaken for a failed launch.
template <typename... KArgs, typename... Args>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shm, hipStream_t s, Args... args) {
  void *ptrs[] = {static_cast<void *>(&args)...};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, shm, s);
  if (e != hipSuccess) {
    g_last_hip_error = e;
    return QG_ERR_LAUNCH;
  }
  return QG_OK;
}

namespace {

int fill_args(int fmt, const void *w, int64_t n, int64_t k, GemvArgs &a) {
  qg_layout L;
  int st = qg_device_layout(fmt, n, k, &L);
  if (st != QG_OK) return st;
  a.w = static_cast<const uint8_t *>(w);
  a.n = n;
  a.k = k;
  a.units = (k + kUnit - 1) / kUnit;
  for (int p = 0; p < 4; ++p) {
    a.poff[p] = L.plane_offset[p];
    a.prb[p] = L.plane_row_bytes[p];
  }
  return QG_OK;
}

constexpr int kMaxWk = 16;
constexpr int64_t kSimds = 1024;           // 256 CUs x 4 SIMDs
constexpr int64_t kWavesPerSimd = 4;       // resident waves the kernels' register use allows
constexpr int kMaxBatches = 32;

template <int F, int R>
int launch_gemv_r(GemvArgs a, int64_t count, hipStream_t s) {
  const int64_t groups_per_matrix = (a.n + R - 1) / R;          // batches of R rows
  const int64_t target = kSimds * kWavesPerSimd / a.wk;         // row groups resident at once
  int64_t nb = (groups_per_matrix * count) / target;
  nb = nb < 1 ? 1 : (nb > kMaxBatches ? kMaxBatches : nb);
  a.nb = (int)nb;
  const int64_t rows_per_block = (int64_t)a.wr * R * nb;
  dim3 grid((unsigned)((a.n + rows_per_block - 1) / rows_per_block), (unsigned)count);
  dim3 block((unsigned)(64 * a.wk * a.wr));
  size_t shm = a.wk > 1 ? (size_t)a.wr * R * nb * a.wk * sizeof(float) : 0;
  return launch(gemv_kernel<F, R>, grid, block, shm, s, a);
}

// Rows per batch: 2 (double-buffered, so four rows of loads per wave in flight at 4 waves per
// SIMD without spilling) when there are enough rows to keep every SIMD busy, else 1: small
// problems are bound by latency, so they get as many waves as possible.
template <int F>
int launch_gemv_t(GemvArgs a, int64_t count, hipStream_t s) {
  const int wk = (int)((a.units + 63) / 64);
  a.wk = wk;
  a.wr = wk >= 4 ? 1 : 4 / wk;
  const int64_t rows = a.n * count, target = kSimds * kWavesPerSimd / wk;
  if (rows >= 2 * target) return launch_gemv_r<F, 2>(a, count, s);
  return launch_gemv_r<F, 1>(a, count, s);
}

int launch_gemv(int fmt, GemvArgs a, int64_t count, hipStream_t s) {
  switch (fmt) {
    case 2: return launch_gemv_t<2>(a, count, s);
    case 3: return launch_gemv_t<3>(a, count, s);
    case 4: return launch_gemv_t<4>(a, count, s);
    case 5: return launch_gemv_t<5>(a, count, s);
    case 6: return launch_gemv_t<6>(a, count, s);
  }
  return QG_ERR_FORMAT;
}

}  // namespace

}  // namespace qg

using namespace qg;

extern "C" {

int qg_gemv_batched(int fmt, const void *w, int64_t w_stride, const uint16_t *x, int64_t x_stride, void *y,
                    int64_t y_stride, int y_f32, int64_t count, int64_t n, int64_t k, void *stream) {
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (n < 0 || k < 0 || count < 0) return QG_ERR_SHAPE;
  if ((fmt == 4 && k % 32) || (fmt != 4 && k % kQK)) return QG_ERR_SHAPE;
  if ((k + kUnit - 1) / kUnit > 64 * kMaxWk) return QG_ERR_SHAPE;
  if (count > 65535) return QG_ERR_SHAPE;
  if (n == 0 || count == 0) return QG_OK;
  if (!y || (k > 0 && (!w || !x))) return QG_ERR_NULL;
  if (!aligned(y, y_f32 ? 4 : 2)) return QG_ERR_ALIGN;
  if (count > 1 && y_stride < n) return QG_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (k == 0) {
    int64_t total = n * count;
    return launch(fill_zero_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, y, total, y_f32,
                  y_stride, n);
  }
  if (!aligned(w, 256) || !aligned(x, 16)) return QG_ERR_ALIGN;
  if (count > 1 && (w_stride % 256 || x_stride % 8)) return QG_ERR_ALIGN;
  GemvArgs a{};
  int st = fill_args(fmt, w, n, k, a);
  if (st != QG_OK) return st;
  a.w_bstride = w_stride;
  a.x = x;
  a.x_bstride = x_stride;
  a.y = y;
  a.y_bstride = y_stride;
  a.y_f32 = y_f32;
  return launch_gemv(fmt, a, count, s);
}

int qg_gemv(int fmt, const void *w, const uint16_t *x, void *y, int y_f32, int64_t n, int64_t k, void *stream) {
  return qg_gemv_batched(fmt, w, 0, x, 0, y, n, y_f32, 1, n, k, stream);
}

int dequant_gemv_q4g32(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(4, w, x, y, 0, n, k, s); }
int dequant_gemv_q2sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(2, w, x, y, 0, n, k, s); }
int dequant_gemv_q3sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(3, w, x, y, 0, n, k, s); }
int dequant_gemv_q5sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(5, w, x, y, 0, n, k, s); }
int dequant_gemv_q6sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(6, w, x, y, 0, n, k, s); }

int qg_dequantize(int fmt, const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream) {
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (n < 0 || k < 0 || (fmt == 4 && k % 32) || (fmt != 4 && k % kQK)) return QG_ERR_SHAPE;
  if (n == 0 || k == 0) return QG_OK;
  if (!w || (!w_out && !codes_out)) return QG_ERR_NULL;
  if (!aligned(w, 256) || (w_out && !aligned(w_out, 4))) return QG_ERR_ALIGN;
  GemvArgs a{};
  int st = fill_args(fmt, w, n, k, a);
  if (st != QG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t total = n * a.units;
  dim3 grid((unsigned)((total + 127) / 128)), block(128);
  switch (fmt) {
    case 2: return launch(dequant_kernel<2>, grid, block, 0, s, a, w_out, codes_out);
    case 3: return launch(dequant_kernel<3>, grid, block, 0, s, a, w_out, codes_out);
    case 4: return launch(dequant_kernel<4>, grid, block, 0, s, a, w_out, codes_out);
    case 5: return launch(dequant_kernel<5>, grid, block, 0, s, a, w_out, codes_out);
    case 6: return launch(dequant_kernel<6>, grid, block, 0, s, a, w_out, codes_out);
  }
  return QG_ERR_FORMAT;
}

const char *qg_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

int qg_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
  if (bytes < 0 || bytes % 16) return QG_ERR_SHAPE;
  if (bytes == 0) return QG_OK;
  if (!buf || !sink) return QG_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QG_ERR_ALIGN;
  const int64_t n16 = bytes / 16;
  return launch(read_probe_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                reinterpret_cast<const u32x4 *>(buf), n16, sink);
}

int dequantize_q4g32(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(4, w, o, c, n, k, s); }
int dequantize_q2sb(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(2, w, o, c, n, k, s); }
int dequantize_q3sb(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(3, w, o, c, n, k, s); }
int dequantize_q5sb(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(5, w, o, c, n, k, s); }
int dequantize_q6sb(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(6, w, o, c, n, k, s); }

}  // extern "C"
