// Host side of libqgemv: fp16 rounding, little-endian bitstreams, the five quantizers, the
// canonical encodings and the canonical <-> device layout permutation.
//
// Quantizers follow the DBHOO-CIM page (INT4: sections 2.1 and 3.1, fp32 arithmetic as its
// PyTorch code) and the "二三五六位量化" page (super-blocks: sections 2.1-2.3) with the
// "range-covering round to nearest" scale rule stated in qgemv.h. Every integer decision is
// made with the same IEEE operations in the same order as the rule states; build with
// -ffp-contract=off so no multiply-add is fused.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/qgemv.h"
#include "layout.h"

namespace qg {
namespace {

// ---------------------------------------------------------------- fp16 -------------------

double half_to_double(uint16_t h) {
  int e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp((double)(1024 + m), e - 25);
  return (h & 0x8000) ? -v : v;
}

// Smallest binary16 value >= v for finite v >= 0, as bits. Returns false on overflow.
bool half_ceil(double v, uint16_t *bits) {
  if (!(v >= 0.0) || v > 65504.0) return false;
  if (v == 0.0) { *bits = 0; return true; }
  if (v < std::ldexp(1.0, -14)) {                        // subnormal range: k * 2^-24
    double k = std::ceil(std::ldexp(v, 24));             // exact power-of-two scaling
    *bits = (uint16_t)k;                                 // k == 1024 is 2^-14 = 0x0400
    return true;
  }
  int ex;
  std::frexp(v, &ex);                                    // v in [2^(ex-1), 2^ex)
  int e = ex - 1;
  double k = std::ceil(std::ldexp(v, 10 - e));           // in [1024, 2048]
  if (k >= 2048.0) { k = 1024.0; e += 1; }
  int be = e + 15;
  if (be >= 31) return false;
  *bits = (uint16_t)((be << 10) | ((int)k - 1024));
  return true;
}

// Nearest binary16 value to v for finite v >= 0 (ties to even), as bits. Returns false on
// overflow (v rounds past 65504).
bool half_rn(double v, uint16_t *bits) {
  if (!(v >= 0.0)) return false;
  if (v == 0.0) { *bits = 0; return true; }
  if (v < std::ldexp(1.0, -14)) {                        // subnormal range: k * 2^-24
    *bits = (uint16_t)std::nearbyint(std::ldexp(v, 24));   // k == 1024 is 2^-14 = 0x0400
    return true;
  }
  int ex;
  std::frexp(v, &ex);
  int e = ex - 1;
  double k = std::nearbyint(std::ldexp(v, 10 - e));      // in [1024, 2048], ties to even
  if (k >= 2048.0) { k = 1024.0; e += 1; }
  int be = e + 15;
  if (be >= 31) return false;
  *bits = (uint16_t)((be << 10) | ((int)k - 1024));
  return true;
}

// Smallest bfloat16 value >= v for finite v >= 0, as bits. Returns false on overflow.
bool bf16_ceil(double v, uint16_t *bits) {
  if (!(v >= 0.0) || !std::isfinite(v)) return false;
  float f = (float)v;                                    // round to nearest
  if ((double)f < v) f = std::nextafterf(f, INFINITY);
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if (u & 0xFFFFu) u = (u & 0xFFFF0000u) + 0x10000u;     // round the dropped half up
  if ((u >> 16) >= 0x7F80u) return false;
  *bits = (uint16_t)(u >> 16);
  return true;
}

double bf16_to_double(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// ---------------------------------------------------------------- bitstreams -------------

void pack_le(const uint8_t *codes, int64_t count, int bits, uint8_t *out) {
  int64_t nbytes = (count * bits + 7) / 8;
  std::memset(out, 0, (size_t)nbytes);
  int64_t pos = 0;
  for (int64_t i = 0; i < count; ++i, pos += bits) {
    uint32_t c = codes[i];
    for (int b = 0; b < bits; ++b)
      if ((c >> b) & 1u) out[(pos + b) >> 3] |= (uint8_t)(1u << ((pos + b) & 7));
  }
}

void unpack_le(const uint8_t *in, int64_t count, int bits, uint8_t *codes) {
  int64_t pos = 0;
  for (int64_t i = 0; i < count; ++i, pos += bits) {
    uint32_t c = 0;
    for (int b = 0; b < bits; ++b) c |= (uint32_t)((in[(pos + b) >> 3] >> ((pos + b) & 7)) & 1u) << b;
    codes[i] = (uint8_t)c;
  }
}

inline void put_half(uint8_t *p, uint16_t h) { p[0] = (uint8_t)(h & 0xFF); p[1] = (uint8_t)(h >> 8); }
inline uint16_t get_half(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

// ---------------------------------------------------------------- format specs -----------

struct SB {
  int bits, nsub, sym, offset, smax, rec;
  bool bf16 = false;                                     // super-scales stored as bf16
  int sub() const { return kQK / nsub; }
  int cmax() const { return (1 << bits) - 1; }
};

bool sb_spec(int fmt, SB *s) {
  switch (sb_base(fmt)) {
    case 2: *s = {2, 16, 0, 0, 15, 84}; break;
    case 3: *s = {3, 16, 1, 4, 63, 110}; break;
    case 5: *s = {5, 8, 0, 0, 63, 176}; break;
    case 6: *s = {6, 16, 1, 32, 127, 210}; break;
    default: return false;
  }
  s->bf16 = sb_bf16(fmt);
  return true;
}

// Super-scale rounding and decoding in the format's 16-bit type (fp16, or bf16).
bool scale_ceil(const SB &s, double v, uint16_t *bits) { return s.bf16 ? bf16_ceil(v, bits) : half_ceil(v, bits); }
double scale_value(const SB &s, uint16_t bits) { return s.bf16 ? bf16_to_double(bits) : half_to_double(bits); }

// ---------------------------------------------------------------- quantizers -------------

// One INT4 row: codes (k/2 bytes, canonical nibble order) and fp32 scales (k/32).
int quantize_row_q4(const float *w, int64_t k, int G, uint8_t *codes, float *scales) {
  for (int64_t g = 0; g < k / G; ++g) {
    const float *v = w + g * G;
    float amax = 0.0f;
    for (int i = 0; i < G; ++i) {
      if (!std::isfinite(v[i])) return QG_ERR_NONFINITE;
      float a = std::fabs(v[i]);
      if (a > amax) amax = a;
    }
    float scale = amax / 8.0f;
    if (scale < 1e-12f) scale = 1e-12f;
    scales[g] = scale;
    for (int i = 0; i < G; i += 2) {
      int u[2];
      for (int t = 0; t < 2; ++t) {
        float r = v[i + t] / scale;                  // fp32 quotient
        float q = std::nearbyint(r);                 // round half to even
        if (q < -8.0f) q = -8.0f;
        if (q > 7.0f) q = 7.0f;
        u[t] = (int)q + 8;
      }
      codes[(g * G + i) / 2] = (uint8_t)(u[0] | (u[1] << 4));
    }
  }
  return QG_OK;
}

// One row of plain group-wise b-bit codes (b = 3 or 5) with an fp32 scale and min per group
// of 32: m = min w (a zero minimum stored as +0), s = max((max w - min w) / (2^b - 1), 1e-12),
// c = clamp(rint((w - m) / s), 0, 2^b - 1), the difference and the quotient in fp32; codes
// packed as one little-endian bitstream (k*b/8 bytes).
int quantize_row_gw(const float *w, int64_t k, int b, uint8_t *codes, float *scales, float *mins) {
  const int qmax = (1 << b) - 1;
  std::vector<uint8_t> c((size_t)k);
  for (int64_t g = 0; g < k / 32; ++g) {
    const float *v = w + g * 32;
    float lo = v[0], hi = v[0];
    for (int i = 0; i < 32; ++i) {
      if (!std::isfinite(v[i])) return QG_ERR_NONFINITE;
      if (v[i] < lo) lo = v[i];
      if (v[i] > hi) hi = v[i];
    }
    float scale = (hi - lo) / (float)qmax;
    if (!std::isfinite(scale)) return QG_ERR_RANGE;
    if (scale < 1e-12f) scale = 1e-12f;
    lo = lo + 0.0f;                                      // a zero minimum is stored as +0
    scales[g] = scale;
    mins[g] = lo;
    for (int i = 0; i < 32; ++i) {
      const float diff = v[i] - lo;
      float q = std::nearbyint(diff / scale);
      q = std::min((float)qmax, std::max(0.0f, q));
      c[(size_t)(g * 32 + i)] = (uint8_t)q;
    }
  }
  pack_le(c.data(), k, b, codes);
  return QG_OK;
}

// One INT4 row with fp16 group scales (groups of 32): the INT4 rule with the scale
// max|w| / 8 (fp32) rounded to the nearest fp16 (0 raised to 2^-24), the codes taken
// against that stored scale.
int quantize_row_q4h(const float *w, int64_t k, uint8_t *codes, uint16_t *scales) {
  for (int64_t g = 0; g < k / 32; ++g) {
    const float *v = w + g * 32;
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
      if (!std::isfinite(v[i])) return QG_ERR_NONFINITE;
      float a = std::fabs(v[i]);
      if (a > amax) amax = a;
    }
    uint16_t sb;
    if (!half_rn((double)(amax / 8.0f), &sb)) return QG_ERR_RANGE;
    if (sb == 0) sb = 1;
    scales[g] = sb;
    const float scale = (float)half_to_double(sb);
    for (int i = 0; i < 32; i += 2) {
      int u[2];
      for (int t = 0; t < 2; ++t) {
        float q = std::nearbyint(v[i + t] / scale);
        q = std::min(7.0f, std::max(-8.0f, q));
        u[t] = (int)q + 8;
      }
      codes[(g * 32 + i) / 2] = (uint8_t)(u[0] | (u[1] << 4));
    }
  }
  return QG_OK;
}

// One asymmetric INT4 row (groups of 32): unsigned codes (k/2 bytes, canonical nibble order),
// fp32 scales and uint8 zero points (k/32 each). The group's range is widened to include 0:
// lo = min(0, min w), hi = max(0, max w), s = max((hi - lo) / 15, 1e-12),
// z = clamp(rint(-lo / s), 0, 15), c = clamp(rint(w / s) + z, 0, 15); fp32 throughout.
int quantize_row_q4a(const float *w, int64_t k, uint8_t *codes, float *scales, uint8_t *zeros) {
  for (int64_t g = 0; g < k / 32; ++g) {
    const float *v = w + g * 32;
    float lo = 0.0f, hi = 0.0f;
    for (int i = 0; i < 32; ++i) {
      if (!std::isfinite(v[i])) return QG_ERR_NONFINITE;
      if (v[i] < lo) lo = v[i];
      if (v[i] > hi) hi = v[i];
    }
    float scale = (hi - lo) / 15.0f;
    if (scale < 1e-12f) scale = 1e-12f;
    float zf = std::nearbyint(-lo / scale);
    zf = std::min(15.0f, std::max(0.0f, zf));
    scales[g] = scale;
    zeros[g] = (uint8_t)zf;
    for (int i = 0; i < 32; i += 2) {
      int u[2];
      for (int t = 0; t < 2; ++t) {
        float q = std::nearbyint(v[i + t] / scale) + zf;
        u[t] = (int)std::min(15.0f, std::max(0.0f, q));
      }
      codes[(g * 32 + i) / 2] = (uint8_t)(u[0] | (u[1] << 4));
    }
  }
  return QG_OK;
}

// One super-block: fp32 w[256] -> canonical record.
int quantize_block_sb(const SB &s, int fmt, const float *w, uint8_t *rec) {
  const int sub = s.sub(), nsub = s.nsub, cmax = s.cmax();
  double t[16], off[16] = {0};
  int sc[16] = {0}, m[16] = {0};
  uint8_t c[256];
  uint16_t dbits = 0, dminbits = 0;
  for (int i = 0; i < kQK; ++i)
    if (!std::isfinite(w[i])) return QG_ERR_NONFINITE;
  if (s.sym) {
    double T = 0.0;
    for (int j = 0; j < nsub; ++j) {
      double M = 0.0;
      for (int i = 0; i < sub; ++i) M = std::max(M, std::fabs((double)w[j * sub + i]));
      t[j] = M / (s.offset - 0.5);
      T = std::max(T, t[j]);
    }
    double d = 0.0;
    if (T != 0.0) {
      if (!scale_ceil(s, T / s.smax, &dbits)) return QG_ERR_RANGE;
      d = scale_value(s, dbits);
      for (int j = 0; j < nsub; ++j) sc[j] = (int)std::min((double)s.smax, std::ceil(t[j] / d));
    }
    for (int j = 0; j < nsub; ++j) {
      double step = d * sc[j];
      for (int i = 0; i < sub; ++i) {
        int q = s.offset;
        if (step != 0.0) {
          double r = std::nearbyint((double)w[j * sub + i] / step) + s.offset;
          q = (int)std::min((double)cmax, std::max(0.0, r));
        }
        c[j * sub + i] = (uint8_t)q;
      }
    }
  } else {
    double lo[16], hi[16], L = 0.0;
    for (int j = 0; j < nsub; ++j) {
      double mn = (double)w[j * sub], mx = (double)w[j * sub];
      for (int i = 1; i < sub; ++i) {
        mn = std::min(mn, (double)w[j * sub + i]);
        mx = std::max(mx, (double)w[j * sub + i]);
      }
      lo[j] = std::min(0.0, mn);
      hi[j] = std::max(0.0, mx);
      L = std::max(L, -lo[j]);
    }
    double dmin = 0.0;
    if (L != 0.0) {
      if (!scale_ceil(s, L / s.smax, &dminbits)) return QG_ERR_RANGE;
      dmin = scale_value(s, dminbits);
      for (int j = 0; j < nsub; ++j) m[j] = (int)std::min((double)s.smax, std::ceil(-lo[j] / dmin));
    }
    double T = 0.0;
    for (int j = 0; j < nsub; ++j) {
      off[j] = dmin * m[j];
      t[j] = (hi[j] + off[j]) / cmax;
      T = std::max(T, t[j]);
    }
    double d = 0.0;
    if (T != 0.0) {
      if (!scale_ceil(s, T / s.smax, &dbits)) return QG_ERR_RANGE;
      d = scale_value(s, dbits);
      for (int j = 0; j < nsub; ++j) sc[j] = (int)std::min((double)s.smax, std::ceil(t[j] / d));
    }
    for (int j = 0; j < nsub; ++j) {
      double step = d * sc[j];
      for (int i = 0; i < sub; ++i) {
        int q = 0;
        if (step != 0.0) {
          double r = std::nearbyint(((double)w[j * sub + i] + off[j]) / step);
          q = (int)std::min((double)cmax, std::max(0.0, r));
        }
        c[j * sub + i] = (uint8_t)q;
      }
    }
  }
  // canonical record, fields in the byte table's column order
  std::memset(rec, 0, (size_t)s.rec);
  if (fmt == 2) {
    pack_le(c, 256, 2, rec);
    for (int j = 0; j < 16; ++j) rec[64 + j] = (uint8_t)(sc[j] | (m[j] << 4));
    put_half(rec + 80, dbits);
    put_half(rec + 82, dminbits);
  } else if (fmt == 3 || fmt == kQ3SBPlanes) {
    if (fmt == 3) {
      pack_le(c, 256, 3, rec);
    } else {                                             // 2-bit plane, then 1-bit plane
      uint8_t lo2[256], hi1[256];
      for (int i = 0; i < 256; ++i) { lo2[i] = c[i] & 3; hi1[i] = c[i] >> 2; }
      pack_le(lo2, 256, 2, rec);
      pack_le(hi1, 256, 1, rec + 64);
    }
    uint8_t f[16];
    for (int j = 0; j < 16; ++j) f[j] = (uint8_t)sc[j];
    pack_le(f, 16, 6, rec + 96);
    put_half(rec + 108, dbits);
  } else if (fmt == 5) {
    uint8_t lo4[256], hi1[256], f[16];
    for (int i = 0; i < 256; ++i) { lo4[i] = c[i] & 15; hi1[i] = c[i] >> 4; }
    pack_le(lo4, 256, 4, rec);
    pack_le(hi1, 256, 1, rec + 128);
    for (int j = 0; j < 8; ++j) { f[j] = (uint8_t)sc[j]; f[8 + j] = (uint8_t)m[j]; }
    pack_le(f, 16, 6, rec + 160);
    put_half(rec + 172, dbits);
    put_half(rec + 174, dminbits);
  } else {
    uint8_t lo4[256], hi2[256];
    for (int i = 0; i < 256; ++i) { lo4[i] = c[i] & 15; hi2[i] = c[i] >> 4; }
    pack_le(lo4, 256, 4, rec);
    pack_le(hi2, 256, 2, rec + 128);
    for (int j = 0; j < 16; ++j) rec[192 + j] = (uint8_t)(int8_t)sc[j];
    put_half(rec + 208, dbits);
  }
  return QG_OK;
}

// Run f(r0, r1) over row ranges on a few threads; returns the first error.
template <class F>
int parallel_rows(int64_t n, int64_t work_per_row, F f) {
  unsigned hw = std::thread::hardware_concurrency();
  int64_t nt = std::max<int64_t>(1, std::min<int64_t>(hw ? hw : 1, 16));
  nt = std::min<int64_t>(nt, std::max<int64_t>(1, n * work_per_row / (1 << 18)));
  if (nt <= 1) return f((int64_t)0, n);
  std::vector<std::thread> th;
  std::vector<int> st((size_t)nt, QG_OK);
  int64_t per = (n + nt - 1) / nt;
  for (int64_t t = 0; t < nt; ++t) {
    int64_t r0 = t * per, r1 = std::min(n, r0 + per);
    if (r0 >= r1) break;
    th.emplace_back([&, t, r0, r1] { st[(size_t)t] = f(r0, r1); });
  }
  for (auto &x : th) x.join();
  for (int s : st)
    if (s != QG_OK) return s;
  return QG_OK;
}

bool shape_ok(int fmt, int64_t n, int64_t k) {
  if (n < 0 || k < 0) return false;
  return k % k_multiple(fmt) == 0;
}

// ---------------------------------------------------------------- device layout ----------

inline void setbit(uint32_t *w, int pos, uint32_t v) { if (v) w[pos >> 5] |= 1u << (pos & 31); }
inline uint32_t getbit(const uint32_t *w, int pos) { return (w[pos >> 5] >> (pos & 31)) & 1u; }

// Bit position (dword index within the unit's code dwords * 32 + bit) of bit b of the code
// at unit position k, for the code planes of each format. For q5sb/q6sb this is the low
// nibble (b < 4) in the nibble dwords; high bits are placed by hi_pos().
int code_pos(int fmt, int k, int b) {
  if (q4_group(fmt) || fmt == kQ4A32 || fmt == kQ4G32H || fmt == 5 || fmt == 6) {   // nibble dwords
    int i = k >> 3, e = k & 7;
    return i * 32 + q4_slot(e) * 4 + b;
  }
  if (fmt == 2) {
    int j = k >> 4, t = k >> 1, h = k & 1, r = t & 7;
    return (r >> 1) * 32 + 16 * h + 8 * (r & 1) + 2 * j + b;
  }
  // q3sb chunks
  static const int ta[8][2] = {{0, 0}, {0, 3}, {1, 0}, {1, 3}, {2, 0}, {2, 3}, {0, 1}, {0, 4}};
  static const int tb[8][2] = {{1, 1}, {1, 4}, {2, 1}, {2, 4}, {0, 2}, {1, 2}, {2, 2}, {-1, -1}};
  int c = k >> 5, cp = k & 31, sub = cp >> 4, r = (cp & 15) >> 1, h = cp & 1;
  const int *e = sub ? tb[r] : ta[r];
  if (e[0] < 0) return (3 * c + b) * 32 + 15 + 16 * h;                // spare pair
  return (3 * c + e[0]) * 32 + 16 * h + 3 * e[1] + b;
}

// High-plane bit position of high bit hb of the code at unit position k (q5sb: hb = 0;
// q6sb: hb = 0, 1).
int hi_pos(int fmt, int k, int hb) {
  int i = k >> 3, e = k & 7, pk = e >> 1, h = e & 1;
  static const int base[4] = {4, 8, 12, 16};
  if (fmt == 5) {
    int ip = i & 3, dw = i >> 2;
    return dw * 32 + ((base[pk] + 16 * h + ip) & 31);
  }
  int ip = i & 1, dw = i >> 1;
  return dw * 32 + ((base[pk] + 16 * h + 2 * ip) & 31) + hb;
}

struct Planes {
  uint8_t *p[4];
  int64_t rb[4];
};

// Canonical row -> logical codes + canonical metadata pointers, then scatter to planes.
void row_to_device(int fmt, const uint8_t *canon, int64_t k, int64_t r, int64_t n, Planes P) {
  const int64_t units = (k + kUnit - 1) / kUnit;
  std::vector<uint8_t> codes((size_t)(units * kUnit), 0);
  if (q4_group(fmt) || fmt == kQ4A32 || fmt == kQ4G32H) {
    const int G = q4_group(fmt) ? q4_group(fmt) : 32;
    const uint8_t *cr = canon + r * (k / 2);
    for (int64_t i = 0; i < k; ++i) codes[(size_t)i] = (cr[i >> 1] >> (4 * (i & 1))) & 15;
    uint8_t *ds = P.p[1] + r * P.rb[1];
    if (fmt == kQ4G32H) {                                // fp16 scales, in group order
      std::memcpy(ds, canon + n * (k / 2) + r * (k / 32) * 2, (size_t)(k / 32) * 2);
    } else {
      const uint8_t *sr = canon + n * (k / 2) + r * (k / G) * 4;
      for (int64_t g = 0; g < k / G; ++g) std::memcpy(ds + q4_scale_off(G, units, g), sr + g * 4, 4);
    }
    if (fmt == kQ4A32)                                   // zero points, in group order
      std::memcpy(P.p[2] + r * P.rb[2], canon + n * (k / 2) + n * (k / 32) * 4 + r * (k / 32), (size_t)(k / 32));
    uint8_t *dst = P.p[0] + r * P.rb[0];
    for (int64_t u = 0; u < units; ++u) {
      uint32_t wv[8] = {0};
      for (int kk = 0; kk < kUnit; ++kk)
        for (int b = 0; b < 4; ++b) setbit(wv, code_pos(4, kk, b), (codes[(size_t)(u * kUnit + kk)] >> b) & 1u);
      std::memcpy(dst + split_off(units, u, 0, 16), wv, 16);
      if (k / 2 - u * 32 > 16) std::memcpy(dst + split_off(units, u, 1, 16), wv + 4, 16);
    }
    return;
  }
  int pf = fmt;                                         // code placement: a super-block format
  if (gw_bits(fmt)) {
    const int b = gw_bits(fmt);
    unpack_le(canon + r * (k * b / 8), k, b, codes.data());
    const uint8_t *meta = canon + n * (k * b / 8);        // scales [n][k/32], then mins
    std::memcpy(P.p[2] + r * P.rb[2], meta + r * (k / 32) * 4, (size_t)(k / 32) * 4);
    std::memcpy(P.p[3] + r * P.rb[3], meta + n * (k / 32) * 4 + r * (k / 32) * 4, (size_t)(k / 32) * 4);
    pf = b == 3 ? 3 : 5;
  } else {
  if (fmt == kQ3SBPlanes) pf = 3;
  SB s;
  sb_spec(fmt, &s);
  const int64_t S = k / kQK;
  const uint8_t *row = canon + r * S * s.rec;
  for (int64_t sbi = 0; sbi < S; ++sbi) {
    const uint8_t *rec = row + sbi * s.rec;
    uint8_t *c = &codes[(size_t)(sbi * kQK)];
    if (fmt == 2) {
      unpack_le(rec, 256, 2, c);
      std::memcpy(P.p[1] + r * P.rb[1] + sbi * 16, rec + 64, 16);
      std::memcpy(P.p[2] + r * P.rb[2] + sbi * 4, rec + 80, 4);
    } else if (fmt == 3 || fmt == kQ3SBPlanes) {
      if (fmt == 3) {
        unpack_le(rec, 256, 3, c);
      } else {
        uint8_t lo2[256], hi1[256];
        unpack_le(rec, 256, 2, lo2);
        unpack_le(rec + 64, 256, 1, hi1);
        for (int i = 0; i < 256; ++i) c[i] = (uint8_t)(lo2[i] | (hi1[i] << 2));
      }
      std::memcpy(P.p[2] + r * P.rb[2] + sbi * 12, rec + 96, 12);
      std::memcpy(P.p[3] + r * P.rb[3] + sbi * 2, rec + 108, 2);
    } else if (fmt == 5) {
      uint8_t lo[256], hi[256], f[16], g[16];
      unpack_le(rec, 256, 4, lo);
      unpack_le(rec + 128, 256, 1, hi);
      for (int i = 0; i < 256; ++i) c[i] = (uint8_t)(lo[i] | (hi[i] << 4));
      unpack_le(rec + 160, 16, 6, f);
      for (int q = 0; q < 4; ++q) {                    // [sc_2q, sc_2q+1, m_2q, m_2q+1]
        g[4 * q + 0] = f[2 * q];
        g[4 * q + 1] = f[2 * q + 1];
        g[4 * q + 2] = f[8 + 2 * q];
        g[4 * q + 3] = f[8 + 2 * q + 1];
      }
      pack_le(g, 16, 6, P.p[2] + r * P.rb[2] + sbi * 12);
      std::memcpy(P.p[3] + r * P.rb[3] + sbi * 4, rec + 172, 4);
    } else {
      uint8_t lo[256], hi[256];
      unpack_le(rec, 256, 4, lo);
      unpack_le(rec + 128, 256, 2, hi);
      for (int i = 0; i < 256; ++i) c[i] = (uint8_t)(lo[i] | (hi[i] << 4));
      std::memcpy(P.p[2] + r * P.rb[2] + sbi * 16, rec + 192, 16);
      std::memcpy(P.p[3] + r * P.rb[3] + sbi * 2, rec + 208, 2);
    }
  }
  }
  FmtPlanes fp = fmt_planes(fmt);
  for (int64_t u = 0; u < units; ++u) {
    const uint8_t *cu = &codes[(size_t)(u * kUnit)];
    uint32_t a[8] = {0}, hb[4] = {0};
    for (int kk = 0; kk < kUnit; ++kk) {
      uint32_t cv = cu[kk];
      if (pf == 2) {
        for (int b = 0; b < 2; ++b) setbit(a, code_pos(2, kk, b), (cv >> b) & 1u);
      } else if (pf == 3) {
        for (int b = 0; b < 3; ++b) setbit(a, code_pos(3, kk, b), (cv >> b) & 1u);
      } else {
        for (int b = 0; b < 4; ++b) setbit(a, code_pos(pf, kk, b), (cv >> b) & 1u);
        int nh = pf == 5 ? 1 : 2;
        for (int b = 0; b < nh; ++b) setbit(hb, hi_pos(pf, kk, b), (cv >> (4 + b)) & 1u);
      }
    }
    uint8_t *d0 = P.p[0] + r * P.rb[0] + u * fp.unit_bytes[0];   // (q2sb, q3sb)
    uint8_t *d1 = P.p[1] + r * P.rb[1] + u * fp.unit_bytes[1];
    if (pf == 2) {
      std::memcpy(d0, a, 16);
    } else if (pf == 3) {
      std::memcpy(d0, a, 16);
      std::memcpy(d1, a + 4, 8);
    } else {
      uint8_t *row0 = P.p[0] + r * P.rb[0];
      std::memcpy(row0 + split_off(units, u, 0, 16), a, 16);
      std::memcpy(row0 + split_off(units, u, 1, 16), a + 4, 16);
      std::memcpy(d1, hb, (size_t)fp.unit_bytes[1]);
    }
  }
}

void row_from_device(int fmt, const uint8_t *const *pl, const int64_t *rb, int64_t k, int64_t r, int64_t n,
                     uint8_t *canon) {
  const int64_t units = (k + kUnit - 1) / kUnit;
  FmtPlanes fp = fmt_planes(fmt);
  const int pf = gw_bits(fmt) == 3 || fmt == kQ3SBPlanes ? 3 : gw_bits(fmt) == 5 ? 5 : fmt;   // code placement
  std::vector<uint8_t> codes((size_t)(units * kUnit), 0);
  for (int64_t u = 0; u < units; ++u) {
    uint32_t a[8] = {0}, hb[4] = {0};
    if (q4_group(pf) || pf == kQ4A32 || pf == kQ4G32H) {
      std::memcpy(a, pl[0] + r * rb[0] + split_off(units, u, 0, 16), 16);
      if (k / 2 - u * 32 > 16) std::memcpy(a + 4, pl[0] + r * rb[0] + split_off(units, u, 1, 16), 16);
    } else if (pf == 2) {
      std::memcpy(a, pl[0] + r * rb[0] + u * 16, 16);
    } else if (pf == 3) {
      std::memcpy(a, pl[0] + r * rb[0] + u * 16, 16);
      std::memcpy(a + 4, pl[1] + r * rb[1] + u * 8, 8);
    } else {
      std::memcpy(a, pl[0] + r * rb[0] + split_off(units, u, 0, 16), 16);
      std::memcpy(a + 4, pl[0] + r * rb[0] + split_off(units, u, 1, 16), 16);
      std::memcpy(hb, pl[1] + r * rb[1] + u * fp.unit_bytes[1], (size_t)fp.unit_bytes[1]);
    }
    for (int kk = 0; kk < kUnit; ++kk) {
      uint32_t cv = 0;
      int nb = pf == 2 ? 2 : pf == 3 ? 3 : 4;
      for (int b = 0; b < nb; ++b) cv |= getbit(a, code_pos(pf, kk, b)) << b;
      if (pf == 5 || pf == 6) {
        int nh = pf == 5 ? 1 : 2;
        for (int b = 0; b < nh; ++b) cv |= getbit(hb, hi_pos(pf, kk, b)) << (4 + b);
      }
      codes[(size_t)(u * kUnit + kk)] = (uint8_t)cv;
    }
  }
  if (gw_bits(fmt)) {
    const int b = gw_bits(fmt);
    pack_le(codes.data(), k, b, canon + r * (k * b / 8));
    uint8_t *meta = canon + n * (k * b / 8);
    std::memcpy(meta + r * (k / 32) * 4, pl[2] + r * rb[2], (size_t)(k / 32) * 4);
    std::memcpy(meta + n * (k / 32) * 4 + r * (k / 32) * 4, pl[3] + r * rb[3], (size_t)(k / 32) * 4);
    return;
  }
  if (q4_group(fmt) || fmt == kQ4A32 || fmt == kQ4G32H) {
    const int G = q4_group(fmt) ? q4_group(fmt) : 32;
    uint8_t *cr = canon + r * (k / 2);
    for (int64_t i = 0; i < k; i += 2) cr[i / 2] = (uint8_t)(codes[(size_t)i] | (codes[(size_t)i + 1] << 4));
    if (fmt == kQ4G32H) {
      std::memcpy(canon + n * (k / 2) + r * (k / 32) * 2, pl[1] + r * rb[1], (size_t)(k / 32) * 2);
      return;
    }
    for (int64_t g = 0; g < k / G; ++g)
      std::memcpy(canon + n * (k / 2) + r * (k / G) * 4 + g * 4, pl[1] + r * rb[1] + q4_scale_off(G, units, g), 4);
    if (fmt == kQ4A32)
      std::memcpy(canon + n * (k / 2) + n * (k / 32) * 4 + r * (k / 32), pl[2] + r * rb[2], (size_t)(k / 32));
    return;
  }
  SB s;
  sb_spec(fmt, &s);
  const int64_t S = k / kQK;
  for (int64_t sbi = 0; sbi < S; ++sbi) {
    uint8_t *rec = canon + (r * S + sbi) * s.rec;
    const uint8_t *c = &codes[(size_t)(sbi * kQK)];
    std::memset(rec, 0, (size_t)s.rec);
    if (fmt == 2) {
      pack_le(c, 256, 2, rec);
      std::memcpy(rec + 64, pl[1] + r * rb[1] + sbi * 16, 16);
      std::memcpy(rec + 80, pl[2] + r * rb[2] + sbi * 4, 4);
    } else if (fmt == 3 || fmt == kQ3SBPlanes) {
      if (fmt == 3) {
        pack_le(c, 256, 3, rec);
      } else {
        uint8_t lo2[256], hi1[256];
        for (int i = 0; i < 256; ++i) { lo2[i] = c[i] & 3; hi1[i] = c[i] >> 2; }
        pack_le(lo2, 256, 2, rec);
        pack_le(hi1, 256, 1, rec + 64);
      }
      std::memcpy(rec + 96, pl[2] + r * rb[2] + sbi * 12, 12);
      std::memcpy(rec + 108, pl[3] + r * rb[3] + sbi * 2, 2);
    } else if (fmt == 5) {
      uint8_t lo[256], hi[256], f[16], g[16];
      for (int i = 0; i < 256; ++i) { lo[i] = c[i] & 15; hi[i] = c[i] >> 4; }
      pack_le(lo, 256, 4, rec);
      pack_le(hi, 256, 1, rec + 128);
      unpack_le(pl[2] + r * rb[2] + sbi * 12, 16, 6, g);
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = g[4 * q + 0];
        f[2 * q + 1] = g[4 * q + 1];
        f[8 + 2 * q] = g[4 * q + 2];
        f[8 + 2 * q + 1] = g[4 * q + 3];
      }
      pack_le(f, 16, 6, rec + 160);
      std::memcpy(rec + 172, pl[3] + r * rb[3] + sbi * 4, 4);
    } else {
      uint8_t lo[256], hi[256];
      for (int i = 0; i < 256; ++i) { lo[i] = c[i] & 15; hi[i] = c[i] >> 4; }
      pack_le(lo, 256, 4, rec);
      pack_le(hi, 256, 2, rec + 128);
      std::memcpy(rec + 192, pl[2] + r * rb[2] + sbi * 16, 16);
      std::memcpy(rec + 208, pl[3] + r * rb[3] + sbi * 2, 2);
    }
  }
}

}  // namespace

int layout(int fmt, int64_t n, int64_t k, qg_layout *out) {
  FmtPlanes f = fmt_planes(fmt);
  std::memset(out, 0, sizeof(*out));
  out->nplanes = f.nplanes;
  int64_t off = 0, alg = 0;
  for (int p = 0; p < f.nplanes; ++p) {
    int64_t rbytes = plane_row_bytes(fmt, p, k);
    off = align_up(off, kPlaneAlign);
    out->plane_offset[p] = off;
    out->plane_row_bytes[p] = rbytes;
    off += rbytes * n;
    alg += rbytes * n;
  }
  out->total_bytes = align_up(off, kPlaneAlign);
  out->algorithmic_bytes = alg;
  return QG_OK;
}

}  // namespace qg

using namespace qg;

extern "C" {

int qg_abi_version(void) { return QG_ABI_VERSION; }

const char *qg_strerror(int status) {
  switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "a required pointer is NULL";
    case QG_ERR_SHAPE: return "n, k or m out of range (k must be a multiple of 256 for the super-block formats, of 32 for q4g32, 64 for q4g16, q4g64, q4a32, q4g32h, q3g32 and q5g32, 128 for q4g128)";
    case QG_ERR_ALIGN: return "misaligned device pointer or leading dimension";
    case QG_ERR_NONFINITE: return "a weight is NaN or infinite";
    case QG_ERR_RANGE: return "a super-block scale does not fit fp16 (or bf16), or an fp16 group scale overflows, or a code does not fit its width";
    case QG_ERR_FORMAT: return "unknown format or bit width";
    case QG_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case QG_ERR_DEVICE: return "no usable gfx950 device or HIP runtime error";
    default: return "unknown status";
  }
}

int qg_canonical_bytes(int fmt, int64_t n, int64_t k, int64_t *bytes) {
  if (!bytes) return QG_ERR_NULL;
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (!shape_ok(fmt, n, k)) return QG_ERR_SHAPE;
  if (q4_group(fmt)) { *bytes = n * (k / 2) + n * (k / q4_group(fmt)) * 4; return QG_OK; }
  if (fmt == kQ4A32) { *bytes = n * (k / 2) + n * (k / 32) * 5; return QG_OK; }
  if (fmt == kQ4G32H) { *bytes = n * (k / 2) + n * (k / 32) * 2; return QG_OK; }
  if (gw_bits(fmt)) { *bytes = n * (k * gw_bits(fmt) / 8) + n * (k / 32) * 8; return QG_OK; }
  SB s;
  sb_spec(fmt, &s);
  *bytes = n * (k / kQK) * s.rec;
  return QG_OK;
}

int qg_device_layout(int fmt, int64_t n, int64_t k, qg_layout *out) {
  if (!out) return QG_ERR_NULL;
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (!shape_ok(fmt, n, k)) return QG_ERR_SHAPE;
  return qg::layout(fmt, n, k, out);
}

int qg_packed_bytes(int fmt, int64_t n, int64_t k, int64_t *total, int64_t *algorithmic) {
  qg_layout l;
  const int st = qg_device_layout(fmt, n, k, &l);
  if (st != QG_OK) return st;
  if (total) *total = l.total_bytes;
  if (algorithmic) *algorithmic = l.algorithmic_bytes;
  return QG_OK;
}

int qg_pack_bits(int bits, const uint8_t *codes, int64_t count, uint8_t *out) {
  if (bits < 1 || bits > 8) return QG_ERR_FORMAT;
  if (count < 0) return QG_ERR_SHAPE;
  if (count && (!codes || !out)) return QG_ERR_NULL;
  for (int64_t i = 0; i < count; ++i)
    if (bits < 8 && codes[i] >> bits) return QG_ERR_RANGE;
  pack_le(codes, count, bits, out);
  return QG_OK;
}

int qg_unpack_bits(int bits, const uint8_t *in, int64_t count, uint8_t *codes) {
  if (bits < 1 || bits > 8) return QG_ERR_FORMAT;
  if (count < 0) return QG_ERR_SHAPE;
  if (count && (!codes || !in)) return QG_ERR_NULL;
  unpack_le(in, count, bits, codes);
  return QG_OK;
}

int qg_quantize(int fmt, const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical) {
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (!shape_ok(fmt, n, k) || ldw < k) return QG_ERR_SHAPE;
  if (n == 0 || k == 0) return QG_OK;
  if (!w || !canonical) return QG_ERR_NULL;
  if (q4_group(fmt)) {
    const int G = q4_group(fmt);
    uint8_t *codes = canonical;
    float *scales = reinterpret_cast<float *>(canonical + n * (k / 2));
    // scales start at n*k/2 bytes, a multiple of 16: aligned for float
    return parallel_rows(n, k, [&](int64_t r0, int64_t r1) {
      for (int64_t r = r0; r < r1; ++r) {
        int st = quantize_row_q4(w + r * ldw, k, G, codes + r * (k / 2), scales + r * (k / G));
        if (st != QG_OK) return st;
      }
      return (int)QG_OK;
    });
  }
  if (gw_bits(fmt)) {
    const int b = gw_bits(fmt);
    float *scales = reinterpret_cast<float *>(canonical + n * (k * b / 8));   // k % 64: 4-byte aligned
    float *mins = scales + n * (k / 32);
    return parallel_rows(n, k, [&](int64_t r0, int64_t r1) {
      for (int64_t r = r0; r < r1; ++r) {
        int st = quantize_row_gw(w + r * ldw, k, b, canonical + r * (k * b / 8), scales + r * (k / 32), mins + r * (k / 32));
        if (st != QG_OK) return st;
      }
      return (int)QG_OK;
    });
  }
  if (fmt == kQ4G32H) {
    uint8_t *codes = canonical;
    uint16_t *scales = reinterpret_cast<uint16_t *>(canonical + n * (k / 2));
    return parallel_rows(n, k, [&](int64_t r0, int64_t r1) {
      for (int64_t r = r0; r < r1; ++r) {
        int st = quantize_row_q4h(w + r * ldw, k, codes + r * (k / 2), scales + r * (k / 32));
        if (st != QG_OK) return st;
      }
      return (int)QG_OK;
    });
  }
  if (fmt == kQ4A32) {
    uint8_t *codes = canonical;
    float *scales = reinterpret_cast<float *>(canonical + n * (k / 2));
    uint8_t *zeros = canonical + n * (k / 2) + n * (k / 32) * 4;
    return parallel_rows(n, k, [&](int64_t r0, int64_t r1) {
      for (int64_t r = r0; r < r1; ++r) {
        int st = quantize_row_q4a(w + r * ldw, k, codes + r * (k / 2), scales + r * (k / 32), zeros + r * (k / 32));
        if (st != QG_OK) return st;
      }
      return (int)QG_OK;
    });
  }
  SB s;
  sb_spec(fmt, &s);
  const int64_t S = k / kQK;
  return parallel_rows(n, k, [&](int64_t r0, int64_t r1) {
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t b = 0; b < S; ++b) {
        int st = quantize_block_sb(s, fmt == kQ3SBPlanes ? fmt : sb_base(fmt), w + r * ldw + b * kQK,
                                   canonical + (r * S + b) * s.rec);
        if (st != QG_OK) return st;
      }
    return (int)QG_OK;
  });
}

int quantize_q4g32(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(4, w, n, k, ldw, c); }
int quantize_q4g16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(7, w, n, k, ldw, c); }
int quantize_q4g64(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(8, w, n, k, ldw, c); }
int quantize_q4g128(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(9, w, n, k, ldw, c); }
int quantize_q4a32(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(10, w, n, k, ldw, c); }
int quantize_q4g32h(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(11, w, n, k, ldw, c); }
int quantize_q2sb_bf16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(12, w, n, k, ldw, c); }
int quantize_q3sb_bf16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(13, w, n, k, ldw, c); }
int quantize_q5sb_bf16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(15, w, n, k, ldw, c); }
int quantize_q6sb_bf16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(16, w, n, k, ldw, c); }
int quantize_q3g32(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(17, w, n, k, ldw, c); }
int quantize_q3sb_planes(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(14, w, n, k, ldw, c); }
int quantize_q5g32(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(18, w, n, k, ldw, c); }
int quantize_q2sb(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(2, w, n, k, ldw, c); }
int quantize_q3sb(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(3, w, n, k, ldw, c); }
int quantize_q5sb(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(5, w, n, k, ldw, c); }
int quantize_q6sb(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *c) { return qg_quantize(6, w, n, k, ldw, c); }

int qg_to_device_layout(int fmt, const uint8_t *canonical, int64_t n, int64_t k, uint8_t *dev) {
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (!shape_ok(fmt, n, k)) return QG_ERR_SHAPE;
  qg_layout L;
  qg::layout(fmt, n, k, &L);
  if (L.total_bytes == 0) return QG_OK;
  if (!canonical || !dev) return QG_ERR_NULL;
  std::memset(dev, 0, (size_t)L.total_bytes);
  Planes P;
  for (int p = 0; p < 4; ++p) {
    P.p[p] = dev + L.plane_offset[p];
    P.rb[p] = L.plane_row_bytes[p];
  }
  return parallel_rows(n, k * 4, [&](int64_t r0, int64_t r1) {
    for (int64_t r = r0; r < r1; ++r) row_to_device(fmt == kQ3SBPlanes ? fmt : sb_base(fmt), canonical, k, r, n, P);
    return (int)QG_OK;
  });
}

int qg_from_device_layout(int fmt, const uint8_t *dev, int64_t n, int64_t k, uint8_t *canonical) {
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (!shape_ok(fmt, n, k)) return QG_ERR_SHAPE;
  qg_layout L;
  qg::layout(fmt, n, k, &L);
  if (L.total_bytes == 0) return QG_OK;
  if (!canonical || !dev) return QG_ERR_NULL;
  const uint8_t *pl[4];
  int64_t rb[4];
  for (int p = 0; p < 4; ++p) {
    pl[p] = dev + L.plane_offset[p];
    rb[p] = L.plane_row_bytes[p];
  }
  return parallel_rows(n, k * 4, [&](int64_t r0, int64_t r1) {
    for (int64_t r = r0; r < r1; ++r) row_from_device(fmt == kQ3SBPlanes ? fmt : sb_base(fmt), pl, rb, k, r, n, canonical);
    return (int)QG_OK;
  });
}

}  // extern "C"
