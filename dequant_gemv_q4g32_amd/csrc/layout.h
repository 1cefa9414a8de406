// Device layout of the packed formats: planes, per-lane units and bit placement.
//
// The unit of work of one lane is 64 consecutive weights of one row ("lane unit"). Every
// plane is [n][row_bytes] row-major with row_bytes = (k / 64) * unit_bytes, so that lane u
// of a wave reads its unit with one or two 128-bit (or 64/32-bit) loads and consecutive
// lanes read consecutive bytes.
//
// Inside a unit the codes are placed so that one v_and_or_b32 (mask, | 0x6400 in both
// halves) yields a pair of fp16 values (1024 + p*c_a, 1024 + p*c_b) for a power of two p,
// which v_dot2_f32_f16 multiplies with the activation pair (x[2t], x[2t+1]). The 1024 and
// the code offsets are folded into per-lane constants computed once from x.
//
// Placement per format (positions are unit-relative weight indices 0..63; "pair t" means
// weights 2t (low fp16 half, bits 0..15) and 2t+1 (high half, bits 16..31)):
//
//  q4g32  plane 0 codes: 8 dwords/unit, dword i holds weights 8i..8i+7, weight 8i+e in
//         nibble slot (e>>1) + 4*(e&1); plane 1 fp32 scales (one per group of 32).
//  q4a32  (asymmetric) planes 0 and 1 as q4g32 (unsigned codes), plane 2 uint8 zero points,
//         2 bytes per unit in group order (not split).
//  q4g32h plane 0 as q4g32; plane 1 fp16 scales in group order (one dword per unit).
//  q3g32  planes 0 and 1 as q3sb (a unit's two chunks of 32 codes are its two groups);
//         planes 2 and 3 fp32 scales and fp32 mins, two per unit in group order.
//  q5g32  planes 0 and 1 as q5sb (a unit's two sub-blocks of 32 are its two groups); planes
//         2 and 3 fp32 scales and fp32 mins, two per unit in group order.
//         Split halves (also the q5sb/q6sb nibble planes): a row of a 32-byte-per-unit plane
//         stores the first 16 bytes of every unit, then the second 16 bytes of every unit
//         (dwords 0-3 of unit u at 16u, dwords 4-7 at 16 units + 16u); the q4g32 scale plane
//         likewise stores every unit's first scale, then every unit's second scale. Each
//         128-bit (32-bit) load of a wave then reads one contiguous run of 1 KB (256 B).
//         A ragged q4g32 row (k % 64 == 32) has no second half for its last unit.
//  q2sb   plane 0 codes: 4 dwords/unit (a quarter super-block, 4 sub-blocks j of 16).
//         Pair t of sub-block j = t>>3, r = t&7 sits in dword r>>1 at bit 2j + 8*(r&1)
//         (+16 for the high half). Extraction mask 0x00030003 << 2j, class p = 4^j.
//         plane 1 sub-block bytes (sc | m<<4, 4 per unit), plane 2 (fp16 d, fp16 dmin).
//  q3sb   plane 0 (16 B/unit) + plane 1 (8 B/unit): two chunks of three dwords E0..E2, each
//         chunk holding 32 codes = sub-blocks a (first 16) and b. Each 16-bit half holds five
//         3-bit fields f0..f4 at bits 0,3,6,9,12; bit 15 is a spare. Sub-block a pairs
//         r=0..7 -> (E0,f0) (E0,f3) (E1,f0) (E1,f3) (E2,f0) (E2,f3) (E0,f1) (E0,f4);
//         sub-block b pairs -> (E1,f1) (E1,f4) (E2,f1) (E2,f4) (E0,f2) (E1,f2) (E2,f2) spare,
//         where the spare pair's code bits 0,1,2 are bit 15 of E0,E1,E2 (low half) and
//         bit 31 (high half). Plane 0 = chunk0 E0 E1 E2, chunk1 E0; plane 1 = chunk1 E1 E2.
//         plane 2: 12 B/super-block of 6-bit sub-scales (canonical order), plane 3 fp16 d.
//  q5sb   plane 0 low nibbles: 8 dwords/unit in the q4g32 nibble placement. plane 1 high
//         bits: 2 dwords/unit; dword h serves nibble dwords 4h..4h+3 (sub-block h). For
//         nibble dword i (i' = i & 3) and its pairs k = 0..3 (weights (2k, 2k+1) of the
//         dword) the high bits sit at bits {4,20}+i', {8,24}+i', {12,28}+i', {16,0}+i'.
//         plane 2: 3 B/unit of 6-bit fields [sc_2q, sc_2q+1, m_2q, m_2q+1]; plane 3 (d, dmin).
//  q6sb   plane 0 low nibbles as q5sb. plane 1 high 2-bit fields: 4 dwords/unit; dword h
//         serves nibble dwords 2h, 2h+1 (sub-block h); for i' = i & 1 the 2-bit fields sit at
//         bits {4,20}+2i', {8,24}+2i', {12,28}+2i', {16,0}+2i'. plane 2 int8 sub-scales,
//         plane 3 fp16 d.
#pragma once
#include <stdint.h>

namespace qg {

constexpr int kUnit = 64;          // weights per lane unit
constexpr int kQK = 256;           // weights per super-block
constexpr int64_t kPlaneAlign = 256;

// Byte offset, within a row of a split-halves plane, of half `second` of unit u (each half
// `hb` bytes; `units` units per row). Shared by the host packer and the device decoder.
#if defined(__HIP__)
#define QG_HOST_DEVICE __host__ __device__
#else
#define QG_HOST_DEVICE
#endif
QG_HOST_DEVICE inline int64_t split_off(int64_t units, int64_t u, int second, int hb) { return (second ? units * hb : 0) + u * hb; }

// Byte offset, within a row of an INT4 group format's scale plane, of the fp32 scale of
// group g (G weights per group; units lane units per row).
QG_HOST_DEVICE inline int64_t q4_scale_off(int G, int64_t units, int64_t g) {
  if (G == 32) return split_off(units, g >> 1, (int)(g & 1), 4);
  if (G == 16) return split_off(units, g >> 2, (int)((g >> 1) & 1), 8) + 4 * (g & 1);
  return 4 * g;                                     // groups of 64 and 128: in order
}

// Bytes per lane unit of each plane, and the number of planes.
struct FmtPlanes {
  int nplanes;
  int unit_bytes[4];   // bytes per 64-weight unit; 0 for planes sized per super-block
  int sb_bytes[4];     // bytes per 256-weight super-block (when unit_bytes == 0)
};

// INT4 symmetric group formats: group size of the format code (0 for the super-block formats).
// Codes 7, 8 and 9 are groups of 16, 64 and 128; they share q4g32's code plane (units of 64
// weights, split halves) and differ only in the fp32 scale plane: 4 scales per unit in split
// halves of 8 bytes (group 16; half h of unit u holds groups 4u + 2h, 4u + 2h + 1), one per
// unit (group 64), one per two units (group 128).
QG_HOST_DEVICE constexpr int q4_group(int fmt) { return fmt == 4 ? 32 : fmt == 7 ? 16 : fmt == 8 ? 64 : fmt == 9 ? 128 : 0; }

// INT4 asymmetric, groups of 32 with a zero point (code 10); INT4 symmetric, groups of 32
// with fp16 scales (code 11).
constexpr int kQ4A32 = 10;
constexpr int kQ4G32H = 11;

// Super-block formats with bf16 super-scales d (and dmin): the base format's code + 10
// (12, 13, 15, 16 for q2sb, q3sb, q5sb, q6sb). Same records, planes and kernels as the base
// format; only the 16-bit super-scale fields hold bf16 instead of fp16.
// q3sb_planes (code 14) is q3sb with the record's codes in a 2-bit and a 1-bit plane: its
// device layout is q3sb's.
constexpr int kQ3SBPlanes = 14;
QG_HOST_DEVICE constexpr bool sb_bf16(int fmt) { return fmt == 12 || fmt == 13 || fmt == 15 || fmt == 16; }
QG_HOST_DEVICE constexpr int sb_base(int fmt) { return sb_bf16(fmt) ? fmt - 10 : fmt == kQ3SBPlanes ? 3 : fmt; }

// Plain group-wise codes with an fp32 scale and min per group of 32: 3-bit (code 17) and
// 5-bit (code 18); code bits of the format (0 for the others).
constexpr int kQ3G32 = 17;
constexpr int kQ5G32 = 18;
QG_HOST_DEVICE constexpr int gw_bits(int fmt) { return fmt == kQ3G32 ? 3 : fmt == kQ5G32 ? 5 : 0; }

inline bool fmt_valid(int fmt) {
  return (fmt >= 2 && fmt <= 6) || q4_group(fmt) != 0 || fmt == kQ4A32 || fmt == kQ4G32H || sb_bf16(fmt) ||
         gw_bits(fmt) != 0 || fmt == kQ3SBPlanes;
}

// K must be a multiple of this: 32 for q4g32 (a row may end in half a unit), whole units
// (64) for q4g16, q4g64, q4a32, q4g32h, q3g32 and q5g32, 128 for q4g128, a super-block
// (256) for the other formats.
inline int64_t k_multiple(int fmt) {
  if (fmt == kQ4A32 || fmt == kQ4G32H || gw_bits(fmt)) return kUnit;
  const int G = q4_group(fmt);
  return G == 32 ? 32 : G ? (G > kUnit ? G : kUnit) : kQK;
}

inline FmtPlanes fmt_planes(int fmt) {
  switch (sb_base(fmt)) {
    case 4: return {2, {32, 8, 0, 0}, {0, 0, 0, 0}};          // codes, fp32 scales
    case 2: return {3, {16, 4, 0, 0}, {0, 0, 4, 0}};          // codes, sc|m, (d, dmin)
    case 3: return {4, {16, 8, 0, 0}, {0, 0, 12, 2}};         // codes A, codes B, sc, d
    case 5: return {4, {32, 8, 0, 0}, {0, 0, 12, 4}};         // lo, hi, sc/m, (d, dmin)
    case 6: return {4, {32, 16, 4, 0}, {0, 0, 0, 2}};         // lo, hi, sc, d
    case 7: return {2, {32, 16, 0, 0}, {0, 0, 0, 0}};         // codes, 4 fp32 scales per unit
    case 8: return {2, {32, 4, 0, 0}, {0, 0, 0, 0}};          // codes, 1 fp32 scale per unit
    case 9: return {2, {32, 2, 0, 0}, {0, 0, 0, 0}};          // codes, 1 fp32 scale per 2 units
    case 10: return {3, {32, 8, 2, 0}, {0, 0, 0, 0}};         // codes, fp32 scales, zero points
    case 11: return {2, {32, 4, 0, 0}, {0, 0, 0, 0}};         // codes, fp16 scales
    case 17: return {4, {16, 8, 8, 8}, {0, 0, 0, 0}};         // codes A, codes B, scales, mins
    case 18: return {4, {32, 8, 8, 8}, {0, 0, 0, 0}};         // lo, hi, scales, mins
    default: return {0, {0, 0, 0, 0}, {0, 0, 0, 0}};
  }
}

// Row bytes of plane p for a row of k weights (k a multiple of 256 for the super-block
// formats, of 32 for q4g32, of 64 for q4g16, q4g64, q4a32, q4g32h, q3g32 and q5g32, of 128
// for q4g128).
inline int64_t plane_row_bytes(int fmt, int p, int64_t k) {
  FmtPlanes f = fmt_planes(fmt);
  if (fmt == 4) return p == 0 ? k / 2 : (k / 32) * 4;
  if (fmt == kQ4A32) return p == 0 ? k / 2 : p == 1 ? (k / 32) * 4 : k / 32;
  if (fmt == kQ4G32H) return p == 0 ? k / 2 : (k / 32) * 2;
  if (q4_group(fmt)) return p == 0 ? k / 2 : (k / q4_group(fmt)) * 4;
  if (f.unit_bytes[p]) return (k / kUnit) * f.unit_bytes[p];
  return (k / kQK) * f.sb_bytes[p];
}

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// q4g32 nibble slot of weight e (0..7) inside a code dword.
inline int q4_slot(int e) { return (e >> 1) + 4 * (e & 1); }

}  // namespace qg
