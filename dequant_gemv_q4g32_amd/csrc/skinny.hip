// Dequant GEMM for a decode batch of 5 to 32 activation rows on the matrix cores, gfx950.
//
// Method: "二三五六位量化" page section 1.2 and DBHOO-CIM page section 5.2 (a decode batch is
// the GEMV with several activation rows, still bound by the weight stream). On the vector
// units every code pair costs one v_dot2 per activation row, so 8 rows need about 300 TFLOP/s
// at 8 TB/s, twice what v_dot2 delivers. Here each code is decoded once to fp16 w_hat (the
// per-format `wide` decode of units.h, as in the prefill kernel) and the products with all
// activation rows (padded to 16, or to 32 as two blocks of 16 that share each decoded
// fragment) come from v_mfma_f32_16x16x32_f16 with fp32 accumulation. Each block's sums are
// formed as a 16-row launch on its rows forms them, so the result of a 32-row launch equals
// that of two 16-row launches bit for bit.
//
// Mapping: a wave covers 16 weight rows and 4 * DW units of K per pass. Lane l serves weight
// row l % 16 (the MFMA's N index) and lane group g = l / 16 serves unit g of each group of 4
// consecutive units: it decodes those 64 weights to 32 fp16 pairs, which are the B operands
// of 8 MFMAs (4 pairs each). The A operands are the activations of the same k indices for
// activation row l % 16, loaded once per pass into registers and reused for every row tile
// of the wave. Waves of a workgroup split K; each keeps its partial 16 x 16 tiles in its own
// LDS slots (summed over its passes), and after one barrier the slots are added in wave
// order, so the result does not depend on timing.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/qgemv.h"
#include "device_common.h"
#include "launch.h"
#include "layout.h"
#include "units.h"

namespace qg {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct SkinnyArgs {
  const uint8_t *w;
  int64_t poff[4];
  int64_t prb[4];
  int64_t n, k, units;
  const uint16_t *x;
  int64_t ldx;
  void *y;
  int64_t ldy;
  int m;
  int y_f32;
  int wk;            // waves along K in a workgroup
  int kpasses;       // passes over K
  int nb;            // row tiles (16 rows each) per workgroup
};

constexpr int kDW = 1;                     // steps of 4 units per wave and pass
constexpr int kStages = 2;                  // register stages over row tiles (3 and 4 measured slower)
constexpr int kSkinnyMaxWk = 8;
constexpr int kSkinnyMaxNb = 32;           // row tiles per workgroup (a multiple of kStages)
constexpr int kStageLine = 144;            // bytes per staged activation line (128 + 16 of padding)
constexpr int64_t kStageBytes = 64 * kStageLine;   // one wave's staged activations
constexpr int64_t kSkinnyLds = 160 * 1024; // LDS: staging for every wave, then wk * nb * 256 (32 rows: 512) floats
constexpr uint32_t kSkX = 0x7FFFFFF0u;     // activation buffer range; offsets past it read 0
constexpr int64_t kSkinnyWaves = 4096;     // about 4 waves per SIMD

// MB blocks of 16 activation rows (1: up to 16 rows, 2: up to 32): each decoded weight
// fragment is the B operand of MB MFMAs.
template <int F, int MB>
__global__ __launch_bounds__(64 * kSkinnyMaxWk) void skinny_kernel(SkinnyArgs a) {
  using U = Unit<F>;
  using Raw = typename U::Raw;
  static_assert(kDW == 1, "one step of 4 units per wave and pass");
  static_assert(MB == 1 || MB == 2, "16 or 32 activation rows");
  // [wk][64 lines of kStageLine bytes] staged activations, then [wk][nb][MB][256] partial tiles
  extern __shared__ float red[];
  const int lane = threadIdx.x & 63;
  const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane & 15, g = lane >> 4;
  const int64_t tile0 = (int64_t)blockIdx.x * a.nb;

  Lane L;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    L.rs[p] = make_rsrc(a.w + a.poff[p], (uint32_t)(a.prb[p] * a.n));
    L.prb[p] = (uint32_t)a.prb[p];
  }
  L.set_halves(a.units);
  uint8_t *stage = reinterpret_cast<uint8_t *>(red) + wk * kStageBytes;   // this wave's lines
  float *const tiles = red + (a.wk * kStageBytes) / 4;                    // every wave's partial tiles
  float *slots = tiles + (size_t)wk * a.nb * MB * 256;                     // this wave's
  const rsrc_t xr = make_rsrc(a.x, kSkX);
  const int cl = lane & 7, li = lane >> 3;         // staging loads: chunk, line within 8

  // This wave's units in pass kp: 4 consecutive units; lane group g takes unit 4 * step + g,
  // so a load instruction reads 4 units (64 B or more) of each of its 16 rows contiguously.
  auto step_of = [&](int kp) -> int64_t { return (int64_t)kp * a.wk + wk; };
  auto unit_of = [&](int kp) -> int64_t {
    const int64_t u = 4 * step_of(kp) + g;
    return u < a.units ? u : a.units - 1;
  };
  // activations (A operands) of pass kp: lane (rl, g) needs the 128 bytes of activation row
  // rl in unit g, the "line" rl + 16 g. Loaded with 8 consecutive lanes per line (instruction
  // j reads lines 8j..8j+7, one cache line each), written to this wave's LDS lines, and each
  // lane reads its own line back: for MFMA s of a unit, local pairs 4 (s & 3).. of half s >> 2.
  // With 32 rows, block b (rows 16 b ..) goes through the same lines after block 0.
  half8_t A[MB][8];
  auto a_load = [&](u32x4 *v, int kp, int b) {
    const int64_t step0 = step_of(kp);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int line = 8 * j + li, arow = (line & 15) + 16 * b;
      const int64_t u = 4 * step0 + (line >> 4), kk = u * kUnit + 8 * cl;
      const bool ok = arow < a.m && u < a.units && kk < a.k;
      v[j] = bld4c(xr, ok ? (uint32_t)(arow * a.ldx * 2 + kk * 2) : kSkX, 0);
    }
  };
  auto a_stage = [&](const u32x4 *v, int b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4 *>(stage + (8 * j + li) * kStageLine + 16 * cl) = v[j];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8)
      A[b][s8] = *reinterpret_cast<const half8_t *>(stage + lane * kStageLine + 4 * U::pidx(s8 >> 2, 4 * (s8 & 3), 2));
  };
  // every block of pass kp: loaded together, staged one after the other through the same
  // lines (a wave's LDS accesses complete in order, so block 0's reads precede block 1's writes)
  auto a_load_all = [&](u32x4 (*v)[8], int kp) {
#pragma unroll
    for (int b = 0; b < MB; ++b) a_load(v[b], kp, b);
  };
  auto a_stage_all = [&](u32x4 (*v)[8]) {
#pragma unroll
    for (int b = 0; b < MB; ++b) a_stage(v[b], b);
  };

  // weights of row tile j in pass kp (a tile past the workgroup's last re-loads that one)
  auto load = [&](Raw *q, int kp, int j) {
    const int64_t t = tile0 + (j < a.nb ? j : a.nb - 1);
    int64_t row = t * 16 + rl;
    row = row < a.n ? row : a.n - 1;
    const int64_t unit = unit_of(kp);
#pragma unroll
    for (int d = 0; d < kDW; ++d) {
      Lane Ld = L;
#pragma unroll
      for (int p = 0; p < 4; ++p) Ld.off[p] = 0;
      U::offsets(unit, Ld.off);
      Ld.sh = fields_sh(unit);
#pragma unroll
      for (int p = 0; p < 4; ++p) Ld.off[p] += (uint32_t)row * Ld.prb[p];
      const bool half = (F == 4) && (unit == a.units - 1) && (a.k % 64 != 0);
      // default cache policy: a load reads 64 bytes of each of its 16 rows, and the other half
      // of those 128-byte lines belongs to the next wave's units in the same pass; with the
      // non-temporal hint the lines were often gone by then (HBM fetch 1.25 x the weight bytes
      // on 28672 x 8192, and 3-10% slower)
      U::template load<0>(q[d], Ld, 0, half);
    }
  };
  auto finish = [&](const Raw *q, int kp, int j) {
    // two accumulators per row block (one per unit half), so that consecutive MFMAs are
    // independent
    f32x4 acc2[MB][2];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc2[b][0] = acc2[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint32_t pr[16];
      U::wide(q[0], hh, pr);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const half8_t B = __builtin_bit_cast(half8_t, u32x4{pr[4 * s], pr[4 * s + 1], pr[4 * s + 2], pr[4 * s + 3]});
#pragma unroll
        for (int b = 0; b < MB; ++b)
          acc2[b][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[b][4 * hh + s], B, acc2[b][s & 1], 0, 0, 0);
      }
    }
    // D of a 16 x 16 MFMA: lane l holds column l % 16 (weight row) and rows 4 (l / 16) + e
    // (activation rows of the block); tile index (j MB + b) 256 + m * 16 + n
    // (each lane owns 4 of the block's 256 sums; the first pass stores, later passes add)
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const f32x4 acc = acc2[b][0] + acc2[b][1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float &slot = slots[(j * MB + b) * 256 + (4 * g + e) * 16 + rl];
        slot = kp == 0 ? acc[e] : slot + acc[e];
      }
    }
  };

  u32x4 v[MB][8];
  Raw qa[kDW], qb[kDW];
  if (a.nb == 1) {
    // one tile per workgroup (small grids): nothing to pipeline
    for (int kp = 0; kp < a.kpasses; ++kp) {
      a_load_all(v, kp);
      load(qa, kp, 0);
      a_stage_all(v);
      finish(qa, kp, 0);
    }
  } else {
    // Two register stages over the (pass, tile) sequence, without a drain at the pass
    // boundaries: the last two tiles of a pass also issue the next pass's activation loads
    // and its first tile's weight loads, and the activations are staged after the pass's
    // last MFMAs. (nb is even; every load is unconditional, the last pass "prefetching"
    // itself, so that each wait covers only the oldest stage.)
    a_load_all(v, 0);
    load(qa, 0, 0);
    a_stage_all(v);
    for (int kp = 0; kp < a.kpasses; ++kp) {
      const int kn = kp + 1 < a.kpasses ? kp + 1 : kp;
      for (int j = 0; j + 2 < a.nb; j += 2) {
        load(qb, kp, j + 1);
        finish(qa, kp, j);
        load(qa, kp, j + 2);
        finish(qb, kp, j + 1);
      }
      load(qb, kp, a.nb - 1);
      finish(qa, kp, a.nb - 2);
      a_load_all(v, kn);
      load(qa, kn, 0);
      finish(qb, kp, a.nb - 1);
      a_stage_all(v);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.nb * MB * 256; i += blockDim.x) {
    const int j = i / (MB * 256), b = (i >> 8) % MB, idx = i & 255, mm = 16 * b + (idx >> 4);
    const int64_t row = (tile0 + j) * 16 + (idx & 15);
    if (mm >= a.m || row >= a.n) continue;
    float sum = tiles[i];
    for (int w = 1; w < a.wk; ++w) sum += tiles[(size_t)w * a.nb * MB * 256 + i];
    const int64_t o = (int64_t)mm * a.ldy + row;
    if (a.y_f32) reinterpret_cast<float *>(a.y)[o] = sum;
    else reinterpret_cast<_Float16 *>(a.y)[o] = (_Float16)sum;
  }
}

template <int MB>
static int launch_fmt(int fmt, dim3 grid, dim3 block, size_t shm, hipStream_t s, const SkinnyArgs &a) {
  switch (fmt) {
    case 2: return launch(skinny_kernel<2, MB>, grid, block, shm, s, a);
    case 3: return launch(skinny_kernel<3, MB>, grid, block, shm, s, a);
    case 4: return launch(skinny_kernel<4, MB>, grid, block, shm, s, a);
    case 5: return launch(skinny_kernel<5, MB>, grid, block, shm, s, a);
    case 6: return launch(skinny_kernel<6, MB>, grid, block, shm, s, a);
    case 7: return launch(skinny_kernel<7, MB>, grid, block, shm, s, a);
    case 8: return launch(skinny_kernel<8, MB>, grid, block, shm, s, a);
    case 9: return launch(skinny_kernel<9, MB>, grid, block, shm, s, a);
    case 10: return launch(skinny_kernel<10, MB>, grid, block, shm, s, a);
    case 11: return launch(skinny_kernel<11, MB>, grid, block, shm, s, a);
    case 12: return launch(skinny_kernel<12, MB>, grid, block, shm, s, a);
    case 13: return launch(skinny_kernel<13, MB>, grid, block, shm, s, a);
    case 14: return launch(skinny_kernel<3, MB>, grid, block, shm, s, a);   // q3sb's device layout
    case 15: return launch(skinny_kernel<15, MB>, grid, block, shm, s, a);
    case 16: return launch(skinny_kernel<16, MB>, grid, block, shm, s, a);
    case 17: return launch(skinny_kernel<17, MB>, grid, block, shm, s, a);
    case 18: return launch(skinny_kernel<18, MB>, grid, block, shm, s, a);
  }
  return QG_ERR_FORMAT;
}

// Launch shape of the kernel for m x n x k (m <= 32): waves per workgroup (each a slice of
// K), passes over K, row tiles per workgroup, workgroups, LDS bytes.
struct SkinnyPlan {
  int mb, wk, kpasses, nb;
  int64_t units, wgs;
  size_t shm;
};

static SkinnyPlan skinny_plan(int64_t m, int64_t n, int64_t k) {
  SkinnyPlan p{};
  p.mb = m > 16 ? 2 : 1;                                  // blocks of 16 activation rows
  p.units = (k + kUnit - 1) / kUnit;
  const int64_t waves_k = (p.units + 4 * kDW - 1) / (4 * kDW);
  const int64_t passes = (waves_k + kSkinnyMaxWk - 1) / kSkinnyMaxWk;
  p.kpasses = (int)passes;
  p.wk = (int)((waves_k + passes - 1) / passes);
  const int64_t tiles = (n + 15) / 16;
  // Row tiles per workgroup: each wave reuses its activation registers for every tile, so
  // more tiles per wave means less activation traffic per weight byte; the grid is kept at
  // about kSkinnyWaves waves so that the CUs stay busy.
  int64_t nb = tiles * p.wk / kSkinnyWaves;
  nb = nb < 1 ? 1 : (nb > kSkinnyMaxNb ? kSkinnyMaxNb : nb);
  nb = (nb + kStages - 1) / kStages * kStages;      // whole pipeline rounds; extra tiles are past n
  // staging and every wave's partial tiles fit in the CU's LDS
  const int64_t nb_lds = (kSkinnyLds - p.wk * kStageBytes) / (p.wk * p.mb * 256 * (int64_t)sizeof(float)) / kStages * kStages;
  if (nb > nb_lds) nb = nb_lds;
  // A grid of more than one workgroup per CU runs in two rounds, and every workgroup
  // re-reads all the activation rows of its K range: the next larger tile count (by one or
  // two pipeline rounds) whose grid fits one round and still keeps half the CUs busy
  // instead (measured on one MI355X, q4g32: 11008 x 4096 at 8 or 16 rows, 344 workgroups of
  // 2 tiles 16.4 us, 172 of 4 tiles 13.1 us; 12288 x 4096 at 16 rows, 384 of 2 18.9 us,
  // 192 of 4 15.3 us; 14336 x 4096 at 16 rows, 448 of 2 19.1 us, 224 of 4 15.2 us;
  // 28672 x 8192 at 16 rows, 448 of 4 50.7 us, 224 of 8 44.8 us; 22016 x 4096 at 16 rows,
  // 688 of 2 27.9 us, 230 of 6 20.1 us).
  if ((tiles + nb - 1) / nb > 256) {
    for (int64_t nb2 = nb + kStages; nb2 <= nb + 2 * kStages; nb2 += kStages) {
      const int64_t wgs2 = (tiles + nb2 - 1) / nb2;
      if (wgs2 <= 256 && wgs2 >= 128 && nb2 <= kSkinnyMaxNb && nb2 <= nb_lds) {
        nb = nb2;
        break;
      }
    }
  }
  // At most 256 tiles: two tiles per workgroup would leave at least half the CUs idle, so
  // each workgroup takes one (an unpipelined tile).
  if (nb == kStages && tiles <= 256) nb = 1;
  p.nb = (int)nb;
  p.wgs = (tiles + nb - 1) / nb;
  p.shm = (size_t)p.wk * kStageBytes + (size_t)p.wk * nb * p.mb * 256 * sizeof(float);
  return p;
}

double skinny_us(int fmt, int64_t m, int64_t n, int64_t k) {
  qg_layout lay;
  if (m < 1 || m > 32 || n < 1 || k < 1 || qg_device_layout(fmt, n, k, &lay) != QG_OK) return 1e30;
  const SkinnyPlan p = skinny_plan(m, n, k);
  // workgroups resident per CU: LDS, and VGPRs (about 136 per lane with 16 rows, 200 with 32:
  // 3 or 2 waves per SIMD)
  int64_t per_cu = kSkinnyLds / (int64_t)p.shm;
  const int64_t by_vgpr = 4 * (p.mb == 2 ? 2 : 3) / p.wk;
  if (by_vgpr < per_cu) per_cu = by_vgpr;
  if (per_cu < 1) per_cu = 1;
  const int64_t rounds = (p.wgs + 256 * per_cu - 1) / (256 * per_cu);
  // fitted to one MI355X over 4096-28672 x 4096-11008 in q3sb, q4g32 and q5sb: a (tile, pass)
  // of a CU's work 1.3 us, a further round 4 us, 2 us fixed; bytes per weight relative to
  // q4g32's 0.625 enter with the square root; 32 rows 1.35 x the time of 16
  const double rel = std::sqrt((double)lay.algorithmic_bytes / ((double)n * (double)k * 0.625));
  const double t = 2.0 + 1.3 * (double)(p.kpasses * p.nb * rounds) + 4.0 * (double)(rounds - 1);
  return t * rel * (p.mb == 2 ? 1.35 : 1.0);
}

int launch_skinny(int fmt, const void *w, const uint16_t *X, int64_t ldx, void *Y, int64_t ldy, int y_f32,
                  int64_t m, int64_t n, int64_t k, hipStream_t s) {
  qg_layout lay;
  int st = qg_device_layout(fmt, n, k, &lay);
  if (st != QG_OK) return st;
  if (m < 1 || m > 32) return QG_ERR_SHAPE;
  const SkinnyPlan p = skinny_plan(m, n, k);
  if (16 * p.mb * ldx * 2 >= (int64_t)kSkX) return QG_ERR_SHAPE;  // 32-bit activation offsets
  SkinnyArgs a{};
  a.w = static_cast<const uint8_t *>(w);
  for (int q = 0; q < 4; ++q) {
    a.poff[q] = lay.plane_offset[q];
    a.prb[q] = lay.plane_row_bytes[q];
  }
  a.n = n;
  a.k = k;
  a.units = p.units;
  a.x = X;
  a.ldx = ldx;
  a.y = Y;
  a.ldy = ldy;
  a.m = (int)m;
  a.y_f32 = y_f32;
  a.kpasses = p.kpasses;
  a.wk = p.wk;
  a.nb = p.nb;
  const dim3 grid((unsigned)p.wgs), block((unsigned)(64 * p.wk));
  return p.mb == 2 ? launch_fmt<2>(fmt, grid, block, p.shm, s, a) : launch_fmt<1>(fmt, grid, block, p.shm, s, a);
}

}  // namespace qg

