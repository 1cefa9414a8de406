// Dequant GEMM for a decode batch of 5 to 16 activation rows on the matrix cores, gfx950.
//
// Method: "二三五六位量化" page section 1.2 and DBHOO-CIM page section 5.2 (a decode batch is
// the GEMV with several activation rows, still bound by the weight stream). On the vector
// units every code pair costs one v_dot2 per activation row, so 8 rows need about 300 TFLOP/s
// at 8 TB/s, twice what v_dot2 delivers. Here each code is decoded once to fp16 w_hat (the
// per-format `wide` decode of units.h, as in the prefill kernel) and the products with all
// activation rows (padded to 16) come from v_mfma_f32_16x16x32_f16 with fp32 accumulation.
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
constexpr int64_t kSkinnyLds = 128 * 1024; // LDS: staging for every wave, then wk * nb * 256 floats
constexpr uint32_t kSkX = 0x7FFFFFF0u;     // activation buffer range; offsets past it read 0
constexpr int64_t kSkinnyWaves = 4096;     // about 4 waves per SIMD

template <int F>
__global__ __launch_bounds__(64 * kSkinnyMaxWk) void skinny_kernel(SkinnyArgs a) {
  using U = Unit<F>;
  using Raw = typename U::Raw;
  static_assert(kDW == 1, "one step of 4 units per wave and pass");
  // [wk][64 lines of kStageLine bytes] staged activations, then [wk][nb][256] partial tiles
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
  float *slots = tiles + (size_t)wk * a.nb * 256;                          // this wave's
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
  half8_t A[kDW][8];
  auto a_load = [&](u32x4 *v, int kp) {
    const int64_t step0 = step_of(kp);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int line = 8 * j + li, arow = line & 15;
      const int64_t u = 4 * step0 + (line >> 4), kk = u * kUnit + 8 * cl;
      const bool ok = arow < a.m && u < a.units && kk < a.k;
      v[j] = bld4c(xr, ok ? (uint32_t)(arow * a.ldx * 2 + kk * 2) : kSkX, 0);
    }
  };
  auto a_stage = [&](const u32x4 *v) {
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4 *>(stage + (8 * j + li) * kStageLine + 16 * cl) = v[j];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8)
      A[0][s8] = *reinterpret_cast<const half8_t *>(stage + lane * kStageLine + 4 * U::pidx(s8 >> 2, 4 * (s8 & 3), 2));
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
    // two accumulators (one per unit half), so that consecutive MFMAs are independent
    f32x4 acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int d = 0; d < kDW; ++d)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t pr[16];
        U::wide(q[d], hh, pr);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const half8_t B = __builtin_bit_cast(half8_t, u32x4{pr[4 * s], pr[4 * s + 1], pr[4 * s + 2], pr[4 * s + 3]});
          acc2[s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[d][4 * hh + s], B, acc2[s & 1], 0, 0, 0);
        }
      }
    const f32x4 acc = acc2[0] + acc2[1];
    // D of a 16 x 16 MFMA: lane l holds column l % 16 (weight row) and rows 4 (l / 16) + e
    // (activation rows); tile index m * 16 + n
    // (each lane owns 4 of the tile's 256 sums; the first pass stores, later passes add)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float &slot = slots[j * 256 + (4 * g + e) * 16 + rl];
      slot = kp == 0 ? acc[e] : slot + acc[e];
    }
  };

  u32x4 v[8];
  Raw qa[kDW], qb[kDW];
  if (a.nb == 1) {
    // one tile per workgroup (small grids): nothing to pipeline
    for (int kp = 0; kp < a.kpasses; ++kp) {
      a_load(v, kp);
      load(qa, kp, 0);
      a_stage(v);
      finish(qa, kp, 0);
    }
  } else {
    // Two register stages over the (pass, tile) sequence, without a drain at the pass
    // boundaries: the last two tiles of a pass also issue the next pass's activation loads
    // and its first tile's weight loads, and the activations are staged after the pass's
    // last MFMAs. (nb is even; every load is unconditional, the last pass "prefetching"
    // itself, so that each wait covers only the oldest stage.)
    a_load(v, 0);
    load(qa, 0, 0);
    a_stage(v);
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
      a_load(v, kn);
      load(qa, kn, 0);
      finish(qb, kp, a.nb - 1);
      a_stage(v);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.nb * 256; i += blockDim.x) {
    const int j = i >> 8, idx = i & 255, mm = idx >> 4;
    const int64_t row = (tile0 + j) * 16 + (idx & 15);
    if (mm >= a.m || row >= a.n) continue;
    float sum = tiles[i];
    for (int w = 1; w < a.wk; ++w) sum += tiles[(size_t)w * a.nb * 256 + i];
    const int64_t o = (int64_t)mm * a.ldy + row;
    if (a.y_f32) reinterpret_cast<float *>(a.y)[o] = sum;
    else reinterpret_cast<_Float16 *>(a.y)[o] = (_Float16)sum;
  }
}

int launch_skinny(int fmt, const void *w, const uint16_t *X, int64_t ldx, void *Y, int64_t ldy, int y_f32,
                  int64_t m, int64_t n, int64_t k, hipStream_t s) {
  qg_layout lay;
  int st = qg_device_layout(fmt, n, k, &lay);
  if (st != QG_OK) return st;
  if (m < 1 || m > 16) return QG_ERR_SHAPE;
  if (16 * ldx * 2 >= (int64_t)kSkX) return QG_ERR_SHAPE;         // 32-bit activation offsets
  SkinnyArgs a{};
  a.w = static_cast<const uint8_t *>(w);
  for (int p = 0; p < 4; ++p) {
    a.poff[p] = lay.plane_offset[p];
    a.prb[p] = lay.plane_row_bytes[p];
  }
  a.n = n;
  a.k = k;
  a.units = (k + kUnit - 1) / kUnit;
  a.x = X;
  a.ldx = ldx;
  a.y = Y;
  a.ldy = ldy;
  a.m = (int)m;
  a.y_f32 = y_f32;
  const int64_t waves_k = (a.units + 4 * kDW - 1) / (4 * kDW);
  const int64_t passes = (waves_k + kSkinnyMaxWk - 1) / kSkinnyMaxWk;
  a.kpasses = (int)passes;
  a.wk = (int)((waves_k + passes - 1) / passes);
  const int64_t tiles = (n + 15) / 16;
  // Row tiles per workgroup: each wave reuses its activation registers for every tile, so
  // more tiles per wave means less activation traffic per weight byte; the grid is kept at
  // about kSkinnyWaves waves so that the CUs stay busy.
  int64_t nb = tiles * a.wk / kSkinnyWaves;
  nb = nb < 1 ? 1 : (nb > kSkinnyMaxNb ? kSkinnyMaxNb : nb);
  nb = (nb + kStages - 1) / kStages * kStages;      // whole pipeline rounds; extra tiles are past n
  const int64_t nb_lds = (kSkinnyLds - a.wk * kStageBytes) / (a.wk * 256 * (int64_t)sizeof(float)) / kStages * kStages;
  if (nb > nb_lds) nb = nb_lds;                     // staging and every wave's partial tiles fit in LDS
  // A grid a little over one workgroup per CU gives most CUs one workgroup and a few two,
  // and every workgroup re-reads all the activation rows of its K range: twice the tiles per
  // workgroup instead, while that still keeps half the CUs busy (11008 x 4096 with 8 or 16
  // rows: 344 workgroups of 2 tiles 16.4 us, 172 of 4 tiles 13.1 us, measured on one MI355X).
  const int64_t wgs = (tiles + nb - 1) / nb, nb2 = nb + kStages;
  if (wgs > 256 && wgs < 384 && nb2 <= kSkinnyMaxNb && nb2 <= nb_lds && (tiles + nb2 - 1) / nb2 >= 128) nb = nb2;
  // At most 256 tiles: two tiles per workgroup would leave at least half the CUs idle, so
  // each workgroup takes one (an unpipelined tile).
  if (nb == kStages && tiles <= 256) nb = 1;
  a.nb = (int)nb;
  const dim3 grid((unsigned)((tiles + nb - 1) / nb)), block((unsigned)(64 * a.wk));
  const size_t shm = (size_t)a.wk * kStageBytes + (size_t)a.wk * nb * 256 * sizeof(float);
  switch (fmt) {
    case 2: return launch(skinny_kernel<2>, grid, block, shm, s, a);
    case 3: return launch(skinny_kernel<3>, grid, block, shm, s, a);
    case 4: return launch(skinny_kernel<4>, grid, block, shm, s, a);
    case 5: return launch(skinny_kernel<5>, grid, block, shm, s, a);
    case 6: return launch(skinny_kernel<6>, grid, block, shm, s, a);
    case 7: return launch(skinny_kernel<7>, grid, block, shm, s, a);
    case 8: return launch(skinny_kernel<8>, grid, block, shm, s, a);
    case 9: return launch(skinny_kernel<9>, grid, block, shm, s, a);
    case 10: return launch(skinny_kernel<10>, grid, block, shm, s, a);
    case 11: return launch(skinny_kernel<11>, grid, block, shm, s, a);
    case 12: return launch(skinny_kernel<12>, grid, block, shm, s, a);
    case 13: return launch(skinny_kernel<13>, grid, block, shm, s, a);
    case 14: return launch(skinny_kernel<3>, grid, block, shm, s, a);   // q3sb's device layout
    case 15: return launch(skinny_kernel<15>, grid, block, shm, s, a);
    case 16: return launch(skinny_kernel<16>, grid, block, shm, s, a);
    case 17: return launch(skinny_kernel<17>, grid, block, shm, s, a);
    case 18: return launch(skinny_kernel<18>, grid, block, shm, s, a);
  }
  return QG_ERR_FORMAT;
}

}  // namespace qg
