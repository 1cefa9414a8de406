// Dequant GEMM for prefill-sized m, gfx950: Y = X * W_hat^T with W_hat tiles dequantized to
// fp16 in LDS and multiplied on the matrix cores (v_mfma_f32_32x32x16_f16, fp32 accumulate).
//
// Method: "二三五六位量化" page section 1.2 (prefill multiplies the same low-bit weights by
// many activation rows, so the work is a dense contraction; the dequantized weights are fp16)
// and DBHOO-CIM page section 5.2 (large prefill batches turn compute-bound). The codes are turned
// into fp16 w_hat by the same per-format unit decode as the GEMV (units.h, `wide`), written
// once per K step into an LDS tile that every wave of the workgroup reads.
//
// Tiling: a workgroup of 4 waves computes a 128 x BN tile of Y (128 activation rows x BN =
// 128 or 96 weight rows) and walks K in steps of one 64-weight unit. Each step, every thread
// loads half a unit of one weight row (the first 2 * BN threads) and 16 bytes of each of 4
// activation rows (two steps ahead, into one of two register stages), decodes its half unit
// to 16 fp16 pairs and stores both into one of two LDS buffers. Each wave then runs 2 x 2
// (BN = 128) or 1 x 3 (BN = 96) MFMA tiles of 32 x 32 over the step's 4 K-slices of 16.
// Workgroups are numbered so that the M tiles sharing a weight tile run on one XCD and share
// its L2.
#include <hip/hip_runtime.h>

#include "../../include/qgemv.h"
#include "device_common.h"
#include "launch.h"
#include "layout.h"
#include "units.h"

namespace qg {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct PrefillArgs {
  const uint8_t *w;
  int64_t poff[4];
  int64_t prb[4];
  int64_t n, k, units;
  const uint16_t *x;
  int64_t ldx;
  void *y;
  int64_t ldy;
  int64_t m;
  int y_f32;
  int mtiles, ntiles, per_xcd;
};

constexpr int kBM = 128;                 // activation rows per workgroup tile
// Weight rows per workgroup tile, BN: 128 (4 waves as 2 x 2 of 64 x 64) or 96 (4 waves along
// M, each 32 x 96). The launch takes the one whose busiest CU has the fewest weight rows.
constexpr int kLdsRow = kUnit + 8;       // halfs per LDS row: 64 + 8 of padding (bank spread)
constexpr uint32_t kXRange = 0x7FFFFFF0u; // activation buffer range; offsets at or past it read 0

template <int F, int BN>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  using U = Unit<F>;
  using Raw = typename U::Raw;
  static_assert(BN == 128 || BN == 96, "weight rows per tile");
  constexpr int WM = BN == 128 ? 2 : 4;                   // waves along M
  constexpr int TM = kBM / WM / 32, TN = BN / (4 / WM) / 32;   // 32 x 32 MFMA tiles per wave
  // two LDS buffers per operand: the MFMAs of step u read one while step u+1 is stored into
  // the other, so one barrier per step suffices
  __shared__ __attribute__((aligned(16))) _Float16 xs[2][kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) _Float16 ws[2][BN * kLdsRow];

  // Workgroups are dispatched round-robin over the 8 XCDs; tile numbers are assigned so that
  // consecutive tiles (the M tiles of one weight tile) fall on the same XCD.
  const int bid = blockIdx.x;
  const int tile = (bid & 7) * a.per_xcd + (bid >> 3);
  if (tile >= a.mtiles * a.ntiles) return;
  // (integer division runs on the vector unit; readfirstlane keeps the tile indices scalar,
  // so that the buffer resources built from them stay in scalar registers)
  const int mt = __builtin_amdgcn_readfirstlane(tile % a.mtiles);
  const int nt = __builtin_amdgcn_readfirstlane(tile / a.mtiles);
  const int64_t m0 = (int64_t)mt * kBM, r0 = (int64_t)nt * BN;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave % WM, wn = wave / WM;        // this wave's (TM x 32) x (TN x 32) block

  // weight loader role: LDS row t >> 1 of the weight tile, half h = t & 1 of the unit
  const int lrow = t >> 1, h = t & 1;
  const bool wload = BN == 128 || lrow < BN;       // wave-uniform: threads 2 * BN.. load no weights
  const int64_t wrow = r0 + lrow < a.n ? r0 + lrow : a.n - 1;   // rows past n are not stored
  // activation loader role: rows (t >> 3) + 32 i, 16-byte chunk t & 7 of the step's 128 bytes,
  // so that 8 consecutive lanes read one row's 128 bytes (whole cache lines)
  const int xr0 = t >> 3, xc = t & 7;
  // activations through a buffer resource based at this tile's first row: a dead row or the
  // missing half of a ragged q4g32 unit gets an offset past the range, which loads zeros (a
  // select on the loaded data instead would make every step wait for its own loads)
  const rsrc_t xr = make_rsrc(a.x + m0 * a.ldx, kXRange);

  Lane L;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    L.rs[p] = make_rsrc(a.w + a.poff[p], (uint32_t)(a.prb[p] * a.n));
    L.prb[p] = (uint32_t)a.prb[p];
  }
  L.h = h;

  // Global loads of step u into one register stage. Steps past the end re-load the last
  // step, so that every step issues the same loads and waits only for the older stage.
  auto gload = [&](Raw &q, u32x4 *xv, int64_t u) {
    u = u < a.units ? u : a.units - 1;
#pragma unroll
    for (int p = 0; p < 4; ++p) L.off[p] = 0;
    U::offsets(u, L.off);
    L.sh = fields_sh(u);
    L.set_halves(a.units);
    // the weight row differs per lane here, so it goes into the per-lane offset (a row in
    // the scalar offset would force one load per distinct row)
#pragma unroll
    for (int p = 0; p < 4; ++p) L.off[p] += (uint32_t)wrow * L.prb[p];
    const bool half = (F == 4) && (u == a.units - 1) && (a.k % 64 != 0);
    // only this thread's half of the unit; cached: the weight tile is read again by the
    // workgroups of the other M tiles
    if (wload) U::template load<0, 2>(q, L, 0, half);
    const int64_t kk = u * kUnit + 8 * xc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int xrow = xr0 + 32 * i;
      const bool ok = m0 + xrow < a.m && kk < a.k;
      xv[i] = bld4c(xr, ok ? (uint32_t)(xrow * a.ldx * 2 + kk * 2) : kXRange, 0);
    }
  };
  // decode a register stage to fp16 and store it, with its activations, into LDS buffer b
  auto lds_store = [&](const Raw &q, const u32x4 *xv, int b) {
    if (wload) {
      uint32_t pr[16];
      U::template wide<2>(q, h, pr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // local pairs 4i..4i+3 are the unit's consecutive pairs pidx(h, 4i).. (k = 2 * pair)
        const int g = U::pidx(h, 4 * i, 2);
        *reinterpret_cast<u32x4 *>(&ws[b][lrow * kLdsRow + 2 * g]) =
            u32x4{pr[4 * i], pr[4 * i + 1], pr[4 * i + 2], pr[4 * i + 3]};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4 *>(&xs[b][(xr0 + 32 * i) * kLdsRow + 8 * xc]) = xv[i];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int arow = lane & 31, akoff = 8 * (lane >> 5);
  auto mfma_step = [&](int b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t A[TM], B[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        A[i] = *reinterpret_cast<const half8_t *>(&xs[b][(wm * TM * 32 + 32 * i + arow) * kLdsRow + 16 * s + akoff]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        B[j] = *reinterpret_cast<const half8_t *>(&ws[b][(wn * TN * 32 + 32 * j + arow) * kLdsRow + 16 * s + akoff]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[j], acc[i][j], 0, 0, 0);
    }
  };

  // Pipeline: at step u, LDS buffer u & 1 holds step u, one register stage holds step u + 1
  // (loaded during step u - 1) and the other is free, so it receives the loads of step u + 2.
  Raw q0, q1;
  u32x4 x0[4], x1[4];
  gload(q0, x0, 0);
  gload(q1, x1, 1);
  lds_store(q0, x0, 0);
  __syncthreads();
  // No branches inside a step: past the last step the stage and LDS buffer written are never
  // read. Two steps per iteration keep the stages in fixed registers.
  auto body = [&](Raw &ql, u32x4 *xl, const Raw &qs, const u32x4 *xs_, int b, int64_t u) {
    gload(ql, xl, u + 2);
    mfma_step(b);
    lds_store(qs, xs_, b ^ 1);
    __syncthreads();
  };
  int64_t u = 0;
  for (; u + 2 <= a.units; u += 2) {
    body(q0, x0, q1, x1, 0, u);
    body(q1, x1, q0, x0, 1, u + 1);
  }
  if (u < a.units) body(q0, x0, q1, x1, 0, u);

  // D of a 32 x 32 MFMA: lane l holds column l % 32 and rows 8 (e / 4) + 4 (l / 32) + e % 4
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * TM * 32 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t col = r0 + wn * TN * 32 + 32 * j + (lane & 31);
        if (row < a.m && col < a.n) {
          const int64_t idx = row * a.ldy + col;
          if (a.y_f32) reinterpret_cast<float *>(a.y)[idx] = acc[i][j][e];
          else reinterpret_cast<_Float16 *>(a.y)[idx] = (_Float16)acc[i][j][e];
        }
      }
}

int launch_prefill(int fmt, const void *w, const uint16_t *X, int64_t ldx, void *Y, int64_t ldy, int y_f32,
                   int64_t m, int64_t n, int64_t k, hipStream_t s) {
  qg_layout lay;
  int st = qg_device_layout(fmt, n, k, &lay);
  if (st != QG_OK) return st;
  PrefillArgs a{};
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
  a.m = m;
  a.y_f32 = y_f32;
  if (kBM * ldx * 2 >= (int64_t)kXRange) return QG_ERR_SHAPE;     // 32-bit activation offsets
  // weight rows on the busiest CU: ceil(tiles / 256) tiles of BN rows (the workgroups go out one
  // per CU first); 96-row tiles when they leave it fewer rows (512 x 11008: 460 tiles, 192 rows
  // against 344 tiles and 256 rows)
  const int64_t mtiles = (m + kBM - 1) / kBM;
  const int64_t t128 = mtiles * ((n + 127) / 128), t96 = mtiles * ((n + 95) / 96);
  const int BN = (t96 + 255) / 256 * 96 < (t128 + 255) / 256 * 128 ? 96 : 128;
  const int64_t ntiles = (n + BN - 1) / BN;
  const int64_t total = mtiles * ntiles;
  if (total > (int64_t(1) << 30)) return QG_ERR_SHAPE;
  a.mtiles = (int)mtiles;
  a.ntiles = (int)ntiles;
  a.per_xcd = (int)((total + 7) / 8);
  const dim3 grid((unsigned)(8 * a.per_xcd)), block(256);
  auto go = [&](auto kern128, auto kern96) {
    return BN == 96 ? launch(kern96, grid, block, 0, s, a) : launch(kern128, grid, block, 0, s, a);
  };
  switch (fmt) {
    case 2: return go(prefill_kernel<2, 128>, prefill_kernel<2, 96>);
    case 3: return go(prefill_kernel<3, 128>, prefill_kernel<3, 96>);
    case 4: return go(prefill_kernel<4, 128>, prefill_kernel<4, 96>);
    case 5: return go(prefill_kernel<5, 128>, prefill_kernel<5, 96>);
    case 6: return go(prefill_kernel<6, 128>, prefill_kernel<6, 96>);
    case 7: return go(prefill_kernel<7, 128>, prefill_kernel<7, 96>);
    case 8: return go(prefill_kernel<8, 128>, prefill_kernel<8, 96>);
    case 9: return go(prefill_kernel<9, 128>, prefill_kernel<9, 96>);
    case 10: return go(prefill_kernel<10, 128>, prefill_kernel<10, 96>);
    case 11: return go(prefill_kernel<11, 128>, prefill_kernel<11, 96>);
    case 12: return go(prefill_kernel<12, 128>, prefill_kernel<12, 96>);
    case 13: return go(prefill_kernel<13, 128>, prefill_kernel<13, 96>);
    case 14: return go(prefill_kernel<3, 128>, prefill_kernel<3, 96>);   // q3sb's device layout
    case 15: return go(prefill_kernel<15, 128>, prefill_kernel<15, 96>);
    case 16: return go(prefill_kernel<16, 128>, prefill_kernel<16, 96>);
    case 17: return go(prefill_kernel<17, 128>, prefill_kernel<17, 96>);
    case 18: return go(prefill_kernel<18, 128>, prefill_kernel<18, 96>);
  }
  return QG_ERR_FORMAT;
}

}  // namespace qg
