// Dequant GEMM for prefill-sized m, gfx950: Y = X * W_hat^T with W_hat tiles dequantized to
// fp16 in LDS and multiplied on the matrix cores (v_mfma_f32_32x32x16_f16, fp32 accumulate).
//
// Method: "二三五六位量化" page section 1.2 (prefill multiplies the same low-bit weights by
// many activation rows, so the work is a dense contraction; the dequantized weights are fp16)
// and DBHOO-CIM page section 5.2 (large prefill batches turn compute-bound). The codes are turned
// into fp16 w_hat by the same per-format unit decode as the GEMV (units.h, `wide`), written
// once per K step into an LDS tile that every wave of the workgroup reads.
//
// Tiling: a workgroup of NW waves computes a BM x BN tile of Y and walks K in steps of one
// 64-weight unit. Three shapes:
//   * 256 x 64 (4 waves, each a 64 x 64 block of 2 x 2 MFMA tiles): each weight is decoded
//     once per 256 activation rows, and the 32 KB of activations a step brings in feed 2 MFLOP;
//   * 256 x 96 (8 waves, each 32 x 96) where its rounds of workgroups fill the CUs better
//     (prefill_tile): its 132 KB of LDS leave one workgroup per CU, and 8 waves put two on
//     each SIMD;
//   * 128 x 32 (4 waves, each one 32 x 32 MFMA tile) where 256 x 64 tiles would leave CUs without
//     a workgroup (512 x 4096 has 128 of them, 128 x 11008 has 172): four times the tiles.
// Roles per step:
//   * activations: a later step's tile (BM rows x 128 bytes) goes straight into LDS with
//     buffer_load ... lds (no registers, no LDS store instructions). With 96 columns, and
//     with 64 for the formats of uni_rows64, every wave streams the rows it multiplies itself
//     (and waits for its own loads only); otherwise waves 2 and 3 stream the tile;
//   * weights: the first 2 BN threads (waves 0 and 1, waves 0-2, or wave 0) load a later
//     step's weights (thread t: half t & 1 of the unit of weight row t >> 1) and decode the
//     next step's to fp16 into the LDS weight tile. Wave 1 of the 32-column tiles, and waves
//     2-3 of the 64-column tiles of uni_rows64, load and decode a copy of row 0 and store
//     nothing, so that the waves of one role run branch-free code;
//   * all waves run the current step's MFMAs (4 K-slices of 16).
// P stages of both tiles in distinct LDS arrays (so that the compiler can see that the
// loads into one buffer do not alias the reads of another) and one barrier per step: the
// 256 x 64 tiles take two (two workgroups fit on a CU, each hiding the other's waits), the
// 256 x 96 and 128 x 32 tiles three, so that an activation DMA and a weight load each have
// two steps to arrive. Rows are stored with their 16-byte chunks XOR-swizzled (swz below), so
// that the rows an MFMA operand read touches fall on different banks.
// Workgroups are numbered so that each XCD works through the tiles of one M tile, whose
// activation rows then stay in its L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "../../include/qgemv.h"
#include "device_common.h"
#include "launch.h"
#include "layout.h"
#include "units.h"

namespace qg {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

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

constexpr int kMaxBM = 256;                   // activation rows per workgroup tile (256 or 128)
constexpr int kRowBytes = kUnit * 2;          // one K step of one row in fp16: 128 bytes
constexpr uint32_t kXRange = 0x7FFFFFF0u;    // activation buffer range; offsets at or past it read 0

// Byte offset of 16-byte chunk c of row r in a swizzled tile: the chunk goes to position
// c ^ f(r) of its row, f(r) = (r ^ (r >> 3)) & 7. A 128-bit LDS read serves 16 lanes per
// cycle (256 bytes, 64 banks): an MFMA operand read has those lanes on 16 consecutive rows
// at one chunk, and f is one-to-one on the even and on the odd rows of any 16 aligned rows
// (and on any 8 aligned rows), so those reads hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t swz(uint32_t r, uint32_t c) { return r * kRowBytes + 16u * (c ^ ((r ^ (r >> 3)) & 7u)); }

// Formats whose 64-column tiles let every wave stream its own activation rows, the two spare
// waves decoding a copy of weight row 0 (instead of waves 2-3 streaming all rows): measured
// on 1024-4096 x 11008 x 4096 (one session), q4g32 and q5sb 1-13% faster; q6sb 2-4% slower.
// (The 96-column tiles stream each wave's own rows for every format, with no spare decode.)
template <int F> constexpr bool uni_rows64() { return F == 4 || F == 5 || F == 15; }

// s_waitcnt: wait until at most N vector memory loads of this wave are in flight
template <int N> __device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int F, int BM, int BN>
__global__ __launch_bounds__(BN == 96 ? 512 : 256) void prefill_kernel(PrefillArgs a) {
  using U = Unit<F>;
  using Raw = typename U::Raw;
  static_assert((BM == 256 && (BN == 64 || BN == 96)) || (BM == 128 && BN == 32), "tile shape");
  constexpr int NW = BN == 96 ? 8 : 4;          // waves
  constexpr int TM = BM / (32 * NW);            // 32-row MFMA tiles per wave (rows BM / NW)
  constexpr int WN = BN / 32;                   // 32-column MFMA tiles per wave
  constexpr bool UNI = BN == 64 && uni_rows64<F>();   // every wave streams its rows, spare decode
  constexpr bool OWN = UNI || BN == 96;         // every wave streams the activation rows it uses
  constexpr int XW0 = UNI ? 0 : (BN == 96 ? 3 : 2);   // first x-wave (2 BN threads decode weights)
  constexpr int NX = OWN ? BM / (8 * NW) : BM / 8 / (4 - XW0);   // 1 KB activation DMA instructions per x-wave
  constexpr int P = BN == 64 ? 2 : 3;           // pipeline stages
  __shared__ __attribute__((aligned(16))) uint8_t X0[BM * kRowBytes], X1[BM * kRowBytes], X2[P > 2 ? BM * kRowBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t W0[BN * kRowBytes], W1[BN * kRowBytes], W2[P > 2 ? BN * kRowBytes : 16];

  // Workgroups are dispatched round-robin over the 8 XCDs; tile numbers are assigned so that
  // each XCD runs a contiguous range of tiles, M tile major: an XCD's L2 then holds the
  // activation rows of one M tile (2 MB at K = 4096 and BM = 256), which every step of every
  // tile reads BM x 128 bytes of, while a weight tile (BN rows of one unit) is read once per M
  // tile.
  const int bid = blockIdx.x;
  const int tile = (bid & 7) * a.per_xcd + (bid >> 3);
  if (tile >= a.mtiles * a.ntiles) return;
  // (integer division runs on the vector unit; readfirstlane keeps the tile indices scalar)
  const int mt = __builtin_amdgcn_readfirstlane(tile / a.ntiles);
  const int nt = __builtin_amdgcn_readfirstlane(tile % a.ntiles);
  const int64_t m0 = (int64_t)mt * BM, r0 = (int64_t)nt * BN;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool xwave = wave >= XW0;               // wave-uniform role

  // ---- weights (waves below XW0, or every wave in the uni_rows64 layout): thread t < 2 BN
  // decodes half t & 1 of weight row t >> 1. The loads and the decode run in every thread of
  // the weight waves (threads past 2 BN re-read the tile's first row); only the stores depend
  // on wload.
  // With no branch around them, the compiler counts the loads in flight exactly, and the
  // wait before a decode covers only the stage it reads.
  const bool wload = UNI ? t < 2 * BN : (64 * XW0 <= 2 * BN || t < 2 * BN);   // wave-uniform
  const int lrow = (t >> 1) < BN ? t >> 1 : 0, h = t & 1;
  const int64_t wrow = r0 + lrow < a.n ? r0 + lrow : a.n - 1;   // rows past n are not stored
  Lane L;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    L.rs[p] = make_rsrc(a.w + a.poff[p], (uint32_t)(a.prb[p] * a.n));
    L.prb[p] = (uint32_t)a.prb[p];
  }
  L.h = h;
  // global loads of step u (steps past the end re-load the last one, never read)
  auto gload = [&](Raw &q, int64_t u) {
    u = u < a.units ? u : a.units - 1;
#pragma unroll
    for (int p = 0; p < 4; ++p) L.off[p] = 0;
    U::offsets(u, L.off);
    L.sh = fields_sh(u);
    L.set_halves(a.units);
    // the weight row differs per lane, so it goes into the per-lane offset
#pragma unroll
    for (int p = 0; p < 4; ++p) L.off[p] += (uint32_t)wrow * L.prb[p];
    const bool half = (F == 4) && (u == a.units - 1) && (a.k % 64 != 0);
    // cached: the workgroups of the other M tiles read the same weight tile
    U::template load<0, 2>(q, L, 0, half);
  };
  // decode a register stage to fp16 and store it into the weight tile W
  auto wstore = [&](const Raw &q, uint8_t *W) {
    uint32_t pr[16];
    U::template wide<2>(q, h, pr);
    if (!wload) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // local pairs 4i..4i+3 are the unit's consecutive pairs pidx(h, 4i).. (k = 2 * pair), so
      // they fill 16-byte chunk pidx / 4 of the row
      const int c = U::pidx(h, 4 * i, 2) >> 2;
      *reinterpret_cast<u32x4 *>(W + swz(lrow, c)) = u32x4{pr[4 * i], pr[4 * i + 1], pr[4 * i + 2], pr[4 * i + 3]};
    }
  };

  // ---- activations (waves 2 and 3, or every wave, which then fills the rows it multiplies):
  // instruction i of x-wave xw fills tile rows 8 R .. 8 R + 7,
  // R = NX xw + i (1 KB, written in lane order); lane l loads row 8 R + (l >> 3), chunk
  // (l & 7) ^ f(row) of the step's 128 bytes, which lands at LDS position l & 7 of that row:
  // the swizzled layout (f(8 R + j) = (j ^ R) & 7). A dead row, or the missing half of a ragged
  // q4g32 unit, gets an offset past the range and reads zeros.
  const int xw = OWN ? wave : (wave - XW0 < 0 ? 0 : wave - XW0);
  const int xrow_l = lane >> 3;
  const rsrc_t xr = make_rsrc(a.x + m0 * a.ldx, kXRange);
  // 256-row tiles: each instruction's lane offset is fixed (row and chunk) and the step adds
  // u * 128 bytes as the scalar offset; xcs marks the lanes whose chunk is in the second half
  // of a unit, which a ragged q4g32 K (k % 64 == 32) leaves past k in the last unit. 128-row
  // tiles compute each offset per step instead. (Measured in one session: the fixed offsets
  // took 4-7% off the 256 x 64 launches and added 7-9% to the q3sb and q5sb 128 x 32 ones.)
  uint32_t xoff[NX];
  uint32_t xcs = 0;
  if constexpr (BM == 256) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int row = 8 * (NX * xw + i) + xrow_l;
      const int xc = (lane & 7) ^ ((xrow_l ^ (NX * xw + i)) & 7);
      xoff[i] = m0 + row < a.m ? (uint32_t)(row * a.ldx * 2 + 16 * xc) : kXRange;
      xcs |= (xc >= 4 ? 1u : 0u) << i;
    }
  }
  const bool ragged = (F == 4) && (a.k % 64 != 0);
  auto xdma = [&](int64_t u, uint8_t *X) {
    u = u < a.units ? u : a.units - 1;
    if constexpr (BM == 256) {
      const uint32_t so = (uint32_t)(u * kRowBytes);
      const bool cut = ragged && u == a.units - 1;
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const uint32_t voff = cut && ((xcs >> i) & 1u) ? kXRange : xoff[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t *)(X + (NX * xw + i) * 1024), 16, voff, so, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const int row = 8 * (NX * xw + i) + xrow_l;
        const int xc = (lane & 7) ^ ((xrow_l ^ (NX * xw + i)) & 7);
        const int64_t kk = u * kUnit + 8 * xc;
        const bool ok = m0 + row < a.m && kk < a.k;
        const uint32_t voff = ok ? (uint32_t)(row * a.ldx * 2 + kk * 2) : kXRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t *)(X + (NX * xw + i) * 1024), 16, voff, 0, 0, 0);
      }
    }
  };

  // ---- MFMAs of one step: wave w covers tile rows BM w / NW .., each of its TM 32-row blocks
  // against every 32-column block of the weight tile
  f32x16 acc[TM][WN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const uint32_t arow = (uint32_t)(BM / NW * wave + (lane & 31)), brow = (uint32_t)(lane & 31), kh = (uint32_t)(lane >> 5);
  auto mfma_step = [&](const uint8_t *X, const uint8_t *W) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t A[TM], B[WN];
#pragma unroll
      for (int i = 0; i < TM; ++i) A[i] = *reinterpret_cast<const half8_t *>(X + swz(arow + 32 * i, 2 * s + kh));
#pragma unroll
      for (int j = 0; j < WN; ++j) B[j] = *reinterpret_cast<const half8_t *>(W + swz(brow + 32 * j, 2 * s + kh));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[j], acc[i][j], 0, 0, 0);
    }
  };
  const int64_t units = a.units;
  if constexpr (P == 2 && UNI) {
    // two stages, every wave on its own activation rows (the DMA of step u + 1 may still be in
    // flight at the barrier: the compiler's wait before the wave's LDS reads covers it)
    auto wg_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    Raw q0, q1;
    xdma(0, X0);
    gload(q0, 0);
    gload(q1, 1);
    wstore(q0, W0);
    wg_barrier();
    int64_t u = 0;
    for (; u + 2 <= units; u += 2) {
      xdma(u + 1, X1);
      gload(q0, u + 2);
      mfma_step(X0, W0);
      wstore(q1, W1);
      wg_barrier();
      xdma(u + 2, X0);
      gload(q1, u + 3);
      mfma_step(X1, W1);
      wstore(q0, W0);
      wg_barrier();
    }
    if (u < units) {
      xdma(u + 1, X1);
      gload(q0, u + 2);
      mfma_step(X0, W0);
      wstore(q1, W1);
      wg_barrier();
    }
    vm_wait<0>();   // no DMA into the workgroup's LDS outlives it
  } else if constexpr (P == 2) {
    // x-waves: their LDS loads of this step are complete before they reach the barrier
    auto xwait = [&]() { __builtin_amdgcn_s_waitcnt(0); };

    // Two stages, two steps per iteration so that every buffer and register stage is fixed:
    // step u computes from X_{u&1}, W_{u&1}; the x-waves fill X_{(u+1)&1}, the weight waves store
    // the decoded step u + 1 into W_{(u+1)&1} and load step u + 2.
    if (xwave) {
      xdma(0, X0);
      xwait();
      __syncthreads();
      int64_t u = 0;
      for (; u + 2 <= units; u += 2) {
        xdma(u + 1, X1);
        mfma_step(X0, W0);
        xwait();
        __syncthreads();
        xdma(u + 2, X0);
        mfma_step(X1, W1);
        xwait();
        __syncthreads();
      }
      if (u < units) {
        xdma(u + 1, X1);
        mfma_step(X0, W0);
        xwait();
        __syncthreads();
      }
    } else {
      Raw q0, q1;
      gload(q0, 0);
      gload(q1, 1);
      wstore(q0, W0);
      __syncthreads();
      int64_t u = 0;
      for (; u + 2 <= units; u += 2) {
        gload(q0, u + 2);
        mfma_step(X0, W0);
        wstore(q1, W1);
        __syncthreads();
        gload(q1, u + 3);
        mfma_step(X1, W1);
        wstore(q0, W0);
        __syncthreads();
      }
      if (u < units) {
        gload(q0, u + 2);
        mfma_step(X0, W0);
        wstore(q1, W1);
        __syncthreads();
      }
    }
  } else {
    // Three stages, three steps per iteration: step u computes from X_{u%3}, W_{u%3}; at its
    // start the activation DMA of step u + 2 is issued and the weight waves issue the loads of
    // step u + 3 (into the register stage decoded at step u - 1); at its end the weight waves
    // decode step u + 1, loaded two steps earlier. 96 columns: every wave streams its own rows
    // and reads only those, so the compiler's wait before those LDS reads (for that wave's DMA
    // into that buffer) is all they need. 32 columns: the x-waves wait for the DMA of step
    // u + 1 only. The barrier is s_barrier after the wave's own LDS writes: __syncthreads would
    // add a fence that also waits for the DMA still in flight. (The memory clobber keeps every
    // LDS access on its side of the barrier.)
    auto wg_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    auto XB = [&](auto J) -> uint8_t * {
      if constexpr (decltype(J)::value == 0) return X0;
      else if constexpr (decltype(J)::value == 1) return X1;
      else return X2;
    };
    auto WB = [&](auto J) -> uint8_t * {
      if constexpr (decltype(J)::value == 0) return W0;
      else if constexpr (decltype(J)::value == 1) return W1;
      else return W2;
    };
    if constexpr (OWN) {
      if (xwave) {   // waves 3-7: their activation rows only
        xdma(0, X0);
        xdma(1, X1);
        wg_barrier();
        auto step = [&](auto J, int64_t u) {
          xdma(u + 2, XB(std::integral_constant<int, (decltype(J)::value + 2) % 3>{}));
          mfma_step(XB(J), WB(J));
          wg_barrier();
        };
        for (int64_t u = 0; u < units; u += 3) {
          step(I0{}, u);
          if (u + 1 < units) step(I1{}, u + 1);
          if (u + 2 < units) step(I2{}, u + 2);
        }
      } else {
        Raw q0, q1, q2;
        auto QB = [&](auto J) -> Raw & {
          if constexpr (decltype(J)::value == 0) return q0;
          else if constexpr (decltype(J)::value == 1) return q1;
          else return q2;
        };
        xdma(0, X0);
        xdma(1, X1);
        gload(q0, 0);
        gload(q1, 1);
        gload(q2, 2);
        wstore(q0, W0);
        wg_barrier();
        auto step = [&](auto J, int64_t u) {
          using JN = std::integral_constant<int, (decltype(J)::value + 1) % 3>;
          xdma(u + 2, XB(std::integral_constant<int, (decltype(J)::value + 2) % 3>{}));
          gload(QB(J), u + 3);
          mfma_step(XB(J), WB(J));
          wstore(QB(JN{}), WB(JN{}));
          wg_barrier();
        };
        for (int64_t u = 0; u < units; u += 3) {
          step(I0{}, u);
          if (u + 1 < units) step(I1{}, u + 1);
          if (u + 2 < units) step(I2{}, u + 2);
        }
      }
      vm_wait<0>();   // no DMA into the workgroup's LDS outlives it
    } else if (xwave) {
      xdma(0, X0);
      xdma(1, X1);
      vm_wait<NX>();
      wg_barrier();
      auto step = [&](auto J, int64_t u) {
        xdma(u + 2, XB(std::integral_constant<int, (decltype(J)::value + 2) % 3>{}));
        mfma_step(XB(J), WB(J));
        vm_wait<NX>();
        wg_barrier();
      };
      for (int64_t u = 0; u < units; u += 3) {
        step(I0{}, u);
        if (u + 1 < units) step(I1{}, u + 1);
        if (u + 2 < units) step(I2{}, u + 2);
      }
      vm_wait<0>();   // no DMA into the workgroup's LDS outlives it
    } else {
      Raw q0, q1, q2;
      auto QB = [&](auto J) -> Raw & {
        if constexpr (decltype(J)::value == 0) return q0;
        else if constexpr (decltype(J)::value == 1) return q1;
        else return q2;
      };
      gload(q0, 0);
      gload(q1, 1);
      gload(q2, 2);
      wstore(q0, W0);
      wg_barrier();
      auto step = [&](auto J, int64_t u) {
        using JN = std::integral_constant<int, (decltype(J)::value + 1) % 3>;
        gload(QB(J), u + 3);
        mfma_step(XB(J), WB(J));
        wstore(QB(JN{}), WB(JN{}));
        wg_barrier();
      };
      for (int64_t u = 0; u < units; u += 3) {
        step(I0{}, u);
        if (u + 1 < units) step(I1{}, u + 1);
        if (u + 2 < units) step(I2{}, u + 2);
      }
    }
  }

  // D of a 32 x 32 MFMA: lane l holds column l % 32 and rows 8 (e / 4) + 4 (l / 32) + e % 4
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + BM / NW * wave + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t col = r0 + 32 * j + (lane & 31);
        if (row < a.m && col < a.n) {
          const int64_t idx = row * a.ldy + col;
          if (a.y_f32) reinterpret_cast<float *>(a.y)[idx] = acc[i][j][e];
          else reinterpret_cast<_Float16 *>(a.y)[idx] = (_Float16)acc[i][j][e];
        }
      }
}

// Tile shape for m x n: 256 rows when 256 x 64 tiles give every CU a workgroup, else 128 x 32,
// four times the tiles (each K step of a tile is then short, and more of them run at once).
// Between 64 and 96 columns, the one whose rounds of workgroups fill more of the CUs: two
// 256 x 64 workgroups run on a CU at once, one 256 x 96 (8 waves, two per SIMD); at equal
// fill the 96-column tiles are 2-5% faster, hence the margin. Measured on one MI355X (q3sb,
// q4g32, q5sb, q6sb; 96 against 64 columns): 1024 x 11008 x 4096 460 tiles against 688,
// 8-20% faster; 2048 x 28672 x 8192 2392 against 3584, 5%; 2048 x 4096 x 4096 344 against
// 512, 16-22% slower.
void prefill_tile(int64_t m, int64_t n, int *bm, int *bn) {
  const int64_t mt = (m + 255) / 256, t64 = mt * ((n + 63) / 64), t96 = mt * ((n + 95) / 96);
  const bool big = t64 >= 256;
  const int64_t r64 = (t64 + 511) / 512, r96 = (t96 + 255) / 256;   // rounds on 256 CUs
  const double fill64 = (double)t64 / (double)(512 * r64), fill96 = (double)t96 / (double)(256 * r96);
  *bm = big ? 256 : 128;
  *bn = !big ? 32 : (fill96 + 0.07 >= fill64 ? 96 : 64);
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
  if (kMaxBM * ldx * 2 >= (int64_t)kXRange) return QG_ERR_SHAPE;     // 32-bit activation offsets
  int BM, BN;
  prefill_tile(m, n, &BM, &BN);
  const int64_t mtiles = (m + BM - 1) / BM;
  const int64_t ntiles = (n + BN - 1) / BN;
  const int64_t total = mtiles * ntiles;
  if (total > (int64_t(1) << 30)) return QG_ERR_SHAPE;
  a.mtiles = (int)mtiles;
  a.ntiles = (int)ntiles;
  a.per_xcd = (int)((total + 7) / 8);
  const dim3 grid((unsigned)(8 * a.per_xcd)), block(BN == 96 ? 512 : 256);
  auto go = [&](auto big, auto small, auto wide) {
    if (BM == 128) return launch(small, grid, block, 0, s, a);
    return BN == 96 ? launch(wide, grid, block, 0, s, a) : launch(big, grid, block, 0, s, a);
  };
#define QG_PF(F) go(prefill_kernel<F, 256, 64>, prefill_kernel<F, 128, 32>, prefill_kernel<F, 256, 96>)
  switch (fmt) {
    case 2: return QG_PF(2);
    case 3: return QG_PF(3);
    case 4: return QG_PF(4);
    case 5: return QG_PF(5);
    case 6: return QG_PF(6);
    case 7: return QG_PF(7);
    case 8: return QG_PF(8);
    case 9: return QG_PF(9);
    case 10: return QG_PF(10);
    case 11: return QG_PF(11);
    case 12: return QG_PF(12);
    case 13: return QG_PF(13);
    case 14: return QG_PF(3);   // q3sb's device layout
    case 15: return QG_PF(15);
    case 16: return QG_PF(16);
    case 17: return QG_PF(17);
    case 18: return QG_PF(18);
  }
#undef QG_PF
  return QG_ERR_FORMAT;
}

}  // namespace qg
