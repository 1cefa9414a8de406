// The streaming dequant GEMV / small-M kernel (mv_kernel, mv_group_kernel), its launch
// planner and its launchers, shared by gemv.hip (the C ABI) and the per-format translation
// units mv_*.hip, which instantiate the launchers of a few formats each so that the device
// code compiles in parallel.
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
// (B + c) pairs with one v_and_or_b32 each and multiplied with v_dot2_f32_f16; the code
// offsets cancel against per-lane constants computed once from x. Each wave reduces its R
// row partials with DPP; K longer than 4096 weights is split across the waves of a
// workgroup and reduced through LDS.
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/qgemv.h"
#include "device_common.h"
#include "launch.h"
#include "layout.h"
#include "units.h"

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
  int64_t m;                // activation rows (1 for the GEMV)
  const int32_t *perm;      // act-order column permutation (k entries) or null
  int64_t xl_off;           // act-order: float offset of the activations staged in LDS, or -1
  int64_t ldx, ldy;         // elements between activation rows / output rows
  int y_f32;
  int wk;                   // waves per workgroup along K
  int wr;                   // row groups per workgroup
  int kpasses;              // passes over K (wk > 1 whenever kpasses > 1)
  int nb;                   // most row batches (each R rows) of any row group
  int64_t groups;           // row batches per matrix
  int64_t rgroups;          // row groups per matrix (gridDim.x * wr); they split the batches evenly:
  int64_t gq, gr;           // row group g starts at batch g * gq + min(g, gr) (gq = groups / rgroups,
                            // gr = groups % rgroups), so the first gr groups take one batch more
};

// ------------------------------------------------------------------ GEMV / small-M kernel -
//
// Template parameters: F format, M activation rows that share every decoded code (1 for the
// GEMV), S lanes per 64-weight unit (1, or 2 to halve the activation registers when M is
// large), R rows per pipelined batch, MP more than one pass over K, ONE a single batch of R
// (2 or 4) rows per row group with no pipeline: launches that fit one resident round of
// waves, where a second round trip to memory, not the stream rate, would set the time. DYN
// (K in one wave): the row batches of a workgroup are handed to its waves one at a time from
// an LDS counter instead of in fixed runs. Waves of one CU that run the same number of
// batches were measured to end up to 10 us apart in a 41 us launch (the CU's memory
// pipeline serves them unevenly), so that each CU ran its last quarter with few loads in
// flight; with a shared queue the waves of a workgroup end within about one batch.

// Register pipeline stages over row batches. Deeper pipelines spill or lose occupancy and
// measured no faster.
constexpr int kGemvDepth = 2;

// Largest workgroup of the streaming kernels: it bounds their registers (a workgroup must fit
// on the 4 SIMDs of one CU) and the waves along K of one pass. Eight activation rows need
// more than the 128 VGPRs a 1024-thread bound leaves.
template <int M> constexpr int mv_threads() { return M > 4 ? 512 : 1024; }

// One workgroup of the streaming kernel over matrix b of a (block bx along the rows). Waves
// past wk * wr (a grouped launch whose workgroup is sized for another matrix) have no rows
// but still reach the barrier.
// PERM (act-order): 0 none; 1 the activations staged in LDS in stored-column order, read as
// contiguous pieces; 2 each lane gathers its own, from a natural-order copy in LDS (when it
// fits) or from global memory.
template <int F, int M, int S, int R, bool MP, int PERM = 0, bool ONE = false, bool DYN = false>
__device__ __forceinline__ void mv_body(const GemvArgs &a, int64_t bx, int64_t b) {
  constexpr int D = ONE ? 1 : kGemvDepth;      // pipeline stages
  using U = Unit<F>;
  using Raw = typename U::Raw;
  static_assert(R == 1 || R == 2 || (ONE && R == 4), "rows per batch");
  static_assert(!ONE || (!MP && !PERM), "one-shot batches: a single pass, no permutation");
  static_assert(!DYN || (!MP && !PERM && !ONE && D == 2), "shared batch queue: one pass, K in one wave");
  constexpr int UPW = 64 / S;                  // units per wave
  constexpr int NP = 32 / S;                   // activation pairs per lane and row
  constexpr int NK = U::NKS(S);
  extern __shared__ float red[];               // [wr][R * nb][M][wk] partial sums when wk > 1
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int wk = wave % a.wk;
  const int wr = wave / a.wk;
  const int h = S == 1 ? 0 : (lane & 1);

  const uint8_t *w = a.w + b * a.w_bstride;
  const uint16_t *x = a.x + b * a.x_bstride;

  Lane L;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    L.rs[p] = make_rsrc(w + a.poff[p], (uint32_t)(a.prb[p] * a.n));
    L.prb[p] = (uint32_t)a.prb[p];
  }

  // This row group's rows: batches [begin, end) of R rows, an even split of the matrix's
  // batches over the grid's row groups (they differ by at most one batch); rows past n
  // re-read row n-1.
  const int64_t grp = bx * a.wr + wr;
  const bool idle = wr >= a.wr;
  auto gbegin = [&](int64_t g) -> int64_t { return g * a.gq + (g < a.gr ? g : a.gr); };
  const int64_t begin = idle ? 0 : gbegin(grp), end = idle ? 0 : gbegin(grp + 1);
  const int nbh = (int)(end - begin);          // batches of this row group (0 only for tiny n)
  const int rows_max = R * a.nb;               // LDS stride of a row group: a.nb >= every nbh
  auto row_of = [&](int j, int i) -> int64_t { return (begin + j) * R + i; };
  // DYN: the workgroup's batches [dyn_begin, dyn_begin + dyn_total), handed out by dyn_next
  __shared__ uint32_t dyn_next;
  int64_t dyn_begin = 0;
  int dyn_total = 0;
  if constexpr (DYN) {
    dyn_begin = gbegin(bx * a.wr);
    dyn_total = (int)(gbegin(bx * a.wr + a.wr) - dyn_begin);
    if (threadIdx.x == 0) dyn_next = 0;
    __syncthreads();
  }
  auto claim = [&]() -> int {                  // the next batch of the workgroup (wave-uniform)
    uint32_t v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(&dyn_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return (int)__builtin_amdgcn_readfirstlane(v);
  };
  // first row of batch c (a batch past the end re-reads the last one; its results are dropped)
  auto dyn_row = [&](int c) -> int64_t { return (dyn_begin + (c < dyn_total ? c : dyn_total - 1)) * R; };
  auto store_y = [&](int mm, int64_t r, float v) {
    const int64_t i = b * a.y_bstride + (int64_t)mm * a.ldy + r;
    if (a.y_f32) reinterpret_cast<float *>(a.y)[i] = v;
    else reinterpret_cast<_Float16 *>(a.y)[i] = (_Float16)v;
  };

  // K passes: the wk waves of a row group cover wk * UPW units per pass. With more than one
  // pass (long K with many activation rows) each wave accumulates its partial sums in LDS.
  // Act-order, PERM = 1: the workgroup copies its m rows of x into LDS (contiguous 16-byte
  // loads), then writes them again in stored-column order (column c holds x[perm[c]], an
  // index outside [0, k) gives 0): each thread reads 8 permutation entries with two 16-byte
  // loads, gathers the 8 values from the first copy and stores them as one 16-byte piece.
  // Each lane then reads its activations from the second copy as contiguous 16-byte pieces,
  // as without a permutation. PERM = 2 (one copy fits): only the natural-order copy, which
  // each lane gathers from through its own permutation entries.
  const uint16_t *xq = nullptr, *xl = nullptr;
  if (PERM && a.xl_off >= 0) {
    uint16_t *xn = reinterpret_cast<uint16_t *>(red + a.xl_off);   // [m][k], natural order
    const int64_t chunks = a.k / 8;                          // 16-byte chunks per row
    for (int64_t i = threadIdx.x; i < a.m * chunks; i += blockDim.x) {
      const int64_t mm = i / chunks, c = i % chunks;
      *reinterpret_cast<u32x4 *>(xn + mm * a.k + 8 * c) = ld4(reinterpret_cast<const uint8_t *>(x + mm * a.ldx + 8 * c));
    }
    __syncthreads();
    xl = xn;
    if constexpr (PERM == 1) {
      uint16_t *xs = xn + a.m * a.k;                         // [m][k], stored-column order
      const rsrc_t pr = make_rsrc(a.perm, (uint32_t)(a.k * 4));
      for (int64_t i = threadIdx.x; i < a.m * chunks; i += blockDim.x) {
        const int64_t mm = i / chunks, c = i % chunks;
        const u32x4 i0 = bld4c(pr, (uint32_t)(c * 32), 0), i1 = bld4c(pr, (uint32_t)(c * 32 + 16), 0);
        const uint32_t idx[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
        uint32_t hv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) hv[j] = idx[j] < (uint32_t)a.k ? xn[mm * a.k + idx[j]] : 0u;
        *reinterpret_cast<u32x4 *>(xs + mm * a.k + 8 * c) =
            u32x4{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16)};
      }
      __syncthreads();
      xq = xs;
    }
  }

  const int passes = MP ? a.kpasses : 1;
  for (int kp = 0; kp < passes; ++kp) {
    if (DYN ? dyn_total == 0 : nbh == 0) break;   // wave-uniform: no batch for this wave
    const int64_t u_raw = ((int64_t)kp * a.wk + wk) * UPW + (S == 1 ? lane : lane >> 1);
    const bool act = u_raw < a.units;
    const int64_t u = act ? u_raw : 0;         // inactive lanes read unit 0 and contribute 0
    const bool half = (F == 4) && act && (u == a.units - 1) && (a.k % 64 != 0);
#pragma unroll
    for (int p = 0; p < 4; ++p) L.off[p] = 0;
    U::offsets(u, L.off);
    L.sh = fields_sh(u);
    L.set_halves(a.units);
    L.h = h;

    auto load_batch = [&](Raw *q, int64_t r0) {
#pragma unroll
      for (int i = 0; i < R; ++i) U::template load<kNT, S>(q[i], L, r0 + i < a.n ? r0 + i : a.n - 1, half);
    };
    // D register stages: the loads of D - 1 batches are in flight while one is computed.
    // Prefetches past this row group's last batch re-load that batch (no extra HBM traffic).
    Raw qs[D][R];
    auto load_batch_j = [&](Raw *q, int jb) { load_batch(q, row_of(jb < nbh ? jb : nbh - 1, 0)); };

    // The lane's activation pairs, 16 bytes (4 pairs) at a time: local pairs 4i..4i+3 are the
    // unit's pairs pidx(h, 4i).. (consecutive), i.e. bytes 4 * pidx(h, 4i) of its 128.
    // With an act-order permutation, the activation of stored column c is x[perm[c]]: read
    // from the workgroup's copy in stored-column order, or gathered by the lane (an index
    // outside [0, k) reads 0, never past x).
    uint32_t xp[M][NP];
    auto load_x = [&]() {
    // (separate instantiations: the gather's registers at a branch made the register
    // allocator spill the kernels with 4 and 8 activation rows)
    if constexpr (PERM == 1) {
#pragma unroll
      for (int mm = 0; mm < M; ++mm) {
        const bool live = mm < a.m;
        const uint16_t *px = xq + (int64_t)(live ? mm : 0) * a.k + u * kUnit;
#pragma unroll
        for (int i = 0; i < NP / 4; ++i) {
          uint32_t off = 4u * (uint32_t)U::pidx(h, 4 * i, S);
          bool keepx = live;
          if (F == 4 && half && off >= 64) { off -= 64; keepx = false; }
          const u32x4 v = *reinterpret_cast<const u32x4 *>(px + off / 2);
          xp[mm][4 * i + 0] = keepx ? v.x : 0u;
          xp[mm][4 * i + 1] = keepx ? v.y : 0u;
          xp[mm][4 * i + 2] = keepx ? v.z : 0u;
          xp[mm][4 * i + 3] = keepx ? v.w : 0u;
        }
      }
    } else if constexpr (PERM == 2) {
      // the lane gathers its 8 activations per group of 4 pairs through 32-bit buffer loads
      // of the indices and reads of the LDS copy, or 16-bit buffer loads of x
      const rsrc_t pr = make_rsrc(a.perm, (uint32_t)(a.k * 4));
#pragma unroll
      for (int i = 0; i < NP / 4; ++i) {
        uint32_t off = 4u * (uint32_t)U::pidx(h, 4 * i, S);
        bool keepx = true;
        if (F == 4 && half && off >= 64) { off -= 64; keepx = false; }
        const uint32_t kb = (uint32_t)(u * kUnit) + off / 2;   // first of the 8 stored columns
        const u32x4 i0 = bld4c(pr, kb * 4, 0), i1 = bld4c(pr, kb * 4 + 16, 0);
        const uint32_t idx[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
        for (int mm = 0; mm < M; ++mm) {
          const bool live = mm < a.m && keepx;
          const int64_t row = mm < a.m ? mm : 0;
          uint32_t hv[8];
          if (xl) {
#pragma unroll
            for (int j = 0; j < 8; ++j) hv[j] = idx[j] < (uint32_t)a.k ? xl[row * a.k + idx[j]] : 0u;
          } else {
            const rsrc_t xr = make_rsrc(x + row * a.ldx, (uint32_t)(a.k * 2));
#pragma unroll
            for (int j = 0; j < 8; ++j) hv[j] = bldh(xr, idx[j] * 2, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) xp[mm][4 * i + r] = live ? (hv[2 * r] | (hv[2 * r + 1] << 16)) : 0u;
        }
      }
    } else {
#pragma unroll
      for (int mm = 0; mm < M; ++mm) {
        const bool live = mm < a.m;
        const uint8_t *px =
            reinterpret_cast<const uint8_t *>(x + (int64_t)(live ? mm : 0) * a.ldx) + (uint32_t)(u * 128);
#pragma unroll
        for (int i = 0; i < NP / 4; ++i) {
          uint32_t off = 4u * (uint32_t)U::pidx(h, 4 * i, S);
          bool keepx = live;
          // a half unit (k % 64 == 32) has only 32 activations: re-read the first half, zero it
          if (F == 4 && half && off >= 64) { off -= 64; keepx = false; }
          const u32x4 v = ld4(px + off);
          xp[mm][4 * i + 0] = keepx ? v.x : 0u;
          xp[mm][4 * i + 1] = keepx ? v.y : 0u;
          xp[mm][4 * i + 2] = keepx ? v.z : 0u;
          xp[mm][4 * i + 3] = keepx ? v.w : 0u;
        }
      }
    }
    };
    // Activations first: loads complete in order, so the wait for them before prep leaves the
    // first batch's weight loads in flight (with ONE, every row of the wave: each row is then
    // computed as its data arrives). The scheduling barrier keeps every one of these loads
    // ahead of the first wait; without it the scheduler moved most weight loads behind the
    // wait for the activations, so that a wave paid two round trips to memory before its
    // first row instead of one.
    int dyn_c0 = 0;
    if constexpr (DYN) dyn_c0 = claim();
    load_x();
    if constexpr (ONE) {
      load_batch(qs[0], row_of(0, 0));
    } else if constexpr (DYN) {
      load_batch(qs[0], dyn_row(dyn_c0));
    } else {
#pragma unroll
      for (int d = 0; d + 1 < D; ++d) load_batch_j(qs[d], d);
    }
    __builtin_amdgcn_sched_barrier(0);
    float kc[M][NK];
#pragma unroll
    for (int mm = 0; mm < M; ++mm) U::template prep<S>(xp[mm], kc[mm]);

    auto finish_batch = [&](const Raw *q, int64_t r0, int j) {
      // the batch's R x M partial sums, reduced over the wave together
      constexpr int T = R * M;
      float v[T];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float o[M];
#pragma unroll
        for (int mm = 0; mm < M; ++mm) o[mm] = 0.f;
        U::template dot<M, S>(q[i], h, xp, kc, o);
#pragma unroll
        for (int mm = 0; mm < M; ++mm) v[i * M + mm] = act ? o[mm] : 0.f;
      }
      wave_sums<T>(v);
      auto emit = [&](float val, int vi) {
        const int i = vi / M, mm = vi % M;
        if (mm >= a.m) return;
        if (a.wk == 1) {
          if (r0 + i < a.n) store_y(mm, r0 + i, val);
        } else {
          float &slot = red[((wr * rows_max + j * R + i) * M + mm) * a.wk + wk];
          slot = (MP && kp) ? slot + val : val;
        }
      };
      if constexpr (T == 1) {
        if (lane == 63) emit(v[0], 0);
      } else if constexpr (T == 2) {
        if ((lane & 31) == 31) emit(v[0], lane >> 5);
      } else {
        if ((lane & 15) == 15) {
          const int r = lane >> 4, pr = r == 1 ? 2 : (r == 2 ? 1 : r);
#pragma unroll
          for (int jj = 0; jj < T / 4; ++jj) emit(v[jj], 4 * jj + pr);
        }
      }
    };

    // Software pipeline, D batches per iteration so that every stage stays in fixed registers.
    // Loads are unconditional, so the wait before each compute covers only the oldest stage
    // (a conditional prefetch would force a wait for everything in flight).
    if constexpr (ONE) {
      finish_batch(qs[0], row_of(0, 0), 0);    // the row group's only batch (nbh == 1)
      continue;
    }
    if constexpr (DYN) {
      // two stages as below; each prefetch claims the next batch of the workgroup
      int c0 = dyn_c0;
      for (;;) {
        const int c1 = claim();
        load_batch(qs[1], dyn_row(c1));
        if (c0 >= dyn_total) break;
        finish_batch(qs[0], dyn_row(c0), 0);
        c0 = claim();
        load_batch(qs[0], dyn_row(c0));
        if (c1 >= dyn_total) break;
        finish_batch(qs[1], dyn_row(c1), 0);
      }
      continue;
    }
    for (int j = 0; j < nbh; j += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (j + d >= nbh) break;
        load_batch_j(qs[(d + D - 1) % D], j + d + D - 1);
        finish_batch(qs[d], row_of(j + d, 0), j + d);
      }
    }
  }
  if (a.wk == 1) return;
  // K split over wk waves: one barrier, then the first wave of the row group adds the
  // partial sums of all its (row, m) outputs and writes them (one output per lane)
  __syncthreads();
  if (wk == 0) {
    for (int i = lane; i < R * nbh * M; i += 64) {
      const int64_t r = row_of(i / M / R, i / M % R);
      const int mm = i % M;
      float sum = 0.f;
      for (int jj = 0; jj < a.wk; ++jj) sum += red[(wr * rows_max * M + i) * a.wk + jj];
      if (r < a.n && mm < a.m) store_y(mm, r, sum);
    }
  }
}

template <int F, int M, int S, int R, bool MP, int PERM, bool ONE = false, bool DYN = false>
__global__ __launch_bounds__(mv_threads<M>()) void mv_kernel(GemvArgs a) {
  mv_body<F, M, S, R, MP, PERM, ONE, DYN>(a, blockIdx.x, blockIdx.y);
}

// Several matrices (any shapes, one activation-row count) in one launch: blocks
// [block_end[g-1], block_end[g]) serve matrix g.
constexpr int kMaxGroup = 8;
struct GemvGroup {
  int count;
  int64_t block_end[kMaxGroup];
  GemvArgs g[kMaxGroup];
};

template <int F, int M, int S, int R, bool MP, bool ONE = false, bool DYN = false>
__global__ __launch_bounds__(mv_threads<M>()) void mv_group_kernel(GemvGroup G) {
  const int64_t bx = blockIdx.x;
  int gi = 0;
  while (gi + 1 < G.count && bx >= G.block_end[gi]) ++gi;
  mv_body<F, M, S, R, MP, false, ONE, DYN>(G.g[gi], bx - (gi ? G.block_end[gi - 1] : 0), 0);
}

// ------------------------------------------------------------------ launch planning ------


constexpr int64_t kMaxK = int64_t(1) << 20;   // at most 64 K passes in every configuration
constexpr int64_t kMaxPlaneBytes = (int64_t(1) << 32) - 1;   // buffer resources are 32-bit ranges

inline int fill_args(int fmt, const void *w, int64_t n, int64_t k, GemvArgs &a) {
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
    if (a.prb[p] * n > kMaxPlaneBytes) return QG_ERR_SHAPE;
  }
  return QG_OK;
}

constexpr int64_t kSimds = 1024;           // 256 CUs x 4 SIMDs
constexpr int kMaxBatches = 32;
constexpr int64_t kActOrderLds = 128 * 1024;  // most LDS an act-order launch stages activations in (two copies)
constexpr int kMinBatches = 4;
constexpr int kMaxM = 8;                   // activation rows one streaming launch serves
constexpr int kSkinnyMaxM = 16;            // activation rows of the matrix-core decode kernel
constexpr int kGemmStreamMaxM = 4;         // qg_gemm's streaming rows (grouped and act-order: kMaxM)

// Resident waves per SIMD that a kernel's register and LDS use allow (asked once per kernel).
inline int waves_per_simd(const void *kernel) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 64, 0) != hipSuccess || blocks < 4) return 1;
  return blocks / 4 > 8 ? 8 : blocks / 4;
}

// Row groups of one matrix: about nbt batches (of R rows) each, at most kMaxBatches (the
// partial sums of a row group fit in LDS), whole workgroups of wr row groups, batches split
// evenly. Returns the workgroups along the rows.
inline int64_t split_rows(GemvArgs &a, int R, int64_t nbt) {
  const int64_t groups = (a.n + R - 1) / R;
  int64_t rg = groups / nbt;
  const int64_t rg_cap = (groups + kMaxBatches - 1) / kMaxBatches;
  rg = rg < rg_cap ? rg_cap : rg;
  rg = rg < 1 ? 1 : (rg > groups ? groups : rg);
  const int64_t blocks = (rg + a.wr - 1) / a.wr;
  a.groups = groups;
  a.rgroups = blocks * a.wr;
  a.gq = groups / a.rgroups;
  a.gr = groups % a.rgroups;
  a.nb = (int)((groups + a.rgroups - 1) / a.rgroups);
  return blocks;
}

inline size_t red_bytes(const GemvArgs &a, int R, int M) {
  return a.wk > 1 ? (size_t)a.wr * R * a.nb * M * a.wk * sizeof(float) : 0;
}

// Launch shape of the streaming kernel over `ng` matrix shapes (count[g] matrices of n[g]
// rows and wk[g] waves along K each). Every workgroup has W waves; matrix g gets
// wr_g = W / wk_g row groups per workgroup, and waves past wr_g * wk_g idle until the
// workgroup's barrier. Whole workgroups fit a CU's wave slots floor(slots / W) times. Row
// groups take nbt batches each: one resident round of waves (no tail round), but at least
// kMinBatches, so that a wave's activation load and first load latency are spread over
// several rows (fewer, longer waves beat a full grid of very short ones here), and longer
// still for large single-row launches (kLongWaves below). W is chosen
// for the fewest wasted wave slots, times the fraction of the 256 CUs that get a workgroup
// at all (a small matrix in large workgroups would leave most CUs idle); the smaller W on
// ties, and no more than kMaxPlanW waves unless one matrix needs more along K (idle waves
// and coarse workgroups cost more than the score shows: workgroups of 10 to 16 waves
// measured up to 40% slower than 3 to 8 on the same grouped launch).
constexpr int kMaxPlanW = 8;
constexpr int64_t kLdsPerCu = 160 * 1024;   // LDS bytes per CU on gfx950
// Large single-row launches: every wave first loads its activation slice (8 KB for a whole
// wave of units), which a full grid of short waves re-reads from L2 thousands of times.
// When there is enough work, waves take more batches so that about kLongWaves of them
// (two per SIMD) cover it, up to a per-format cap: the 2- and 3-bit decodes spend about twice
// the VALU per weight byte and need the wave slots to hide it (cap 16 batches), the others
// stream best with the longest waves (32).
constexpr int64_t kLongWaves = 2048;
template <int F> constexpr bool light_bits() {   // q2sb, q3sb, their bf16-scale forms and q3g32
  return F == 2 || F == 3 || F == 12 || F == 13 || F == kQ3G32;
}
template <int F> constexpr int long_nbt() { return light_bits<F>() ? 16 : kMaxBatches; }
// Among equally scored workgroup sizes, the 2- and 3-bit single-row kernels take 4 waves when
// that still gives every CU at least 4 workgroups: measured 1.3% (q3sb) and 4% (q2sb) faster
// than 1 on 32 4096^2 GEMVs per launch; the other formats were as fast or up to 2% slower.
template <int F> constexpr int prefer_w() { return light_bits<F>() ? 4 : 0; }
struct MvPlan {
  int W;
  int64_t nbt;
};
inline MvPlan plan_mv(int ng, const int64_t *n, const int *wk, const int64_t *count, int R, int wps, int max_w,
               int64_t lds_block = 0, int long_cap = 0, int prefer_w = 0) {
  const int slots = 4 * wps;
  int64_t work[kMaxGroup], total = 0;
  int wk_max = 1;
  for (int g = 0; g < ng; ++g) {
    work[g] = (n[g] + R - 1) / R * wk[g] * count[g];           // row batches x waves along K
    total += work[g];
    wk_max = wk[g] > wk_max ? wk[g] : wk_max;
  }
  // workgroups of W waves when row groups take nbt batches (split_rows' split)
  auto blocks_for = [&](int W, int64_t nbt) {
    int64_t blocks = 0;
    for (int g = 0; g < ng; ++g) {
      const int64_t groups = (n[g] + R - 1) / R;
      int64_t rg = groups / nbt;
      const int64_t rg_cap = (groups + kMaxBatches - 1) / kMaxBatches;
      rg = rg < rg_cap ? rg_cap : rg;
      rg = rg < 1 ? 1 : (rg > groups ? groups : rg);
      blocks += count[g] * ((rg + W / wk[g] - 1) / (W / wk[g]));
    }
    return blocks;
  };
  MvPlan best{wk_max, kMinBatches}, best_plain{wk_max, kMinBatches};
  double best_score = -1.0, plain_score = -1.0;
  for (int W = wk_max; W <= max_w && W <= slots && (W <= kMaxPlanW || W == wk_max || lds_block > 0); ++W) {
    double used = 0.0;
    for (int g = 0; g < ng; ++g) used += (double)work[g] * (W / wk[g] * wk[g]) / W;
    int64_t per_cu = slots / W;
    if (lds_block > 0 && kLdsPerCu / lds_block < per_cu) per_cu = kLdsPerCu / lds_block;
    const int64_t resident = (int64_t)256 * per_cu * W;
    int64_t nbt = (total + resident - 1) / resident;
    nbt = nbt < kMinBatches ? kMinBatches : nbt;
    const int64_t blocks = blocks_for(W, nbt);
    const double score = used / (double)total * (double)(per_cu * W) / slots *
                         (blocks >= 256 ? 1.0 : (double)blocks / 256);
    if (score > best_score + 1e-9 || (W == prefer_w && score > best_score - 1e-9 && blocks >= 4 * 256)) {
      best_score = score;
      best = {W, nbt};
    }
    if (score > plain_score + 1e-9) {
      plain_score = score;
      best_plain = {W, nbt};
    }
  }
  // Long waves (single-row kernels): about kLongWaves waves, i.e. bpc workgroups of W waves
  // on every CU, each row group taking nbt_long batches, when that is longer than the plan's
  // and within the format's cap. Taken only if the workgroups still fit one even round
  // (blocks <= 256 * bpc): a grid a little larger than that leaves some CUs a second round.
  auto lengthen = [&](MvPlan p) {
    if (long_cap > 0) {
      const int64_t per_wave_slots = kLongWaves / 256;                  // waves per CU
      const int64_t bpc = p.W < per_wave_slots ? per_wave_slots / p.W : 1;
      const int64_t denom = (int64_t)256 * p.W * bpc;
      const int64_t nbt_long = (total + denom - 1) / denom;
      if (nbt_long > p.nbt && nbt_long <= long_cap && blocks_for(p.W, nbt_long) <= 256 * bpc) p.nbt = nbt_long;
    }
    return p;
  };
  best = lengthen(best);
  // the preferred workgroup size only where the final plan still gives every CU 4 workgroups
  if (best.W == prefer_w && blocks_for(best.W, best.nbt) < 4 * 256) best = lengthen(best_plain);
  return best;
}

// Shared batch queues (DYN): workgroups of dyn_waves<F>() waves (fewer if the kernel's
// registers leave fewer wave slots per CU), exactly one resident round of them, every row
// group taking an even share of the batches (its workgroup's waves then share them
// dynamically). Taken for single-row launches with K in one wave and at least kDynMinBatches
// batches. Measured on the benchmark's launch of 32 4096^2 GEMVs over 1.2 GB of rotating
// copies, against the fixed runs (three alternating runs, medians): q3sb 40.7 -> 39.1 us with
// workgroups of 16 waves (40.0 with 8), q4g32 54.4 -> 52.8 with 8 (53.7 with 16), q5sb
// 59.1 -> 59.6 (within noise). With fewer than about 8 batches per wave of one resident round
// the claims cost more than the balance gains (the 7B gate and up projections in one launch,
// 11008 batches: 11.8 -> 13.6 us).
template <int F> constexpr int dyn_waves() { return light_bits<F>() ? 16 : 8; }
constexpr int64_t kDynMinBatches = 4 * kSimds * 8;
inline MvPlan plan_dyn(const int64_t *n, int ng, int64_t count, int R, int wps, int max_w) {
  const int W = 4 * wps < max_w ? 4 * wps : max_w;
  const int64_t per_cu = (4 * wps) / W;
  int64_t batches = 0;
  for (int g = 0; g < ng; ++g) batches += (n[g] + R - 1) / R * count;
  const int64_t round = (int64_t)256 * per_cu * W;
  return {W, (batches + round - 1) / round};
}

template <int F, int M, int S, int R, bool MP, int PERM, bool ONE, bool DYN = false>
int launch_mv_k(GemvArgs a, int64_t count, hipStream_t s) {
  const GemvArgs a0 = a;
  void (*kern)(GemvArgs) = mv_kernel<F, M, S, R, MP, PERM, ONE, DYN>;
  static const int wps = waves_per_simd(reinterpret_cast<const void *>(kern));
  // act-order activations staged in LDS when they fit beside the partial sums: two copies
  // (natural and stored-column order) for PERM = 1, the natural-order one for PERM = 2
  const int64_t xl_bytes = PERM == 1 ? 2 * a.m * a.k * 2 : PERM == 2 ? a.m * a.k * 2 : 0;
  const bool stage = PERM && xl_bytes <= kActOrderLds;
  MvPlan P = plan_mv(1, &a.n, &a.wk, &count, R, wps, mv_threads<M>() / 64, stage ? xl_bytes : 0,
                     M == 1 && !ONE ? long_nbt<F>() : 0, M == 1 && !PERM && !ONE ? prefer_w<F>() : 0);
  if (ONE) P.nbt = 1;
  if (DYN) P = plan_dyn(&a.n, 1, count, R, wps, dyn_waves<F>());
  a.wr = P.W / a.wk;
  const int64_t blocks = split_rows(a, R, P.nbt);
  size_t shm = red_bytes(a, R, M);
  a.xl_off = -1;
  const bool fits = stage && (int64_t)((shm + 15) / 16 * 16) + xl_bytes <= kLdsPerCu;
  // PERM = 1 reads only the staged copy: without room for it, the per-lane gathers instead
  if constexpr (PERM == 1) {
    if (!fits) return launch_mv_k<F, M, S, R, MP, 2, ONE, DYN>(a0, count, s);
  }
  if (fits) {
    a.xl_off = (int64_t)((shm + 15) / 16 * 4);
    shm = (size_t)a.xl_off * 4 + (size_t)xl_bytes;
  }
  dim3 grid((unsigned)blocks, (unsigned)count);
  return launch(kern, grid, dim3((unsigned)(64 * P.W)), shm, s, a);
}

template <int F, int M, int S, int R, bool MP, bool ONE = false, bool DYN = false>
int launch_mv(GemvArgs a, int64_t count, hipStream_t s) {
  if constexpr (ONE) return launch_mv_k<F, M, S, R, MP, 0, true>(a, count, s);
  else if constexpr (DYN) return launch_mv_k<F, M, S, R, MP, 0, false, true>(a, count, s);
  else return a.perm ? launch_mv_k<F, M, S, R, MP, 1, false>(a, count, s)
                     : launch_mv_k<F, M, S, R, MP, 0, false>(a, count, s);
}

template <int F, int M, int S, int R, bool MP, bool ONE = false, bool DYN = false>
int launch_mv_group(GemvGroup &G, hipStream_t s) {
  void (*kern)(GemvGroup) = mv_group_kernel<F, M, S, R, MP, ONE, DYN>;
  static const int wps = waves_per_simd(reinterpret_cast<const void *>(kern));
  int64_t n[kMaxGroup], count[kMaxGroup];
  int wk[kMaxGroup];
  for (int g = 0; g < G.count; ++g) {
    n[g] = G.g[g].n;
    wk[g] = G.g[g].wk;
    count[g] = 1;
  }
  MvPlan P = plan_mv(G.count, n, wk, count, R, wps, mv_threads<M>() / 64, 0, M == 1 && !ONE ? long_nbt<F>() : 0);
  if (ONE) P.nbt = 1;
  if (DYN) P = plan_dyn(n, G.count, 1, R, wps, dyn_waves<F>());
  int64_t blocks = 0;
  size_t shm = 0;
  for (int g = 0; g < G.count; ++g) {
    G.g[g].xl_off = -1;
    G.g[g].wr = P.W / G.g[g].wk;
    blocks += split_rows(G.g[g], R, P.nbt);
    G.block_end[g] = blocks;
    const size_t r = red_bytes(G.g[g], R, M);
    shm = r > shm ? r : shm;
  }
  if (blocks > 0x7FFFFFFF) return QG_ERR_SHAPE;
  return launch(kern, dim3((unsigned)blocks), dim3((unsigned)(64 * P.W)), shm, s, G);
}

// Waves along K: one per 64 / S units, in passes of at most the workgroup's waves.
template <int M, int S>
int set_k_split(GemvArgs &a) {
  constexpr int UPW = 64 / S;
  constexpr int max_wk = mv_threads<M>() / 64;                // the kernel's block-size bound
  const int64_t waves_k = (a.units + UPW - 1) / UPW;
  const int64_t passes = (waves_k + max_wk - 1) / max_wk;
  if (passes > 64) return QG_ERR_SHAPE;
  a.kpasses = (int)passes;
  a.wk = (int)((waves_k + passes - 1) / passes);
  return QG_OK;
}

// One-shot launches (single-row kernels whose K fits one wave): when one wave per kOneRows
// rows needs at most kOneMaxWaves waves, every wave loads all its rows at once and the launch
// takes one memory round trip; larger launches stream through the pipelined kernel. Measured
// on q2sb / q3sb / q4g32 / q5sb / q6sb (graph-timed, HBM-resident copies): one 4096^2 matrix
// 5.3-6.3 -> 4.4-5.8 us, two per launch 7.2 -> 6.9 us; at four 4096^2 matrices, on 8192^2
// and on 4096 x 11008 (two or three waves along K) the pipelined kernel was 0.6-1.3 us faster.
constexpr int kOneRows = 4;
constexpr int64_t kOneMaxWaves = 2 * kSimds;
inline bool one_shot(int64_t rows, int wk) { return wk == 1 && (rows + kOneRows - 1) / kOneRows <= kOneMaxWaves; }

// Rows per batch: 2 (double-buffered, so four rows of loads per wave in flight without
// spilling) when there are enough rows to keep every SIMD busy, else 1: small problems are
// bound by latency and get as many waves as possible. With M > 2 the activation registers
// leave room for one row per batch only.
template <int F, int M, int S>
int launch_mv_s(GemvArgs a, int64_t count, hipStream_t s) {
  int st = set_k_split<M, S>(a);
  if (st != QG_OK) return st;
  if (a.kpasses > 1) return launch_mv<F, M, S, 1, true>(a, count, s);
  if constexpr (M == 1)
    if (!a.perm && one_shot(a.n * count, a.wk)) return launch_mv<F, M, S, kOneRows, false, true>(a, count, s);
  if constexpr (M <= 2)
    if (a.n * count * a.wk >= 2 * kSimds * 4) {
      if constexpr (M == 1)
        if (!a.perm && a.wk == 1 && (a.n + 1) / 2 * count >= kDynMinBatches)
          return launch_mv<F, M, S, 2, false, false, true>(a, count, s);
      return launch_mv<F, M, S, 2, false>(a, count, s);
    }
  return launch_mv<F, M, S, 1, false>(a, count, s);
}

template <int F, int M, int S>
int launch_mv_group_s(GemvGroup &G, hipStream_t s) {
  int64_t rows = 0, rows_1 = 0;
  bool mp = false;
  int wk_max = 1;
  for (int g = 0; g < G.count; ++g) {
    int st = set_k_split<M, S>(G.g[g]);
    if (st != QG_OK) return st;
    mp = mp || G.g[g].kpasses > 1;
    rows += G.g[g].n * G.g[g].wk;
    rows_1 += G.g[g].n;
    wk_max = G.g[g].wk > wk_max ? G.g[g].wk : wk_max;
  }
  if (mp) return launch_mv_group<F, M, S, 1, true>(G, s);
  if constexpr (M == 1)
    if (one_shot(rows_1, wk_max)) return launch_mv_group<F, M, S, kOneRows, false, true>(G, s);
  if constexpr (M <= 2)
    if (rows >= 2 * kSimds * 4) {
      if constexpr (M == 1)
        if (wk_max == 1 && (rows_1 + G.count) / 2 >= kDynMinBatches) return launch_mv_group<F, M, S, 2, false, false, true>(G, s);
      return launch_mv_group<F, M, S, 2, false>(G, s);
    }
  return launch_mv_group<F, M, S, 1, false>(G, s);
}

// M = 1: a lane owns a whole unit (32 activation VGPRs). M = 2..8: two lanes share a unit, so
// eight rows of activations take 128 VGPRs; rows beyond m are zero and not stored.
template <int F>
int launch_mv_f(GemvArgs a, int64_t count, hipStream_t s) {
  switch (a.m) {
    case 1: return launch_mv_s<F, 1, 1>(a, count, s);
    case 2: return launch_mv_s<F, 2, 2>(a, count, s);
    case 3:
    case 4: return launch_mv_s<F, 4, 2>(a, count, s);
    default: return launch_mv_s<F, 8, 2>(a, count, s);
  }
}

template <int F>
int launch_mv_group_f(GemvGroup &G, hipStream_t s) {
  switch (G.g[0].m) {
    case 1: return launch_mv_group_s<F, 1, 1>(G, s);
    case 2: return launch_mv_group_s<F, 2, 2>(G, s);
    case 3:
    case 4: return launch_mv_group_s<F, 4, 2>(G, s);
    default: return launch_mv_group_s<F, 8, 2>(G, s);
  }
}

// Instantiations: every format's launchers live in one of the mv_*.hip translation units.
#define QG_MV_INSTANTIATE(F)                                                \
  template int launch_mv_f<F>(GemvArgs, int64_t, hipStream_t);             \
  template int launch_mv_group_f<F>(GemvGroup &, hipStream_t);
#define QG_MV_DECLARE(F)                                                    \
  extern template int launch_mv_f<F>(GemvArgs, int64_t, hipStream_t);      \
  extern template int launch_mv_group_f<F>(GemvGroup &, hipStream_t);
#define QG_MV_FORMATS(X) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(15) X(16) X(17) X(18)

}  // namespace qg
