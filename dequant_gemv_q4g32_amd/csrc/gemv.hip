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
  int64_t rgroups;          // row groups per matrix (gridDim.x * wr); they split the batches evenly
};

// ------------------------------------------------------------------ GEMV / small-M kernel -
//
// Template parameters: F format, M activation rows that share every decoded code (1 for the
// GEMV), S lanes per 64-weight unit (1, or 2 to halve the activation registers when M is
// large), R rows per pipelined batch, MP more than one pass over K.

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
template <int F, int M, int S, int R, bool MP, bool PERM = false>
__device__ __forceinline__ void mv_body(const GemvArgs &a, int64_t bx, int64_t b) {
  constexpr int D = kGemvDepth;                // pipeline stages
  using U = Unit<F>;
  using Raw = typename U::Raw;
  static_assert(R == 1 || R == 2, "rows per batch");
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
  const int64_t begin = idle ? 0 : grp * a.groups / a.rgroups, end = idle ? 0 : (grp + 1) * a.groups / a.rgroups;
  const int nbh = (int)(end - begin);          // batches of this row group (0 only for tiny n)
  const int rows_max = R * a.nb;               // LDS stride of a row group: a.nb >= every nbh
  auto row_of = [&](int j, int i) -> int64_t { return (begin + j) * R + i; };
  auto store_y = [&](int mm, int64_t r, float v) {
    const int64_t i = b * a.y_bstride + (int64_t)mm * a.ldy + r;
    if (a.y_f32) reinterpret_cast<float *>(a.y)[i] = v;
    else reinterpret_cast<_Float16 *>(a.y)[i] = (_Float16)v;
  };

  // K passes: the wk waves of a row group cover wk * UPW units per pass. With more than one
  // pass (long K with many activation rows) each wave accumulates its partial sums in LDS.
  // Act-order with the activations staged in LDS: the workgroup copies its m rows of x
  // (contiguous 16-byte loads) once, so that each lane's gather by the permutation reads LDS
  // instead of issuing 2-byte global loads that touch a cache line each.
  const uint16_t *xl = a.xl_off >= 0 ? reinterpret_cast<const uint16_t *>(red + a.xl_off) : nullptr;
  if (PERM && xl) {
    uint16_t *xw = reinterpret_cast<uint16_t *>(red + a.xl_off);
    const int64_t chunks = a.k / 8;                          // 16-byte chunks per row
    for (int64_t i = threadIdx.x; i < a.m * chunks; i += blockDim.x) {
      const int64_t mm = i / chunks, c = i % chunks;
      *reinterpret_cast<u32x4 *>(xw + mm * a.k + 8 * c) = ld4(reinterpret_cast<const uint8_t *>(x + mm * a.ldx + 8 * c));
    }
    __syncthreads();
  }

  const int passes = MP ? a.kpasses : 1;
  for (int kp = 0; kp < passes; ++kp) {
    if (nbh == 0) break;                       // wave-uniform: a row group past the last batch
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
#pragma unroll
    for (int d = 0; d + 1 < D; ++d) load_batch_j(qs[d], d);   // weights first: their latency covers the x work

    // The lane's activation pairs, 16 bytes (4 pairs) at a time: local pairs 4i..4i+3 are the
    // unit's pairs pidx(h, 4i).. (consecutive), i.e. bytes 4 * pidx(h, 4i) of its 128.
    // With an act-order permutation, the activation of stored column c is x[perm[c]]: the
    // lane gathers its 8 activations per group of 4 pairs through 32-bit buffer loads of the
    // indices and 16-bit buffer loads of x (an index outside [0, k) reads 0, never past x).
    uint32_t xp[M][NP];
    // (a separate instantiation: the gather's registers at the branch made the register
    // allocator spill the kernels with 4 and 8 activation rows)
    if constexpr (PERM) {
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
    float kc[M][NK];
#pragma unroll
    for (int mm = 0; mm < M; ++mm) U::template prep<S>(xp[mm], kc[mm]);

    auto finish_batch = [&](const Raw *q, int j) {
      const int64_t r0 = row_of(j, 0);
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
    for (int j = 0; j < nbh; j += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (j + d >= nbh) break;
        load_batch_j(qs[(d + D - 1) % D], j + d + D - 1);
        finish_batch(qs[d], j + d);
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

template <int F, int M, int S, int R, bool MP, bool PERM>
__global__ __launch_bounds__(mv_threads<M>()) void mv_kernel(GemvArgs a) {
  mv_body<F, M, S, R, MP, PERM>(a, blockIdx.x, blockIdx.y);
}

// Several matrices (any shapes, one activation-row count) in one launch: blocks
// [block_end[g-1], block_end[g]) serve matrix g.
constexpr int kMaxGroup = 8;
struct GemvGroup {
  int count;
  int64_t block_end[kMaxGroup];
  GemvArgs g[kMaxGroup];
};

template <int F, int M, int S, int R, bool MP>
__global__ __launch_bounds__(mv_threads<M>()) void mv_group_kernel(GemvGroup G) {
  const int64_t bx = blockIdx.x;
  int gi = 0;
  while (gi + 1 < G.count && bx >= G.block_end[gi]) ++gi;
  mv_body<F, M, S, R, MP>(G.g[gi], bx - (gi ? G.block_end[gi - 1] : 0), 0);
}

__global__ void fill_zero_kernel(void *y, int64_t count, int f32, int64_t bstride, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  int64_t b = i / n, r = i % n;
  if (f32) reinterpret_cast<float *>(y)[b * bstride + r] = 0.f;
  else reinterpret_cast<_Float16 *>(y)[b * bstride + r] = (_Float16)0.f;
}

// ------------------------------------------------------------------ read ceiling ---------
// Streaming read of `bytes` bytes with a xor reduction: the achievable HBM read bandwidth
// that a GEMV kernel can be compared with (the DBHOO-CIM page, section 5.3, measures the
// machine's ceiling with STREAM before tuning kernels against it). The fastest pattern
// measured on gfx950: a grid-stride loop over a fixed grid, four non-temporal 128-bit loads
// in flight per thread (about 10% above one cached load per thread over a one-shot grid).
constexpr int kProbeBlocks = 4096;
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *p, int64_t n16, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  uint32_t s = 0;
  for (int64_t base = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; base < n16; base += stride) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = base + 256 * j;
      v[j] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) s ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
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

// Group-wise formats: w_hat = s * c + m (one rounding), group = the unit's half
__device__ void gw_values(const GemvArgs &a, const uint8_t *w, int64_t r, int64_t u, const uint8_t *c, uint8_t *codes,
                          float *vals) {
  const uint8_t *ps = w + a.poff[2] + r * a.prb[2] + u * 8;
  const uint8_t *pm = w + a.poff[3] + r * a.prb[3] + u * 8;
  for (int k = 0; k < 64; ++k) {
    const int g = k >> 5;
    codes[k] = c[k];
    vals[k] = __builtin_fmaf(__builtin_bit_cast(float, ld1(ps + 4 * g)), (float)c[k],
                             __builtin_bit_cast(float, ld1(pm + 4 * g)));
  }
}

template <int F>
__device__ void decode_unit(const GemvArgs &a, const uint8_t *w, int64_t r, int64_t u, uint8_t *codes, float *vals,
                            int nvalid) {
  uint8_t c[64];
  float step[4] = {0, 0, 0, 0}, off[4] = {0, 0, 0, 0};
  if constexpr (q4_group(F) != 0) {
    constexpr int G = q4_group(F);
    const uint8_t *pc = w + a.poff[0] + r * a.prb[0];
    const uint8_t *ps = w + a.poff[1] + r * a.prb[1];
    for (int i = 0; i < 8; ++i) {
      uint32_t v = (i < 4 || nvalid > 32) ? ld1(pc + split_off(a.units, u, i >> 2, 16) + 4 * (i & 3)) : 0u;
      for (int e = 0; e < 8; ++e) c[8 * i + e] = (v >> (4 * ((e >> 1) + 4 * (e & 1)))) & 15u;
    }
    for (int i = 0; i < nvalid; ++i) {
      const int64_t g = (u * kUnit + i) / G;
      codes[i] = c[i];
      vals[i] = (float)((int)c[i] - 8) * __builtin_bit_cast(float, ld1(ps + q4_scale_off(G, a.units, g)));
    }
    return;
  }
  if constexpr (F == kQ4G32H) {
    const uint8_t *pc = w + a.poff[0] + r * a.prb[0];
    const uint32_t sc = ld1(w + a.poff[1] + r * a.prb[1] + u * 4);
    for (int i = 0; i < 8; ++i) {
      uint32_t v = ld1(pc + split_off(a.units, u, i >> 2, 16) + 4 * (i & 3));
      for (int e = 0; e < 8; ++e) c[8 * i + e] = (v >> (4 * ((e >> 1) + 4 * (e & 1)))) & 15u;
    }
    for (int i = 0; i < nvalid; ++i) {
      codes[i] = c[i];
      vals[i] = (float)((int)c[i] - 8) * (i < 32 ? half_lo(sc) : half_hi(sc));
    }
    return;
  }
  if constexpr (F == kQ4A32) {
    const uint8_t *pc = w + a.poff[0] + r * a.prb[0];
    const uint8_t *ps = w + a.poff[1] + r * a.prb[1];
    const uint32_t zz = ldh(w + a.poff[2] + r * a.prb[2] + u * 2);
    for (int i = 0; i < 8; ++i) {
      uint32_t v = ld1(pc + split_off(a.units, u, i >> 2, 16) + 4 * (i & 3));
      for (int e = 0; e < 8; ++e) c[8 * i + e] = (v >> (4 * ((e >> 1) + 4 * (e & 1)))) & 15u;
    }
    for (int i = 0; i < nvalid; ++i) {
      const int gi = i >> 5;                       // group of the unit
      const int z = (int)((zz >> (8 * gi)) & 0xFFu);
      codes[i] = c[i];
      vals[i] = (float)((int)c[i] - z) * __builtin_bit_cast(float, ld1(ps + split_off(a.units, u, gi, 4)));
    }
    return;
  }
  constexpr int B = F == kQ3G32 ? 3 : F == kQ5G32 ? 5 : sb_base(F);   // code placement
  constexpr bool BF = sb_bf16(F);
  if (B == 2) {
    const uint8_t *pc = w + a.poff[0] + r * a.prb[0] + u * 16;
    uint32_t d[4];
    for (int i = 0; i < 4; ++i) d[i] = ld1(pc + 4 * i);
    for (int k = 0; k < 64; ++k) {
      int j = k >> 4, t = k >> 1, h = k & 1, rr = t & 7;
      c[k] = (d[rr >> 1] >> (16 * h + 8 * (rr & 1) + 2 * j)) & 3u;
    }
    uint32_t s = ld1(w + a.poff[1] + r * a.prb[1] + u * 4);
    uint32_t dd = ld1(w + a.poff[2] + r * a.prb[2] + (u >> 2) * 4);
    float dv = ss_lo<BF>(dd), dm = ss_hi<BF>(dd);
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
  if (B == 3) {
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
    if constexpr (F == kQ3G32) {
      gw_values(a, w, r, u, c, codes, vals);
      return;
    }
    uint32_t f = load_fields24(w + a.poff[2] + r * a.prb[2] + (u >> 2) * 12, (int)(u & 3));
    float dv = ss_one<BF>(ldh(w + a.poff[3] + r * a.prb[3] + (u >> 2) * 2));
    for (int k = 0; k < 64; ++k) {
      codes[k] = c[k];
      float st = dv * (float)((f >> (6 * (k >> 4))) & 63u);
      vals[k] = st * (float)((int)c[k] - 4);
    }
    return;
  }
  // q5sb / q6sb
  const uint8_t *pl = w + a.poff[0] + r * a.prb[0];
  uint32_t L[8], H[4];
  for (int i = 0; i < 8; ++i) L[i] = ld1(pl + split_off(a.units, u, i >> 2, 16) + 4 * (i & 3));
  const int hbytes = B == 5 ? 8 : 16;
  const uint8_t *ph = w + a.poff[1] + r * a.prb[1] + u * hbytes;
  for (int i = 0; i < hbytes / 4; ++i) H[i] = ld1(ph + 4 * i);
  const int base[4] = {4, 8, 12, 16};
  for (int k = 0; k < 64; ++k) {
    int i = k >> 3, e = k & 7, pk = e >> 1, h = e & 1;
    uint32_t lo = (L[i] >> (4 * ((e >> 1) + 4 * (e & 1)))) & 15u, hi;
    if (B == 5) hi = (H[i >> 2] >> ((base[pk] + 16 * h + (i & 3)) & 31)) & 1u;
    else hi = (H[i >> 1] >> ((base[pk] + 16 * h + 2 * (i & 1)) & 31)) & 3u;
    c[k] = (uint8_t)(lo | (hi << 4));
  }
  if constexpr (F == kQ5G32) {
    gw_values(a, w, r, u, c, codes, vals);
    return;
  }
  if (B == 5) {
    uint32_t f = load_fields24(w + a.poff[2] + r * a.prb[2] + (u >> 2) * 12, (int)(u & 3));
    uint32_t dd = ld1(w + a.poff[3] + r * a.prb[3] + (u >> 2) * 4);
    float dv = ss_lo<BF>(dd), dm = ss_hi<BF>(dd);
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
    float dv = ss_one<BF>(ldh(w + a.poff[3] + r * a.prb[3] + (u >> 2) * 2));
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

namespace {

constexpr int64_t kMaxK = int64_t(1) << 20;   // at most 64 K passes in every configuration
constexpr int64_t kMaxPlaneBytes = (int64_t(1) << 32) - 1;   // buffer resources are 32-bit ranges

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
    if (a.prb[p] * n > kMaxPlaneBytes) return QG_ERR_SHAPE;
  }
  return QG_OK;
}

constexpr int64_t kSimds = 1024;           // 256 CUs x 4 SIMDs
constexpr int kMaxBatches = 32;
constexpr int64_t kActOrderLds = 64 * 1024;   // most activation bytes an act-order launch stages in LDS
constexpr int kMinBatches = 4;
constexpr int kMaxM = 8;                   // activation rows one streaming launch serves
constexpr int kSkinnyMaxM = 16;            // activation rows of the matrix-core decode kernel
constexpr int kGemmStreamMaxM = 4;         // qg_gemm's streaming rows (grouped and act-order: kMaxM)

// Resident waves per SIMD that a kernel's register and LDS use allow (asked once per kernel).
int waves_per_simd(const void *kernel) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 64, 0) != hipSuccess || blocks < 4) return 1;
  return blocks / 4 > 8 ? 8 : blocks / 4;
}

// Row groups of one matrix: about nbt batches (of R rows) each, at most kMaxBatches (the
// partial sums of a row group fit in LDS), whole workgroups of wr row groups, batches split
// evenly. Returns the workgroups along the rows.
int64_t split_rows(GemvArgs &a, int R, int64_t nbt) {
  const int64_t groups = (a.n + R - 1) / R;
  int64_t rg = groups / nbt;
  const int64_t rg_cap = (groups + kMaxBatches - 1) / kMaxBatches;
  rg = rg < rg_cap ? rg_cap : rg;
  rg = rg < 1 ? 1 : (rg > groups ? groups : rg);
  const int64_t blocks = (rg + a.wr - 1) / a.wr;
  a.groups = groups;
  a.rgroups = blocks * a.wr;
  a.nb = (int)((groups + a.rgroups - 1) / a.rgroups);
  return blocks;
}

size_t red_bytes(const GemvArgs &a, int R, int M) {
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
MvPlan plan_mv(int ng, const int64_t *n, const int *wk, const int64_t *count, int R, int wps, int max_w,
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
  MvPlan best{wk_max, kMinBatches};
  double best_score = -1.0;
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
  }
  // Long waves (single-row kernels): about kLongWaves waves, i.e. bpc workgroups of W waves
  // on every CU, each row group taking nbt_long batches, when that is longer than the plan's
  // and within the format's cap. Taken only if the workgroups still fit one even round
  // (blocks <= 256 * bpc): a grid a little larger than that leaves some CUs a second round.
  if (long_cap > 0) {
    const int64_t per_wave_slots = kLongWaves / 256;                  // waves per CU
    const int64_t bpc = best.W < per_wave_slots ? per_wave_slots / best.W : 1;
    const int64_t denom = (int64_t)256 * best.W * bpc;
    const int64_t nbt_long = (total + denom - 1) / denom;
    if (nbt_long > best.nbt && nbt_long <= long_cap && blocks_for(best.W, nbt_long) <= 256 * bpc) best.nbt = nbt_long;
  }
  return best;
}

template <int F, int M, int S, int R, bool MP, bool PERM>
int launch_mv_k(GemvArgs a, int64_t count, hipStream_t s) {
  void (*kern)(GemvArgs) = mv_kernel<F, M, S, R, MP, PERM>;
  static const int wps = waves_per_simd(reinterpret_cast<const void *>(kern));
  // act-order activations staged in LDS when they fit beside the partial sums
  const int64_t xl_bytes = a.perm ? a.m * a.k * 2 : 0;
  const bool stage = a.perm && xl_bytes <= kActOrderLds;
  const MvPlan P = plan_mv(1, &a.n, &a.wk, &count, R, wps, mv_threads<M>() / 64, stage ? xl_bytes : 0,
                           M == 1 ? long_nbt<F>() : 0, M == 1 && !PERM ? prefer_w<F>() : 0);
  a.wr = P.W / a.wk;
  const int64_t blocks = split_rows(a, R, P.nbt);
  size_t shm = red_bytes(a, R, M);
  a.xl_off = -1;
  if (stage) {
    a.xl_off = (int64_t)((shm + 15) / 16 * 4);
    shm = (size_t)a.xl_off * 4 + (size_t)xl_bytes;
  }
  dim3 grid((unsigned)blocks, (unsigned)count);
  return launch(kern, grid, dim3((unsigned)(64 * P.W)), shm, s, a);
}

template <int F, int M, int S, int R, bool MP>
int launch_mv(GemvArgs a, int64_t count, hipStream_t s) {
  return a.perm ? launch_mv_k<F, M, S, R, MP, true>(a, count, s) : launch_mv_k<F, M, S, R, MP, false>(a, count, s);
}

template <int F, int M, int S, int R, bool MP>
int launch_mv_group(GemvGroup &G, hipStream_t s) {
  void (*kern)(GemvGroup) = mv_group_kernel<F, M, S, R, MP>;
  static const int wps = waves_per_simd(reinterpret_cast<const void *>(kern));
  int64_t n[kMaxGroup], count[kMaxGroup];
  int wk[kMaxGroup];
  for (int g = 0; g < G.count; ++g) {
    n[g] = G.g[g].n;
    wk[g] = G.g[g].wk;
    count[g] = 1;
  }
  const MvPlan P = plan_mv(G.count, n, wk, count, R, wps, mv_threads<M>() / 64, 0, M == 1 ? long_nbt<F>() : 0);
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

// Rows per batch: 2 (double-buffered, so four rows of loads per wave in flight without
// spilling) when there are enough rows to keep every SIMD busy, else 1: small problems are
// bound by latency and get as many waves as possible. With M > 2 the activation registers
// leave room for one row per batch only.
template <int F, int M, int S>
int launch_mv_s(GemvArgs a, int64_t count, hipStream_t s) {
  int st = set_k_split<M, S>(a);
  if (st != QG_OK) return st;
  if (a.kpasses > 1) return launch_mv<F, M, S, 1, true>(a, count, s);
  if constexpr (M <= 2)
    if (a.n * count * a.wk >= 2 * kSimds * 4) return launch_mv<F, M, S, 2, false>(a, count, s);
  return launch_mv<F, M, S, 1, false>(a, count, s);
}

template <int F, int M, int S>
int launch_mv_group_s(GemvGroup &G, hipStream_t s) {
  int64_t rows = 0;
  bool mp = false;
  for (int g = 0; g < G.count; ++g) {
    int st = set_k_split<M, S>(G.g[g]);
    if (st != QG_OK) return st;
    mp = mp || G.g[g].kpasses > 1;
    rows += G.g[g].n * G.g[g].wk;
  }
  if (mp) return launch_mv_group<F, M, S, 1, true>(G, s);
  if constexpr (M <= 2)
    if (rows >= 2 * kSimds * 4) return launch_mv_group<F, M, S, 2, false>(G, s);
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

int launch_mv_fmt(int fmt, GemvArgs a, int64_t count, hipStream_t s) {
  if (a.m < 1 || a.m > kMaxM) return QG_ERR_SHAPE;
  switch (fmt) {
    case 2: return launch_mv_f<2>(a, count, s);
    case 3: return launch_mv_f<3>(a, count, s);
    case 4: return launch_mv_f<4>(a, count, s);
    case 5: return launch_mv_f<5>(a, count, s);
    case 6: return launch_mv_f<6>(a, count, s);
    case 7: return launch_mv_f<7>(a, count, s);
    case 8: return launch_mv_f<8>(a, count, s);
    case 9: return launch_mv_f<9>(a, count, s);
    case 10: return launch_mv_f<10>(a, count, s);
    case 11: return launch_mv_f<11>(a, count, s);
    case 12: return launch_mv_f<12>(a, count, s);
    case 13: return launch_mv_f<13>(a, count, s);
    case 14: return launch_mv_f<3>(a, count, s);   // q3sb's device layout
    case 15: return launch_mv_f<15>(a, count, s);
    case 16: return launch_mv_f<16>(a, count, s);
    case 17: return launch_mv_f<17>(a, count, s);
    case 18: return launch_mv_f<18>(a, count, s);
  }
  return QG_ERR_FORMAT;
}

int launch_mv_group_fmt(int fmt, GemvGroup &G, hipStream_t s) {
  switch (fmt) {
    case 2: return launch_mv_group_f<2>(G, s);
    case 3: return launch_mv_group_f<3>(G, s);
    case 4: return launch_mv_group_f<4>(G, s);
    case 5: return launch_mv_group_f<5>(G, s);
    case 6: return launch_mv_group_f<6>(G, s);
    case 7: return launch_mv_group_f<7>(G, s);
    case 8: return launch_mv_group_f<8>(G, s);
    case 9: return launch_mv_group_f<9>(G, s);
    case 10: return launch_mv_group_f<10>(G, s);
    case 11: return launch_mv_group_f<11>(G, s);
    case 12: return launch_mv_group_f<12>(G, s);
    case 13: return launch_mv_group_f<13>(G, s);
    case 14: return launch_mv_group_f<3>(G, s);   // q3sb's device layout
    case 15: return launch_mv_group_f<15>(G, s);
    case 16: return launch_mv_group_f<16>(G, s);
    case 17: return launch_mv_group_f<17>(G, s);
    case 18: return launch_mv_group_f<18>(G, s);
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
  if (k % k_multiple(fmt)) return QG_ERR_SHAPE;
  if (k > kMaxK) return QG_ERR_SHAPE;
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
  a.m = 1;
  return launch_mv_fmt(fmt, a, count, s);
}

int qg_gemv(int fmt, const void *w, const uint16_t *x, void *y, int y_f32, int64_t n, int64_t k, void *stream) {
  return qg_gemv_batched(fmt, w, 0, x, 0, y, 0, y_f32, 1, n, k, stream);
}

int qg_gemm(int fmt, const void *w, const uint16_t *X, int64_t ldx, void *Y, int64_t ldy, int y_f32, int64_t m,
            int64_t n, int64_t k, void *stream) {
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (n < 0 || k < 0 || m < 0) return QG_ERR_SHAPE;
  if (k % k_multiple(fmt)) return QG_ERR_SHAPE;
  if (m > 1 && (ldx < k || ldy < n)) return QG_ERR_SHAPE;
  if (k > kMaxK) return QG_ERR_SHAPE;
  if (n == 0 || m == 0) return QG_OK;
  if (!Y || (k > 0 && (!w || !X))) return QG_ERR_NULL;
  if (!aligned(Y, y_f32 ? 4 : 2)) return QG_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t esz = y_f32 ? 4 : 2;
  if (k == 0) {
    for (int64_t i = 0; i < m; ++i) {
      int st = launch(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                      static_cast<void *>(static_cast<char *>(Y) + i * ldy * esz), n, y_f32, (int64_t)0, n);
      if (st != QG_OK) return st;
    }
    return QG_OK;
  }
  if (!aligned(w, 256) || !aligned(X, 16) || (m > 1 && ldx % 8)) return QG_ERR_ALIGN;
  GemvArgs a{};
  int st = fill_args(fmt, w, n, k, a);
  if (st != QG_OK) return st;
  // up to 4 activation rows: the streaming kernel (every decoded code pair meets each row in
  // a v_dot2); 5 to 16: fp16 w_hat on the matrix cores in one weight stream (from 5 rows
  // on, the v_dot2 per row and code pair cost more than the decode that the matrix cores
  // need once); more rows: LDS-staged fp16 tiles on the matrix cores
  if (m > kGemmStreamMaxM && m <= kSkinnyMaxM) return launch_skinny(fmt, w, X, ldx, Y, ldy, y_f32, m, n, k, s);
  if (m > kSkinnyMaxM) return launch_prefill(fmt, w, X, ldx, Y, ldy, y_f32, m, n, k, s);
  a.x = X;
  a.ldx = ldx;
  a.y = Y;
  a.ldy = ldy;
  a.y_f32 = y_f32;
  a.m = m;
  return launch_mv_fmt(fmt, a, 1, s);
}

int qg_gemm_act_order(int fmt, const void *w, const uint16_t *X, int64_t ldx, const int32_t *perm, void *Y,
                      int64_t ldy, int y_f32, int64_t m, int64_t n, int64_t k, void *stream) {
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (n < 0 || k < 0 || m < 0 || m > kMaxM) return QG_ERR_SHAPE;
  if (k % k_multiple(fmt)) return QG_ERR_SHAPE;
  if (m > 1 && (ldx < k || ldy < n)) return QG_ERR_SHAPE;
  if (k > kMaxK) return QG_ERR_SHAPE;
  if (n == 0 || m == 0) return QG_OK;
  if (!Y || (k > 0 && (!w || !X || !perm))) return QG_ERR_NULL;
  if (!aligned(Y, y_f32 ? 4 : 2)) return QG_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (k == 0) return qg_gemm(fmt, w, X, ldx, Y, ldy, y_f32, m, n, k, stream);
  if (!aligned(w, 256) || !aligned(X, 16) || !aligned(perm, 16) || (m > 1 && ldx % 8)) return QG_ERR_ALIGN;
  GemvArgs a{};
  int st = fill_args(fmt, w, n, k, a);
  if (st != QG_OK) return st;
  a.x = X;
  a.ldx = m > 1 ? ldx : k;
  a.y = Y;
  a.ldy = m > 1 ? ldy : n;
  a.y_f32 = y_f32;
  a.m = m;
  a.perm = perm;
  return launch_mv_fmt(fmt, a, 1, s);
}

int qg_gemm_grouped(int fmt, int count, const void *const *w, const uint16_t *const *X, const int64_t *ldx,
                    void *const *Y, const int64_t *ldy, const int64_t *n, const int64_t *k, int64_t m, int y_f32,
                    void *stream) {
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (count < 0 || count > kMaxGroup || m < 0 || m > kMaxM) return QG_ERR_SHAPE;
  if (count > 0 && (!w || !X || !Y || !n || !k || (m > 1 && (!ldx || !ldy)))) return QG_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t esz = y_f32 ? 4 : 2;
  GemvGroup G{};
  // every matrix is checked before anything is launched
  for (int g = 0; g < count; ++g) {
    const int64_t lx = m > 1 ? ldx[g] : k[g], ly = m > 1 ? ldy[g] : n[g];
    if (n[g] < 0 || k[g] < 0) return QG_ERR_SHAPE;
    if (k[g] % k_multiple(fmt)) return QG_ERR_SHAPE;
    if (m > 1 && (lx < k[g] || ly < n[g])) return QG_ERR_SHAPE;
    if (k[g] > kMaxK) return QG_ERR_SHAPE;
    if (n[g] == 0 || m == 0) continue;
    if (!Y[g] || (k[g] > 0 && (!w[g] || !X[g]))) return QG_ERR_NULL;
    if (!aligned(Y[g], esz)) return QG_ERR_ALIGN;
    if (k[g] == 0) continue;
    if (!aligned(w[g], 256) || !aligned(X[g], 16) || (m > 1 && lx % 8)) return QG_ERR_ALIGN;
    GemvArgs &a = G.g[G.count];
    int st = fill_args(fmt, w[g], n[g], k[g], a);
    if (st != QG_OK) return st;
    a.x = X[g];
    a.ldx = lx;
    a.y = Y[g];
    a.ldy = ly;
    a.y_f32 = y_f32;
    a.m = m;
    ++G.count;
  }
  for (int g = 0; g < count && m > 0; ++g) {
    if (n[g] == 0 || k[g] != 0) continue;
    for (int64_t i = 0; i < m; ++i) {
      const int64_t ly = m > 1 ? ldy[g] : n[g];
      int st = launch(fill_zero_kernel, dim3((unsigned)((n[g] + 255) / 256)), dim3(256), 0, s,
                      static_cast<void *>(static_cast<char *>(Y[g]) + i * ly * esz), n[g], y_f32, (int64_t)0, n[g]);
      if (st != QG_OK) return st;
    }
  }
  if (G.count == 0) return QG_OK;
  return launch_mv_group_fmt(fmt, G, s);
}

int dequant_gemv_q4g32(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(4, w, x, y, 0, n, k, s); }
int dequant_gemv_q2sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(2, w, x, y, 0, n, k, s); }
int dequant_gemv_q3sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(3, w, x, y, 0, n, k, s); }
int dequant_gemv_q5sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(5, w, x, y, 0, n, k, s); }
int dequant_gemv_q6sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(6, w, x, y, 0, n, k, s); }
int dequant_gemv_q4g16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(7, w, x, y, 0, n, k, s); }
int dequant_gemv_q4g64(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(8, w, x, y, 0, n, k, s); }
int dequant_gemv_q4g128(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(9, w, x, y, 0, n, k, s); }
int dequant_gemv_q4a32(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(10, w, x, y, 0, n, k, s); }
int dequant_gemv_q4g32h(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(11, w, x, y, 0, n, k, s); }
int dequant_gemv_q2sb_bf16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(12, w, x, y, 0, n, k, s); }
int dequant_gemv_q3sb_bf16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(13, w, x, y, 0, n, k, s); }
int dequant_gemv_q5sb_bf16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(15, w, x, y, 0, n, k, s); }
int dequant_gemv_q6sb_bf16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(16, w, x, y, 0, n, k, s); }
int dequant_gemv_q3g32(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(17, w, x, y, 0, n, k, s); }
int dequant_gemv_q5g32(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(18, w, x, y, 0, n, k, s); }
int dequant_gemv_q3sb_planes(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *s) { return qg_gemv(14, w, x, y, 0, n, k, s); }
int dequant_gemm_q4g32(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                       int64_t k, void *s) {
  return qg_gemm(4, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q2sb(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                      int64_t k, void *s) {
  return qg_gemm(2, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q3sb(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                      int64_t k, void *s) {
  return qg_gemm(3, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q5sb(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                      int64_t k, void *s) {
  return qg_gemm(5, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q6sb(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                      int64_t k, void *s) {
  return qg_gemm(6, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q4g16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                      int64_t k, void *s) {
  return qg_gemm(7, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q4g64(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                      int64_t k, void *s) {
  return qg_gemm(8, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q4g128(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                      int64_t k, void *s) {
  return qg_gemm(9, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q4a32(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                       int64_t k, void *s) {
  return qg_gemm(10, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q4g32h(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                        int64_t k, void *s) {
  return qg_gemm(11, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q2sb_bf16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                            int64_t k, void *s) {
  return qg_gemm(12, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q3sb_bf16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                            int64_t k, void *s) {
  return qg_gemm(13, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q5sb_bf16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                            int64_t k, void *s) {
  return qg_gemm(15, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q6sb_bf16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                            int64_t k, void *s) {
  return qg_gemm(16, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q3g32(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                        int64_t k, void *s) {
  return qg_gemm(17, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q5g32(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m, int64_t n,
                        int64_t k, void *s) {
  return qg_gemm(18, w, X, ldx, Y, ldy, 0, m, n, k, s);
}
int dequant_gemm_q3sb_planes(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy, int64_t m,
                              int64_t n, int64_t k, void *s) {
  return qg_gemm(14, w, X, ldx, Y, ldy, 0, m, n, k, s);
}

int qg_dequantize(int fmt, const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream) {
  if (!fmt_valid(fmt)) return QG_ERR_FORMAT;
  if (n < 0 || k < 0 || k % k_multiple(fmt)) return QG_ERR_SHAPE;
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
    case 7: return launch(dequant_kernel<7>, grid, block, 0, s, a, w_out, codes_out);
    case 8: return launch(dequant_kernel<8>, grid, block, 0, s, a, w_out, codes_out);
    case 9: return launch(dequant_kernel<9>, grid, block, 0, s, a, w_out, codes_out);
    case 10: return launch(dequant_kernel<10>, grid, block, 0, s, a, w_out, codes_out);
    case 11: return launch(dequant_kernel<11>, grid, block, 0, s, a, w_out, codes_out);
    case 12: return launch(dequant_kernel<12>, grid, block, 0, s, a, w_out, codes_out);
    case 13: return launch(dequant_kernel<13>, grid, block, 0, s, a, w_out, codes_out);
    case 14: return launch(dequant_kernel<3>, grid, block, 0, s, a, w_out, codes_out);   // q3sb's device layout
    case 15: return launch(dequant_kernel<15>, grid, block, 0, s, a, w_out, codes_out);
    case 16: return launch(dequant_kernel<16>, grid, block, 0, s, a, w_out, codes_out);
    case 17: return launch(dequant_kernel<17>, grid, block, 0, s, a, w_out, codes_out);
    case 18: return launch(dequant_kernel<18>, grid, block, 0, s, a, w_out, codes_out);
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
  const int64_t need = (n16 + 1023) / 1024;               // blocks of 256 threads x 4 loads
  const unsigned blocks = (unsigned)(need < kProbeBlocks ? need : kProbeBlocks);
  return launch(read_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                reinterpret_cast<const u32x4 *>(buf), n16, sink);
}

int dequantize_q4g32(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(4, w, o, c, n, k, s); }
int dequantize_q2sb(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(2, w, o, c, n, k, s); }
int dequantize_q3sb(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(3, w, o, c, n, k, s); }
int dequantize_q5sb(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(5, w, o, c, n, k, s); }
int dequantize_q6sb(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(6, w, o, c, n, k, s); }
int dequantize_q4g16(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(7, w, o, c, n, k, s); }
int dequantize_q4g64(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(8, w, o, c, n, k, s); }
int dequantize_q4g128(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(9, w, o, c, n, k, s); }
int dequantize_q4a32(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(10, w, o, c, n, k, s); }
int dequantize_q4g32h(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(11, w, o, c, n, k, s); }
int dequantize_q2sb_bf16(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(12, w, o, c, n, k, s); }
int dequantize_q3sb_bf16(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(13, w, o, c, n, k, s); }
int dequantize_q5sb_bf16(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(15, w, o, c, n, k, s); }
int dequantize_q6sb_bf16(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(16, w, o, c, n, k, s); }
int dequantize_q3g32(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(17, w, o, c, n, k, s); }
int dequantize_q5g32(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(18, w, o, c, n, k, s); }
int dequantize_q3sb_planes(const void *w, float *o, uint8_t *c, int64_t n, int64_t k, void *s) { return qg_dequantize(14, w, o, c, n, k, s); }

}  // extern "C"
