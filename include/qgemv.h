/*
 * qgemv.h - C ABI of libqgemv: weight-only low-bit dequantize-and-multiply on MI355X (gfx950).
 *
 * Formats (one byte table per 256 weights, "二三五六位量化" page section 2.3; INT4 from the
 * DBHOO-CIM page sections 2.1, 3.1, 3.2 and 4.1):
 *
 *   QG_Q4G32  INT4 symmetric, groups of 32 consecutive weights of a row, fp32 scale per group:
 *             scale = max(max|w| / 8, 1e-12), q = clamp(rint(w / scale), -8, 7) in fp32,
 *             w_hat = q * scale; 16 B of codes + 4 B of scale per group (5.0 bpw).
 *   QG_Q4G16, QG_Q4G64, QG_Q4G128  the same INT4 code with groups of 16, 64 or 128 weights
 *             (6.0, 4.5, 4.25 bpw; DBHOO-CIM page section 5.1 advises groups of 16 against
 *             outlier weights). k must be a multiple of 64 (of 128 for QG_Q4G128).
 *   QG_Q4A32  INT4 asymmetric, groups of 32, fp32 scale s and uint8 zero point z per group
 *             ("二三五六位量化" page section 2.1's x = s (q - z); DBHOO-CIM page section 5.1
 *             keeps asymmetric quantization for layers the symmetric grid serves badly):
 *             lo = min(0, min w), hi = max(0, max w), s = max((hi - lo) / 15, 1e-12),
 *             z = clamp(rint(-lo / s), 0, 15), c = clamp(rint(w / s) + z, 0, 15) in fp32,
 *             w_hat = s * (c - z); 16 B of codes + 4 B of scale + 1 B of zero point per group
 *             (5.25 bpw). k must be a multiple of 64.
 *   QG_Q4G32H INT4 symmetric, groups of 32, fp16 scale ("二三五六位量化" page section 2.1: a
 *             16-bit scale per group of 32): s = fp16_rn(max|w| / 8 in fp32) (0 raised to
 *             2^-24; past 65504 QG_ERR_RANGE), q = clamp(rint(w / s), -8, 7) in fp32 against
 *             that stored s, w_hat = q * s; 16 B of codes + 2 B of scale per group (4.5 bpw).
 *             k must be a multiple of 64.
 *   QG_Q2SB   256-weight super-block, 16 sub-blocks of 16, 2-bit codes c, 4-bit sub-scale sc
 *             and 4-bit sub-min m, fp16 d and dmin: w_hat = d*sc*c - dmin*m  (84 B, 2.625 bpw).
 *   QG_Q3SB   16 sub-blocks of 16, 3-bit codes, 6-bit sc, fp16 d: w_hat = d*sc*(c - 4)
 *             (110 B, 3.4375 bpw).
 *   QG_Q5SB   8 sub-blocks of 32, 5-bit codes (low-4-bit plane + high-bit plane), 6-bit sc and
 *             m, fp16 d and dmin: w_hat = d*sc*c - dmin*m  (176 B, 5.5 bpw).
 *   QG_Q6SB   16 sub-blocks of 16, 6-bit codes (low-4-bit plane + high-2-bit plane), int8 sc,
 *             fp16 d: w_hat = d*sc*(c - 32)  (210 B, 6.5625 bpw).
 *   QG_Q2SB_BF16, QG_Q3SB_BF16, QG_Q5SB_BF16, QG_Q6SB_BF16  the same four formats with the
 *             super-scales d (and dmin) stored as bf16 instead of fp16 ("二三五六位量化" page
 *             section 2.3: against fp16 overflow of the super-scale); same records and sizes,
 *             bf16_ceil in place of fp16_ceil in the rule below. The GEMM paths for m > 4
 *             multiply fp16 W_hat on the matrix cores: weights beyond the fp16 range (which
 *             only bf16 super-scales can express) need the streaming kernel (qg_gemm with
 *             m <= 4, qg_gemm_grouped or qg_gemm_act_order with m <= 8).
 *   QG_Q3SB_PLANES  q3sb with the record's 96 code bytes stored as a 64-byte plane of the low
 *             2 bits (2-bit stream) and a 32-byte plane of the high bit (1-bit stream)
 *             ("二三五六位量化" page section 2.3: split widths that do not divide a byte into
 *             planes); same fields, rule and device layout as QG_Q3SB (110 B, 3.4375 bpw).
 *   QG_Q3G32, QG_Q5G32  plain group-wise 3- and 5-bit codes c with an fp32 scale s and an fp32
 *             min m per group of 32 (the form of "二三五六位量化" page section 3.3's gemv_q3:
 *             w_hat = s*c + m): m = min w (+0 for a zero minimum), s = max((max w - min w) / (2^b - 1), 1e-12),
 *             c = clamp(rint((w - m) / s), 0, 2^b - 1), difference and quotient in fp32.
 *             12 or 20 B of codes + 8 B per group (5.0 and 7.0 bpw). k a multiple of 64.
 *
 * Super-block scales are chosen by "range-covering round to nearest" (the pages give the
 * layouts, not the rule): with fp16_ceil(v) = smallest fp16 >= v, symmetric formats take
 * t_j = max|w_j| / (o - 0.5), d = fp16_ceil(max_j t_j / Smax), sc_j = min(Smax, ceil(t_j / d));
 * asymmetric formats take dmin = fp16_ceil(max_j(-min(0, min w_j)) / Smax),
 * m_j = min(Smax, ceil(-min(0, min w_j) / dmin)), t_j = (max(0, max w_j) + dmin*m_j) / (2^b - 1)
 * and d, sc_j as above; codes are rint (half to even) of w / (d*sc_j) (+ o), or of
 * (w + dmin*m_j) / (d*sc_j), clamped. All in fp64. Every weight is then within d*sc_j / 2.
 * Smax = 15 (q2sb), 63 (q3sb, q5sb), 127 (q6sb).
 *
 * Two encodings of a quantized matrix W [n][k] (W is out_features x in_features):
 *   canonical  the pages' interchange layout. q4g32: codes [n][k/2] (byte = u[2j] | u[2j+1] << 4
 *              with u = q + 8) followed by fp32 scales [n][k/32] (q4gG: [n][k/G]). q4a32: codes
 *              [n][k/2] (u = c), fp32 scales [n][k/32], uint8 zero points [n][k/32]. q4g32h: codes
 *              as q4g32, then fp16 scales [n][k/32]. q3g32 / q5g32: each row's codes as one
 *              little-endian b-bit stream [n][k*b/8], then fp32 scales [n][k/32], then fp32
 *              mins [n][k/32]. Super-block formats: records
 *              [n][k/256] of 84/110/176/210 bytes; fields in the byte table's column order
 *              (codes [, high-bit plane], sub-scales, d [, dmin]; q3sb_planes: low-2-bit plane,
 *              high-bit plane, sub-scales, d); every bit field is a
 *              little-endian bitstream (code i at bits [b*i, b*i + b), section 2.2's unpack3
 *              and unpack5); q2sb sub-block byte = sc | m << 4; q5sb's 12 bytes hold sixteen
 *              6-bit fields sc0..sc7, m0..m7; fp16 values little-endian.
 *   device     a planar, bit-permuted rearrangement of exactly the same bits, built for
 *              128-bit coalesced lane loads and single-instruction field extraction on CDNA4.
 *              Each plane is [n][row_bytes] row-major and starts 256-byte aligned. The planes
 *              hold the same number of bytes as the canonical encoding (plus < 1 KiB of
 *              inter-plane padding, never read). It is opaque: build it with
 *              qg_to_device_layout and read it back with qg_from_device_layout.
 *
 * Conventions: all sizes are int64_t. fp16 values are passed as uint16_t bit patterns.
 * `stream` is a hipStream_t (NULL = the default stream). Every function returns a qg_status.
 *
 * Ownership: the caller allocates and owns every buffer, host and device. The library never
 * allocates, frees or synchronizes, and keeps no pointer past the call. Host functions are
 * pure and thread-safe. Device functions validate their arguments on the host, return an
 * error without launching anything if they are invalid, and otherwise enqueue kernels on
 * `stream` and return; execution faults surface at the caller's next synchronization.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QG_ABI_VERSION 1

typedef enum qg_format {
  QG_Q2SB = 2,
  QG_Q3SB = 3,
  QG_Q4G32 = 4,
  QG_Q5SB = 5,
  QG_Q6SB = 6,
  QG_Q4G16 = 7,
  QG_Q4G64 = 8,
  QG_Q4G128 = 9,
  QG_Q4A32 = 10,
  QG_Q4G32H = 11,
  QG_Q2SB_BF16 = 12,
  QG_Q3SB_BF16 = 13,
  QG_Q3SB_PLANES = 14,
  QG_Q5SB_BF16 = 15,
  QG_Q6SB_BF16 = 16,
  QG_Q3G32 = 17,
  QG_Q5G32 = 18
} qg_format;

typedef enum qg_status {
  QG_OK = 0,
  QG_ERR_NULL = -1,      /* a required pointer is NULL                                      */
  QG_ERR_SHAPE = -2,     /* n, k or m out of range (k % 256 super-blocks, % 32 q4g32, ...)   */
  QG_ERR_ALIGN = -3,     /* a device pointer or leading dimension is misaligned              */
  QG_ERR_NONFINITE = -4, /* a weight is NaN or infinite                                     */
  QG_ERR_RANGE = -5,     /* d or dmin does not fit fp16 (section 2.3's overflow warning)     */
  QG_ERR_FORMAT = -6,    /* unknown format or bit width                                     */
  QG_ERR_LAUNCH = -7,    /* the HIP runtime refused a launch                                 */
  QG_ERR_DEVICE = -8     /* no usable gfx950 device / HIP runtime error                       */
} qg_status;

#define QG_MAX_PLANES 4

/* Device layout of one n x k matrix. */
typedef struct qg_layout {
  int64_t total_bytes;                        /* bytes to allocate (planes + padding)        */
  int64_t algorithmic_bytes;                  /* bytes one dequant-GEMV must read            */
  int32_t nplanes;
  int32_t reserved;
  int64_t plane_offset[QG_MAX_PLANES];        /* from the buffer start, 256-byte aligned     */
  int64_t plane_row_bytes[QG_MAX_PLANES];     /* bytes per row of each plane                 */
} qg_layout;

int qg_abi_version(void);
const char *qg_strerror(int status);
/* HIP's description of the last launch the library saw fail on this thread (QG_ERR_LAUNCH). */
const char *qg_last_hip_error(void);

/* ---- sizes and layouts (host) ------------------------------------------------------- */

/* Bytes of the canonical encoding of an n x k matrix: n * k / 256 records of 84 / 110 / 176 /
 * 210 bytes for the super-block formats ("二三五六位量化" page section 2.3, byte table), and
 * for INT4 16 bytes of codes plus the scale bytes per group (DBHOO-CIM page sections 3.2, 4.1).
 * Errors: QG_ERR_NULL, QG_ERR_FORMAT, QG_ERR_SHAPE. */
int qg_canonical_bytes(int fmt, int64_t n, int64_t k, int64_t *bytes);
/* Device layout of an n x k matrix: the planes (codes, high-bit planes, sub-scales,
 * super-scales) kept apart, as the pages advise for the scales (DBHOO-CIM page section 4.1,
 * "二三五六位量化" page section 2.3), with their offsets and row strides; algorithmic_bytes
 * equals the canonical size. Errors: QG_ERR_NULL, QG_ERR_FORMAT, QG_ERR_SHAPE. */
int qg_device_layout(int fmt, int64_t n, int64_t k, qg_layout *out);
/* The two sizes a caller needs, in one call: *total = bytes to allocate for the device layout
 * (planes and padding), *algorithmic = the bytes one dequant GEMV reads (the canonical size,
 * which the effective-bandwidth figure of DBHOO-CIM page section 4.4 divides by the time).
 * Either pointer may be NULL. Errors: QG_ERR_FORMAT, QG_ERR_SHAPE. */
int qg_packed_bytes(int fmt, int64_t n, int64_t k, int64_t *total, int64_t *algorithmic);

/* ---- bitstreams (host; "二三五六位量化" page section 2.2) ---------------------------- */

/* Pack count codes of `bits` bits (1..8) into a little-endian bitstream of
 * ceil(count*bits/8) bytes; code i occupies stream bits [bits*i, bits*i + bits).
 * Codes must be < 2^bits (QG_ERR_RANGE otherwise). */
int qg_pack_bits(int bits, const uint8_t *codes, int64_t count, uint8_t *out);
/* Inverse of qg_pack_bits. */
int qg_unpack_bits(int bits, const uint8_t *in, int64_t count, uint8_t *codes);

/* ---- quantizers (host, synchronous) -------------------------------------------------- */

/* Quantize fp32 W [n][ldw] (first k columns used, ldw >= k) into the canonical encoding
 * `canonical` (qg_canonical_bytes(fmt, n, k) bytes). Multi-threaded over rows; the output is
 * independent of the thread count. Errors: QG_ERR_SHAPE, QG_ERR_NONFINITE, QG_ERR_RANGE. */
int qg_quantize(int fmt, const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q4g32(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q2sb(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q3sb(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q5sb(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q6sb(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q4g16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q4g64(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q4g128(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q4a32(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q4g32h(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q2sb_bf16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q3sb_bf16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q5sb_bf16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q6sb_bf16(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q3g32(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q5g32(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);
int quantize_q3sb_planes(const float *w, int64_t n, int64_t k, int64_t ldw, uint8_t *canonical);

/* Canonical encoding (host) -> device layout (host buffer of qg_device_layout().total_bytes;
 * padding is zeroed). A pure bit permutation: the scales move to planes of their own
 * (DBHOO-CIM page section 4.1 keeps scales in a separate array) and the codes to planes of
 * whole bit fields ("二三五六位量化" page section 2.3 splits 5- and 6-bit codes into a low
 * plane and a high-bit plane). Errors: QG_ERR_NULL, QG_ERR_FORMAT, QG_ERR_SHAPE. */
int qg_to_device_layout(int fmt, const uint8_t *canonical, int64_t n, int64_t k, uint8_t *device_layout);
/* Device layout (host copy) -> canonical encoding. Inverse of qg_to_device_layout; same
 * errors. */
int qg_from_device_layout(int fmt, const uint8_t *device_layout, int64_t n, int64_t k, uint8_t *canonical);

/* ---- dequant GEMV, batch 1 (device) ------------------------------------------------------
 * y[r] = sum_c W_hat[r][c] * x[c] for r < n, with W in device layout (`w`, 256-byte aligned),
 * x fp16 [k] (16-byte aligned), y fp16 [n]; fp32 accumulation, one fp16 rounding at the end.
 * The packed weights are streamed once with 128-bit loads and decoded in registers; no
 * dequantized weight is ever written to memory (DBHOO-CIM page section 3.3; "二三五六位量化"
 * page section 3.3's gemv_q3 and its Sigma-x rewrite). Limits: k <= 2^20 and every plane
 * of the device layout under 4 GiB. n == 0 is a no-op; k == 0 writes zeros.
 * Errors: QG_ERR_NULL, QG_ERR_SHAPE, QG_ERR_ALIGN, QG_ERR_FORMAT, QG_ERR_LAUNCH. */
int dequant_gemv_q4g32(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q2sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q3sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q5sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q6sb(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q4g16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q4g64(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q4g128(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q4a32(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q4g32h(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q2sb_bf16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q3sb_bf16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q5sb_bf16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q6sb_bf16(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q3g32(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q5g32(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);
int dequant_gemv_q3sb_planes(const void *w, const uint16_t *x, uint16_t *y, int64_t n, int64_t k, void *stream);

/* Generic form: y_f32 != 0 writes fp32 y (4-byte aligned) instead of fp16. */
int qg_gemv(int fmt, const void *w, const uint16_t *x, void *y, int y_f32, int64_t n, int64_t k, void *stream);

/* Strided batch of independent GEMVs of one shape in one launch: for b < count,
 * y_b = W_b x_b with W_b at w + b*w_stride (bytes, multiple of 256), x_b at x + b*x_stride
 * and y_b at y + b*y_stride (elements; x_stride a multiple of 8). Same numerics as qg_gemv.
 * This is how a decode step issues several same-shape projections (or experts) without a
 * launch per matrix ("二三五六位量化" page section 1.2: decode reads every weight once per
 * token, one stream bound by bandwidth). count == 0 is a no-op. Errors as qg_gemv, and
 * QG_ERR_SHAPE for count < 0, QG_ERR_ALIGN for a misaligned stride. */
int qg_gemv_batched(int fmt, const void *w, int64_t w_stride, const uint16_t *x, int64_t x_stride,
                    void *y, int64_t y_stride, int y_f32, int64_t count, int64_t n, int64_t k, void *stream);

/* ---- dequant GEMM with a few activation rows (device) ------------------------------------
 * Y[i][r] = sum_c X[i][c] * W_hat[r][c] for i < m, r < n: X fp16 [m][ldx] (16-byte aligned,
 * ldx >= k and a multiple of 8 when m > 1), Y fp16 [m][ldy] (ldy >= n when m > 1). Batched
 * decode: the weights are streamed once per launch and each decoded code meets all the
 * launch's activation rows, up to 16 of them ("二三五六位量化" page section 1.2: decode
 * batches and prefill are the same contraction with more activation rows; DBHOO-CIM page
 * section 5.2: still bandwidth-bound at small batch, compute-bound at large batch). Any m >= 1:
 * m <= 4 runs on the vector units (each decoded code pair meets every activation row in a
 * v_dot2; the kernel of qg_gemv, qg_gemm_grouped and qg_gemm_act_order), 5 <= m <= 16
 * decodes each code once to fp16 and multiplies on the matrix cores in the same single
 * weight stream, and m > 16 (prefill) stages fp16 weight and activation tiles in LDS for
 * 32x32 matrix-core tiles. For 17 <= m <= 128, when a cost estimate says so (the prefill
 * tiles then carry mostly dead rows), the rows run instead as launches of that decode
 * kernel of up to 32 rows each (two 16-row blocks share each decoded fragment; a 32-row
 * launch gives the same bits as two 16-row launches). Limits as dequant_gemv_*; also
 * ldx < 2^26 for 5 <= m <= 16 and
 * ldx < 2^22 for m > 16 (32-bit activation offsets within a 16-row or a 256-row tile).
 * m == 0 or n == 0 is a no-op; k == 0 writes zeros. Errors as dequant_gemv_*.
 * Precision: m <= 4 works on the codes in fp32 (the 2e-3 * sum |W_hat x| bound holds at any
 * weight and activation scale). The matrix-core paths (m > 4) round each decoded weight to
 * fp16, which keeps 11 significant bits down to 2^-14 only: they hold the bound while the
 * quantization steps (an INT4 group scale, a super-block's d * sc) are at least 2^-14 and
 * the weights stay within +-65504; smaller steps lose relative precision (fp16 subnormals)
 * and weights beyond the fp16 range (the _bf16 formats only) are not representable. Such
 * layers take m <= 4 launches, or qg_gemm_grouped / qg_gemm_act_order up to 8 rows. */
int dequant_gemm_q4g32(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                       int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q2sb(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                      int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q3sb(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                      int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q5sb(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                      int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q6sb(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                      int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q4g16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                      int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q4g64(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                      int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q4g128(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                      int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q4a32(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                       int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q4g32h(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                        int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q2sb_bf16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                            int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q3sb_bf16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                            int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q5sb_bf16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                            int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q6sb_bf16(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                            int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q3g32(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                        int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q5g32(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                        int64_t m, int64_t n, int64_t k, void *stream);
int dequant_gemm_q3sb_planes(const void *w, const uint16_t *X, int64_t ldx, uint16_t *Y, int64_t ldy,
                              int64_t m, int64_t n, int64_t k, void *stream);
/* Generic form; y_f32 != 0 writes fp32 Y (4-byte aligned). */
int qg_gemm(int fmt, const void *w, const uint16_t *X, int64_t ldx, void *Y, int64_t ldy, int y_f32,
            int64_t m, int64_t n, int64_t k, void *stream);

/* Act-order weights ("二三五六位量化" page section 2.4 and section 3.2, stage 3: GPTQ
 * quantizes the columns in an activation-dependent order and stores that permutation, which
 * inference must apply): W was quantized with its columns permuted, stored column c being
 * original column perm[c], so Y[i][r] = sum_c X[i][perm[c]] * W_hat[r][c]. perm: int32 [k] on
 * the device (16-byte aligned), entries in [0, k) (an entry outside that range reads an
 * activation of 0; it never reads outside X). The gather is fused into the streaming
 * kernel's activation load, so the result equals that kernel's on the gathered activations
 * bit for bit (qg_gemm_grouped's for any m, qg_gemm's for m <= 4). Activation rows of more
 * than 128 KB (m * k * 2 bytes) run as several launches of half, a quarter, ... of the rows,
 * the first size that fits; each such chunk equals qg_gemm_grouped's launch on its rows.
 * m: 0..8 activation rows (the streaming kernel); other arguments, limits and errors as
 * qg_gemm. */
int qg_gemm_act_order(int fmt, const void *w, const uint16_t *X, int64_t ldx, const int32_t *perm, void *Y,
                      int64_t ldy, int y_f32, int64_t m, int64_t n, int64_t k, void *stream);

/* Several matrices of any shapes, one activation-row count m (0..8), in one launch: for
 * g < count (at most 8), Y_g [m][ldy[g]] = X_g [m][ldx[g]] * W_hat_g^T with W_g of n[g] x k[g]
 * at w[g]. The arrays are host arrays read during the call; ldx and ldy are read only when
 * m > 1 (else the rows are dense). Each matrix is checked as by qg_gemm (for m <= 8) before
 * anything is launched; a matrix with n[g] == 0 is skipped and one with k[g] == 0 gets
 * zeros. Every matrix runs on the streaming vector-unit kernel of qg_gemv and shares its
 * numerics (qg_gemm's for m <= 4; for 5 <= m <= 8 qg_gemm uses the matrix cores and agrees
 * within the tolerance, not bit for bit). This serves the projections of a decode step that read one activation (q, k and
 * v; gate and up) or simply follow each other, with one launch's start and drain instead
 * of one per matrix ("二三五六位量化" page section 1.2: the decode pass is one weight stream
 * bound by bandwidth). Errors: QG_ERR_SHAPE (count > 8, m > 8, or a matrix's shape),
 * QG_ERR_NULL, QG_ERR_ALIGN, QG_ERR_FORMAT, QG_ERR_LAUNCH. */
int qg_gemm_grouped(int fmt, int count, const void *const *w, const uint16_t *const *X, const int64_t *ldx,
                    void *const *Y, const int64_t *ldy, const int64_t *n, const int64_t *k, int64_t m, int y_f32,
                    void *stream);

/* ---- 8-bit KV-cache group codec (device) --------------------------------------------------
 * "二三五六位量化" page section 4.1: the KV cache quantized to 8 bits, every 32 elements
 * sharing one fp16 scale (about 1.06 bytes per element, half of fp16). Codes are symmetric
 * int8 in [-127, 127]; the scale d of a group is the smallest fp16 >= max|x| / 127, q is
 * rint(x / d) on the exact quotient (halves to even), an all-zero group has d = 0 and q = 0,
 * and every element is within d/2 of d * q.
 *
 * qg_kv_quantize (on append): src fp16 [rows][ld_src] (first cols used; 16-byte aligned,
 * ld_src a multiple of 8 when rows > 1) -> codes int8 [rows][cols] (8-byte aligned) and scales
 * fp16 [rows][cols/32] (2-byte aligned). qg_kv_dequantize (on read): codes and scales ->
 * dst fp16 [rows][ld_dst] (16-byte aligned, ld_dst a multiple of 8 when rows > 1), each value
 * d * q rounded once to fp16 and saturated at +-65504 (d * q exceeds it only for code
 * +-127 at d = 516, the scale of a group whose maximum is above 65469; the saturated value
 * is still within d/2 of the input). cols must be a multiple of 32. Inputs must be finite
 * (a NaN or Inf gives unspecified codes for its group). rows == 0 or cols == 0 is a no-op.
 * Errors: QG_ERR_SHAPE, QG_ERR_NULL, QG_ERR_ALIGN, QG_ERR_LAUNCH. */
int qg_kv_quantize(const uint16_t *src, int64_t ld_src, int64_t rows, int64_t cols, int8_t *codes, uint16_t *scales,
                   void *stream);
int qg_kv_dequantize(const int8_t *codes, const uint16_t *scales, int64_t rows, int64_t cols, uint16_t *dst,
                     int64_t ld_dst, void *stream);

/* ---- decode to memory (device; for verification, not for inference) ----------------------
 * Writes W_hat as fp32 [n][k] to w_out (if non-NULL) and the integer codes as uint8 [n][k]
 * to codes_out (if non-NULL; q4g32 writes the unsigned nibble u = q + 8, q4a32 the code c).
 * fp32 values are single-rounding products (q*scale, (c - z)*s, d*sc*(c - o),
 * fma(d*sc, c, -dmin*m), fma(s, c, m)), hence exactly fp32(W_hat). */
int dequantize_q4g32(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q2sb(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q3sb(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q5sb(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q6sb(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q4g16(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q4g64(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q4g128(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q4a32(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q4g32h(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q2sb_bf16(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q3sb_bf16(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q5sb_bf16(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q6sb_bf16(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q3g32(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q5g32(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int dequantize_q3sb_planes(const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);
int qg_dequantize(int fmt, const void *w, float *w_out, uint8_t *codes_out, int64_t n, int64_t k, void *stream);

/* ---- measurement (device) -----------------------------------------------------------------
 * Streams `bytes` bytes (a multiple of 16; buf 16-byte aligned) through non-temporal 128-bit
 * loads (a grid-stride loop, four loads in flight per thread) and writes nothing except, with
 * negligible probability, one word of `sink`: the achievable HBM
 * read rate the GEMV kernels are measured against (the DBHOO-CIM page, section 5.3,
 * measures the machine's ceiling with STREAM first). */
int qg_read_probe(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
