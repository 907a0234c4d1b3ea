/*
 * qfa_oracle.c -- plain, slow CPU oracle for the QK4PV8 attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links or calls this
 * file; only the test-suite, the smoke check and the benchmark's CPU-baseline leg
 * load it.  It shares no code, header, table or constant generator with the HIP
 * path.  Arithmetic is IEEE binary64 unless a step says otherwise.
 *
 * Sources (web pages; cited by title and section):
 *  [MpFA]  "MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on
 *          Blackwell GPUs" (arxivdaily entry), English abstract: Q/K in 4-bit
 *          with block scales, P and V in FP8 (QK4PV8), online quantisation of P
 *          after softmax, rank-one smoothing compensation as one extra MMA,
 *          split partitioning for prefill and decode.
 *  [FA4tut] "FlashAttention压到4位：矩阵乘快一倍多，训练却只快14%" (bloombook
 *          tutorial): section "注意力慢在哪儿" (tiling + online softmax with a
 *          running max m and running sum l, exact against full softmax; LSE per
 *          row), section "FP4 只有约 15 个可表示的数" (E2M1 magnitudes
 *          0, 1/2, 1, 3/2, 2, 3, 4, 6; MXFP4 = 32 elements + one E8M0
 *          power-of-two scale), section "Direct-P" (the softmax denominator
 *          must use the same rounded codes that the PV product consumes).
 *  [MXnotes] hnwysp.cn notes on MXAttention / MXFP4 KV-cache compression,
 *          section 2.3 (block amax -> power-of-two scale -> divide -> round ->
 *          store codes and scale) and section 5.2 (round to nearest even, not
 *          floor).
 *  [Blog]  "Blackwell免训练4-bit注意力MpFA：QK4V8量化与FlashAttention内核解析"
 *          (sheratonhq blog), section 2.1: S = QK^T/sqrt(d), P = softmax(S),
 *          O = PV, and softmax is unchanged by a per-row constant.
 *
 * Readings where the pages leave a step open (each is also listed in the
 * design notes of the repository):
 *  - QK format: MXFP4 (E2M1 elements, one E8M0 scale per 32 consecutive
 *    elements along D).  Scale exponent e = ceil(log2 amax) - 2, clamped to
 *    [-127, 127]; amax == 0 gives e = -127 (code 0); a block holding a NaN or
 *    an infinity gets scale code 0xFF and element codes 0.
 *  - V format: E4M3 (OCP "FN": bias 7, max 448, 0x7F/0xFF NaN) with one E8M0
 *    scale per 32 consecutive tokens of one channel, e = ceil(log2 amax) - 8.
 *    Codes are stored block-contiguous: [B][H][S/32][D][32].
 *  - Element rounding: round-to-nearest, ties to the even code, applied once to
 *    the exact value x * 2^-e; the sign of zero is kept; magnitudes beyond the
 *    largest finite value saturate to it.
 *  - Softmax scale: S = Q K^T / sqrt(d) is exponentiated in base 2, so the
 *    factor c2 = fl32(softmax_scale * log2 e) is applied to Q before Q is
 *    quantised (Q' = fl32(q * c2), then MXFP4).  The pages do not say where
 *    the scale enters; applied to Q, the product Q'K^T is already the
 *    exponent argument in log2 units.
 *  - P is E4M3(256 * 2^(s - m)) with m the running max in log2 units kept on
 *    the integer grid: after every 128-token key tile (ascending order)
 *    m <- max(m, ceil(max_j s_j)).  Online softmax only needs m to bound the
 *    row max from above; an integer m makes every rescale factor 2^(m - m')
 *    an exact power of two and, because E4M3 rounding commutes with powers of
 *    two, makes the P codes independent of the tile and split schedule (up to
 *    the subnormal range).  The denominator l sums the decoded P codes.  O is
 *    returned in binary64 here, LSE in natural-log units referring to the
 *    compensated logits.
 *  - Rank-one smoothing compensation: K is smoothed per 128-token block by its
 *    channel mean Kbar: the block's values of the channel summed in binary64
 *    in token order (exact unless they span more than 2^38 in magnitude),
 *    divided by the count of present tokens in binary64, rounded to bf16 (an
 *    infinite or NaN mean stays one).  Every logit of a block gets back the
 *    rank-one term q_bf16 . Kbar_block.
 *  - Causal masks are bottom-right aligned: key j is visible to query i iff
 *    j <= i + (L - Sq).  Query head h reads kv head h / (Hq / Hkv).
 *  - Decode splits are contiguous runs of whole 128-token tiles, merged by
 *    log-sum-exp.
 *  - The exponent argument of P and its exponential (which decide an integer
 *    code) are binary32, the precision the kernels decide in (fp32_arg = 1):
 *    y = fl32(fl32(S) + fl32(c2 * fl32(delta))), m' = max(m, ceil(max y)),
 *    P = E4M3(256 * fl32(2^(y - m'))) with fl32 the correctly rounded binary32
 *    value (ties of the E4M3 rounding go to the even code).  Without the
 *    compensation y = S exactly.  Every other exponential, sum and product is
 *    evaluated in binary64.
 *  - Contrast cases (not the method; see tile_p): P in E4M3 with one E8M0
 *    scale per (row, 32 keys) instead of one per row, and MXFP4 P and V
 *    ("QK4PV4": E2M1 codes, one E8M0 scale per 32 keys of a row for P and per
 *    32 tokens of a channel for V).  A block's scale exponent is the ceiling of
 *    its max, floored at 64 below the row's running max.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QFA_ORC_TILE 128
#define QFA_ORC_BLOCK 32

/* ------------------------------------------------------------------------- */
/* Element formats                                                           */
/* ------------------------------------------------------------------------- */

/* E2M1 code layout s e1 e0 m.  Exponent field 0 encodes 0 and 1/2; otherwise
 * (1 + m/2) * 2^(e-1).  [FA4tut, "FP4 只有约 15 个可表示的数"] */
double orc_e2m1_value(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* Nearest of the eight E2M1 magnitudes; on an exact tie the code with mantissa
 * bit 0 wins (round half to even).  Values beyond 6 land on 6. */
int orc_e2m1_encode(double v) {
  int sign = signbit(v) ? 8 : 0;
  double a = fabs(v);
  /* above the largest value 6 the nearest value is 6 (saturation); taken
   * first, because for huge a every distance a - value rounds to a itself */
  if (a > 6.0) return sign | 7;
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double d = fabs(orc_e2m1_value(c) - a);
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      bestd = d;
      best = c;
    }
  }
  return sign | best;
}

/* OCP E4M3 ("FN"): bias 7, exponent field 0 is subnormal m/8 * 2^-6,
 * S.1111.111 is NaN, no infinities, largest finite 448. */
double orc_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(8.0 + m, e - 10);
  return s ? -mag : mag;
}

/* Round to nearest, ties to even, of an exact binary64 value; saturating to
 * +-448; NaN -> 0x7F. */
int orc_e4m3_encode(double v) {
  if (isnan(v)) return 0x7F;
  int sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: units of 2^-9, 0..8 (8 becomes the smallest normal) */
    double n = nearbyint(ldexp(a, 9));
    return sign | (int)n; /* n == 8 is exactly code 0x08 = 2^-6 */
  }
  int ex;
  frexp(a, &ex);      /* a = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;     /* a in [2^e, 2^(e+1)) */
  double n = nearbyint(ldexp(a, 3 - e)); /* 8..16 */
  int code = ((e + 7) << 3) + ((int)n - 8); /* n == 16 carries into the exponent */
  if (code > 0x7E) code = 0x7E;
  return sign | code;
}

/* E8M0: 2^(code - 127), 0xFF is NaN. */
double orc_e8m0_value(int code) {
  if ((code & 0xFF) == 0xFF) return NAN;
  return ldexp(1.0, (code & 0xFF) - 127);
}

/* ceil(log2 a) for finite a > 0, from frexp (exact, subnormals included). */
static int ceil_log2(double a) {
  int ex;
  double f = frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  return (f == 0.5) ? ex - 1 : ex;
}

/* Shared-scale exponent of an MX block: ceil(log2 amax) - k, clamped to
 * [-127, 127]; amax == 0 -> -127.  k = 2 for E2M1 (block maximum lands in
 * (2, 4]) and k = 8 for E4M3 (block maximum lands in (128, 256]). */
int orc_mx_exponent(double amax, int k) {
  if (!(amax > 0.0)) return -127;
  int e = ceil_log2(amax) - k;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* bfloat16 */
double orc_bf16_value(uint16_t bits) {
  union { uint32_t u; float f; } x;
  x.u = (uint32_t)bits << 16;
  return (double)x.f;
}

/* Round an exact binary64 value to bfloat16, nearest-even. */
uint16_t orc_bf16_from_double(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7FC0;
  if (isinf(v)) return sign | 0x7F80;
  if (a == 0.0) return sign;
  if (a < ldexp(1.0, -126)) { /* subnormal: units of 2^-133 */
    double n = nearbyint(ldexp(a, 133));
    return sign | (uint16_t)n; /* n == 128 is the smallest normal */
  }
  int ex;
  frexp(a, &ex);
  int e = ex - 1;
  double n = nearbyint(ldexp(a, 7 - e)); /* 128..256 */
  int32_t biased = e + 127;
  int32_t bits = (biased << 7) + ((int32_t)n - 128);
  if (bits >= 0x7F80) bits = 0x7F80; /* overflow -> inf */
  return sign | (uint16_t)bits;
}

/* ------------------------------------------------------------------------- */
/* Quantizers                                                                */
/* ------------------------------------------------------------------------- */

/* Channel means of K per 128-token block: the binary64 sum in token order
 * (exact while the block's values of the channel span at most 2^38 in
 * magnitude: then every partial sum is an integer multiple of the smallest
 * value's bf16 unit below 2^53 of them), divided by the count of present
 * tokens and rounded to bf16.  kbar layout [B][H][ceil(S/128)][D]. */
static void kbar_of(const uint16_t* x, int64_t S, int64_t D, uint16_t* kbar) {
  int64_t nt = (S + QFA_ORC_TILE - 1) / QFA_ORC_TILE;
  for (int64_t t = 0; t < nt; ++t) {
    int64_t j0 = t * QFA_ORC_TILE, j1 = j0 + QFA_ORC_TILE < S ? j0 + QFA_ORC_TILE : S;
    for (int64_t c = 0; c < D; ++c) {
      double sum = 0.0;
      for (int64_t j = j0; j < j1; ++j) sum += orc_bf16_value(x[j * D + c]);
      kbar[t * D + c] = orc_bf16_from_double(sum / (double)(j1 - j0));
    }
  }
}

/* MXFP4 quantisation of one run of 32 elements given as binary64 values that
 * are exactly binary32 numbers.  Writes 16 code bytes (even element in the
 * low nibble) and returns the scale code.  [MXnotes 2.3, 5.2] */
static int mxfp4_block(const double* x, uint8_t* codes) {
  double amax = 0.0;
  int finite = 1;
  for (int i = 0; i < QFA_ORC_BLOCK; ++i) {
    if (!isfinite(x[i])) finite = 0;
    else if (fabs(x[i]) > amax) amax = fabs(x[i]);
  }
  if (!finite) {
    memset(codes, 0, QFA_ORC_BLOCK / 2);
    return 0xFF;
  }
  int e = orc_mx_exponent(amax, 2);
  for (int i = 0; i < QFA_ORC_BLOCK; i += 2) {
    int lo = orc_e2m1_encode(ldexp(x[i], -e));
    int hi = orc_e2m1_encode(ldexp(x[i + 1], -e));
    codes[i / 2] = (uint8_t)(lo | (hi << 4));
  }
  return e + 127;
}

/* Q or K [B][H][S][D] bf16 -> codes [B][H][S][D/2], scales [B][H][S][D/32].
 * With smooth != 0 the 128-token channel means are written to kbar
 * [B][H][ceil(S/128)][D] and the quantised tensor is fl32(K - Kbar) (one
 * correctly rounded binary32 subtraction).  Each element is then multiplied
 * by prescale in binary32 (fl32(v * prescale); 1 leaves it unchanged): Q is
 * quantised as fl32(q * c2) with c2 = fl32(softmax_scale * log2 e), so that
 * Q'K^T is already the exponent argument in log2 units.  D must be a
 * multiple of 32. */
void orc_quantize_qk4(const uint16_t* x, int64_t B, int64_t H, int64_t S, int64_t D, int smooth, float prescale,
                      uint8_t* codes, uint8_t* scales, uint16_t* kbar) {
  int64_t nt = (S + QFA_ORC_TILE - 1) / QFA_ORC_TILE;
  int64_t nb = D / QFA_ORC_BLOCK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const uint16_t* xs = x + bh * S * D;
    uint16_t* kb = smooth ? kbar + bh * nt * D : NULL;
    if (smooth) kbar_of(xs, S, D, kb);
    double buf[QFA_ORC_BLOCK];
    for (int64_t s = 0; s < S; ++s) {
      for (int64_t blk = 0; blk < nb; ++blk) {
        for (int i = 0; i < QFA_ORC_BLOCK; ++i) {
          int64_t c = blk * QFA_ORC_BLOCK + i;
          double v = orc_bf16_value(xs[s * D + c]);
          if (smooth) v = (double)(float)(v - orc_bf16_value(kb[(s / QFA_ORC_TILE) * D + c]));
          if (prescale != 1.0f) v = (double)((float)v * prescale);
          buf[i] = v;
        }
        int64_t row = bh * S + s;
        scales[row * nb + blk] =
            (uint8_t)mxfp4_block(buf, codes + row * (D / 2) + blk * (QFA_ORC_BLOCK / 2));
      }
    }
  }
}

/* V [B][H][S][D] bf16 -> E4M3 codes [B][H][ceil(S/32)][D][32] and E8M0 scales
 * [B][H][ceil(S/32)][D]; one block = 32 consecutive tokens of one channel.
 * Tokens past S in the last block are absent: they do not enter amax and get
 * code 0. */
void orc_quantize_v8(const uint16_t* v, int64_t B, int64_t H, int64_t S, int64_t D,
                     uint8_t* codes, uint8_t* scales) {
  int64_t nblk = (S + QFA_ORC_BLOCK - 1) / QFA_ORC_BLOCK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const uint16_t* vs = v + bh * S * D;
    for (int64_t blk = 0; blk < nblk; ++blk) {
      int64_t j0 = blk * QFA_ORC_BLOCK;
      int64_t n = S - j0 < QFA_ORC_BLOCK ? S - j0 : QFA_ORC_BLOCK;
      for (int64_t c = 0; c < D; ++c) {
        uint8_t* out = codes + ((bh * nblk + blk) * D + c) * QFA_ORC_BLOCK;
        double amax = 0.0;
        int finite = 1;
        for (int64_t t = 0; t < n; ++t) {
          double x = orc_bf16_value(vs[(j0 + t) * D + c]);
          if (!isfinite(x)) finite = 0;
          else if (fabs(x) > amax) amax = fabs(x);
        }
        memset(out, 0, QFA_ORC_BLOCK);
        if (!finite) {
          scales[(bh * nblk + blk) * D + c] = 0xFF;
          continue;
        }
        int e = orc_mx_exponent(amax, 8);
        for (int64_t t = 0; t < n; ++t)
          out[t] = (uint8_t)orc_e4m3_encode(ldexp(orc_bf16_value(vs[(j0 + t) * D + c]), -e));
        scales[(bh * nblk + blk) * D + c] = (uint8_t)(e + 127);
      }
    }
  }
}

/* V [B][H][S][D] bf16 -> MXFP4 codes [B][H][ceil(S/32)][D][16] and E8M0
 * scales [B][H][ceil(S/32)][D]: the MXFP4 rule of the Q/K quantiser (e =
 * ceil(log2 amax) - 2) applied to each block of 32 consecutive tokens of one
 * channel, token 2k in the low nibble of byte k.  Tokens past S in the last
 * block count as 0 (no effect on amax, code 0).  This is the V side of the
 * full-FP4 "QK4PV4" contrast case ([MpFA] abstract; [FA4tut] "Direct-P": P
 * and V in MXFP4 with one E8M0 scale per 32). */
void orc_quantize_v4(const uint16_t* v, int64_t B, int64_t H, int64_t S, int64_t D,
                     uint8_t* codes, uint8_t* scales) {
  int64_t nblk = (S + QFA_ORC_BLOCK - 1) / QFA_ORC_BLOCK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const uint16_t* vs = v + bh * S * D;
    double buf[QFA_ORC_BLOCK];
    for (int64_t blk = 0; blk < nblk; ++blk) {
      int64_t j0 = blk * QFA_ORC_BLOCK;
      int64_t n = S - j0 < QFA_ORC_BLOCK ? S - j0 : QFA_ORC_BLOCK;
      for (int64_t c = 0; c < D; ++c) {
        for (int64_t t = 0; t < QFA_ORC_BLOCK; ++t) buf[t] = t < n ? orc_bf16_value(vs[(j0 + t) * D + c]) : 0.0;
        scales[(bh * nblk + blk) * D + c] =
            (uint8_t)mxfp4_block(buf, codes + ((bh * nblk + blk) * D + c) * (QFA_ORC_BLOCK / 2));
      }
    }
  }
}

/* NVFP4 quantisation of one run of 16 elements given as binary32 values, with
 * the per-tensor scale g (a power of two): the block scale is the E4M3 code
 * (RNE, saturating at 448) of the binary32 quotient fl32(fl32(amax / g) / 6),
 * 6 being the largest E2M1 magnitude; each element is the E2M1 code (RNE,
 * saturating at 6) of the binary32 quotient fl32(x / (s g)) with s the
 * decoded scale.  A scale of 0 gives zero codes; a block holding a NaN or an
 * infinity gets scale code 0x7F and zero codes.  Writes 8 code bytes (even
 * element in the low nibble) and returns the scale code.  [FA4tut] "FP4 只有约
 * 15 个可表示的数" (NVFP4: blocks of 16, E4M3 scale, optional FP32 tensor
 * scale; about 4.5 bits per value) and [MpFA] abstract (NVFP4 for QK). */
static int nvfp4_block(const float* x, float g, uint8_t* codes) {
  float amax = 0.0f;
  int finite = 1;
  for (int i = 0; i < 16; ++i) {
    if (!isfinite(x[i])) finite = 0;
    else if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
  }
  memset(codes, 0, 8);
  if (!finite) return 0x7F;
  volatile float q = amax / g; /* exact: g is a power of two */
  q = q / 6.0f;                /* binary32, correctly rounded */
  int sc = orc_e4m3_encode((double)q);
  float t = (float)orc_e4m3_value(sc) * g; /* exact */
  if (t == 0.0f) return sc;
  for (int i = 0; i < 16; i += 2) {
    volatile float a = x[i] / t, b = x[i + 1] / t;
    int lo = orc_e2m1_encode((double)a);
    int hi = orc_e2m1_encode((double)b);
    codes[i / 2] = (uint8_t)(lo | (hi << 4));
  }
  return sc;
}

/* Q or K [B][H][S][D] bf16 -> NVFP4 codes [B][H][S][D/2] and E4M3 block scales
 * [B][H][S][D/16], with the per-tensor scale g (a power of two).  smooth and
 * prescale as for orc_quantize_qk4: the quantised value is fl32(fl32(K - Kbar)
 * * prescale). */
void orc_quantize_nvfp4(const uint16_t* x, int64_t B, int64_t H, int64_t S, int64_t D, int smooth, float prescale,
                        float g, uint8_t* codes, uint8_t* scales, uint16_t* kbar) {
  int64_t nt = (S + QFA_ORC_TILE - 1) / QFA_ORC_TILE;
  int64_t nb = D / 16;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const uint16_t* xs = x + bh * S * D;
    uint16_t* kb = smooth ? kbar + bh * nt * D : NULL;
    if (smooth) kbar_of(xs, S, D, kb);
    float buf[16];
    for (int64_t s = 0; s < S; ++s) {
      for (int64_t blk = 0; blk < nb; ++blk) {
        for (int i = 0; i < 16; ++i) {
          int64_t c = blk * 16 + i;
          double v = orc_bf16_value(xs[s * D + c]);
          if (smooth) v = (double)(float)(v - orc_bf16_value(kb[(s / QFA_ORC_TILE) * D + c]));
          if (prescale != 1.0f) v = (double)((float)v * prescale);
          buf[i] = (float)v;
        }
        int64_t row = bh * S + s;
        scales[row * nb + blk] = (uint8_t)nvfp4_block(buf, g, codes + row * (D / 2) + blk * 8);
      }
    }
  }
}

/* ------------------------------------------------------------------------- */
/* Dequantizers (exact in binary64)                                          */
/* ------------------------------------------------------------------------- */

void orc_dequant_qk4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t D, double* out) {
  int64_t nb = D / QFA_ORC_BLOCK;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < D; ++c) {
      uint8_t byte = codes[r * (D / 2) + c / 2];
      int code = (c & 1) ? (byte >> 4) : (byte & 15);
      out[r * D + c] = orc_e2m1_value(code) * orc_e8m0_value(scales[r * nb + c / QFA_ORC_BLOCK]);
    }
}

/* NVFP4 rows: codes [rows][D/2], E4M3 scales [rows][D/16], tensor scale g -> v * s * g. */
void orc_dequant_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t D, double g, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < D; ++c) {
      uint8_t byte = codes[r * (D / 2) + c / 2];
      int code = (c & 1) ? (byte >> 4) : (byte & 15);
      out[r * D + c] = orc_e2m1_value(code) * orc_e4m3_value(scales[r * (D / 16) + c / 16]) * g;
    }
}

/* One (b, h) slice: codes [ceil(S/32)][D][32], scales [ceil(S/32)][D] -> [S][D]. */
void orc_dequant_v8(const uint8_t* codes, const uint8_t* scales, int64_t S, int64_t D, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < S; ++j)
    for (int64_t c = 0; c < D; ++c) {
      int64_t blk = j / QFA_ORC_BLOCK;
      out[j * D + c] = orc_e4m3_value(codes[(blk * D + c) * QFA_ORC_BLOCK + j % QFA_ORC_BLOCK]) *
                       orc_e8m0_value(scales[blk * D + c]);
    }
}

/* One (b, h) slice: codes [ceil(S/32)][D][16], scales [ceil(S/32)][D] -> [S][D]. */
void orc_dequant_v4(const uint8_t* codes, const uint8_t* scales, int64_t S, int64_t D, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < S; ++j)
    for (int64_t c = 0; c < D; ++c) {
      int64_t blk = j / QFA_ORC_BLOCK, t = j % QFA_ORC_BLOCK;
      uint8_t byte = codes[(blk * D + c) * (QFA_ORC_BLOCK / 2) + t / 2];
      int code = (t & 1) ? (byte >> 4) : (byte & 15);
      out[j * D + c] = orc_e2m1_value(code) * orc_e8m0_value(scales[blk * D + c]);
    }
}

/* ------------------------------------------------------------------------- */
/* (a) exact softmax attention, binary64, two passes.  [Blog 2.1]            */
/* ------------------------------------------------------------------------- */

static int visible(int64_t i, int64_t j, int64_t L, int64_t Sq, int causal) {
  return !causal || j <= i + (L - Sq);
}

/* Q [n][D] rows at positions qpos against one kv head K, V [L][D]. */
void orc_attn_exact_rows(const double* Q, const int64_t* qpos, int64_t n, const double* K, const double* V,
                         int64_t L, int64_t Sq, int64_t D, int causal, double softmax_scale, double* O,
                         double* lse) {
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < n; ++r) {
    const double* q = Q + r * D;
    int64_t i = qpos[r];
    double* o = O + r * D;
    double mx = -INFINITY;
    for (int64_t j = 0; j < L; ++j) {
      if (!visible(i, j, L, Sq, causal)) continue;
      double s = 0.0;
      for (int64_t c = 0; c < D; ++c) s += q[c] * K[j * D + c];
      s *= softmax_scale;
      if (s > mx) mx = s;
    }
    for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
    if (mx == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double den = 0.0;
    for (int64_t j = 0; j < L; ++j) {
      if (!visible(i, j, L, Sq, causal)) continue;
      double s = 0.0;
      for (int64_t c = 0; c < D; ++c) s += q[c] * K[j * D + c];
      double w = exp(s * softmax_scale - mx);
      den += w;
      for (int64_t c = 0; c < D; ++c) o[c] += w * V[j * D + c];
    }
    for (int64_t c = 0; c < D; ++c) o[c] /= den;
    lse[r] = mx + log(den);
  }
}

/* ------------------------------------------------------------------------- */
/* (c) quantised attention with the method's online-softmax schedule         */
/* ------------------------------------------------------------------------- */

#define LOG2E_F32 1.44269502162933349609375f /* binary32 nearest to log2(e) */

/* P of one tile from the exponent arguments y[0..n) (masked keys -inf) and
 * the row's new running max mnew, written as the values that multiply V and
 * enter the denominator, in the frame of mnew:
 *   QFA_P_EXACT        256 * 2^(y - mnew), not rounded (identity quantiser)
 *   QFA_P_E4M3         E4M3(256 * 2^(y - mnew)): the method (QK4PV8), one
 *                      power-of-two P scale per row
 *   QFA_P_E4M3_BLOCK   per 32-key block b of the tile (keys 32b .. 32b+31
 *                      from the tile start), e_b = max(ceil(max_{j in b} y_j),
 *                      mnew - 64) and 2^(e_b - mnew) * E4M3(256 * 2^(y - e_b)):
 *                      a dynamic E8M0 P scale per (row, 32 keys)
 *   QFA_P_E2M1_BLOCK   the same blocks with 2^(e_b - mnew) * E2M1(4 * 2^(y - e_b)):
 *                      MXFP4 P (the full-FP4 "QK4PV4" contrast case).  For
 *                      a block whose max is the row's, e_b - 2 is the MX
 *                      rule's ceil(log2 amax) - 2 with amax = 2^(max y - mnew).
 * The floor mnew - 64 bounds how far below the row a block's scale may go
 * (a block that far down holds no weight at binary32 precision); a block
 * with no visible key gets it too and contributes 0.  The scale per (row, 32
 * keys) follows [FA4tut] "Direct-P" (one E8M0 power-of-two scale per 32
 * probabilities) and [MpFA] abstract (QK4PV8 vs fully FP4 attention). */
#define QFA_P_EXACT 0
#define QFA_P_E4M3 1
#define QFA_P_E4M3_BLOCK 2
#define QFA_P_E2M1_BLOCK 3
#define QFA_P_BLOCK_FLOOR 64.0
/* 2^x, rounded to binary32 when the exponential is taken in binary32 (exp32):
 * the P code is an integer decided by floating point, and the kernels decide
 * it from a binary32 exponential.  exp2 in binary64 is far more accurate than
 * half a binary32 ulp, so the cast gives the correctly rounded binary32 value
 * (up to double rounding within 2^-53 of a binary32 midpoint). */
static double pexp2(double x, int exp32) {
  double e = exp2(x);
  return exp32 ? (double)(float)e : e;
}

static void tile_p(const double* y, int64_t n, double mnew, int p_mode, int exp32, double* P) {
  if (p_mode == QFA_P_EXACT || p_mode == QFA_P_E4M3) {
    for (int64_t j = 0; j < n; ++j) {
      if (y[j] == -INFINITY) {
        P[j] = 0.0;
        continue;
      }
      double p = ldexp(pexp2(y[j] - mnew, exp32 && p_mode == QFA_P_E4M3), 8);
      P[j] = p_mode == QFA_P_E4M3 ? orc_e4m3_value(orc_e4m3_encode(p)) : p;
    }
    return;
  }
  for (int64_t b0 = 0; b0 < n; b0 += QFA_ORC_BLOCK) {
    int64_t b1 = b0 + QFA_ORC_BLOCK < n ? b0 + QFA_ORC_BLOCK : n;
    double mu = -INFINITY;
    for (int64_t j = b0; j < b1; ++j)
      if (y[j] > mu) mu = y[j];
    double e = ceil(mu);
    if (!(e >= mnew - QFA_P_BLOCK_FLOOR)) e = mnew - QFA_P_BLOCK_FLOOR; /* also for mu = -inf */
    for (int64_t j = b0; j < b1; ++j) {
      if (y[j] == -INFINITY) {
        P[j] = 0.0;
        continue;
      }
      double v;
      if (p_mode == QFA_P_E4M3_BLOCK)
        v = orc_e4m3_value(orc_e4m3_encode(ldexp(pexp2(y[j] - e, exp32), 8)));
      else
        v = orc_e2m1_value(orc_e2m1_encode(ldexp(pexp2(y[j] - e, exp32), 2)));
      P[j] = ldexp(v, (int)(e - mnew));
    }
  }
}

/* One split [t0, t1) of 128-token tiles for one query row.  q is the
 * pre-scaled query row (q' = c2 q, so q' . k is in log2 units).  Returns 0 if
 * no key of the split is visible (the split then has weight 0), else fills o
 * (already divided by l) and *lse_out. */
static int split_row(const double* q, const double* qc, int64_t i, const double* K, const double* Kbar,
                     const double* V, int64_t L, int64_t Sq, int64_t D, int causal, float scale32,
                     int64_t t0, int64_t t1, int p_mode, int fp32_arg, double* o, double* lse_out,
                     double* S, double* P) {
  const float c2f = scale32 * LOG2E_F32;          /* binary32 product, as the kernel */
  const double c2d = (double)scale32 * M_LOG2E;   /* binary64 */
  double m = -INFINITY, l = 0.0;
  int any = 0;
  for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
  for (int64_t t = t0; t < t1; ++t) {
    int64_t j0 = t * QFA_ORC_TILE, j1 = j0 + QFA_ORC_TILE < L ? j0 + QFA_ORC_TILE : L;
    if (j0 >= L) break;
    /* logits of the tile in log2 units (exact); masked keys marked with -inf */
    double smax = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
      if (!visible(i, j, L, Sq, causal)) {
        S[j - j0] = -INFINITY;
        continue;
      }
      double s = 0.0;
      for (int64_t c = 0; c < D; ++c) s += q[c] * K[j * D + c];
      S[j - j0] = s;
      if (s > smax) smax = s;
    }
    if (smax == -INFINITY) continue; /* fully masked tile: skipped */
    any = 1;
    /* rank-one compensation term of this (row, tile): q_bf16 . Kbar_t */
    double delta = 0.0;
    if (Kbar)
      for (int64_t c = 0; c < D; ++c) delta += qc[c] * Kbar[t * D + c];
    /* exponent argument y_j of P (from here S holds y; masked keys stay -inf)
     * and the new running max m' = max(m, ceil(max_j y_j)) */
    double ymax = -INFINITY;
    if (fp32_arg) {
      /* in binary32, as the kernel forms it:
       *   y_j = fl32(fl32(S_j) + delta32),  delta32 = fl32(c2 * fl32(delta)) */
      const float d32 = Kbar ? c2f * (float)delta : 0.0f;
      for (int64_t j = 0; j < j1 - j0; ++j) {
        if (S[j] == -INFINITY) continue;
        float y = (float)S[j] + d32;
        S[j] = (double)y;
        if (S[j] > ymax) ymax = S[j];
      }
    } else {
      for (int64_t j = 0; j < j1 - j0; ++j) {
        if (S[j] == -INFINITY) continue;
        S[j] += c2d * delta;
        if (S[j] > ymax) ymax = S[j];
      }
    }
    const double mt = ceil(ymax);
    const double mnew = (m == -INFINITY || mt > m) ? mt : m;
    const double alpha = (m == -INFINITY) ? 0.0 : exp2(m - mnew);
    tile_p(S, j1 - j0, mnew, p_mode, fp32_arg, P);
    /* running sum of the same (decoded) P values that multiply V, and output
     * rescale  [FA4tut "Direct-P"; "注意力慢在哪儿"] */
    double lt = 0.0;
    for (int64_t j = 0; j < j1 - j0; ++j) lt += P[j];
    l = alpha * l + lt;
    for (int64_t c = 0; c < D; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < j1 - j0; ++j)
        if (P[j] != 0.0) acc += P[j] * V[(j0 + j) * D + c];
      o[c] = alpha * o[c] + acc;
    }
    m = mnew;
  }
  if (!any) return 0;
  for (int64_t c = 0; c < D; ++c) o[c] /= l;
  *lse_out = M_LN2 * (m + log2(l / (p_mode == QFA_P_E2M1_BLOCK ? 4.0 : 256.0)));
  return 1;
}

/*
 * Quantised attention for n query rows of one (batch, kv head):
 *   Q  [n][D]   pre-scaled query rows q' = c2 q (decoded MXFP4 of fl32(q c2),
 *               or exact values for the identity path), so q' . k is the
 *               logit in log2 units
 *   Qc [n][D]   bf16 query rows for the compensation term, or NULL
 *   qpos[n]     query index i in [0, Sq)
 *   K, V [L][D] keys and values (decoded), Kbar [ceil(L/128)][D] or NULL
 *   split_tiles 0: one split over all tiles; else tiles per decode split
 *   p_mode      how P is quantised: QFA_P_EXACT (0, identity), QFA_P_E4M3
 *               (1, the method), QFA_P_E4M3_BLOCK (2), QFA_P_E2M1_BLOCK (3);
 *               see tile_p
 *   fp32_arg    1: exponent argument and the exponential of quantised P
 *                  in binary32 (see split_row, tile_p);
 *               0: everything in binary64
 * Outputs O [n][D], lse [n].  Rows with no visible key get O = 0, lse = -inf.
 */
void orc_attn_quant_rows(const double* Q, const double* Qc, const int64_t* qpos, int64_t n, const double* K,
                         const double* Kbar, const double* V, int64_t L, int64_t Sq, int64_t D, int causal,
                         float softmax_scale, int64_t split_tiles, int p_mode, int fp32_arg, double* O,
                         double* lse) {
  int64_t nt = (L + QFA_ORC_TILE - 1) / QFA_ORC_TILE;
  int64_t per = split_tiles > 0 ? split_tiles : (nt > 0 ? nt : 1);
  int64_t nsplit = nt > 0 ? (nt + per - 1) / per : 0;
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * QFA_ORC_TILE);
    double* P = (double*)malloc(sizeof(double) * QFA_ORC_TILE);
    double* os = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
      double* o = O + r * D;
      for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
      /* log-sum-exp merge of the splits, binary64 */
      double big = -INFINITY;
      double* lses = (double*)malloc(sizeof(double) * (nsplit > 0 ? nsplit : 1));
      double* outs = (double*)malloc(sizeof(double) * D * (nsplit > 0 ? nsplit : 1));
      int* ok = (int*)malloc(sizeof(int) * (nsplit > 0 ? nsplit : 1));
      for (int64_t sp = 0; sp < nsplit; ++sp) {
        int64_t t0 = sp * per, t1 = t0 + per < nt ? t0 + per : nt;
        ok[sp] = split_row(Q + r * D, Qc ? Qc + r * D : NULL, qpos[r], K, Kbar, V, L, Sq, D, causal,
                           softmax_scale, t0, t1, p_mode, fp32_arg, os, &lses[sp], S, P);
        if (ok[sp]) {
          memcpy(outs + sp * D, os, sizeof(double) * D);
          if (lses[sp] > big) big = lses[sp];
        }
      }
      if (big == -INFINITY) {
        lse[r] = -INFINITY;
      } else {
        double den = 0.0;
        for (int64_t sp = 0; sp < nsplit; ++sp)
          if (ok[sp]) den += exp(lses[sp] - big);
        double tot = big + log(den);
        for (int64_t sp = 0; sp < nsplit; ++sp) {
          if (!ok[sp]) continue;
          double w = exp(lses[sp] - tot);
          for (int64_t c = 0; c < D; ++c) o[c] += w * outs[sp * D + c];
        }
        lse[r] = tot;
      }
      free(lses);
      free(outs);
      free(ok);
    }
    free(S);
    free(P);
    free(os);
  }
}

/* Array helpers for tests (vectorised codec access). */
void orc_e4m3_encode_array(const double* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e4m3_encode(x[i]);
}
void orc_e2m1_encode_array(const double* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_encode(x[i]);
}
void orc_bf16_from_double_array(const double* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_double(x[i]);
}
int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
