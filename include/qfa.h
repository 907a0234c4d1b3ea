/*
 * qfa.h -- C ABI of the QK4PV8 mixed-precision attention forward library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method ("MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels
 * on Blackwell GPUs", abstract): Q and K are quantised on the fly to 4-bit
 * floating point with per-block shared scales, S = Q K^T / sqrt(d) runs on the
 * 4-bit operands, softmax is computed online (running max, running sum, output
 * rescale) without writing S or P to memory, P and V are quantised to FP8 E4M3
 * and O = P V accumulates in FP32; an optional rank-one smoothing compensation
 * adds one extra matrix-multiply term; prefill and split-KV decode are covered
 * with an adaptive parallel partition.
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are DEVICE pointers to contiguous, 16-byte aligned
 *    buffers owned by the caller.  The library never allocates, frees or
 *    retains device memory; buffers must stay alive until `stream` has
 *    finished the enqueued work.
 *  - Every call validates its arguments on the host, synchronously.  On any
 *    error nothing is launched and no output is written.  On success the work
 *    is enqueued on `stream` (NULL = the legacy default stream) and the call
 *    returns without synchronising.  Launch failures are reported as
 *    QFA_ERR_HIP.
 *  - Stateless and thread-safe; no C++ exception crosses the ABI.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - MX block size: 32 (`block_size` must be 32).  Head dimension D: 64 or
 *    128 for attention; any multiple of 32 up to 256 for the quantisers.
 *  - E8M0 scale codes: value 2^(code - 127); 0xFF marks a block that held a
 *    NaN or an infinity (its element codes are 0).  Inputs are expected finite.
 *
 * Formats (the MXFP4 block of 32 elements with one E8M0 power-of-two scale and
 * the E2M1 element values 0, 1/2, 1, 3/2, 2, 3, 4, 6 follow the FP4 tutorial
 * "FlashAttention压到4位", section "FP4 只有约 15 个可表示的数"; the block
 * quantiser -- amax, power-of-two scale, divide, round to nearest even, store
 * codes and scales in separate pools -- follows the hnwysp.cn MXAttention /
 * MXFP4 notes, sections 2.3, 5.2 and 5.4):
 *  - Q/K codes  [B][H][S][D/2]   E2M1, element 2k in bits 3:0, 2k+1 in bits 7:4
 *  - Q/K scales [B][H][S][D/32]  E8M0, one per 32 consecutive channels,
 *                                exponent ceil(log2 amax) - 2 (clamped to
 *                                [-127, 127]; amax = 0 gives code 0)
 *  - Kbar       [B][Hkv][ceil(S/128)][D] bf16: channel mean of K over each
 *                                128-token block (present tokens only)
 *  - V codes    [B][Hkv][ceil(S/32)][D][32] E4M3 (OCP, bias 7, max 448):
 *                                the 32 tokens of one MX block of one channel
 *                                are contiguous; absent tokens of a ragged
 *                                last block hold code 0
 *  - V scales   [B][Hkv][ceil(S/32)][D] E8M0, exponent ceil(log2 amax) - 8
 *  - O          [B][Hq][S_q][D] float32,  LSE [B][Hq][S_q] float32 (natural log)
 */
#ifndef QFA_H
#define QFA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qfa_status {
  QFA_OK = 0,
  QFA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, Hq % Hkv != 0 */
  QFA_ERR_UNSUPPORTED = 2, /* D or block_size outside what the kernels support */
  QFA_ERR_WORKSPACE = 3,   /* decode workspace missing or too small */
  QFA_ERR_HIP = 4          /* kernel launch failed (hipGetLastError) */
} qfa_status;

/*
 * The factor Q is multiplied by before it is quantised:
 * c2 = fl32(softmax_scale * fl32(log2 e)).  S = Q K^T / sqrt(d) is
 * exponentiated in base 2, and with c2 applied to Q the product Q'K^T is the
 * exponent argument in log2 units (the pages do not say where the scale
 * enters).  Host arithmetic only.
 */
float qfa_exp2_scale(float softmax_scale);

/*
 * Online Q or K quantisation to MXFP4 (MpFA abstract: "online quantization";
 * block quantiser of the MXFP4 notes, sections 2.3 and 5.2).
 *   x         bf16 [B][H][S][D]
 *   smooth    0: quantise x.  1 (K only): also write kbar and quantise the
 *             smoothed tensor fl32(x - Kbar_block) -- the K side of the rank-one
 *             smoothing compensation.  kbar must be NULL iff smooth == 0.
 *   prescale  each element is multiplied by it in binary32 before quantisation:
 *             qfa_exp2_scale(softmax_scale) for Q, 1 for K.  Must be finite and > 0.
 *   codes     out [B][H][S][D/2], scales out [B][H][S][D/32], kbar out as above.
 * Deterministic: codes, scales and kbar are bit-exact functions of x.
 */
qfa_status qfa_quantize_qk4(const uint16_t* x, int B, int H, int S, int D, int block_size, int smooth,
                            float prescale, uint8_t* codes, uint8_t* scales, uint16_t* kbar, hipStream_t stream);

/*
 * V quantisation to FP8 E4M3 with one E8M0 scale per (32 consecutive tokens,
 * channel) -- the contraction axis of P V (MpFA abstract: FP8 for PV).
 *   v      bf16 [B][H][S][D]
 *   codes  out [B][H][ceil(S/32)][D][32], scales out [B][H][ceil(S/32)][D].
 */
qfa_status qfa_quantize_v8(const uint16_t* v, int B, int H, int S, int D, int block_size, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream);

/*
 * V quantisation to MXFP4 for the QFA_PV_FP4 contrast case (below): the Q/K
 * block rule (E2M1 elements, E8M0 scale 2^(ceil(log2 amax) - 2)) applied to
 * each (32 consecutive tokens, channel) block, token 2k in the low nibble of
 * byte k; tokens past S count as 0.  FP4 tutorial, section "Direct-P" (P and
 * V in MXFP4, one E8M0 scale per 32).
 *   v      bf16 [B][H][S][D]
 *   codes  out [B][H][ceil(S/32)][D][16], scales out [B][H][ceil(S/32)][D].
 */
qfa_status qfa_quantize_v4(const uint16_t* v, int B, int H, int S, int D, int block_size, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream);

/*
 * Prefill forward (MpFA abstract; online softmax per the FP4 tutorial's
 * section "注意力慢在哪儿").  Q must be quantised with prescale
 * qfa_exp2_scale(softmax_scale), so s_j = q4 . k4_j is the logit of key j in
 * log2 units.  For each query row i of head h (kv head h / (Hq/Hkv)) the
 * 128-token key tiles are visited in ascending order:
 *   y_j  = fl32(s_j + fl32(c2 * delta))   (delta = q_bf16 . Kbar_tile, only
 *                                          when kbar != NULL)
 *   m'   = max(m, ceil(max_j y_j))        (an integer bound on the row max)
 *   P8_j = E4M3(256 * 2^(y_j - m'))
 *   l    = 2^(m - m') l + sum_j P8_j;  O = 2^(m - m') O + sum_j P8_j V8_j
 * and O / l, LSE = ln(l / 256) + m ln 2 are written.  Because m is an integer
 * the rescale factors are exact powers of two, and E4M3 rounding commutes
 * with them, so without the compensation the P codes do not depend on how
 * the key range is cut into tiles or splits.  delta is the exactly rounded
 * binary32 value of the bf16 dot product.  S and P never reach memory.
 * Causal masks are bottom-right aligned: key j is visible to query i iff
 * j <= i + (S_kv - S_q); a row with no visible key gets O = 0, LSE = -inf.
 *   q4, q4s      MXFP4 Q [B][Hq][S_q][D/2], [B][Hq][S_q][D/32] -- or both NULL:
 *                the kernel then quantises q_bf16 itself (each row read once,
 *                times qfa_exp2_scale(softmax_scale), the MXFP4 block rule),
 *                producing the same codes as qfa_quantize_qk4 and so the same
 *                O and LSE, without the separate pass over Q (the "online
 *                quantization" of the MpFA abstract, fused)
 *   k4, k4s      MXFP4 K [B][Hkv][S_kv][D/2], [..][D/32] (smoothed if kbar)
 *   kbar         NULL (no compensation) or bf16 [B][Hkv][ceil(S_kv/128)][D]
 *   q_bf16       bf16 Q [B][Hq][S_q][D]; required when kbar is set or q4 is
 *                NULL, ignored otherwise
 *   v8, v8s      E4M3 V and its scales (layout above)
 *   O            out float32 [B][Hq][S_q][D];  lse out float32 [B][Hq][S_q] or NULL
 */
qfa_status qfa_fwd_prefill(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                           const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                           int B, int Hq, int Hkv, int S_q, int S_kv, int D, int causal, float softmax_scale,
                           int block_size, float* O, float* lse, hipStream_t stream);

/*
 * Split-KV decode forward, one query token per sequence (MpFA abstract:
 * adaptive parallel partitioning across prefill and decode).  Sequence b uses
 * its first L_b = kv_lens[b] keys (kv_lens: device int32 [B], or NULL for
 * S_kv_max everywhere; 0 <= L_b <= S_kv_max).  Its ceil(L_b/128) tiles are cut
 * into num_splits contiguous runs of ceil(tiles/num_splits) tiles; each run
 * yields a normalised partial (O_s, LSE_s) in `workspace`, and a second kernel
 * merges them: LSE = log sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s.  Runs
 * with no key get weight 0.  No causal mask.
 *   q4, q4s        MXFP4 Q [B][Hq][1][D/2], [B][Hq][1][D/32], quantised with
 *                  prescale qfa_exp2_scale(softmax_scale) as for prefill, or
 *                  both NULL to have the kernel quantise q_bf16 (as for prefill)
 *   k4, k4s, v8, v8s   the pre-quantised KV cache, S_kv_max tokens per sequence
 *   kbar, q_bf16   as for prefill (q_bf16 [B][Hq][1][D])
 *   num_splits     in/out: 0 lets the library choose (written back); > 0 is used
 *   workspace      device buffer of at least qfa_decode_workspace_bytes(...)
 *   O, lse         out float32 [B][Hq][D], [B][Hq] (lse may be NULL)
 */
qfa_status qfa_fwd_decode(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                          const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                          int B, int Hq, int Hkv, int S_kv_max, const int32_t* kv_lens, int D,
                          float softmax_scale, int block_size, int* num_splits, void* workspace,
                          size_t workspace_bytes, float* O, float* lse, hipStream_t stream);

/*
 * qfa_fwd_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * qfa_fwd_decode (P/V format QFA_PV_FP8).  The split partials go to a
 * library-owned device array of QFA_DECODE_NOALLOC_MAX_BYTES per GPU, created
 * with the library's code object on each device and held until the process
 * ends; the call itself allocates and frees nothing.  Its address is looked
 * up once per device, on the first call made with that device current (the
 * current device must be the one `stream` belongs to).
 *   - A shape whose partials need more than QFA_DECODE_NOALLOC_MAX_BYTES
 *     (qfa_decode_workspace_bytes(B, Hq, D, splits) with the split count
 *     used) is rejected with QFA_ERR_WORKSPACE before anything is launched.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (concurrent streams, or host threads) race and must be
 *     serialised by the caller.  No contents carry over between calls: every
 *     partial is written before it is read.
 */
#define QFA_DECODE_NOALLOC_MAX_BYTES (32u << 20)
qfa_status qfa_fwd_decode_noalloc(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                                  const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8,
                                  const uint8_t* v8s, int B, int Hq, int Hkv, int S_kv_max, const int32_t* kv_lens,
                                  int D, float softmax_scale, int block_size, int* num_splits, float* O, float* lse,
                                  hipStream_t stream);

/*
 * P/V formats.  QFA_PV_FP8 is the method described above.  The other two are
 * contrast cases: the MpFA abstract sets QK4PV8 against fully FP4 attention,
 * and the FP4 tutorial's "Direct-P" section gives P one E8M0 power-of-two
 * scale per 32 probabilities.
 *   QFA_PV_FP8_BLOCKP  P in E4M3 with one E8M0 scale per (row, 32 keys): key
 *                      block b (32 keys from a multiple of 32) of a tile is
 *                      coded as E4M3(256 * 2^(y_j - e_b)) with
 *                      e_b = max(ceil(max_{j in b} y_j), m' - 64), and those
 *                      codes count 2^(e_b - m') in O and l.  V as for QFA_PV_FP8.
 *   QFA_PV_FP4         P in MXFP4, E2M1(4 * 2^(y_j - e_b)) on the same blocks,
 *                      and V in MXFP4 (qfa_quantize_v4); LSE = ln(l / 4) + m ln 2.
 */
typedef enum qfa_pv_format { QFA_PV_FP8 = 0, QFA_PV_FP8_BLOCKP = 1, QFA_PV_FP4 = 2 } qfa_pv_format;

/*
 * qfa_fwd_prefill and qfa_fwd_decode with the P/V format as an argument; the
 * plain entry points are pv_format = QFA_PV_FP8.  For QFA_PV_FP4, v8 and v8s
 * carry the MXFP4 V of qfa_quantize_v4.  An unknown format gives
 * QFA_ERR_INVALID_ARG.  Everything else is as for the plain entry points.
 */
qfa_status qfa_fwd_prefill_ex(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                              const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                              int B, int Hq, int Hkv, int S_q, int S_kv, int D, int causal, float softmax_scale,
                              int block_size, int pv_format, float* O, float* lse, hipStream_t stream);
qfa_status qfa_fwd_decode_ex(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                             const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                             int B, int Hq, int Hkv, int S_kv_max, const int32_t* kv_lens, int D,
                             float softmax_scale, int block_size, int pv_format, int* num_splits, void* workspace,
                             size_t workspace_bytes, float* O, float* lse, hipStream_t stream);

/*
 * KV-cache writer: append n_new tokens to every sequence of a pre-quantised
 * cache (quantise on write: hnwysp.cn MXAttention/MXFP4 notes, sections 3.4
 * and 5.4; the cache feeds qfa_fwd_decode).  Sequence b holds L_b tokens
 * (kv_lens: device int32 [B], or NULL for all 0) and receives tokens
 * [L_b, L_b + n_new), clamped to S_kv_max; the caller advances kv_lens.
 * Afterwards the cache holds, for tokens [0, L_b + n_new), exactly the bytes
 * qfa_quantize_qk4 (K, smoothing as given) and qfa_quantize_v8 would write
 * for the whole sequence: the V block of 32 tokens the append starts in is
 * quantised again (its scale may change), and with smoothing so are all rows
 * of the 128-token tile it starts in (K-bar changes).  Their earlier raw values
 * come from the tails.
 *   k_new, v_new   bf16 [B][Hkv][n_new][D]
 *   k4, k4s, kbar  the K cache [B][Hkv][S_kv_max][D/2], [..][D/32],
 *                  kbar [B][Hkv][ceil(S_kv_max/128)][D] or NULL (no smoothing)
 *   v8, v8s        the V cache [B][Hkv][ceil(S_kv_max/32)][D][32], [..][D]
 *   k_tail, v_tail bf16 [B][Hkv][128][D], caller-owned and kept between calls:
 *                  the raw values of each sequence's last partial 128-token
 *                  tile (rows 0 .. L_b - 128 floor(L_b/128) - 1 are read,
 *                  the new partial tile's rows written).  k_tail is NULL iff
 *                  kbar is NULL.  Start them with the cache: for L_b = 0
 *                  nothing is read.
 * Three kernels on `stream`; calls for the same cache must not overlap.
 */
qfa_status qfa_kv_append(const uint16_t* k_new, const uint16_t* v_new, int B, int Hkv, int n_new, int D,
                         int S_kv_max, int block_size, const int32_t* kv_lens, uint8_t* k4, uint8_t* k4s,
                         uint16_t* kbar, uint8_t* v8, uint8_t* v8s, uint16_t* k_tail, uint16_t* v_tail,
                         hipStream_t stream);

/*
 * NVFP4 contrast case for Q and K (MpFA abstract: NVFP4 for QK; the FP4
 * tutorial's section "FP4 只有约 15 个可表示的数": blocks of 16 values with an
 * E4M3 scale and a per-tensor FP32 scale, about 4.5 bits per value).
 *
 * qfa_quantize_nvfp4: x -> E2M1 codes [B][H][S][D/2] (element 2k in the low
 * nibble of byte k) and E4M3 block scales [B][H][S][D/16].  block_size must
 * be 16.  tensor_scale g must be a positive power of two (else
 * QFA_ERR_INVALID_ARG); the smallest 2^k with amax / (6 * 2^k) <= 448 uses
 * E4M3's whole range.  Per block of 16 values (after smoothing and prescale,
 * as for qfa_quantize_qk4) the scale is the E4M3 code (RNE, saturating at 448)
 * of fl32(fl32(amax / g) / 6) and each value the E2M1 code (RNE, saturating at
 * 6) of fl32(x / (s g)).  A scale of 0 gives zero codes; a block holding a
 * non-finite value gets scale 0x7F (E4M3 NaN) and zero codes.
 *
 * qfa_fwd_prefill_nvfp4 / qfa_fwd_decode_nvfp4: qfa_fwd_prefill / qfa_fwd_decode
 * with Q and K in NVFP4 (q4 and q4s required, from qfa_quantize_nvfp4 with
 * prescale qfa_exp2_scale(softmax_scale) and tensor scale q_tensor_scale; K
 * with k_tensor_scale) and P and V as in the method.  S is computed exactly
 * from the decoded values (each lane decodes to bf16 and S runs on the bf16
 * MFMA): an emulation of NVFP4 numerics on gfx950, slower than the MXFP4 path.
 */
qfa_status qfa_quantize_nvfp4(const uint16_t* x, int B, int H, int S, int D, int block_size, int smooth,
                              float prescale, float tensor_scale, uint8_t* codes, uint8_t* scales, uint16_t* kbar,
                              hipStream_t stream);
qfa_status qfa_fwd_prefill_nvfp4(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                                 const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                                 int B, int Hq, int Hkv, int S_q, int S_kv, int D, int causal, float softmax_scale,
                                 float q_tensor_scale, float k_tensor_scale, float* O, float* lse, hipStream_t stream);
qfa_status qfa_fwd_decode_nvfp4(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                                const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                                int B, int Hq, int Hkv, int S_kv_max, const int32_t* kv_lens, int D,
                                float softmax_scale, float q_tensor_scale, float k_tensor_scale, int* num_splits,
                                void* workspace, size_t workspace_bytes, float* O, float* lse, hipStream_t stream);

/*
 * qfa_kv_append for the caches of the contrast formats: pv_format QFA_PV_FP4
 * keeps V in MXFP4 (records and scales as written by qfa_quantize_v4; the
 * other formats keep E4M3 V), and k_tensor_scale > 0 (a power of two) keeps K
 * in NVFP4 with that tensor scale (codes [..][D/2], E4M3 scales [..][D/16], as
 * qfa_quantize_nvfp4 writes them; 0 keeps MXFP4 K).  The contract is the one
 * of qfa_kv_append: afterwards the cache holds the bytes the matching
 * quantisers write for the whole sequence at once.  qfa_kv_append is
 * pv_format = QFA_PV_FP8, k_tensor_scale = 0.
 */
qfa_status qfa_kv_append_ex(const uint16_t* k_new, const uint16_t* v_new, int B, int Hkv, int n_new, int D,
                            int S_kv_max, int block_size, const int32_t* kv_lens, uint8_t* k4, uint8_t* k4s,
                            uint16_t* kbar, uint8_t* v8, uint8_t* v8s, uint16_t* k_tail, uint16_t* v_tail,
                            int pv_format, float k_tensor_scale, hipStream_t stream);

/* Bytes of decode workspace for the given shape and split count (> 0). */
size_t qfa_decode_workspace_bytes(int B, int Hq, int D, int num_splits);

/* The split count the library picks for num_splits == 0 (host arithmetic only):
 * enough (sequence, kv head, split) work units to give every compute unit
 * several, never more splits than tiles. */
int qfa_decode_default_splits(int B, int Hkv, int S_kv_max);

/* Human-readable name of a status code (static storage). */
const char* qfa_status_string(qfa_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int qfa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QFA_H */
