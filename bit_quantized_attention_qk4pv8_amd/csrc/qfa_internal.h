// Internal declarations shared by the HIP translation units of libqfa.
// gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qfa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kTile = 128;   // keys per online-softmax step (the running max is updated per tile)
constexpr int kBlock = 32;   // MX block size
constexpr int kRows = 32;    // query rows per wave (one 32x32 MFMA column block)

// E8M0 code 127 = 1.0
constexpr int kScaleOne = 127;
// Cache-policy operand of a buffer load on gfx950: the non-temporal hint
// (`nt`).  Measured on MI355X: streaming 3.4 GB once through LDS with
// buffer_load ... lds reads at 6.95 TB/s with it against 6.18 without.
constexpr int kCpolNT = 2;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// 2^k for k in [-126, 127] as an exact float.
__device__ __forceinline__ float exp2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// ceil(log2 a) for a finite, positive binary32 value given by its bits.
__device__ __forceinline__ int ceil_log2_f32bits(uint32_t u) {
  uint32_t E = u >> 23, M = u & 0x7FFFFFu;
  if (E == 0) {  // subnormal: a = M * 2^-149
    int c = (M <= 1u) ? 0 : 32 - __clz(M - 1u);
    return c - 149;
  }
  return (int)E - 127 + (M != 0u);
}

// Shared E8M0 exponent of an MX block from its (finite) amax bits:
// ceil(log2 amax) - k clamped to [-127, 127]; amax == 0 -> -127.
__device__ __forceinline__ int mx_block_exponent(uint32_t amax_bits, int k) {
  if (amax_bits == 0u) return -127;
  int e = ceil_log2_f32bits(amax_bits) - k;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// One MXFP4 block: 32 binary32 values -> 16 bytes of E2M1 codes (element 2k
// in the low nibble of byte k, RNE by the hardware converter on the exact
// x * 2^-e) and its E8M0 scale code (e + 127).  A block holding a non-finite
// value gets scale 0xFF and zero codes.  Used by the quantiser kernel and by
// the attention kernels that quantise Q themselves, so both produce the same
// bytes.
__device__ __forceinline__ void mxfp4_block(const float (&v)[kBlock], uint4& codes, uint8_t& scale) {
  uint32_t amax = 0u, nonfinite = 0u;
#pragma unroll
  for (int i = 0; i < kBlock; ++i) {
    const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;
    nonfinite |= (a >= 0x7F800000u);
    amax = a > amax ? a : amax;
  }
  codes = make_uint4(0u, 0u, 0u, 0u);
  scale = 0xFF;
  if (nonfinite) return;
  const int e = mx_block_exponent(amax, 2);
  const float inv = exp2i(-e);  // e in [-127, 126] for finite binary32 input
  uint32_t wd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t r = 0u;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[q * 8 + 0] * inv, v[q * 8 + 1] * inv, 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[q * 8 + 2] * inv, v[q * 8 + 3] * inv, 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[q * 8 + 4] * inv, v[q * 8 + 5] * inv, 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[q * 8 + 6] * inv, v[q * 8 + 7] * inv, 1.0f, 3);
    wd[q] = r;
  }
  codes = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  scale = (uint8_t)(e + 127);
}

// E4M3 byte `sel` (0..3, a constant after unrolling) of w as binary32 (exact).
__device__ __forceinline__ float e4m3_byte_to_f32(int w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(w, 3);
  }
}

// One NVFP4 block: 16 binary32 values -> 8 bytes of E2M1 codes (element 2k in
// the low nibble of byte k) and the E4M3 scale code, with the per-tensor scale
// g (a power of two).  The scale is the E4M3 code (RNE, saturating at 448) of
// fl32(fl32(amax / g) / 6), each element the E2M1 code (RNE, saturating at 6)
// of fl32(x / (s g)): both divisions are IEEE binary32 ones (correctly
// rounded), so the decisions are those of the binary32 definition.  A zero
// scale gives zero codes; a non-finite block gets scale 0x7F and zero codes.
// Used by the NVFP4 quantiser; the attention kernels only decode.
__device__ __forceinline__ void nvfp4_block(const float (&v)[16], float g, uint2& codes, uint8_t& scale) {
  uint32_t amax = 0u, nonfinite = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;
    nonfinite |= (a >= 0x7F800000u);
    amax = a > amax ? a : amax;
  }
  codes = make_uint2(0u, 0u);
  scale = 0x7F;
  if (nonfinite) return;
  const float q = __builtin_fminf((__uint_as_float(amax) / g) / 6.0f, 448.0f);
  const int sc = __builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xFF;
  scale = (uint8_t)sc;
  const float t = __builtin_amdgcn_cvt_f32_fp8(sc, 0) * g;
  if (t == 0.0f) return;
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float q8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q8[j] = __builtin_fminf(__builtin_fmaxf(v[8 * h + j] / t, -6.0f), 6.0f);
    uint32_t r = 0u;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q8[0], q8[1], 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q8[2], q8[3], 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q8[4], q8[5], 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q8[6], q8[7], 1.0f, 3);
    w[h] = r;
  }
  codes = make_uint2(w[0], w[1]);
}

// 32 consecutive bf16 values (64 bytes, 16-byte aligned) -> binary32.
__device__ __forceinline__ void load_bf16_block(const uint16_t* src, float (&v)[kBlock]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = reinterpret_cast<const uint4*>(src)[q];
    const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[q * 8 + 2 * k] = bf16_bits_to_float(wds[k] & 0xFFFFu);
      v[q * 8 + 2 * k + 1] = bf16_bits_to_float(wds[k] >> 16);
    }
  }
}

// MFMA wrappers (gfx950 block-scaled f8f6f4).  Format codes: 0 = FP8 E4M3, 4 = FP4 E2M1.
// 32x32x64: lane l supplies row (l % 32) and K-block (l / 32); the scale byte
// (bits 7:0 of the scale operand) applies to that lane's 32-element K-block.
__device__ __forceinline__ v16f mfma_fp4_32x32x64(v4i a, v4i b, v16f c, int sa, int sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}
// E2M1 x E2M1 with the scale byte SEL (0..3) of sa and sb selected by the
// instruction's byte select.
template <int SEL>
__device__ __forceinline__ v16f mfma_fp4_32x32x64_sel(v4i a, v4i b, v16f c, int sa, int sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, SEL, sa, SEL, sb);
}
__device__ __forceinline__ v16f mfma_fp8_32x32x64(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
// 16x16x128, E2M1 A (four VGPRs) x E4M3 B, unit scales.  Lane l supplies row
// (or column) l % 16.  For E4M3 operands lane group g = l / 16 holds
// contraction indices 16g + (0..15) in bytes 0..15 and 64 + 16g + (0..15) in
// bytes 16..31, and the scale of each 32-index block is taken from one lane
// group, so a block mixes bytes of two lane groups; E2M1 operands hold
// indices 32g + (0..31) in nibble order (both measured on MI355X).
__device__ __forceinline__ v4f mfma_fp4_fp8_16x16x128(v4i a, v8i b, v4f c) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, 4, 0, 0, kScaleOne, 0, kScaleOne);
}

// ---------------------------------------------------------------- launchers (host side)
hipError_t launch_quant_qk4(const uint16_t* x, int B, int H, int S, int D, int smooth, float prescale,
                            uint8_t* codes, uint8_t* scales, uint16_t* kbar, hipStream_t s);
hipError_t launch_quant_v8(const uint16_t* v, int B, int H, int S, int D, uint8_t* codes, uint8_t* scales,
                           hipStream_t s);
hipError_t launch_quant_nvfp4(const uint16_t* x, int B, int H, int S, int D, int smooth, float prescale, float g,
                              uint8_t* codes, uint8_t* scales, uint16_t* kbar, hipStream_t s);
hipError_t launch_quant_v4(const uint16_t* v, int B, int H, int S, int D, uint8_t* codes, uint8_t* scales,
                           hipStream_t s);

// Kernel formats (the attention kernels' template argument; see attn_common.h):
// the method, two P/V contrast formats, and NVFP4 Q/K with the method's P/V.
constexpr int PV_FP8 = 0, PV_FP8_BLOCKP = 1, PV_FP4 = 2, QK_NVFP4 = 3;

struct AttnArgs {
  const uint8_t* q4;
  const uint8_t* q4s;
  const uint8_t* k4;
  const uint8_t* k4s;
  const uint8_t* v8;
  const uint8_t* v8s;
  const uint16_t* kbar;   // may be null
  const uint16_t* qbf;    // bf16 Q: for the compensation and, when q4 is null, quantised in the kernel
  const int32_t* kv_lens; // decode only, may be null
  float* O;               // prefill: final O; decode: partial O workspace
  float* lse;             // prefill: final LSE (may be null); decode: partial LSE workspace
  int B, Hq, Hkv, Sq, Skv, D, G;
  int causal;
  float c2;               // softmax_scale * log2(e), rounded to binary32
  int num_splits;         // decode
  int pv;                 // kernel format (PV_FP8, PV_FP8_BLOCKP, PV_FP4, QK_NVFP4)
  float nv_gq, nv_gk;     // QK_NVFP4: the tensor scales of Q and K (powers of two)
};

hipError_t launch_prefill(const AttnArgs& a, hipStream_t s);

struct AppendArgs {
  const uint16_t* k_new;   // bf16 [B][Hkv][n][D]
  const uint16_t* v_new;
  const int32_t* kv_lens;  // device int32 [B] (tokens already cached) or null (all 0)
  uint8_t* k4;             // cache, S tokens per (b, kv head)
  uint8_t* k4s;
  uint16_t* kbar;          // null: no smoothing
  uint8_t* v8;
  uint8_t* v8s;
  uint16_t* k_tail;        // bf16 [B][Hkv][128][D]; null iff kbar null
  uint16_t* v_tail;        // bf16 [B][Hkv][128][D]
  int B, Hkv, n, S;
  int v_fp4;               // V records in MXFP4 (16 bytes) instead of E4M3 (32 bytes)
  float k_nv_g;            // > 0: K in NVFP4 with this tensor scale; 0: K in MXFP4
};
hipError_t launch_kv_append(const AppendArgs& a, int D, hipStream_t s);
hipError_t launch_decode(const AttnArgs& a, float* O, float* lse, hipStream_t s);

}  // namespace qfa
