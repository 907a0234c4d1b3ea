// Test-only HIP library for the GPU-side pins of the QK4PV8 kernels (gfx950).
// Not part of libqfa: it exposes, one at a time, the building blocks whose
// exactness the attention kernels rely on, so the tests can compare them with
// the CPU oracle in isolation.
//
//  - probe_cvt: the hardware conversions the kernels use, applied to an array
//    of binary32 values: v_cvt_scalef32_pk_fp4_f32 (E2M1; the MXFP4 quantiser
//    with scale 1 and the FP4 P of the contrast format with power-of-two
//    scales), v_cvt_scalef32_pk_fp8_f32 (E4M3 P with scale 2^(m - 8)) and
//    v_cvt_pk_fp8_f32 (the V quantiser and the NVFP4 scale code).  E2M1 and
//    E4M3 follow the FP4 tutorial "FlashAttention压到4位", section
//    "FP4 只有约 15 个可表示的数", and the MXFP4 notes (hnwysp.cn), section 5.2
//    (round to nearest even).
//  - probe_s_tile: one 128-key tile of S' = Q'4 K4^T for 32 query rows, through
//    the kernels' own tile DMA, operand reads and block-scaled FP4 MFMAs
//    (attn_common.h), written out as binary32 scores.
//  - probe_s_tile_seeded: the same tile with the S accumulator started at a
//    per-row offset d[row], built by offset_block as the compensated kernels
//    build it.
//  - probe_tile_rowsum: the E4M3-P denominator of two tiles (tile_rowsum on
//    each 64-key half, then fold_rowsum with each tile's P scale code), for
//    P operands given in the 32x32x64 B layout of the P V product.
//  - probe_delta: the rank-one compensation term of 32 tiles x 32 query rows
//    (compute_delta: K-bar . Q_bf16 on the FP64 MFMA), written out as the
//    LDS slab the kernels read, dl[tile][row].
//  - probe_exp2: v_exp_f32 (the kernels' exponential) applied to an array.
//  - probe_lds_fill: fills the LDS of every compute unit with a byte pattern
//    (a regression check that no kernel reads LDS bytes it did not write).
//
// Host functions launch on the null stream and return the hipError_t of the
// launch; the caller synchronises.
#include "../../bit_quantized_attention_qk4pv8_amd/csrc/attn_common.h"

namespace {

using namespace qfa;

// kind 0: E2M1 pairs, one byte per pair (element 2i low nibble, 2i+1 high);
// kind 1: E4M3 with scale, one byte per element; kind 2: E4M3 without scale.
__global__ void k_cvt(int kind, const float* __restrict__ x, long n, float scale, uint8_t* __restrict__ out) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; 4 * i < n; i += stride) {
    const long j = 4 * i;
    const float a = x[j], b = j + 1 < n ? x[j + 1] : 0.0f, c = j + 2 < n ? x[j + 2] : 0.0f,
                d = j + 3 < n ? x[j + 3] : 0.0f;
    if (kind == 0) {
      uint32_t r = 0u;
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, a, b, scale, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c, d, scale, 1);
      out[j / 2] = (uint8_t)(r & 0xFF);
      if (j + 2 < n) out[j / 2 + 1] = (uint8_t)((r >> 8) & 0xFF);
    } else {
      uint32_t r;
      if (kind == 1) {
        v2s w = v2s{0, 0};
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, scale, false);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, scale, true);
        r = __builtin_bit_cast(uint32_t, w);
      } else {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
        r = (uint32_t)w;
      }
      for (int k = 0; k < 4 && j + k < n; ++k) out[j + k] = (uint8_t)(r >> (8 * k));
    }
  }
}

// One wave: query rows 0..31 (codes q4 [32][D/2], scales [32][D/32]) against
// keys [128 t, 128 t + 128) of k4 [L][D/2], k4s [L][D/32].  S[row][key] for
// the keys present (a ragged last tile writes only its L - 128 t keys).
// d: null, or 32 per-row start values of the accumulator.
template <int D>
__global__ void __launch_bounds__(64) k_s_tile(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4,
                                               const uint8_t* k4s, const float* d, int L, int t, float* S) {
  using TL = TileLayout<D, PV_FP8>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  TileLoader<D, 1, PV_FP8> ld;
  ld.init(k4, k4s, k4, k4s, 0, L, L, 0);  // (V regions unused)
  ld.issue_k(t, smem, 0);
  wait_vmem_all();
  ld.fixup(t, smem);
  __syncthreads();
  RowState<D> st;
  load_q<D, PV_FP8>(st, q4 + (size_t)n * (D / 2), q4s + (size_t)n * (D / 32), nullptr, 1.0f, true);
  LaneOffs<D, PV_FP8> lo;
  lo.init();
  v16f s[4];
  v16f init = v16f{};
  if (d) init = offset_block(d[n]);  // as the compensated kernels build it
  qk_tile<D, PV_FP8>(st, lo, smem, s, init);
  const int nk = min(kTile, L - kTile * t);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = score_key<PV_FP8>(c, g, rr);
      if (key < nk) S[n * kTile + key] = s[c][rr];
    }
}

__global__ void k_exp2(const float* __restrict__ x, long n, float* __restrict__ out) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] = __builtin_amdgcn_exp2f(x[i]);
}

__global__ void __launch_bounds__(256) k_lds_fill(uint32_t pattern, int words) {
  extern __shared__ uint32_t lds_words[];
  for (int i = threadIdx.x; i < words; i += blockDim.x) lds_words[i] = pattern;
  __syncthreads();
}

}  // namespace

// pb: per lane 32 dwords (tile t, half h at dwords 16t + 8h .. +7); ps: per
// lane the P scale codes of the two tiles.  ts_out[(t * 64 + lane) * 4 + v]:
// element v of tile t's row sums; lsum_out[lane]: the denominator after both.
__global__ void __launch_bounds__(64) k_tile_rowsum(const int* pb, const int* ps, float* ts_out, float* lsum_out) {
  const int lane = threadIdx.x;
  RowState<64> st;
  load_q<64, PV_FP8>(st, nullptr, nullptr, nullptr, 1.0f, false);
  for (int t = 0; t < 2; ++t) {
    v8i p0, p1;
    for (int r = 0; r < 8; ++r) {
      p0[r] = pb[lane * 32 + 16 * t + r];
      p1[r] = pb[lane * 32 + 16 * t + 8 + r];
    }
    v4f ts = tile_rowsum(st.sel, p0, v4f{});
    ts = tile_rowsum(st.sel, p1, ts);
    fold_rowsum(st, ts, ps[lane * 2 + t]);
    for (int v = 0; v < 4; ++v) ts_out[(t * 64 + lane) * 4 + v] = ts[v];
  }
  lsum_out[lane] = st.lsum;
}

template <int D>
__global__ void __launch_bounds__(64) k_delta(const uint16_t* kbar, int tlim, int tau0, const uint16_t* q,
                                               int q_stride, int nrows, float* out) {
  __shared__ float dl[32 * 32];
  for (int o = threadIdx.x; o < 32 * 32; o += 64) dl[o] = __builtin_nanf("");
  __syncthreads();
  compute_delta<D>(dl, kbar, tlim, tau0, q, q_stride, nrows);
  __syncthreads();
  for (int o = threadIdx.x; o < 32 * 32; o += 64) out[o] = dl[o];
}

extern "C" {

int probe_cvt(int kind, const float* x, long n, float scale, uint8_t* out) {
  if (kind < 0 || kind > 2 || n <= 0) return (int)hipErrorInvalidValue;
  const long threads = (n + 3) / 4;
  const int blocks = (int)((threads + 255) / 256 < 65536 ? (threads + 255) / 256 : 65536);
  hipLaunchKernelGGL(k_cvt, dim3(blocks), dim3(256), 0, 0, kind, x, n, scale, out);
  return (int)hipGetLastError();
}

int probe_s_tile_seeded(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s, const float* d,
                        int D, int L, int t, float* S) {
  if (L <= 0 || t < 0 || kTile * t >= L) return (int)hipErrorInvalidValue;
  if (D == 64) {
    constexpr size_t lds = TileLayout<64, PV_FP8>::KREG;
    hipLaunchKernelGGL(k_s_tile<64>, dim3(1), dim3(64), lds, 0, q4, q4s, k4, k4s, d, L, t, S);
  } else if (D == 128) {
    constexpr size_t lds = TileLayout<128, PV_FP8>::KREG;
    hipLaunchKernelGGL(k_s_tile<128>, dim3(1), dim3(64), lds, 0, q4, q4s, k4, k4s, d, L, t, S);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int probe_s_tile(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s, int D, int L, int t,
                 float* S) {
  return probe_s_tile_seeded(q4, q4s, k4, k4s, nullptr, D, L, t, S);
}

// Every workgroup takes `bytes` of LDS (at most 160 KB) and writes the pattern into all of it.
int probe_tile_rowsum(const int* pb, const int* ps, float* ts_out, float* lsum_out) {
  hipLaunchKernelGGL(k_tile_rowsum, dim3(1), dim3(64), 0, 0, pb, ps, ts_out, lsum_out);
  return (int)hipGetLastError();
}

// kbar: the K-bar rows of one slice (tile-major, D bf16 each; at least one
// row, and every row below tlim); q: the first of 32 query rows, q_stride
// elements apart (rows below nrows are read); out: 32 x 32 floats.
int probe_delta(const uint16_t* kbar, int tlim, int tau0, const uint16_t* q, int q_stride, int nrows, int D,
                float* out) {
  if (D == 64)
    hipLaunchKernelGGL(k_delta<64>, dim3(1), dim3(64), 0, 0, kbar, tlim, tau0, q, q_stride, nrows, out);
  else if (D == 128)
    hipLaunchKernelGGL(k_delta<128>, dim3(1), dim3(64), 0, 0, kbar, tlim, tau0, q, q_stride, nrows, out);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int probe_exp2(const float* x, long n, float* out) {
  if (n <= 0) return (int)hipErrorInvalidValue;
  const int blocks = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  hipLaunchKernelGGL(k_exp2, dim3(blocks), dim3(256), 0, 0, x, n, out);
  return (int)hipGetLastError();
}

int probe_lds_fill(uint32_t pattern, int nwg, int bytes) {
  if (nwg <= 0 || bytes <= 0 || bytes > 160 * 1024 || (bytes & 3)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_lds_fill, dim3(nwg), dim3(256), (size_t)bytes, 0, pattern, bytes / 4);
  return (int)hipGetLastError();
}

}  // extern "C"
