// Online block quantisers (HBM-bound, one read of bf16 and one write of codes).
//
//  * Q/K -> MXFP4: E2M1 elements, one E8M0 scale per 32 consecutive channels,
//    exponent ceil(log2 amax) - 2 ("MpFA: Hardware-Efficient Train-Free QK4V8
//    FlashAttention Kernels on Blackwell GPUs", abstract: online quantisation of
//    Q and K to 4 bits with block scales; block recipe per the hnwysp.cn
//    MXAttention/MXFP4 notes, sections 2.3 and 5.2: amax -> power-of-two scale ->
//    divide -> round to nearest even).
//  * Q is multiplied by c2 = fl32(softmax_scale * log2 e) in binary32 first
//    (prescale), so that Q'K^T is the softmax exponent in log2 units.
//  * K smoothing for the rank-one compensation: per 128-token block channel
//    means, the binary64 sum in token order (exact unless the values span more
//    than 2^38 in magnitude), divided by the number of present tokens and
//    rounded to bf16; the quantised tensor is fl32(K - Kbar).
//  * V -> E4M3 with one E8M0 scale per 32 consecutive tokens of one channel
//    (exponent ceil(log2 amax) - 8), stored block-contiguous [.., S/32, D, 32].
//
// The element conversions use gfx950's RNE converters on the exactly
// pre-scaled value x * 2^-e (a power-of-two multiply, exact).
#include "qfa_internal.h"

namespace qfa {

// binary64 -> bf16 bits, round to nearest even (correct for every finite value).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  double a = fabs(d);
  if (a != a) return 0x7FC0u;
  if (a == 0.0) return sign;
  if (a < 1.1754943508222875e-38) {  // below 2^-126: bf16 subnormal, units of 2^-133
    double n = rint(a * 0x1p133);
    return sign | (uint16_t)n;
  }
  uint64_t ua = u & 0x7FFFFFFFFFFFFFFFull;
  uint64_t r = ua + 0xFFFFFFFFFFFull + ((ua >> 45) & 1ull);  // drop 45 bits (52 - 7): bias 2^44 - 1 + lsb
  int ex = (int)(r >> 52) - 1023 + 127;
  uint32_t man = (uint32_t)(r >> 45) & 0x7Fu;
  if (ex >= 255) return sign | 0x7F80u;
  return sign | (uint16_t)((ex << 7) | man);
}

// K-bar of one 128-token tile: for each channel c, bf16_RNE(s_c / n) with
// s_c = sum_j x[j][c] over the tile's n present rows, accumulated in binary64
// in row order.  Run by the workgroup's 256 threads: with RG = 256 / (D/8)
// row groups, thread t < RG * D/8 reads the 16-byte chunk t % (D/8) (8
// channels) of rows t / (D/8), + RG, ... (coalesced, all loads in flight
// together) and keeps 8 partial sums, which meet in red (LDS, RG * D <= 2048
// doubles).  A different order of the additions
// gives the same s_c whenever every partial sum is exact: a bf16 value with
// exponent field E >= 1 is an integer multiple of 2^(E-134) below 2^(E-126)
// (subnormals: multiples of 2^-133), so a sum of at most 128 of them whose
// nonzero exponent fields lie within E_min..E_max is an integer multiple of
// 2^(max(E_min,1)-134) below 2^(E_max-119), exact in binary64 while
// E_max - max(E_min,1) <= 38.  The tile-wide exponent range is tracked on the
// way; a tile outside it (or holding an infinity or a NaN) is summed again in
// row order by thread c.  Writes kb[c] (binary32) and kbar_out[c] (bf16 bits);
// ends with the workgroup synchronised.  row(j) gives row j's first element.
template <int D, class Row>
__device__ __forceinline__ void tile_kbar(const Row& row, int n, float* kb, uint16_t* kbar_out, double* red,
                                          uint32_t* erange) {
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int RG = 256 / CH;                // row groups (threads from RG * CH on only reduce)
  constexpr int PER = (kTile + RG - 1) / RG;  // rows per thread
  static_assert(D % 8 == 0 && CH <= 256 && RG * D <= 2048, "row groups");
  const int t = threadIdx.x, ch = t % CH, rg = t / CH;
  const bool act = rg < RG;
  uint4 u[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = rg + i * RG;
    u[i] = (act && j < n) ? *reinterpret_cast<const uint4*>(row(j) + 8 * ch) : uint4{0u, 0u, 0u, 0u};
  }
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  uint32_t amax = 0u, amin = 0x7FFFu;  // largest / smallest nonzero magnitude bits
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t wds[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t h = (k & 1) ? (wds[k >> 1] >> 16) : (wds[k >> 1] & 0xFFFFu);
      const uint32_t m = h & 0x7FFFu;
      amax = max(amax, m);
      amin = min(amin, m ? m : 0x7FFFu);
      acc[k] += (double)bf16_bits_to_float(h);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, o));
    amin = min(amin, (uint32_t)__shfl_xor((int)amin, o));
  }
  if ((t & 63) == 0) {
    erange[2 * (t >> 6)] = amax;
    erange[2 * (t >> 6) + 1] = amin;
  }
  if (act) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rg * D + 8 * ch + i] = acc[i];
  }
  __syncthreads();
  if (t < D) {
    uint32_t mx = 0u, mn = 0x7FFFu;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mx = max(mx, erange[2 * w]);
      mn = min(mn, erange[2 * w + 1]);
    }
    const int emax = (int)(mx >> 7), emin = max((int)(mn >> 7), 1);
    double sum = 0.0;
    if (emax - emin <= 38) {
      for (int r = 0; r < RG; ++r) sum += red[r * D + t];
    } else {
      for (int j = 0; j < n; ++j) sum += (double)bf16_bits_to_float(row(j)[t]);
    }
    const uint16_t b = f64_to_bf16_rne(sum / (double)n);
    kb[t] = bf16_bits_to_float(b);
    kbar_out[t] = b;
  }
  __syncthreads();
}

template <int D>
__global__ void __launch_bounds__(256) k_quant_qk4(const uint16_t* __restrict__ x, int S, int ntiles, int smooth,
                                                   float prescale, uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales, uint16_t* __restrict__ kbar) {
  constexpr int NB = D / kBlock;
  __shared__ float kb[D];
  const int tile = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int t0 = tile * kTile;
  const int n = min(kTile, S - t0);
  const uint16_t* xs = x + (bh * (size_t)S + t0) * D;
  if (smooth) {
    __shared__ double red[256 * 8];
    __shared__ uint32_t erange[8];
    tile_kbar<D>([&](int j) { return xs + (size_t)j * D; }, n, kb, kbar + (bh * ntiles + tile) * D, red, erange);
  }
  for (int w = threadIdx.x; w < n * NB; w += blockDim.x) {
    const int j = w / NB, blk = w % NB;
    float v[kBlock];
    load_bf16_block(xs + (size_t)j * D + blk * kBlock, v);
    if (smooth) {
#pragma unroll
      for (int i = 0; i < kBlock; ++i) v[i] = v[i] - kb[blk * kBlock + i];
    }
    if (prescale != 1.0f) {  // Q: fl32(q * c2)
#pragma unroll
      for (int i = 0; i < kBlock; ++i) v[i] = v[i] * prescale;
    }
    const size_t row = bh * (size_t)S + t0 + j;
    uint4 out;
    uint8_t sc;
    mxfp4_block(v, out, sc);
    *reinterpret_cast<uint4*>(codes + row * (D / 2) + blk * (kBlock / 2)) = out;
    scales[row * NB + blk] = sc;
  }
}

// Q/K -> NVFP4 (the QK format of the NVFP4 contrast case): as k_quant_qk4 with
// blocks of 16 channels, E4M3 block scales and the per-tensor scale g.
template <int D>
__global__ void __launch_bounds__(256) k_quant_nvfp4(const uint16_t* __restrict__ x, int S, int ntiles, int smooth,
                                                     float prescale, float g, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, uint16_t* __restrict__ kbar) {
  constexpr int NB = D / 16;
  __shared__ float kb[D];
  const int tile = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int t0 = tile * kTile;
  const int n = min(kTile, S - t0);
  const uint16_t* xs = x + (bh * (size_t)S + t0) * D;
  if (smooth) {
    __shared__ double red[256 * 8];
    __shared__ uint32_t erange[8];
    tile_kbar<D>([&](int j) { return xs + (size_t)j * D; }, n, kb, kbar + (bh * ntiles + tile) * D, red, erange);
  }
  for (int w = threadIdx.x; w < n * NB; w += blockDim.x) {
    const int j = w / NB, blk = w % NB;
    float v[16];
    const uint16_t* src = xs + (size_t)j * D + blk * 16;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 u = reinterpret_cast<const uint4*>(src)[q];
      const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[q * 8 + 2 * k] = bf16_bits_to_float(wds[k] & 0xFFFFu);
        v[q * 8 + 2 * k + 1] = bf16_bits_to_float(wds[k] >> 16);
      }
    }
    if (smooth) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = v[i] - kb[blk * 16 + i];
    }
    if (prescale != 1.0f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = v[i] * prescale;
    }
    const size_t row = bh * (size_t)S + t0 + j;
    uint2 out;
    uint8_t sc;
    nvfp4_block(v, g, out, sc);
    *reinterpret_cast<uint2*>(codes + row * (D / 2) + blk * 8) = out;
    scales[row * NB + blk] = sc;
  }
}

// One V record: the 32 token values of one channel (missing tokens 0) -> 32
// E4M3 codes, RNE by the hardware converter on the exact x * 2^-e, and the
// E8M0 code of e = ceil(log2 amax) - 8; a non-finite record gets scale 0xFF
// and zero codes.  Shared by the V quantiser and the cache writer.
__device__ __forceinline__ void fp8_block_store(const float (&x)[kBlock], uint8_t* dst, uint8_t* scale) {
  uint32_t amax = 0u, nonfinite = 0u;
#pragma unroll
  for (int t = 0; t < kBlock; ++t) {
    const uint32_t a = __float_as_uint(x[t]) & 0x7FFFFFFFu;
    nonfinite |= (a >= 0x7F800000u);
    amax = a > amax ? a : amax;
  }
  uint32_t wd[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  uint8_t sc = 0xFF;
  if (!nonfinite) {
    const int e = mx_block_exponent(amax, 8);
    const float inv = exp2i(-e);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      int r = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q] * inv, x[4 * q + 1] * inv, 0, false);
      r = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q + 2] * inv, x[4 * q + 3] * inv, r, true);
      wd[q] = (uint32_t)r;
    }
    sc = (uint8_t)(e + 127);
  }
  reinterpret_cast<uint4*>(dst)[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  reinterpret_cast<uint4*>(dst)[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
  *scale = sc;
}

// One workgroup per (b, h, 32-token block); thread c handles channel c.
template <int D>
__global__ void __launch_bounds__(D) k_quant_v8(const uint16_t* __restrict__ v, int S, int nblk,
                                                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ uint16_t tile[kBlock * D];
  const int blk = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int j0 = blk * kBlock;
  const int n = min(kBlock, S - j0);
  const uint16_t* src = v + (bh * (size_t)S + j0) * D;
  // stage the block (n * D bf16, a multiple of 16 bytes) through LDS with 16-byte loads
  const int chunks = n * D / 8;
  for (int i = threadIdx.x; i < chunks; i += D)
    reinterpret_cast<uint4*>(tile)[i] = reinterpret_cast<const uint4*>(src)[i];
  __syncthreads();
  const int c = threadIdx.x;
  float x[kBlock];
#pragma unroll
  for (int t = 0; t < kBlock; ++t) x[t] = (t < n) ? bf16_bits_to_float(tile[t * D + c]) : 0.0f;
  fp8_block_store(x, codes + ((bh * nblk + blk) * D + c) * kBlock, scales + (bh * nblk + blk) * D + c);
}

// V -> MXFP4 along tokens (the full-FP4 contrast case): one workgroup per
// 32-token block stages it through LDS as for E4M3; thread c quantises channel
// c's 32 tokens with the Q/K block rule (tokens past S count as 0).
template <int D>
__global__ void __launch_bounds__(D) k_quant_v4(const uint16_t* __restrict__ v, int S, int nblk,
                                                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ uint16_t tile[kBlock * D];
  const int blk = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int j0 = blk * kBlock;
  const int n = min(kBlock, S - j0);
  const uint16_t* src = v + (bh * (size_t)S + j0) * D;
  const int chunks = n * D / 8;
  for (int i = threadIdx.x; i < chunks; i += D)
    reinterpret_cast<uint4*>(tile)[i] = reinterpret_cast<const uint4*>(src)[i];
  __syncthreads();
  const int c = threadIdx.x;
  float x[kBlock];
#pragma unroll
  for (int t = 0; t < kBlock; ++t) x[t] = (t < n) ? bf16_bits_to_float(tile[t * D + c]) : 0.0f;
  uint4 cd;
  uint8_t sc;
  mxfp4_block(x, cd, sc);
  *reinterpret_cast<uint4*>(codes + ((bh * nblk + blk) * D + c) * (kBlock / 2)) = cd;
  scales[(bh * nblk + blk) * D + c] = sc;
}

// ---------------------------------------------------------------- KV-cache writer
// Appending n tokens to a sequence that holds L: the V records of the 32-token
// blocks from floor(L/32) on and (with smoothing) every K row of the 128-token
// tiles from floor(L/128) on are quantised again from raw bf16 values, which
// for tokens below L come from the tail (the raw values of the sequence's
// current partial 128-token tile), so the cache ends up with the bytes the
// quantisers would write for the whole sequence at once.  Quantise-on-write:
// hnwysp.cn MXAttention/MXFP4 notes, sections 3.4 and 5.4.

// Valid range of sequence bg's append: tokens [L, L2), clamped to the cache.
__device__ __forceinline__ void append_range(const AppendArgs& a, size_t bg, int& L, int& L2) {
  const int b = (int)(bg / a.Hkv);
  int l = a.kv_lens ? a.kv_lens[b] : 0;
  l = min(max(l, 0), a.S);
  L = l;
  L2 = min(l + a.n, a.S);
}

// Raw bf16 row of token tau: the tail (base 128 floor(L/128)) below L, the new tokens from L.
template <int D>
__device__ __forceinline__ const uint16_t* tok_row(const uint16_t* tail, const uint16_t* nw, size_t bg, int n, int L,
                                                   int tau) {
  if (tau < L) return tail + (bg * kTile + (tau - (L / kTile) * kTile)) * D;
  return nw + (bg * (size_t)n + (tau - L)) * D;
}

// One workgroup per (affected 32-token V block, sequence slice); thread c = channel c.
template <int D>
__global__ void __launch_bounds__(D) k_append_v(AppendArgs a) {
  const size_t bg = blockIdx.y;
  int L, L2;
  append_range(a, bg, L, L2);
  const int blk = L / kBlock + (int)blockIdx.x;
  const int j0 = blk * kBlock;
  if (j0 >= L2) return;
  const int np = min(kBlock, L2 - j0);
  const int c = threadIdx.x;
  float x[kBlock];
#pragma unroll
  for (int t = 0; t < kBlock; ++t)
    x[t] = (t < np) ? bf16_bits_to_float(tok_row<D>(a.v_tail, a.v_new, bg, a.n, L, j0 + t)[c]) : 0.0f;
  const size_t nvb = (size_t)(a.S + kBlock - 1) / kBlock;
  if (a.v_fp4) {  // MXFP4 record of the full-FP4 cache
    uint4 cd;
    uint8_t sc;
    mxfp4_block(x, cd, sc);
    *reinterpret_cast<uint4*>(a.v8 + ((bg * nvb + blk) * D + c) * (kBlock / 2)) = cd;
    a.v8s[(bg * nvb + blk) * D + c] = sc;
  } else {
    fp8_block_store(x, a.v8 + ((bg * nvb + blk) * D + c) * kBlock, a.v8s + (bg * nvb + blk) * D + c);
  }
}

// One workgroup per (affected 128-token K tile, sequence slice): K-bar of the
// tile's present tokens (smoothing), then the MXFP4 rows -- all of the tile's
// rows when K-bar changed, else only the new ones.
template <int D>
__global__ void __launch_bounds__(256) k_append_k(AppendArgs a, int smooth) {
  constexpr int NB = D / kBlock;
  __shared__ float kb[D];
  const size_t bg = blockIdx.y;
  int L, L2;
  append_range(a, bg, L, L2);
  const int tile = L / kTile + (int)blockIdx.x;
  const int t0 = tile * kTile;
  if (t0 >= L2) return;
  const int np = min(kTile, L2 - t0);
  const int lo = smooth ? t0 : max(t0, L);
  if (smooth) {
    const size_t ntiles = (size_t)(a.S + kTile - 1) / kTile;
    __shared__ double red[256 * 8];
    __shared__ uint32_t erange[8];
    tile_kbar<D>([&](int j) { return tok_row<D>(a.k_tail, a.k_new, bg, a.n, L, t0 + j); }, np, kb,
                 a.kbar + (bg * ntiles + tile) * D, red, erange);
  }
  const int nrows = t0 + np - lo;
  if (a.k_nv_g > 0.0f) {  // NVFP4 rows (blocks of 16, E4M3 scales)
    constexpr int NB16 = D / 16;
    for (int w = threadIdx.x; w < nrows * NB16; w += blockDim.x) {
      const int j = lo + w / NB16, blk = w % NB16;
      const uint16_t* src = tok_row<D>(a.k_tail, a.k_new, bg, a.n, L, j) + blk * 16;
      float v[16];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 u = reinterpret_cast<const uint4*>(src)[q];
        const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[q * 8 + 2 * k] = bf16_bits_to_float(wds[k] & 0xFFFFu);
          v[q * 8 + 2 * k + 1] = bf16_bits_to_float(wds[k] >> 16);
        }
      }
      if (smooth) {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = v[i] - kb[blk * 16 + i];
      }
      uint2 out;
      uint8_t sc;
      nvfp4_block(v, a.k_nv_g, out, sc);
      const size_t row = bg * (size_t)a.S + j;
      *reinterpret_cast<uint2*>(a.k4 + row * (D / 2) + blk * 8) = out;
      a.k4s[row * NB16 + blk] = sc;
    }
    return;
  }
  for (int w = threadIdx.x; w < nrows * NB; w += blockDim.x) {
    const int j = lo + w / NB, blk = w % NB;
    float v[kBlock];
    load_bf16_block(tok_row<D>(a.k_tail, a.k_new, bg, a.n, L, j) + blk * kBlock, v);
    if (smooth) {
#pragma unroll
      for (int i = 0; i < kBlock; ++i) v[i] = v[i] - kb[blk * kBlock + i];
    }
    uint4 out;
    uint8_t sc;
    mxfp4_block(v, out, sc);
    const size_t row = bg * (size_t)a.S + j;
    *reinterpret_cast<uint4*>(a.k4 + row * (D / 2) + blk * (kBlock / 2)) = out;
    a.k4s[row * NB + blk] = sc;
  }
}

// After the two kernels above: the tail takes the raw values of the new
// partial tile's new tokens (its older tokens, if any, are already in place).
template <int D>
__global__ void __launch_bounds__(256) k_append_tail(AppendArgs a) {
  const size_t bg = blockIdx.x;
  int L, L2;
  append_range(a, bg, L, L2);
  const int base2 = (L2 / kTile) * kTile;
  const int from = max(base2, L);
  constexpr int CH = D / 8;  // 16-byte chunks per row
  for (int w = threadIdx.x; w < (L2 - from) * CH; w += blockDim.x) {
    const int tau = from + w / CH, ch = w % CH;
    const size_t src = (bg * (size_t)a.n + (tau - L)) * D + ch * 8;
    const size_t dst = (bg * kTile + (tau - base2)) * D + ch * 8;
    *reinterpret_cast<uint4*>(a.v_tail + dst) = *reinterpret_cast<const uint4*>(a.v_new + src);
    if (a.k_tail) *reinterpret_cast<uint4*>(a.k_tail + dst) = *reinterpret_cast<const uint4*>(a.k_new + src);
  }
}

template <int D>
static hipError_t append_d(const AppendArgs& a, hipStream_t s) {
  const unsigned nbg = (unsigned)(a.B * a.Hkv);
  const int smooth = a.kbar != nullptr;
  hipLaunchKernelGGL(k_append_v<D>, dim3((unsigned)((a.n + kBlock - 1) / kBlock + 1), nbg), dim3(D), 0, s, a);
  hipLaunchKernelGGL(k_append_k<D>, dim3((unsigned)((a.n + kTile - 1) / kTile + 1), nbg), dim3(256), 0, s, a, smooth);
  hipLaunchKernelGGL(k_append_tail<D>, dim3(nbg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, int D, hipStream_t s) {
  switch (D) {
#define QFA_APPEND_CASE(DD) \
  case DD: return append_d<DD>(a, s);
    QFA_APPEND_CASE(32) QFA_APPEND_CASE(64) QFA_APPEND_CASE(96) QFA_APPEND_CASE(128) QFA_APPEND_CASE(160)
    QFA_APPEND_CASE(192) QFA_APPEND_CASE(224) QFA_APPEND_CASE(256)
#undef QFA_APPEND_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quant_qk4(const uint16_t* x, int B, int H, int S, int D, int smooth, float prescale,
                            uint8_t* codes, uint8_t* scales, uint16_t* kbar, hipStream_t s) {
  const int ntiles = (S + kTile - 1) / kTile;
  dim3 grid(ntiles, B * H);
  switch (D) {
#define QFA_QK4_CASE(DD) \
  case DD: hipLaunchKernelGGL(k_quant_qk4<DD>, grid, dim3(256), 0, s, x, S, ntiles, smooth, prescale, codes, scales, kbar); break;
    QFA_QK4_CASE(32) QFA_QK4_CASE(64) QFA_QK4_CASE(96) QFA_QK4_CASE(128) QFA_QK4_CASE(160) QFA_QK4_CASE(192)
    QFA_QK4_CASE(224) QFA_QK4_CASE(256)
#undef QFA_QK4_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_v8(const uint16_t* v, int B, int H, int S, int D, uint8_t* codes, uint8_t* scales,
                           hipStream_t s) {
  const int nblk = (S + kBlock - 1) / kBlock;
  dim3 grid(nblk, B * H);
  switch (D) {
#define QFA_V8_CASE(DD) \
  case DD: hipLaunchKernelGGL(k_quant_v8<DD>, grid, dim3(DD), 0, s, v, S, nblk, codes, scales); break;
    QFA_V8_CASE(32) QFA_V8_CASE(64) QFA_V8_CASE(96) QFA_V8_CASE(128) QFA_V8_CASE(160) QFA_V8_CASE(192)
    QFA_V8_CASE(224) QFA_V8_CASE(256)
#undef QFA_V8_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const uint16_t* x, int B, int H, int S, int D, int smooth, float prescale, float g,
                              uint8_t* codes, uint8_t* scales, uint16_t* kbar, hipStream_t s) {
  const int ntiles = (S + kTile - 1) / kTile;
  dim3 grid(ntiles, B * H);
  switch (D) {
#define QFA_NV_CASE(DD)                                                                                       \
  case DD:                                                                                                    \
    hipLaunchKernelGGL(k_quant_nvfp4<DD>, grid, dim3(256), 0, s, x, S, ntiles, smooth, prescale, g, codes, scales, \
                       kbar);                                                                                 \
    break;
    QFA_NV_CASE(32) QFA_NV_CASE(64) QFA_NV_CASE(96) QFA_NV_CASE(128) QFA_NV_CASE(160) QFA_NV_CASE(192)
    QFA_NV_CASE(224) QFA_NV_CASE(256)
#undef QFA_NV_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_v4(const uint16_t* v, int B, int H, int S, int D, uint8_t* codes, uint8_t* scales,
                           hipStream_t s) {
  const int nblk = (S + kBlock - 1) / kBlock;
  dim3 grid(nblk, B * H);
  switch (D) {
#define QFA_V4_CASE(DD) \
  case DD: hipLaunchKernelGGL(k_quant_v4<DD>, grid, dim3(DD), 0, s, v, S, nblk, codes, scales); break;
    QFA_V4_CASE(32) QFA_V4_CASE(64) QFA_V4_CASE(96) QFA_V4_CASE(128) QFA_V4_CASE(160) QFA_V4_CASE(192)
    QFA_V4_CASE(224) QFA_V4_CASE(256)
#undef QFA_V4_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qfa
