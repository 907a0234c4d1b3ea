// QK4PV8 attention forward for gfx950: prefill, split-KV decode, LSE merge.
//
// Method ("MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on
// Blackwell GPUs", abstract): S = Q K^T / sqrt(d) on 4-bit block-scaled
// operands, online softmax with a running max / running sum / output rescale
// (FP4 tutorial "FlashAttention压到4位", section "注意力慢在哪儿"), P quantised
// to FP8 E4M3 after the softmax, O = P V on FP8 operands with FP32
// accumulation, the denominator summed from the same rounded P codes that
// feed P V (same tutorial, section "Direct-P"), and the rank-one smoothing
// compensation added as one extra matrix product.
//
// Mapping onto CDNA4:
//  * One wave owns 32 query rows.  S is produced transposed, S^T = K Q^T, on
//    v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands and the E8M0 block
//    scales fed straight into the instruction.  Lane l then holds 64 scores of
//    query row l % 32, so the row max is 63 in-lane maxima and one lane swap.
//  * K rows are fed to the MFMA in a permuted token order chosen so that the
//    S accumulator registers, converted to FP8, are already the B operand of
//    the P V MFMA (O^T = V^T P^T), and so that every 32-token K-group of that
//    operand is exactly one 32-token E8M0 block of V.  No S or P value leaves
//    the register file.
//  * The softmax denominator is a P V product against a row of ones, so it is
//    the exact sum of the decoded P codes and costs MFMA time, not VALU time.
//  * A workgroup holds all query heads of one KV head (GQA packing) for one
//    32-row query block, so each 128-token K/V tile is loaded into LDS once
//    and read by every head.  Tiles are double-buffered in LDS and fed by
//    global_load_lds_dwordx4 (no VGPR staging).
//  * Rank-one compensation: delta(row, tile) = q_bf16 . Kbar_tile is computed
//    for 32 tiles at a time with v_mfma_f32_32x32x16_bf16 (Kbar Q^T), kept in
//    LDS, and folded into the per-row exponent offset (no per-score work).
//  * Workgroups are ordered longest-causal-range first and KV-head groups are
//    pinned to XCDs (workgroup i runs on XCD i % 8) so a KV head's K/V stays
//    in one XCD's L2.
#include "qfa_internal.h"

namespace qfa {

// A zero page: the source of out-of-range chunks of a ragged last tile.
static __device__ __attribute__((aligned(16))) uint8_t g_zero_page[16];

template <int D>
struct TileLayout {
  static constexpr int KC = kTile * D / 2;   // K codes  [128][D/2]
  static constexpr int KS = kTile * D / 32;  // K scales [128][D/32]
  static constexpr int VC = kTile * D;       // V codes  [4][D][32]
  static constexpr int VS = (kTile / 32) * D;  // V scales [4][D]
  static constexpr int BYTES = KC + KS + VC + VS;
  static constexpr int CHUNKS = BYTES / 16;
  // LDS stride of one tile buffer: whole 1 KB DMA instructions (64 lanes x 16 B),
  // so the tail lanes of the last instruction land in padding.
  static constexpr int STRIDE = (BYTES + 1023) / 1024 * 1024;
};

// Token of MFMA row rho inside a 32-token block: lane group g = (rho/4)%2 of
// the S^T output then holds tokens 16g .. 16g+15 in register order.
__device__ __forceinline__ int perm_token(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Issue the loads of one K/V tile into an LDS buffer.  Full tiles go through
// the LDS-DMA path; a ragged last tile (fewer than 128 tokens) is copied with
// ordinary loads and zero-filled.
__device__ __forceinline__ bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Issue the loads of one K/V tile into an LDS buffer.  Full tiles whose four
// source ranges are 16-byte aligned go through the LDS-DMA path
// (global_load_lds_dwordx4, 1 KB per wave instruction); otherwise (a ragged
// last tile, or unaligned scale arrays) the tile is copied with ordinary loads,
// byte-wise where a chunk is unaligned or partial, and zero-filled past the
// valid bytes.  Every read stays inside the caller's buffers.
template <int D>
__device__ __forceinline__ void load_tile(uint8_t* lbuf, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                                          const uint8_t* vs, int n_tok, int n_vblk, int nwaves) {
  using TL = TileLayout<D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (n_tok == kTile && aligned16(kc) && aligned16(ks) && aligned16(vc) && aligned16(vs)) {
    for (int ins = wave; ins * 64 < TL::CHUNKS; ins += nwaves) {
      const int off = (ins * 64 + lane) * 16;  // byte offset inside the tile buffer
      const uint8_t* src;
      if (off < TL::KC) src = kc + off;
      else if (off < TL::KC + TL::KS) src = ks + (off - TL::KC);
      else if (off < TL::KC + TL::KS + TL::VC) src = vc + (off - TL::KC - TL::KS);
      else src = vs + (off - TL::KC - TL::KS - TL::VC);
      if (off >= TL::BYTES) src = g_zero_page;  // tail lanes of the last instruction (padding)
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lbuf + ins * 1024), 16, 0, 0);
    }
  } else {
    const int kc_valid = n_tok * (D / 2), ks_valid = n_tok * (D / 32);
    const int vc_valid = n_vblk * D * 32, vs_valid = n_vblk * D;
    for (int ch = threadIdx.x; ch < TL::CHUNKS; ch += nwaves * 64) {
      const int off = ch * 16;
      const uint8_t* base;
      int rel, valid;
      if (off < TL::KC) { base = kc; rel = off; valid = kc_valid; }
      else if (off < TL::KC + TL::KS) { base = ks; rel = off - TL::KC; valid = ks_valid; }
      else if (off < TL::KC + TL::KS + TL::VC) { base = vc; rel = off - TL::KC - TL::KS; valid = vc_valid; }
      else { base = vs; rel = off - TL::KC - TL::KS - TL::VC; valid = vs_valid; }
      uint4 v = {0u, 0u, 0u, 0u};
      if (rel + 16 <= valid && aligned16(base + rel)) {
        v = *reinterpret_cast<const uint4*>(base + rel);
      } else if (rel < valid) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (rel + i < valid) w[i >> 2] |= (uint32_t)base[rel + i] << (8 * (i & 3));
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
      *reinterpret_cast<uint4*>(lbuf + off) = v;
    }
  }
}

// Per-wave state of 32 query rows.
template <int D>
struct RowState {
  v4i qa[D / 64];  // Q fragments (B operand of S^T = K Q^T)
  int qs[D / 64];  // their E8M0 scale bytes
  v16f o[D / 32];  // O^T accumulators: o[cb][rr] = channel 32cb + (rr/4)*8 + 4g + rr%4
  v16f lv;         // denominator (every element equals the row sum)
  float m;         // running max in log2 units
};

// One 128-token tile for one wave.  jlim: last visible key index for this
// lane's row (keys > jlim are masked), L: number of keys.
template <int D>
__device__ __forceinline__ void process_tile(RowState<D>& st, const uint8_t* lbuf, int t, bool need_mask, int jlim,
                                             float c2, float delta) {
  using TL = TileLayout<D>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const uint8_t* Kl = lbuf;
  const uint8_t* Ksl = lbuf + TL::KC;
  const uint8_t* Vl = lbuf + TL::KC + TL::KS;
  const uint8_t* Vsl = lbuf + TL::KC + TL::KS + TL::VC;

  // ---- S^T = K Q^T on E2M1 x E2M1 with E8M0 block scales
  v16f s[4];
  const int rho = lane & 31;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int tok = 32 * c + perm_token(rho);
    s[c] = v16f{};
#pragma unroll
    for (int dh = 0; dh < D / 64; ++dh) {
      const v4i ka = *reinterpret_cast<const v4i*>(Kl + tok * (D / 2) + 32 * dh + 16 * g);
      const int sa = Ksl[tok * (D / 32) + 2 * dh + g];
      s[c] = mfma_fp4_32x32x64(ka, st.qa[dh], s[c], sa, st.qs[dh]);
    }
  }

  // ---- mask (diagonal / ragged tiles only); score s[c][rr] is key 128t + 32c + 16g + rr
  if (need_mask) {
    const int jb = kTile * t + 16 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        if (jb + 32 * c + rr > jlim) s[c][rr] = -__builtin_inff();
  }

  // ---- running max (log2 units), rescale factor
  float mx = -__builtin_inff();
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int rr = 0; rr < 16; rr += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[c][rr], s[c][rr + 1]));
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  const float dlt = c2 * delta;
  const float mt = __builtin_fmaf(mx, c2, dlt);
  const float mn = __builtin_fmaxf(st.m, mt);
  const float alpha = (mn == st.m) ? 1.0f : __builtin_amdgcn_exp2f(st.m - mn);
  const float beta = (mn == -__builtin_inff()) ? 0.0f : dlt - mn;
  st.m = mn;

  // ---- P8 = E4M3(256 * 2^(s*c2 + beta)); packed as the B operand of O^T += V^T P^T
  v8i pb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = 2 * h + (k >> 2);
      const int r0 = 4 * (k & 3);
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][r0 + 0], c2, beta));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][r0 + 1], c2, beta));
      const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][r0 + 2], c2, beta));
      const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c][r0 + 3], c2, beta));
      v2s w = {0, 0};
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, p0, p1, 0x1p-8f, false);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, p2, p3, 0x1p-8f, true);
      pb[h][k] = __builtin_bit_cast(int, w);
    }

  // ---- rescale O and l when any row's max moved
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) st.o[cb] *= alpha;
    st.lv *= alpha;
  }

  // ---- O^T += V^T P^T (FP8 x FP8, V's E8M0 scale per 32 tokens x channel), l += 1 . P^T
  const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                    0x38383838, 0x38383838, 0x38383838, 0x38383838};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const int ch = 32 * cb + rho;
      const v4i a0 = *reinterpret_cast<const v4i*>(Vl + ((2 * h) * D + ch) * 32 + 16 * g);
      const v4i a1 = *reinterpret_cast<const v4i*>(Vl + ((2 * h + 1) * D + ch) * 32 + 16 * g);
      const int sa = Vsl[(2 * h + g) * D + ch];
      const v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      st.o[cb] = mfma_fp8_32x32x64(a, pb[h], st.o[cb], sa, kScaleOne);
    }
    st.lv = mfma_fp8_32x32x64(ones, pb[h], st.lv, kScaleOne, kScaleOne);
  }
}

// delta^T for 32 tiles starting at tau0: Kbar[tau0 .. tau0+31] . Q_bf16^T, into
// the wave's LDS slab dl[tile][row].
template <int D>
__device__ __forceinline__ void compute_delta(float* dl, const uint16_t* kbar_bg, int ntk, int tau0,
                                              const uint16_t* qrow, bool qvalid) {
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int tau = tau0 + n;
  v16f acc = v16f{};
#pragma unroll
  for (int step = 0; step < D / 16; ++step) {
    const int c0 = 16 * step + 8 * g;
    uint4 ua = {0u, 0u, 0u, 0u}, ub = {0u, 0u, 0u, 0u};
    if (tau < ntk) ua = *reinterpret_cast<const uint4*>(kbar_bg + (size_t)tau * D + c0);
    if (qvalid) ub = *reinterpret_cast<const uint4*>(qrow + c0);
    bf16x8 a, b;
    __builtin_memcpy(&a, &ua, 16);
    __builtin_memcpy(&b, &ub, 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) dl[((rr >> 2) * 8 + 4 * g + (rr & 3)) * 32 + n] = acc[rr];
}

template <int D>
__device__ __forceinline__ void load_q(RowState<D>& st, const uint8_t* q4row, const uint8_t* q4srow, bool valid) {
  const int g = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int dh = 0; dh < D / 64; ++dh) {
    st.qa[dh] = valid ? *reinterpret_cast<const v4i*>(q4row + 32 * dh + 16 * g) : v4i{0, 0, 0, 0};
    st.qs[dh] = valid ? (int)q4srow[2 * dh + g] : 0;
  }
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) st.o[cb] = v16f{};
  st.lv = v16f{};
  st.m = -__builtin_inff();
}

// Workgroup = (batch b, kv head g, head chunk hc, 32-row query block qb);
// wave w = query head g*G + hc*hpw + w.
template <int D, bool COMP>
__global__ void __launch_bounds__(512) k_prefill(AttnArgs a, int hpw, int nhc, int nq) {
  using TL = TileLayout<D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int g_lane = lane >> 5, n = lane & 31;

  // ---- workgroup -> (group, query block): longest first, groups pinned to XCDs
  const int ngroups = a.B * a.Hkv * nhc;
  int grp, qrank;
  const int x = blockIdx.x;
  if ((ngroups & 7) == 0) {
    const int xcd = x & 7, slot = x >> 3, gpx = ngroups >> 3;
    qrank = slot / gpx;
    grp = xcd + 8 * (slot % gpx);
  } else {
    qrank = x / ngroups;
    grp = x % ngroups;
  }
  const int qb = a.causal ? (nq - 1 - qrank) : qrank;
  const int hc = grp % nhc;
  const int bg = grp / nhc;  // b * Hkv + g
  const int b = bg / a.Hkv, gk = bg % a.Hkv;
  const int h = gk * a.G + hc * hpw + wave;
  const bool wave_active = (hc * hpw + wave) < a.G;

  const int Sq = a.Sq, L = a.Skv;
  const int off = L - Sq;
  const int i0 = qb * kRows;
  const int ntk = (L + kTile - 1) / kTile;
  const int nvb = (L + 31) / 32;
  const int imax = min(i0 + kRows - 1, Sq - 1);
  int t_end = ntk;
  if (a.causal) {
    const int jl = imax + off;
    t_end = (jl < 0) ? 0 : min(ntk, jl / kTile + 1);
  }

  // ---- per-wave row state
  RowState<D> st;
  const int i = i0 + n;
  const bool rvalid = wave_active && i < Sq;
  const size_t qrow = ((size_t)b * a.Hq + h) * Sq + i;
  load_q<D>(st, a.q4 + qrow * (D / 2), a.q4s + qrow * (D / 32), rvalid);
  const int jlim = a.causal ? min(i + off, L - 1) : (L - 1);
  const int jmin_row0 = a.causal ? (i0 + off) : (L - 1);  // smallest limit over the block's rows

  uint8_t* bufs = smem;
  float* dl = reinterpret_cast<float*>(smem + 2 * TL::STRIDE) + wave * 32 * 32;

  const size_t kbase = (size_t)bg * L;
  const size_t vbase = (size_t)bg * nvb;
  auto issue = [&](int t) {
    const int n_tok = min(kTile, L - t * kTile);
    const int n_vblk = min(4, nvb - 4 * t);
    load_tile<D>(bufs + (t & 1) * TL::STRIDE, a.k4 + (kbase + (size_t)t * kTile) * (D / 2),
                 a.k4s + (kbase + (size_t)t * kTile) * (D / 32), a.v8 + (vbase + (size_t)4 * t) * D * 32,
                 a.v8s + (vbase + (size_t)4 * t) * D, n_tok, n_vblk, nwaves);
  };

  if (t_end > 0) issue(0);
  wait_vmem_all();
  __syncthreads();
  for (int t = 0; t < t_end; ++t) {
    if (t + 1 < t_end) issue(t + 1);
    if (wave_active) {
      float delta = 0.0f;
      if (COMP) {
        if ((t & 31) == 0)
          compute_delta<D>(dl, a.kbar + (size_t)bg * ntk * D, ntk, t, a.qbf + qrow * D, rvalid);
        delta = dl[(t & 31) * 32 + n];
      }
      const bool need_mask = (kTile * t + kTile - 1 > jmin_row0) || (kTile * t + kTile > L);
      process_tile<D>(st, bufs + (t & 1) * TL::STRIDE, t, need_mask, jlim, a.c2, delta);
    }
    wait_vmem_all();
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2(l / 256))
  if (!rvalid) return;
  const float l = st.lv[0];
  const bool empty = (st.m == -__builtin_inff());
  const float inv = empty ? 0.0f : 1.0f / l;
  float* orow = a.O + qrow * D;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) orow[32 * cb + (rr >> 2) * 8 + 4 * g_lane + (rr & 3)] = st.o[cb][rr] * inv;
  if (a.lse && g_lane == 0)
    a.lse[qrow] = empty ? -__builtin_inff() : 0.69314718055994531f * (st.m + __builtin_log2f(l * 0x1p-8f));
}

// Decode: workgroup = one wave = (b, kv head g, row chunk rc, split s); lane row n
// = query head g*G + 32*rc + n.  Writes normalised partials to the workspace.
template <int D, bool COMP>
__global__ void __launch_bounds__(64) k_decode_split(AttnArgs a, int nrc) {
  using TL = TileLayout<D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int g_lane = lane >> 5, n = lane & 31;
  const int S = a.num_splits;
  // blockIdx.x = ((bg * nrc) + rc) * S + s; (bg, rc) groups of consecutive splits land on different XCDs
  const int x = blockIdx.x;
  const int s = x % S;
  const int rc = (x / S) % nrc;
  const int bg = x / (S * nrc);
  const int b = bg / a.Hkv, gk = bg % a.Hkv;
  const int hrow = 32 * rc + n;
  const bool rvalid = hrow < a.G;
  const int h = gk * a.G + hrow;

  const int Lmax = a.Skv;
  const int L = a.kv_lens ? min(max(a.kv_lens[b], 0), Lmax) : Lmax;
  const int ntk = (L + kTile - 1) / kTile;
  const int per = (ntk + S - 1) / S;
  const int t0 = s * per, t1 = min(ntk, t0 + per);
  const int ntk_max = (Lmax + kTile - 1) / kTile;
  const int nvb_max = (Lmax + 31) / 32;
  const int nvb = (L + 31) / 32;

  RowState<D> st;
  const size_t qrow = (size_t)b * a.Hq + (rvalid ? h : 0);
  load_q<D>(st, a.q4 + qrow * (D / 2), a.q4s + qrow * (D / 32), rvalid);

  uint8_t* bufs = smem;
  float* dl = reinterpret_cast<float*>(smem + 2 * TL::STRIDE);
  const size_t kbase = (size_t)bg * Lmax;
  const size_t vbase = (size_t)bg * nvb_max;
  auto issue = [&](int t) {
    const int n_tok = min(kTile, L - t * kTile);
    const int n_vblk = min(4, nvb - 4 * t);
    load_tile<D>(bufs + (t & 1) * TL::STRIDE, a.k4 + (kbase + (size_t)t * kTile) * (D / 2),
                 a.k4s + (kbase + (size_t)t * kTile) * (D / 32), a.v8 + (vbase + (size_t)4 * t) * D * 32,
                 a.v8s + (vbase + (size_t)4 * t) * D, n_tok, n_vblk, 1);
  };
  if (t0 < t1) issue(t0);
  wait_vmem_all();
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    if (t + 1 < t1) issue(t + 1);
    float delta = 0.0f;
    if (COMP) {
      if (t == t0 || (t & 31) == 0)
        compute_delta<D>(dl, a.kbar + (size_t)bg * ntk_max * D, ntk, t & ~31, a.qbf + qrow * D, rvalid);
      delta = dl[(t & 31) * 32 + n];
    }
    process_tile<D>(st, bufs + (t & 1) * TL::STRIDE, t, kTile * t + kTile > L, L - 1, a.c2, delta);
    wait_vmem_all();
    __syncthreads();
  }
  if (!rvalid) return;
  const size_t prow = ((size_t)b * a.Hq + h) * S + s;
  const float l = st.lv[0];
  const bool empty = (st.m == -__builtin_inff());
  const float inv = empty ? 0.0f : 1.0f / l;
  float* orow = a.O + prow * D;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) orow[32 * cb + (rr >> 2) * 8 + 4 * g_lane + (rr & 3)] = st.o[cb][rr] * inv;
  if (g_lane == 0) a.lse[prow] = empty ? -__builtin_inff() : 0.69314718055994531f * (st.m + __builtin_log2f(l * 0x1p-8f));
}

// LSE merge: one wave per (b, h) row.  LSE = log sum_s e^{LSE_s};  O = sum_s e^{LSE_s - LSE} O_s.
template <int D>
__global__ void __launch_bounds__(256) k_decode_merge(const float* __restrict__ Op, const float* __restrict__ Lp,
                                                      int rows, int S, float* __restrict__ O, float* __restrict__ lse) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* lp = Lp + (size_t)row * S;
  float mx = -__builtin_inff();
  for (int s = 0; s < S; ++s) mx = __builtin_fmaxf(mx, lp[s]);
  float acc[D / 64];
#pragma unroll
  for (int k = 0; k < D / 64; ++k) acc[k] = 0.0f;
  float den = 0.0f;
  if (mx != -__builtin_inff()) {
    for (int s = 0; s < S; ++s) {
      const float w = __expf(lp[s] - mx);
      den += w;
      const float* op = Op + ((size_t)row * S + s) * D;
#pragma unroll
      for (int k = 0; k < D / 64; ++k) acc[k] += w * op[64 * k + lane];
    }
  }
  const float inv = (den > 0.0f) ? 1.0f / den : 0.0f;
#pragma unroll
  for (int k = 0; k < D / 64; ++k) O[(size_t)row * D + 64 * k + lane] = acc[k] * inv;
  if (lse && lane == 0) lse[row] = (den > 0.0f) ? mx + __logf(den) : -__builtin_inff();
}

template <int D>
static hipError_t prefill_d(const AttnArgs& a, hipStream_t s) {
  using TL = TileLayout<D>;
  const int hpw = a.G < 8 ? a.G : 8;
  const int nhc = (a.G + hpw - 1) / hpw;
  const int nq = (a.Sq + kRows - 1) / kRows;
  const long long nwg = (long long)a.B * a.Hkv * nhc * nq;
  if (nwg == 0) return hipSuccess;
  const bool comp = a.kbar != nullptr;
  const size_t lds = 2 * TL::STRIDE + (comp ? (size_t)hpw * 32 * 32 * 4 : 0);
  if (comp)
    hipLaunchKernelGGL((k_prefill<D, true>), dim3((unsigned)nwg), dim3(64 * hpw), lds, s, a, hpw, nhc, nq);
  else
    hipLaunchKernelGGL((k_prefill<D, false>), dim3((unsigned)nwg), dim3(64 * hpw), lds, s, a, hpw, nhc, nq);
  return hipGetLastError();
}

hipError_t launch_prefill(const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) return prefill_d<64>(a, s);
  if (a.D == 128) return prefill_d<128>(a, s);
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t decode_d(const AttnArgs& a, float* O, float* lse, hipStream_t s) {
  using TL = TileLayout<D>;
  const int nrc = (a.G + 31) / 32;
  const long long nwg = (long long)a.B * a.Hkv * nrc * a.num_splits;
  if (nwg == 0) return hipSuccess;
  const bool comp = a.kbar != nullptr;
  const size_t lds = 2 * TL::STRIDE + (comp ? 32 * 32 * 4 : 0);
  if (comp)
    hipLaunchKernelGGL((k_decode_split<D, true>), dim3((unsigned)nwg), dim3(64), lds, s, a, nrc);
  else
    hipLaunchKernelGGL((k_decode_split<D, false>), dim3((unsigned)nwg), dim3(64), lds, s, a, nrc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = a.B * a.Hq;
  hipLaunchKernelGGL(k_decode_merge<D>, dim3((rows + 3) / 4), dim3(256), 0, s, a.O, a.lse, rows, a.num_splits, O,
                     lse);
  return hipGetLastError();
}

hipError_t launch_decode(const AttnArgs& a, float* O, float* lse, hipStream_t s) {
  if (a.D == 64) return decode_d<64>(a, O, lse, s);
  if (a.D == 128) return decode_d<128>(a, O, lse, s);
  return hipErrorInvalidValue;
}

}  // namespace qfa
