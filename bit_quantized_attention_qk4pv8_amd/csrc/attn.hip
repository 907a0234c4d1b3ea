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
//  * The running max is kept on the integer grid (log2 units): m only has to
//    bound the row max from above, and an integer m makes each rescale an
//    exact power of two.  P is converted against a per-row frame m_ref, and
//    the factor 2^(m_ref - m) is applied through the E8M0 scale operand of
//    the P V and denominator MFMAs, so O and l are never rescaled by VALU
//    work except when m drifts more than 64 above the frame.
//  * A workgroup holds all query heads of one KV head (GQA packing) for one
//    32-row query block, so each 128-token K/V tile is loaded into LDS once
//    and read by every head.  Tiles are double-buffered in LDS and fed by
//    buffer_load ... lds (no VGPR staging, hardware range checks).
//  * Rank-one compensation: delta(row, tile) = q_bf16 . Kbar_tile is computed
//    for 32 tiles at a time with v_mfma_f64_16x16x4f64 (Kbar Q^T, exact for
//    bf16 operands, then rounded once to binary32), kept in LDS, and folded
//    into the per-row exponent offset (no per-score work).
//  * Workgroups are ordered longest-causal-range first and KV-head groups are
//    pinned to XCDs (workgroup i runs on XCD i % 8) so a KV head's K/V stays
//    in one XCD's L2.
#include "qfa_internal.h"

namespace qfa {

// LDS image of one K/V tile (128 keys):
//   [K codes 128 x D/2][K scales, 1 KB area][V codes 4 x D x 32][V scales, 1 KB area]
// K and V codes are stored with an XOR swizzle of their 16-byte chunks (see
// kswz / vswz) so that the MFMA operand reads are free of bank conflicts.
template <int D>
struct TileLayout {
  static constexpr int KC = kTile * D / 2;
  static constexpr int KS_BYTES = kTile * D / 32;
  static constexpr int VC = kTile * D;
  static constexpr int VS_BYTES = (kTile / 32) * D;
  static constexpr int K_OFF = 0;
  static constexpr int KS_OFF = KC;
  static constexpr int V_OFF = KC + 1024;
  static constexpr int VS_OFF = V_OFF + VC;
  static constexpr int STRIDE = VS_OFF + 1024;
  static constexpr int NK = KC / 1024;  // 1 KB DMA instructions per region
  static constexpr int NV = VC / 1024;
  static constexpr int NKS = D == 128 ? 2 : 1;  // dword DMA instructions (256 B each) for K scales
  static constexpr int NINS = NK + NKS + NV + 1;
};

// Token of MFMA row rho inside a 32-token block: lane group g = (rho/4)%2 of
// the S^T output then holds tokens 16g .. 16g+15 in register order.
__device__ __forceinline__ int perm_token(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

// K row of token tok (D/2 bytes): chunk k is stored at k ^ kswz(tok).
template <int D>
__device__ __forceinline__ int kswz(int tok) {
  if (D == 128) return (((tok >> 1) ^ (tok >> 2)) & 1) | (((tok >> 4) & 1) << 1);
  return ((tok >> 1) ^ (tok >> 2) ^ (tok >> 4)) & 1;
}
// V record (block, channel) = 32 token bytes = 2 chunks: half h stored at h ^ vswz(ch).
__device__ __forceinline__ int vswz(int ch) { return ((ch >> 2) ^ (ch >> 3)) & 1; }

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Streams the K/V tiles of one (batch, kv head) slice into LDS with
// buffer_load ... lds (no VGPR staging).  For each tile a buffer resource per
// region starts at the tile and covers only the slice's remaining valid bytes,
// so the hardware range check (applied to voffset + inst_offset) zero-fills a
// ragged last tile and V blocks past the end, and no read leaves the slice.
// Per-lane offsets (which carry the LDS swizzle) are loop-invariant.
template <int D>
struct TileLoader {
  using TL = TileLayout<D>;
  const uint8_t* kc;  // slice bases
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  uint32_t kc_bytes, ks_bytes, vc_bytes, vs_bytes;  // valid bytes of each slice region
  uint32_t vk0, vk1, vv;
  int L;

  __device__ __forceinline__ void init(const uint8_t* k4, const uint8_t* k4s, const uint8_t* v8, const uint8_t* v8s,
                                       size_t bg, int L_storage, int L_valid) {
    const int nvb_storage = (L_storage + 31) / 32, nvb = (L_valid + 31) / 32;
    L = L_valid;
    kc = k4 + bg * L_storage * (D / 2);
    ks = k4s + bg * L_storage * (D / 32);
    vc = v8 + bg * nvb_storage * D * 32;
    vs = v8s + bg * nvb_storage * D;
    kc_bytes = (uint32_t)L_valid * (D / 2);
    ks_bytes = (uint32_t)L_valid * (D / 32);
    vc_bytes = (uint32_t)nvb * D * 32;
    vs_bytes = (uint32_t)nvb * D;
    const int p = threadIdx.x & 63;
    if (D == 128) {  // 16 tokens of 64 B per KB; kswz uses token bits 1, 2 and 4 (= KB parity)
      const int tl = p >> 2, kpos = p & 3;
      vk0 = tl * 64 + 16 * (kpos ^ kswz<D>(tl));
      vk1 = tl * 64 + 16 * (kpos ^ kswz<D>(tl + 16));
    } else {         // 32 tokens of 32 B per KB
      const int tl = p >> 1, kpos = p & 1;
      vk0 = vk1 = tl * 32 + 16 * (kpos ^ kswz<D>(tl));
    }
    const int rl = p >> 1, hpos = p & 1;  // 32 records of 32 B per KB; vswz uses record bits 2, 3
    vv = rl * 32 + 16 * (hpos ^ vswz(rl));
  }

  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, uint32_t bytes, uint32_t t0) {
    const uint32_t rem = bytes > t0 ? bytes - t0 : 0u;
    // raw buffer (stride 0): voffset + inst_offset >= rem reads as zero
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + t0), (short)0, (int)rem, 0x00020000);
  }

  // Issue tile t into lbuf; the wave issues every nwaves-th 1 KB (or 256 B) instruction.
  __device__ __forceinline__ void issue(int t, uint8_t* lbuf, int wave, int nwaves) const {
    const int lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc, kc_bytes, (uint32_t)t * TL::KC);
    const __amdgpu_buffer_rsrc_t rks = tile_rsrc(ks, ks_bytes, (uint32_t)t * TL::KS_BYTES);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc, vc_bytes, (uint32_t)t * TL::VC);
    const __amdgpu_buffer_rsrc_t rvs = tile_rsrc(vs, vs_bytes, (uint32_t)t * TL::VS_BYTES);
    for (int ins = wave; ins < TL::NINS; ins += nwaves) {
      if (ins < TL::NK) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(lbuf + TL::K_OFF + ins * 1024), 16,
                                                 ((ins & 1) ? vk1 : vk0) + ins * 1024, 0, 0, 0);
      } else if (ins < TL::NK + TL::NKS) {
        const int j = ins - TL::NK;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, (lds_ptr_t)(lbuf + TL::KS_OFF + j * 256), 4, lane * 4 + j * 256, 0,
                                                 0, 0);
      } else if (ins < TL::NK + TL::NKS + TL::NV) {
        const int i = ins - TL::NK - TL::NKS;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(lbuf + TL::V_OFF + i * 1024), 16, vv + i * 1024, 0, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rvs, (lds_ptr_t)(lbuf + TL::VS_OFF), 16, lane * 16, 0, 0, 0);
      }
    }
  }

  // D = 64 with an odd key count: the last token's two scale bytes share a
  // dword with bytes past the end, which the range check zeroes; patch them
  // after the DMA has landed (called between the wait and the barrier).
  __device__ __forceinline__ void fixup(int t, uint8_t* lbuf) const {
    if (D == 64 && (L & 1) && t == (L - 1) / kTile && threadIdx.x == 0) {
      const int j = (L - 1) - t * kTile;
      lbuf[TL::KS_OFF + 2 * j] = ks[2 * (L - 1)];
      lbuf[TL::KS_OFF + 2 * j + 1] = ks[2 * (L - 1) + 1];
    }
  }
};

// Per-wave state of 32 query rows.
template <int D>
struct RowState {
  v4i qa[D / 64];  // Q fragments (B operand of S^T = K Q^T)
  int qs[D / 64];  // their E8M0 scale bytes
  v16f o[D / 32];  // O^T accumulators: o[cb][rr] = channel 32cb + (rr/4)*8 + 4g + rr%4
  v16f lv;         // denominator 1 . P^T (every element equals the row sum), in the m_ref frame
  float m;         // running max in log2 units, on the integer grid (-inf before any key)
  float m_ref;     // frame of o and lv: both hold sum 2^(m_t - m_ref) P_t (V_t | 1)
  v8i ones;        // FP8 1.0 in every byte: the A operand of the denominator product
};

// One 128-token tile for one wave.  jlim: last visible key index for this
// lane's row (keys > jlim are masked), L: number of keys.
template <int D>
__device__ __forceinline__ void process_tile(RowState<D>& st, const uint8_t* lbuf, int t, bool need_mask, int jlim,
                                             float c2, float delta) {
  using TL = TileLayout<D>;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const uint8_t* Kl = lbuf + TL::K_OFF;
  const uint8_t* Ksl = lbuf + TL::KS_OFF;
  const uint8_t* Vl = lbuf + TL::V_OFF;
  const uint8_t* Vsl = lbuf + TL::VS_OFF;

  // ---- S^T = K Q^T on E2M1 x E2M1 with E8M0 block scales
  v16f s[4];
  const int rho = lane & 31;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int tok = 32 * c + perm_token(rho);
    const int sw = kswz<D>(tok);
    // the token's D/32 scale bytes; byte 2*dh + g feeds this lane's K-block
    const uint32_t sc_word = D == 128 ? *reinterpret_cast<const uint32_t*>(Ksl + tok * 4)
                                      : (uint32_t)*reinterpret_cast<const uint16_t*>(Ksl + tok * 2);
    s[c] = v16f{};
#pragma unroll
    for (int dh = 0; dh < D / 64; ++dh) {
      const v4i ka = *reinterpret_cast<const v4i*>(Kl + tok * (D / 2) + 16 * ((2 * dh + g) ^ sw));
      const int sa = (int)(sc_word >> (8 * (2 * dh + g)));
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

  // ---- running max (log2 units), rescale factor.  Two left-associated chains
  // (max(max(m, a), b) compiles to v_max3_f32: one instruction per two scores).
  float mx0 = s[0][0], mx1 = s[2][0];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int rr = (c == 0 ? 1 : 0); rr < 16; rr += 2) {
      if (rr + 1 < 16) {
        mx0 = __builtin_fmaxf(__builtin_fmaxf(mx0, s[c][rr]), s[c][rr + 1]);
        mx1 = __builtin_fmaxf(__builtin_fmaxf(mx1, s[c + 2][rr]), s[c + 2][rr + 1]);
      } else {
        mx0 = __builtin_fmaxf(mx0, s[c][rr]);
        mx1 = __builtin_fmaxf(mx1, s[c + 2][rr]);
      }
    }
  float mx = __builtin_fmaxf(mx0, mx1);
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  // Running max on the integer grid: every rescale factor is an exact power of
  // two, applied below through the E8M0 scale of the P operand (no VALU work).
  const float dlt = c2 * delta;
  const float mt = __builtin_ceilf(__builtin_fmaf(mx, c2, dlt));
  const float mn = __builtin_fmaxf(st.m, mt);
  const float beta = (mn == -__builtin_inff()) ? 0.0f : dlt - mn;
  if (st.m_ref == -__builtin_inff()) st.m_ref = mn;  // first visible key fixes the frame
  st.m = mn;
  // Keep 2^(m - m_ref) inside the E8M0 range: rebase the frame when it grows
  // past 2^64 (rare: the row max would have to climb 64 binades).
  if (__builtin_amdgcn_ballot_w64(mn - st.m_ref > 64.0f)) {
    const float f = (mn - st.m_ref > 64.0f) ? __builtin_ldexpf(1.0f, (int)(st.m_ref - mn)) : 1.0f;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(st.o[cb][rr]) : "v"(f));
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(st.lv[rr]) : "v"(f));
    if (mn - st.m_ref > 64.0f) st.m_ref = mn;
  }
  const int pscale = (mn == -__builtin_inff()) ? kScaleOne : kScaleOne + (int)(mn - st.m_ref);

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
      // the old value of the destination is dead (both halves are written): reuse p0's register
      v2s w = __builtin_bit_cast(v2s, p0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, p0, p1, 0x1p-8f, false);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, p2, p3, 0x1p-8f, true);
      pb[h][k] = __builtin_bit_cast(int, w);
    }

  // ---- O^T += 2^(m - m_ref) V^T P^T (FP8 x FP8; V's E8M0 scale per 32 tokens x
  // channel, P's per row); the denominator is the same product against ones
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const int ch = 32 * cb + rho;
      const int hv = 16 * (g ^ vswz(ch));
      const v4i a0 = *reinterpret_cast<const v4i*>(Vl + ((2 * h) * D + ch) * 32 + hv);
      const v4i a1 = *reinterpret_cast<const v4i*>(Vl + ((2 * h + 1) * D + ch) * 32 + hv);
      const int sa = Vsl[(2 * h + g) * D + ch];
      const v8i a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      st.o[cb] = mfma_fp8_32x32x64(a, pb[h], st.o[cb], sa, pscale);
    }
    st.lv = mfma_fp8_32x32x64(st.ones, pb[h], st.lv, kScaleOne, pscale);
  }
}

// delta^T for 32 tiles starting at tau0: Kbar[tau0 .. tau0+31] . Q_bf16^T,
// into the wave's LDS slab dl[tile][row] as binary32.  The products of two bf16
// values are exact in binary64 and a sum of D of them stays exact there, so the
// FP64 MFMA (v_mfma_f64_16x16x4f64) yields the exactly rounded binary32 value:
// the per-(row, tile) exponent offset, which decides P codes, is then the same
// number the binary64 definition gives.  Four 16x16 blocks (2 tile halves x 2
// row halves); the contraction index of step s, lane group g is channel
// 32 g + s (any pairing works as long as A and B agree).
template <int D>
__device__ __forceinline__ void compute_delta(float* dl, const uint16_t* kbar_bg, int ntk, int tau0,
                                              const uint16_t* qbase, int q_stride, int nrows_valid) {
  typedef double v4d __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  constexpr int CPG = D / 4;  // channels per lane group
  v4d acc[2][2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[tb][rb] = v4d{0.0, 0.0, 0.0, 0.0};
  const int tau_a = tau0 + r16, tau_b = tau0 + 16 + r16;
  const int row_a = r16, row_b = 16 + r16;
#pragma unroll
  for (int s8 = 0; s8 < CPG; s8 += 8) {
    const int c0 = CPG * g + s8;
    uint4 ka = {0u, 0u, 0u, 0u}, kb = {0u, 0u, 0u, 0u}, qa = {0u, 0u, 0u, 0u}, qb = {0u, 0u, 0u, 0u};
    if (tau_a < ntk) ka = *reinterpret_cast<const uint4*>(kbar_bg + (size_t)tau_a * D + c0);
    if (tau_b < ntk) kb = *reinterpret_cast<const uint4*>(kbar_bg + (size_t)tau_b * D + c0);
    if (row_a < nrows_valid) qa = *reinterpret_cast<const uint4*>(qbase + (size_t)row_a * q_stride + c0);
    if (row_b < nrows_valid) qb = *reinterpret_cast<const uint4*>(qbase + (size_t)row_b * q_stride + c0);
    const uint32_t kaw[4] = {ka.x, ka.y, ka.z, ka.w}, kbw[4] = {kb.x, kb.y, kb.z, kb.w};
    const uint32_t qaw[4] = {qa.x, qa.y, qa.z, qa.w}, qbw[4] = {qb.x, qb.y, qb.z, qb.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) ? 16 : 0;
      const double A0 = (double)bf16_bits_to_float((kaw[e >> 1] >> sh) & 0xFFFFu);
      const double A1 = (double)bf16_bits_to_float((kbw[e >> 1] >> sh) & 0xFFFFu);
      const double B0 = (double)bf16_bits_to_float((qaw[e >> 1] >> sh) & 0xFFFFu);
      const double B1 = (double)bf16_bits_to_float((qbw[e >> 1] >> sh) & 0xFFFFu);
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(A0, B0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(A0, B1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(A1, B0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(A1, B1, acc[1][1], 0, 0, 0);
    }
  }
  // FP64 16x16 result layout: register r of lane l holds entry (i, j) = (l / 16 + 4 r, l % 16), i.e.
  // tile 16 tb + lane / 16 + 4 r and query row 16 rb + lane % 16 of block (tb, rb)
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dl[(16 * tb + g + 4 * r) * 32 + 16 * rb + r16] = (float)acc[tb][rb][r];
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
  st.m_ref = -__builtin_inff();
  st.ones = v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838};
  asm volatile("" : "+v"(st.ones));  // resident in VGPRs for the whole loop (no per-tile rebuild)
}

// Workgroup = (batch b, kv head g, head chunk hc, 32-row query block qb);
// wave w = query head g*G + hc*hpw + w.
template <int D, bool COMP>
__global__ void __launch_bounds__(512) k_prefill(AttnArgs a, int hpw, int nhc, int nq) {
  using TL = TileLayout<D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar control flow
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

  // Both tile buffers start zeroed: bytes a ragged tile does not cover then hold
  // zeros or codes of an earlier tile, never uninitialised (possibly NaN) codes.
  for (int o = threadIdx.x * 16; o < 2 * TL::STRIDE; o += blockDim.x * 16)
    *reinterpret_cast<uint4*>(bufs + o) = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  TileLoader<D> ld;
  ld.init(a.k4, a.k4s, a.v8, a.v8s, (size_t)bg, L, L);

  if (t_end > 0) ld.issue(0, bufs, wave, nwaves);
  wait_vmem_all();
  if (t_end > 0) ld.fixup(0, bufs);
  __syncthreads();
  for (int t = 0; t < t_end; ++t) {
    if (t + 1 < t_end) ld.issue(t + 1, bufs + ((t + 1) & 1) * TL::STRIDE, wave, nwaves);
    if (wave_active) {
      float delta = 0.0f;
      if (COMP) {
        if ((t & 31) == 0)
          compute_delta<D>(dl, a.kbar + (size_t)bg * ntk * D, ntk, t, a.qbf + (((size_t)b * a.Hq + h) * Sq + i0) * D,
                           D, wave_active ? Sq - i0 : 0);
        delta = dl[(t & 31) * 32 + n];
      }
      const bool need_mask = (kTile * t + kTile - 1 > jmin_row0) || (kTile * t + kTile > L);
      process_tile<D>(st, bufs + (t & 1) * TL::STRIDE, t, need_mask, jlim, a.c2, delta);
    }
    wait_vmem_all();
    if (t + 1 < t_end) ld.fixup(t + 1, bufs + ((t + 1) & 1) * TL::STRIDE);
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
    a.lse[qrow] = empty ? -__builtin_inff() : 0.69314718055994531f * (st.m_ref + __builtin_log2f(l * 0x1p-8f));
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

  RowState<D> st;
  const size_t qrow = (size_t)b * a.Hq + (rvalid ? h : 0);
  load_q<D>(st, a.q4 + qrow * (D / 2), a.q4s + qrow * (D / 32), rvalid);

  uint8_t* bufs = smem;
  float* dl = reinterpret_cast<float*>(smem + 2 * TL::STRIDE);
  for (int o = threadIdx.x * 16; o < 2 * TL::STRIDE; o += blockDim.x * 16)
    *reinterpret_cast<uint4*>(bufs + o) = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  TileLoader<D> ld;
  ld.init(a.k4, a.k4s, a.v8, a.v8s, (size_t)bg, Lmax, L);
  if (t0 < t1) ld.issue(t0, bufs + (t0 & 1) * TL::STRIDE, 0, 1);
  wait_vmem_all();
  if (t0 < t1) ld.fixup(t0, bufs + (t0 & 1) * TL::STRIDE);
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    if (t + 1 < t1) ld.issue(t + 1, bufs + ((t + 1) & 1) * TL::STRIDE, 0, 1);
    float delta = 0.0f;
    if (COMP) {
      if (t == t0 || (t & 31) == 0)
        compute_delta<D>(dl, a.kbar + (size_t)bg * ntk_max * D, ntk, t & ~31,
                         a.qbf + ((size_t)b * a.Hq + gk * a.G + 32 * rc) * D, D, a.G - 32 * rc);
      delta = dl[(t & 31) * 32 + n];
    }
    process_tile<D>(st, bufs + (t & 1) * TL::STRIDE, t, kTile * t + kTile > L, L - 1, a.c2, delta);
    wait_vmem_all();
    if (t + 1 < t1) ld.fixup(t + 1, bufs + ((t + 1) & 1) * TL::STRIDE);
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
  if (g_lane == 0)
    a.lse[prow] = empty ? -__builtin_inff() : 0.69314718055994531f * (st.m_ref + __builtin_log2f(l * 0x1p-8f));
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
