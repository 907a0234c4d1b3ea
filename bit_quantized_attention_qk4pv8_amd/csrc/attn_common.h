// Building blocks shared by the prefill and decode attention kernels (gfx950).
//
// A 128-key tile is processed by one wave for 32 query rows in three steps:
//   S^T = K Q^T   on v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1 x E2M1, E8M0 block
//                 scales fed to the instruction)                 [qk_tile]
//   softmax       mask, running max on the integer grid, P = E4M3(256 * 2^(.))
//                 packed directly as the B operand of the P V product
//                                                                [softmax_tile]
//   P V           O^T += V^T P^T on the FP8 MFMA, with the rescale
//                 2^(m - m_ref) riding on P's E8M0 scale, and the tile's row
//                 sums of P on one 16x16x128 MFMA per 64 keys   [pv_tile]
// pv_then_qk runs the P V of one tile and the S^T of the next back to back.
// Every step is templated on the kernel format: the method (above) or one of
// the contrast formats described at pv_of below.
// Method: "MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on
// Blackwell GPUs" (abstract); online softmax per the FP4 tutorial
// "FlashAttention压到4位", section "注意力慢在哪儿"; the denominator uses the
// rounded P codes (same tutorial, section "Direct-P").
#pragma once

#include <type_traits>

#include "qfa_internal.h"

namespace qfa {

// Kernel formats.  PV_FP8 is the method: P = E4M3(256 * 2^(y - m)) with one
// power-of-two scale per row (the running max m) and V in E4M3.
// PV_FP8_BLOCKP gives P one E8M0 scale per (row, 32 keys): block b is coded
// as E4M3(256 * 2^(y - e_b)) with e_b = max(ceil(max_{j in b} y_j), m - 64)
// and weighted 2^(e_b - m_ref) through the MFMA's scale operand.  PV_FP4
// codes P the same way in E2M1 (E2M1(4 * 2^(y - e_b))) and takes V in MXFP4,
// and both products run on the FP4 MFMA.  ([FA4tut] "Direct-P": one E8M0
// scale per 32 probabilities; [MpFA] abstract: FP8 P/V versus fully FP4
// attention.)
// QK_NVFP4: Q and K in NVFP4 (blocks of 16, E4M3 scales, power-of-two tensor
// scales) with the method's E4M3 P and V.  The K tile keeps the MXFP4 code
// layout (with twice the scale bytes); each lane decodes its codes to bf16
// right before the product, exactly (an E2M1 value times an E4M3 scale times
// a power of two has at most six significant bits), and S runs on the bf16
// MFMA: an emulation of NVFP4 numerics, not a fast path.  ([MpFA] abstract:
// NVFP4 for QK; [FA4tut] "FP4 只有约 15 个可表示的数": blocks of 16 with an
// E4M3 scale and an FP32 tensor scale.)
// The P/V format of a kernel format: QK_NVFP4 keeps the method's.
constexpr int pv_of(int fmt) { return fmt == QK_NVFP4 ? PV_FP8 : fmt; }
// V bytes per (32-token block, channel) record
template <int PV>
constexpr int v_record() { return PV == PV_FP4 ? 16 : 32; }

// LDS image of one K/V tile (128 keys):
//   K region [K codes 128 x D/2][K scales, 1 KB area]
//   V region [V codes 4 x D x VR][V scales, 1 KB area]  (VR = 32 bytes per
//            (32-token block, channel) record in E4M3, 16 in MXFP4)
// The two regions may live in separate buffers (KREG / VREG bytes each).
// K codes and E4M3 V records are stored with an XOR swizzle of their 16-byte
// chunks (see kswz / vswz) so that the MFMA operand reads are free of bank
// conflicts; an MXFP4 V record is one 16-byte chunk and needs none.
template <int D, int PV = PV_FP8>
struct TileLayout {
  static constexpr int KC = kTile * D / 2;
  static constexpr int KSB = PV == QK_NVFP4 ? D / 16 : D / 32;  // K scale bytes per token
  static constexpr int KS_BYTES = kTile * KSB;
  static constexpr int VC = (kTile / 32) * D * v_record<PV>();
  static constexpr int VS_BYTES = (kTile / 32) * D;
  static constexpr int K_OFF = 0;
  static constexpr int KS_OFF = KC;
  static constexpr int V_OFF = KC + 1024;
  static constexpr int VS_OFF = V_OFF + VC;
  static constexpr int STRIDE = VS_OFF + 1024;
  static constexpr int KREG = KC + 1024;  // K region bytes (codes, then scales at KC)
  static constexpr int VREG = VC + 1024;  // V region bytes (codes, then scales at VC)
  static constexpr int NK = KC / 1024;  // 1 KB DMA instructions per region
  static constexpr int NV = VC / 1024;
  static constexpr int NKS = KS_BYTES / 256;  // dword DMA instructions (256 B each) for K scales
  static constexpr int NINS = NK + NKS + NV + 1;
};

// Token of MFMA row rho inside a 32-token block: lane group g = (rho/4)%2 of
// the S^T output then holds tokens 16g .. 16g+15 in register order.
__device__ __forceinline__ int perm_token(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }
// PV_FP4: MFMA c = 2h + w of a tile covers, for lane group g, keys
// 64h + 32g + 16w .. +15, so a lane holds all 32 keys of block 2h + g (the
// FP4 P operand of one lane is one whole 32-key block).  Row rho reads token
// 64h + 16w + perm64(rho).
__device__ __forceinline__ int perm64(int rho) { return 32 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }
// Key (from the tile start) of score s[c][rr] in lane group g.
template <int PV>
__device__ __forceinline__ int score_key(int c, int g, int rr) {
  return PV == PV_FP4 ? 64 * (c >> 1) + 32 * g + 16 * (c & 1) + rr : 32 * c + 16 * g + rr;
}

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

// Streams the K/V tiles of one (batch, kv head) slice into LDS (NW waves
// share the issue) with
// buffer_load ... lds (no VGPR staging).  Each 1 KB (or 256 B) instruction
// gets its own buffer resource, built with scalar arithmetic, that starts at
// the instruction's bytes and covers only the slice's remaining valid bytes:
// the hardware range check (on voffset + inst_offset) zero-fills a ragged last
// tile and V blocks past the end, no read leaves the slice, and the per-lane
// voffsets (which carry the LDS swizzle) stay loop-invariant, so issuing a
// tile costs no VALU work.  CPOL is the loads' cache-policy operand: kCpolNT
// (non-temporal) for a stream whose bytes are read once (the decode), 0 for
// tiles that other workgroups read again through L2 (the prefill).
template <int D, int NW, int PV = PV_FP8, int CPOL = 0>
struct TileLoader {
  using TL = TileLayout<D, PV>;
  static constexpr int VR = v_record<PV>();
  const uint8_t* kc;  // slice bases
  const uint8_t* ks;
  const uint8_t* vc;
  const uint8_t* vs;
  uint32_t kc_bytes, ks_bytes, vc_bytes, vs_bytes;  // valid bytes of each slice region
  uint32_t vk0, vk1, vkw, vv;                        // per-lane voffsets (vkw: K codes, parity of `wave`)
  int L;

  // Point the loader at slice bg (a (batch, kv head) pair) of the K/V tensors.
  __device__ __forceinline__ void slice(const uint8_t* k4, const uint8_t* k4s, const uint8_t* v8, const uint8_t* v8s,
                                        size_t bg, int L_storage, int L_valid) {
    const int nvb_storage = (L_storage + 31) / 32, nvb = (L_valid + 31) / 32;
    L = L_valid;
    kc = k4 + bg * L_storage * (D / 2);
    ks = k4s + bg * L_storage * TL::KSB;
    vc = v8 + bg * nvb_storage * D * VR;
    vs = v8s + bg * nvb_storage * D;
    kc_bytes = (uint32_t)L_valid * (D / 2);
    ks_bytes = (uint32_t)L_valid * TL::KSB;
    vc_bytes = (uint32_t)nvb * D * VR;
    vs_bytes = (uint32_t)nvb * D;
  }

  // wave: index of the issuing wave when several waves split a tile (only its
  // parity matters); 0 when one wave issues everything.
  __device__ __forceinline__ void init(const uint8_t* k4, const uint8_t* k4s, const uint8_t* v8, const uint8_t* v8s,
                                       size_t bg, int L_storage, int L_valid, int wave) {
    slice(k4, k4s, v8, v8s, bg, L_storage, L_valid);
    const int p = threadIdx.x & 63;
    if (D == 128) {  // 16 tokens of 64 B per KB; kswz uses token bits 1, 2 and 4 (= KB parity)
      const int tl = p >> 2, kpos = p & 3;
      vk0 = tl * 64 + 16 * (kpos ^ kswz<D>(tl));
      vk1 = tl * 64 + 16 * (kpos ^ kswz<D>(tl + 16));
    } else {         // 32 tokens of 32 B per KB
      const int tl = p >> 1, kpos = p & 1;
      vk0 = vk1 = tl * 32 + 16 * (kpos ^ kswz<D>(tl));
    }
    vkw = (wave & 1) ? vk1 : vk0;
    if (PV == PV_FP4) {  // 64 records of 16 B per KB, not swizzled
      vv = p * 16;
    } else {             // 32 records of 32 B per KB; vswz uses record bits 2, 3
      const int rl = p >> 1, hpos = p & 1;
      vv = rl * 32 + 16 * (hpos ^ vswz(rl));
    }
  }

  // Resource for the bytes [off, bytes) of a slice region (empty when off >=
  // bytes, whatever off is), so every access it allows lies inside the
  // region.  The saturating subtract is written as two scalar instructions
  // (the borrow of s_sub_u32 selects 0): left to the compiler it becomes a
  // VALU clamp plus a readfirstlane in the middle of the MFMA sequence.
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const uint8_t* base, uint32_t bytes, uint32_t off) {
    uint32_t r;
    asm("s_sub_u32 %0, %1, %2\n\ts_cselect_b32 %0, 0, %0" : "=s"(r) : "s"(bytes), "s"(off) : "scc");
    const int rem = (int)r;
    // raw buffer (stride 0): voffset + inst_offset >= rem reads as zero
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + off), (short)0, rem, 0x00020000);
  }

  // Issue the K region (codes + scales) of tile t into kreg.  NW waves split
  // the instructions: this wave issues indices wave, wave + NW, ...
  __device__ __forceinline__ void issue_k(int t, uint8_t* kreg, int wave) const {
    const int lane = threadIdx.x & 63;
    constexpr int N = TL::NK + TL::NKS;
#pragma unroll
    for (int j = 0; j < (N + NW - 1) / NW; ++j) {
      const int ins = wave + NW * j;
      // (the descriptor is bound to a local: passing the call's result straight
      // to the builtin loses the host launch stub of later kernel instances)
      if (ins < TL::NK) {
        const uint32_t voff = (NW % 2 == 0) ? vkw : ((ins & 1) ? vk1 : vk0);
        const __amdgpu_buffer_rsrc_t r = rsrc_at(kc, kc_bytes, (uint32_t)t * TL::KC + ins * 1024);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(kreg + ins * 1024), 16, voff, 0, 0, CPOL);
      } else if (ins < N) {
        const int i = ins - TL::NK;
        const __amdgpu_buffer_rsrc_t r = rsrc_at(ks, ks_bytes, (uint32_t)t * TL::KS_BYTES + i * 256);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(kreg + TL::KC + i * 256), 4, lane * 4, 0, 0, CPOL);
      }
    }
  }
  // Issue the V region (codes + scales) of tile t into vreg.
  __device__ __forceinline__ void issue_v(int t, uint8_t* vreg, int wave) const {
    const int lane = threadIdx.x & 63;
    constexpr int N = TL::NV + 1;
#pragma unroll
    for (int j = 0; j < (N + NW - 1) / NW; ++j) {
      const int ins = wave + NW * j;
      if (ins < TL::NV) {
        const __amdgpu_buffer_rsrc_t r = rsrc_at(vc, vc_bytes, (uint32_t)t * TL::VC + ins * 1024);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(vreg + ins * 1024), 16, vv, 0, 0, CPOL);
      } else if (ins < N) {
        const __amdgpu_buffer_rsrc_t r = rsrc_at(vs, vs_bytes, (uint32_t)t * TL::VS_BYTES);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(vreg + TL::VC), 16, lane * 16, 0, 0, CPOL);
      }
    }
  }

  // Fixed-shape issue of the code instructions: each of the NW waves makes
  // the same SLOTS instructions per (K, V) tile pair, so they can sit between
  // MFMAs without a branch.  Slot k (a compile-time value after unrolling):
  //   k <  KCS   K codes, instruction wave + NW * k
  //   k >= KCS   V codes, instruction wave + NW * (k - KCS)
  // An instruction past the end of its region, or of a tile that is not
  // wanted (ek / ev false), reads nothing (range 0) and writes its zeros to
  // `trash`, 1 KB of LDS that nothing reads.  The scale instructions are
  // issued by issue_scales.
  static constexpr int KCS = (TL::NK + NW - 1) / NW;
  static constexpr int VCS = (TL::NV + NW - 1) / NW;
  static constexpr int SLOTS = KCS + VCS;
  __device__ __forceinline__ void dma_slot(int k, int tk, uint8_t* kreg, bool ek, int tv, uint8_t* vreg, bool ev,
                                           int wave, uint8_t* trash) const {
    if (k < KCS) {
      const int ins = wave + NW * k;
      const bool e = ek && ins < TL::NK;
      const __amdgpu_buffer_rsrc_t r = rsrc_at(kc, e ? kc_bytes : 0u, (uint32_t)tk * TL::KC + (e ? ins : 0) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(e ? kreg + ins * 1024 : trash), 16, vkw, 0, 0, CPOL);
    } else if (k < SLOTS) {
      const int ins = wave + NW * (k - KCS);
      const bool e = ev && ins < TL::NV;
      const __amdgpu_buffer_rsrc_t r = rsrc_at(vc, e ? vc_bytes : 0u, (uint32_t)tv * TL::VC + (e ? ins : 0) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(e ? vreg + ins * 1024 : trash), 16, vv, 0, 0, CPOL);
    }
  }
  // The scale bytes of a tile pair as dword loads of 256 B, one per wave:
  // waves 0 .. NKS-1 the K-scale blocks, the next NVS waves the V-scale
  // blocks, every other wave (or an unwanted tile) a load of nothing into
  // `trash`.  Branch-free like dma_slot.
  static constexpr int NVS = TL::VS_BYTES / 256;
  __device__ __forceinline__ void scale_slot(int tk, uint8_t* kreg, bool ek, int tv, uint8_t* vreg, bool ev,
                                             int wave, uint8_t* trash) const {
    static_assert(TL::NKS + NVS <= NW, "one scale load per wave");
    const int lane = threadIdx.x & 63;
    const bool isk = wave < TL::NKS, isv = !isk && wave < TL::NKS + NVS;
    const int i = isk ? wave : (isv ? wave - TL::NKS : 0);
    const bool e = (isk && ek) || (isv && ev);
    const uint8_t* base = isk ? ks : vs;
    const uint32_t bytes = e ? (isk ? ks_bytes : vs_bytes) : 0u;
    const uint32_t off = (uint32_t)(isk ? tk * TL::KS_BYTES : tv * TL::VS_BYTES) + i * 256;
    uint8_t* dst = !e ? trash : (isk ? kreg + TL::KC : vreg + TL::VC) + i * 256;
    const __amdgpu_buffer_rsrc_t r = rsrc_at(base, bytes, off);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 4, lane * 4, 0, 0, CPOL);
  }

  // Two scale bytes per token (MXFP4, D = 64) with an odd key count: the last
  // token's scale bytes share a dword with bytes past the end, which the
  // range check zeroes; patch them after the DMA has landed (called between
  // the wait and the barrier).
  __device__ __forceinline__ void fixup(int t, uint8_t* kreg) const {
    if (TL::KSB == 2 && (L & 1) && t == (L - 1) / kTile && (threadIdx.x & 63) == 0) {
      const int j = (L - 1) - t * kTile;
      kreg[TL::KC + 2 * j] = ks[2 * (L - 1)];
      kreg[TL::KC + 2 * j + 1] = ks[2 * (L - 1) + 1];
    }
  }
};

// Channel-block assignment of the QK^T contraction.  MFMA k of a 32-key block
// takes, in lane group g (lanes 32g .. 32g+31), the 32 channels of block
// kblock(g, k): {2g, 2g+1} for D = 128, so a lane's two E8M0 bytes are
// adjacent in a token's scale word (one 16-bit LDS read, picked by the
// MFMA's byte select), and block g for D = 64.  Q uses the same assignment.
template <int D>
__device__ __forceinline__ int kblock(int g, int k) { return D == 128 ? 2 * g + k : g; }

// Per-lane LDS byte offsets of a wave's operand reads, relative to a tile's K
// or V region; the compile-time part of each address goes into the
// instruction's offset field, so a read costs no VALU work.
template <int D, int PV = PV_FP8>
struct LaneOffs {
  // K fragment of MFMA k.  E4M3 P: key block c adds 32c * D/2.  PV_FP4: MFMA
  // c = 2h + w adds (64h + 16w) * D/2 to k1 (w = 1) or k (w = 0): adding 16
  // flips token bit 4, which the K swizzle uses.
  uint32_t k[D / 64];
  uint32_t k1[PV == PV_FP4 ? D / 64 : 1];
  uint32_t ks;  // K scale bytes (KC included); key block c adds 32c * D/32 (PV_FP4: (64h + 16w) * D/32)
  // V fragment.  E4M3: (half h, part w, channel block cb) adds ((2h + w) * D + 32cb) * 32.
  // MXFP4: the lane's whole record of block 2h + g; (h, cb) adds (2h * D + 32cb) * 16.
  uint32_t v;
  uint32_t vs;  // V scale byte (VC included); adds 2h * D + 32cb

  __device__ __forceinline__ void init() {
    using TL = TileLayout<D, PV>;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 5, rho = lane & 31;
    // kswz depends on token bits 1, 2, 4 only: for the E4M3 formats the same for every key block
    const int tok = PV == PV_FP4 ? perm64(rho) : perm_token(rho);
    const int sw = kswz<D>(tok);
#pragma unroll
    for (int k = 0; k < D / 64; ++k) this->k[k] = tok * (D / 2) + 16 * (kblock<D>(g, k) ^ sw);
    if constexpr (PV == PV_FP4) {
      const int sw1 = kswz<D>(tok + 16);
#pragma unroll
      for (int k = 0; k < D / 64; ++k) k1[k] = tok * (D / 2) + 16 * (kblock<D>(g, k) ^ sw1);
    }
    ks = TL::KC + tok * TL::KSB + (D == 128 ? 2 * g : g) * (TL::KSB / (D / 32));
    if (PV == PV_FP4)
      v = (g * D + rho) * 16;
    else
      v = rho * 32 + 16 * (g ^ vswz(rho));  // vswz depends on channel bits 2, 3 only
    vs = TL::VC + g * D + rho;
  }
};

// Per-wave state of 32 query rows.
template <int D>
struct RowState {
  v4i qa[D / 64];  // Q fragments (B operand of S^T = K Q^T), channel blocks kblock(g, k)
  int qs;          // their E8M0 scale bytes: byte k feeds MFMA k
  v16f o[D / 32];  // O^T accumulators: o[cb][rr] = channel 32cb + (rr/4)*8 + 4g + rr%4
  float lsum;      // E4M3 P: the denominator, sum of 2^(m_t - m_ref) times tile t's row sum of P codes
  v4i sel;         // E4M3 P: the E2M1 selector operand of the row sums (see tile_rowsum)
  v16f lv;         // block-scaled P: denominator 1 . P^T (every element equals the row sum)
  float m;         // running max in log2 units, on the integer grid (-inf before any key)
  float m_ref;     // frame of o and the denominator: sum 2^(m_t - m_ref) P_t (V_t | 1)
  v8i ones;        // block-scaled P: 1.0 in every element (E4M3 0x38, or E2M1 0x2 in the first four
                   // dwords), the A operand of the denominator product
  bf16x8 qn[D / 16];  // QK_NVFP4: Q decoded to bf16, 8 channels per bf16 MFMA (see qk_blk)
  float gk;           // QK_NVFP4: K's tensor scale
};

// The P and V operand types of the P V product: 32 E4M3 bytes or 32 E2M1 nibbles per lane.
template <int PV>
using POp = typename std::conditional<pv_of(PV) == PV_FP4, v4i, v8i>::type;

// ---- O^T in fixed accumulation registers (method prefill, no compensation)
// In that kernel O^T lives in AGPRs a0 .. a(D/2 - 1), block cb in
// a[16 cb .. 16 cb + 15], and only inline assembly touches it: the P V MFMAs
// accumulate there, the rare frame rebase and the epilogue go through
// v_accvgpr_read/write.  (The MFMA builtins pick one register file for every
// MFMA of a kernel, and S has to stay in VGPRs for the softmax.)  With O in
// AGPRs an MFMA issue holds back the other wave's VALU work for fewer cycles:
// llama16k measured 4% faster on MI355X.
// The compiler does not know these registers hold a value between the
// statements, so the kernel is correct only while the compiler allocates no
// AGPR of its own in it; a test compiles the kernel and checks exactly that
// (it needs about 124 VGPRs, inside the 128 the compiler keeps for VGPRs in a
// kernel that uses AGPRs).  Hazards the compiler cannot see: VALU code reads
// or rewrites O only after ofix_settle (24 wait states, more than a 16-pass
// MFMA's result needs); two MFMAs on one block are four MFMAs apart; the P, V
// and scale operands come from LDS loads (which the compiler's waits cover) or
// from VALU writes a whole softmax phase before the MFMA.
__device__ __forceinline__ void ofix_settle() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7");
#endif
}
// O^T block cb += V^T P^T (E4M3 x E4M3 with block scales sa, sb).
__device__ __forceinline__ void ofix_mfma(int cb, const v8i& a, const v8i& b, int sa, int sb) {
#if defined(__HIP_DEVICE_COMPILE__)
  switch (cb) {
    case 0:
      asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 a[0:15], %0, %1, a[0:15], %2, %3 op_sel_hi:[0,0,0]"
                   :
                   : "v"(a), "v"(b), "v"(sa), "v"(sb)
                   : "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15");
      break;
    case 1:
      asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 a[16:31], %0, %1, a[16:31], %2, %3 op_sel_hi:[0,0,0]"
                   :
                   : "v"(a), "v"(b), "v"(sa), "v"(sb)
                   : "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31");
      break;
    case 2:
      asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 a[32:47], %0, %1, a[32:47], %2, %3 op_sel_hi:[0,0,0]"
                   :
                   : "v"(a), "v"(b), "v"(sa), "v"(sb)
                   : "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47");
      break;
    case 3:
      asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 a[48:63], %0, %1, a[48:63], %2, %3 op_sel_hi:[0,0,0]"
                   :
                   : "v"(a), "v"(b), "v"(sa), "v"(sb)
                   : "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63");
      break;
  }
#endif
}
#if defined(__HIP_DEVICE_COMPILE__)
#define QFA_OFIX_Z(N) asm volatile("v_accvgpr_write_b32 a" #N ", 0" ::: "a" #N)
#define QFA_OFIX_RD(N) asm volatile("v_accvgpr_read_b32 %0, a" #N : "=v"(x[N]))
#define QFA_OFIX_SC(N)                                                                                  \
  asm volatile("v_accvgpr_read_b32 %0, a" #N "\n v_mul_f32 %0, %0, %1\n v_accvgpr_write_b32 a" #N ", %0" \
               : "=&v"(t)                                                                               \
               : "v"(f)                                                                                 \
               : "a" #N)
#else
#define QFA_OFIX_Z(N)
#define QFA_OFIX_RD(N) x[N] = 0.0f
#define QFA_OFIX_SC(N) (void)t
#endif
// O^T = 0 for the first NB blocks (plain AGPR writes: an MFMA would read
// operands the compiler does not know are read).
template <int NB>
__device__ __forceinline__ void ofix_zero() {
  if constexpr (NB > 0) {
    QFA_OFIX_Z(0); QFA_OFIX_Z(1); QFA_OFIX_Z(2); QFA_OFIX_Z(3); QFA_OFIX_Z(4); QFA_OFIX_Z(5); QFA_OFIX_Z(6); QFA_OFIX_Z(7);
    QFA_OFIX_Z(8); QFA_OFIX_Z(9); QFA_OFIX_Z(10); QFA_OFIX_Z(11); QFA_OFIX_Z(12); QFA_OFIX_Z(13); QFA_OFIX_Z(14); QFA_OFIX_Z(15);
  }
  if constexpr (NB > 1) {
    QFA_OFIX_Z(16); QFA_OFIX_Z(17); QFA_OFIX_Z(18); QFA_OFIX_Z(19); QFA_OFIX_Z(20); QFA_OFIX_Z(21); QFA_OFIX_Z(22); QFA_OFIX_Z(23);
    QFA_OFIX_Z(24); QFA_OFIX_Z(25); QFA_OFIX_Z(26); QFA_OFIX_Z(27); QFA_OFIX_Z(28); QFA_OFIX_Z(29); QFA_OFIX_Z(30); QFA_OFIX_Z(31);
  }
  if constexpr (NB > 2) {
    QFA_OFIX_Z(32); QFA_OFIX_Z(33); QFA_OFIX_Z(34); QFA_OFIX_Z(35); QFA_OFIX_Z(36); QFA_OFIX_Z(37); QFA_OFIX_Z(38); QFA_OFIX_Z(39);
    QFA_OFIX_Z(40); QFA_OFIX_Z(41); QFA_OFIX_Z(42); QFA_OFIX_Z(43); QFA_OFIX_Z(44); QFA_OFIX_Z(45); QFA_OFIX_Z(46); QFA_OFIX_Z(47);
  }
  if constexpr (NB > 3) {
    QFA_OFIX_Z(48); QFA_OFIX_Z(49); QFA_OFIX_Z(50); QFA_OFIX_Z(51); QFA_OFIX_Z(52); QFA_OFIX_Z(53); QFA_OFIX_Z(54); QFA_OFIX_Z(55);
    QFA_OFIX_Z(56); QFA_OFIX_Z(57); QFA_OFIX_Z(58); QFA_OFIX_Z(59); QFA_OFIX_Z(60); QFA_OFIX_Z(61); QFA_OFIX_Z(62); QFA_OFIX_Z(63);
  }
}
// x[16 cb + rr] = O^T block cb, element rr.
template <int NB>
__device__ __forceinline__ void ofix_read(float (&x)[64]) {
  if constexpr (NB > 0) {
    QFA_OFIX_RD(0); QFA_OFIX_RD(1); QFA_OFIX_RD(2); QFA_OFIX_RD(3); QFA_OFIX_RD(4); QFA_OFIX_RD(5); QFA_OFIX_RD(6); QFA_OFIX_RD(7);
    QFA_OFIX_RD(8); QFA_OFIX_RD(9); QFA_OFIX_RD(10); QFA_OFIX_RD(11); QFA_OFIX_RD(12); QFA_OFIX_RD(13); QFA_OFIX_RD(14); QFA_OFIX_RD(15);
  }
  if constexpr (NB > 1) {
    QFA_OFIX_RD(16); QFA_OFIX_RD(17); QFA_OFIX_RD(18); QFA_OFIX_RD(19); QFA_OFIX_RD(20); QFA_OFIX_RD(21); QFA_OFIX_RD(22); QFA_OFIX_RD(23);
    QFA_OFIX_RD(24); QFA_OFIX_RD(25); QFA_OFIX_RD(26); QFA_OFIX_RD(27); QFA_OFIX_RD(28); QFA_OFIX_RD(29); QFA_OFIX_RD(30); QFA_OFIX_RD(31);
  }
  if constexpr (NB > 2) {
    QFA_OFIX_RD(32); QFA_OFIX_RD(33); QFA_OFIX_RD(34); QFA_OFIX_RD(35); QFA_OFIX_RD(36); QFA_OFIX_RD(37); QFA_OFIX_RD(38); QFA_OFIX_RD(39);
    QFA_OFIX_RD(40); QFA_OFIX_RD(41); QFA_OFIX_RD(42); QFA_OFIX_RD(43); QFA_OFIX_RD(44); QFA_OFIX_RD(45); QFA_OFIX_RD(46); QFA_OFIX_RD(47);
  }
  if constexpr (NB > 3) {
    QFA_OFIX_RD(48); QFA_OFIX_RD(49); QFA_OFIX_RD(50); QFA_OFIX_RD(51); QFA_OFIX_RD(52); QFA_OFIX_RD(53); QFA_OFIX_RD(54); QFA_OFIX_RD(55);
    QFA_OFIX_RD(56); QFA_OFIX_RD(57); QFA_OFIX_RD(58); QFA_OFIX_RD(59); QFA_OFIX_RD(60); QFA_OFIX_RD(61); QFA_OFIX_RD(62); QFA_OFIX_RD(63);
  }
}
// O^T *= f.
template <int NB>
__device__ __forceinline__ void ofix_scale(float f) {
  float t = 0.0f;
  if constexpr (NB > 0) {
    QFA_OFIX_SC(0); QFA_OFIX_SC(1); QFA_OFIX_SC(2); QFA_OFIX_SC(3); QFA_OFIX_SC(4); QFA_OFIX_SC(5); QFA_OFIX_SC(6); QFA_OFIX_SC(7);
    QFA_OFIX_SC(8); QFA_OFIX_SC(9); QFA_OFIX_SC(10); QFA_OFIX_SC(11); QFA_OFIX_SC(12); QFA_OFIX_SC(13); QFA_OFIX_SC(14); QFA_OFIX_SC(15);
  }
  if constexpr (NB > 1) {
    QFA_OFIX_SC(16); QFA_OFIX_SC(17); QFA_OFIX_SC(18); QFA_OFIX_SC(19); QFA_OFIX_SC(20); QFA_OFIX_SC(21); QFA_OFIX_SC(22); QFA_OFIX_SC(23);
    QFA_OFIX_SC(24); QFA_OFIX_SC(25); QFA_OFIX_SC(26); QFA_OFIX_SC(27); QFA_OFIX_SC(28); QFA_OFIX_SC(29); QFA_OFIX_SC(30); QFA_OFIX_SC(31);
  }
  if constexpr (NB > 2) {
    QFA_OFIX_SC(32); QFA_OFIX_SC(33); QFA_OFIX_SC(34); QFA_OFIX_SC(35); QFA_OFIX_SC(36); QFA_OFIX_SC(37); QFA_OFIX_SC(38); QFA_OFIX_SC(39);
    QFA_OFIX_SC(40); QFA_OFIX_SC(41); QFA_OFIX_SC(42); QFA_OFIX_SC(43); QFA_OFIX_SC(44); QFA_OFIX_SC(45); QFA_OFIX_SC(46); QFA_OFIX_SC(47);
  }
  if constexpr (NB > 3) {
    QFA_OFIX_SC(48); QFA_OFIX_SC(49); QFA_OFIX_SC(50); QFA_OFIX_SC(51); QFA_OFIX_SC(52); QFA_OFIX_SC(53); QFA_OFIX_SC(54); QFA_OFIX_SC(55);
    QFA_OFIX_SC(56); QFA_OFIX_SC(57); QFA_OFIX_SC(58); QFA_OFIX_SC(59); QFA_OFIX_SC(60); QFA_OFIX_SC(61); QFA_OFIX_SC(62); QFA_OFIX_SC(63);
  }
}
#undef QFA_OFIX_Z
#undef QFA_OFIX_RD
#undef QFA_OFIX_SC

// Softmax step of one tile.  s holds S' = Q'K^T, the logits in log2 units
// (Q carries the factor softmax_scale * log2 e).  Masks keys > jlim (when
// need_mask), adds the compensation offset d32 = fl32(c2 * delta) (COMP),
// moves the running max m on the integer grid and converts P (see PV_FP8)
// into pb, the B operand of the P V product (pb[h] covers keys 64h .. 64h+63).
// pscale[h] receives the E8M0 code that the P V product of half h applies:
// 2^(m - m_ref) (PV_FP8), or 2^(e_b - m_ref) of the key block b = 2h + g
// whose scale this lane supplies (PV_FP8_BLOCKP, PV_FP4).  O and l are
// touched only by the rare frame rebase.
template <int D, bool COMP, int PV, bool OF = false>
__device__ __forceinline__ void softmax_tile(RowState<D>& st, v16f (&s)[4], int t, bool need_mask, int jlim,
                                             float d32, POp<PV> (&pb)[2], int (&pscale)[2]) {
  constexpr int P = pv_of(PV);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  // ---- mask (diagonal / ragged tiles only); score s[c][rr] is key
  // 128t + score_key(c, g, rr).  A lane's 16 keys of MFMA c are consecutive,
  // so the visible ones are a prefix rr <= nvm1; the select is done on the
  // bits ((nvm1 - rr) >> 31 is -1 for a masked key), which keeps 64
  // comparison masks out of the SGPRs.
  if (need_mask) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int nvm1 = jlim - (kTile * t + score_key<PV>(c, g, 0));
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int msk = (nvm1 - rr) >> 31;
        s[c][rr] = __int_as_float((__float_as_int(s[c][rr]) & ~msk) | (int)(0xFF800000u & (uint32_t)msk));
      }
    }
  }
  if (COMP) {  // y = fl32(S' + d32)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s[c][rr] += d32;
  }

  // ---- row max (two left-associated chains: max(max(m, a), b) compiles to
  // v_max3_f32, one instruction per two scores) and one lane swap
  float mx;
  float bmax[4];  // PV_FP8_BLOCKP: max of key block c (both lanes of the row); PV_FP4: [h] of block 2h + g
  if constexpr (P == PV_FP4) {
    // a lane holds all 32 keys of block 2h + g: its max needs no other lane
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float x = __builtin_fmaxf(s[2 * h][0], s[2 * h][1]);
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int rr = (w == 0 ? 2 : 0); rr < 16; rr += 2)
          x = __builtin_fmaxf(__builtin_fmaxf(x, s[2 * h + w][rr]), s[2 * h + w][rr + 1]);
      bmax[h] = x;
    }
    mx = __builtin_fmaxf(bmax[0], bmax[1]);
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  } else if constexpr (P == PV_FP8) {
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
    mx = __builtin_fmaxf(mx0, mx1);
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  } else {
    // this lane's 16 keys of each block, then the partner lane's (l ^ 32)
    // half: the first swap of (block 2h, block 2h+1) leaves in lane group g
    // both halves of block 2h + g; the second hands each lane the other block
    float pm[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float x = __builtin_fmaxf(s[c][0], s[c][1]);
#pragma unroll
      for (int rr = 2; rr < 16; rr += 2) x = __builtin_fmaxf(__builtin_fmaxf(x, s[c][rr]), s[c][rr + 1]);
      pm[c] = x;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm[2 * h]), __float_as_uint(pm[2 * h + 1]), false,
                                                 false);
      const float f = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(f), __float_as_uint(f), false, false);
      bmax[2 * h] = __uint_as_float(sw2[0]);
      bmax[2 * h + 1] = __uint_as_float(sw2[1]);
    }
    mx = __builtin_fmaxf(__builtin_fmaxf(bmax[0], bmax[1]), __builtin_fmaxf(bmax[2], bmax[3]));
  }
  // Running max on the integer grid: every rescale factor is an exact power of
  // two, applied through the E8M0 scale of the P operand (no VALU work on O).
  const float mn = __builtin_fmaxf(st.m, __builtin_ceilf(mx));
  if (st.m_ref == -__builtin_inff()) st.m_ref = mn;  // first visible key fixes the frame
  st.m = mn;
  // Keep 2^(m - m_ref) inside the E8M0 range: rebase the frame when it grows
  // past 2^64 (rare: the row max would have to climb 64 binades).
  if (__builtin_amdgcn_ballot_w64(mn - st.m_ref > 64.0f)) {
    const float f = (mn - st.m_ref > 64.0f) ? __builtin_ldexpf(1.0f, (int)(st.m_ref - mn)) : 1.0f;
    if constexpr (OF) {
      ofix_settle();
      ofix_scale<D / 32>(f);
    } else {
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(st.o[cb][rr]) : "v"(f));
    }
    if constexpr (P == PV_FP8) {
      st.lsum *= f;
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(st.lv[rr]) : "v"(f));
    }
    if (mn - st.m_ref > 64.0f) st.m_ref = mn;
  }
  // ---- P8 = E4M3(256 * 2^(y - e)), packed as the B operand of O^T += V^T P^T,
  // with e = m (PV_FP8) or e = e_c of the key block (PV_FP8_BLOCKP).  The
  // conversion divides by its scale operand, so 2^(e - 8) there turns 2^y
  // into 256 * 2^(y - e) exactly, with no per-score subtraction.  That needs
  // 2^y and the scale in binary32 range: while e lies in [-100, 100] the keys
  // that can give a non-zero code (y > e - 18) have 2^y in [2^-118, 2^100].
  // A wave with an exponent outside subtracts it from the scores first.
  float e[4];
  if constexpr (P == PV_FP4) {  // e[c]: the exponent of MFMA c's keys (block 2h + g for c = 2h + w)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float eh = (mn == -__builtin_inff()) ? 0.0f : __builtin_fmaxf(__builtin_ceilf(bmax[h]), mn - 64.0f);
      e[2 * h] = e[2 * h + 1] = eh;
      pscale[h] = (mn == -__builtin_inff()) ? kScaleOne : kScaleOne + (int)(eh - st.m_ref);
    }
  } else if constexpr (P == PV_FP8) {
    pscale[0] = pscale[1] = (mn == -__builtin_inff()) ? kScaleOne : kScaleOne + (int)(mn - st.m_ref);
    e[0] = e[1] = e[2] = e[3] = (mn == -__builtin_inff()) ? 0.0f : mn;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)  // also for a block with no visible key: the floor
      e[c] = (mn == -__builtin_inff()) ? 0.0f : __builtin_fmaxf(__builtin_ceilf(bmax[c]), mn - 64.0f);
    // lane group g supplies the scale of block 2h + g (a mask select: an
    // indexed e[2h + g] would put e in scratch memory)
    const int gm = -((threadIdx.x & 63) >> 5);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d0 = (int)(e[2 * h] - st.m_ref), d1 = (int)(e[2 * h + 1] - st.m_ref);
      pscale[h] = (mn == -__builtin_inff()) ? kScaleOne : kScaleOne + (d0 ^ ((d0 ^ d1) & gm));
    }
  }
  bool out_of_range = false;
#pragma unroll
  for (int c = 0; c < (P == PV_FP8 ? 1 : 4); ++c) out_of_range |= __builtin_fabsf(e[c]) > 100.0f;
  const bool far = __builtin_amdgcn_ballot_w64(out_of_range) != 0;
  if (far) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s[c][rr] -= e[c];
  }
  // the conversion's scale: 2^(e - 8) for E4M3 (codes 256 * 2^(y - e)),
  // 2^(e - 2) for E2M1 (codes 4 * 2^(y - e))
  constexpr int PB = P == PV_FP4 ? 2 : 8;
  float cs[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) cs[c] = far ? (P == PV_FP4 ? 0x1p-2f : 0x1p-8f) : __builtin_ldexpf(1.0f, (int)e[c] - PB);
  if constexpr (P == PV_FP4) {
    // pb[h] register r holds keys 8r .. 8r+7 of block 2h + g (s[2h + r/2][8(r%2) ..]),
    // two E2M1 codes per byte, the lower key in the low nibble
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 2 * h + (r >> 1), r0 = 8 * (r & 1);
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(s[c][r0 + j]);
        uint32_t w = __float_as_uint(p[0]);  // dead old value: every byte is written
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[0], p[1], cs[c], 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[2], p[3], cs[c], 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[4], p[5], cs[c], 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[6], p[7], cs[c], 3);
        pb[h][r] = (int)w;
      }
    return;
  } else {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = 2 * h + (k >> 2);
      const int r0 = 4 * (k & 3);
      const float p0 = __builtin_amdgcn_exp2f(s[c][r0 + 0]);
      const float p1 = __builtin_amdgcn_exp2f(s[c][r0 + 1]);
      const float p2 = __builtin_amdgcn_exp2f(s[c][r0 + 2]);
      const float p3 = __builtin_amdgcn_exp2f(s[c][r0 + 3]);
      // the old value of the destination is dead (both halves are written): reuse p0's register
      v2s w = __builtin_bit_cast(v2s, p0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, p0, p1, cs[c], false);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, p2, p3, cs[c], true);
      pb[h][k] = __builtin_bit_cast(int, w);
    }
  }
}

// Start block of the S^T accumulator for the compensated kernels: the 32 x 32
// block (key, row) with every entry equal to the row's offset d (this lane's
// d, lane l holding row l % 32), built on the matrix unit instead of by 16
// VALU moves.  One FP32 MFMA (v_mfma_f32_32x32x2f32): A = 1 everywhere, B = d
// at contraction index 0 (lanes 0..31) and 0 at index 1 (lanes 32..63), so
// entry (key, row) = 1 * d + 1 * 0 = d exactly, infinities included.
__device__ __forceinline__ v16f offset_block(float d) {
  const float b = (threadIdx.x & 32) ? 0.0f : d;
  return __builtin_amdgcn_mfma_f32_32x32x2f32(1.0f, b, v16f{}, 0, 0, 0);
}

// One K operand block (32 keys x all channels): the A operands of the D/64
// MFMAs of key block c and their scale bytes (byte k feeds MFMA k).
template <int D>
struct KBlk {
  v4i ka[D / 64];
  int sc;
};

template <int D, int PV>
__device__ __forceinline__ void load_k_blk(const uint8_t* kreg, const LaneOffs<D, PV>& lo, int c, KBlk<D>& k) {
  // first token of MFMA c's rows (plus the lane's own token offset)
  const int t0 = PV == PV_FP4 ? 64 * (c >> 1) + 16 * (c & 1) : 32 * c;
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk) {
    const uint32_t lk = (PV == PV_FP4 && (c & 1)) ? lo.k1[PV == PV_FP4 ? kk : 0] : lo.k[kk];
    k.ka[kk] = *reinterpret_cast<const v4i*>(kreg + lk + t0 * (D / 2));
  }
  using TL = TileLayout<D, PV>;
  const uint8_t* sp = kreg + lo.ks + t0 * TL::KSB;
  if (PV == QK_NVFP4)  // four (D = 128) or two E4M3 scales of this lane's channels
    k.sc = D == 128 ? (int)*reinterpret_cast<const uint32_t*>(sp) : (int)*reinterpret_cast<const uint16_t*>(sp);
  else                 // two (D = 128) or one E8M0 scale
    k.sc = D == 128 ? (int)*reinterpret_cast<const uint16_t*>(sp) : (int)*sp;
}

// S^T block c = K_c Q^T: sc_[rr] is the score of this lane's row (l % 32)
// against key 32c + 16g + rr of the tile (g = l / 32).
// QK_NVFP4: eight E2M1 codes (one dword, channels 8r .. 8r+7 of a 32-channel
// chunk) times their E4M3 block scale s times the tensor scale g, as bf16.
// The scaled FP4 conversions apply only the exponent of their scale operand
// (an E8M0 scale), so the codes are converted with g (a power of two) to
// binary32, multiplied by s there (exact: at most six significant bits) and
// packed to bf16 (exact for the same reason).
__device__ __forceinline__ bf16x8 nvfp4_decode8(uint32_t w, float s, float g) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, g, 0);
  const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, g, 1);
  const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, g, 2);
  const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, g, 3);
  return bf16x8{(__bf16)(p0[0] * s), (__bf16)(p0[1] * s), (__bf16)(p1[0] * s), (__bf16)(p1[1] * s),
                (__bf16)(p2[0] * s), (__bf16)(p2[1] * s), (__bf16)(p3[0] * s), (__bf16)(p3[1] * s)};
}

// init: the accumulator's start value (zero, or the compensation offset of
// this lane's row, which then enters the exponent argument through the MFMA's
// accumulate instead of one add per score).
template <int D, int PV = PV_FP8>
__device__ __forceinline__ void qk_blk(const RowState<D>& st, const KBlk<D>& k, v16f& sc_,
                                       const v16f& init = v16f{}) {
  sc_ = init;
  if constexpr (PV == QK_NVFP4) {
    // lane group g holds chunk kblock(g, kk) (32 channels); bf16 MFMA 4kk + r
    // contracts its channels 8r .. 8r+7 against the same channels of Q
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = e4m3_byte_to_f32(k.sc, 2 * kk + (r >> 1));
        const bf16x8 a = nvfp4_decode8((uint32_t)k.ka[kk][r], s, st.gk);
        sc_ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.qn[4 * kk + r], sc_, 0, 0, 0);
      }
  } else {
    sc_ = mfma_fp4_32x32x64_sel<0>(k.ka[0], st.qa[0], sc_, k.sc, st.qs);
    if (D == 128) sc_ = mfma_fp4_32x32x64_sel<1>(k.ka[D / 64 - 1], st.qa[D / 64 - 1], sc_, k.sc, st.qs);
  }
}

// One V operand (64 keys x 32 channels: half h = q / (D/32), channel block
// cb = q % (D/32)) and its E8M0 scale byte.
template <int D, int PV>
__device__ __forceinline__ void load_v_op(const uint8_t* vreg, const LaneOffs<D, PV>& lo, int q, POp<PV>& a,
                                          int& sa) {
  const int h = q / (D / 32), cb = q % (D / 32);
  if constexpr (PV == PV_FP4) {
    a = *reinterpret_cast<const v4i*>(vreg + lo.v + (2 * h * D + 32 * cb) * 16);
  } else {
    const v4i a0 = *reinterpret_cast<const v4i*>(vreg + lo.v + ((2 * h) * D + 32 * cb) * 32);
    const v4i a1 = *reinterpret_cast<const v4i*>(vreg + lo.v + ((2 * h + 1) * D + 32 * cb) * 32);
    a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  sa = vreg[lo.vs + 2 * h * D + 32 * cb];
}

// O^T or l += V^T P^T of one (half, channel block) on the FP8 or the FP4 MFMA.
template <int PV>
__device__ __forceinline__ v16f mfma_pv(const POp<PV>& a, const POp<PV>& b, v16f c, int sa, int sb) {
  if constexpr (PV == PV_FP4)
    return mfma_fp4_32x32x64(a, b, c, sa, sb);
  else
    return mfma_fp8_32x32x64(a, b, c, sa, sb);
}
template <int PV>
__device__ __forceinline__ POp<PV> ones_op(const v8i& ones) {
  if constexpr (PV == PV_FP4)
    return v4i{ones[0], ones[1], ones[2], ones[3]};
  else
    return ones;
}

// O^T block cb += V^T P^T, in VGPRs or (OF) in the fixed accumulation registers.
template <int D, int PV, bool OF>
__device__ __forceinline__ void o_acc(RowState<D>& st, int cb, const POp<PV>& a, const POp<PV>& b, int sa, int sb) {
  if constexpr (OF)
    ofix_mfma(cb, a, b, sa, sb);
  else
    st.o[cb] = mfma_pv<PV>(a, b, st.o[cb], sa, sb);
}

// Row sums of the E4M3 P codes of one 64-key half, accumulated into ts, on
// one 16x16x128 MFMA at unit scales.  Read as the B operand of that product,
// the 32x32x64 P operand pb (lane l: query l % 32) gives output column c the
// codes of query c from lane groups 0 and 2 and of query c + 16 from groups 1
// and 3; with the E4M3 index layout (see mfma_fp4_fp8_16x16x128) these are
// exactly the contraction indices with bit 4 clear and set.  The selector
// operand st.sel holds E2M1 ones in nibbles 0..15 (indices with bit 4 clear)
// for rows r with bit 2 clear and in nibbles 16..31 for the others, so output
// (r, c) sums query c + 16 ((r >> 2) & 1); the rows lane l holds,
// 4 (l / 16) .. 4 (l / 16) + 3, then make all four of its elements the sum of
// its own query l % 32.  P's row scale cannot ride on this product (a 32-index
// scale block mixes two queries), so the sum is taken in P's own frame and
// folded into st.lsum with the factor 2^(m - m_ref) by one FMA.  The result is
// bit-identical to the 32x32x64 product against E4M3 ones at unit scale
// (checked on MI355X), at half the matrix time and a quarter of the registers.
__device__ __forceinline__ v4f tile_rowsum(const v4i& sel, const v8i& pb, const v4f& ts) {
  return mfma_fp4_fp8_16x16x128(sel, pb, ts);
}
// lsum += 2^(m - m_ref) * (tile row sum), the factor read from P's scale code.
template <int D>
__device__ __forceinline__ void fold_rowsum(RowState<D>& st, const v4f& ts, int pscale) {
  st.lsum = __builtin_fmaf(ts[0], __builtin_ldexpf(1.0f, pscale - kScaleOne), st.lsum);
}

// O^T += 2^(m - m_ref) V^T P^T of one tile (FP8 x FP8; V's E8M0 scale per 32
// tokens x channel, P's per row) and the denominator (tile_rowsum for E4M3 P;
// for block-scaled P the same product against ones), followed by S = K Q^T of
// the next tile.  Software-pipelined
// over a small ring of operand registers: V operands are read three products
// ahead and the first two K blocks during the last P V products, so the MFMAs
// issue back to back while LDS reads stay in flight.  The scheduler fences
// keep this order within the register budget of two waves per SIMD.
struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// hook(k) runs after the k-th MFMA step (k = 0 .. 2 D/32 + 3), inside the
// scheduling fences: a place for instructions that should issue while the
// matrix unit is busy.  KEEP_INIT (a non-zero start block) keeps init live
// through the S products: otherwise the last block's MFMA takes over init's
// registers and the result is copied out again (8 v_mov_b64 per tile).
template <int D, int PV, class Hook = NoHook, bool KEEP_INIT = false, bool OF = false>
__device__ __forceinline__ void pv_then_qk(RowState<D>& st, const LaneOffs<D, PV>& lo, const uint8_t* vreg,
                                           const POp<PV> (&pb)[2], const int (&pscale)[2], const uint8_t* kreg,
                                           v16f (&s)[4], const v16f& init, const Hook& hook = Hook()) {
  constexpr int NQ = 2 * (D / 32);  // P V products (excluding the denominator)
  constexpr int R = 3;              // V operands in flight
  constexpr bool TS = pv_of(PV) == PV_FP8;
  POp<PV> va[R];
  int vs[R];
  KBlk<D> kb[2];
  v4f ts = v4f{};
#pragma unroll
  for (int q = 0; q < R; ++q) load_v_op<D, PV>(vreg, lo, q, va[q], vs[q]);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    __builtin_amdgcn_sched_barrier(0);
    const int h = q / (D / 32), cb = q % (D / 32);
    o_acc<D, PV, OF>(st, cb, va[q % R], pb[h], vs[q % R], pscale[h]);
    if (cb == D / 32 - 1) {
      if constexpr (TS)
        ts = tile_rowsum(st.sel, pb[h], ts);
      else
        st.lv = mfma_pv<PV>(ones_op<PV>(st.ones), pb[h], st.lv, kScaleOne, pscale[h]);
    }
    if (q + R < NQ)
      load_v_op<D, PV>(vreg, lo, q + R, va[q % R], vs[q % R]);
    else if (q + R - NQ < 2)
      load_k_blk<D, PV>(kreg, lo, q + R - NQ, kb[q + R - NQ]);
    hook(q);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    __builtin_amdgcn_sched_barrier(0);
    qk_blk<D, PV>(st, kb[c & 1], s[c], init);
    if (c + 2 < 4) load_k_blk<D, PV>(kreg, lo, c + 2, kb[c & 1]);
    hook(NQ + c);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (KEEP_INIT) asm volatile("" ::"v"(init));
  // (the row sums finished during the S products)
  if constexpr (TS) fold_rowsum(st, ts, pscale[0]);
}

// P V of one tile alone, pipelined like pv_then_qk.
template <int D, int PV>
__device__ __forceinline__ void pv_tile(RowState<D>& st, const LaneOffs<D, PV>& lo, const uint8_t* vreg,
                                        const POp<PV> (&pb)[2], const int (&pscale)[2]) {
  constexpr int NQ = 2 * (D / 32);
  constexpr int R = 3;
  constexpr bool TS = pv_of(PV) == PV_FP8;
  POp<PV> va[R];
  int vs[R];
  v4f ts = v4f{};
#pragma unroll
  for (int q = 0; q < R; ++q) load_v_op<D, PV>(vreg, lo, q, va[q], vs[q]);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    __builtin_amdgcn_sched_barrier(0);
    const int h = q / (D / 32), cb = q % (D / 32);
    o_acc<D, PV, false>(st, cb, va[q % R], pb[h], vs[q % R], pscale[h]);
    if (cb == D / 32 - 1) {
      if constexpr (TS)
        ts = tile_rowsum(st.sel, pb[h], ts);
      else
        st.lv = mfma_pv<PV>(ones_op<PV>(st.ones), pb[h], st.lv, kScaleOne, pscale[h]);
    }
    if (q + R < NQ) load_v_op<D, PV>(vreg, lo, q + R, va[q % R], vs[q % R]);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (TS) fold_rowsum(st, ts, pscale[0]);
}

// S = K Q^T of one tile alone, two K blocks in flight.
template <int D, int PV>
__device__ __forceinline__ void qk_tile(const RowState<D>& st, const LaneOffs<D, PV>& lo, const uint8_t* kreg,
                                        v16f (&s)[4], const v16f& init = v16f{}) {
  KBlk<D> kb[2];
  load_k_blk<D, PV>(kreg, lo, 0, kb[0]);
  load_k_blk<D, PV>(kreg, lo, 1, kb[1]);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    __builtin_amdgcn_sched_barrier(0);
    qk_blk<D, PV>(st, kb[c & 1], s[c], init);
    if (c + 2 < 4) load_k_blk<D, PV>(kreg, lo, c + 2, kb[c & 1]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Epilogue of one row: O = O^T / l (this lane writes half of the row's
// channels) and LSE = ln2 * (m_ref + log2(l / 256)) (E4M3 P: codes of
// 256 * 2^(y - e); E2M1 P: 4 * 2^(y - e), so l / 4).  lse_row may be null.
template <int D, int PV = PV_FP8, bool OF = false>
__device__ __forceinline__ void store_row(const RowState<D>& st, float* orow, float* lse_row) {
  const int g = (threadIdx.x & 63) >> 5;
  const float l = pv_of(PV) == PV_FP8 ? st.lsum : st.lv[0];
  const bool empty = (st.m == -__builtin_inff());
  const float inv = empty ? 0.0f : 1.0f / l;
  if constexpr (OF) {
    float x[64];
    ofix_settle();
    ofix_read<D / 32>(x);
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) orow[32 * cb + (rr >> 2) * 8 + 4 * g + (rr & 3)] = x[16 * cb + rr] * inv;
  } else {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) orow[32 * cb + (rr >> 2) * 8 + 4 * g + (rr & 3)] = st.o[cb][rr] * inv;
  }
  if (lse_row && g == 0)
    *lse_row = empty ? -__builtin_inff()
                     : 0.69314718055994531f * (st.m_ref + __builtin_log2f(l * (PV == PV_FP4 ? 0x1p-2f : 0x1p-8f)));
}

// delta^T for 32 tiles starting at tau0: Kbar[tau0 .. tau0+31] . Q_bf16^T,
// into the wave's LDS slab dl[tile][row] as binary32.  The products of two bf16
// values are exact in binary64 and a sum of D of them stays exact there, so the
// FP64 MFMA (v_mfma_f64_16x16x4f64) yields the exactly rounded binary32 value:
// the per-(row, tile) exponent offset, which decides P codes, is then the same
// number the binary64 definition gives.  Four 16x16 blocks (2 tile halves x 2
// row halves), each in D/32 steps of 8 channels per lane; the contraction
// index of step s, element e, lane group g is channel D/4 g + 8 s + e (any
// pairing works as long as A and B agree).  The operands of a step are loaded
// one step ahead, across block boundaries, so the FP64 MFMAs do not wait on
// global-memory latency.  Tiles from tlim on are not needed: their K-bar rows
// read as zeros, and the blocks of a tile half that starts there are skipped.
template <int D>
__device__ __forceinline__ void compute_delta(float* dl, const uint16_t* kbar_bg, int tlim, int tau0,
                                              const uint16_t* qbase, int q_stride, int nrows_valid) {
  typedef double v4d __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  constexpr int CPG = D / 4;          // channels per lane group
  constexpr int NS = CPG / 8;         // steps per block
  constexpr int NSTEP = 4 * NS;       // steps of the call
  constexpr int PF = 1;               // steps whose operands are in flight
  const int nblk = (tau0 + 16 < tlim) ? 4 : 2;  // wave-uniform
  uint4 ka[PF], qa[PF];
  auto load = [&](int i, uint4& k, uint4& q) {
    const int blk = i / NS, c0 = CPG * g + 8 * (i % NS);
    const int tau = tau0 + 16 * (blk >> 1) + r16, row = 16 * (blk & 1) + r16;
    k = make_uint4(0u, 0u, 0u, 0u);
    q = make_uint4(0u, 0u, 0u, 0u);
    if (blk < nblk && tau < tlim) k = *reinterpret_cast<const uint4*>(kbar_bg + (size_t)tau * D + c0);
    if (blk < nblk && row < nrows_valid) q = *reinterpret_cast<const uint4*>(qbase + (size_t)row * q_stride + c0);
  };
  auto widen = [](const uint4& w, int e) {
    const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
    return (double)bf16_bits_to_float((x >> ((e & 1) ? 16 : 0)) & 0xFFFFu);
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) load(i, ka[i], qa[i]);
  // two independent accumulation chains (even and odd elements), so one
  // MFMA need not wait for the previous one's result; their sum is exact too
  v4d acc[2] = {v4d{0.0, 0.0, 0.0, 0.0}, v4d{0.0, 0.0, 0.0, 0.0}};
#pragma unroll
  for (int i = 0; i < NSTEP; ++i) {
    const int blk = i / NS;
    if (blk >= nblk) break;
    const uint4 k = ka[i % PF], q = qa[i % PF];
    if (i + PF < NSTEP) load(i + PF, ka[i % PF], qa[i % PF]);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc[e & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64(widen(k, e), widen(q, e), acc[e & 1], 0, 0, 0);
    if (i % NS == NS - 1) {
      // FP64 16x16 result layout: register r of lane l holds entry (i, j) = (l / 16 + 4 r, l % 16):
      // tile 16 tb + lane / 16 + 4 r, query row 16 rb + lane % 16
      const int tb = blk >> 1, rb = blk & 1;
#pragma unroll
      for (int r = 0; r < 4; ++r) dl[(16 * tb + g + 4 * r) * 32 + 16 * rb + r16] = (float)(acc[0][r] + acc[1][r]);
      acc[0] = acc[1] = v4d{0.0, 0.0, 0.0, 0.0};
    }
  }
}

// Q fragments of this lane's row (zeros when invalid) and a fresh row state.
// With q4row null, the row is quantised here from its bf16 values qbfrow
// (times c2, then the MXFP4 block rule): the same bytes the quantiser kernel
// writes for Q with prescale c2.  QK_NVFP4 takes the quantised row (codes, E4M3
// scales) and the tensor scales gq, gk, and keeps Q as bf16.
template <int D, int PV = PV_FP8, bool OF = false>
__device__ __forceinline__ void load_q(RowState<D>& st, const uint8_t* q4row, const uint8_t* q4srow,
                                       const uint16_t* qbfrow, float c2, bool valid, float gq = 1.0f,
                                       float gk = 1.0f) {
  const int g = (threadIdx.x & 63) >> 5;
  st.qs = 0;
  if constexpr (PV == QK_NVFP4) {  // NVFP4 Q (codes and E4M3 scales) decoded to bf16
    st.gk = gk;
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
      const int b = kblock<D>(g, kk);
      const v4i c = valid ? *reinterpret_cast<const v4i*>(q4row + 16 * b) : v4i{0, 0, 0, 0};
      const int sc = valid ? (int)*reinterpret_cast<const uint16_t*>(q4srow + 2 * b) : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        st.qn[4 * kk + r] = nvfp4_decode8((uint32_t)c[r], e4m3_byte_to_f32(sc, r >> 1), gq);
    }
  } else {
#pragma unroll
  for (int k = 0; k < D / 64; ++k) {
    const int b = kblock<D>(g, k);
    if (!valid) {
      st.qa[k] = v4i{0, 0, 0, 0};
    } else if (q4row) {
      st.qa[k] = *reinterpret_cast<const v4i*>(q4row + 16 * b);
      st.qs |= (int)q4srow[b] << (8 * k);
    } else {
      float v[kBlock];
      load_bf16_block(qbfrow + kBlock * b, v);
#pragma unroll
      for (int i = 0; i < kBlock; ++i) v[i] = v[i] * c2;
      uint4 c;
      uint8_t sc;
      mxfp4_block(v, c, sc);
      st.qa[k] = v4i{(int)c.x, (int)c.y, (int)c.z, (int)c.w};
      st.qs |= (int)sc << (8 * k);
    }
  }
  }
  if constexpr (OF) {
    ofix_zero<D / 32>();
  } else {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) st.o[cb] = v16f{};
  }
  st.m = -__builtin_inff();
  st.m_ref = -__builtin_inff();
  if constexpr (pv_of(PV) == PV_FP8) {
    st.lsum = 0.0f;
    // tile_rowsum's selector: E2M1 1.0 (0x2) in nibbles 0..15 for rows r = lane % 16
    // with bit 2 clear, in nibbles 16..31 for the others
    constexpr int e = 0x22222222;
    const bool hi = (threadIdx.x >> 2) & 1;
    st.sel = v4i{hi ? 0 : e, hi ? 0 : e, hi ? e : 0, hi ? e : 0};
    asm volatile("" : "+v"(st.sel));  // resident in VGPRs for the whole loop (no per-tile rebuild)
  } else {
    st.lv = v16f{};
    constexpr int one = PV == PV_FP4 ? 0x22222222 : 0x38383838;  // E2M1 / E4M3 1.0 in every element
    st.ones = v8i{one, one, one, one, one, one, one, one};
    asm volatile("" : "+v"(st.ones));  // resident in VGPRs for the whole loop (no per-tile rebuild)
  }
}

}  // namespace qfa
