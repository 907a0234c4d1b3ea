// QK4PV8 prefill forward for gfx950: two waves per SIMD in ping-pong.
//
// Method ("MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on
// Blackwell GPUs", abstract): S = Q K^T / sqrt(d) on 4-bit block-scaled
// operands, online softmax (FP4 tutorial "FlashAttention压到4位", section
// "注意力慢在哪儿"), P quantised to FP8 after the softmax, O = P V on FP8
// operands with FP32 accumulation, and the rank-one smoothing compensation as
// one extra matrix product.  The per-tile steps live in attn_common.h.
//
// Schedule.  On gfx950 a wave's MFMA and VALU instructions do not overlap each
// other, but an MFMA of one wave runs alongside VALU work of another wave on
// the same SIMD.  The softmax of a tile is pure VALU (exp, FP8 conversion,
// max) and the two products are pure MFMA, so each SIMD hosts two waves that
// run the same loop -- products of tile t (P V(t-1), S(t) = K(t) Q^T), then
// the softmax of tile t -- half an iteration apart.  One workgroup barrier per
// iteration keeps them there: wave A (rows 0..31 of a unit) arrives after its
// softmax, wave B (rows 32..63) after its products, so between two barriers
//
//   wave A:  products(t+1)   softmax(t+1)
//   wave B:  softmax(t)      products(t+1)
//
// and each side may run ahead into its second half while the other finishes
// its first.  The products run at raised issue priority, so an MFMA issues as
// soon as the matrix unit is free and the VALU work of the other wave fills
// the gaps.
//
// A workgroup is 8 waves: waves w and w+4 share SIMD w % 4 and own one unit
// (query head, 64-row block).  The 4 units of a workgroup belong to one KV
// head, so every K/V tile staged in LDS serves all of them.  K and V tiles
// rotate through three LDS buffers each: in the window between barriers j-1
// and j the products read K(j) and V(j-1), and the A waves issue K(j+2) and
// V(j+1) (buffer_load ... lds), which must land by barriers j+1 and j+1; the
// buffer each overwrites was last read two windows earlier.  Units are
// numbered head-fastest within a KV head (u = qb * G + head), 4 consecutive
// units per workgroup; workgroups run longest causal range first, and KV heads
// are pinned to XCDs (workgroup i runs on XCD i % 8) so a head's K/V stays in
// one L2.
#include "attn_common.h"

namespace qfa {

#ifndef QFA_PREFILL_BUFFERS
#define QFA_PREFILL_BUFFERS 3
#endif
constexpr int kPrefillBuffers = QFA_PREFILL_BUFFERS;
static_assert(kPrefillBuffers == 3 || kPrefillBuffers == 4, "3 or 4 LDS buffers per operand");

__device__ __forceinline__ void wait_lgkm_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// vmcnt(n) for a wave-uniform n in [0, 16]: waits until at most n of this
// wave's vector-memory loads are outstanding.
__device__ __forceinline__ void wait_vmem_le(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    case 15: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
    default: __builtin_amdgcn_s_waitcnt(0x4F70); break;  // 16: vmcnt bits 5:4 live in simm16 bits 15:14
  }
}

// Workgroup barrier without a memory fence: the waits the schedule needs
// (DMA completion, LDS stores) are explicit.  The scheduler does not move
// instructions across it.
__device__ __forceinline__ void window_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool COMP, int PV>
__global__ void __launch_bounds__(512) k_prefill(AttnArgs a, int nwg_per_group) {
  using TL = TileLayout<D, PV>;
  constexpr int NB = kPrefillBuffers;  // LDS buffers per operand
  // O^T in the fixed accumulation registers (attn_common.h, ofix_*): the
  // method's kernel without the compensation, the one whose register budget
  // leaves the compiler no reason to allocate accumulation registers itself
  constexpr bool OF = !COMP && PV == PV_FP8;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar control flow
  // half 0 (rows 0..31 of a unit) runs products then softmax in a window,
  // half 1 (rows 32..63) softmax then products.  Waves 0..3 (the older wave of
  // each SIMD) take half 1.  Measured on MI355X: the products of the younger
  // wave of a SIMD can run up to twice as long beside the older wave's
  // softmax, whatever the issue priorities, and this assignment is about 3%
  // faster than the reverse one.
  const int pair = wave & 3, half = 1 - (wave >> 2);
  const int n = lane & 31;

  // ---- workgroup -> (KV group, rank): longest first, groups pinned to XCDs
  const int ngroups = a.B * a.Hkv;
  const int x = blockIdx.x;
  int grp, rank;
  if ((ngroups & 7) == 0) {
    const int xcd = x & 7, slot = x >> 3, gpx = ngroups >> 3;
    rank = slot / gpx;
    grp = xcd + 8 * (slot % gpx);
  } else {
    rank = x / ngroups;
    grp = x % ngroups;
  }
  const int b = grp / a.Hkv, gk = grp % a.Hkv;
  const int wg_local = a.causal ? (nwg_per_group - 1 - rank) : rank;
  const int G = a.G, Sq = a.Sq, L = a.Skv, off = L - Sq;
  const int U = G * ((Sq + 63) / 64);  // units of this KV group
  const int u = 4 * wg_local + pair;
  const bool unit_valid = u < U;
  const int qb = unit_valid ? u / G : 0;
  const int h = gk * G + (unit_valid ? u % G : 0);
  const int i0 = 64 * qb + 32 * half;  // first row of this wave
  const bool wave_active = unit_valid && i0 < Sq;

  // ---- tile ranges: the workgroup's (union over its units) and this wave's
  const int ntk = (L + kTile - 1) / kTile;
  const int u_last = min(4 * wg_local + 3, U - 1);
  int T = ntk, Tw = 0;
  if (a.causal) {
    const int jl = min(64 * (u_last / G) + 63, Sq - 1) + off;
    T = jl < 0 ? 0 : min(ntk, jl / kTile + 1);
  }
  if (wave_active) {
    Tw = ntk;
    if (a.causal) {
      const int jl = min(i0 + 31, Sq - 1) + off;
      Tw = jl < 0 ? 0 : min(ntk, jl / kTile + 1);
    }
  }

  // ---- per-wave row state
  RowState<D> st;
  const int i = i0 + n;
  const bool rvalid = wave_active && i < Sq;
  const size_t qrow = ((size_t)b * a.Hq + h) * Sq + (rvalid ? i : 0);
  const int jlim = a.causal ? min(i + off, L - 1) : (L - 1);
  const int jmin_w = a.causal ? (i0 + off) : (L - 1);  // smallest limit over the wave's rows

  uint8_t* kbuf = smem;                                   // NB x K region
  uint8_t* vbuf = smem + NB * TL::KREG;                   // NB x V region
  uint8_t* trash = smem + NB * (TL::KREG + TL::VREG);     // 1 KB sink of unused DMA slots
  float* dl = reinterpret_cast<float*>(trash + 1024) + wave * 32 * 32;

  // Every byte a tile step reads is written by that tile's DMA first, and the
  // DMA writes zeros for the lanes its range check cuts off, so a ragged tile
  // reads zeros without this (the decode relies on exactly that).  The buffers
  // are zeroed once anyway, at about 0.3% of the kernel's time, so that a
  // byte read outside the DMA's coverage could only ever be zero, never a
  // leftover NaN code.
  for (int o = threadIdx.x * 16; o < NB * (TL::KREG + TL::VREG); o += blockDim.x * 16)
    *reinterpret_cast<uint4*>(smem + o) = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  TileLoader<D, 8, PV> ld;  // all 8 waves share the DMA
  ld.init(a.k4, a.k4s, a.v8, a.v8s, (size_t)grp, L, L, wave);
  LaneOffs<D, PV> lo;
  lo.init();
  constexpr int SLOTS = TileLoader<D, 8, PV>::SLOTS;  // code DMA instructions per wave and window
  // K(0 .. NB-2), V(0 .. NB-3) before the loop; Q (and its quantisation)
  // while they are in flight
  for (int j = 0; j < NB - 1 && j < T; ++j) ld.issue_k(j, kbuf + j * TL::KREG, wave);
  for (int j = 0; j < NB - 2 && j < T; ++j) ld.issue_v(j, vbuf + j * TL::VREG, wave);
  load_q<D, PV, OF>(st, a.q4 ? a.q4 + qrow * (D / 2) : nullptr, a.q4 ? a.q4s + qrow * TileLayout<D, PV>::KSB : nullptr,
                a.qbf ? a.qbf + qrow * D : nullptr, a.c2, rvalid, a.nv_gq, a.nv_gk);
  wait_vmem_le(0);
  __syncthreads();  // every wave's loads have landed before the scale patch
  if (wave == 0) {
    for (int j = 0; j < NB - 1 && j < T; ++j) ld.fixup(j, kbuf + j * TL::KREG);
    wait_lgkm_all();
  }
  __syncthreads();

  POp<PV> pb[2];  // P of the last softmax, consumed by the next products
  int pscale[2] = {kScaleOne, kScaleOne};
  int kb_cur = 0, vb_prev = NB - 1;  // buffer of K(t) and of V(t-1)
#pragma nounroll
  for (int t = 0; t <= T; ++t) {
    // ---- DMA of K(t+NB-1) and V(t+NB-2) into the buffers last read in the
    // previous window (tile j lives in buffer j % NB): one load per MFMA step
    // of the products, the same count on every wave (one scale slot, then the
    // code slots)
    const bool dk = t + NB - 1 < T, dv = t + NB - 2 < T;
    uint8_t* kdst = kbuf + (kb_cur == 0 ? NB - 1 : kb_cur - 1) * TL::KREG;
    int vb2 = vb_prev + NB - 1;
    vb2 -= vb2 >= NB ? NB : 0;
    uint8_t* vdst = vbuf + vb2 * TL::VREG;
    constexpr int issued = SLOTS + 1;  // loads per wave and window: the code slots and one scale slot
    auto dma = [&](int k) {
      if (k == 0)
        ld.scale_slot(t + NB - 1, kdst, dk, t + NB - 2, vdst, dv, wave, trash);
      else if (k <= SLOTS)
        ld.dma_slot(k - 1, t + NB - 1, kdst, dk, t + NB - 2, vdst, dv, wave, trash);
    };
    // ---- products of tile t at raised priority: P V(t-1), then S(t) = K(t) Q^T
    const bool do_pv = t >= 1 && t - 1 < Tw, do_qk = t < Tw;
    v16f s[4];  // S of tile t: written here, consumed by this iteration's softmax
    if (COMP && do_qk && (t & 31) == 0)
      compute_delta<D>(dl, a.kbar + (size_t)grp * ntk * D, Tw, t, a.qbf + (((size_t)b * a.Hq + h) * Sq + i0) * D, D,
                       Sq - i0);
    // The compensation offset d = fl32(c2 fl32(delta)) of this lane's row and
    // tile starts the S accumulator (offset_block), so the exponent argument
    // y = fl32(fl32(d + S'_0) + S'_1) (S'_k: the exact partial product of
    // MFMA k) needs no add per score.  (NVFP4 Q/K, a contrast format on the
    // bf16 MFMA, keeps the add: its register budget has no room for the
    // start value.)
    constexpr bool SEED = COMP && PV != QK_NVFP4;
    v16f init = v16f{};
    if (SEED) init = offset_block(a.c2 * dl[(t & 31) * 32 + n]);
    __builtin_amdgcn_s_setprio(2);
    // (a wave's last P V also computes a product of whatever K buffer kb_cur
    // holds; that S is never used: one code path keeps the register budget)
    if (do_pv) {
      pv_then_qk<D, PV, decltype(dma), SEED, OF>(st, lo, vbuf + vb_prev * TL::VREG, pb, pscale, kbuf + kb_cur * TL::KREG,
                                             s, init, dma);
    } else {
#pragma unroll
      for (int k = 0; k <= SLOTS; ++k) dma(k);
      if (do_qk) qk_tile<D, PV>(st, lo, kbuf + kb_cur * TL::KREG, s, init);
    }
    __builtin_amdgcn_s_setprio(0);
    // ---- end of this wave's window: its loads of K(t+1) and V(t) (issued
    // NB-2 windows ago) have landed, the K-scale patch of K(t+1) is written
    // by the wave that loaded those scales, then the barrier
    auto end_window = [&]() {
      wait_vmem_le((NB - 2) * issued);
      if (wave == 0 && t + 1 < T) {
        ld.fixup(t + 1, kbuf + (kb_cur + 1 == NB ? 0 : kb_cur + 1) * TL::KREG);
        wait_lgkm_all();
      }
      window_barrier();
    };
    if (half == 1) end_window();
    // ---- softmax of tile t
    if (t < Tw) {
      const float d32 = (COMP && !SEED) ? a.c2 * dl[(t & 31) * 32 + n] : 0.0f;
      const bool need_mask = (kTile * t + kTile - 1 > jmin_w) || (kTile * t + kTile > L);
      softmax_tile<D, COMP && !SEED, PV, OF>(st, s, t, need_mask, jlim, d32, pb, pscale);
    }
    if (half == 0) end_window();
    kb_cur = kb_cur + 1 == NB ? 0 : kb_cur + 1;
    vb_prev = vb_prev + 1 == NB ? 0 : vb_prev + 1;
  }

  if (rvalid) store_row<D, PV, OF>(st, a.O + qrow * D, a.lse ? a.lse + qrow : nullptr);
}

template <int D, int PV>
static hipError_t prefill_dp(const AttnArgs& a, hipStream_t s) {
  using TL = TileLayout<D, PV>;
  const int U = a.G * ((a.Sq + 63) / 64);
  const int nwg_per_group = (U + 3) / 4;
  const long long nwg = (long long)a.B * a.Hkv * nwg_per_group;
  if (nwg == 0) return hipSuccess;
  const bool comp = a.kbar != nullptr;
  const size_t lds = kPrefillBuffers * (TL::KREG + TL::VREG) + 1024 + (comp ? (size_t)8 * 32 * 32 * 4 : 0);
  if (comp)
    hipLaunchKernelGGL((k_prefill<D, true, PV>), dim3((unsigned)nwg), dim3(512), lds, s, a, nwg_per_group);
  else
    hipLaunchKernelGGL((k_prefill<D, false, PV>), dim3((unsigned)nwg), dim3(512), lds, s, a, nwg_per_group);
  return hipGetLastError();
}

template <int D>
static hipError_t prefill_d(const AttnArgs& a, hipStream_t s) {
  switch (a.pv) {
    case PV_FP8: return prefill_dp<D, PV_FP8>(a, s);
    case PV_FP8_BLOCKP: return prefill_dp<D, PV_FP8_BLOCKP>(a, s);
    case PV_FP4: return prefill_dp<D, PV_FP4>(a, s);
    case QK_NVFP4: return prefill_dp<D, QK_NVFP4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) return prefill_d<64>(a, s);
  if (a.D == 128) return prefill_d<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace qfa
