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
// max) and the two products are pure MFMA, so each SIMD hosts two waves whose
// phases are kept opposite by workgroup barriers:
//
//   phase   wave A (rows 0..31 of a unit)     wave B (rows 32..63 of the unit)
//   2t      P V(t-1), S(t) = K(t) Q^T          softmax(t-1)
//   2t+1    softmax(t)                         P V(t-1), S(t)
//
// A workgroup is 8 waves: waves w and w+4 share SIMD w % 4 and own one unit
// (query head, 64-row block).  The 4 units of a workgroup belong to one KV
// head, so every K/V tile staged in LDS serves all of them.  K and V have
// their own double buffers: K(t+1) and V(t) are issued by the A waves in phase
// 2t (buffer_load ... lds) and waited for at the end of phase 2t+1, two phases
// before their first use.  Units are numbered head-fastest within a KV head
// (u = qb * G + head), 4 consecutive units per workgroup; workgroups run
// longest causal range first, and KV heads are pinned to XCDs (workgroup i
// runs on XCD i % 8) so a head's K/V stays in one L2.
#include "attn_common.h"

namespace qfa {

// Workgroup barrier without a memory fence: the waits the schedule needs
// (DMA completion, LDS stores) are explicit.  The scheduler does not move
// instructions across it, which keeps the two phases apart.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wait_lgkm_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

template <int D, bool COMP>
__global__ void __launch_bounds__(512) k_prefill(AttnArgs a, int nwg_per_group) {
  using TL = TileLayout<D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar control flow
  const int pair = wave & 3, half = wave >> 2;
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
  load_q<D>(st, a.q4 + qrow * (D / 2), a.q4s + qrow * (D / 32), rvalid);
  const int jlim = a.causal ? min(i + off, L - 1) : (L - 1);
  const int jmin_w = a.causal ? (i0 + off) : (L - 1);  // smallest limit over the wave's rows

  uint8_t* kbuf = smem;                 // 2 x K region
  uint8_t* vbuf = smem + 2 * TL::KREG;  // 2 x V region
  float* dl = reinterpret_cast<float*>(smem + 2 * (TL::KREG + TL::VREG)) + wave * 32 * 32;

  // Both buffer pairs start zeroed: bytes a ragged tile does not cover then hold
  // zeros or codes of an earlier tile, never uninitialised (possibly NaN) codes.
  for (int o = threadIdx.x * 16; o < 2 * (TL::KREG + TL::VREG); o += blockDim.x * 16)
    *reinterpret_cast<uint4*>(smem + o) = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  TileLoader<D, 4> ld;
  ld.init(a.k4, a.k4s, a.v8, a.v8s, (size_t)grp, L, L, pair);
  LaneOffs<D> lo;
  lo.init();
  if (half == 0 && T > 0) ld.issue_k(0, kbuf, pair);
  wait_vmem_all();
  if (wave == 0 && T > 0) {
    ld.fixup(0, kbuf);
    wait_lgkm_all();
  }
  __syncthreads();

  v8i pb[2];  // P of the last softmax, consumed by the next MFMA phase
  int pscale = kScaleOne;
  if (half == 1) phase_barrier();  // B runs one phase behind A
  for (int t = 0; t <= T; ++t) {
    // ---- MFMA phase: P V of tile t-1 and S of tile t; A waves also issue K(t+1), V(t)
    if (half == 0) {
      if (t + 1 < T) ld.issue_k(t + 1, kbuf + ((t + 1) & 1) * TL::KREG, pair);
      if (t < T) ld.issue_v(t, vbuf + (t & 1) * TL::VREG, pair);
    }
    const bool do_pv = t >= 1 && t - 1 < Tw, do_qk = t < Tw;
    v16f s[4];  // S of tile t: written here, consumed by this iteration's softmax
    if (COMP && do_qk && (t & 31) == 0)
      compute_delta<D>(dl, a.kbar + (size_t)grp * ntk * D, ntk, t, a.qbf + (((size_t)b * a.Hq + h) * Sq + i0) * D, D,
                       Sq - i0);
    // all LDS operand reads first, then the products back to back
    // (a wave's last P V also computes a product of whatever K buffer t & 1
    // holds; that S is never used: one code path keeps the register budget)
    if (do_pv) {
      pv_then_qk<D>(st, lo, vbuf + ((t - 1) & 1) * TL::VREG, pb, pscale, kbuf + (t & 1) * TL::KREG, s);
    } else if (do_qk) {
      qk_tile<D>(st, lo, kbuf + (t & 1) * TL::KREG, s);
    }
    phase_barrier();
    // ---- softmax phase of tile t; A waves then wait for the DMA issued above
    if (t < Tw) {
      const float d32 = COMP ? a.c2 * dl[(t & 31) * 32 + n] : 0.0f;
      const bool need_mask = (kTile * t + kTile - 1 > jmin_w) || (kTile * t + kTile > L);
      softmax_tile<D, COMP>(st, s, t, need_mask, jlim, d32, pb, pscale);
    }
    if (half == 0) {
      wait_vmem_all();
      if (wave == 0 && t + 1 < T) {
        ld.fixup(t + 1, kbuf + ((t + 1) & 1) * TL::KREG);
        wait_lgkm_all();
      }
    }
    phase_barrier();
  }
  if (half == 0) phase_barrier();  // A matches B's extra leading barrier

  if (rvalid) store_row<D>(st, a.O + qrow * D, a.lse ? a.lse + qrow : nullptr);
}

template <int D>
static hipError_t prefill_d(const AttnArgs& a, hipStream_t s) {
  using TL = TileLayout<D>;
  const int U = a.G * ((a.Sq + 63) / 64);
  const int nwg_per_group = (U + 3) / 4;
  const long long nwg = (long long)a.B * a.Hkv * nwg_per_group;
  if (nwg == 0) return hipSuccess;
  const bool comp = a.kbar != nullptr;
  const size_t lds = 2 * (TL::KREG + TL::VREG) + (comp ? (size_t)8 * 32 * 32 * 4 : 0);
  if (comp)
    hipLaunchKernelGGL((k_prefill<D, true>), dim3((unsigned)nwg), dim3(512), lds, s, a, nwg_per_group);
  else
    hipLaunchKernelGGL((k_prefill<D, false>), dim3((unsigned)nwg), dim3(512), lds, s, a, nwg_per_group);
  return hipGetLastError();
}

hipError_t launch_prefill(const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) return prefill_d<64>(a, s);
  if (a.D == 128) return prefill_d<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace qfa
