// QK4PV8 split-KV decode for gfx950: per-split partials and the log-sum-exp merge.
//
// Method ("MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on
// Blackwell GPUs", abstract: prefill and decode, adaptive partitioning).  One
// query token per sequence; the Hq/Hkv query heads of a KV head form the 32
// MFMA rows of one wave, so the KV cache is read once per KV head.  A split is
// a contiguous run of whole 128-key tiles; its normalised partial O and its
// LSE go to the caller's workspace, and k_decode_merge combines them:
// LSE = log sum_s e^{LSE_s},  O = sum_s e^{LSE_s - LSE} O_s.  The tile loop is
// the same three steps as the prefill (attn_common.h), over a ring of two or
// three LDS tiles (decode_ring).
#include "attn_common.h"

namespace qfa {

// LDS tile ring of the decode: three tiles (two workgroups per CU) for the
// E4M3-V formats, two (three or more per CU) for MXFP4 V and NVFP4 Q/K, whose
// decodes need the extra workgroups.  Measured on MI355X with the B64 x 32768
// decode: 3 tiles 0.760 / 2 tiles 0.754 of 8 TB/s for the method, 0.671 / 0.714
// for MXFP4 V, 0.623 / 0.729 for NVFP4 Q/K.
template <int PV>
constexpr int decode_ring() { return (PV == PV_FP8 || PV == PV_FP8_BLOCKP) ? 3 : 2; }

// Decode: workgroup = one wave = (b, kv head g, row chunk rc, split s); lane row n
// = query head g*G + 32*rc + n.  Writes normalised partials to the workspace.
template <int D, bool COMP, int PV>
__global__ void __launch_bounds__(64) k_decode_split(AttnArgs a, int nrc) {
  using TL = TileLayout<D, PV>;
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
  load_q<D, PV>(st, a.q4 ? a.q4 + qrow * (D / 2) : nullptr, a.q4 ? a.q4s + qrow * TileLayout<D, PV>::KSB : nullptr,
                a.qbf ? a.qbf + qrow * D : nullptr, a.c2, rvalid, a.nv_gq, a.nv_gk);

  // (no zeroing of the tile buffers: every byte a tile step reads is written by
  // that tile's DMA first, and the DMA writes zeros for the lanes its range
  // check cuts off -- measured on MI355X -- so a ragged tile reads zeros)
  constexpr int NBD = decode_ring<PV>();  // tile t lives in buffer t % NBD
  uint8_t* bufs = smem;
  float* dl = reinterpret_cast<float*>(smem + NBD * TL::STRIDE);
  TileLoader<D, 1, PV, kCpolNT> ld;  // each cached byte is read once: non-temporal loads
  ld.init(a.k4, a.k4s, a.v8, a.v8s, (size_t)bg, Lmax, L, 0);
  LaneOffs<D, PV> lo;
  lo.init();
  auto buf_of = [&](int t) { return bufs + (unsigned)t % NBD * TL::STRIDE; };
  // tiles t0 .. t0+NBD-2 in flight before the loop; then tile t+NBD-1 is
  // issued while tile t is computed, into the buffer tile t-1 used
  for (int j = t0; j < t0 + NBD - 1 && j < t1; ++j) {
    ld.issue_k(j, buf_of(j), 0);
    ld.issue_v(j, buf_of(j) + TL::V_OFF, 0);
  }
  wait_vmem_all();
  for (int j = t0; j < t0 + NBD - 1 && j < t1; ++j) ld.fixup(j, buf_of(j));
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    if (t + NBD - 1 < t1) {
      ld.issue_k(t + NBD - 1, buf_of(t + NBD - 1), 0);
      ld.issue_v(t + NBD - 1, buf_of(t + NBD - 1) + TL::V_OFF, 0);
    }
    float d32 = 0.0f;
    if (COMP) {
      if (t == t0 || (t & 31) == 0)
        compute_delta<D>(dl, a.kbar + (size_t)bg * ntk_max * D, t1, t & ~31,
                         a.qbf + ((size_t)b * a.Hq + gk * a.G + 32 * rc) * D, D, a.G - 32 * rc);
      d32 = a.c2 * dl[(t & 31) * 32 + n];
    }
    uint8_t* buf = buf_of(t);
    v16f s[4];
    POp<PV> pb[2];
    int pscale[2];
    // the compensation offset starts the S accumulator, as in the prefill
    // (NVFP4 Q/K keeps the add per score)
    constexpr bool SEED = COMP && PV != QK_NVFP4;
    v16f init = v16f{};
    if (SEED) init = offset_block(d32);
    qk_tile<D, PV>(st, lo, buf, s, init);
    softmax_tile<D, COMP && !SEED, PV>(st, s, t, kTile * t + kTile > L, L - 1, d32, pb, pscale);
    pv_tile<D, PV>(st, lo, buf + TL::V_OFF, pb, pscale);
    // tile t+1 has landed once only the loads of tile t+2 (issued this
    // iteration, NBD = 3) may still be outstanding
    if (NBD == 3 && t + 2 < t1) {
      static_assert(TL::NINS <= 63, "vmcnt field");
      __builtin_amdgcn_s_waitcnt((TL::NINS & 15) | 0x0F70 | ((TL::NINS >> 4) << 14));
    } else {
      wait_vmem_all();
    }
    if (t + 1 < t1) ld.fixup(t + 1, buf_of(t + 1));
    __syncthreads();
  }
  if (!rvalid) return;
  const size_t prow = ((size_t)b * a.Hq + h) * S + s;
  store_row<D, PV>(st, a.O + prow * D, a.lse + prow);
}

// LSE merge: one wave per (b, h) row.  LSE = log sum_s e^{LSE_s};  O = sum_s e^{LSE_s - LSE} O_s.
// Lane s holds split s's LSE and weight (64 splits per pass, broadcast by
// readlane); the partial-O loads of eight splits are issued together, so
// their latencies overlap.
template <int D>
__global__ void __launch_bounds__(256) k_decode_merge(const float* __restrict__ Op, const float* __restrict__ Lp,
                                                      int rows, int S, float* __restrict__ O, float* __restrict__ lse) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* lp = Lp + (size_t)row * S;
  const float* op = Op + (size_t)row * S * D;
  float mx = -__builtin_inff();
  for (int s0 = 0; s0 < S; s0 += 64)
    if (s0 + lane < S) mx = __builtin_fmaxf(mx, lp[s0 + lane]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
  float acc[D / 64];
#pragma unroll
  for (int k = 0; k < D / 64; ++k) acc[k] = 0.0f;
  float den = 0.0f;
  if (mx != -__builtin_inff()) {
    for (int s0 = 0; s0 < S; s0 += 64) {
      const int ns = min(64, S - s0);
      const float w = lane < ns ? __expf(lp[s0 + lane] - mx) : 0.0f;
      den += w;
      int s = 0;
      for (; s + 8 <= ns; s += 8) {
        float v[8][D / 64], ws[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          ws[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s + j));
#pragma unroll
          for (int k = 0; k < D / 64; ++k) v[j][k] = op[(size_t)(s0 + s + j) * D + 64 * k + lane];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int k = 0; k < D / 64; ++k) acc[k] += ws[j] * v[j][k];
      }
      for (; s < ns; ++s) {
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
#pragma unroll
        for (int k = 0; k < D / 64; ++k) acc[k] += ws * op[(size_t)(s0 + s) * D + 64 * k + lane];
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
  }
  const float inv = (den > 0.0f) ? 1.0f / den : 0.0f;
#pragma unroll
  for (int k = 0; k < D / 64; ++k) O[(size_t)row * D + 64 * k + lane] = acc[k] * inv;
  if (lse && lane == 0) lse[row] = (den > 0.0f) ? mx + __logf(den) : -__builtin_inff();
}

template <int D, int PV>
static hipError_t decode_dp(const AttnArgs& a, float* O, float* lse, hipStream_t s) {
  using TL = TileLayout<D, PV>;
  const int nrc = (a.G + 31) / 32;
  const long long nwg = (long long)a.B * a.Hkv * nrc * a.num_splits;
  if (nwg == 0) return hipSuccess;
  const bool comp = a.kbar != nullptr;
  const size_t lds = decode_ring<PV>() * TL::STRIDE + (comp ? 32 * 32 * 4 : 0);
  if (comp)
    hipLaunchKernelGGL((k_decode_split<D, true, PV>), dim3((unsigned)nwg), dim3(64), lds, s, a, nrc);
  else
    hipLaunchKernelGGL((k_decode_split<D, false, PV>), dim3((unsigned)nwg), dim3(64), lds, s, a, nrc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = a.B * a.Hq;
  hipLaunchKernelGGL(k_decode_merge<D>, dim3((rows + 3) / 4), dim3(256), 0, s, a.O, a.lse, rows, a.num_splits, O,
                     lse);
  return hipGetLastError();
}

template <int D>
static hipError_t decode_d(const AttnArgs& a, float* O, float* lse, hipStream_t s) {
  switch (a.pv) {
    case PV_FP8: return decode_dp<D, PV_FP8>(a, O, lse, s);
    case PV_FP8_BLOCKP: return decode_dp<D, PV_FP8_BLOCKP>(a, O, lse, s);
    case PV_FP4: return decode_dp<D, PV_FP4>(a, O, lse, s);
    case QK_NVFP4: return decode_dp<D, QK_NVFP4>(a, O, lse, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const AttnArgs& a, float* O, float* lse, hipStream_t s) {
  if (a.D == 64) return decode_d<64>(a, O, lse, s);
  if (a.D == 128) return decode_d<128>(a, O, lse, s);
  return hipErrorInvalidValue;
}

}  // namespace qfa
