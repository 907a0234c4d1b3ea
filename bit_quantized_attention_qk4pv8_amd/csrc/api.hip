// extern "C" entry points of libqfa: argument validation on the host, then
// kernel launches on the caller's stream.  See include/qfa.h for the contract.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/qfa.h"
#include "qfa_internal.h"

// Decode partials of qfa_fwd_decode_noalloc: one array per GPU, kept until the
// process ends.  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress (scratch_on_current_device).
static __device__ __align__(256) uint8_t scratch[QFA_DECODE_NOALLOC_MAX_BYTES];

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool qk_dim_ok(int D) { return D >= 32 && D <= 256 && D % 32 == 0; }
bool attn_dim_ok(int D) { return D == 64 || D == 128; }

qfa_status from_hip(hipError_t e) { return e == hipSuccess ? QFA_OK : QFA_ERR_HIP; }

// log2(e) rounded to binary32; the kernels form the exponent argument from
// c2 = fl32(softmax_scale * log2e).
constexpr float kLog2e = 1.44269502162933349609375f;

size_t ws_bytes(int B, int Hq, int D, int splits) {
  const size_t rows = (size_t)B * Hq * splits;
  size_t o = rows * D * sizeof(float);
  o = (o + 255) / 256 * 256;
  return o + (rows * sizeof(float) + 255) / 256 * 256;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, resolved once

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with that device current).
qfa_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QFA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return QFA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QFA_OK;
}

}  // namespace

extern "C" {

const char* qfa_status_string(qfa_status status) {
  switch (status) {
    case QFA_OK: return "QFA_OK";
    case QFA_ERR_INVALID_ARG: return "QFA_ERR_INVALID_ARG";
    case QFA_ERR_UNSUPPORTED: return "QFA_ERR_UNSUPPORTED";
    case QFA_ERR_WORKSPACE: return "QFA_ERR_WORKSPACE";
    case QFA_ERR_HIP: return "QFA_ERR_HIP";
  }
  return "QFA_ERR_UNKNOWN";
}

int qfa_version(void) { return kVersion; }

float qfa_exp2_scale(float softmax_scale) { return softmax_scale * kLog2e; }

qfa_status qfa_quantize_qk4(const uint16_t* x, int B, int H, int S, int D, int block_size, int smooth,
                            float prescale, uint8_t* codes, uint8_t* scales, uint16_t* kbar, hipStream_t stream) {
  if (block_size != 32 || !qk_dim_ok(D)) return QFA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || S < 0 || (long long)B * H > 65535) return QFA_ERR_INVALID_ARG;
  if (smooth != 0 && smooth != 1) return QFA_ERR_INVALID_ARG;
  if (!(prescale > 0.0f) || !isfinite(prescale)) return QFA_ERR_INVALID_ARG;
  if ((smooth == 1) != (kbar != nullptr)) return QFA_ERR_INVALID_ARG;
  if ((long long)B * H * S == 0) return QFA_OK;
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)) return QFA_ERR_INVALID_ARG;
  if (kbar && !aligned16(kbar)) return QFA_ERR_INVALID_ARG;
  return from_hip(qfa::launch_quant_qk4(x, B, H, S, D, smooth, prescale, codes, scales, kbar, stream));
}

qfa_status qfa_quantize_v8(const uint16_t* v, int B, int H, int S, int D, int block_size, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream) {
  if (block_size != 32 || !qk_dim_ok(D)) return QFA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || S < 0 || (long long)B * H > 65535) return QFA_ERR_INVALID_ARG;
  if ((long long)B * H * S == 0) return QFA_OK;
  if (!v || !codes || !scales || !aligned16(v) || !aligned16(codes)) return QFA_ERR_INVALID_ARG;
  return from_hip(qfa::launch_quant_v8(v, B, H, S, D, codes, scales, stream));
}

// a positive, finite power of two (the per-tensor NVFP4 scale)
static bool pow2_ok(float g) {
  if (!(g > 0.0f) || !isfinite(g)) return false;
  int e;
  return frexpf(g, &e) == 0.5f;
}

qfa_status qfa_quantize_nvfp4(const uint16_t* x, int B, int H, int S, int D, int block_size, int smooth,
                              float prescale, float tensor_scale, uint8_t* codes, uint8_t* scales, uint16_t* kbar,
                              hipStream_t stream) {
  if (block_size != 16 || !qk_dim_ok(D)) return QFA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || S < 0 || (long long)B * H > 65535) return QFA_ERR_INVALID_ARG;
  if (smooth != 0 && smooth != 1) return QFA_ERR_INVALID_ARG;
  if ((smooth != 0) != (kbar != nullptr)) return QFA_ERR_INVALID_ARG;
  if (!(prescale > 0.0f) || !isfinite(prescale) || !pow2_ok(tensor_scale)) return QFA_ERR_INVALID_ARG;
  if ((long long)B * H * S == 0) return QFA_OK;
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)) return QFA_ERR_INVALID_ARG;
  if (kbar && !aligned16(kbar)) return QFA_ERR_INVALID_ARG;
  return from_hip(qfa::launch_quant_nvfp4(x, B, H, S, D, smooth, prescale, tensor_scale, codes, scales, kbar, stream));
}

qfa_status qfa_quantize_v4(const uint16_t* v, int B, int H, int S, int D, int block_size, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream) {
  if (block_size != 32 || !qk_dim_ok(D)) return QFA_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || S < 0 || (long long)B * H > 65535) return QFA_ERR_INVALID_ARG;
  if ((long long)B * H * S == 0) return QFA_OK;
  if (!v || !codes || !scales || !aligned16(v) || !aligned16(codes)) return QFA_ERR_INVALID_ARG;
  return from_hip(qfa::launch_quant_v4(v, B, H, S, D, codes, scales, stream));
}

static qfa_status check_attn_common(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                                    const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8,
                                    const uint8_t* v8s, int B, int Hq, int Hkv, int D, float softmax_scale,
                                    int block_size, const float* O) {
  if (block_size != 32 || !attn_dim_ok(D)) return QFA_ERR_UNSUPPORTED;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return QFA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return QFA_ERR_INVALID_ARG;
  // Q comes quantised (q4 and q4s) or as bf16 to be quantised in the kernel
  // (both null, q_bf16 set); the compensation (kbar) also needs q_bf16.
  if ((q4 == nullptr) != (q4s == nullptr)) return QFA_ERR_INVALID_ARG;
  if ((q4 == nullptr || kbar != nullptr) && q_bf16 == nullptr) return QFA_ERR_INVALID_ARG;
  const void* ptrs[] = {k4, v8, O};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return QFA_ERR_INVALID_ARG;
  if (!k4s || !v8s) return QFA_ERR_INVALID_ARG;
  if (q4 && !aligned16(q4)) return QFA_ERR_INVALID_ARG;
  if (q_bf16 && !aligned16(q_bf16)) return QFA_ERR_INVALID_ARG;
  if (kbar && !aligned16(kbar)) return QFA_ERR_INVALID_ARG;
  return QFA_OK;
}

static qfa_status check_pv_format(int pv_format) {
  if (pv_format == QFA_PV_FP8 || pv_format == QFA_PV_FP8_BLOCKP || pv_format == QFA_PV_FP4) return QFA_OK;
  return QFA_ERR_INVALID_ARG;
}

qfa_status qfa_fwd_prefill(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                           const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                           int B, int Hq, int Hkv, int S_q, int S_kv, int D, int causal, float softmax_scale,
                           int block_size, float* O, float* lse, hipStream_t stream) {
  return qfa_fwd_prefill_ex(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_q, S_kv, D, causal,
                            softmax_scale, block_size, QFA_PV_FP8, O, lse, stream);
}

qfa_status qfa_fwd_prefill_ex(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                              const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                              int B, int Hq, int Hkv, int S_q, int S_kv, int D, int causal, float softmax_scale,
                              int block_size, int pv_format, float* O, float* lse, hipStream_t stream) {
  if (S_q < 0 || S_kv < 0 || (causal != 0 && causal != 1)) return QFA_ERR_INVALID_ARG;
  if (qfa_status f = check_pv_format(pv_format); f != QFA_OK) return f;
  if ((long long)B * Hq * S_q == 0) return QFA_OK;
  qfa_status st = check_attn_common(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, D, softmax_scale,
                                    block_size, O);
  if (st != QFA_OK) return st;
  const long long nq = (S_q + 31) / 32;
  const int G = Hq / Hkv;
  const long long nwg = (long long)B * Hkv * ((G + 7) / 8) * nq;
  if (nwg > 0x7FFFFFFFLL) return QFA_ERR_INVALID_ARG;
  qfa::AttnArgs a{};
  a.q4 = q4; a.q4s = q4s; a.k4 = k4; a.k4s = k4s; a.v8 = v8; a.v8s = v8s;
  a.kbar = kbar; a.qbf = q_bf16; a.kv_lens = nullptr;
  a.O = O; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = S_q; a.Skv = S_kv; a.D = D; a.G = G;
  a.causal = causal;
  a.c2 = softmax_scale * kLog2e;
  a.num_splits = 1;
  a.pv = pv_format;
  return from_hip(qfa::launch_prefill(a, stream));
}

qfa_status qfa_fwd_prefill_nvfp4(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                                 const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                                 int B, int Hq, int Hkv, int S_q, int S_kv, int D, int causal, float softmax_scale,
                                 float q_tensor_scale, float k_tensor_scale, float* O, float* lse, hipStream_t stream) {
  if (S_q < 0 || S_kv < 0 || (causal != 0 && causal != 1)) return QFA_ERR_INVALID_ARG;
  if (!pow2_ok(q_tensor_scale) || !pow2_ok(k_tensor_scale)) return QFA_ERR_INVALID_ARG;
  if ((long long)B * Hq * S_q == 0) return QFA_OK;
  if (!q4 || !q4s) return QFA_ERR_INVALID_ARG;  // NVFP4 Q comes quantised
  qfa_status st = check_attn_common(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, D, softmax_scale, 32, O);
  if (st != QFA_OK) return st;
  const long long nq = (S_q + 31) / 32;
  const int G = Hq / Hkv;
  const long long nwg = (long long)B * Hkv * ((G + 7) / 8) * nq;
  if (nwg > 0x7FFFFFFFLL) return QFA_ERR_INVALID_ARG;
  qfa::AttnArgs a{};
  a.q4 = q4; a.q4s = q4s; a.k4 = k4; a.k4s = k4s; a.v8 = v8; a.v8s = v8s;
  a.kbar = kbar; a.qbf = q_bf16; a.kv_lens = nullptr;
  a.O = O; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = S_q; a.Skv = S_kv; a.D = D; a.G = G;
  a.causal = causal;
  a.c2 = softmax_scale * kLog2e;
  a.num_splits = 1;
  a.pv = qfa::QK_NVFP4;
  a.nv_gq = q_tensor_scale;
  a.nv_gk = k_tensor_scale;
  return from_hip(qfa::launch_prefill(a, stream));
}

qfa_status qfa_kv_append(const uint16_t* k_new, const uint16_t* v_new, int B, int Hkv, int n_new, int D,
                         int S_kv_max, int block_size, const int32_t* kv_lens, uint8_t* k4, uint8_t* k4s,
                         uint16_t* kbar, uint8_t* v8, uint8_t* v8s, uint16_t* k_tail, uint16_t* v_tail,
                         hipStream_t stream) {
  return qfa_kv_append_ex(k_new, v_new, B, Hkv, n_new, D, S_kv_max, block_size, kv_lens, k4, k4s, kbar, v8, v8s,
                          k_tail, v_tail, QFA_PV_FP8, 0.0f, stream);
}

qfa_status qfa_kv_append_ex(const uint16_t* k_new, const uint16_t* v_new, int B, int Hkv, int n_new, int D,
                            int S_kv_max, int block_size, const int32_t* kv_lens, uint8_t* k4, uint8_t* k4s,
                            uint16_t* kbar, uint8_t* v8, uint8_t* v8s, uint16_t* k_tail, uint16_t* v_tail,
                            int pv_format, float k_tensor_scale, hipStream_t stream) {
  if (block_size != 32 || !qk_dim_ok(D)) return QFA_ERR_UNSUPPORTED;
  if (qfa_status f = check_pv_format(pv_format); f != QFA_OK) return f;
  if (k_tensor_scale != 0.0f && !pow2_ok(k_tensor_scale)) return QFA_ERR_INVALID_ARG;
  if (B < 0 || Hkv < 0 || n_new < 0 || S_kv_max < 0 || (long long)B * Hkv > 65535) return QFA_ERR_INVALID_ARG;
  if ((kbar == nullptr) != (k_tail == nullptr)) return QFA_ERR_INVALID_ARG;
  if ((long long)B * Hkv * n_new == 0 || S_kv_max == 0) return QFA_OK;
  const void* ptrs[] = {k_new, v_new, k4, v8, v_tail};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return QFA_ERR_INVALID_ARG;
  if (!k4s || !v8s) return QFA_ERR_INVALID_ARG;
  if (kbar && (!aligned16(kbar) || !aligned16(k_tail))) return QFA_ERR_INVALID_ARG;
  qfa::AppendArgs a{};
  a.k_new = k_new; a.v_new = v_new; a.kv_lens = kv_lens;
  a.k4 = k4; a.k4s = k4s; a.kbar = kbar; a.v8 = v8; a.v8s = v8s;
  a.k_tail = k_tail; a.v_tail = v_tail;
  a.B = B; a.Hkv = Hkv; a.n = n_new; a.S = S_kv_max;
  a.v_fp4 = pv_format == QFA_PV_FP4;
  a.k_nv_g = k_tensor_scale;
  return from_hip(qfa::launch_kv_append(a, D, stream));
}

int qfa_decode_default_splits(int B, int Hkv, int S_kv_max) {
  const long long units = (long long)(B > 0 ? B : 1) * (Hkv > 0 ? Hkv : 1);
  const int tiles = S_kv_max > 0 ? (S_kv_max + 127) / 128 : 1;
  const long long target = 8LL * 256;  // several work units for each of the 256 compute units
  long long s = (target + units - 1) / units;
  if (s > tiles) s = tiles;
  if (s > 256) s = 256;
  return s < 1 ? 1 : (int)s;
}

size_t qfa_decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
  if (B <= 0 || Hq <= 0 || D <= 0 || num_splits <= 0) return 0;
  return ws_bytes(B, Hq, D, num_splits);
}

qfa_status qfa_fwd_decode(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                          const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                          int B, int Hq, int Hkv, int S_kv_max, const int32_t* kv_lens, int D,
                          float softmax_scale, int block_size, int* num_splits, void* workspace,
                          size_t workspace_bytes, float* O, float* lse, hipStream_t stream) {
  return qfa_fwd_decode_ex(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D,
                           softmax_scale, block_size, QFA_PV_FP8, num_splits, workspace, workspace_bytes, O, lse,
                           stream);
}

static qfa_status decode_common(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                                const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                                int B, int Hq, int Hkv, int S_kv_max, const int32_t* kv_lens, int D,
                                float softmax_scale, int block_size, int fmt, float gq, float gk, int* num_splits,
                                void* workspace, size_t workspace_bytes, float* O, float* lse, hipStream_t stream) {
  if (!num_splits || S_kv_max < 0 || *num_splits < 0 || *num_splits > 4096) return QFA_ERR_INVALID_ARG;
  qfa_status st = check_attn_common(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, D, softmax_scale,
                                    block_size, O);
  if (st != QFA_OK) return st;
  int splits = *num_splits == 0 ? qfa_decode_default_splits(B, Hkv, S_kv_max) : *num_splits;
  if (B == 0) {
    *num_splits = splits;
    return QFA_OK;
  }
  const size_t need = ws_bytes(B, Hq, D, splits);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return QFA_ERR_WORKSPACE;
  const int G = Hq / Hkv;
  const long long nwg = (long long)B * Hkv * ((G + 31) / 32) * splits;
  if (nwg > 0x7FFFFFFFLL) return QFA_ERR_INVALID_ARG;
  *num_splits = splits;
  const size_t rows = (size_t)B * Hq * splits;
  float* Op = static_cast<float*>(workspace);
  float* Lp = reinterpret_cast<float*>(static_cast<char*>(workspace) + (rows * D * sizeof(float) + 255) / 256 * 256);
  qfa::AttnArgs a{};
  a.q4 = q4; a.q4s = q4s; a.k4 = k4; a.k4s = k4s; a.v8 = v8; a.v8s = v8s;
  a.kbar = kbar; a.qbf = q_bf16; a.kv_lens = kv_lens;
  a.O = Op; a.lse = Lp;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = 1; a.Skv = S_kv_max; a.D = D; a.G = G;
  a.causal = 0;
  a.c2 = softmax_scale * kLog2e;
  a.num_splits = splits;
  a.pv = fmt;
  a.nv_gq = gq;
  a.nv_gk = gk;
  return from_hip(qfa::launch_decode(a, O, lse, stream));
}

qfa_status qfa_fwd_decode_noalloc(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                                  const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8,
                                  const uint8_t* v8s, int B, int Hq, int Hkv, int S_kv_max, const int32_t* kv_lens,
                                  int D, float softmax_scale, int block_size, int* num_splits, float* O, float* lse,
                                  hipStream_t stream) {
  // host checks first: a call that is rejected makes no HIP call at all
  if (!num_splits || S_kv_max < 0 || *num_splits < 0 || *num_splits > 4096) return QFA_ERR_INVALID_ARG;
  qfa_status st = check_attn_common(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, D, softmax_scale,
                                    block_size, O);
  if (st != QFA_OK) return st;
  if (B == 0)
    return decode_common(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D, softmax_scale,
                         block_size, QFA_PV_FP8, 1.0f, 1.0f, num_splits, nullptr, 0, O, lse, stream);
  const int splits = *num_splits == 0 ? qfa_decode_default_splits(B, Hkv, S_kv_max) : *num_splits;
  if (ws_bytes(B, Hq, D, splits) > (size_t)QFA_DECODE_NOALLOC_MAX_BYTES) return QFA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != QFA_OK) return st;
  return decode_common(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D, softmax_scale,
                       block_size, QFA_PV_FP8, 1.0f, 1.0f, num_splits, ws, (size_t)QFA_DECODE_NOALLOC_MAX_BYTES, O,
                       lse, stream);
}

qfa_status qfa_fwd_decode_ex(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                             const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                             int B, int Hq, int Hkv, int S_kv_max, const int32_t* kv_lens, int D,
                             float softmax_scale, int block_size, int pv_format, int* num_splits, void* workspace,
                             size_t workspace_bytes, float* O, float* lse, hipStream_t stream) {
  if (qfa_status f = check_pv_format(pv_format); f != QFA_OK) return f;
  return decode_common(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D, softmax_scale,
                       block_size, pv_format, 1.0f, 1.0f, num_splits, workspace, workspace_bytes, O, lse, stream);
}

qfa_status qfa_fwd_decode_nvfp4(const uint8_t* q4, const uint8_t* q4s, const uint8_t* k4, const uint8_t* k4s,
                                const uint16_t* kbar, const uint16_t* q_bf16, const uint8_t* v8, const uint8_t* v8s,
                                int B, int Hq, int Hkv, int S_kv_max, const int32_t* kv_lens, int D,
                                float softmax_scale, float q_tensor_scale, float k_tensor_scale, int* num_splits,
                                void* workspace, size_t workspace_bytes, float* O, float* lse, hipStream_t stream) {
  if (!pow2_ok(q_tensor_scale) || !pow2_ok(k_tensor_scale)) return QFA_ERR_INVALID_ARG;
  if (!q4 || !q4s) return QFA_ERR_INVALID_ARG;
  return decode_common(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D, softmax_scale,
                       32, qfa::QK_NVFP4, q_tensor_scale, k_tensor_scale, num_splits, workspace, workspace_bytes, O,
                       lse, stream);
}

}  // extern "C"
