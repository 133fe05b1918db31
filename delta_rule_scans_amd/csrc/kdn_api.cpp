// kdn_api.cpp -- the exported C ABI: argument checks, workspace sizing and
// dispatch to the HIP kernels. Every check runs before anything is enqueued,
// so a rejected call touches no device state.
#include "../../include/kdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kdn_internal.h"

#define KDN_EXPORT extern "C" __attribute__((visibility("default")))

namespace kdn {

bool trace_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("KDN_TRACE");
    return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
  }();
  return on;
}

void trace_launch(const char* kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  std::fprintf(stderr, "kdn: launch %s grid (%u,%u,%u) block (%u,%u,%u) lds %zu stream %p\n",
               kernel, grid.x, grid.y, grid.z, block.x, block.y, block.z, lds,
               static_cast<void*>(s));
}

void trace_call(const char* fmt, ...) {
  if (!trace_enabled()) return;
  std::va_list ap;
  va_start(ap, fmt);
  std::fputs("kdn: ", stderr);
  std::vfprintf(stderr, fmt, ap);
  std::fputc('\n', stderr);
  va_end(ap);
}

}  // namespace kdn

namespace {

constexpr int kMaxDim = 128;
constexpr int kMaxFullDk = 64;
constexpr int kMaxCapacity = 256;
constexpr int kMaxGridYZ = 65535;
constexpr int kMaxPrefillBlock = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_chunk(int c) { return c == 16 || c == 32 || c == 64 || c == 128; }

// The chunk the kernels run. 128 runs as 64-token chunks: the chunk form gives
// the same result for any chunk length up to rounding, and the matrix-core
// kernels are built for 64 while the float32 kernel's LDS grows with C^2.
int run_chunk(int c) { return c == 128 ? 64 : c; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout, 256-byte aligned parts:
//   [maps (DIAG, ISO) | gains (DIAG, FULL) or write strengths and key norms (ISO)
//    | per-chunk records of the matrix-core path | residuals for the scores].
// Gains are fp16 for bf16 inputs and float32 otherwise. The residual part holds
// fp16 residuals (matrix-core path) or per-tile squared norms (float32 path),
// sized for the larger of the two since the path is chosen at call time.
struct WsLayout {
  size_t maps_off, maps_bytes, gains_off, gains_bytes, t_off, t_bytes, s_off, s_bytes, total;
};

bool use_mfma_path(int in_dtype, int d_k, int d_v, int chunk) {
  return in_dtype == KDN_BF16 && kdn::scan_mfma_supported(d_k, d_v, chunk);
}

WsLayout ws_layout(int B, int H, int L, int dk, int dv, int chunk, int mode, int in_dtype,
                   bool scores) {
  WsLayout w{0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (L <= 0) return w;
  const size_t BH = (size_t)B * H;
  const size_t nchunks = ((size_t)L + chunk - 1) / chunk;
  // the diagonal write on the matrix-core path scans half chunks and keeps
  // their starting variances after the maps
  const bool half = use_mfma_path(in_dtype, dk, dv, chunk);
  const size_t nmaps = half ? ((size_t)L + chunk / 2 - 1) / (chunk / 2) : nchunks;
  if (mode == KDN_GAIN_DIAG) w.maps_bytes = BH * nmaps * dk * (half ? 5 : 4) * sizeof(float);
  if (mode == KDN_GAIN_ISO) w.maps_bytes = BH * nchunks * 4 * sizeof(float);
  if (mode == KDN_GAIN_DIAG || mode == KDN_GAIN_FULL)
    w.gains_bytes = BH * (size_t)L * dk * (in_dtype == KDN_BF16 ? 2 : 4);
  if (mode == KDN_GAIN_ISO) w.gains_bytes = 2 * BH * (size_t)L * sizeof(float);
  const bool gain = mode == KDN_GAIN_DIAG || mode == KDN_GAIN_FULL;
  if (use_mfma_path(in_dtype, dk, dv, chunk)) w.t_bytes = kdn::scan_mfma_workspace_bytes((int)BH, L, gain);
  if (scores) {
    const int cols = kdn::scan_f32_tile_cols(dk, chunk);
    const size_t ntiles = cols > 0 ? (size_t)(dv + cols - 1) / cols : 0;
    w.s_bytes = BH * ntiles * (size_t)L * sizeof(float);
    if (use_mfma_path(in_dtype, dk, dv, chunk)) {
      const size_t u = kdn::scan_mfma_ubuf_bytes((int)BH, L, dv);
      if (u > w.s_bytes) w.s_bytes = u;
    }
  }
  w.maps_off = 0;
  w.gains_off = round_up(w.maps_bytes, 256);
  w.t_off = w.gains_off + round_up(w.gains_bytes, 256);
  w.s_off = w.t_off + round_up(w.t_bytes, 256);
  w.total = w.s_off + round_up(w.s_bytes, 256);
  return w;
}

int map_hip(hipError_t e) { return e == hipSuccess ? KDN_OK : static_cast<int>(e); }

}  // namespace

KDN_EXPORT const char* kdn_status_string(int status) {
  switch (status) {
    case KDN_OK: return "ok";
    case KDN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case KDN_ERR_BAD_SHAPE: return "a size argument is out of range";
    case KDN_ERR_BAD_CHUNK: return "chunk must be 16, 32, 64 or 128";
    case KDN_ERR_BAD_MODE: return "unknown write mode or residual form, or plain residual with a Kalman gain";
    case KDN_ERR_BAD_DTYPE: return "unknown element type";
    case KDN_ERR_UNSUPPORTED: return "valid arguments that this library does not implement (e.g. full covariance with d_k > 64)";
    case KDN_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than kdn_scan_workspace_size";
    case KDN_ERR_BAD_CAPACITY: return "cache capacity w must be in [1, 256]";
    case KDN_ERR_BAD_ALIGNMENT: return "a pointer is not 16-byte aligned";
    case KDN_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch than the library's static scratch array holds "
             "(KDN_STATIC_SCRATCH_BYTES per GPU); use kdn_scan_fwd with a workspace";
    default: break;
  }
  if (status > 0) return hipGetErrorString(static_cast<hipError_t>(status));
  return "unknown status";
}

KDN_EXPORT int kdn_version(void) { return 100; }

KDN_EXPORT size_t kdn_scan_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk,
                                          int mode, int in_dtype, int with_scores) {
  if (B < 1 || H < 1 || L < 0 || d_k < 1 || d_v < 1 || !valid_chunk(chunk)) return 0;
  return ws_layout(B, H, L, d_k, d_v, run_chunk(chunk), mode, in_dtype, with_scores != 0).total;
}

namespace kdn {

// Every check of kdn_scan_fwd_phase that does not involve the workspace; host
// only, no HIP call.
int scan_args_status(int phase, const void* q, const void* k, const void* v, int in_dtype,
                     const float* beta, const float* cov_in, float q_noise_var, void* o,
                     int out_dtype, const float* m, int score_kind, int B, int H, int L, int d_k,
                     int d_v, int chunk, int mode, int resid) {
  if (phase != KDN_PHASE_ALL && phase != KDN_PHASE_PREPARE && phase != KDN_PHASE_STATE)
    return KDN_ERR_BAD_MODE;
  if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return KDN_ERR_BAD_DTYPE;
  if (out_dtype != KDN_F32 && out_dtype != KDN_BF16) return KDN_ERR_BAD_DTYPE;
  if (mode != KDN_GAIN_DELTA && mode != KDN_GAIN_DIAG && mode != KDN_GAIN_FULL &&
      mode != KDN_GAIN_ISO)
    return KDN_ERR_BAD_MODE;
  if (resid != KDN_RESID_GATED && resid != KDN_RESID_PLAIN && resid != KDN_RESID_NOERASE)
    return KDN_ERR_BAD_MODE;
  if (resid != KDN_RESID_GATED && mode != KDN_GAIN_DELTA) return KDN_ERR_BAD_MODE;
  if (m && (score_kind < KDN_SCORE_WRITE || score_kind > KDN_SCORE_VALUE)) return KDN_ERR_BAD_MODE;
  if (B < 1 || H < 1 || L < 0 || d_k < 1 || d_v < 1 || d_k > kMaxDim || d_v > kMaxDim)
    return KDN_ERR_BAD_SHAPE;
  if ((long long)B * H > (1LL << 24)) return KDN_ERR_BAD_SHAPE;
  if (!valid_chunk(chunk)) return KDN_ERR_BAD_CHUNK;
  chunk = run_chunk(chunk);
  if ((long long)(L + chunk - 1) / chunk > kMaxGridYZ) return KDN_ERR_BAD_SHAPE;
  if (mode == KDN_GAIN_FULL && d_k > kMaxFullDk) return KDN_ERR_UNSUPPORTED;
  if (mode != KDN_GAIN_DELTA && cov_in == nullptr) return KDN_ERR_NULL_POINTER;
  if (!std::isfinite(q_noise_var) || q_noise_var < 0.f) return KDN_ERR_BAD_SHAPE;
  if (L > 0) {
    if (!q || !k || !v || !o) return KDN_ERR_NULL_POINTER;
    if (mode == KDN_GAIN_DELTA && beta == nullptr) return KDN_ERR_NULL_POINTER;
  }
  if (kdn::scan_f32_lds_bytes(d_k, chunk) == 0 &&
      !(in_dtype == KDN_BF16 && kdn::scan_mfma_supported(d_k, d_v, chunk)))
    return KDN_ERR_UNSUPPORTED;
  return KDN_OK;
}

}  // namespace kdn

KDN_EXPORT int kdn_scan_fwd_phase(int phase, const void* q, const void* k, const void* v,
                                  int in_dtype, const float* alpha, const float* beta,
                                  const float* r, const float* cov_in, float* cov_out,
                                  float q_noise_var, const float* state_in, float* state_out,
                                  void* o, int out_dtype, float* m, int score_kind, int B, int H,
                                  int L, int d_k, int d_v, int chunk, int mode, int resid,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const int st = kdn::scan_args_status(phase, q, k, v, in_dtype, beta, cov_in, q_noise_var, o,
                                       out_dtype, m, score_kind, B, H, L, d_k, d_v, chunk, mode,
                                       resid);
  if (st != KDN_OK) return st;
  chunk = run_chunk(chunk);
  const bool do_prep = phase != KDN_PHASE_STATE, do_state = phase != KDN_PHASE_PREPARE;
  const WsLayout ws = ws_layout(B, H, L, d_k, d_v, chunk, mode, in_dtype, m != nullptr);
  if (ws.total > 0 && (workspace == nullptr || workspace_bytes < ws.total || !aligned16(workspace)))
    return KDN_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int BH = B * H;
  const size_t cov_elems = mode == KDN_GAIN_DIAG   ? (size_t)BH * d_k
                           : mode == KDN_GAIN_FULL ? (size_t)BH * d_k * d_k
                           : mode == KDN_GAIN_ISO  ? (size_t)BH
                                                   : 0;
  if (L == 0) {
    hipError_t e = hipSuccess;
    if (do_state && state_out)
      e = kdn::launch_copy_f32(state_in, state_out, (size_t)BH * d_k * d_v, s);
    if (do_prep && e == hipSuccess && cov_out && cov_elems)
      e = kdn::launch_copy_f32(cov_in, cov_out, cov_elems, s);
    return map_hip(e);
  }

  const bool in_bf16 = in_dtype == KDN_BF16;
  const bool has_gain = mode == KDN_GAIN_DIAG || mode == KDN_GAIN_FULL;
  const void* gains = nullptr;
  if (has_gain) {
    char* base = static_cast<char*>(workspace);
    void* g = base + ws.gains_off;
    gains = g;
  }
  // the isotropic write runs as the delta write with the beta it computes here
  float* iso_beta = mode == KDN_GAIN_ISO
                        ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.gains_off)
                        : nullptr;
  if (do_prep && mode == KDN_GAIN_ISO) {
    char* base = static_cast<char*>(workspace);
    const hipError_t e = kdn::launch_iso_beta(
        k, in_bf16, alpha, r, cov_in, cov_out, q_noise_var, iso_beta, iso_beta + (size_t)BH * L,
        reinterpret_cast<float*>(base + ws.maps_off), BH, L, d_k, chunk, s);
    if (e != hipSuccess) return map_hip(e);
  }
  const bool mfma_ok = use_mfma_path(in_dtype, d_k, d_v, chunk) && aligned16(q) &&
                       aligned16(k) && aligned16(v) && aligned16(o) &&
                       (gains == nullptr || aligned16(gains));
  // the diagonal write on the matrix-core path: the covariance scan over half
  // chunks gives their starting variances and the prepare kernel forms the
  // gains from them
  const bool diag_fused = mode == KDN_GAIN_DIAG && mfma_ok;
  float* diag_maps = nullptr;    // [BH, half chunks, d_k] float4, then
  float* diag_starts = nullptr;  // [BH, half chunks, d_k] starting variances
  if (diag_fused) {
    diag_maps = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.maps_off);
    diag_starts = diag_maps + (size_t)BH * ((L + chunk / 2 - 1) / (chunk / 2)) * d_k * 4;
  }
  if (do_prep && diag_fused) {
    const hipError_t e = kdn::launch_diag_starts(k, in_bf16, alpha, r, cov_in, q_noise_var,
                                                 diag_maps, diag_starts, BH, L, d_k, chunk / 2, s);
    if (e != hipSuccess) return map_hip(e);
  } else if (do_prep && has_gain) {
    char* base = static_cast<char*>(workspace);
    void* g = base + ws.gains_off;
    hipError_t e;
    if (mode == KDN_GAIN_DIAG)
      e = kdn::launch_diag_gains(k, in_bf16, alpha, r, cov_in, cov_out, q_noise_var, g, in_bf16,
                                 reinterpret_cast<float*>(base + ws.maps_off), BH, L, d_k, chunk,
                                 s);
    else
      e = kdn::launch_full_gains(k, in_bf16, alpha, r, cov_in, cov_out, q_noise_var, g, in_bf16,
                                 BH, L, d_k, s);
    if (e != hipSuccess) return map_hip(e);
  }

  kdn::ScanArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = mode == KDN_GAIN_DELTA ? beta : iso_beta;
  a.gain = gains;
  a.state_in = state_in;
  a.state_out = state_out;
  a.o = o;
  a.BH = BH;
  a.L = L;
  a.dk = d_k;
  a.dv = d_v;
  a.chunk = chunk;
  a.plain = resid == KDN_RESID_PLAIN ? 1 : 0;
  a.noerase = resid == KDN_RESID_NOERASE ? 1 : 0;

  if (diag_fused) {
    a.dmaps = diag_starts;
    a.r = r;
    a.qvar = q_noise_var;
    a.cov_out = cov_out;
  }

  const bool out_bf16 = out_dtype == KDN_BF16;
  kdn::trace_call("kdn_scan_fwd phase %d B %d H %d L %d d_k %d d_v %d chunk %d mode %d resid %d "
                  "in %s -> %s path", phase, B, H, L, d_k, d_v, chunk, mode, resid,
                  in_bf16 ? "bf16" : "f32", mfma_ok ? "matrix-core" : "float32");
  kdn::ScoreArgs sc{};
  if (m) {
    void* sbuf = static_cast<char*>(workspace) + ws.s_off;
    if (mfma_ok) a.ubuf = sbuf;
    else a.esq = static_cast<float*>(sbuf);
    const int cols = kdn::scan_f32_tile_cols(d_k, chunk);
    sc.kind = score_kind;
    sc.v = v;
    sc.v_bf16 = in_bf16 ? 1 : 0;
    sc.esq = a.esq;
    sc.ubuf = a.ubuf;
    sc.uexp = a.ubuf ? kdn::scan_mfma_ubuf_exps(a.ubuf, BH, L, d_v) : nullptr;
    sc.ntiles = mfma_ok ? d_v / 32 : (d_v + cols - 1) / cols;
    sc.beta = a.beta;
    sc.iso_beta = iso_beta;
    sc.iso_kk = iso_beta ? iso_beta + (size_t)BH * L : nullptr;
    sc.gains = gains;
    sc.gains_f16 = in_bf16 ? 1 : 0;
    sc.m = m;
    sc.BH = BH;
    sc.L = L;
    sc.dk = d_k;
    sc.dv = d_v;
  }
  hipError_t e = hipSuccess;
  if (mfma_ok) {
    void* tbuf = static_cast<char*>(workspace) + ws.t_off;
    if (do_prep) {
      e = kdn::launch_tinv_mfma(a, tbuf, s);
      if (e != hipSuccess) return map_hip(e);
    }
    if (do_state) e = kdn::launch_state_mfma(a, out_bf16, tbuf, s);
  } else if (do_state) {
    e = kdn::launch_scan_f32(a, in_bf16, out_bf16, in_bf16, s);
  }
  if (e == hipSuccess && do_state && m) e = kdn::launch_scores(sc, s);
  return map_hip(e);
}

KDN_EXPORT int kdn_scan_fwd(const void* q, const void* k, const void* v, int in_dtype,
                            const float* alpha, const float* beta, const float* r,
                            const float* cov_in, float* cov_out, float q_noise_var,
                            const float* state_in, float* state_out, void* o, int out_dtype,
                            float* m, int score_kind, int B, int H, int L, int d_k, int d_v,
                            int chunk, int mode, int resid, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return kdn_scan_fwd_phase(KDN_PHASE_ALL, q, k, v, in_dtype, alpha, beta, r, cov_in, cov_out,
                            q_noise_var, state_in, state_out, o, out_dtype, m, score_kind, B, H, L,
                            d_k, d_v, chunk, mode, resid, workspace, workspace_bytes, stream);
}

KDN_EXPORT int kdn_step_decode(const float* q, const float* k, const float* v, const float* alpha,
                               const float* beta, const float* r, float* cov, float q_noise_var,
                               float* state, float* o, float* m, int score_kind, int B, int H,
                               int d_k, int d_v, int mode, int resid, void* stream) {
  if (mode != KDN_GAIN_DELTA && mode != KDN_GAIN_DIAG && mode != KDN_GAIN_FULL &&
      mode != KDN_GAIN_ISO)
    return KDN_ERR_BAD_MODE;
  if (resid != KDN_RESID_GATED && resid != KDN_RESID_PLAIN && resid != KDN_RESID_NOERASE)
    return KDN_ERR_BAD_MODE;
  if (resid != KDN_RESID_GATED && mode != KDN_GAIN_DELTA) return KDN_ERR_BAD_MODE;
  if (m && (score_kind < KDN_SCORE_WRITE || score_kind > KDN_SCORE_VALUE)) return KDN_ERR_BAD_MODE;
  if (B < 1 || H < 1 || d_k < 1 || d_v < 1 || d_k > kMaxDim || d_v > kMaxDim)
    return KDN_ERR_BAD_SHAPE;
  if ((long long)B * H > (1LL << 30)) return KDN_ERR_BAD_SHAPE;
  if (mode == KDN_GAIN_FULL) return KDN_ERR_UNSUPPORTED;
  if (!std::isfinite(q_noise_var) || q_noise_var < 0.f) return KDN_ERR_BAD_SHAPE;
  if (!q || !k || !v || !state || !o) return KDN_ERR_NULL_POINTER;
  if (mode == KDN_GAIN_DELTA && beta == nullptr) return KDN_ERR_NULL_POINTER;
  if ((mode == KDN_GAIN_DIAG || mode == KDN_GAIN_ISO) && cov == nullptr)
    return KDN_ERR_NULL_POINTER;
  return map_hip(kdn::launch_decode(q, k, v, alpha, beta, r, cov, q_noise_var, state, o, m, B * H,
                                    d_k, d_v,
                                    mode == KDN_GAIN_DIAG  ? 1
                                    : mode == KDN_GAIN_ISO ? 2
                                                           : 0,
                                    resid, m ? score_kind : 0, static_cast<hipStream_t>(stream)));
}

KDN_EXPORT int hola_cache_update(const float* q, const float* k, const float* v, const float* m,
                                 int32_t t, float* cache_k, float* cache_v, float* cache_m,
                                 int32_t* cache_pos, int32_t* cache_count,
                                 const float* sink_logit, float* o_cache, float rms_eps, int B,
                                 int H, int d_k, int d_v, int w, int policy, void* stream) {
  if (w < 1 || w > kMaxCapacity) return KDN_ERR_BAD_CAPACITY;
  if (policy != KDN_EVICT_SCORE && policy != KDN_EVICT_RECENCY) return KDN_ERR_BAD_MODE;
  if (B < 1 || H < 1 || d_k < 1 || d_v < 1 || d_k > kMaxDim || d_v > kMaxDim)
    return KDN_ERR_BAD_SHAPE;
  if ((long long)B * H > (1LL << 30)) return KDN_ERR_BAD_SHAPE;
  if (!(rms_eps >= 0.f) || !std::isfinite(rms_eps)) return KDN_ERR_BAD_SHAPE;
  if (!q || !k || !v || !m || !cache_k || !cache_v || !cache_m || !cache_pos || !cache_count ||
      !o_cache)
    return KDN_ERR_NULL_POINTER;
  return map_hip(kdn::launch_hola(q, k, v, m, t, cache_k, cache_v, cache_m, cache_pos, cache_count,
                                  sink_logit, o_cache, rms_eps, B, H, d_k, d_v, w, policy,
                                  static_cast<hipStream_t>(stream)));
}

KDN_EXPORT size_t hola_prefill_workspace_size(int B, int H, int L, int d_k, int d_v, int w,
                                              int block) {
  if (B < 1 || H < 1 || L < 1 || d_k < 1 || d_v < 1 || w < 1 || block < 1) return 0;
  return kdn::prefill_workspace_bytes(B * H, L, d_k, d_v, w, block);
}

KDN_EXPORT int hola_prefill(const void* q, const void* k, const void* v, int in_dtype,
                            const float* m, int32_t t0, int block, float* cache_k, float* cache_v,
                            float* cache_m, int32_t* cache_pos, int32_t* cache_count,
                            const float* sink_logit, float* o_cache, float rms_eps, int B, int H,
                            int L, int d_k, int d_v, int w, int policy, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return KDN_ERR_BAD_DTYPE;
  if (w < 1 || w > kMaxCapacity) return KDN_ERR_BAD_CAPACITY;
  if (policy != KDN_EVICT_SCORE && policy != KDN_EVICT_RECENCY) return KDN_ERR_BAD_MODE;
  if (B < 1 || H < 1 || L < 0 || d_k < 1 || d_v < 1 || d_k > kMaxDim || d_v > kMaxDim)
    return KDN_ERR_BAD_SHAPE;
  if (block < 1 || block > kMaxPrefillBlock) return KDN_ERR_BAD_SHAPE;
  if ((long long)B * H > (1LL << 24)) return KDN_ERR_BAD_SHAPE;
  if ((long long)(L + block - 1) / block > kMaxGridYZ) return KDN_ERR_BAD_SHAPE;
  if ((long long)t0 + L > INT32_MAX) return KDN_ERR_BAD_SHAPE;
  if (!(rms_eps >= 0.f) || !std::isfinite(rms_eps)) return KDN_ERR_BAD_SHAPE;
  if (!cache_k || !cache_v || !cache_m || !cache_pos || !cache_count) return KDN_ERR_NULL_POINTER;
  if (L == 0) return KDN_OK;
  if (!q || !k || !v || !m || !o_cache) return KDN_ERR_NULL_POINTER;
  const size_t need = kdn::prefill_workspace_bytes(B * H, L, d_k, d_v, w, block);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return KDN_ERR_WORKSPACE;
  kdn::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.m = m;
  a.t0 = t0;
  a.block = block;
  a.cache_k = cache_k;
  a.cache_v = cache_v;
  a.cache_m = cache_m;
  a.cache_pos = cache_pos;
  a.cache_count = cache_count;
  a.sink_logit = sink_logit;
  a.o_cache = o_cache;
  a.rms_eps = rms_eps;
  a.BH = B * H;
  a.H = H;
  a.L = L;
  a.dk = d_k;
  a.dv = d_v;
  a.w = w;
  a.policy = policy;
  kdn::prefill_bind_workspace(a, workspace);
  return map_hip(kdn::launch_prefill(a, in_dtype == KDN_BF16, static_cast<hipStream_t>(stream)));
}

KDN_EXPORT size_t kdn_scan_bwd_workspace_size(int B, int H, int L, int d_k, int d_v) {
  if (B < 1 || H < 1 || L < 1 || d_k < 1 || d_v < 1 || d_k > kMaxDim || d_v > kMaxDim) return 0;
  return kdn::scan_bwd_workspace_bytes(B * H, L, d_k, d_v);
}

KDN_EXPORT int kdn_scan_bwd(const float* q, const float* k, const float* v, const float* alpha,
                            const float* beta, const float* state_in, const float* d_o,
                            const float* dstate_out, float* dq, float* dk, float* dv,
                            float* dalpha, float* dbeta, float* dstate_in, int B, int H, int L,
                            int d_k, int d_v, int resid, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (resid != KDN_RESID_GATED && resid != KDN_RESID_PLAIN && resid != KDN_RESID_NOERASE)
    return KDN_ERR_BAD_MODE;
  if (B < 1 || H < 1 || L < 0 || d_k < 1 || d_v < 1 || d_k > kMaxDim || d_v > kMaxDim)
    return KDN_ERR_BAD_SHAPE;
  if ((long long)B * H > (1LL << 24) || (long long)(d_v + 31) / 32 > kMaxGridYZ ||
      ((long long)L + 63) / 64 > kMaxGridYZ)
    return KDN_ERR_BAD_SHAPE;
  if (L == 0) {
    // no tokens: the initial state's gradient is the final state's
    hipError_t e = hipSuccess;
    if (dstate_in)
      e = kdn::launch_copy_f32(dstate_out, dstate_in, (size_t)B * H * d_k * d_v,
                               static_cast<hipStream_t>(stream));
    return map_hip(e);
  }
  if (!q || !k || !v || !beta || !d_o || !dq || !dk || !dv || !dbeta) return KDN_ERR_NULL_POINTER;
  if (alpha && !dalpha) return KDN_ERR_NULL_POINTER;
  const size_t need = kdn::scan_bwd_workspace_bytes(B * H, L, d_k, d_v);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return KDN_ERR_WORKSPACE;
  kdn::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.state_in = state_in;
  a.d_o = d_o;
  a.dstate_out = dstate_out;
  a.dq = dq;
  a.dk_out = dk;
  a.dv_out = dv;
  a.dalpha = alpha ? dalpha : nullptr;
  a.dbeta = dbeta;
  a.dstate_in = dstate_in;
  a.BH = B * H;
  a.L = L;
  a.dk = d_k;
  a.dv = d_v;
  a.resid = resid;
  return map_hip(kdn::launch_scan_bwd(a, workspace, static_cast<hipStream_t>(stream)));
}


// ------------------------------------------------------------ kdn_scan_bwd_ex
namespace {

// Workspace of kdn_scan_bwd_ex, 256-byte aligned parts:
//   [float32 copies of bf16 q, k, v, d_o | Kalman forward recompute: gains or
//    write strengths, variance before each token, s_t or ||k||^2, chunk maps |
//    dL/d(gain rows) or dL/dbeta | covariance-adjoint scratch | the state
//    backward's workspace]
struct BwdExLayout {
  size_t cvt_q, cvt_k, cvt_v, cvt_o, gain, pprev, sden, maps, dgain, adj, bwd, total;
};

BwdExLayout bwd_ex_layout(int B, int H, int L, int dk, int dv, int mode, int in_dtype) {
  BwdExLayout w{};
  const size_t BH = (size_t)B * H, T = BH * (size_t)L, nch = ((size_t)L + 63) / 64;
  const bool bf = in_dtype == KDN_BF16, diag = mode == KDN_GAIN_DIAG, iso = mode == KDN_GAIN_ISO;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes, 256);
    return at;
  };
  w.cvt_q = take(bf ? T * dk * 4 : 0);
  w.cvt_k = take(bf ? T * dk * 4 : 0);
  w.cvt_v = take(bf ? T * dv * 4 : 0);
  w.cvt_o = take(bf ? T * dv * 4 : 0);
  w.gain = take(diag ? T * dk * 4 : iso ? 2 * T * 4 : 0);        // gains / (beta, ||k||^2)
  w.pprev = take(diag ? T * dk * 4 : iso ? T * 4 : 0);
  w.sden = take(diag ? T * 4 : 0);
  w.maps = take(diag ? BH * nch * dk * 16 : iso ? BH * nch * 16 : 0);
  w.dgain = take(diag ? T * dk * 4 : iso ? T * 4 : 0);           // dL/dgain / dL/dbeta
  w.adj = take((diag || iso) ? kdn::cov_adj_scratch_floats((int)BH, L, dk, diag) * 4 : 0);
  w.bwd = take(kdn::scan_bwd_workspace_bytes((int)BH, L, dk, dv));
  w.total = o;
  return w;
}

}  // namespace

KDN_EXPORT size_t kdn_scan_bwd_ex_workspace_size(int B, int H, int L, int d_k, int d_v, int mode,
                                                 int in_dtype) {
  if (B < 1 || H < 1 || L < 1 || d_k < 1 || d_v < 1 || d_k > kMaxDim || d_v > kMaxDim) return 0;
  if (mode != KDN_GAIN_DELTA && mode != KDN_GAIN_DIAG && mode != KDN_GAIN_ISO) return 0;
  if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return 0;
  return bwd_ex_layout(B, H, L, d_k, d_v, mode, in_dtype).total;
}

KDN_EXPORT int kdn_scan_bwd_ex(const void* q, const void* k, const void* v, const void* d_o,
                               int in_dtype, const float* alpha, const float* beta, const float* r,
                               const float* cov_in, float q_noise_var, const float* state_in,
                               const float* dstate_out, const float* dcov_out, float* dq, float* dk,
                               float* dv, float* dalpha, float* dbeta, float* dr, float* dcov_in,
                               float* dstate_in, int B, int H, int L, int d_k, int d_v, int mode,
                               int resid, void* workspace, size_t workspace_bytes, void* stream) {
  if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return KDN_ERR_BAD_DTYPE;
  if (mode == KDN_GAIN_FULL) return KDN_ERR_UNSUPPORTED;
  if (mode != KDN_GAIN_DELTA && mode != KDN_GAIN_DIAG && mode != KDN_GAIN_ISO)
    return KDN_ERR_BAD_MODE;
  if (resid != KDN_RESID_GATED && resid != KDN_RESID_PLAIN && resid != KDN_RESID_NOERASE)
    return KDN_ERR_BAD_MODE;
  if (resid != KDN_RESID_GATED && mode != KDN_GAIN_DELTA) return KDN_ERR_BAD_MODE;
  if (B < 1 || H < 1 || L < 0 || d_k < 1 || d_v < 1 || d_k > kMaxDim || d_v > kMaxDim)
    return KDN_ERR_BAD_SHAPE;
  if ((long long)B * H > (1LL << 24) || (long long)(d_v + 31) / 32 > kMaxGridYZ ||
      ((long long)L + 63) / 64 > kMaxGridYZ)
    return KDN_ERR_BAD_SHAPE;
  if (!std::isfinite(q_noise_var) || q_noise_var < 0.f) return KDN_ERR_BAD_SHAPE;
  const bool kalman = mode != KDN_GAIN_DELTA;
  if (kalman && cov_in == nullptr) return KDN_ERR_NULL_POINTER;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int BH = B * H;
  const size_t np = mode == KDN_GAIN_DIAG ? (size_t)d_k : 1;
  if (L == 0) {
    // no tokens: the initial state's and covariance's gradients are the final ones'
    hipError_t e = hipSuccess;
    if (dstate_in) e = kdn::launch_copy_f32(dstate_out, dstate_in, (size_t)BH * d_k * d_v, s);
    if (e == hipSuccess && kalman && dcov_in) e = kdn::launch_copy_f32(dcov_out, dcov_in, BH * np, s);
    return map_hip(e);
  }
  if (!q || !k || !v || !d_o || !dq || !dk || !dv) return KDN_ERR_NULL_POINTER;
  if (!kalman && (!beta || !dbeta)) return KDN_ERR_NULL_POINTER;
  if (alpha && !dalpha) return KDN_ERR_NULL_POINTER;
  if (kalman && r && !dr) return KDN_ERR_NULL_POINTER;
  const BwdExLayout w = bwd_ex_layout(B, H, L, d_k, d_v, mode, in_dtype);
  if (workspace == nullptr || workspace_bytes < w.total || !aligned16(workspace))
    return KDN_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const size_t T = (size_t)BH * L;
  hipError_t e = hipSuccess;
  const float *qf = static_cast<const float*>(q), *kf = static_cast<const float*>(k);
  const float *vf = static_cast<const float*>(v), *of = static_cast<const float*>(d_o);
  if (in_dtype == KDN_BF16) {
    float* cq = reinterpret_cast<float*>(ws + w.cvt_q);
    float* ck = reinterpret_cast<float*>(ws + w.cvt_k);
    float* cv = reinterpret_cast<float*>(ws + w.cvt_v);
    float* co = reinterpret_cast<float*>(ws + w.cvt_o);
    e = kdn::launch_bf16_to_f32(static_cast<const uint16_t*>(q), cq, T * d_k, s);
    if (e == hipSuccess) e = kdn::launch_bf16_to_f32(static_cast<const uint16_t*>(k), ck, T * d_k, s);
    if (e == hipSuccess) e = kdn::launch_bf16_to_f32(static_cast<const uint16_t*>(v), cv, T * d_v, s);
    if (e == hipSuccess) e = kdn::launch_bf16_to_f32(static_cast<const uint16_t*>(d_o), co, T * d_v, s);
    if (e != hipSuccess) return map_hip(e);
    qf = cq;
    kf = ck;
    vf = cv;
    of = co;
  }
  kdn::BwdArgs a{};
  a.q = qf;
  a.k = kf;
  a.v = vf;
  a.alpha = alpha;
  a.beta = beta;
  a.state_in = state_in;
  a.d_o = of;
  a.dstate_out = dstate_out;
  a.dq = dq;
  a.dk_out = dk;
  a.dv_out = dv;
  a.dalpha = alpha ? dalpha : nullptr;
  a.dbeta = dbeta;
  a.dstate_in = dstate_in;
  a.BH = BH;
  a.L = L;
  a.dk = d_k;
  a.dv = d_v;
  a.resid = resid;
  kdn::CovAdjArgs c{};
  float* gain = reinterpret_cast<float*>(ws + w.gain);
  float* pprev = reinterpret_cast<float*>(ws + w.pprev);
  float* dgain = reinterpret_cast<float*>(ws + w.dgain);
  if (mode == KDN_GAIN_DIAG) {
    // forward: the gains, the variance before each token and s_t
    float* sden = reinterpret_cast<float*>(ws + w.sden);
    e = kdn::launch_diag_gains(kf, false, alpha, r, cov_in, nullptr, q_noise_var, gain, false,
                               reinterpret_cast<float*>(ws + w.maps), BH, L, d_k, 64, s, pprev,
                               sden);
    if (e != hipSuccess) return map_hip(e);
    a.beta = nullptr;
    a.dbeta = nullptr;
    a.gain = gain;
    a.dgain = dgain;
    c.sden = sden;
    c.gains = gain;
    c.dgain = dgain;
  } else if (mode == KDN_GAIN_ISO) {
    // forward: the write strengths beta_t (the delta write), ||k||^2, variances
    float* kk = gain + T;
    e = kdn::launch_iso_beta(kf, false, alpha, r, cov_in, nullptr, q_noise_var, gain, kk,
                             reinterpret_cast<float*>(ws + w.maps), BH, L, d_k, 64, s, pprev);
    if (e != hipSuccess) return map_hip(e);
    a.beta = gain;
    a.dbeta = dgain;
    c.kk = kk;
    c.dbeta = dgain;
  }
  e = kdn::launch_scan_bwd(a, ws + w.bwd, s);
  if (e != hipSuccess || !kalman) return map_hip(e);
  c.diag = mode == KDN_GAIN_DIAG;
  c.k = kf;
  c.alpha = alpha;
  c.r = r;
  c.qvar = q_noise_var;
  c.pprev = pprev;
  c.dcov_out = dcov_out;
  c.dk_out = dk;
  c.dalpha = alpha ? dalpha : nullptr;
  c.dr = r ? dr : nullptr;
  c.dcov_in = dcov_in;
  c.BH = BH;
  c.L = L;
  c.dk = d_k;
  return map_hip(kdn::launch_cov_adjoint(c, reinterpret_cast<float*>(ws + w.adj), s));
}
