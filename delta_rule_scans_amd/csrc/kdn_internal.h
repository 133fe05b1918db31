// kdn_internal.h -- declarations shared by the HIP translation units of the
// library (device helpers and the host-side launchers the C ABI calls).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kdn {

// Launch tracing: with KDN_TRACE=1 in the environment every kernel launch is
// written to stderr (kernel, grid, workgroup, LDS bytes, stream) as it is
// enqueued; otherwise the cost is one test of a cached flag.
bool trace_enabled();
void trace_launch(const char* kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s);
void trace_call(const char* fmt, ...);
#define KDN_LAUNCH_NAMED(name, kernel, grid, block, lds, stream, ...)                          \
  do {                                                                                        \
    if (::kdn::trace_enabled()) ::kdn::trace_launch(name, dim3(grid), dim3(block), (lds), (stream)); \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                        \
  } while (0)
#define KDN_LAUNCH(kernel, grid, block, lds, stream, ...) \
  KDN_LAUNCH_NAMED(#kernel, kernel, grid, block, lds, stream, __VA_ARGS__)

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
// Two floats -> two bf16 (lo in the low half), round to nearest even, in one
// v_cvt_pk_bf16_f32.
typedef float kdn_float2v __attribute__((ext_vector_type(2)));
typedef __bf16 kdn_bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(kdn_float2v{lo, hi}, kdn_bf16x2v));
}
// One float -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Raw buffer resource over [base, base + bytes): loads past the end read 0,
// stores past it are dropped. The base must be uniform across the wavefront.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes > 0x7fffffffu ? 0x7fffffffu : bytes),
                                           0x00020000);
}

// Streaming store (cache policy sc0 nt): written once and not read back by the
// kernel, so it does not allocate in L2.
constexpr int kStreamStore = 3;
__device__ __forceinline__ void stream_store16(__amdgpu_buffer_rsrc_t r, int off, float4 x) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(
      u4{__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)}, r,
      off, 0, kStreamStore);
}
// Streaming load (sc0 nt) for data read exactly once by the whole grid. Data
// that other workgroups read again must use ordinary loads.
__device__ __forceinline__ float4 stream_load16(__amdgpu_buffer_rsrc_t r, int off) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamStore);
  return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                     __uint_as_float(x[3]));
}
__device__ __forceinline__ void stream_store4(__amdgpu_buffer_rsrc_t r, int off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, kStreamStore);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<_Float16> {
  __device__ static __forceinline__ float load(const _Float16* p, size_t i) { return (float)p[i]; }
  __device__ static __forceinline__ void store(_Float16* p, size_t i, float x) { p[i] = (_Float16)x; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float load(const uint16_t* p, size_t i) {
    return bf16_to_f32(p[i]);
  }
  __device__ static __forceinline__ void store(uint16_t* p, size_t i, float x) {
    p[i] = f32_to_bf16(x);
  }
};

// ------------------------------------------------------------- scan arguments
// Everything a scan kernel needs; device pointers, element counts in elements.
struct ScanArgs {
  const void* q;       // [BH, L, dk]
  const void* k;       // [BH, L, dk]
  const void* v;       // [BH, L, dv]
  const float* alpha;  // [BH, L] or null (= 1)
  const float* beta;   // [BH, L] (delta) or null
  const void* gain;    // [BH, L, dk] precomputed write vectors (Kalman modes) or null
  const float* state_in;  // [BH, dk, dv] or null (= 0)
  float* state_out;       // [BH, dk, dv] or null
  void* o;                // [BH, L, dv]
  int BH, L, dk, dv, chunk;
  int plain;  // 1: plain residual e = v - S^T k (delta only): exclusive decay in A and K S0
  int noerase = 0;  // 1: e = v (no prediction subtracted, delta only)
  // Residuals for the write scores, or null: the float32 path writes per-tile
  // sums of e_t^2 to esq [BH, d_v tiles, L]; the matrix-core path writes the
  // residuals themselves (fp16) to ubuf, see scan_mfma_ubuf_bytes.
  float* esq = nullptr;
  void* ubuf = nullptr;
  // Diagonal Kalman write on the matrix-core path with the gains formed by the
  // prepare kernel (else null): the variances at the start of every half chunk
  // ([BH, half chunks, dk] floats from launch_diag_starts with chunk / 2),
  // r [BH, L] (null: 1), the process noise variance and the final variances
  // [BH, dk] (or null); the gains go to `gain`, which the state kernel reads.
  const float* dmaps = nullptr;
  const float* r = nullptr;
  float qvar = 0.f;
  float* cov_out = nullptr;
};

// Status of kdn_scan_fwd_phase's argument checks other than the workspace
// (KDN_OK or a negative KDN_ERR_*); host only, makes no HIP call.
int scan_args_status(int phase, const void* q, const void* k, const void* v, int in_dtype,
                     const float* beta, const float* cov_in, float q_noise_var, void* o,
                     int out_dtype, const float* m, int score_kind, int B, int H, int L, int d_k,
                     int d_v, int chunk, int mode, int resid);

// ------------------------------------------------------------------ launchers
// Each returns a hipError_t (hipSuccess when the launch was enqueued).

// Float32 vector-path chunk scan; in/out element types chosen at run time.
// Gains (Kalman modes) are fp16 when gain_f16, else float32.
hipError_t launch_scan_f32(const ScanArgs& a, bool in_bf16, bool out_bf16, bool gain_f16,
                           hipStream_t s);
// LDS bytes the float32 path needs for (dk, chunk), or 0 when it cannot run them.
size_t scan_f32_lds_bytes(int dk, int chunk);
// Value columns per workgroup of the float32 path (its d_v tile).
int scan_f32_tile_cols(int dk, int chunk);

// Matrix-core chunk scan for bf16 inputs (dk == 128, dv % 32 == 0, chunk == 64);
// gains (if any) are fp16. `tbuf` holds scan_mfma_workspace_bytes(BH, L, gain)
// bytes: per chunk (I + A)^-1, the masked query-key product for the Kalman
// writes, and the token scalars.
hipError_t launch_tinv_mfma(const ScanArgs& a, void* tbuf, hipStream_t s);
hipError_t launch_state_mfma(const ScanArgs& a, bool out_bf16, const void* tbuf, hipStream_t s);
bool scan_mfma_supported(int dk, int dv, int chunk);
size_t scan_mfma_workspace_bytes(int BH, int L, bool gain);
// Bytes of the residual buffer of the matrix-core path (fp16 residuals of
// every token and value column).
size_t scan_mfma_ubuf_bytes(int BH, int L, int dv);
// The residuals there are times 2^e_S, one int exponent per (head, 32-column
// slice, chunk), stored after them: their address.
const int* scan_mfma_ubuf_exps(const void* ubuf, int BH, int L, int dv);

// Write scores m_t = s_t ||e_t|| ("A Hippocampus for Linear Attention", sec.
// 3.3 eq. (6)) from the residuals a scan left in esq (float32 path, `ntiles`
// d_v tiles) or ubuf (matrix-core path, dv / 32 tiles). The write scale s_t is
// beta_t for the delta write, beta_t ||k_t|| for the isotropic gain (iso_beta, iso_kk = ||k||^2), and
// ||g_t|| for the diagonal / full gains (gains [BH, L, dk], fp16 or f32).
struct ScoreArgs {
  int kind;  // 0: s ||e||, 1: ||e||, 2: s ||v|| (s: the write scale below)
  const void* v;  // [BH, L, dv] input values (kind 2)
  int v_bf16;
  const float* esq;
  const void* ubuf;
  const int* uexp;  // exponents of the residuals in ubuf (see scan_mfma_ubuf_exps)
  int ntiles;
  const float* beta;
  const float* iso_beta;
  const float* iso_kk;
  const void* gains;
  int gains_f16;
  float* m;
  int BH, L, dk, dv;
};
hipError_t launch_scores(const ScoreArgs& a, hipStream_t s);

// Diagonal-covariance Kalman gains: writes gains [BH, L, dk] (fp16 or f32) and
// the final covariance. `maps` is scratch of BH * nchunks * dk * 4 floats.
// pprev (optional, [BH, L, dk] float32): the variance before every token; sden
// (optional, [BH, L]): s_t = r_t + sum_i p-_i k_i^2 (the backward reads both).
hipError_t launch_diag_gains(const void* k, bool k_bf16, const float* alpha, const float* r,
                             const float* cov_in, float* cov_out, float q_noise_var,
                             void* gains, bool gains_f16, float* maps, int BH, int L, int dk,
                             int chunk, hipStream_t s, float* pprev = nullptr,
                             float* sden = nullptr);
// The first two passes of launch_diag_gains only: every chunk's starting
// variances into `starts` ([BH, nchunks, dk] floats); `maps` is scratch of
// BH * nchunks * dk float4. d_k must be a multiple of 64. The matrix-core
// prepare kernel then forms the gains itself.
hipError_t launch_diag_starts(const void* k, bool k_bf16, const float* alpha, const float* r,
                              const float* cov_in, float q_noise_var, float* maps, float* starts,
                              int BH, int L, int dk, int chunk, hipStream_t s);

// Isotropic Kalman write: the per-token write strengths beta [BH, L] (the gain
// is beta_t k_t) and the final variance [BH]. `kk` is scratch of BH * L floats,
// `maps` of BH * nchunks * 4 floats (16-byte aligned). chunk <= 64.
// pprev (optional, [BH, L]): the variance before every token.
hipError_t launch_iso_beta(const void* k, bool k_bf16, const float* alpha, const float* r,
                          const float* cov_in, float* cov_out, float q_noise_var, float* beta,
                          float* kk, float* maps, int BH, int L, int dk, int chunk,
                          hipStream_t s, float* pprev = nullptr);

// Backward through the Kalman gains and the covariance recursion (see cov.hip):
// adds the gain and covariance terms to dk_out and dalpha, writes dr and
// dcov_in. DIAG reads the gains and dL/d(gain rows), ISO reads ||k||^2 and
// dL/dbeta. All arrays float32; k [BH, L, dk].
struct CovAdjArgs {
  bool diag;
  const float* k;
  const float* alpha;    // [BH, L] or null
  const float* r;        // [BH, L] or null
  float qvar;
  const float* pprev;    // [BH, L, dk] (DIAG) / [BH, L] (ISO): variance before each token
  const float* sden;     // [BH, L] (DIAG): the gain's denominator s_t
  const float* gains;    // [BH, L, dk] (DIAG)
  const float* dgain;    // [BH, L, dk] (DIAG)
  const float* kk;       // [BH, L] (ISO): ||k_t||^2
  const float* dbeta;    // [BH, L] (ISO): dL/dbeta_t of the equivalent delta write
  const float* dcov_out; // [BH, dk] / [BH] or null
  float* dk_out;         // [BH, L, dk], added to
  float* dalpha;         // [BH, L] or null, added to
  float* dr;             // [BH, L] or null
  float* dcov_in;        // [BH, dk] / [BH] or null
  int BH, L, dk;
};
size_t cov_adj_scratch_floats(int BH, int L, int dk, bool diag);
hipError_t launch_cov_adjoint(const CovAdjArgs& a, float* scratch, hipStream_t s);

// bf16 -> float32, n elements (the backward takes float32 operands).
hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, size_t n, hipStream_t s);

// Full-covariance Kalman gains (dk <= 64): gains [BH, L, dk] and the final covariance.
hipError_t launch_full_gains(const void* k, bool k_bf16, const float* alpha, const float* r,
                             const float* cov_in, float* cov_out, float q_noise_var,
                             void* gains, bool gains_f16, int BH, int L, int dk, hipStream_t s);

// Copy the covariance / state through unchanged (L == 0).
hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t s);

// One decode token per head; gmode 0 = delta, 1 = diagonal, 2 = isotropic gain;
// resid 0 gated, 1 plain, 2 no erase; score kind as ScoreArgs::kind.
hipError_t launch_decode(const float* q, const float* k, const float* v, const float* alpha,
                         const float* beta, const float* r, float* cov, float q_noise_var,
                         float* state, float* o, float* m, int BH, int dk, int dv, int gmode,
                         int resid, int score_kind, hipStream_t s);

// HOLA cache read + insert for one decode token per head.
hipError_t launch_hola(const float* q, const float* k, const float* v, const float* m, int32_t t,
                       float* cache_k, float* cache_v, float* cache_m, int32_t* cache_pos,
                       int32_t* cache_count, const float* sink_logit, float* o_cache,
                       float rms_eps, int B, int H, int dk, int dv, int w, int policy,
                       hipStream_t s);

// Gradients of the delta-write scan (float32); see scan_bwd.hip.
struct BwdArgs {
  const float* q;           // [BH, L, dk]
  const float* k;           // [BH, L, dk]
  const float* v;           // [BH, L, dv]
  const float* alpha;       // [BH, L] or null (= 1)
  const float* beta;        // [BH, L]
  const float* state_in;    // [BH, dk, dv] or null (= 0)
  const float* d_o;         // [BH, L, dv]
  const float* dstate_out;  // [BH, dk, dv] or null (= 0)
  float* dq;                // [BH, L, dk]
  float* dk_out;            // [BH, L, dk]
  float* dv_out;            // [BH, L, dv]
  float* dalpha;            // [BH, L] or null
  float* dbeta;             // [BH, L]
  float* dstate_in;         // [BH, dk, dv] or null
  int BH, L, dk, dv;
  int resid;                // 0 gated, 1 plain, 2 no erase
  // gain mode (Kalman writes): write vectors given as rows, beta unused
  const float* gain = nullptr;  // [BH, L, dk] or null (delta write)
  float* dgain = nullptr;       // [BH, L, dk] out: dL/d(gain rows) (gain mode)
  // workspace parts (set by launch_scan_bwd)
  float* S0s = nullptr;  // [BH, chunks, dk, dv] state at each chunk start
  float* Gs = nullptr;   // [BH, chunks, dk, dv] state gradient at each chunk end
  float* E = nullptr;    // [BH, chunks * 64, dv] residuals
  float* dR = nullptr;   // [BH, chunks * 64, dv] residual-input gradients
  float* Am = nullptr;   // [BH, chunks, 64, 64]
  float* Tm = nullptr;   // [BH, chunks, 64, 64]
  float* Pm = nullptr;   // [BH, chunks, 64, 64]
  float* M1 = nullptr;   // [BH, chunks * 64, dk] dO S0^T
  float* M2 = nullptr;   // [BH, chunks * 64, dk] dR S0^T
  float* M3 = nullptr;   // [BH, chunks * 64, dk] E G^T
  float* dPm = nullptr;  // [BH, chunks, 64, 64] dO E^T
  float* dA = nullptr;   // [BH, chunks, 64, 64] dR E^T
  float* gs0 = nullptr;  // [BH, chunks] <G, S0>
};
size_t scan_bwd_workspace_bytes(int BH, int L, int dk, int dv);
hipError_t launch_scan_bwd(BwdArgs a, void* ws, hipStream_t s);

// HOLA cache over a whole prompt in blocks; see hola_prefill.hip.
struct PrefillArgs {
  const void* q;   // [BH, L, dk] (bf16 or float32)
  const void* k;   // [BH, L, dk]
  const void* v;   // [BH, L, dv]
  const float* m;  // [BH, L] scores
  int t0, block;
  float* cache_k;  // [BH, w, dk]
  float* cache_v;  // [BH, w, dv]
  float* cache_m;  // [BH, w]
  int32_t* cache_pos;
  int32_t* cache_count;
  const float* sink_logit;  // [H] or null
  float* o_cache;           // [BH, L, dv]
  float rms_eps;
  int BH, H, L, dk, dv, w;
  int policy;  // 0: top-w by score, 1: the w most recent
  // workspace parts (prefill_bind_workspace)
  int* members;       // [BH, blocks, w] cache members each block reads
  int* member_count;  // [BH, blocks]
  int* final_src;     // [BH, w]
  float* final_m;     // [BH, w]
  int* final_pos;     // [BH, w]
  int* final_count;   // [BH]
  float* stage;       // [BH, w, dk + dv]
  float* top_m;       // [BH, blocks, w] each block's own top-w, in rank order
  int* top_pos;       // [BH, blocks, w]
  int* top_src;       // [BH, blocks, w]
};
size_t prefill_workspace_bytes(int BH, int L, int dk, int dv, int w, int block);
void prefill_bind_workspace(PrefillArgs& a, void* ws);
hipError_t launch_prefill(const PrefillArgs& a, bool in_bf16, hipStream_t s);

}  // namespace kdn
