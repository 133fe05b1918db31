// scan_mfma.hip -- chunkwise scan on the gfx950 matrix cores (d_k = 128, chunk 64).
//
// Recurrence ("A Hippocampus for Linear Attention", sec. 3.3 eq. (5), sec. 3.5)
//   e_t = v_t - alpha_t S_{t-1}^T k_t,  S_t = alpha_t S_{t-1} + b_t e_t^T,  o_t = S_t^T q_t
// in chunk form (one chunk of n <= 64 tokens, incoming state S0, chunk-local
// decay g_i = prod_{l<=i} alpha_l, write vectors b_l = beta_l k_l or the gain):
//   A = strict_lower((K B^T) * G),  G_il = g_i / g_l,  T = (I + A)^-1
//   P = lower_incl((Q B^T) * G)
//   X = V - (diag(g) K) S0,  U = T X  (U are the residuals e_t)
//   O = (diag(g) Q) S0 + P U
//   S = g_n S0 + (diag(w) B)^T U,  w_l = (g_n / g_l) beta_l  (1 in place of beta for a gain)
// The plain residual e_t = v_t - S_{t-1}^T k_t (same update) unrolls to the
// same form with the exclusive decay g_{t-1} = g_t / alpha_t in the rows of A
// and in X: A_tl = (k_t . b_l) g_{t-1} / g_l, X = V - diag(g_{t-1}) K S0;
// every decay ratio stays <= 1, so no factor grows when alpha_t is small.
// The write without its erase term (e_t = v_t, decayed linear attention) is
// the same form with no decay at all in the residual: A = 0, T = I, X = V.
//
// Two kernels:
//  * prep_kernel: every chunk independent of the others; a workgroup takes
//    one chunk of one head (two consecutive ones past 16384 chunks, loading
//    the second one's inputs while it computes the first).
//    Everything that does not depend on the state: the per-token decay
//    scalars g_t, w_t; for the diagonal Kalman write the gains themselves
//    (each coordinate's variance carried through the chunk's two 32-token
//    halves from the starting variances of the covariance scan, the gains
//    written out for the state kernel); the Grams K B^T and Q B^T on the
//    matrix cores; and
//    T = (I + A)^-1 by blocks of 16: the four diagonal blocks are inverted in
//    float32 registers (one wavefront per block, four lanes per column, quad
//    reductions through DPP), the six off-diagonal blocks follow by block
//    products on the matrix cores, diagonal by diagonal:
//    T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj.
//    Output per (head, chunk): T (and P for the Kalman writes) in fp16, and
//    the token scalars.
//  * state_kernel: one workgroup per (head, 32-column slice of d_v); the loop
//    over chunks is sequential. One wavefront carries the chain (K S, U = T X,
//    state update) with the float32 state slice (128 x 32) in its matrix-core
//    accumulators for the whole sequence, one writes the outputs of the chunk
//    before, two stage the inputs; details at the kernel.
//
// Matrix products are fp16 x fp16 -> fp32: v_mfma_f32_16x16x32_f16 in the
// prepare kernel, v_mfma_f32_32x32x16_f16 in the state kernel. bf16 inputs are
// converted to fp16 when staged (exact for bf16 values of magnitude in
// [2^-14, 65504]). fp16 rather than bf16 operands because the intermediate
// operands (S, X, U, P, T) need the 3 extra significand bits: with bf16
// operands the output error at the gated-delta workload is ~3.7e-2 RMS(o),
// with fp16 ~5e-3.
//
// Range: fp16 operands overflow above 65504. The state, the values and the
// residuals are therefore carried scaled by powers of two, which is exact:
// the producers stage a chunk's values times 2^e_p when its largest finite
// |v| reaches 2^12 (e_p = 11 - floor(log2 max), else 0), and the chain keeps
// S * 2^e_S in its accumulators. It checks max |S * 2^e_S| while a chunk's
// K S products run; at the next chunk start, if that reached 2^11 (or stayed
// below 2^5 with e_S < 0), e_S is recomputed from the state so that its
// largest finite entry lies in [2^9, 2^10) (e_S = 0 if the state is below
// 2^11). Then e_S is lowered to the chunk's value exponents if they are
// lower, and value rows staged at a higher exponent are scaled down in
// place, so one exponent holds for the whole chunk. The recurrence is linear
// in (V, S, U, O), so the residuals and outputs come out scaled and are
// unscaled when stored. With values and states below 2^11 nothing is scaled;
// the step itself never branches on the range.
//
// Operand layouts: an MFMA reads A as [m][k] and B as [n][k] with k contiguous
// (16-byte LDS reads); its result gives each lane 4 consecutive rows of one
// column, which is written either as [n][m] (one 8-byte write) or [m][n]
// (four 2-byte writes). Every buffer below is laid out for its reader.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <utility>

#include "kdn_internal.h"

namespace kdn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int C = 64;          // chunk length
constexpr int DK = 128;        // key dimension
constexpr int DV = 32;         // value columns per workgroup
constexpr int KP = DK + 8;     // fp16 pitch of [token][d_k] tiles (272 B: conflict-free rows)
constexpr int CP = C + 8;      // fp16 pitch of [.][token] tiles (144 B)

// Per (head, chunk) record written by prep_kernel and read by state_kernel:
//   T  = (I + A)^-1 as its three nonzero 32 x 32 blocks (rows/cols 0-31,
//        rows 32-63 x cols 0-31, rows/cols 32-63), fp16, row-major per block;
//   P  (Kalman writes only) in the same three-block form;
//   scalars, three float4 per token: (g_x, w, log2 g, write scale),
//        (R, Cf, f0, f1), (value scale, extreme, g, 0), where g_x is the decay
//        the residual sees (g_{t-1} for the plain residual, else g). They factor the decay
//        ratio of the masked query-key product bs_l g_i / g_l (l <= i):
//        across the two 32-token halves as f0_l f1_i with
//        f0_l = bs_l g_31 / g_l (l < 32), f1_i = g_i / g_31 (i >= 32), both
//        <= bs_l resp. 1; inside a half b as R_l Cf_i with
//        R_l = bs_l g_r / g_l, Cf_i = g_i / g_r, r = 32 b + 15. Those can
//        overflow only for decay faster than 2^-100 over 16 tokens; the chunk's
//        `extreme` flag (1.0) then selects exp2 of log2 g differences instead.
// The delta write's P is formed by the state kernel from the staged Q and K.
constexpr size_t kTriBytes = 3 * 32 * 32 * 2;     // 6144
constexpr size_t kRecT = 0;
__host__ __device__ constexpr size_t rec_p_off(bool gain) { return gain ? kTriBytes : 0; }
__host__ __device__ constexpr size_t rec_s_off(bool gain) { return gain ? 2 * kTriBytes : kTriBytes; }
__host__ __device__ constexpr size_t rec_bytes(bool gain) { return rec_s_off(gain) + (size_t)C * 48; }
// element (row, col) of a lower-triangular 64 x 64 matrix in three-block form (col <= row block)
__host__ __device__ constexpr int tri_index(int row, int col) {
  return row < 32 ? row * 32 + col : (col < 32 ? 1024 + (row - 32) * 32 + col : 2048 + (row - 32) * 32 + col - 32);
}

__device__ __forceinline__ floatx4 mfma(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 ld8(const _Float16* p) {
  return *reinterpret_cast<const half8*>(p);
}
__device__ __forceinline__ void st4(_Float16* p, floatx4 x) {
  half4 h;
  h[0] = (_Float16)x[0];
  h[1] = (_Float16)x[1];
  h[2] = (_Float16)x[2];
  h[3] = (_Float16)x[3];
  *reinterpret_cast<half4*>(p) = h;
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Two floats -> two fp16 in one dword (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pk_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{lo, hi}, half2v));
}

// 8 bf16 values (one 16-byte load), each times `scale`, -> 8 fp16 values.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 u, float scale) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pk_f16(__uint_as_float(w[i] << 16) * scale, __uint_as_float(w[i] & 0xffff0000u) * scale);
  return make_uint4(r[0], r[1], r[2], r[3]);
}
// The same without a scale.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pk_f16(__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xffff0000u));
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// 8 fp16 values times `scale` -> 8 fp16 values.
__device__ __forceinline__ uint4 f16x8_scale(uint4 u, float scale) {
  half8 h = __builtin_bit_cast(half8, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)((float)h[i] * scale);
  return __builtin_bit_cast(uint4, h);
}

__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_prefix(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Lower 16x16 tile number tl (0..9) -> (ti, tj), ti >= tj, row-major order.
__device__ __forceinline__ void tile_ij(int tl, int& ti, int& tj) {
  ti = tl < 1 ? 0 : tl < 3 ? 1 : tl < 6 ? 2 : 3;
  tj = tl - ti * (ti + 1) / 2;
}

// =====================================================================  prep kernel

struct PrepArgs {
  const uint16_t* q;      // bf16 [BH, L, DK]
  const uint16_t* k;      // bf16 [BH, L, DK]
  const _Float16* gain;   // fp16 [BH, L, DK] or null (delta write)
  const float* alpha;     // [BH, L] or null
  const float* beta;      // [BH, L]
  unsigned char* rec;     // [BH, nchunks] records of rec_bytes(gain)
  int L, nchunks, plain, noerase;
  int cpw;                // consecutive chunks per workgroup
  // diagonal Kalman write with its gains formed here (else null): the starting
  // variances of every half chunk [BH, nsub, DK], observation noise
  // [BH, L] (null: 1), process noise variance, the fp16 gains written out
  // [BH, L, DK], and the variances after the last token [BH, DK] (or null)
  int nsub = 0;
  const float* dmaps = nullptr;
  const float* r = nullptr;
  float qvar = 0.f;
  _Float16* gain_out = nullptr;
  float* cov_out = nullptr;
};

constexpr int kAdP = 17;  // fp32 pitch of the diagonal blocks of A
constexpr int kPrepR1 = (C * KP > 2 * C * CP ? C * KP : 2 * C * CP) * 2;  // a tile, later sT + sTt

// The delta write stages only K, which then shares the first region with T.
// The Kalman writes stage K, then Q, then P in one tile, and the gains in the
// first region, which then takes T (53.5 KB: three workgroups per CU). The
// diagonal Kalman write with its gains formed here adds a token array.
size_t prep_lds_bytes(bool gain, bool diagf = false) {
  return (size_t)kPrepR1 + (gain ? (size_t)C * KP * 2 : 0) +
         (size_t)C * CP * 2 + (size_t)4 * 16 * kAdP * 4 + (size_t)4 * 16 * 24 * 2 +
         (size_t)3 * C * 4 + (diagf ? (size_t)C * 4 : 0);
}
// fp32 pitch of the per-(token, coordinate) terms p-_i k_i^2 summed for the
// gain denominators (they borrow the region from the gains tile to the end of
// the per-wavefront scratch)
constexpr int kKuP = DK + 1;

// Cache policy of the prepare kernel's stores for the Kalman writes: nt
// (marked for early eviction). Their records and gains, 130 MB at the gated
// workload's shape, then leave the caches to the state kernel's other reads
// (diagonal write: 275 -> 264 us per step); the delta write keeps the default
// policy for its records (its state kernel was 101 against 107 us).
constexpr int kNtStore = 2;

// One chunk's inputs in registers: this thread's four 16-byte pieces of K
// (and of Q and the gains), token `lane`'s alpha and beta (and r), and with
// the gains formed here the variance of coordinate tid mod d_k at the start of
// half tid / d_k of the chunk.
template <bool GAIN>
struct PrepIn {
  uint4 k[4], q[GAIN ? 4 : 1], g[GAIN ? 4 : 1];
  float al, be, rn, pv;
};

// Loads chunk cc of head bh through buffer descriptors over the head's rows:
// rows past the sequence read as zero, and so does every load when `has` is
// false (descriptor range 0, no memory access). No load sits behind a branch,
// which keeps the compiler's wait counts exact.
template <bool GAIN, bool DIAGF>
__device__ __forceinline__ void prep_load(const PrepArgs& a, int bh, int cc, bool has, int tid, int lane,
                                          PrepIn<GAIN>& x) {
  const size_t head_tok = (size_t)bh * a.L;
  const size_t rows = has ? (size_t)a.L * DK * 2 : 0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + head_tok * DK, rows);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int seg = tid + NT * i, row = seg >> 4, c8 = seg & 15;
    const int off = ((cc * C + row) * DK + c8 * 8) * 2;
    x.k[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    if (GAIN) {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + head_tok * DK, rows);
      x.q[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      if (!DIAGF) {
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gain + head_tok * DK, rows);
        x.g[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
      }
    }
  }
  const int toff = (cc * C + lane) * 4;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.alpha + (a.alpha ? head_tok : 0), has && a.alpha ? (size_t)a.L * 4 : 0);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.beta + (a.beta ? head_tok : 0), has && a.beta ? (size_t)a.L * 4 : 0);
  x.al = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, toff, 0, 0));
  x.be = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, toff, 0, 0));
  if (DIAGF) {
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.r + (a.r ? head_tok : 0), has && a.r ? (size_t)a.L * 4 : 0);
    x.rn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, toff, 0, 0));
    // a half past the sequence reads zero (its tokens are all padding)
    const __amdgpu_buffer_rsrc_t rm =
        make_rsrc(a.dmaps + (size_t)bh * a.nsub * DK, has ? (size_t)a.nsub * DK * 4 : 0);
    x.pv = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rm, ((2 * cc + (tid >> 7)) * DK + (tid & (DK - 1))) * 4, 0, 0));
  } else {
    x.rn = x.pv = 0.f;
  }
}

template <bool GAIN, bool DIAGF>
__global__ __launch_bounds__(NT) void prep_kernel(PrepArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  constexpr bool gain = GAIN;
  static_assert(GAIN || !DIAGF, "the gains are formed here only for the diagonal Kalman write");
  unsigned char* p = lds_raw;
  // delta write: K [C][KP] (phases 1-2) in the first region, then T;
  // Kalman writes: K, then Q (phase 2), then P [C][CP] in one tile, the
  // gains [C][KP] (phases 1-2) in the first region, then T
  _Float16* sK = reinterpret_cast<_Float16*>(p);
  if (gain) p += C * KP * 2;
  _Float16* sB = reinterpret_cast<_Float16*>(p);   // write vectors (K for the delta write)
  _Float16* sT = sB;                               // [C][CP] (phases 3-5)
  _Float16* sTt = sT + C * CP;                     // [C][CP] T transposed
  p += kPrepR1;
  _Float16* sQ = sK;                               // [C][KP] (phase 2, Kalman writes)
  _Float16* sP = sK;                               // [C][CP] (phases 3-5, Kalman writes)
  _Float16* sAh = reinterpret_cast<_Float16*>(p);  // [C][CP] A in fp16
  p += C * CP * 2;
  float* sAd = reinterpret_cast<float*>(p);        // [4][16][kAdP] diagonal blocks of A
  p += 4 * 16 * kAdP * 4;
  _Float16* sM = reinterpret_cast<_Float16*>(p);   // [4][16][24] per-wavefront scratch
  p += 4 * 16 * 24 * 2;
  float* sLg = reinterpret_cast<float*>(p);        // [C] log2 of g
  float* sBs = sLg + C;                            // [C] write scale
  float* sLgx = sBs + C;                           // [C] log2 of g_x (rows of A)
  // diagonal Kalman write, gains formed here: per token sum_i p-_i k_i^2, and
  // the terms of those sums (they borrow the gains tile and what follows it)
  float* sSd = sLgx + C;                           // [C]
  float* sKu = reinterpret_cast<float*>(sB);       // [C][kKuP] p-_i k_i^2 (before the Grams)
  static_assert(C * kKuP * 4 <= kPrepR1 + C * CP * 2 + 4 * 16 * kAdP * 4 + 4 * 16 * 24 * 2,
                "the terms of the gain denominators fit from the gains tile to the token arrays");

  const int bh = blockIdx.x;
  const int cbeg = blockIdx.y * a.cpw, cend = min(cbeg + a.cpw, a.nchunks);

  PrepIn<GAIN> in;
  prep_load<GAIN, DIAGF>(a, bh, cbeg, true, threadIdx.x, threadIdx.x & 63, in);
  // As many stores as a chunk issues after its next chunk's loads (3 scalar
  // pieces, 2 rounds of T and P pieces; with the gains formed here 4 pieces of
  // gains and a variance), all dropped (range 0): the wait for a
  // chunk's inputs is then the same on entry as around the loop, and the
  // compiler does not fall back to waiting for every store in flight.
  {
    const __amdgpu_buffer_rsrc_t none = make_rsrc(a.rec, 0);
    const v4u32 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 3 + 2 * (GAIN ? 2 : 1) + (DIAGF ? 4 : 0); ++i)
      __builtin_amdgcn_raw_buffer_store_b128(z, none, 0, 0, 0);
    if (DIAGF) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 0, 0, 0);
  }
  for (int c = cbeg; c < cend; ++c) {
    // The lane index passes through an empty asm statement each chunk: the
    // compiler then forms the many LDS addresses that derive from it where they
    // are used, instead of hoisting them out of the loop and holding them all
    // in registers (which would cost occupancy or spill).
    int lane_opaque = threadIdx.x & 63;
    asm volatile("" : "+v"(lane_opaque));
    const int lane = lane_opaque, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tid = wave * 64 + lane;
    const int r16 = lane & 15, kq = lane >> 4, k8 = kq * 8;
    const int c0 = c * C, n = min(C, a.L - c0);
    unsigned char* rec = a.rec + ((size_t)bh * a.nchunks + c) * rec_bytes(gain);

    // phase 1: stage K (and the gains when they come from the gains kernel)
    // as fp16 from the registers, start loading the next chunk, per-token
    // scalars (Kalman writes: Q is staged over K once the A Gram is done; its
    // pieces wait in registers)
    uint4 q_cur[GAIN ? 4 : 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int seg = tid + NT * i, row = seg >> 4, c8 = seg & 15;
      *reinterpret_cast<uint4*>(sK + row * KP + c8 * 8) = bf16x8_to_f16x8(in.k[i]);
      if (GAIN) {
        q_cur[GAIN ? i : 0] = in.q[GAIN ? i : 0];
        if (!DIAGF) *reinterpret_cast<uint4*>(sB + row * KP + c8 * 8) = in.g[GAIN ? i : 0];
      }
    }
    const float al_in = in.al, be_in = in.be, rn_in = in.rn, pv_in = in.pv;
    prep_load<GAIN, DIAGF>(a, bh, c + 1, c + 1 < cend, tid, lane, in);
    // Every wavefront forms the scalars (token = lane); wavefront 0 keeps them
    // in LDS and stores them. The record is written through buffer stores
    // that every wavefront issues, the others at an offset past the record
    // (dropped), so the number of stores in flight is the same on every path
    // and the wait for the next chunk's loads does not include them.
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, rec_bytes(gain));
    constexpr int kDrop = 1 << 30;  // past any record
    {
      float la = 0.f, bs = 0.f;
      const float vs = 1.f;
      if (lane < n) {
        const float al = a.alpha ? al_in : 1.f;
        la = log2f(al);
        bs = gain ? 1.f : be_in;
      }
      const float lg = wave_prefix(la, lane);
      // the residual's decay: exclusive for plain, none (g_x = 0: A = 0,
      // T = I and X = V) for the write without its erase term
      const float lgx = a.noerase ? -INFINITY : a.plain ? lg - la : lg;
      const float lgn = __shfl(lg, n - 1, 64);
      const float lg31 = __shfl(lg, 31, 64);
      const float lgr = __shfl(lg, (lane & 32) + 15, 64);   // reference of this half
      if (wave == 0) {
        sLg[lane] = lg;
        sBs[lane] = bs;
        sLgx[lane] = lgx;
      }
      const float w = lane < n ? exp2f(lgn - lg) * bs : 0.f;
      // exponents of R and Cf stay in [-100, 100] unless the decay is extreme
      const float span = fabsf(lgr - lg);
      const bool extreme = __ballot(span > 100.f) != 0;
      // default (write-back) stores: the state kernel reads the records soon after
      const int so = wave == 0 ? (int)rec_s_off(gain) + 48 * lane : kDrop;
      const float4 s0 = make_float4(exp2f(lgx), w, lg, bs);
      const float4 s1 = make_float4(extreme ? 0.f : bs * exp2f(lgr - lg), extreme ? 0.f : exp2f(lg - lgr),
                                    lane < 32 ? bs * exp2f(lg31 - lg) : 0.f,
                                    lane >= 32 ? exp2f(lg - lg31) : 0.f);
      const float4 s2 = make_float4(vs, extreme ? 1.f : 0.f, exp2f(lg), 0.f);
      constexpr int rpol = GAIN ? kNtStore : 0;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, s0), rr, so, 0, rpol);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, s1), rr, so + 16, 0, rpol);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, s2), rr, so + 32, 0, rpol);
    }
    __syncthreads();

    if constexpr (DIAGF) {
      // The diagonal Kalman gains of this chunk ("Kalman Delta Networks",
      // abstract: the mean-field diagonal covariance), as the separate gains
      // kernel forms them. Lane i of wavefronts 0 and 1 carries coordinate i's
      // variance through the first half of the chunk's tokens, wavefronts 2
      // and 3 through the second half, each from the variance the covariance
      // scan gives at the start of its half (p- = a^2 p + Q, u = p- k,
      // p = p- r / (r + p- k^2)). The denominators s_t = r_t + sum_i p-_i k_i^2
      // are summed through LDS; the gains u_t / s_t go to the write-vector tile
      // and to the gains buffer. The per-token scalars are read across lanes
      // (token = lane in every wavefront), the keys from the staged tile.
      constexpr int TH = C / 2;
      const int ci = 64 * (wave & 1) + lane, t0h = TH * (wave >> 1);
      // tokens past the sequence: alpha = r = 1 and no process noise (their
      // zero keys then leave p alone)
      const float al = lane < n && a.alpha ? al_in : 1.f;
      const float a2l = al * al, qnl = (1.f - al) * (1.f + al) * a.qvar;
      const float rl = lane < n && a.r ? rn_in : 1.f;
      float kf[TH], u[TH];
#pragma unroll
      for (int t = 0; t < TH; ++t) kf[t] = (float)sK[(t0h + t) * KP + ci];
      float pv = pv_in;
#pragma unroll
      for (int t = 0; t < TH; ++t) {
        const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a2l), t0h + t));
        const float qn = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qnl), t0h + t));
        const float rt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rl), t0h + t));
        const float pm = fmaf(a2, pv, qn);
        u[t] = pm * kf[t];
        pv = pm * rt * __builtin_amdgcn_rcpf(fmaf(u[t], kf[t], rt));
      }
#pragma unroll
      for (int t = 0; t < TH; ++t) sKu[(t0h + t) * kKuP + ci] = u[t] * kf[t];
      {  // the variances after the sequence's last token: from the half that holds it
        const bool last = c == a.nchunks - 1 && (wave >> 1) == (n - 1) / TH;
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(a.cov_out + (a.cov_out ? (size_t)bh * DK : 0), a.cov_out ? (size_t)DK * 4 : 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pv), rc, last ? ci * 4 : kDrop, 0, 0);
      }
      __syncthreads();
      {  // sum_i p-_i k_i^2: four lanes per token
        const int t = tid >> 2, part = tid & 3;
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < DK / 4; ++j) sum += sKu[t * kKuP + part + 4 * j];
        sum += __shfl_xor(sum, 1, 64);
        sum += __shfl_xor(sum, 2, 64);
        if (part == 0) sSd[t] = sum;
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < TH; ++t) {
        const float rt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rl), t0h + t));
        // reciprocal by v_rcp_f32 (1 ulp), as in the gains kernel
        sB[(t0h + t) * KP + ci] = (_Float16)(u[t] * __builtin_amdgcn_rcpf(rt + sSd[t0h + t]));
      }
      __syncthreads();
      {  // gains rows to the buffer the state kernel reads (rows past the sequence dropped)
        const size_t head_tok = (size_t)bh * a.L;
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gain_out + head_tok * DK, (size_t)a.L * DK * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int seg = tid + NT * i, row = seg >> 4, c8 = seg & 15;
          const uint4 gv = *reinterpret_cast<const uint4*>(sB + row * KP + c8 * 8);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, gv), rg,
                                                 ((c * C + row) * DK + c8 * 8) * 2, 0, kNtStore);
        }
      }
    }

    // phase 2: 20 lower Gram tiles, A (tiles 0-9) from K and P (tiles 10-19) from Q;
    // wavefront w takes tiles w, w + 4, ..., w + 16. The Kalman writes stage
    // Q over K between the A and the P tiles.
    floatx4 pacc[3];
    int pti[3], ptj[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      pacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
      pti[j] = ptj[j] = -1;
    }
    int np = 0;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int tl = wave + 4 * j;
      const bool isP = tl >= 10;
      if (isP && !gain) continue;
      if (gain && tl == 10 + (wave + 2) % 4) {
        // the first P tile of this wavefront: every wavefront's A tiles (its
        // tiles below 10) are done reading K
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int seg = tid + NT * i, row = seg >> 4, c8 = seg & 15;
          *reinterpret_cast<uint4*>(sQ + row * KP + c8 * 8) = bf16x8_to_f16x8(q_cur[GAIN ? i : 0]);
        }
        __syncthreads();
      }
      int ti, tj;
      tile_ij(isP ? tl - 10 : tl, ti, tj);
      const _Float16* srcA = isP ? sQ : sK;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
        acc = mfma(ld8(srcA + (16 * ti + r16) * KP + 32 * ks + k8),
                   ld8(sB + (16 * tj + r16) * KP + 32 * ks + k8), acc);
      const int col = 16 * tj + r16;
      const float lgc = sLg[col], bsc = sBs[col];
      // rows of A take the residual's decay, rows of P the read-out's
      const float4 lgr = *reinterpret_cast<const float4*>((isP ? sLg : sLgx) + 16 * ti + kq * 4);
      const float lgrv[4] = {lgr.x, lgr.y, lgr.z, lgr.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = 16 * ti + kq * 4 + jj;
        const float e = __builtin_amdgcn_exp2f(fminf(lgrv[jj] - lgc, 0.f)) * bsc;
        const bool keep = isP ? row >= col : row > col;
        acc[jj] = keep ? acc[jj] * e : 0.f;
      }
      if (isP) {
        // wave-uniform slot index: tiles 10-19 of this wavefront in order
        if (np == 0) { pacc[0] = acc; pti[0] = ti; ptj[0] = tj; }
        else if (np == 1) { pacc[1] = acc; pti[1] = ti; ptj[1] = tj; }
        else { pacc[2] = acc; pti[2] = ti; ptj[2] = tj; }
        ++np;
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int row = 16 * ti + kq * 4 + jj;
          sAh[row * CP + col] = (_Float16)acc[jj];
          if (ti == tj) sAd[(ti * 16 + (row & 15)) * kAdP + (col & 15)] = acc[jj];
        }
      }
    }
    __syncthreads();
    // P tiles into LDS (sK is free now)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (pti[j] >= 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          sP[(16 * pti[j] + kq * 4 + jj) * CP + 16 * ptj[j] + r16] = (_Float16)pacc[j][jj];
      }
    }

    // phase 3: diagonal blocks D_b = (I + A_bb)^-1 in float32.
    // Lane (j = lane / 4, q = lane % 4) owns rows 4q..4q+3 of column j.
    {
      const int b = wave, j = lane >> 2, q = lane & 3;
      float am[16][4];
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) am[i][m] = sAd[(b * 16 + i) * kAdP + 4 * q + m];
      float x[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) x[m] = (4 * q + m == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        float s = am[i][0] * x[0];
        s = fmaf(am[i][1], x[1], s);
        s = fmaf(am[i][2], x[2], s);
        s = fmaf(am[i][3], x[3], s);
        s += dpp_xor1(s);
        s += dpp_xor2(s);
        const float t = (i == j ? 1.f : 0.f) - s;
        if ((i >> 2) == q) x[i & 3] = t;
      }
      const int r0 = 16 * b + 4 * q, cc = 16 * b + j;
#pragma unroll
      for (int m = 0; m < 4; ++m) sT[(r0 + m) * CP + cc] = (_Float16)x[m];
      floatx4 xv = {x[0], x[1], x[2], x[3]};
      st4(sTt + cc * CP + r0, xv);
    }
    __syncthreads();

    // phase 4: off-diagonal blocks, one diagonal at a time.
    {
      _Float16* myM = sM + wave * 16 * 24;
      const half8 zero8 = {};
      for (int d = 1; d < 4; ++d) {
        const int i = wave + d, j = wave;
        const bool active = wave < 4 - d;
        if (active) {
          // M = sum_{k=j}^{i-1} A_ik T_kj  (contraction over columns [16j, 16i))
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          for (int kb = 16 * j; kb < 16 * i; kb += 32) {
            const int kk = kb + k8;
            const bool ok = kk < 16 * i;
            const half8 av = ok ? ld8(sAh + (16 * i + r16) * CP + kk) : zero8;
            const half8 bv = ok ? ld8(sTt + (16 * j + r16) * CP + kk) : zero8;
            acc = mfma(av, bv, acc);
          }
          st4(myM + r16 * 24 + kq * 4, acc);  // M^T[col][rows]
        }
        // no barrier: M is this wavefront's own scratch (LDS accesses of one
        // wavefront stay in order), D_i was written before the last barrier,
        // and no wavefront reads a block of this diagonal during it
        if (active) {
          // T_ij = -D_i M
          const bool ok = kq < 2;
          const half8 av = ok ? ld8(sT + (16 * i + r16) * CP + 16 * i + k8) : zero8;
          const half8 bv = ok ? ld8(myM + r16 * 24 + k8) : zero8;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = mfma(av, bv, acc);
          acc = -acc;
          const int row0 = 16 * i + kq * 4, col = 16 * j + r16;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) sT[(row0 + jj) * CP + col] = (_Float16)acc[jj];
          st4(sTt + col * CP + row0, acc);
        }
        __syncthreads();
      }
    }

    // phase 5: T (and P) to the record in three-block form. Each block is 32
    // rows x 64 bytes = 128 pieces of 16 bytes, 384 pieces in all: two rounds
    // over the workgroup, the second one's pieces past 384 dropped.
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      const int seg = tid + NT * round;
      const bool ok = seg < 384;
      const int sg = ok ? seg : seg - NT;  // a piece to read; its store is dropped
      const int blk = sg >> 7, brow = (sg >> 2) & 31, piece = sg & 3;
      const int row = (blk == 0 ? 0 : 32) + brow, col = (blk == 2 ? 32 : 0) + 8 * piece;
      const int off = ok ? 2 * (blk * 1024 + brow * 32 + 8 * piece) : kDrop;
      // 16 x 16 blocks above the diagonal were never written: zeros
      const bool lower = (col >> 4) <= (row >> 4);
      uint4 tv = *reinterpret_cast<const uint4*>(sT + row * CP + col);
      if (!lower) tv = make_uint4(0, 0, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, tv), rr, (int)kRecT + off, 0,
                                             GAIN ? kNtStore : 0);
      if (gain) {
        uint4 pv = *reinterpret_cast<const uint4*>(sP + row * CP + col);
        if (!lower) pv = make_uint4(0, 0, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, pv), rr,
                                               ok ? (int)rec_p_off(gain) + off : kDrop, 0, kNtStore);
      }
    }
    __syncthreads();  // the next chunk's staging overwrites sT, sP and the scalars
  }
}

// =====================================================================  state kernel
//
// One workgroup per (head, 32-column slice of d_v), four wavefronts with
// fixed roles and one workgroup barrier per step. Step c:
//  * wavefront 0 carries the sequential chain of chunk c:
//      K S (16 products), X = v_scale V - g K S, U = T X (6), and the state
//      update S = g_n S + (diag(w) B)^T U (16).
//    The float32 state slice (128 x 32) lives in its 32x32 accumulators for
//    the whole sequence, and every intermediate (S, X, U in fp16) goes from
//    one product's accumulator straight into the next product's operand
//    registers (see "operand k order" below). The transposed write vectors
//    come from the staged [token][d_k] tile by ds_read_b64_tr_b16. Chunk c's
//    incoming state and its residuals U go to an exchange buffer.
//  * wavefront 1 writes the outputs of chunk c - 1 from the exchange buffer:
//    O = diag(g) Q S + P U. For the delta write it also forms P from the
//    staged Q and K as P^T = K Q^T (masked, scaled by the decay ratios), whose
//    accumulator layout is directly the operand layout of P U; for the Kalman
//    writes P comes with the prepare record.
//  * wavefronts 2-3 stage into LDS what wavefront 0 reads for chunk c + 1 (K,
//    the gains for the Kalman writes, V scaled by the value scale, T, token
//    scalars) and what wavefront 1 reads for chunk c (Q, or P for the Kalman
//    writes), from registers loaded two steps earlier with 1 KB loads of
//    consecutive bytes. Wavefronts 0 and 1 never wait on global memory.
//    Chain stages are triple-buffered for the delta write (wavefront 1 reads
//    chunk c - 1's K and scalars while chunk c + 1 is staged).
// Each wavefront's products are software-pipelined by hand: operand reads are
// issued a few products ahead and scheduling fences keep the compiler from
// regrouping them (the LDS counter tracks at most 15 reads, so issuing
// everything up front would serialise). Loads of rows past the end of the
// sequence go through buffer descriptors sized to the head, which return
// zeros; output stores past it are dropped the same way.
//
// Operand k order: the 32x32x16 accumulator gives lane (h = lane / 32, col)
// the rows 8 j + 4 h + r (j, r = 0..3) of a 32-row block. Registers 8 i ..
// 8 i + 7 of such a block are used as the operand of k step i + 2 (block),
// so within a 16-wide k step, operand slot e of half h stands for index
// 8 (e / 4) + 4 h + e % 4. Operands read from memory follow the same order:
// two 8-byte reads at columns 4 h and 8 + 4 h of the k step.

typedef float floatx16 __attribute__((ext_vector_type(16)));

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N - 1>).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
typedef short short4v __attribute__((ext_vector_type(4)));
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 cat(half4 a, half4 b) {
  return half8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ half4 ld4(const _Float16* p) {
  return *reinterpret_cast<const half4*>(p);
}
// operand of one 16-wide k step from a row whose k step starts at p
__device__ __forceinline__ half8 ld_op(const _Float16* p, int h) {
  return cat(ld4(p + 4 * h), ld4(p + 8 + 4 * h));
}

// Transposing LDS read: within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte blocks addressed by lanes i / 4, i / 4 + 4, i / 4 + 8,
// i / 4 + 12. A group whose lanes address 4 rows x 4 column quads
// (lane 4 r + q: row r, quad q) returns one column per lane, 4 rows deep.
__device__ __forceinline__ half4 ld_tr(const _Float16* p) {
  const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p));
  return __builtin_bit_cast(half4, v);
}

// The delta write's output stores stream on the 32-column tiling
// (kStreamStore, kdn_internal.h): the outputs are never read back by the
// kernel, and keeping them out of L2 leaves it to the keys, queries and
// records that the four d_v slices of a head share (measured: its state kernel
// 98 against 116 us with default stores). With default stores the slices'
// pieces of each output row meet in L2 before they go to HBM instead; that
// wins for the Kalman writes' state kernel, which also reads the gain rows and
// the output's Q rows (153 against 169 us on the diagonal write at the gated
// workload's shape), and for the 16-column tiling, whose eight slices store
// 64-byte pieces of each row (the long workload's step 1.74 against 1.81 ms).
// Non-temporal loads are much slower and are not used.
template <bool GAIN, bool NARROW>
constexpr int out_store_policy() { return GAIN || NARROW ? 0 : kStreamStore; }

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// 4 bf16 values (8 bytes) -> 4 fp16 values.
__device__ __forceinline__ half4 bf16x4_to_f16x4(uint2 u) {
  return __builtin_bit_cast(half4, make_uint2(pk_f16(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u)),
                                              pk_f16(__uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u))));
}

struct StateArgs {
  int* uexp;             // e_S of every (head, slice, chunk) for the write scores, or null
  const uint16_t* q;     // bf16 [BH, L, DK]
  const uint16_t* k;     // bf16 [BH, L, DK]
  const uint16_t* v;     // bf16 [BH, L, dv]
  const _Float16* gain;  // fp16 [BH, L, DK] or null
  const unsigned char* rec;
  const float* state_in;
  float* state_out;
  void* o;
  half8* ubuf;           // residuals for the write scores, or null
  int BH, L, dv, nchunks, ntiles;
};

constexpr int NT_STATE = 256;
constexpr int VP = DV + 8;  // fp16 pitch of the staged V rows

// LDS, per chain stage (3 for the delta write, 2 for the Kalman writes):
//   K [C][KP]; gains [C][KP] (Kalman); T [C][CP] (lower blocks only);
//   V times 2^e_p [C][VP]; nine token scalars [9][C] (g_x, w, log2 g, write
//   scale, R, Cf, f0, f1, g), the chunk's extreme-decay flag and the two
//   producers' value exponents (floor log2 of their rows' largest finite |v|);
// per output stage (2): Q [C][KP] (delta) or P [C][CP] and g [C] (Kalman);
// per exchange buffer (2): S (8 k steps) and U (4 k steps), 16 bytes per lane
// and k step in wavefront-0 register order.
constexpr size_t kStK = (size_t)C * KP * 2;
constexpr size_t kStT = (size_t)C * CP * 2;
constexpr size_t kStV = (size_t)C * VP * 2;
constexpr size_t kStSc = (size_t)9 * C * 4 + 16;
constexpr size_t kExBytes = (size_t)12 * 64 * 16 + 16;  // S, U, then their exponent
__host__ __device__ constexpr int n_chain_stages(bool gain) { return gain ? 2 : 3; }
__host__ __device__ constexpr size_t chain_stage_bytes(bool gain) {
  return kStK * (gain ? 2 : 1) + kStT + kStV + kStSc;
}
__host__ __device__ constexpr size_t out_stage_bytes(bool gain) {
  return gain ? kStT + (size_t)C * 4 : kStK;
}
size_t state_lds_bytes(bool gain) {
  return n_chain_stages(gain) * chain_stage_bytes(gain) + 2 * out_stage_bytes(gain) + 2 * kExBytes;
}

struct ChainStage {
  _Float16* k;   // K
  _Float16* b;   // write vectors: K (delta) or the gains
  _Float16* t;
  _Float16* v;
  float* g;      // token scalars: g_x (the residual's decay)
  float* w;
  float* lg;
  float* bs;
  float* f0;
  float* f1;
  float* rr;
  float* cf;
  float* go;     // g (the read-out's decay)
  float* extreme;
  int* vexp;     // [2] exponents of the largest finite |v| of rows 0-31, 32-63 (< 12: all below 2^12)
};
struct OutStage {
  _Float16* q;   // delta write
  _Float16* p;   // Kalman writes
  float* g;      // Kalman writes
};
template <bool GAIN>
__device__ __forceinline__ ChainStage chain_stage(unsigned char* lds, int buf) {
  unsigned char* p = lds + (size_t)buf * chain_stage_bytes(GAIN);
  ChainStage s;
  s.k = reinterpret_cast<_Float16*>(p); p += kStK;
  s.b = s.k;
  if (GAIN) { s.b = reinterpret_cast<_Float16*>(p); p += kStK; }
  s.t = reinterpret_cast<_Float16*>(p); p += kStT;
  s.v = reinterpret_cast<_Float16*>(p); p += kStV;
  float* f = reinterpret_cast<float*>(p);
  s.g = f; s.w = f + C; s.lg = f + 2 * C; s.bs = f + 3 * C; s.f0 = f + 4 * C; s.f1 = f + 5 * C;
  s.rr = f + 6 * C; s.cf = f + 7 * C; s.go = f + 8 * C; s.extreme = f + 9 * C;
  s.vexp = reinterpret_cast<int*>(f + 9 * C + 1);
  return s;
}
template <bool GAIN>
__device__ __forceinline__ OutStage out_stage(unsigned char* lds, int buf) {
  unsigned char* p = lds + n_chain_stages(GAIN) * chain_stage_bytes(GAIN) +
                     (size_t)buf * out_stage_bytes(GAIN);
  OutStage s;
  s.q = reinterpret_cast<_Float16*>(p);
  s.p = reinterpret_cast<_Float16*>(p);
  s.g = reinterpret_cast<float*>(p + kStT);
  return s;
}
template <bool GAIN>
__device__ __forceinline__ half8* exch_at(unsigned char* lds, int buf) {
  return reinterpret_cast<half8*>(lds + n_chain_stages(GAIN) * chain_stage_bytes(GAIN) +
                                  2 * out_stage_bytes(GAIN) + (size_t)buf * kExBytes);
}

// ---- wavefronts 2-3 (pw = 0, 1). Each load instruction of a wavefront reads
// 1 KB of consecutive bytes. Chain fields belong to one chunk, output fields
// to the one before it.
template <bool GAIN> struct ProdX {
  uint4 gn[8];  // gains: rows 32 pw + 4 i + l / 16, piece l % 16 (chain chunk)
  uint4 p[3];   // P, three-block form: 1 KB pieces 3 pw + i (output chunk)
  float go;     // g of token l (output chunk)
};
template <> struct ProdX<false> {
  uint4 q[8];   // Q: rows 32 pw + 4 i + l / 16, piece l % 16 (output chunk)
};
template <bool GAIN>
struct ProdBuf : ProdX<GAIN> {
  uint4 k[8];    // K: rows 32 pw + 4 i + l / 16, 16-byte piece l % 16
  uint4 t[3];    // T, three-block form: 1 KB pieces 3 pw + i
  uint4 v[2];    // V slice: rows 32 pw + 16 i + l / 4, piece l % 4
  float4 sc0;    // scalars of token l (chain chunk): g, w, log2 g, write scale
  float4 sc1;    //   R, Cf, f0, f1
  float4 sc2;    //   value scale, extreme, g, 0
};

struct ProdCtx {
  __amdgpu_buffer_rsrc_t rk, rx, rv;
  const unsigned char* rec;   // records of this head
  int pw, lane;
};

// T / P piece j (0..5) of the three-block form: block j / 2, block rows
// 16 (j % 2) + l / 4, columns 8 (l % 4) .. + 8 -> matrix (row, col)
__device__ __forceinline__ void tri_piece(int j, int l, int& row, int& col) {
  const int blk = j >> 1, brow = 16 * (j & 1) + (l >> 2);
  row = (blk == 0 ? 0 : 32) + brow;
  col = (blk == 2 ? 32 : 0) + 8 * (l & 3);
}

template <bool GAIN>
__device__ __forceinline__ void prod_load(const ProdCtx& x, ProdBuf<GAIN>& b, int cc, int co, int dv) {
  const int l = x.lane, r0 = 32 * x.pw;
  const unsigned char* rc = x.rec + (size_t)cc * rec_bytes(GAIN);
  const unsigned char* ro = x.rec + (size_t)co * rec_bytes(GAIN);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int off_c = (cc * C + r0 + 4 * i) * (DK * 2) + l * 16;
    b.k[i] = bload16(x.rk, off_c);
    if constexpr (GAIN) b.gn[i] = bload16(x.rx, off_c);
    else b.q[i] = bload16(x.rx, (co * C + r0 + 4 * i) * (DK * 2) + l * 16);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    b.t[i] = reinterpret_cast<const uint4*>(rc + kRecT)[(3 * x.pw + i) * 64 + l];
    if constexpr (GAIN) b.p[i] = reinterpret_cast<const uint4*>(ro + rec_p_off(true))[(3 * x.pw + i) * 64 + l];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
    b.v[i] = bload16(x.rv, (cc * C + r0 + 16 * i + (l >> 2)) * dv * 2 + (l & 3) * 16);
  const float4* sc = reinterpret_cast<const float4*>(rc + rec_s_off(GAIN));
  b.sc0 = sc[3 * l];
  b.sc1 = sc[3 * l + 1];
  b.sc2 = sc[3 * l + 2];
  if constexpr (GAIN) b.go = reinterpret_cast<const float4*>(ro + rec_s_off(true))[3 * l].x;
}

// Maximum over the 64 lanes (every lane gets it; all lanes active).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true));  // ^1
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true));  // ^2
  x = max(x, (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (4 << 10)));
  x = max(x, (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (8 << 10)));
  x = max(x, (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (16 << 10)));
  const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(x, __lane_id() < 32 ? sw[1] : sw[0]);
}
// 2^e as a float, -126 <= e <= 127
__device__ __forceinline__ float pow2i(int e) { return __int_as_float((127 + e) << 23); }
// Largest of three, a NaN propagating (one v_maximum3_f32, abs folded into
// its operands; no quieting of the inputs as the number-preferring maximum needs)
__device__ __forceinline__ float max3_nan(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
// Exponent floor(log2 |v|) of the largest finite |v| among the bf16 values in
// `n` dwords of every lane, when it is at least 12; any smaller result (-127
// here) means that every finite |v| is below 2^12. A ballot on the lanes'
// packed maxima decides whether some |v| reaches 4096 or is not finite; only
// then are the non-finite ones masked and the maximum taken over the wave.
template <int N>
__device__ __forceinline__ int bf16_max_exponent(const uint32_t (&w)[N]) {
  typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
  ushort2v m = {0, 0};
#pragma unroll
  for (int i = 0; i < N; ++i)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2v, w[i] & 0x7fff7fffu));
  if (__ballot(max((uint32_t)m[0], (uint32_t)m[1]) >= 0x4580u) == 0) return -127;
  uint32_t f = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
    f = max(f, max(lo < 0x7f80u ? lo : 0u, hi < 0x7f80u ? hi : 0u));
  }
  return (int)(__builtin_amdgcn_readfirstlane(wave_max_u32(f)) >> 7) - 127;
}
// The staging exponent for values whose largest |v| has exponent E.
__device__ __forceinline__ int value_shift(int E) { return E >= 12 ? max(11 - E, -120) : 0; }

template <bool GAIN>
__device__ __forceinline__ void prod_stage(const ProdCtx& x, const ProdBuf<GAIN>& b,
                                           const ChainStage& cs, const OutStage& os) {
  const int l = x.lane, r0 = 32 * x.pw;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int off = (r0 + 4 * i + (l >> 4)) * KP + (l & 15) * 8;
    *reinterpret_cast<uint4*>(cs.k + off) = bf16x8_to_f16x8(b.k[i]);
    if constexpr (GAIN) *reinterpret_cast<uint4*>(cs.b + off) = b.gn[i];
    else *reinterpret_cast<uint4*>(os.q + off) = bf16x8_to_f16x8(b.q[i]);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    int row, col;
    tri_piece(3 * x.pw + i, l, row, col);
    *reinterpret_cast<uint4*>(cs.t + row * CP + col) = b.t[i];
    if constexpr (GAIN) *reinterpret_cast<uint4*>(os.p + row * CP + col) = b.p[i];
  }
  // V times 2^e_p, e_p from the largest finite |v| of this producer's rows
  {
    const uint32_t vw[8] = {b.v[0].x, b.v[0].y, b.v[0].z, b.v[0].w,
                            b.v[1].x, b.v[1].y, b.v[1].z, b.v[1].w};
    const int E = bf16_max_exponent(vw);
    uint4 vh[2];
    if (E >= 12) {
      const float vsc = pow2i(value_shift(E));
      vh[0] = bf16x8_to_f16x8(b.v[0], vsc);
      vh[1] = bf16x8_to_f16x8(b.v[1], vsc);
    } else {
      vh[0] = bf16x8_to_f16x8(b.v[0]);
      vh[1] = bf16x8_to_f16x8(b.v[1]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4*>(cs.v + (r0 + 16 * i + (l >> 2)) * VP + (l & 3) * 8) = vh[i];
    if (l == 0) cs.vexp[x.pw] = E;
  }
  if (x.pw == 0) {
    cs.g[l] = b.sc0.x;
    cs.w[l] = b.sc0.y;
    cs.lg[l] = b.sc0.z;
    cs.bs[l] = b.sc0.w;
    if (l == 0) cs.extreme[0] = b.sc2.y;
  } else {
    cs.rr[l] = b.sc1.x;
    cs.cf[l] = b.sc1.y;
    cs.f0[l] = b.sc1.z;
    cs.f1[l] = b.sc1.w;
    cs.go[l] = b.sc2.z;
    if constexpr (GAIN) os.g[l] = b.go;
  }
}

// ---- wavefront 1 (Kalman writes): Q rows of one chunk straight from global
// memory, in operand k order.
// Q rows of one chunk as the output wavefront's operands, loaded from global
// memory two steps ahead (Kalman writes: no LDS is left for a Q stage). Lane
// (h, m) loads the 16 bytes of columns 16 s + 8 h .. + 8 of token 32 tb + m;
// q_operand swaps 8-byte halves with lane ^ 32 into the operand k order
// (columns 16 s + 4 h .. + 4 and 16 s + 8 + 4 h .. + 4). Sixteen loads per
// chunk instead of 32 eight-byte ones keep two chunks of loads plus the
// stores between them under the 63 memory operations a wavefront can have in
// flight.
struct QBuf {
  uint4 q[2][8];  // [token block][k step]
};
__device__ __forceinline__ void q_load(__amdgpu_buffer_rsrc_t rq, QBuf& b, int c, int lane) {
  const int m = lane & 31, h = lane >> 5;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int off = (c * C + 32 * tb + m) * (DK * 2) + 16 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s) b.q[tb][s] = bload16(rq, off + 32 * s);
  }
}
__device__ __forceinline__ half8 q_operand(uint4 raw) {
  // lane h = 0 keeps columns 0-3 and receives 8-11 from lane + 32; lane h = 1
  // receives 4-7 from lane - 32 and keeps 12-15 (all relative to 16 s)
  const auto d0 = __builtin_amdgcn_permlane32_swap(raw.x, raw.z, false, false);
  const auto d1 = __builtin_amdgcn_permlane32_swap(raw.y, raw.w, false, false);
  return cat(bf16x4_to_f16x4(make_uint2(d0[0], d1[0])), bf16x4_to_f16x4(make_uint2(d0[1], d1[1])));
}

template <bool GAIN, bool OBF16, bool NARROW>
__global__ __launch_bounds__(NT_STATE) void state_kernel(StateArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  constexpr int NCH = n_chain_stages(GAIN);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c32 = lane & 31;

  int bh, tile;
  {
    // the d_v slices of one head land on one XCD (blocks are dealt to the 8
    // XCDs round-robin), so they share that XCD's L2
    const int id = blockIdx.x;
    if ((a.BH & 7) == 0) {
      const int xcd = id & 7, slot = id >> 3;
      bh = (slot / a.ntiles) * 8 + xcd;
      tile = slot % a.ntiles;
    } else {
      bh = id / a.ntiles;
      tile = id % a.ntiles;
    }
  }
  const int j0 = tile * (NARROW ? 16 : DV);
  const int last = a.nchunks - 1;
  const int nsteps = (a.nchunks + 2) & ~1;  // chunks + 1 (output lag), even
  if constexpr (NARROW) {
    // the exchange's columns 16-31 and its second exponent are never written
    // by the narrow chain: zero them once (the roles' first barrier orders it)
    uint4* ex0 = reinterpret_cast<uint4*>(exch_at<GAIN>(lds_raw, 0));
    for (int i = tid; i < (int)(2 * kExBytes / 16); i += NT_STATE) ex0[i] = make_uint4(0, 0, 0, 0);
  }
  const unsigned char* rec_head = a.rec + (size_t)bh * a.nchunks * rec_bytes(GAIN);
  const size_t head_tok = (size_t)bh * a.L;

  // transposed reads: group G = lane / 16 covers columns 16 (G % 2) .. + 16 and
  // rows 4 (G / 2) .. + 4 of an 8-row half step; lane jj of the group
  // addresses row jj / 4 and column quad jj % 4
  const int G = lane >> 4, jj = lane & 15;
  const int tr_row = 4 * (G >> 1) + (jj >> 2);
  const int tr_col = 16 * (G & 1) + 4 * (jj & 3);

  if (wv >= 2) {
    // ------------------------------------------------------------ producers
    ProdCtx x;
    x.rk = make_rsrc(a.k + head_tok * DK, (size_t)a.L * DK * 2);
    x.rx = GAIN ? make_rsrc(a.gain + head_tok * DK, (size_t)a.L * DK * 2)
                : make_rsrc(a.q + head_tok * DK, (size_t)a.L * DK * 2);
    x.rv = make_rsrc(a.v + head_tok * a.dv + j0, ((size_t)a.L * a.dv - j0) * 2);
    x.rec = rec_head;
    x.pw = wv - 2;
    x.lane = lane;
    // step c stages the chain inputs of chunk c + 1 and the output inputs of
    // chunk c from the register buffer that holds them, then reloads it with
    // chunks c + 3 and c + 2. Chunk indices are clamped to the last chunk;
    // restaging it into a buffer no one reads this step is harmless.
    ProdBuf<GAIN> r0, r1;
    prod_load<GAIN>(x, r0, 0, 0, a.dv);
    prod_load<GAIN>(x, r1, min(1, last), 0, a.dv);
    prod_stage<GAIN>(x, r0, chain_stage<GAIN>(lds_raw, 0), out_stage<GAIN>(lds_raw, 1));
    prod_load<GAIN>(x, r0, min(2, last), min(1, last), a.dv);
    __syncthreads();
    int cs_next = 1 % NCH;  // chain stage of chunk c + 1
    auto body = [&](int c, ProdBuf<GAIN>& r) {
      __builtin_amdgcn_sched_barrier(0);
      prod_stage<GAIN>(x, r, chain_stage<GAIN>(lds_raw, cs_next), out_stage<GAIN>(lds_raw, c & 1));
      prod_load<GAIN>(x, r, min(c + 3, last), min(c + 2, last), a.dv);
      cs_next = cs_next + 1 == NCH ? 0 : cs_next + 1;
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int c = 0; c < nsteps; c += 2) {
      body(c, r1);
      body(c + 1, r0);
    }
    return;
  }

  if (wv == 1) {
    // ------------------------------------------------------------ outputs
    constexpr int esz = OBF16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(static_cast<unsigned char*>(a.o) + (head_tok * a.dv + j0) * esz,
                  ((size_t)a.L * a.dv - j0) * esz);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + head_tok * DK, (size_t)a.L * DK * 2);
    // residuals for the write scores: this (head, slice)'s chunks, or range 0
    const __amdgpu_buffer_rsrc_t ru =
        make_rsrc(a.ubuf + (a.ubuf ? (size_t)(bh * a.ntiles + tile) * a.nchunks * 256 : 0),
                  a.ubuf ? (size_t)a.nchunks * 256 * 16 : 0);
    // the chunk's state exponent e_S beside the residuals (scaled by 2^e_S)
    const __amdgpu_buffer_rsrc_t rue =
        make_rsrc(a.uexp + (a.uexp ? (size_t)(bh * a.ntiles + tile) * a.nchunks : 0),
                  a.uexp ? (size_t)a.nchunks * 4 : 0);
    QBuf b0, b1;
    // Kalman writes: every step runs the same memory operations (Q loads of
    // chunk c + 1, 8 output stores (4 for bf16 outputs), 4 residual stores).
    // On the steps without a chunk (the first, and the last when the chunk
    // count is even) the outputs are formed from stale LDS data and their
    // stores fall outside the buffers (dropped). With no branch around them,
    // and the operations before the loop issued in the loop's order (Q of
    // chunk 0, then dropped stores), the compiler's wait for a chunk's Q does
    // not take in the loads issued one step later: measured, the state kernel
    // of the diagonal Kalman write 191 -> 167 us. The delta write loads
    // nothing here and skips the steps without a chunk.
    if constexpr (GAIN) {
      q_load(rq, b0, 0, lane);
      const __amdgpu_buffer_rsrc_t none = make_rsrc(a.o, 0);
      const v4u32 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < (OBF16 ? 4 : 8) + 4; ++i) __builtin_amdgcn_raw_buffer_store_b128(z, none, 0, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(0u, none, 0, 0, 0);
    }
    __syncthreads();
    int cs_prev = NCH - 1;  // chain stage of chunk c - 1
    // step c (1 <= c <= nchunks) writes the outputs of chunk c - 1
    auto body = [&](int c, QBuf& b) {
      __builtin_amdgcn_sched_barrier(0);
      const int cc = c - 1;
      if (GAIN || (cc >= 0 && cc <= last)) {
        const half8* ex = exch_at<GAIN>(lds_raw, cc & 1);
        const OutStage os = out_stage<GAIN>(lds_raw, cc & 1);
        const ChainStage cs = chain_stage<GAIN>(lds_raw, cs_prev);
        // Q operands: product i = token block i / 8, k step i % 8
        auto q_op = [&](int i) -> half8 {
          const int tb = i >> 3, s = i & 7;
          if constexpr (GAIN)
            return q_operand(b.q[tb][s]);
          else
            return ld_op(os.q + (32 * tb + c32) * KP + 16 * s, h);
        };
        half8 sv[8], uv[4], qa[16], pa[6];
        floatx16 o[2] = {floatx16{}, floatx16{}};
#pragma unroll
        for (int i = 0; i < 4; ++i) qa[i] = q_op(i);
#pragma unroll
        for (int s = 0; s < 8; ++s) sv[s] = ex[s * 64 + lane];
        if constexpr (!GAIN) {
          // P^T = K Q^T on blocks (token block of K, of Q) = (0,0), (0,1), (1,1),
          // k step outer so that every Q operand is read once, in order
          floatx16 pt[3] = {floatx16{}, floatx16{}, floatx16{}};
          half8 kb[2][8];
          float4 fac[3][4];   // row factors: R (diagonal blocks 0, 2), f0 (block 1)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            kb[0][s] = ld_op(cs.k + c32 * KP + 16 * s, h);
            kb[1][s] = ld_op(cs.k + (32 + c32) * KP + 16 * s, h);
          }
#pragma unroll
          for (int i = 8; i < 12; ++i) qa[i] = q_op(i);
          __builtin_amdgcn_sched_barrier(0);
          static_for<24>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int s = i / 3, blk = i % 3;          // 0: (0,0) 1: (0,1) 2: (1,1)
            constexpr int lb = blk == 2 ? 1 : 0, qb = blk == 0 ? 0 : 1;
            pt[blk] = mfma32(kb[lb][s], qa[8 * qb + s], pt[blk]);
            if constexpr (blk == 2 && s + 2 < 8) {
              kb[0][s + 2] = ld_op(cs.k + c32 * KP + 16 * (s + 2), h);
              kb[1][s + 2] = ld_op(cs.k + (32 + c32) * KP + 16 * (s + 2), h);
            }
            // Q operands: token block 0 k step s + 2 and block 1 k step s + 2
            if constexpr (blk == 0 && s + 4 < 8) qa[s + 4] = q_op(s + 4);
            if constexpr (blk == 1 && s + 4 < 8) qa[8 + s + 4] = q_op(8 + s + 4);
            if constexpr (i >= 12) {
              constexpr int q = i - 12, fb = q / 4, fj = q % 4;
              const float* src = fb == 1 ? cs.f0 : cs.rr;
              fac[fb][fj] = *reinterpret_cast<const float4*>(src + 32 * (fb == 2 ? 1 : 0) + 8 * fj + 4 * h);
            }
            __builtin_amdgcn_sched_barrier(0);
          });
          // P_il = (q_i . k_l) bs_l g_i / g_l for l <= i. Lane (h, c32) holds
          // column i = 32 qb + c32 and rows l = 32 lb + 8 j + 4 h + r. The
          // off-diagonal block multiplies f0_l f1_i; the diagonal blocks
          // R_l Cf_i, or exp2 of log2 g differences in an extreme chunk.
          const bool extreme =
              __builtin_amdgcn_readfirstlane(__float_as_int(cs.extreme[0])) != 0;
          const float f1i = cs.f1[32 + c32];
          const float cfi[2] = {cs.cf[c32], cs.cf[32 + c32]};
          const float lgi[2] = {cs.lg[c32], cs.lg[32 + c32]};
          auto scale_quad = [&](int blk, int j, auto exact_c) {
            constexpr bool exact = decltype(exact_c)::value;
            const int lb = blk == 2 ? 1 : 0;
            const int l0 = 32 * lb + 8 * j + 4 * h;
            if (blk == 1) {
              const float4 f0l = fac[1][j];
              pt[1][4 * j + 0] *= f0l.x * f1i;
              pt[1][4 * j + 1] *= f0l.y * f1i;
              pt[1][4 * j + 2] *= f0l.z * f1i;
              pt[1][4 * j + 3] *= f0l.w * f1i;
            } else {
              const int di = c32 - (8 * j + 4 * h);   // i - l for r = 0
              if constexpr (!exact) {
                const float4 rl = fac[blk][j];
                const float rv[4] = {rl.x, rl.y, rl.z, rl.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  pt[blk][4 * j + r] = di >= r ? pt[blk][4 * j + r] * (rv[r] * cfi[lb]) : 0.f;
              } else {
                const float4 lgl = *reinterpret_cast<const float4*>(cs.lg + l0);
                const float4 bsl = *reinterpret_cast<const float4*>(cs.bs + l0);
                const float lgv[4] = {lgl.x, lgl.y, lgl.z, lgl.w};
                const float bsv[4] = {bsl.x, bsl.y, bsl.z, bsl.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const float e = __builtin_amdgcn_exp2f(lgi[lb] - lgv[r]) * bsv[r];
                  pt[blk][4 * j + r] = di >= r ? pt[blk][4 * j + r] * e : 0.f;
                }
              }
            }
          };
          // Q S (16 products) with the scaling of P^T under it
          auto qs_scaled = [&](auto exact_c) {
            static_for<16>([&](auto ic) {
              constexpr int i = decltype(ic)::value;
              o[i & 1] = mfma32(sv[i >> 1], qa[8 * (i & 1) + (i >> 1)], o[i & 1]);
              if constexpr (i < 12) scale_quad(i / 4, i % 4, exact_c);
              if constexpr (i == 12) {
#pragma unroll
                for (int s = 0; s < 4; ++s) uv[s] = ex[(8 + s) * 64 + lane];
              }
              __builtin_amdgcn_sched_barrier(0);
            });
          };
          if (!extreme) qs_scaled(std::false_type{});
          else qs_scaled(std::true_type{});
          // operands of P U: output token block ib, k step s over l
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pa[0][e] = (_Float16)pt[0][e];
            pa[1][e] = (_Float16)pt[0][8 + e];
            pa[2][e] = (_Float16)pt[1][e];
            pa[3][e] = (_Float16)pt[1][8 + e];
            pa[4][e] = (_Float16)pt[2][e];
            pa[5][e] = (_Float16)pt[2][8 + e];
          }
        } else {
#pragma unroll
          for (int i = 4; i < 16; ++i) qa[i] = q_op(i);
          __builtin_amdgcn_sched_barrier(0);
          static_for<16>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            o[i & 1] = mfma32(sv[i >> 1], qa[8 * (i & 1) + (i >> 1)], o[i & 1]);
            __builtin_amdgcn_sched_barrier(0);
          });
#pragma unroll
          for (int s = 0; s < 4; ++s) uv[s] = ex[(8 + s) * 64 + lane];
          pa[0] = ld_op(os.p + c32 * CP, h);
          pa[1] = ld_op(os.p + c32 * CP + 16, h);
#pragma unroll
          for (int s = 0; s < 4; ++s) pa[2 + s] = ld_op(os.p + (32 + c32) * CP + 16 * s, h);
        }
        // The products run transposed, O^T = S^T Q^T + U^T P^T (the operand
        // registers are the same, A and B swap), so that each lane ends with 4
        // consecutive value columns of one token: 16-byte stores. Columns of
        // O^T are tokens: O^T = (S^T Q^T) diag(g) + U^T P^T.
        const float* gsrc = GAIN ? os.g : cs.go;
        // S and U came times 2^eo
        const int eo = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(ex + 12 * 64)[0]);
        const float gt[2] = {gsrc[c32], gsrc[32 + c32]};
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[tb][e] *= gt[tb];
        o[0] = mfma32(uv[0], pa[0], o[0]);
        o[1] = mfma32(uv[0], pa[2], o[1]);
        o[0] = mfma32(uv[1], pa[1], o[0]);
        o[1] = mfma32(uv[1], pa[3], o[1]);
        o[1] = mfma32(uv[2], pa[4], o[1]);
        o[1] = mfma32(uv[3], pa[5], o[1]);
        __builtin_amdgcn_sched_barrier(0);
        // U came times 2^eo, and so did o
        if (eo != 0) {
          const float f = pow2i(-eo);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[tb][e] *= f;
        }
        if (GAIN || a.uexp)
          __builtin_amdgcn_raw_buffer_store_b32((uint32_t)eo, rue, lane == 0 ? cc * 4 : 1 << 30, 0, 0);
        // residuals U of this chunk and d_v slice, in wavefront-0 register
        // order (Kalman writes: issued, and dropped, without them too)
        if (GAIN || a.ubuf) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, uv[s]), ru,
                                                   (cc * 256 + s * 64 + lane) * 16, 0, 0);
        }
        if constexpr (GAIN) q_load(rq, b, min(cc + 2, last), lane);
        // o[tb] registers 4 q .. 4 q + 3: token 32 tb + c32, columns 8 q + 4 h .. + 4
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int tok = cc * C + 32 * tb + c32;
          if constexpr (OBF16) {
            // Lanes l and l ^ 32 hold the two 8-byte halves of each 16-byte
            // piece of bf16 columns. One lane swap per dword gives lane h the
            // whole pieces of column groups pr + 2 h (pr = 0, 1): streaming
            // stores stay 16 bytes (8-byte ones reach HBM as partial writes).
            uint2 pk[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              pk[q4] = make_uint2(pk_bf16(o[tb][4 * q4], o[tb][4 * q4 + 1]),
                                  pk_bf16(o[tb][4 * q4 + 2], o[tb][4 * q4 + 3]));
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
              // lane h = 0 keeps its group pr and receives lane + 32's half of it;
              // lane h = 1 receives lane - 32's half of group pr + 2 and keeps its own
              const auto lo = __builtin_amdgcn_permlane32_swap(pk[pr].x, pk[pr + 2].x, false, false);
              const auto hi = __builtin_amdgcn_permlane32_swap(pk[pr].y, pk[pr + 2].y, false, false);
              const uint4 w4 = make_uint4(lo[0], hi[0], lo[1], hi[1]);
              const int off = (tok * a.dv + 8 * (pr + 2 * h)) * esz;
              // (a narrow slice holds columns 0-15 only: lanes h = 1 store nothing)
              if (!NARROW || h == 0)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, w4), ro, off, 0, out_store_policy<GAIN, NARROW>());
            }
          } else {
#pragma unroll
            for (int q4 = 0; q4 < (NARROW ? 2 : 4); ++q4) {
              const int off = (tok * a.dv + 8 * q4 + 4 * h) * esz;
              const uint4 w4 = make_uint4(__float_as_uint(o[tb][4 * q4]), __float_as_uint(o[tb][4 * q4 + 1]),
                                          __float_as_uint(o[tb][4 * q4 + 2]), __float_as_uint(o[tb][4 * q4 + 3]));
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, w4), ro, off, 0,
                                                     out_store_policy<GAIN, NARROW>());
            }
          }
        }
      }
      cs_prev = cs_prev + 1 == NCH ? 0 : cs_prev + 1;
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int c = 0; c < nsteps; c += 2) {
      body(c, b1);
      body(c + 1, b0);
    }
    return;
  }

  if constexpr (!NARROW) {
  // -------------------------------------------------------------- chain
  floatx16 S[4];  // S[b] register j: d_k row 32 b + 8 (j / 4) + 4 h + j % 4, column c32
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int d = 32 * b + 8 * (j >> 2) + 4 * h + (j & 3);
      S[b][j] = a.state_in ? a.state_in[((size_t)bh * DK + d) * a.dv + j0 + c32] : 0.f;
    }
  // The state is carried as S * 2^eS (see "Range" at the top). The state
  // entering each chunk is checked while the chunk runs (largest |S 2^eS|, a
  // NaN propagating: its column is NaN from then on); at the next chunk start
  // a check that reached 2^11, or one below 2^5 with eS < 0, has the exponent
  // recomputed from the state at hand.
  auto absmax16 = [](const floatx16& x) {
    float m = max3_nan(fabsf(x[0]), fabsf(x[1]), fabsf(x[2]));
#pragma unroll
    for (int j = 3; j < 15; j += 2) m = max3_nan(m, fabsf(x[j]), fabsf(x[j + 1]));
    return __builtin_elementwise_maximum(m, fabsf(x[15]));
  };
  int eS = 0;
  // eS that brings the largest finite |S| into [2^9, 2^10), or 0 if it is below 2^11
  auto rescale_state = [&]() {
    float f = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) f = fabsf(S[b][j]) < INFINITY ? fmaxf(f, fabsf(S[b][j])) : f;
    const uint32_t mb = __builtin_amdgcn_readfirstlane(wave_max_u32(__float_as_uint(f)));
    const int Et = (int)(mb >> 23) - 127 - eS;  // exponent of the largest true |S|
    const int e = Et >= 11 ? max(9 - Et, -120) : 0;
    if (e != eS) {
      const float sc = pow2i(e - eS);
#pragma unroll
      for (int b = 0; b < 4; ++b) S[b] = S[b] * sc;
      eS = e;
    }
  };
  bool s_chk = false;  // the last check asks for a recomputed exponent
  {
    float smax = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) smax = fmaxf(smax, absmax16(S[b]));
    s_chk = __ballot(smax >= 2048.f) != 0;
  }
  __syncthreads();

  // One step is 38 products issued back to back, one per "slot"; the
  // conversions between them and all LDS reads are placed in the slots of
  // earlier products so that they run under the matrix core instead of
  // between its products:
  //   slots  0- 7  K S, token block 0        S -> fp16 (blocks 1-3), V, g reads
  //   slots  8-15  K S, token block 1        S *= g_n, X of block 0, w, T reads
  //   slots 16-17  U0  = T00 X0              B^T reads (transposed)
  //   slots 18-19  U1  = T10 X0              X of block 1
  //   slots 20-21  U1 += T11 X1              U0 -> fp16, w U0 -> fp16
  //   slots 22-29  S  += B^T w U, tokens 0-31    U1 -> fp16, w U1 -> fp16
  //   slots 30-37  S  += B^T w U, tokens 32-63
  int cs_cur = 0;  // chain stage of chunk c
  for (int c = 0; c < nsteps; ++c) {
    __builtin_amdgcn_sched_barrier(0);
    if (c <= last) {
      const ChainStage st = chain_stage<GAIN>(lds_raw, cs_cur);
      half8* ex = exch_at<GAIN>(lds_raw, c & 1);
      const int n = min(C, a.L - c * C);
      half8 s16[8], ka[16], x16[4], u16[4], uw16[4], ta[6];
      half4 vv[2][4], btr[32];
      float4 gg[2][4], ww[2][4];
      floatx16 ks[2] = {floatx16{}, floatx16{}}, u[2] = {floatx16{}, floatx16{}};
      // product i of K S: token block i / 8, k step i % 8
      auto k_op = [&](int i) -> half8 {
        return ld_op(st.k + (32 * (i >> 3) + c32) * KP + 16 * (i & 7), h);
      };
      auto s_to_f16 = [&](int b) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s16[2 * b][e] = (_Float16)S[b][e];
          s16[2 * b + 1][e] = (_Float16)S[b][8 + e];
        }
        ex[(2 * b) * 64 + lane] = s16[2 * b];
        ex[(2 * b + 1) * 64 + lane] = s16[2 * b + 1];
      };
      // X = V - g K S for token block blk, column quads g4 (k = token operand)
      auto x_quad = [&](int blk, int g4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = r == 0 ? gg[blk][g4].x : r == 1 ? gg[blk][g4].y : r == 2 ? gg[blk][g4].z : gg[blk][g4].w;
          x16[2 * blk + (g4 >> 1)][4 * (g4 & 1) + r] =
              (_Float16)((float)vv[blk][g4][r] - gv * ks[blk][4 * g4 + r]);
        }
      };
      // U (outputs) and w U (state update) in fp16 for token block blk, quad g4
      auto u_quad = [&](int blk, int g4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float wv = r == 0 ? ww[blk][g4].x : r == 1 ? ww[blk][g4].y : r == 2 ? ww[blk][g4].z : ww[blk][g4].w;
          const float uv = u[blk][4 * g4 + r];
          u16[2 * blk + (g4 >> 1)][4 * (g4 & 1) + r] = (_Float16)uv;
          uw16[2 * blk + (g4 >> 1)][4 * (g4 & 1) + r] = (_Float16)(uv * wv);
        }
      };
      // transposed write vectors, in the order the state update uses them:
      // q = 0..31 -> (k step s, d_k block b) = tokens 0-31 first, b outer
      auto bt_read = [&](int q) {
        const int part = q >> 4, b = (q >> 2) & 3, s = 2 * part + ((q >> 1) & 1), hi = q & 1;
        btr[q] = ld_tr(st.b + (16 * s + 8 * hi + tr_row) * KP + 32 * b + tr_col);
      };
      const int tr_[6] = {0, 0, 32, 32, 32, 32}, tk_[6] = {0, 16, 0, 16, 32, 48};
      float smax = 0.f;  // largest |S 2^eS| entering this chunk

      // the chunk's exponent: the state's, recomputed if the last check asked,
      // and no higher than the staging exponents of the chunk's values, so
      // that |V 2^eS| < 2^12; rows staged at a higher exponent are scaled down
      const int vE0 = st.vexp[0], vE1 = st.vexp[1];
      if (s_chk) rescale_state();
#pragma unroll
      for (int i = 0; i < 4; ++i) ka[i] = k_op(i);
      s_to_f16(0);
      {
        const int p0 = value_shift(__builtin_amdgcn_readfirstlane(vE0));
        const int p1 = value_shift(__builtin_amdgcn_readfirstlane(vE1));
        const int e = min(eS, min(p0, p1));
        if (e != eS || p0 != e || p1 != e) {
          if (e != eS) {
            const float sc = pow2i(e - eS);
#pragma unroll
            for (int b = 0; b < 4; ++b) S[b] = S[b] * sc;
            eS = e;
            s_to_f16(0);
          }
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            const int p = blk ? p1 : p0;
            if (p != e) {
              const float sc = pow2i(e - p);
#pragma unroll
              for (int i = 0; i < 2; ++i) {
                half8* vp = reinterpret_cast<half8*>(st.v + (32 * blk + 16 * i + (lane >> 2)) * VP + (lane & 3) * 8);
                half8 v = *vp;
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = (_Float16)((float)v[j] * sc);
                *vp = v;
              }
            }
          }
        }
        if (lane == 0) reinterpret_cast<int*>(ex + 12 * 64)[0] = eS;
      }
      const float gn = st.go[n - 1];   // the state carries the inclusive decay g_n
      __builtin_amdgcn_sched_barrier(0);
      static_for<38>([&](auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        // ---- the product
        if constexpr (slot < 16) {
          ks[slot >> 3] = mfma32(ka[slot], s16[slot & 7], ks[slot >> 3]);
        } else if constexpr (slot < 22) {
          const int j = slot - 16;  // 0,1: U0 <- T00 ; 2,3: U1 <- T10 ; 4,5: U1 <- T11
          const int acc = j < 2 ? 0 : 1, xs = j < 4 ? (j & 1) : 2 + (j & 1);
          u[acc] = mfma32(ta[j], x16[xs], u[acc]);
        } else {
          const int q = slot - 22, part = q >> 3, b = (q >> 1) & 3, s = 2 * part + (q & 1);
          const int bi = 16 * part + 4 * b + 2 * (q & 1);
          S[b] = mfma32(cat(btr[bi], btr[bi + 1]), uw16[s], S[b]);
        }
        // ---- work placed under it
        if constexpr (slot < 12) ka[slot + 4] = k_op(slot + 4);
        if constexpr (slot == 0) s_to_f16(1);
        if constexpr (slot == 2) s_to_f16(2);
        if constexpr (slot == 4) s_to_f16(3);
        if constexpr (slot >= 1 && slot <= 8) {
          const int q = slot - 1, blk = q >> 2, g4 = q & 3;
          vv[blk][g4] = ld_tr(st.v + (32 * blk + 8 * g4 + tr_row) * VP + tr_col);
          gg[blk][g4] = *reinterpret_cast<const float4*>(st.g + 32 * blk + 8 * g4 + 4 * h);
        }
        // the state entering the chunk: checked block by block once converted
        if constexpr (slot == 1) smax = absmax16(S[0]);
        if constexpr (slot == 3 || slot == 5) smax = __builtin_elementwise_maximum(smax, absmax16(S[(slot - 1) / 2]));
        if constexpr (slot == 7) {
          smax = __builtin_elementwise_maximum(smax, absmax16(S[3]));
          const bool hi = __ballot(smax >= 2048.f) != 0, lo = __ballot(smax >= 32.f) == 0;
          s_chk = hi | (lo & (eS < 0));
        }
        if constexpr (slot >= 8 && slot <= 11) S[slot - 8] = S[slot - 8] * gn;
        if constexpr (slot >= 9 && slot <= 12) {
          const int q = slot - 9;
          ww[q >> 1][2 * (q & 1)] = *reinterpret_cast<const float4*>(st.w + 32 * (q >> 1) + 16 * (q & 1) + 4 * h);
          ww[q >> 1][2 * (q & 1) + 1] = *reinterpret_cast<const float4*>(st.w + 32 * (q >> 1) + 16 * (q & 1) + 8 + 4 * h);
        }
        if constexpr (slot >= 12 && slot <= 14) {
          const int j = 2 * (slot - 12);
          ta[j] = ld_op(st.t + (tr_[j] + c32) * CP + tk_[j], h);
          ta[j + 1] = ld_op(st.t + (tr_[j + 1] + c32) * CP + tk_[j + 1], h);
        }
        if constexpr (slot >= 10 && slot <= 13) x_quad(0, slot - 10);
        if constexpr (slot >= 15 && slot <= 22) {
          const int q0 = 4 * (slot - 15);
          bt_read(q0); bt_read(q0 + 1); bt_read(q0 + 2); bt_read(q0 + 3);
        }
        if constexpr (slot == 17 || slot == 18) {
          x_quad(1, 2 * (slot - 17));
          x_quad(1, 2 * (slot - 17) + 1);
        }
        if constexpr (slot == 20) { u_quad(0, 0); u_quad(0, 1); }
        if constexpr (slot == 21) {
          u_quad(0, 2); u_quad(0, 3);
          ex[8 * 64 + lane] = u16[0];
          ex[9 * 64 + lane] = u16[1];
        }
        if constexpr (slot >= 24 && slot <= 27) u_quad(1, slot - 24);
        if constexpr (slot == 28) {
          ex[10 * 64 + lane] = u16[2];
          ex[11 * 64 + lane] = u16[3];
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    cs_cur = cs_cur + 1 == NCH ? 0 : cs_cur + 1;
    __syncthreads();
  }

  if (a.state_out) {
    const float f = pow2i(-eS);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int d = 32 * b + 8 * (j >> 2) + 4 * h + (j & 3);
        a.state_out[((size_t)bh * DK + d) * a.dv + j0 + c32] = S[b][j] * f;
      }
  }
  } else {
  // ------------------------------------------------- chain, 16 columns
  // The narrow slice (16 columns j0 .. j0 + 16) on 16 x 16 x 32 products. A lane holds column n16 and rows
  // 4 q4 .. + 4 of every 16-row result tile; an operand gives it row (or
  // column) n16 and k positions 8 q4 .. + 8. Over a 32-wide k block, k
  // position 8 q + j stands for row 4 q + j (j < 4) or 16 + 4 q + j - 4
  // (j >= 4) of the block, so that the two result tiles of a block, side by
  // side, are the operand as they are; the other operand reads its rows in
  // the same order (two 8-byte reads, or two transposed reads).
  constexpr int ci = 0;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int col = j0 + 16 * ci + n16;
  floatx4 S[8];  // S[i][r]: d_k row 16 i + 4 q4 + r, column col
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[i][r] = a.state_in ? a.state_in[((size_t)bh * DK + 16 * i + 4 * q4 + r) * a.dv + col] : 0.f;
  auto cvt4 = [](const floatx4& x) -> half4 {
    return __builtin_bit_cast(half4, make_uint2(pk_f16(x[0], x[1]), pk_f16(x[2], x[3])));
  };
  // The state is carried as S * 2^eS (see "Range" at the top). The state
  // entering each chunk is checked while the chunk runs (largest |S 2^eS|, a
  // NaN propagating: its column is NaN from then on); at the next chunk start
  // a check that reached 2^11, or one below 2^5 with eS < 0, has the exponent
  // recomputed from the state at hand.
  auto absmax8 = [&](float m, int i) {   // m and the 8 entries of tiles i, i + 1
    m = max3_nan(m, fabsf(S[i][0]), fabsf(S[i][1]));
    m = max3_nan(m, fabsf(S[i][2]), fabsf(S[i][3]));
    m = max3_nan(m, fabsf(S[i + 1][0]), fabsf(S[i + 1][1]));
    return max3_nan(m, fabsf(S[i + 1][2]), fabsf(S[i + 1][3]));
  };
  int eS = 0;
  // eS that brings the largest finite |S| into [2^9, 2^10), or 0 if it is below 2^11
  auto rescale_state = [&]() {
    float f = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) f = fabsf(S[i][r]) < INFINITY ? fmaxf(f, fabsf(S[i][r])) : f;
    const uint32_t mb = __builtin_amdgcn_readfirstlane(wave_max_u32(__float_as_uint(f)));
    const int Et = (int)(mb >> 23) - 127 - eS;  // exponent of the largest true |S|
    const int e = Et >= 11 ? max(9 - Et, -120) : 0;
    if (e != eS) {
      const float sc = pow2i(e - eS);
#pragma unroll
      for (int i = 0; i < 8; ++i) S[i] = S[i] * sc;
      eS = e;
    }
  };
  bool s_chk;  // the last check asks for a recomputed exponent
  {
    float smax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) smax = absmax8(smax, i);
    s_chk = __ballot(smax >= 2048.f) != 0;
  }
  __syncthreads();

  // One step is 38 products issued back to back, one per "slot"; the
  // conversions between them and the LDS reads are placed under earlier
  // products:
  //   slots  0-15  K S, token tile slot / 4, k block slot % 4
  //   slots 16-21  U = T X (tiles 0, 1 from X block 0; 2, 3 from blocks 0, 1)
  //   slots 22-37  S += B^T w U, state tile (slot - 22) % 8, token block (slot - 22) / 8
  constexpr int KA = 6;   // K operands read this many products ahead
  constexpr int BA = 6;   // transposed write vectors likewise
  int cs_cur = 0;  // chain stage of chunk c
  for (int c = 0; c < nsteps; ++c) {
    __builtin_amdgcn_sched_barrier(0);
    if (c <= last) {
      const ChainStage st = chain_stage<GAIN>(lds_raw, cs_cur);
      half8* ex = exch_at<GAIN>(lds_raw, c & 1);
      const int n = min(C, a.L - c * C);
      half8 s16[4], ka[16], x16[2], uw16[2], ta[6], bt[16];
      half4 vv[4], xt[4], uwt[4];
      float4 gg[4], ww[4];
      floatx4 ks[4] = {floatx4{}, floatx4{}, floatx4{}, floatx4{}};
      floatx4 u[4] = {floatx4{}, floatx4{}, floatx4{}, floatx4{}};
      // product i of K S: token tile i / 4, k block i % 4
      auto k_op = [&](int i) -> half8 {
        const _Float16* p = st.k + (16 * (i >> 2) + n16) * KP + 32 * (i & 3) + 4 * q4;
        return cat(ld4(p), ld4(p + 16));
      };
      // The output wavefront reads S and U as 32 x 32 operands: k step s,
      // lane c32 + 32 h, elements 4 p + r for row 16 s + 8 p + 4 h + r. Tile s
      // of this wavefront goes there as 8-byte pieces.
      auto ex_put = [&](int s, half4 v) {
        reinterpret_cast<half4*>(ex + s * 64 + 16 * ci + n16 + 32 * (q4 & 1))[q4 >> 1] = v;
      };
      auto s_to_f16 = [&](int kb) {
        const half4 h0 = cvt4(S[2 * kb]), h1 = cvt4(S[2 * kb + 1]);
        s16[kb] = cat(h0, h1);
        ex_put(2 * kb, h0);
        ex_put(2 * kb + 1, h1);
      };
      // X = V - g K S of token tile t
      auto x_tile = [&](int t) {
        const float gv[4] = {gg[t].x, gg[t].y, gg[t].z, gg[t].w};
#pragma unroll
        for (int r = 0; r < 4; ++r) xt[t][r] = (_Float16)fmaf(-gv[r], ks[t][r], (float)vv[t][r]);
      };
      // U of token tile t: to the exchange, and w U as the update's operand
      auto u_tile = [&](int t) {
        ex_put(8 + t, cvt4(u[t]));
        const float wv[4] = {ww[t].x, ww[t].y, ww[t].z, ww[t].w};
#pragma unroll
        for (int r = 0; r < 4; ++r) uwt[t][r] = (_Float16)(u[t][r] * wv[r]);
      };
      // T operand of U tile t, token block kb
      auto t_op = [&](int t, int kb) -> half8 {
        const _Float16* p = st.t + (16 * t + n16) * CP + 32 * kb + 4 * q4;
        return cat(ld4(p), ld4(p + 16));
      };
      // transposed write vectors for product q of the update: state tile
      // q % 8, token block q / 8
      auto bt_read = [&](int q) {
        const int i = q & 7, kb = q >> 3;
        const _Float16* p = st.b + (32 * kb + 4 * q4 + (n16 >> 2)) * KP + 16 * i + 4 * (n16 & 3);
        bt[q] = cat(ld_tr(p), ld_tr(p + 16 * KP));
      };
      constexpr int tt_[6] = {0, 1, 2, 3, 2, 3}, tk_[6] = {0, 0, 0, 0, 1, 1};
      float smax = 0.f;  // largest |S 2^eS| entering this chunk

      // the chunk's exponent: the state's, recomputed if the last check asked,
      // and no higher than the staging exponents of the chunk's values, so
      // that |V 2^eS| < 2^12; this wavefront's columns of rows staged at a
      // higher exponent are scaled down in place
      const int vE0 = st.vexp[0], vE1 = st.vexp[1];
      if (s_chk) rescale_state();
#pragma unroll
      for (int i = 0; i < KA; ++i) ka[i] = k_op(i);
      s_to_f16(0);
      s_to_f16(1);
      {
        const int p0 = value_shift(__builtin_amdgcn_readfirstlane(vE0));
        const int p1 = value_shift(__builtin_amdgcn_readfirstlane(vE1));
        const int e = min(eS, min(p0, p1));
        if (e != eS || p0 != e || p1 != e) {
          if (e != eS) {
            const float sc = pow2i(e - eS);
#pragma unroll
            for (int i = 0; i < 8; ++i) S[i] = S[i] * sc;
            eS = e;
            s_to_f16(0);
            s_to_f16(1);
          }
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            const int p = blk ? p1 : p0;
            if (p != e) {
              const float sc = pow2i(e - p);
              half8* vp = reinterpret_cast<half8*>(st.v + (32 * blk + (lane >> 1)) * VP + 16 * ci + 8 * (lane & 1));
              half8 v = *vp;
#pragma unroll
              for (int j = 0; j < 8; ++j) v[j] = (_Float16)((float)v[j] * sc);
              *vp = v;
            }
          }
        }
        if (lane == 0) reinterpret_cast<int*>(ex + 12 * 64)[ci] = eS;
      }
      const float gn = st.go[n - 1];   // the state carries the inclusive decay g_n
      __builtin_amdgcn_sched_barrier(0);
      static_for<38>([&](auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        // ---- the product
        if constexpr (slot < 16) {
          ks[slot >> 2] = mfma(ka[slot], s16[slot & 3], ks[slot >> 2]);
        } else if constexpr (slot < 22) {
          constexpr int j = slot - 16;
          u[tt_[j]] = mfma(ta[j], x16[tk_[j]], u[tt_[j]]);
        } else {
          constexpr int q = slot - 22, i = q & 7, kb = q >> 3;
          S[i] = mfma(bt[q], uw16[kb], S[i]);
        }
        // ---- work placed under it
        if constexpr (slot + KA < 16) ka[slot + KA] = k_op(slot + KA);
        if constexpr (slot == 0) s_to_f16(2);
        if constexpr (slot == 1) s_to_f16(3);
        if constexpr (slot >= 1 && slot <= 4) {
          constexpr int t = slot - 1;
          vv[t] = ld_tr(st.v + (16 * t + 4 * q4 + (n16 >> 2)) * VP + 16 * ci + 4 * (n16 & 3));
          gg[t] = *reinterpret_cast<const float4*>(st.g + 16 * t + 4 * q4);
        }
        // the state entering the chunk, checked once converted
        if constexpr (slot >= 3 && slot <= 6) smax = absmax8(smax, 2 * (slot - 3));
        if constexpr (slot == 6) {
          const bool hi = __ballot(smax >= 2048.f) != 0, lo = __ballot(smax >= 32.f) == 0;
          s_chk = hi | (lo & (eS < 0));
        }
        if constexpr (slot >= 7 && slot <= 14) S[slot - 7] = S[slot - 7] * gn;
        if constexpr (slot == 5 || slot == 9 || slot == 13 || slot == 17) x_tile((slot - 5) / 4);
        if constexpr (slot == 9) x16[0] = cat(xt[0], xt[1]);
        if constexpr (slot == 17) x16[1] = cat(xt[2], xt[3]);
        if constexpr (slot >= 8 && slot <= 13) ta[slot - 8] = t_op(tt_[slot - 8], tk_[slot - 8]);
        if constexpr (slot >= 12 && slot <= 15) {
          constexpr int t = slot - 12;
          ww[t] = *reinterpret_cast<const float4*>(st.w + 16 * t + 4 * q4);
        }
        if constexpr (slot >= 22 - BA && slot - (22 - BA) < 16) bt_read(slot - (22 - BA));
        if constexpr (slot == 18) u_tile(0);
        if constexpr (slot == 19) { u_tile(1); uw16[0] = cat(uwt[0], uwt[1]); }
        if constexpr (slot == 23) u_tile(2);
        if constexpr (slot == 24) { u_tile(3); uw16[1] = cat(uwt[2], uwt[3]); }
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    cs_cur = cs_cur + 1 == NCH ? 0 : cs_cur + 1;
    __syncthreads();
  }

  if (a.state_out) {
    const float f = pow2i(-eS);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a.state_out[((size_t)bh * DK + 16 * i + 4 * q4 + r) * a.dv + col] = S[i][r] * f;
  }
  }
}

}  // namespace

bool scan_mfma_supported(int dk, int dv, int chunk) {
  return dk == DK && chunk == C && dv % DV == 0 && dv >= DV;
}

// residuals, then the int exponent e_S of every (head, slice, chunk)
static size_t ubuf_core_bytes(int BH, int L, int dv) {
  const size_t nchunks = ((size_t)L + C - 1) / C;
  return (size_t)BH * (dv / DV) * nchunks * 256 * sizeof(half8);
}
size_t scan_mfma_ubuf_bytes(int BH, int L, int dv) {
  const size_t nchunks = ((size_t)L + C - 1) / C;
  return ubuf_core_bytes(BH, L, dv) + (size_t)BH * (dv / DV) * nchunks * sizeof(int);
}
const int* scan_mfma_ubuf_exps(const void* ubuf, int BH, int L, int dv) {
  return reinterpret_cast<const int*>(static_cast<const char*>(ubuf) + ubuf_core_bytes(BH, L, dv));
}

size_t scan_mfma_workspace_bytes(int BH, int L, bool gain) {
  const size_t nchunks = ((size_t)L + C - 1) / C;
  return (size_t)BH * nchunks * rec_bytes(gain);
}

// Chunks per prepare workgroup: one, so that the most workgroups are in
// flight; two once there are more than 16384 chunks, where the loads of a
// workgroup's second chunk overlapping its first pay more (measured on MI355X
// over 1, 2, 4, 8: the gated workload's 4096 chunks 34 -> 31 us with one, the
// long workload's 32768 chunks 227 -> 219 us with two).
int prep_chunks_per_workgroup(int BH, int nchunks) {
  return (long long)BH * nchunks > 16384 ? 2 : 1;
}

hipError_t launch_tinv_mfma(const ScanArgs& s, void* tbuf, hipStream_t st) {
  const int nchunks = (s.L + C - 1) / C;
  const bool gain = s.gain != nullptr;
  PrepArgs pa;
  pa.q = static_cast<const uint16_t*>(s.q);
  pa.k = static_cast<const uint16_t*>(s.k);
  pa.gain = static_cast<const _Float16*>(s.gain);
  pa.alpha = s.alpha;
  pa.beta = s.beta;
  pa.rec = static_cast<unsigned char*>(tbuf);
  pa.L = s.L;
  pa.nchunks = nchunks;
  pa.plain = s.plain;
  pa.noerase = s.noerase;
  pa.cpw = prep_chunks_per_workgroup(s.BH, nchunks);
  const bool diagf = s.dmaps != nullptr;
  if (diagf) {
    pa.nsub = (s.L + C / 2 - 1) / (C / 2);
    pa.dmaps = s.dmaps;
    pa.r = s.r;
    pa.qvar = s.qvar;
    pa.gain_out = static_cast<_Float16*>(const_cast<void*>(s.gain));
    pa.cov_out = s.cov_out;
  }
  const size_t lds = prep_lds_bytes(gain, diagf);
  auto kern = diagf ? prep_kernel<true, true> : gain ? prep_kernel<true, false> : prep_kernel<false, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  KDN_LAUNCH_NAMED(diagf ? "prep_kernel<true> (diagonal gains)" : gain ? "prep_kernel<true>" : "prep_kernel<false>",
                   kern, dim3(s.BH, (nchunks + pa.cpw - 1) / pa.cpw), dim3(NT), lds, st, pa);
  return hipGetLastError();
}

template <bool GAIN, bool OBF16, bool NARROW>
hipError_t launch_state_typed(const StateArgs& sa, hipStream_t st) {
  const size_t lds = state_lds_bytes(GAIN);
  auto kern = state_kernel<GAIN, OBF16, NARROW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  KDN_LAUNCH_NAMED(GAIN ? (OBF16 ? "state_kernel<true, true>" : "state_kernel<true, false>")
                   : NARROW ? (OBF16 ? "state_kernel<false, true> (16 columns)"
                                     : "state_kernel<false, false> (16 columns)")
                            : (OBF16 ? "state_kernel<false, true>" : "state_kernel<false, false>"),
                   kern, dim3(sa.BH * sa.ntiles), dim3(NT_STATE), lds, st, sa);
  return hipGetLastError();
}

// Compute units of the current device (cached per device index).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t launch_state_mfma(const ScanArgs& s, bool out_bf16, const void* tbuf, hipStream_t st) {
  StateArgs sa;
  sa.q = static_cast<const uint16_t*>(s.q);
  sa.k = static_cast<const uint16_t*>(s.k);
  sa.v = static_cast<const uint16_t*>(s.v);
  sa.gain = static_cast<const _Float16*>(s.gain);
  sa.rec = static_cast<const unsigned char*>(tbuf);
  sa.state_in = s.state_in;
  sa.state_out = s.state_out;
  sa.o = s.o;
  sa.BH = s.BH;
  sa.L = s.L;
  sa.dv = s.dv;
  sa.nchunks = (s.L + C - 1) / C;
  sa.ubuf = static_cast<half8*>(s.ubuf);
  sa.uexp = s.ubuf ? const_cast<int*>(scan_mfma_ubuf_exps(s.ubuf, s.BH, s.L, s.dv)) : nullptr;
  if (s.gain) {
    sa.ntiles = s.dv / DV;
    return out_bf16 ? launch_state_typed<true, true, false>(sa, st)
                    : launch_state_typed<true, false, false>(sa, st);
  }
  // One workgroup fills a compute unit. When 32-column slices would leave
  // half of them idle, the delta write takes 16-column slices: twice the
  // workgroups, each with half the chain (its residuals are not kept for
  // the write scores, which take the 32-column slices).
  // KDN_STATE_COLS=16 or 32 in the environment forces either.
  bool narrow = s.ubuf == nullptr && (long long)s.BH * (s.dv / DV) * 2 <= device_cus();
  if (const char* f = std::getenv("KDN_STATE_COLS")) {
    if (std::strcmp(f, "16") == 0) narrow = s.ubuf == nullptr;
    else if (std::strcmp(f, "32") == 0) narrow = false;
  }
  sa.ntiles = s.dv / (narrow ? 16 : DV);
  if (narrow)
    return out_bf16 ? launch_state_typed<false, true, true>(sa, st)
                    : launch_state_typed<false, false, true>(sa, st);
  return out_bf16 ? launch_state_typed<false, true, false>(sa, st)
                  : launch_state_typed<false, false, false>(sa, st);
}

}  // namespace kdn
