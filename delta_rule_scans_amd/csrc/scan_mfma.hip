// scan_mfma.hip -- chunkwise scan on the gfx950 matrix cores (d_k = 128, chunk 64).
//
// Recurrence ("A Hippocampus for Linear Attention", sec. 3.3 eq. (5), sec. 3.5)
//   e_t = v_t - alpha_t S_{t-1}^T k_t,  S_t = alpha_t S_{t-1} + b_t e_t^T,  o_t = S_t^T q_t
// in chunk form (one chunk of n <= 64 tokens, incoming state S0, chunk-local
// decay g_i = prod_{l<=i} alpha_l, write vectors b_l = beta_l k_l or the gain):
//   A = strict_lower((K B^T) * G),  G_il = g_i / g_l,  T = (I + A)^-1
//   X = V - diag(g) K S0,  U = T X  (U are the residuals e_t)
//   O = diag(g) Q S0 + lower_incl((Q B^T) * G) U
//   S = g_n S0 + sum_l (g_n / g_l) b_l U_l^T
//
// Two kernels:
//  * tinv_kernel: one workgroup per (head, chunk), all chunks in parallel.
//    Gram K B^T on the matrix cores, then T = (I + A)^-1 by blocks of 16:
//    the four diagonal blocks are inverted in float32 registers (one wavefront
//    per block, four lanes per column, quad reductions through DPP), the six
//    off-diagonal blocks follow by block products on the matrix cores,
//    diagonal by diagonal: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj.
//    T (fp16, 64x64) goes to the workspace. T does not depend on the state.
//  * scan_kernel: one workgroup per (head, 32-column slice of d_v); the loop
//    over chunks is sequential. The float32 state slice (128 x 32) stays in
//    the matrix-core accumulators for the whole sequence; its fp16 copy in LDS
//    feeds the products K S and Q S.
//
// All matrix products are v_mfma_f32_16x16x32_f16: fp16 operands, fp32
// accumulation. bf16 inputs are converted to fp16 when staged in LDS (exact
// for bf16 values of magnitude in [2^-14, 65504]). fp16 rather than bf16
// operands because the intermediate operands (S, X, U, P, T) need the 3 extra
// significand bits: with bf16 operands the output error at the gated-delta
// workload is ~3.7e-2 RMS(o), with fp16 ~5e-3.
//
// Operand layouts: an MFMA reads A as [m][k] and B as [n][k] with k contiguous
// (16-byte LDS reads); its result gives each lane 4 consecutive rows of one
// column, which is written either as [n][m] (one 8-byte write) or [m][n]
// (four 2-byte writes). Every buffer below is laid out for its reader.
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
constexpr int VP = DV + 8;     // fp16 pitch of the value tile
constexpr int OP = DV + 4;     // fp32 pitch of the output staging tile

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

// 8 bf16 values (one 16-byte load) -> 8 fp16 values.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 u) {
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 lo = (_Float16)__uint_as_float(w[i] << 16);
    const _Float16 hi = (_Float16)__uint_as_float(w[i] & 0xffff0000u);
    r[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
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

// Per-token scalars of one chunk, computed by one wavefront (lane = token).
// lg: chunk-local log-decay prefix; bs: write scale (beta, beta/alpha, or 1);
// vs: value scale (alpha for the plain residual, else 1);
// w: state-update weight (g_n / g_t) * bs_t (0 past the tail).
struct TokenScalars {
  float lg, bs, vs, w, gam;
};
__device__ __forceinline__ TokenScalars token_scalars(const float* alpha, const float* beta,
                                                      bool gain, int plain, size_t tok, int lane,
                                                      int n) {
  TokenScalars s;
  float la = 0.f;
  s.bs = 0.f;
  s.vs = 1.f;
  if (lane < n) {
    const float al = alpha ? alpha[tok + lane] : 1.f;
    la = logf(al);
    s.bs = gain ? 1.f : beta[tok + lane];
    if (plain) {
      s.bs /= al;
      s.vs = al;
    }
  }
  s.lg = wave_prefix(la, lane);
  const float lgn = __shfl(s.lg, n - 1, 64);
  s.gam = expf(s.lg);
  s.w = lane < n ? expf(lgn - s.lg) * s.bs : 0.f;
  return s;
}

// =====================================================================  T = (I + A)^-1

struct TinvArgs {
  const uint16_t* k;      // bf16 [BH, L, DK]
  const _Float16* gain;   // fp16 [BH, L, DK] or null (delta write)
  const float* alpha;     // [BH, L] or null
  const float* beta;      // [BH, L]
  _Float16* tout;         // [BH, nchunks, C, C]
  int L, nchunks, plain;
};

constexpr int kTinvR1 = (C * KP > 2 * C * CP ? C * KP : 2 * C * CP) * 2;  // bytes
constexpr int kAdP = 17;                                                  // fp32 pitch

size_t tinv_lds_bytes(bool gain) {
  return (size_t)kTinvR1 + (gain ? (size_t)C * KP * 2 : 0) + (size_t)C * CP * 2 +
         (size_t)4 * 16 * kAdP * 4 + (size_t)4 * 16 * 24 * 2 + (size_t)2 * C * 4;
}

__global__ __launch_bounds__(NT) void tinv_kernel(TinvArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const bool gain = a.gain != nullptr;
  unsigned char* p = lds_raw;
  _Float16* sK = reinterpret_cast<_Float16*>(p);          // [C][KP] (phase 1-2)
  _Float16* sT = reinterpret_cast<_Float16*>(p);          // [C][CP] (phase 3-5, reuses sK)
  _Float16* sTt = sT + C * CP;                            // [C][CP] transposed T
  p += kTinvR1;
  _Float16* sB = sK;
  if (gain) {
    sB = reinterpret_cast<_Float16*>(p);
    p += C * KP * 2;
  }
  _Float16* sAh = reinterpret_cast<_Float16*>(p);  // [C][CP] A in fp16
  p += C * CP * 2;
  float* sAd = reinterpret_cast<float*>(p);        // [4][16][kAdP] diagonal blocks of A
  p += 4 * 16 * kAdP * 4;
  _Float16* sM = reinterpret_cast<_Float16*>(p);   // [4][16][24] per-wavefront scratch
  p += 4 * 16 * 24 * 2;
  float* sLg = reinterpret_cast<float*>(p);
  float* sBs = sLg + C;

  const int bh = blockIdx.x, c = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c0 = c * C, n = min(C, a.L - c0);
  const size_t tok = (size_t)bh * a.L + c0;

  // phase 1: stage K (and the gains) as fp16; per-token scalars
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int seg = tid + NT * i, row = seg >> 4, c8 = seg & 15;
    uint4 kv = make_uint4(0, 0, 0, 0), gv = make_uint4(0, 0, 0, 0);
    if (row < n) {
      kv = bf16x8_to_f16x8(*reinterpret_cast<const uint4*>(a.k + (tok + row) * DK + c8 * 8));
      if (gain) gv = *reinterpret_cast<const uint4*>(a.gain + (tok + row) * DK + c8 * 8);
    }
    *reinterpret_cast<uint4*>(sK + row * KP + c8 * 8) = kv;
    if (gain) *reinterpret_cast<uint4*>(sB + row * KP + c8 * 8) = gv;
  }
  if (wave == 0) {
    const TokenScalars s = token_scalars(a.alpha, a.beta, gain, a.plain, tok, lane, n);
    sLg[lane] = s.lg;
    sBs[lane] = s.bs;
  }
  __syncthreads();

  // phase 2: lower Gram tiles A = strict_lower((K B^T) * G) (10 tiles of 16x16)
  {
    const int r16 = lane & 15, k8 = (lane >> 4) * 8;
    for (int tl = wave; tl < 10; tl += 4) {
      const int ti = tl < 1 ? 0 : tl < 3 ? 1 : tl < 6 ? 2 : 3;
      const int tj = tl - ti * (ti + 1) / 2;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
        acc = mfma(ld8(sK + (16 * ti + r16) * KP + 32 * ks + k8),
                   ld8(sB + (16 * tj + r16) * KP + 32 * ks + k8), acc);
      const int col = 16 * tj + r16;
      const float lgc = sLg[col], bsc = sBs[col];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = 16 * ti + (lane >> 4) * 4 + jj;
        const float val = row > col ? acc[jj] * bsc * expf(sLg[row] - lgc) : 0.f;
        sAh[row * CP + col] = (_Float16)val;
        if (ti == tj) sAd[(ti * 16 + (row & 15)) * kAdP + (col & 15)] = val;
      }
    }
  }
  __syncthreads();

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
    const int r16 = lane & 15, kq = lane >> 4, k8 = kq * 8;
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
      __syncthreads();
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

  // phase 5: T (row-major, zero above the diagonal blocks) to the workspace
  _Float16* dst = a.tout + ((size_t)bh * a.nchunks + c) * C * C;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int seg = tid + NT * i, row = seg >> 3, c8 = seg & 7;
    uint4 val = make_uint4(0, 0, 0, 0);
    if ((c8 >> 1) <= (row >> 4)) val = *reinterpret_cast<const uint4*>(sT + row * CP + c8 * 8);
    *reinterpret_cast<uint4*>(dst + row * C + c8 * 8) = val;
  }
}

// =====================================================================  state scan

struct MainArgs {
  const uint16_t* q;     // bf16 [BH, L, DK]
  const uint16_t* k;     // bf16 [BH, L, DK]
  const uint16_t* v;     // bf16 [BH, L, dv]
  const _Float16* gain;  // fp16 [BH, L, DK] or null
  const float* alpha;
  const float* beta;
  const _Float16* tin;   // [BH, nchunks, C, C]
  const float* state_in;
  float* state_out;
  void* o;
  int out_bf16;
  int BH, L, dv, nchunks, ntiles, plain;
};

size_t main_lds_bytes(bool gain) {
  size_t b = 0;
  b += (size_t)C * KP * 2 * 2;            // sQ, sK
  if (gain) b += (size_t)C * KP * 2;      // sB
  b += (size_t)C * VP * 2;                // sV
  b += (size_t)C * CP * 2 * 2;            // sT, sP
  b += (size_t)DV * KP * 2;               // sST
  b += (size_t)DV * CP * 2 * 3;           // sXT, sUT, sUW
  b += (size_t)C * OP * 4;                // sO
  b += (size_t)5 * C * 4;                 // scalars
  return b;
}

struct ChunkRegs {
  uint4 q[4], k[4], g[4], v, t[2];
  float al, be;
};

__device__ __forceinline__ void load_chunk(const MainArgs& a, ChunkRegs& r, int bh, int j0, int c,
                                           int tid, bool gain) {
  const int c0 = c * C, n = min(C, a.L - c0);
  const size_t tok = (size_t)bh * a.L + c0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int seg = tid + NT * i, row = seg >> 4, c8 = seg & 15;
    const bool ok = row < n;
    const size_t off = (tok + row) * DK + c8 * 8;
    r.q[i] = ok ? *reinterpret_cast<const uint4*>(a.q + off) : make_uint4(0, 0, 0, 0);
    r.k[i] = ok ? *reinterpret_cast<const uint4*>(a.k + off) : make_uint4(0, 0, 0, 0);
    if (gain) r.g[i] = ok ? *reinterpret_cast<const uint4*>(a.gain + off) : make_uint4(0, 0, 0, 0);
  }
  {
    const int row = tid >> 2, c8 = tid & 3;
    r.v = row < n ? *reinterpret_cast<const uint4*>(a.v + (tok + row) * a.dv + j0 + c8 * 8)
                  : make_uint4(0, 0, 0, 0);
  }
  const _Float16* tsrc = a.tin + ((size_t)bh * a.nchunks + c) * C * C;
#pragma unroll
  for (int i = 0; i < 2; ++i) r.t[i] = *reinterpret_cast<const uint4*>(tsrc + (tid + NT * i) * 8);
  if (tid < C && tid < n) {
    r.al = a.alpha ? a.alpha[tok + tid] : 1.f;
    r.be = gain ? 1.f : a.beta[tok + tid];
  } else {
    r.al = 1.f;
    r.be = 0.f;
  }
}

__global__ __launch_bounds__(NT) void scan_kernel(MainArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const bool gain = a.gain != nullptr;
  unsigned char* p = lds_raw;
  _Float16* sQ = reinterpret_cast<_Float16*>(p); p += C * KP * 2;
  _Float16* sK = reinterpret_cast<_Float16*>(p); p += C * KP * 2;
  _Float16* sB = sK;
  if (gain) { sB = reinterpret_cast<_Float16*>(p); p += C * KP * 2; }
  _Float16* sV = reinterpret_cast<_Float16*>(p); p += C * VP * 2;
  _Float16* sT = reinterpret_cast<_Float16*>(p); p += C * CP * 2;
  _Float16* sP = reinterpret_cast<_Float16*>(p); p += C * CP * 2;
  _Float16* sST = reinterpret_cast<_Float16*>(p); p += DV * KP * 2;   // S^T (fp16)
  _Float16* sXT = reinterpret_cast<_Float16*>(p); p += DV * CP * 2;   // X^T
  _Float16* sUT = reinterpret_cast<_Float16*>(p); p += DV * CP * 2;   // U^T
  _Float16* sUW = reinterpret_cast<_Float16*>(p); p += DV * CP * 2;   // (w * U)^T
  float* sO = reinterpret_cast<float*>(p); p += C * OP * 4;
  float* sLg = reinterpret_cast<float*>(p);
  float* sBs = sLg + C;
  float* sVs = sBs + C;
  float* sW = sVs + C;
  float* sGam = sW + C;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4, k8 = kq * 8;

  // (head, d_v slice): the slices of one head land on one XCD (blocks are
  // dealt to the 8 XCDs round-robin), so they share that XCD's L2.
  int bh, tile;
  {
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
  const int j0 = tile * DV;

  // zero the upper tiles of P that the products touch (never written later)
  for (int e = tid; e < 16 * 16; e += NT) {
    const int rr = e >> 4, cc = e & 15;
    sP[rr * CP + 16 + cc] = (_Float16)0.f;
    sP[(32 + rr) * CP + 48 + cc] = (_Float16)0.f;
  }

  // state slice in the accumulators: wavefront w owns d_k rows [32w, 32w + 32)
  floatx4 S[2][2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * wave + 16 * db + kq * 4 + jj, col = 16 * cb + r16;
        S[db][cb][jj] = a.state_in ? a.state_in[((size_t)bh * DK + d) * a.dv + j0 + col] : 0.f;
      }
      st4(sST + (16 * cb + r16) * KP + 32 * wave + 16 * db + kq * 4, S[db][cb]);
    }

  ChunkRegs cur;
  load_chunk(a, cur, bh, j0, 0, tid, gain);

  for (int c = 0; c < a.nchunks; ++c) {
    const int c0 = c * C, n = min(C, a.L - c0);
    const size_t tok = (size_t)bh * a.L + c0;
    // registers -> LDS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int seg = tid + NT * i, row = seg >> 4, c8 = seg & 15;
      *reinterpret_cast<uint4*>(sQ + row * KP + c8 * 8) = bf16x8_to_f16x8(cur.q[i]);
      *reinterpret_cast<uint4*>(sK + row * KP + c8 * 8) = bf16x8_to_f16x8(cur.k[i]);
      if (gain) *reinterpret_cast<uint4*>(sB + row * KP + c8 * 8) = cur.g[i];
    }
    *reinterpret_cast<uint4*>(sV + (tid >> 2) * VP + (tid & 3) * 8) = bf16x8_to_f16x8(cur.v);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int seg = tid + NT * i, row = seg >> 3, c8 = seg & 7;
      *reinterpret_cast<uint4*>(sT + row * CP + c8 * 8) = cur.t[i];
    }
    if (wave == 0) {
      float la = 0.f, bs = 0.f, vs = 1.f;
      if (lane < n) {
        la = logf(cur.al);
        bs = cur.be;
        if (a.plain) {
          bs /= cur.al;
          vs = cur.al;
        }
      }
      const float lg = wave_prefix(la, lane);
      const float lgn = __shfl(lg, n - 1, 64);
      sLg[lane] = lg;
      sBs[lane] = bs;
      sVs[lane] = vs;
      sGam[lane] = expf(lg);
      sW[lane] = lane < n ? expf(lgn - lg) * bs : 0.f;
    }
    __syncthreads();
    if (c + 1 < a.nchunks) load_chunk(a, cur, bh, j0, c + 1, tid, gain);

    // --- phase A: P = lower_incl((Q B^T) * G); K S, Q S; X = V - g K S
    for (int tl = wave; tl < 10; tl += 4) {
      const int ti = tl < 1 ? 0 : tl < 3 ? 1 : tl < 6 ? 2 : 3;
      const int tj = tl - ti * (ti + 1) / 2;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
        acc = mfma(ld8(sQ + (16 * ti + r16) * KP + 32 * ks + k8),
                   ld8(sB + (16 * tj + r16) * KP + 32 * ks + k8), acc);
      const int col = 16 * tj + r16;
      const float lgc = sLg[col], bsc = sBs[col];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = 16 * ti + kq * 4 + jj;
        const float val = row >= col ? acc[jj] * bsc * expf(sLg[row] - lgc) : 0.f;
        sP[row * CP + col] = (_Float16)val;
      }
    }
    floatx4 Opart[2];
    {
      floatx4 ks_acc[2], qs_acc[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        ks_acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
        qs_acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kd = 0; kd < DK / 32; ++kd) {
        const half8 kv = ld8(sK + (16 * wave + r16) * KP + 32 * kd + k8);
        const half8 qv = ld8(sQ + (16 * wave + r16) * KP + 32 * kd + k8);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const half8 sv = ld8(sST + (16 * cb + r16) * KP + 32 * kd + k8);
          ks_acc[cb] = mfma(kv, sv, ks_acc[cb]);
          qs_acc[cb] = mfma(qv, sv, qs_acc[cb]);
        }
      }
      const int t0 = 16 * wave + kq * 4;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int col = 16 * cb + r16;
        floatx4 x;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int t = t0 + jj;
          const float g = sGam[t];
          x[jj] = sVs[t] * (float)sV[t * VP + col] - g * ks_acc[cb][jj];
          Opart[cb][jj] = g * qs_acc[cb][jj];
        }
        st4(sXT + col * CP + t0, x);
      }
    }
    __syncthreads();

    // --- phase B: U = T X (rows of this wavefront's 16-token block)
    {
      const int nks = wave >= 2 ? 2 : 1;
      const int t0 = 16 * wave + kq * 4;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < nks; ++ks)
          acc = mfma(ld8(sT + (16 * wave + r16) * CP + 32 * ks + k8),
                     ld8(sXT + (16 * cb + r16) * CP + 32 * ks + k8), acc);
        const int col = 16 * cb + r16;
        st4(sUT + col * CP + t0, acc);
        floatx4 wu;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) wu[jj] = acc[jj] * sW[t0 + jj];
        st4(sUW + col * CP + t0, wu);
      }
    }
    __syncthreads();

    // --- phase C: O = g Q S + P U;  S = g_n S + sum_t w_t b_t U_t^T
    {
      const int nks = wave >= 2 ? 2 : 1;
      const int t0 = 16 * wave + kq * 4;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        floatx4 acc = Opart[cb];
        for (int ks = 0; ks < nks; ++ks)
          acc = mfma(ld8(sP + (16 * wave + r16) * CP + 32 * ks + k8),
                     ld8(sUT + (16 * cb + r16) * CP + 32 * ks + k8), acc);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sO[(t0 + jj) * OP + 16 * cb + r16] = acc[jj];
      }
      const float gn = sGam[n - 1];
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int dcol = 32 * wave + 16 * db + r16;  // d_k index this lane reads
        half8 bt[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) bt[ks][e] = sB[(32 * ks + k8 + e) * KP + dcol];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          floatx4 acc = S[db][cb] * gn;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            acc = mfma(bt[ks], ld8(sUW + (16 * cb + r16) * CP + 32 * ks + k8), acc);
          S[db][cb] = acc;
          st4(sST + (16 * cb + r16) * KP + 32 * wave + 16 * db + kq * 4, acc);
        }
      }
    }
    __syncthreads();

    // --- phase D: outputs of this chunk
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int seg = tid + NT * i, row = seg >> 3, c4 = seg & 7;
      if (row < n) {
        const float4 val = *reinterpret_cast<const float4*>(sO + row * OP + c4 * 4);
        const size_t off = (tok + row) * a.dv + j0 + c4 * 4;
        if (a.out_bf16) {
          uint16_t* op = static_cast<uint16_t*>(a.o) + off;
          const uint32_t lo = (uint32_t)f32_to_bf16(val.x) | ((uint32_t)f32_to_bf16(val.y) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16(val.z) | ((uint32_t)f32_to_bf16(val.w) << 16);
          *reinterpret_cast<uint2*>(op) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.o) + off) = val;
        }
      }
    }
  }

  if (a.state_out) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = 32 * wave + 16 * db + kq * 4 + jj, col = 16 * cb + r16;
          a.state_out[((size_t)bh * DK + d) * a.dv + j0 + col] = S[db][cb][jj];
        }
  }
}

}  // namespace

bool scan_mfma_supported(int dk, int dv, int chunk) {
  return dk == DK && chunk == C && dv % DV == 0 && dv >= DV;
}

size_t scan_mfma_workspace_bytes(int BH, int L) {
  const size_t nchunks = ((size_t)L + C - 1) / C;
  return (size_t)BH * nchunks * C * C * sizeof(_Float16);
}

hipError_t launch_tinv_mfma(const ScanArgs& s, void* tbuf, hipStream_t st) {
  const int nchunks = (s.L + C - 1) / C;
  const bool gain = s.gain != nullptr;
  TinvArgs ta;
  ta.k = static_cast<const uint16_t*>(s.k);
  ta.gain = static_cast<const _Float16*>(s.gain);
  ta.alpha = s.alpha;
  ta.beta = s.beta;
  ta.tout = static_cast<_Float16*>(tbuf);
  ta.L = s.L;
  ta.nchunks = nchunks;
  ta.plain = s.plain;
  const size_t lds = tinv_lds_bytes(gain);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(tinv_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tinv_kernel, dim3(s.BH, nchunks), dim3(NT), lds, st, ta);
  return hipGetLastError();
}

hipError_t launch_state_mfma(const ScanArgs& s, bool out_bf16, const void* tbuf, hipStream_t st) {
  const bool gain = s.gain != nullptr;
  MainArgs ma;
  ma.q = static_cast<const uint16_t*>(s.q);
  ma.k = static_cast<const uint16_t*>(s.k);
  ma.v = static_cast<const uint16_t*>(s.v);
  ma.gain = static_cast<const _Float16*>(s.gain);
  ma.alpha = s.alpha;
  ma.beta = s.beta;
  ma.tin = static_cast<const _Float16*>(tbuf);
  ma.state_in = s.state_in;
  ma.state_out = s.state_out;
  ma.o = s.o;
  ma.out_bf16 = out_bf16 ? 1 : 0;
  ma.BH = s.BH;
  ma.L = s.L;
  ma.dv = s.dv;
  ma.nchunks = (s.L + C - 1) / C;
  ma.ntiles = s.dv / DV;
  ma.plain = s.plain;
  const size_t lds = main_lds_bytes(gain);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(scan_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(s.BH * ma.ntiles), dim3(NT), lds, st, ma);
  return hipGetLastError();
}

}  // namespace kdn
