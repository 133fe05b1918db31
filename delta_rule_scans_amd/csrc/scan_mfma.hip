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
//
// Two kernels:
//  * prep_kernel: one workgroup per (head, chunk), every chunk in parallel.
//    Everything that does not depend on the state: the per-token decay
//    scalars g_t, w_t; the Grams K B^T and Q B^T on the matrix cores; and
//    T = (I + A)^-1 by blocks of 16: the four diagonal blocks are inverted in
//    float32 registers (one wavefront per block, four lanes per column, quad
//    reductions through DPP), the six off-diagonal blocks follow by block
//    products on the matrix cores, diagonal by diagonal:
//    T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj.
//    Output per (head, chunk): T and P (fp16, 64 x 64 each) and the scalars.
//  * state_kernel: one workgroup per (head, 32-column slice of d_v); the loop
//    over chunks is sequential. The float32 state slice (128 x 32) stays in
//    the matrix-core accumulators for the whole sequence; its fp16 copy in LDS
//    feeds the products K S and Q S. Per chunk: K S and Q S, U = T X, P U and
//    the state update, three workgroup barriers; the next chunk's inputs are
//    prefetched two chunks ahead into registers.
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

// Per (head, chunk) record written by prep_kernel and read by state_kernel.
constexpr size_t kRecT = 0;                       // T, fp16 [C][C]
constexpr size_t kRecP = C * C * 2;               // P, fp16 [C][C]
constexpr size_t kRecS = 2 * C * C * 2;           // scalars, float4 [C]: g, w, value scale, 0
constexpr size_t kRecBytes = kRecS + C * 16;      // 17408

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

// 8 bf16 values (one 16-byte load), each times `scale`, -> 8 fp16 values.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 u, float scale) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 lo = (_Float16)(__uint_as_float(w[i] << 16) * scale);
    const _Float16 hi = (_Float16)(__uint_as_float(w[i] & 0xffff0000u) * scale);
    r[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
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
  unsigned char* rec;     // [BH, nchunks] records of kRecBytes
  int L, nchunks, plain;
};

constexpr int kAdP = 17;  // fp32 pitch of the diagonal blocks of A
constexpr int kPrepR1 = (C * KP > 2 * C * CP ? C * KP : 2 * C * CP) * 2;  // sQ, later sT + sTt

size_t prep_lds_bytes(bool gain) {
  return (size_t)kPrepR1 + (size_t)C * KP * 2 + (gain ? (size_t)C * KP * 2 : 0) +
         (size_t)C * CP * 2 + (size_t)4 * 16 * kAdP * 4 + (size_t)4 * 16 * 24 * 2 +
         (size_t)2 * C * 4;
}

__global__ __launch_bounds__(NT) void prep_kernel(PrepArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const bool gain = a.gain != nullptr;
  unsigned char* p = lds_raw;
  _Float16* sQ = reinterpret_cast<_Float16*>(p);   // [C][KP] (phases 1-2)
  _Float16* sT = reinterpret_cast<_Float16*>(p);   // [C][CP] (phases 3-5, reuses sQ)
  _Float16* sTt = sT + C * CP;                     // [C][CP] T transposed
  p += kPrepR1;
  _Float16* sK = reinterpret_cast<_Float16*>(p);   // [C][KP] (phases 1-2)
  _Float16* sP = sK;                               // [C][CP] (phases 3-5, reuses sK)
  p += C * KP * 2;
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
  float* sLg = reinterpret_cast<float*>(p);        // [C] log2 of g
  float* sBs = sLg + C;                            // [C] write scale

  const int bh = blockIdx.x, c = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4, k8 = kq * 8;
  const int c0 = c * C, n = min(C, a.L - c0);
  const size_t tok = (size_t)bh * a.L + c0;
  unsigned char* rec = a.rec + ((size_t)bh * a.nchunks + c) * kRecBytes;

  // phase 1: stage Q, K (and the gains) as fp16; per-token scalars
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int seg = tid + NT * i, row = seg >> 4, c8 = seg & 15;
    uint4 qv = make_uint4(0, 0, 0, 0), kv = qv, gv = qv;
    if (row < n) {
      const size_t off = (tok + row) * DK + c8 * 8;
      qv = bf16x8_to_f16x8(*reinterpret_cast<const uint4*>(a.q + off), 1.f);
      kv = bf16x8_to_f16x8(*reinterpret_cast<const uint4*>(a.k + off), 1.f);
      if (gain) gv = *reinterpret_cast<const uint4*>(a.gain + off);
    }
    *reinterpret_cast<uint4*>(sQ + row * KP + c8 * 8) = qv;
    *reinterpret_cast<uint4*>(sK + row * KP + c8 * 8) = kv;
    if (gain) *reinterpret_cast<uint4*>(sB + row * KP + c8 * 8) = gv;
  }
  if (wave == 0) {
    float la = 0.f, bs = 0.f, vs = 1.f;
    if (lane < n) {
      const float al = a.alpha ? a.alpha[tok + lane] : 1.f;
      la = log2f(al);
      bs = gain ? 1.f : a.beta[tok + lane];
      if (a.plain) {  // plain residual = gated form with (beta / alpha, alpha v)
        bs /= al;
        vs = al;
      }
    }
    const float lg = wave_prefix(la, lane);
    const float lgn = __shfl(lg, n - 1, 64);
    sLg[lane] = lg;
    sBs[lane] = bs;
    const float w = lane < n ? exp2f(lgn - lg) * bs : 0.f;
    *reinterpret_cast<float4*>(rec + kRecS + lane * 16) = make_float4(exp2f(lg), w, vs, 0.f);
  }
  __syncthreads();

  // phase 2: 20 lower Gram tiles, A (tiles 0-9) from K and P (tiles 10-19) from Q;
  // wavefront w takes tiles w, w + 4, ..., w + 16.
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
    const float4 lgr = *reinterpret_cast<const float4*>(sLg + 16 * ti + kq * 4);
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

  // phase 5: T and P (row-major, zero above the diagonal blocks) to the record
  _Float16* tdst = reinterpret_cast<_Float16*>(rec + kRecT);
  _Float16* pdst = reinterpret_cast<_Float16*>(rec + kRecP);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int seg = tid + NT * i, row = seg >> 3, c8 = seg & 7;
    const bool lower = (c8 >> 1) <= (row >> 4);
    uint4 tv = make_uint4(0, 0, 0, 0), pv = tv;
    if (lower) {
      tv = *reinterpret_cast<const uint4*>(sT + row * CP + c8 * 8);
      pv = *reinterpret_cast<const uint4*>(sP + row * CP + c8 * 8);
    }
    *reinterpret_cast<uint4*>(tdst + row * C + c8 * 8) = tv;
    *reinterpret_cast<uint4*>(pdst + row * C + c8 * 8) = pv;
  }
}

// =====================================================================  state kernel
//
// Warp-specialised: wavefronts 0-7 compute, wavefronts 8-15 move data.
//  * The compute wavefronts never load from global memory (they only store
//    o), so nothing in their chunk loop waits on the memory counters.
//    Wavefront w owns token block rb = w % 4 and value block cb = w / 4 of
//    the 64 x 32 chunk outputs, and the state tiles (d_k blocks 2 rb, 2 rb + 1;
//    value block cb), 128 x 32 in all, in float32 accumulators.
//  * The producer wavefronts load chunk c + 3 while chunk c is computed
//    (two register buffers), and convert chunk c + 1 into the LDS buffer
//    (c + 1) % 2 that chunk c - 1 has released. The two roles run separate
//    loops with the same barriers, so their registers never overlap.

struct StateArgs {
  const uint16_t* q;     // bf16 [BH, L, DK]
  const uint16_t* k;     // bf16 [BH, L, DK]
  const uint16_t* v;     // bf16 [BH, L, dv]
  const _Float16* gain;  // fp16 [BH, L, DK] or null
  const unsigned char* rec;
  const float* state_in;
  float* state_out;
  void* o;
  int out_bf16;
  int BH, L, dv, nchunks, ntiles;
};

constexpr int NW_COMPUTE = 8;
constexpr int NW_PROD = 8;
constexpr int NT_STATE = 64 * (NW_COMPUTE + NW_PROD);
constexpr int NT_PROD = 64 * NW_PROD;

// One LDS buffer of chunk inputs.
struct StageBuf {
  _Float16* q;     // [C][KP] fp16
  _Float16* k;     // [C][KP] fp16
  _Float16* t;     // [C][CP] T
  _Float16* p;     // [C][CP] P
  _Float16* vt;    // [DV][CP] V^T
  float* gam;      // [C] g
  float* w;        // [C] w
  float* vs;       // [C] value scale
};

constexpr size_t kStageBytes = (size_t)2 * C * KP * 2 + (size_t)2 * C * CP * 2 +
                               (size_t)DV * CP * 2 + (size_t)3 * C * 4;

size_t state_lds_bytes(bool gain) {
  return 2 * kStageBytes + (gain ? (size_t)C * KP * 2 : 0)  // stage buffers, gains
         + (size_t)DV * KP * 2                              // S^T
         + (size_t)3 * DV * CP * 2;                         // X^T, U^T, (w U)^T
}

__device__ __forceinline__ StageBuf carve_stage(unsigned char* p) {
  StageBuf b;
  b.q = reinterpret_cast<_Float16*>(p); p += C * KP * 2;
  b.k = reinterpret_cast<_Float16*>(p); p += C * KP * 2;
  b.t = reinterpret_cast<_Float16*>(p); p += C * CP * 2;
  b.p = reinterpret_cast<_Float16*>(p); p += C * CP * 2;
  b.vt = reinterpret_cast<_Float16*>(p); p += DV * CP * 2;
  b.gam = reinterpret_cast<float*>(p); p += C * 4;
  b.w = reinterpret_cast<float*>(p); p += C * 4;
  b.vs = reinterpret_cast<float*>(p);
  return b;
}

// Raw inputs of one chunk in a producer's registers. Loads are unconditional
// (rows past the chunk's end are clamped to its last row) and nothing is
// computed from them until the chunk is staged.
template <bool GAIN> struct BufGain {};
template <> struct BufGain<true> {
  uint4 g0, g1;            // gains of the q/k rows
};

template <bool GAIN>
struct Buf : BufGain<GAIN> {
  uint4 q0, q1, k0, k1;    // rows p / 16 and p / 16 + 32, columns 8 (p % 16) ..
  uint4 t, pm;             // T and P: row p / 8, columns 8 (p % 8) ..
  uint2 v;                 // value row p / 8, columns j0 + 4 (p % 8) ..
  float4 sc;               // scalars of token p % 64
};

template <bool GAIN>
__device__ __forceinline__ void load_buf(const StateArgs& a, Buf<GAIN>& b, int bh, int j0, int c,
                                         int p) {
  const int c0 = c * C, n = min(C, a.L - c0);
  const size_t tok = (size_t)bh * a.L + c0;
  const unsigned char* rec = a.rec + ((size_t)bh * a.nchunks + c) * kRecBytes;
  const float4* sc = reinterpret_cast<const float4*>(rec + kRecS);
  const size_t off0 = (tok + min(p >> 4, n - 1)) * DK + (p & 15) * 8;
  const size_t off1 = (tok + min((p >> 4) + 32, n - 1)) * DK + (p & 15) * 8;
  b.q0 = *reinterpret_cast<const uint4*>(a.q + off0);
  b.q1 = *reinterpret_cast<const uint4*>(a.q + off1);
  b.k0 = *reinterpret_cast<const uint4*>(a.k + off0);
  b.k1 = *reinterpret_cast<const uint4*>(a.k + off1);
  if constexpr (GAIN) {
    b.g0 = *reinterpret_cast<const uint4*>(a.gain + off0);
    b.g1 = *reinterpret_cast<const uint4*>(a.gain + off1);
  }
  b.t = reinterpret_cast<const uint4*>(rec + kRecT)[p];
  b.pm = reinterpret_cast<const uint4*>(rec + kRecP)[p];
  const int vrow = min(p >> 3, n - 1);
  b.v = *reinterpret_cast<const uint2*>(a.v + (tok + vrow) * a.dv + j0 + (p & 7) * 4);
  b.sc = sc[p & 63];
}

// Convert a chunk into LDS (everything but the gains). Every thread consumes
// everything it loaded, on every path: a load consumed only on some paths
// makes the compiler wait for all outstanding loads before reusing its
// registers, which would serialise the prefetch.
template <bool GAIN>
__device__ __forceinline__ void stage_buf(const StateArgs& a, const Buf<GAIN>& b, const StageBuf& s,
                                          int c, int p) {
  const int n = min(C, a.L - c * C);
  {
    const int row = p >> 4, c8 = p & 15;
    const float keep0 = row < n ? 1.f : 0.f, keep1 = row + 32 < n ? 1.f : 0.f;
    *reinterpret_cast<uint4*>(s.q + row * KP + c8 * 8) = bf16x8_to_f16x8(b.q0, keep0);
    *reinterpret_cast<uint4*>(s.k + row * KP + c8 * 8) = bf16x8_to_f16x8(b.k0, keep0);
    *reinterpret_cast<uint4*>(s.q + (row + 32) * KP + c8 * 8) = bf16x8_to_f16x8(b.q1, keep1);
    *reinterpret_cast<uint4*>(s.k + (row + 32) * KP + c8 * 8) = bf16x8_to_f16x8(b.k1, keep1);
  }
  {
    const int row = p >> 3, c8 = p & 7;
    *reinterpret_cast<uint4*>(s.t + row * CP + c8 * 8) = b.t;
    *reinterpret_cast<uint4*>(s.p + row * CP + c8 * 8) = b.pm;
  }
  {
    const int row = p >> 3, c4 = (p & 7) * 4;
    const float keep = row < n ? 1.f : 0.f;
    const uint32_t w[2] = {b.v.x, b.v.y};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      s.vt[(c4 + 2 * e) * CP + row] = (_Float16)(__uint_as_float(w[e] << 16) * keep);
      s.vt[(c4 + 2 * e + 1) * CP + row] = (_Float16)(__uint_as_float(w[e] & 0xffff0000u) * keep);
    }
  }
  // eight threads write each token's scalars (the same values)
  s.gam[p & 63] = b.sc.x;
  s.w[p & 63] = b.sc.y;
  s.vs[p & 63] = b.sc.z;
}

__device__ __forceinline__ void stage_gain(const Buf<true>& b, _Float16* sG, int n, int p) {
  const int row = p >> 4, c8 = p & 15;
  const uint4 z = make_uint4(0, 0, 0, 0);
  *reinterpret_cast<uint4*>(sG + row * KP + c8 * 8) = row < n ? b.g0 : z;
  *reinterpret_cast<uint4*>(sG + (row + 32) * KP + c8 * 8) = row + 32 < n ? b.g1 : z;
}

template <bool GAIN>
__global__ __launch_bounds__(NT_STATE) void state_kernel(StateArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  unsigned char* lp = lds_raw + 2 * kStageBytes;  // two stage buffers first
  _Float16* sG = nullptr;
  if (GAIN) { sG = reinterpret_cast<_Float16*>(lp); lp += C * KP * 2; }
  _Float16* sST = reinterpret_cast<_Float16*>(lp); lp += DV * KP * 2;  // S^T (fp16)
  _Float16* sXT = reinterpret_cast<_Float16*>(lp); lp += DV * CP * 2;  // X^T
  _Float16* sUT = reinterpret_cast<_Float16*>(lp); lp += DV * CP * 2;  // U^T
  _Float16* sUW = reinterpret_cast<_Float16*>(lp);                     // (w U)^T

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4, k8 = kq * 8;
  const bool producer = wave >= NW_COMPUTE;
  const int p = tid - 64 * NW_COMPUTE;          // producer thread index
  const int rb = wave & 3, cb = (wave >> 2) & 1; // compute wavefront's blocks
  const int t0 = 16 * rb + kq * 4;               // this lane's 4 token rows
  const int col = 16 * cb + r16;                 // this lane's value column (in the slice)

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

  // Both loops run an even number of chunk steps (an odd count gets one
  // idle step), three barriers per step, so the barrier counts match.
  const int nsteps = (a.nchunks + 1) & ~1;
  const int last = a.nchunks - 1;

  if (producer) {
    // ---------------------------------------------------------- producers
    // Step c: stage chunk c + 1 from the register buffer that holds it into
    // LDS buffer (c + 1) % 2, then reload that register buffer with chunk
    // c + 3. Every load and stage is unconditional (chunk indices are clamped
    // to the last chunk; restaging it into the idle buffer is harmless), so
    // no path leaves a load pending and the compiler waits only for the
    // buffer being consumed, never for the one still in flight.
    Buf<GAIN> r0, r1;
    load_buf<GAIN>(a, r0, bh, j0, 0, p);
    load_buf<GAIN>(a, r1, bh, j0, min(1, last), p);
    stage_buf<GAIN>(a, r0, carve_stage(lds_raw), 0, p);
    if constexpr (GAIN) stage_gain(r0, sG, min(C, a.L), p);
    load_buf<GAIN>(a, r0, bh, j0, min(2, last), p);
    __syncthreads();
    // The scheduling barriers keep the compiler from hoisting the next
    // step's conversions (and so its waits for loads still in flight) into
    // this step.
    auto pbody = [&](int c, Buf<GAIN>& rn) {
      const int cn = min(c + 1, last);
      __builtin_amdgcn_sched_barrier(0);
      stage_buf<GAIN>(a, rn, carve_stage(lds_raw + ((c + 1) & 1) * kStageBytes), cn, p);
      if constexpr (!GAIN) load_buf<GAIN>(a, rn, bh, j0, min(c + 3, last), p);
      __syncthreads();
      if constexpr (GAIN) {
        // the gains of chunk c + 1 (the compute side read chunk c's before the barrier)
        stage_gain(rn, sG, min(C, a.L - cn * C), p);
        load_buf<GAIN>(a, rn, bh, j0, min(c + 3, last), p);
      }
      __syncthreads();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int c = 0; c < nsteps; c += 2) {
      pbody(c, r1);
      pbody(c + 1, r0);
    }
    return;
  }

  // ------------------------------------------------------------ compute
  floatx4 S[2];  // state tiles (d_k blocks 2 rb, 2 rb + 1; value block cb)
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = 32 * rb + 16 * db + kq * 4 + jj;
      S[db][jj] = a.state_in ? a.state_in[((size_t)bh * DK + d) * a.dv + j0 + col] : 0.f;
    }
    st4(sST + col * KP + 32 * rb + 16 * db + kq * 4, S[db]);
  }
  __syncthreads();

  const int nks = rb >= 2 ? 2 : 1;
  for (int c = 0; c < nsteps; ++c) {
    if (c > last) {  // the idle step of an odd chunk count
      __syncthreads();
      __syncthreads();
      __syncthreads();
      break;
    }
    const StageBuf cur = carve_stage(lds_raw + (c & 1) * kStageBytes);
    const int n = min(C, a.L - c * C);
    // state-update operand B^T for this wavefront's d_k blocks, gathered early
    half8 bt[2][2];
    const _Float16* srcB = GAIN ? sG : cur.k;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          bt[db][ks][e] = srcB[(32 * ks + k8 + e) * KP + 32 * rb + 16 * db + r16];
    // phase A: K S and Q S for (rb, cb); X = v_scale V - g K S; O part g Q S
    floatx4 opart;
    {
      floatx4 ks_acc = {0.f, 0.f, 0.f, 0.f}, qs_acc = ks_acc;
#pragma unroll
      for (int kd = 0; kd < DK / 32; ++kd) {
        const half8 sv = ld8(sST + col * KP + 32 * kd + k8);
        ks_acc = mfma(ld8(cur.k + (16 * rb + r16) * KP + 32 * kd + k8), sv, ks_acc);
        qs_acc = mfma(ld8(cur.q + (16 * rb + r16) * KP + 32 * kd + k8), sv, qs_acc);
      }
      const float4 g4 = *reinterpret_cast<const float4*>(cur.gam + t0);
      const float4 s4 = *reinterpret_cast<const float4*>(cur.vs + t0);
      const half4 v4 = *reinterpret_cast<const half4*>(cur.vt + col * CP + t0);
      const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
      const float sv4[4] = {s4.x, s4.y, s4.z, s4.w};
      floatx4 x;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        x[jj] = sv4[jj] * (float)v4[jj] - gv[jj] * ks_acc[jj];
        opart[jj] = gv[jj] * qs_acc[jj];
      }
      st4(sXT + col * CP + t0, x);
    }
    __syncthreads();

    // phase B: U = T X for (rb, cb)
    {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < nks; ++ks)
        acc = mfma(ld8(cur.t + (16 * rb + r16) * CP + 32 * ks + k8),
                   ld8(sXT + col * CP + 32 * ks + k8), acc);
      st4(sUT + col * CP + t0, acc);
      const float4 w4 = *reinterpret_cast<const float4*>(cur.w + t0);
      floatx4 wu;
      wu[0] = acc[0] * w4.x;
      wu[1] = acc[1] * w4.y;
      wu[2] = acc[2] * w4.z;
      wu[3] = acc[3] * w4.w;
      st4(sUW + col * CP + t0, wu);
    }
    __syncthreads();

    // phase C: O = g Q S + P U;  S = g_n S + B^T (w U)
    {
      floatx4 acc = opart;
      for (int ks = 0; ks < nks; ++ks)
        acc = mfma(ld8(cur.p + (16 * rb + r16) * CP + 32 * ks + k8),
                   ld8(sUT + col * CP + 32 * ks + k8), acc);
      const size_t tok = (size_t)bh * a.L + (size_t)c * C;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (t0 + jj < n) {
          const size_t off = (tok + t0 + jj) * a.dv + j0 + col;
          if (a.out_bf16)
            static_cast<uint16_t*>(a.o)[off] = f32_to_bf16(acc[jj]);
          else
            static_cast<float*>(a.o)[off] = acc[jj];
        }
      }
      const float gn = cur.gam[n - 1];
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        floatx4 st = S[db] * gn;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) st = mfma(bt[db][ks], ld8(sUW + col * CP + 32 * ks + k8), st);
        S[db] = st;
        st4(sST + col * KP + 32 * rb + 16 * db + kq * 4, st);
      }
    }
    __syncthreads();
  }

  if (a.state_out) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * rb + 16 * db + kq * 4 + jj;
        a.state_out[((size_t)bh * DK + d) * a.dv + j0 + col] = S[db][jj];
      }
  }
}

}  // namespace

bool scan_mfma_supported(int dk, int dv, int chunk) {
  return dk == DK && chunk == C && dv % DV == 0 && dv >= DV;
}

size_t scan_mfma_workspace_bytes(int BH, int L) {
  const size_t nchunks = ((size_t)L + C - 1) / C;
  return (size_t)BH * nchunks * kRecBytes;
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
  const size_t lds = prep_lds_bytes(gain);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prep_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prep_kernel, dim3(s.BH, nchunks), dim3(NT), lds, st, pa);
  return hipGetLastError();
}

template <bool GAIN>
hipError_t launch_state_typed(const StateArgs& sa, hipStream_t st) {
  const size_t lds = state_lds_bytes(GAIN);
  auto kern = state_kernel<GAIN>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(sa.BH * sa.ntiles), dim3(NT_STATE), lds, st, sa);
  return hipGetLastError();
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
  sa.out_bf16 = out_bf16 ? 1 : 0;
  sa.BH = s.BH;
  sa.L = s.L;
  sa.dv = s.dv;
  sa.nchunks = (s.L + C - 1) / C;
  sa.ntiles = s.dv / DV;
  return s.gain ? launch_state_typed<true>(sa, st) : launch_state_typed<false>(sa, st);
}

}  // namespace kdn
