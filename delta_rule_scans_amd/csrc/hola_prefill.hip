// hola_prefill.hip -- the HOLA exact cache over a whole prompt, block by block.
//
// "A Hippocampus for Linear Attention", sec. 3.3 (the cache keeps the w tokens
// with the largest write score; the top-w of a set does not depend on the order
// its members arrive in), sec. 3.4 eq. (7) (a token reads over the cache, the
// causal tokens of its own block and an optional null sink, with RMS-normalised
// query and keys at 1/sqrt(d_k)), sec. 3.2 eq. (4) (softmax read).
//
// Block j's tokens read the cache as it stood before block j; then the block
// is inserted. Three kernels:
//  * block top: one workgroup per (head, block), every block in parallel,
//    ranks the block's tokens by score descending, position ascending (or by
//    position descending for the recency control) and keeps the first w.
//  * merge: one workgroup per head walks the blocks in order, records for
//    every block which tokens the cache holds when the block reads it, then
//    merges the block's top list in.
//  * read: one workgroup per (head, block, 64 queries), every block in
//    parallel: streaming softmax over 32-key tiles of (cache members, causal
//    block tokens), float32 on the matrix cores.
//  * commit: one workgroup per (head, member) gathers the final members' keys
//    and values (from the old cache or the prompt) into staging rows, then a
//    second launch writes the cache in rank order.
#include <math.h>

#include "kdn_internal.h"

namespace kdn {
namespace {

constexpr int NT = 256;
constexpr int QT = 64;   // queries per read workgroup
constexpr int KT = 32;   // keys per tile
constexpr int MAXD = 128;
constexpr int kMaxW = 256;       // largest cache capacity
constexpr int kMaxBlock = 1024;  // largest prompt block

// NaN scores rank below every other score.
__device__ __forceinline__ float score_key(float m) { return m == m ? m : -INFINITY; }

// Block tops: the w best tokens of each block on its own, every block in
// parallel. Positions rise with the index inside a block, so the score order
// ties break on the index and the recency order is the reverse index order.
// Each token's rank is counted against the whole block.
__global__ __launch_bounds__(NT) void block_top_kernel(PrefillArgs a) {
  __shared__ __align__(16) float sm[kMaxBlock];
  const int bh = blockIdx.x, j = blockIdx.y, tid = threadIdx.x;
  const int nblk = (a.L + a.block - 1) / a.block;
  const int j0 = j * a.block, nb = min(a.block, a.L - j0);
  const float* mh = a.m + (size_t)bh * a.L + j0;
  for (int i = tid; i < nb; i += NT) sm[i] = score_key(mh[i]);
  for (int i = nb + tid; i < ((nb + 3) & ~3); i += NT) sm[i] = -INFINITY;
  __syncthreads();
  const size_t base = ((size_t)bh * nblk + j) * a.w;
  for (int x = tid; x < nb; x += NT) {
    int rank;
    if (a.policy == 1) {
      rank = nb - 1 - x;
    } else {
      const float mx = sm[x];
      rank = 0;
      // padding slots hold -inf and sit after x, so they never count
      for (int y = 0; y < nb; y += 4) {
        const float4 m4 = *reinterpret_cast<const float4*>(&sm[y]);
        rank += (m4.x > mx) | ((m4.x == mx) & (y < x));
        rank += (m4.y > mx) | ((m4.y == mx) & (y + 1 < x));
        rank += (m4.z > mx) | ((m4.z == mx) & (y + 2 < x));
        rank += (m4.w > mx) | ((m4.w == mx) & (y + 3 < x));
      }
    }
    if (rank < a.w) {
      a.top_m[base + rank] = mh[x];
      a.top_pos[base + rank] = a.t0 + j0 + x;
      a.top_src[base + rank] = j0 + x;
    }
  }
}

// Cache members are coded as src >= 0: prompt token src; src < 0: old slot -1 - src.
//
// The cache a block reads is the top-w of the old cache and every earlier
// block, and the top-w of a union is the top-w of the union of the parts'
// top-w lists, so one workgroup per head merges the block tops in order: two
// sorted lists, each entry's new rank is its own index plus the number of
// entries of the other list ahead of it (a binary search). On a full tie the
// cache entry goes first, as the earlier candidate.
__global__ __launch_bounds__(NT) void merge_kernel(PrefillArgs a) {
  __shared__ float cm[2][kMaxW];
  __shared__ int cp[2][kMaxW], cs[2][kMaxW];
  __shared__ float tm[kMaxW];
  __shared__ int tp[kMaxW];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int nblk = (a.L + a.block - 1) / a.block;
  const bool rec = a.policy == 1;
  int n = min(max(a.cache_count[bh], 0), a.w);
  // the old cache need not be in rank order: rank it by counting, ties by slot
  if (tid < n) {
    cm[1][tid] = a.cache_m[(size_t)bh * a.w + tid];
    cp[1][tid] = a.cache_pos[(size_t)bh * a.w + tid];
  }
  __syncthreads();
  if (tid < n) {
    const float mx = score_key(cm[1][tid]);
    const int px = cp[1][tid];
    int r = 0;
    for (int y = 0; y < n; ++y) {
      const float my = score_key(cm[1][y]);
      const int py = cp[1][y];
      const bool tie_first = y < tid;
      r += rec ? (py > px || (py == px && tie_first))
               : (my > mx || (my == mx && (py < px || (py == px && tie_first))));
    }
    cm[0][r] = cm[1][tid];
    cp[0][r] = px;
    cs[0][r] = -1 - tid;
  }
  int cur = 0;
  // the next block top, loaded a step ahead
  const size_t tbase = (size_t)bh * nblk * a.w;
  float nm = 0.f;
  int npos = 0, nsrc = 0;
  if (tid < min(a.block, a.L) && tid < a.w) {
    nm = a.top_m[tbase + tid];
    npos = a.top_pos[tbase + tid];
    nsrc = a.top_src[tbase + tid];
  }
  __syncthreads();
  for (int j = 0; j < nblk; ++j) {
    const int nt = min(min(a.block, a.L - j * a.block), a.w);
    int* mem = a.members + ((size_t)bh * nblk + j) * a.w;
    if (tid < n) mem[tid] = cs[cur][tid];
    if (tid == 0) a.member_count[(size_t)bh * nblk + j] = n;
    const float fm = nm;
    const int fp = npos, fs = nsrc;
    if (tid < nt) {
      tm[tid] = score_key(fm);
      tp[tid] = fp;
    }
    if (j + 1 < nblk && tid < min(min(a.block, a.L - (j + 1) * a.block), a.w)) {
      const size_t o = tbase + (size_t)(j + 1) * a.w + tid;
      nm = a.top_m[o];
      npos = a.top_pos[o];
      nsrc = a.top_src[o];
    }
    __syncthreads();
    const int nx = cur ^ 1;
    if (tid < n) {  // cache entry: block-top entries strictly ahead of it
      const float mx = score_key(cm[cur][tid]);
      const int px = cp[cur][tid];
      int lo = 0, hi = nt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const bool ahead = rec ? tp[mid] > px : (tm[mid] > mx || (tm[mid] == mx && tp[mid] < px));
        if (ahead) lo = mid + 1;
        else hi = mid;
      }
      const int r = tid + lo;
      if (r < a.w) {
        cm[nx][r] = cm[cur][tid];
        cp[nx][r] = px;
        cs[nx][r] = cs[cur][tid];
      }
    }
    if (tid < nt) {  // block-top entry: cache entries ahead of it or tied with it
      const float mx = tm[tid];
      const int px = fp;
      int lo = 0, hi = n;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const float cmid = score_key(cm[cur][mid]);
        const int pmid = cp[cur][mid];
        const bool ahead = rec ? pmid >= px : (cmid > mx || (cmid == mx && pmid <= px));
        if (ahead) lo = mid + 1;
        else hi = mid;
      }
      const int r = tid + lo;
      if (r < a.w) {
        cm[nx][r] = fm;
        cp[nx][r] = fp;
        cs[nx][r] = fs;
      }
    }
    n = min(n + nt, a.w);
    cur = nx;
    __syncthreads();
  }
  if (tid < n) {
    a.final_src[(size_t)bh * a.w + tid] = cs[cur][tid];
    a.final_m[(size_t)bh * a.w + tid] = cm[cur][tid];
    a.final_pos[(size_t)bh * a.w + tid] = cp[cur][tid];
  }
  if (tid == 0) a.final_count[bh] = n;
}

// Read: 64 queries per workgroup against 32-key tiles on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32: lane l holds A(m0 + l % 16, k) and B(k, n0 + l % 16);
// the block's element (4 (l / 16) + i, l % 16) is accumulator i). Wavefront w
// owns queries 16 w .. 16 w + 15: its logits for a tile are two 16 x 16 blocks,
// the online softmax runs on them in registers (a row's 16 columns sit in 16
// lanes), the weights go through LDS into operand order, and the outputs are
// eight 16 x 16 blocks that stay in registers. Each lane keeps its query
// operands in registers and the keys sit in LDS, both RMS-normalised (the
// queries also times 1/sqrt(d_k)). In step s of a contraction pass of length
// PL, lane group l / 16 takes k = (PL / 4)(l / 16) + s; with row strides of 1
// mod 32 words the key reads are conflict-free. The next key tile is fetched
// into registers while the current one is used.
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

constexpr int KHP = MAXD + 8;  // fp16 pitch of the key tiles [key][d]
constexpr int VTP = KT + 8;    // fp16 pitch of the value tiles, transposed [d][key]
constexpr int PHP = KT + 8;    // fp16 pitch of the weight tiles [query][key]
constexpr size_t kReadLds = (size_t)(2 * KT * KHP + 2 * MAXD * VTP + 2 * QT * PHP) * 2 + KT * 4;

// Four consecutive elements (the index a multiple of 4, rows 16-byte aligned
// for float32 and 8-byte aligned for bf16).
__device__ __forceinline__ float4 ld4(const float* p, size_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
__device__ __forceinline__ float4 ld4(const uint16_t* p, size_t i) {
  const uint2 u = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ bool aligned_rows(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

// x as two fp16 parts: x_h = fp16(x), x_l = fp16(x - x_h). The matrix cores
// take subnormal fp16 inputs as zero, so callers scale x by a power of two
// that keeps x_l normal wherever it matters.
struct Split16 {
  _Float16 h, l;
};
// The high part is converted once and held opaque, so that the operand and
// the residual use the same bits: the compiler would otherwise convert x again
// where it builds the operand, and its two conversions can round a tie (x
// halfway between two fp16 values) in different directions.
__device__ __forceinline__ Split16 split16(float x) {
  uint32_t hb = __builtin_bit_cast(uint16_t, (_Float16)x);
  asm volatile("" : "+v"(hb));
  const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)hb);
  return {h, (_Float16)(x - (float)h)};
}
// c + a b, a and b each given as two fp16 parts (the product of the two low
// parts, below 2^-22 of the product, is left out). The matrix cores align the
// products of one instruction to the largest of them and of the incoming
// accumulator, keeping float32 precision only relative to that (measured: a
// 2^20 accumulator costs products near 2^5 their low bits), so the high and
// the low products each start from zero and meet c in vector adds.
__device__ __forceinline__ floatx4 mfma_split(half8 ah, half8 al, half8 bh, half8 bl, floatx4 c) {
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  const floatx4 hh = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, z, 0, 0, 0);
  floatx4 lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, z, 0, 0, 0);
  lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, lo, 0, 0, 0);
  return c + (hh + lo);
}
// 2^e as a float, -126 <= e <= 127
__device__ __forceinline__ float pow2f(int e) { return __int_as_float((127 + e) << 23); }

// Read: 64 queries per workgroup against 32-key tiles on the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16: lane l holds A(m0 + l % 16, k0 + 8 (l / 16) .. + 8)
// and B(k0 + 8 (l / 16) .. + 8, n0 + l % 16); the block's element
// (4 (l / 16) + i, l % 16) is accumulator i). Every float32 operand goes in as
// two fp16 parts and each product as three (high x high, high x low, low x
// high): about 22 significant bits, float32-level results at a fifth of the
// float32 products' matrix-core time. The parts are formed from exact
// power-of-two multiples that keep the high parts below 2^15 and the low parts
// normal (the matrix cores take fp16 subnormals as zero): RMS-normalised
// queries and keys (no component above sqrt(d_k)) times 2^8 each; weights
// (at most 1) times 2^14; the values of key j times 2^-E_j, E_j the exponent
// that brings the row's largest finite |v| into [2^14, 2^15), with the weight
// of key j for query i times a further 2^(E_j - F_i), F_i the largest E_j
// among the keys query i has seen (its accumulated outputs are rescaled
// with the online softmax when F_i grows). The logits and outputs are scaled
// back. Wavefront w owns queries 16 w .. 16 w + 15: its logits for a
// tile are two 16 x 16 blocks, the online softmax runs on them in registers (a
// row's 16 columns sit in 16 lanes), its weights go through its own rows of
// LDS into operand order, and its outputs are eight 16 x 16 blocks in
// registers. Values are staged transposed ([d][key]) so that every operand is
// one 16-byte read. The next key tile is fetched into registers while the
// current one is used.
//
// Three workgroups per CU (as many as its 47 KB of LDS allows).
template <typename Tin>
__global__ __launch_bounds__(NT, 3) void read_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) _Float16 ldsh[];
  _Float16* sKh = ldsh;                   // [KT][KHP] keys, high parts
  _Float16* sKl = sKh + KT * KHP;         //           low parts
  _Float16* sVh = sKl + KT * KHP;         // [MAXD][VTP] values transposed, high parts
  _Float16* sVl = sVh + MAXD * VTP;       //             low parts
  _Float16* sPh = sVl + MAXD * VTP;       // [QT][PHP] weights, high parts
  _Float16* sPl = sPh + QT * PHP;         //           low parts
  int* sEk = reinterpret_cast<int*>(sPl + QT * PHP);  // [KT] value exponents E_j of the tile's keys
  const int bh = blockIdx.x, j = blockIdx.y, qt = blockIdx.z, tid = threadIdx.x;
  const int dk = a.dk, dv = a.dv;
  const int nblk = (a.L + a.block - 1) / a.block;
  const int j0 = j * a.block, nb = min(a.block, a.L - j0);
  const int q0 = qt * QT;  // first query, relative to the block
  if (q0 >= nb) return;
  const int nq = min(QT, nb - q0);
  const Tin* qh = static_cast<const Tin*>(a.q) + (size_t)bh * a.L * dk;
  const Tin* kh = static_cast<const Tin*>(a.k) + (size_t)bh * a.L * dk;
  const Tin* vh = static_cast<const Tin*>(a.v) + (size_t)bh * a.L * dv;
  const float* ck = a.cache_k + (size_t)bh * a.w * dk;
  const float* cv = a.cache_v + (size_t)bh * a.w * dv;
  const int* mem = a.members + ((size_t)bh * nblk + j) * a.w;
  const int ncache = a.member_count[(size_t)bh * nblk + j];
  // keys: the cache members, then the block's tokens up to the last query here
  const int nkeys = ncache + q0 + nq;
  const int w = tid >> 6, l = tid & 63, r = l & 15, q = l >> 4;

  // This lane's query operands: row 16 w + r, columns 32 s + 8 q .. + 8,
  // RMS-normalised (the row's four lane groups meet by shuffles), in two parts.
  half8 qoh[4], qol[4];
  {
    const int row = 16 * w + r;
    float x[4][8];
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = 32 * s + 8 * q + u;
        x[s][u] = (row < nq && c < dk) ? Elem<Tin>::load(qh, (size_t)(j0 + q0 + row) * dk + c) : 0.f;
        ss = fmaf(x[s][u], x[s][u], ss);
      }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float sc = 256.f / sqrtf(ss / dk + a.rms_eps);  // times 2^8
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const Split16 t = split16(x[s][u] * sc);
        qoh[s][u] = t.h;
        qol[s][u] = t.l;
      }
  }
  const float lscale = (1.f / 65536.f) / sqrtf((float)dk);  // logit scale, less the 2^16
  // key tiles: 8 lanes per key; lane kp takes columns 32 g + 4 kp + v (g, v <
  // 4), four consecutive ones per load. The source of the tile after next is
  // looked up while the next tile's rows are in flight.
  const int kr = tid >> 3, kp = tid & 7;
  auto src_of = [&](int e) { return e < nkeys ? (e < ncache ? mem[e] : j0 + e - ncache) : 0; };
  const bool vec = ((dk | dv) & 3) == 0 && aligned_rows(a.k) && aligned_rows(a.v) &&
                   aligned_rows(a.cache_k) && aligned_rows(a.cache_v);
  float kx[MAXD / 8], vx[MAXD / 8];
  auto fetch = [&](int e, int src) {
    const bool ok = e < nkeys;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 32 * g + 4 * kp;
      float4 xk = make_float4(0.f, 0.f, 0.f, 0.f), xv = xk;
      if (vec) {
        if (ok && c < dk)
          xk = src >= 0 ? ld4(kh, (size_t)src * dk + c) : ld4(ck, (size_t)(-1 - src) * dk + c);
        if (ok && c < dv)
          xv = src >= 0 ? ld4(vh, (size_t)src * dv + c) : ld4(cv, (size_t)(-1 - src) * dv + c);
      } else {
        float tk[4], tv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int cc = c + v;
          tk[v] = (ok && cc < dk) ? (src >= 0 ? Elem<Tin>::load(kh, (size_t)src * dk + cc)
                                               : ck[(size_t)(-1 - src) * dk + cc])
                                   : 0.f;
          tv[v] = (ok && cc < dv) ? (src >= 0 ? Elem<Tin>::load(vh, (size_t)src * dv + cc)
                                               : cv[(size_t)(-1 - src) * dv + cc])
                                   : 0.f;
        }
        xk = make_float4(tk[0], tk[1], tk[2], tk[3]);
        xv = make_float4(tv[0], tv[1], tv[2], tv[3]);
      }
      kx[4 * g] = xk.x;
      kx[4 * g + 1] = xk.y;
      kx[4 * g + 2] = xk.z;
      kx[4 * g + 3] = xk.w;
      vx[4 * g] = xv.x;
      vx[4 * g + 1] = xv.y;
      vx[4 * g + 2] = xv.z;
      vx[4 * g + 3] = xv.w;
    }
  };
  float M[4], Z[4];
  floatx4 acc[MAXD / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    M[i] = a.sink_logit ? a.sink_logit[bh % a.H] : -INFINITY;
    Z[i] = a.sink_logit ? 1.f : 0.f;
  }
#pragma unroll
  for (int cb = 0; cb < MAXD / 16; ++cb) acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  constexpr int kNoE = -1000;  // F_i before the first visible key
  int F[4] = {kNoE, kNoE, kNoE, kNoE};
  fetch(kr, src_of(kr));
  int src_next = src_of(KT + kr);
  for (int e0 = 0; e0 < nkeys; e0 += KT) {
    __syncthreads();
    {  // stage: keys RMS-normalised, values times 2^-E_j, both in two parts
      float ss = 0.f;
      uint32_t mv = 0;  // bits of the row's largest finite |v|
#pragma unroll
      for (int u = 0; u < MAXD / 8; ++u) {
        ss = fmaf(kx[u], kx[u], ss);
        const uint32_t b = __float_as_uint(fabsf(vx[u]));
        mv = b < 0x7f800000u ? max(mv, b) : mv;
      }
      ss += __shfl_xor(ss, 1, 8);
      ss += __shfl_xor(ss, 2, 8);
      ss += __shfl_xor(ss, 4, 8);
      mv = max(mv, (uint32_t)__shfl_xor((int)mv, 1, 8));
      mv = max(mv, (uint32_t)__shfl_xor((int)mv, 2, 8));
      mv = max(mv, (uint32_t)__shfl_xor((int)mv, 4, 8));
      const int ej = max((int)(mv >> 23) - 127 - 14, -100);  // E_j
      if (kp == 0) sEk[kr] = ej;
      const float sc = 256.f / sqrtf(ss / dk + a.rms_eps);  // times 2^8
      const float vsc = pow2f(-ej);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * g + 4 * kp;
        half4 hk, lk;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const Split16 tk = split16(kx[4 * g + v] * sc);
          hk[v] = tk.h;
          lk[v] = tk.l;
          const Split16 tv = split16(vx[4 * g + v] * vsc);
          sVh[(c + v) * VTP + kr] = tv.h;
          sVl[(c + v) * VTP + kr] = tv.l;
        }
        *reinterpret_cast<half4*>(sKh + kr * KHP + c) = hk;
        *reinterpret_cast<half4*>(sKl + kr * KHP + c) = lk;
      }
    }
    if (e0 + KT < nkeys) {
      fetch(e0 + KT + kr, src_next);
      src_next = src_of(e0 + 2 * KT + kr);
    }
    __syncthreads();
    floatx4 lg[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (32 * s >= dk) break;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int off = (16 * b + r) * KHP + 32 * s + 8 * q;
        lg[b] = mfma_split(qoh[s], qol[s], *reinterpret_cast<const half8*>(sKh + off),
                           *reinterpret_cast<const half8*>(sKl + off), lg[b]);
      }
    }
    const int ek[2] = {sEk[r], sEk[16 + r]};  // E_j of this lane's two keys
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qi = 16 * w + 4 * q + i;  // query within the tile
      const int qtok = q0 + qi;           // relative to the block
      float lv[2];
      float tmax = -INFINITY;
      int emax = kNoE;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int e = e0 + 16 * b + r;
        // cache members are always visible; block tokens up to the query itself
        const bool vis = qi < nq && e < nkeys && (e < ncache || e - ncache <= qtok);
        lv[b] = vis ? lg[b][i] * lscale : -INFINITY;
        tmax = fmaxf(tmax, lv[b]);
        emax = vis ? max(emax, ek[b]) : emax;
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 4, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 8, 16));
      emax = max(emax, __shfl_xor(emax, 1, 16));
      emax = max(emax, __shfl_xor(emax, 2, 16));
      emax = max(emax, __shfl_xor(emax, 4, 16));
      emax = max(emax, __shfl_xor(emax, 8, 16));
      const float Mn = fmaxf(M[i], tmax);
      const int Fn = max(F[i], emax);
      // rows with nothing visible yet keep M = -inf; their weights stay 0;
      // the outputs so far move to the scale of F_i's new value
      const float ms = Mn == -INFINITY ? 1.f : __expf(M[i] - Mn);  // the softmax's rescale
      const float scale = ms * pow2f(max(F[i] - Fn, -126));          // and the outputs'
      float ps = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float p = lv[b] == -INFINITY ? 0.f : __expf(lv[b] - Mn);
        // (a key not visible to this query may have E_j above F_i: its weight
        // is 0 and its factor is held finite)
        const Split16 tp = split16(p * pow2f(min(max(14 + ek[b] - Fn, -126), 14)));
        sPh[qi * PHP + 16 * b + r] = tp.h;
        sPl[qi * PHP + 16 * b + r] = tp.l;
        ps += p;
      }
      ps += __shfl_xor(ps, 1, 16);
      ps += __shfl_xor(ps, 2, 16);
      ps += __shfl_xor(ps, 4, 16);
      ps += __shfl_xor(ps, 8, 16);
      Z[i] = fmaf(Z[i], ms, ps);
      M[i] = Mn;
      F[i] = Fn;
#pragma unroll
      for (int cb = 0; cb < MAXD / 16; ++cb) acc[cb][i] *= scale;
    }
    // the weight rows just written are this wavefront's own: in-order LDS
    // access within the wavefront needs no barrier
    const int poff = (16 * w + r) * PHP + 8 * q;
    const half8 ph = *reinterpret_cast<const half8*>(sPh + poff);
    const half8 pl = *reinterpret_cast<const half8*>(sPl + poff);
#pragma unroll
    for (int cb = 0; cb < MAXD / 16; ++cb) {
      if (16 * cb >= dv) break;
      const int voff = (16 * cb + r) * VTP + 8 * q;
      acc[cb] = mfma_split(ph, pl, *reinterpret_cast<const half8*>(sVh + voff),
                           *reinterpret_cast<const half8*>(sVl + voff), acc[cb]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qi = 16 * w + 4 * q + i;
    if (qi < nq) {
      float* o = a.o_cache + ((size_t)bh * a.L + j0 + q0 + qi) * dv;
      const float inv = pow2f(min(max(F[i] - 14, -126), 127)) / Z[i];
#pragma unroll
      for (int cb = 0; cb < MAXD / 16; ++cb)
        if (16 * cb + r < dv) o[16 * cb + r] = acc[cb][i] * inv;
    }
  }
}

// Commit, in two launches so that every (head, member) row has its own
// workgroup: gather the final members' keys and values (from the prompt or an
// old slot) into the staging rows, then write the cache in rank order. The
// gather finishes before any slot is overwritten.
template <typename Tin>
__global__ __launch_bounds__(64) void commit_gather_kernel(PrefillArgs a) {
  const int bh = blockIdx.x, e = blockIdx.y, tid = threadIdx.x;
  if (e >= a.final_count[bh]) return;
  const int src = a.final_src[(size_t)bh * a.w + e];
  const int row = a.dk + a.dv;
  float* st = a.stage + ((size_t)bh * a.w + e) * row;
  const Tin* kh = static_cast<const Tin*>(a.k) + (size_t)bh * a.L * a.dk;
  const Tin* vh = static_cast<const Tin*>(a.v) + (size_t)bh * a.L * a.dv;
  const float* ck = a.cache_k + (size_t)bh * a.w * a.dk;
  const float* cv = a.cache_v + (size_t)bh * a.w * a.dv;
  for (int c = tid; c < row; c += 64) {
    float x;
    if (c < a.dk)
      x = src >= 0 ? Elem<Tin>::load(kh, (size_t)src * a.dk + c) : ck[(size_t)(-1 - src) * a.dk + c];
    else
      x = src >= 0 ? Elem<Tin>::load(vh, (size_t)src * a.dv + c - a.dk)
                   : cv[(size_t)(-1 - src) * a.dv + c - a.dk];
    st[c] = x;
  }
}

__global__ __launch_bounds__(64) void commit_scatter_kernel(PrefillArgs a) {
  const int bh = blockIdx.x, e = blockIdx.y, tid = threadIdx.x;
  const int n = a.final_count[bh];
  if (e == 0 && tid == 0) a.cache_count[bh] = n;
  if (e >= n) return;
  const int row = a.dk + a.dv;
  const float* st = a.stage + ((size_t)bh * a.w + e) * row;
  for (int c = tid; c < row; c += 64) {
    if (c < a.dk) a.cache_k[((size_t)bh * a.w + e) * a.dk + c] = st[c];
    else a.cache_v[((size_t)bh * a.w + e) * a.dv + c - a.dk] = st[c];
  }
  if (tid == 0) {
    a.cache_m[(size_t)bh * a.w + e] = a.final_m[(size_t)bh * a.w + e];
    a.cache_pos[(size_t)bh * a.w + e] = a.final_pos[(size_t)bh * a.w + e];
  }
}

template <typename Tin>
hipError_t prefill_typed(const PrefillArgs& a, hipStream_t s) {
  const int nblk = (a.L + a.block - 1) / a.block;
  if (a.w > kMaxW || a.block > kMaxBlock || a.w > NT) return hipErrorInvalidValue;
  KDN_LAUNCH(block_top_kernel, dim3(a.BH, nblk), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KDN_LAUNCH(merge_kernel, dim3(a.BH), dim3(NT), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t read_lds = kReadLds;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(read_kernel<Tin>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)read_lds);
  if (e != hipSuccess) return e;
  KDN_LAUNCH(read_kernel<Tin>, dim3(a.BH, nblk, (a.block + QT - 1) / QT), dim3(NT),
                     read_lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  KDN_LAUNCH(commit_gather_kernel<Tin>, dim3(a.BH, a.w), dim3(64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  KDN_LAUNCH(commit_scatter_kernel, dim3(a.BH, a.w), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int BH, int L, int dk, int dv, int w, int block) {
  const size_t nblk = ((size_t)L + block - 1) / block;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return 4 * up((size_t)BH * nblk * w * 4) + up((size_t)BH * nblk * 4) +
         3 * up((size_t)BH * w * 4) + up((size_t)BH * 4) + up((size_t)BH * w * (dk + dv) * 4);
}

void prefill_bind_workspace(PrefillArgs& a, void* ws) {
  const size_t nblk = ((size_t)a.L + a.block - 1) / a.block;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* p = static_cast<char*>(ws);
  a.members = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * nblk * a.w * 4);
  a.member_count = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * nblk * 4);
  a.final_src = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * a.w * 4);
  a.final_m = reinterpret_cast<float*>(p);
  p += up((size_t)a.BH * a.w * 4);
  a.final_pos = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * a.w * 4);
  a.final_count = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * 4);
  a.stage = reinterpret_cast<float*>(p);
  p += up((size_t)a.BH * a.w * (a.dk + a.dv) * 4);
  a.top_m = reinterpret_cast<float*>(p);
  p += up((size_t)a.BH * nblk * a.w * 4);
  a.top_pos = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * nblk * a.w * 4);
  a.top_src = reinterpret_cast<int*>(p);
}

hipError_t launch_prefill(const PrefillArgs& a, bool in_bf16, hipStream_t s) {
  return in_bf16 ? prefill_typed<uint16_t>(a, s) : prefill_typed<float>(a, s);
}

}  // namespace kdn
