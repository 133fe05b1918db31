// scan_bwd.hip -- gradients of the delta-write scan (reverse mode).
//
// Forward ("A Hippocampus for Linear Attention", sec. 3.3 eq. (5), sec. 3.5):
//   S_t = M_t S_{t-1} + beta_t k_t v_t^T,  M_t = alpha_t I - c_t beta_t k_t k_t^T,
//   o_t = S_t^T q_t,  e_t = v_t - c_t S_{t-1}^T k_t,
//   c_t = alpha_t (gated residual), 1 (plain), 0 (no erase).
// The pages give no backward pass; its adjoint, with G_t = dL/dS_t:
//   G_t += q_t do_t^T;  dq_t = S_t do_t;  y_t = G_t^T k_t;  dv_t = beta_t y_t;
//   dbeta_t = y_t . e_t;  dk_t = beta_t G_t e_t - c_t beta_t S_{t-1} y_t;
//   dalpha_t = <G_t, S_{t-1}> - [gated] beta_t y_t . (S_{t-1}^T k_t);
//   G_{t-1} = alpha_t G_t - c_t beta_t k_t y_t^T;  dS_0 = G_0.
//
// Every value column is independent, so one workgroup takes one head and 32
// value columns: thread (c, rg) owns column c and rows rg, rg + 8, ... of S
// and G in registers. A first forward pass stores the state at every 64-token
// chunk start; the reverse pass recomputes each chunk's states (kept in a
// per-workgroup history buffer) and walks it backwards. Sums over rows meet in
// LDS (one barrier per forward token, two per backward token); the per-tile
// partial sums of dq, dk, dalpha, dbeta are added over tiles in a fixed order
// by a second kernel. Float32 throughout.
#include "kdn_internal.h"

namespace kdn {
namespace {

constexpr int NT = 256;
constexpr int CW = 32;   // value columns per workgroup
constexpr int CH = 64;   // tokens per recomputation chunk
constexpr int RPT = 16;  // rows per thread (d_k <= 128)

struct BwdLds {
  float k[CH][128];
  float q[CH][128];
  float v[CH][CW];
  float dout[CH][CW];
  float a[CH], b[CH];
  float red[2][8][CW];       // column sums over row groups
  float red2[2][8][CW];
  float red3[2][8][CW];
  float row[2][128][CW + 1];   // row sums over columns (dk)
  float row2[2][128][CW + 1];  // (dq)
};

__global__ __launch_bounds__(NT) void scan_bwd_kernel(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  BwdLds& L_ = *reinterpret_cast<BwdLds*>(lds_raw);
  const int bh = blockIdx.x, tile = blockIdx.y, tid = threadIdx.x;
  const int c = tid & 31, rg = tid >> 5;
  const int dk = a.dk, dv = a.dv, L = a.L;
  const int j0 = tile * CW, col = j0 + c;
  const bool cok = col < dv;
  const int nchunks = (L + CH - 1) / CH;
  const size_t tile_id = (size_t)bh * gridDim.y + tile;
  float* ckpt = a.ckpt + tile_id * (size_t)nchunks * dk * CW;
  float* hist = a.hist + tile_id * (size_t)(CH + 1) * dk * CW;
  const size_t tok0 = (size_t)bh * L;

  float S[RPT], G[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + 8 * i;
    const bool ok = r < dk && cok;
    S[i] = ok && a.state_in ? a.state_in[((size_t)bh * dk + r) * dv + col] : 0.f;
    G[i] = ok && a.dstate_out ? a.dstate_out[((size_t)bh * dk + r) * dv + col] : 0.f;
  }

  // chunk inputs into LDS (zero past the end and past d_v)
  auto load_chunk = [&](int ck, bool with_q) {
    const int t0 = ck * CH, n = min(CH, L - t0);
    __syncthreads();
    for (int idx = tid; idx < CH * dk; idx += NT) {
      const int s = idx / dk, r = idx - s * dk;
      const bool ok = s < n;
      L_.k[s][r] = ok ? a.k[(tok0 + t0 + s) * dk + r] : 0.f;
      if (with_q) L_.q[s][r] = ok ? a.q[(tok0 + t0 + s) * dk + r] : 0.f;
    }
    for (int idx = tid; idx < CH * CW; idx += NT) {
      const int s = idx / CW, cc = idx - s * CW;
      const bool ok = s < n && j0 + cc < dv;
      L_.v[s][cc] = ok ? a.v[(tok0 + t0 + s) * dv + j0 + cc] : 0.f;
      if (with_q) L_.dout[s][cc] = ok ? a.d_o[(tok0 + t0 + s) * dv + j0 + cc] : 0.f;
    }
    if (tid < CH) {
      const bool ok = tid < n;
      L_.a[tid] = ok ? (a.alpha ? a.alpha[tok0 + t0 + tid] : 1.f) : 1.f;
      L_.b[tid] = ok ? a.beta[tok0 + t0 + tid] : 0.f;
    }
    __syncthreads();
  };
  auto coef = [&](float al) { return a.resid == 0 ? al : (a.resid == 1 ? 1.f : 0.f); };
  // one forward token: S <- alpha S + beta k e^T, e = v - c S^T k
  auto forward = [&](int s, int par) {
    float pk = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + 8 * i;
      if (r < dk) pk = fmaf(S[i], L_.k[s][r], pk);
    }
    L_.red[par][rg][c] = pk;
    __syncthreads();
    float p = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) p += L_.red[par][g][c];
    const float al = L_.a[s], be = L_.b[s];
    const float e = L_.v[s][c] - coef(al) * p;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + 8 * i;
      if (r < dk) S[i] = fmaf(al, S[i], be * L_.k[s][r] * e);
    }
  };
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + 8 * i;
      if (r < dk) dst[r * CW + c] = S[i];
    }
  };

  // pass 1: states at the chunk starts
  for (int ck = 0; ck < nchunks; ++ck) {
    store_state(ckpt + (size_t)ck * dk * CW);
    load_chunk(ck, false);
    const int n = min(CH, L - ck * CH);
    for (int s = 0; s < n; ++s) forward(s, s & 1);
  }

  // pass 2: chunks in reverse
  for (int ck = nchunks - 1; ck >= 0; --ck) {
    const int t0 = ck * CH, n = min(CH, L - t0);
    load_chunk(ck, true);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + 8 * i;
      S[i] = r < dk ? ckpt[((size_t)ck * dk + r) * CW + c] : 0.f;
    }
    store_state(hist);
    for (int s = 0; s < n; ++s) {
      forward(s, s & 1);
      store_state(hist + (size_t)(s + 1) * dk * CW);
    }
    __threadfence_block();
    __syncthreads();
    // S now holds S_{t0+n-1}, the state after the chunk's last token
    for (int s = n - 1; s >= 0; --s) {
      const int par = s & 1;
      const size_t t = tok0 + t0 + s;
      const float al = L_.a[s], be = L_.b[s], cf = coef(al);
      const float dout = L_.dout[s][c];
      float Sp[RPT];
      float yp = 0.f, pp = 0.f, gs = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + 8 * i;
        Sp[i] = r < dk ? hist[((size_t)s * dk + r) * CW + c] : 0.f;
        if (r < dk) {
          G[i] = fmaf(L_.q[s][r], dout, G[i]);
          yp = fmaf(G[i], L_.k[s][r], yp);
          pp = fmaf(Sp[i], L_.k[s][r], pp);
          gs = fmaf(G[i], Sp[i], gs);
          L_.row2[par][r][c] = S[i] * dout;  // dq: S_t do_t
        }
      }
      L_.red[par][rg][c] = yp;
      L_.red2[par][rg][c] = pp;
      L_.red3[par][rg][c] = gs;
      __syncthreads();
      float y = 0.f, p = 0.f, g = 0.f;
#pragma unroll
      for (int gg = 0; gg < 8; ++gg) {
        y += L_.red[par][gg][c];
        p += L_.red2[par][gg][c];
        g += L_.red3[par][gg][c];
      }
      const float e = L_.v[s][c] - cf * p;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + 8 * i;
        if (r < dk) L_.row[par][r][c] = be * (G[i] * e - cf * Sp[i] * y);
      }
      if (rg == 0) {
        if (cok) a.dv_out[t * dv + col] = be * y;
        // over the 32 columns of this tile (one half-wavefront)
        float da = g - (a.resid == 0 ? be * y * p : 0.f), db = y * e;
        for (int off = 16; off > 0; off >>= 1) {
          da += __shfl_xor(da, off, 32);
          db += __shfl_xor(db, off, 32);
        }
        if (c == 0) {
          a.da_part[tile_id * L + t0 + s] = da;
          a.db_part[tile_id * L + t0 + s] = db;
        }
      }
      __syncthreads();
      if (tid < dk) {
        float sk = 0.f, sq = 0.f;
        for (int cc = 0; cc < CW; ++cc) {
          sk += L_.row[par][tid][cc];
          sq += L_.row2[par][tid][cc];
        }
        a.dk_part[(tile_id * L + t0 + s) * dk + tid] = sk;
        a.dq_part[(tile_id * L + t0 + s) * dk + tid] = sq;
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + 8 * i;
        if (r < dk) {
          G[i] = fmaf(-cf * be * L_.k[s][r], y, al * G[i]);
          S[i] = Sp[i];
        }
      }
    }
  }
  if (a.dstate_in) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + 8 * i;
      if (r < dk && cok) a.dstate_in[((size_t)bh * dk + r) * dv + col] = G[i];
    }
  }
}

// Sum the per-tile partials in tile order.
__global__ void bwd_reduce_kernel(BwdArgs a, int ntiles) {
  const size_t n = (size_t)a.BH * a.L;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n * a.dk;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = i / ((size_t)a.L * a.dk), rem = i - bh * a.L * a.dk;
    float sq = 0.f, sk = 0.f;
    for (int tl = 0; tl < ntiles; ++tl) {
      const size_t p = ((bh * ntiles + tl) * a.L) * a.dk + rem;
      sq += a.dq_part[p];
      sk += a.dk_part[p];
    }
    a.dq[i] = sq;
    a.dk_out[i] = sk;
  }
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = i / a.L, t = i - bh * a.L;
    float da = 0.f, db = 0.f;
    for (int tl = 0; tl < ntiles; ++tl) {
      da += a.da_part[(bh * ntiles + tl) * a.L + t];
      db += a.db_part[(bh * ntiles + tl) * a.L + t];
    }
    if (a.dalpha) a.dalpha[i] = da;
    a.dbeta[i] = db;
  }
}

}  // namespace

size_t scan_bwd_workspace_bytes(int BH, int L, int dk, int dv) {
  const size_t ntiles = (dv + CW - 1) / CW, nchunks = ((size_t)L + CH - 1) / CH;
  const size_t tiles = (size_t)BH * ntiles;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up(tiles * nchunks * dk * CW * 4) + up(tiles * (CH + 1) * dk * CW * 4) +
         2 * up(tiles * L * dk * 4) + 2 * up(tiles * L * 4);
}

hipError_t launch_scan_bwd(BwdArgs a, void* ws, hipStream_t s) {
  const int ntiles = (a.dv + CW - 1) / CW, nchunks = (a.L + CH - 1) / CH;
  const size_t tiles = (size_t)a.BH * ntiles;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* p = static_cast<char*>(ws);
  a.ckpt = reinterpret_cast<float*>(p);
  p += up(tiles * nchunks * a.dk * CW * 4);
  a.hist = reinterpret_cast<float*>(p);
  p += up(tiles * (CH + 1) * a.dk * CW * 4);
  a.dq_part = reinterpret_cast<float*>(p);
  p += up(tiles * a.L * a.dk * 4);
  a.dk_part = reinterpret_cast<float*>(p);
  p += up(tiles * a.L * a.dk * 4);
  a.da_part = reinterpret_cast<float*>(p);
  p += up(tiles * a.L * 4);
  a.db_part = reinterpret_cast<float*>(p);
  const size_t lds = sizeof(BwdLds);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(scan_bwd_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_bwd_kernel, dim3(a.BH, ntiles), dim3(NT), lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(1024), dim3(256), 0, s, a, ntiles);
  return hipGetLastError();
}

}  // namespace kdn
