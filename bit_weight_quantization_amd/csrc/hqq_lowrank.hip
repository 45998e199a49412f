// hqq_lowrank.hip -- gfx950 kernels of the data-free low-rank compensation of the
// quantization error: the plain SVD compensation described on the EoRA page (section 1):
// Delta W = W - W_hat = U Sigma V^T, LoRA factors B = U_r Sigma_r, A = V_r^T, with W_hat
// = s (W_q - z) the inverse quantizer of section 2 of "Half-Quadratic Quantization of
// Large Machine Learning Models" applied to the stored codes.
//
// The truncated SVD is computed by randomized subspace iteration: Y = Delta W Omega for
// a caller-supplied Gaussian test matrix Omega (n x l, l = r + oversampling), q power
// steps Y <- Delta W basis(Delta W^T basis(Y)), Q = orth(Y), then the SVD of the small
// B_m = Q^T Delta W through the eigendecomposition of B_m B_m^T.  The heavy work is the
// products with Delta W, which is materialized once as binary16 in both layouts so every
// product is a plain matrix-core GEMM with fp32 accumulation.  Bases come from Cholesky
// QR of the l x l Gram matrix in fp64 (Q = Y R^-1, with nearly dependent columns
// dropped): one pass inside the power steps, where only the spanned subspace matters,
// two for the final orthonormal Q.  The SVD of B_m comes from the eigendecomposition of
// B_m B_m^T (Householder tridiagonalization, bisection, inverse iteration) in fp64 in one
// block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "hqq_internal.h"
#include "hqq_lowrank.h"

namespace hqq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float h2f(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f2h(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---------------------------------------------------------------- residual --

constexpr int kTile = 64;

// One 64 x 64 tile of Delta W per block: thread t computes row t / 4, 16 consecutive
// columns (inside one group), w - (s q - s z) in fp32 (s z exact, two roundings), stores
// binary16 to Delta W and, through LDS, to its transpose.
template <int NB>
__global__ __launch_bounds__(kBlock) void residual_kernel(const uint16_t* __restrict__ W,
                                                          const uint8_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ s16,
                                                          const uint16_t* __restrict__ z16,
                                                          int64_t m, int64_t n, int gshift,
                                                          uint16_t* __restrict__ dW,
                                                          uint16_t* __restrict__ dWT) {
  __shared__ uint16_t tile[kTile][kTile + 2];
  const int t = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.y * kTile, k0 = (int64_t)blockIdx.x * kTile;
  const int ri = t >> 2, ck = (t & 3) * 16;
  const int64_t e = (i0 + ri) * n + k0 + ck;  // flat element index of the 16 weights
  const uint4* wp = reinterpret_cast<const uint4*>(W + e);
  const uint4 wa = wp[0], wb = wp[1];
  const uint32_t ww[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
  uint32_t cw[2] = {0u, 0u};  // the 16 codes: 2 NB bytes at byte e NB / 8
  const uint8_t* cp = packed + (e >> 3) * NB;
  if constexpr (NB == 2) {
    cw[0] = *reinterpret_cast<const uint32_t*>(cp);
  } else if constexpr (NB == 3) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(cp);
    cw[0] = (uint32_t)q[0] | ((uint32_t)q[1] << 16);
    cw[1] = q[2];
  } else if constexpr (NB == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(cp);
    cw[0] = v.x; cw[1] = v.y;
  }
  uint32_t cw8[4] = {0u, 0u, 0u, 0u};
  if constexpr (NB == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(cp);
    cw8[0] = v.x; cw8[1] = v.y; cw8[2] = v.z; cw8[3] = v.w;
  }
  const int64_t gi = e >> gshift;
  const float s = h2f(s16[gi]);
  const float sz = s * h2f(z16[gi]);
  uint32_t out[8];
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    uint32_t q0, q1;
    if constexpr (NB == 8) {
      q0 = (cw8[j >> 2] >> (8 * (j & 3))) & 255u;
      q1 = (cw8[(j + 1) >> 2] >> (8 * ((j + 1) & 3))) & 255u;
    } else {
      const int b0 = NB * j, b1 = NB * (j + 1);
      constexpr uint32_t mask = (1u << NB) - 1u;
      q0 = (b0 >> 5) == ((b0 + NB - 1) >> 5)
               ? (cw[b0 >> 5] >> (b0 & 31)) & mask
               : __builtin_amdgcn_alignbit(cw[1], cw[0], b0 & 31) & mask;
      q1 = (b1 >> 5) == ((b1 + NB - 1) >> 5)
               ? (cw[b1 >> 5] >> (b1 & 31)) & mask
               : __builtin_amdgcn_alignbit(cw[1], cw[0], b1 & 31) & mask;
    }
    const float r0 = h2f(ww[j >> 1] & 0xffffu) - __builtin_fmaf(s, (float)q0, -sz);
    const float r1 = h2f(ww[j >> 1] >> 16) - __builtin_fmaf(s, (float)q1, -sz);
    out[j >> 1] = f2h(r0) | (f2h(r1) << 16);
  }
  uint4* dp = reinterpret_cast<uint4*>(dW + e);
  dp[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dp[1] = make_uint4(out[4], out[5], out[6], out[7]);
  if (!dWT) return;  // block-uniform: no transposed copy wanted
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    tile[ri][ck + 2 * j] = (uint16_t)(out[j] & 0xffffu);
    tile[ri][ck + 2 * j + 1] = (uint16_t)(out[j] >> 16);
  }
  __syncthreads();
  const int rk = t >> 2, ci = (t & 3) * 16;  // transposed: row k0 + rk, columns i0 + ci ..
  uint32_t tw[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    tw[j] = (uint32_t)tile[ci + 2 * j][rk] | ((uint32_t)tile[ci + 2 * j + 1][rk] << 16);
  uint4* tp = reinterpret_cast<uint4*>(dWT + (k0 + rk) * m + i0 + ci);
  tp[0] = make_uint4(tw[0], tw[1], tw[2], tw[3]);
  tp[1] = make_uint4(tw[4], tw[5], tw[6], tw[7]);
}

// -------------------------------------------------------------- fp16 GEMM --

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsRow = kBK + 8;

// P[z][i][j] = sum over k in split z's slice of A[i][k] * B[j][k]: A is M x K and B is
// L x K binary16 (K contiguous), P fp32 (M x L per split).  128 x 128 tiles of four
// wavefronts (2 x 2 v_mfma_f32_32x32x16_f16 each), 64-wide K steps through double-buffered
// LDS with two steps of loads in flight.  M and K are multiples of 64; rows of B past L
// are zero.
__global__ __launch_bounds__(kBlock) void gemm16_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B,
                                                        int64_t M, int64_t K, int L,
                                                        int64_t kslice, float* __restrict__ P) {
  __shared__ __align__(16) _Float16 As[2][kBM][kLdsRow];
  __shared__ __align__(16) _Float16 Bs[2][kBN][kLdsRow];
  const int tid = threadIdx.x;
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  const int wm = wid >> 1, wn = wid & 1;
  const int64_t m0 = (int64_t)blockIdx.x * kBM;
  const int n0 = blockIdx.y * kBN;
  const int64_t kb = (int64_t)blockIdx.z * kslice;
  const int64_t ke = kb + kslice < K ? kb + kslice : K;
  // loads: 8 adjacent lanes take one row's 64 K values (128 bytes, 16 each); load i of a
  // thread covers rows lr + 32 i, so one wave's load reads 8 whole rows.  Rows past M or
  // L read row 0 and are stored as zeros.
  const int lr = tid >> 3, lg = tid & 7;
  const uint16_t* arow[4];
  const uint16_t* brow[4];
  bool a_ok[4], b_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lr + 32 * i;
    a_ok[i] = m0 + r < M;
    b_ok[i] = n0 + r < L;
    arow[i] = A + (a_ok[i] ? m0 + r : 0) * K + 8 * lg;
    brow[i] = B + (int64_t)(b_ok[i] ? n0 + r : 0) * K + 8 * lg;
  }
  // two register sets: while step s is multiplied out of LDS, step s + 1 is in flight in
  // one set and step s + 2 is issued into the other (the loop is unrolled by two so the
  // sets stay fixed registers); past the last step the loads repeat it and are unused
  // Each row block starts its slice at its own step (blockIdx.x mod the step count) and
  // wraps around, so that blocks running together read different 128-byte columns of
  // the rows rather than addresses one row stride apart.
  const int nst = kb < ke ? (int)((ke - kb) / kBK) : 0;
  const int rot = nst > 0 ? (int)(blockIdx.x % (unsigned)nst) : 0;
  auto kpos = [&](int st) {
    int q = (st < nst ? st : nst - 1) + rot;
    q = q >= nst ? q - nst : q;
    return kb + (int64_t)q * kBK;
  };
  // native 4 x 32-bit vectors: a select between two of them stays in registers
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4), may_alias));
  auto load_global = [&](u32x4 (&ra)[4], u32x4 (&rb)[4], int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(arow[i] + k0);
      rb[i] = *reinterpret_cast<const u32x4*>(brow[i] + k0);
    }
  };
  auto store_lds = [&](int buf, const u32x4 (&ra)[4], const u32x4 (&rb)[4]) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&As[buf][lr + 32 * i][8 * lg]) = a_ok[i] ? ra[i] : z;
      *reinterpret_cast<u32x4*>(&Bs[buf][lr + 32 * i][8 * lg]) = b_ok[i] ? rb[i] : z;
    }
  };
  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto mfma_step = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kk = ks * 16 + (lane >> 5) * 8;
      half8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(&As[buf][wm * 64 + i * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(&Bs[buf][wn * 64 + j * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  u32x4 a0[4], b0[4], a1[4], b1[4];
  if (nst > 0) {
    load_global(a0, b0, kpos(0));
    load_global(a1, b1, kpos(1));
    store_lds(0, a0, b0);
  }
  __syncthreads();
  // pairs of steps in one straight-line body (even steps in LDS buffer 0, odd in 1), so
  // each wait is for the older set only; an odd last step follows the loop
  int st = 0;
  // (the scheduling barriers keep each half's loads ahead of its products)
  for (; st + 1 < nst; st += 2) {
    load_global(a0, b0, kpos(st + 2));
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(0);
    store_lds(1, a1, b1);
    __syncthreads();
    load_global(a1, b1, kpos(st + 3));
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(1);
    store_lds(0, a0, b0);
    __syncthreads();
  }
  if (st < nst) mfma_step(0);
  float* out = P + (int64_t)blockIdx.z * M * L;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t mm = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (mm < M && n < L) out[mm * L + n] = acc[i][j][v];
      }
    }
  }
}

// out[e] = sum over splits s (in order) of P[s][e], e < count.
__global__ __launch_bounds__(kBlock) void split_sum_kernel(const float* __restrict__ P, int splits,
                                                           int64_t count, float* __restrict__ out) {
  for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < count;
       e += (int64_t)gridDim.x * kBlock) {
    float v = P[e];
    for (int s = 1; s < splits; ++s) v += P[(int64_t)s * count + e];
    out[e] = v;
  }
}

// ------------------------------------------------------------------- Gram --

// Partial Gram matrices: Gp[z][a][b] = sum over the rows i of split z (rows z * rs ..
// + rs) of X[i][a] X[i][b] for X (M x L fp32), for the 32 x 32 tiles on and above the
// diagonal only (block x: tile (A, B), A <= B, in row order; block y: split z); 64-row
// chunks of the two column slabs through LDS, fp32 sums per chunk added in fp64.
// Thread t: entry a0 + t % 32, b0 + 4 (t / 32) .. + 4.
__global__ __launch_bounds__(kBlock) void gram_kernel(const float* __restrict__ X, int64_t M, int L,
                                                      int64_t rs, double* __restrict__ Gp) {
  __shared__ float xa[64][33];
  __shared__ __align__(16) float xb[64][36];  // 16-byte rows: 4 values of a row in one read
  const int t = threadIdx.x;
  const int nt = L / 32;
  int A = 0, idx = blockIdx.x;
  while (idx >= nt - A) {
    idx -= nt - A;
    ++A;
  }
  const int a0 = A * 32, b0 = (A + idx) * 32;
  const int64_t r0 = (int64_t)blockIdx.y * rs;
  const int64_t r1 = r0 + rs < M ? r0 + rs : M;
  const int ta = t & 31, tb = (t >> 5) * 4;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  // a chunk: 64 rows x 32 columns of each slab, two 16-byte loads per slab and thread
  // (rows past r1 read row r1 - 1 and count as zeros); the next chunk is loaded during
  // this chunk's arithmetic, past the end too
  float4 pa[2], pb[2];
  bool pok[2];
  auto load = [&](int64_t i0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = t + u * kBlock, r = e >> 3, g = e & 7;
      const int64_t i = i0 + r;
      const float* row = X + (i < r1 ? i : r1 - 1) * L;
      pa[u] = *reinterpret_cast<const float4*>(row + a0 + 4 * g);
      pb[u] = *reinterpret_cast<const float4*>(row + b0 + 4 * g);
      pok[u] = i < r1;
    }
  };
  if (r0 < r1) load(r0);
  for (int64_t i0 = r0; i0 < r1; i0 += 64) {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = t + u * kBlock, r = e >> 3, g = e & 7;
      const float4 va = pok[u] ? pa[u] : z, vb = pok[u] ? pb[u] : z;
      xa[r][4 * g] = va.x;
      xa[r][4 * g + 1] = va.y;
      xa[r][4 * g + 2] = va.z;
      xa[r][4 * g + 3] = va.w;
      *reinterpret_cast<float4*>(&xb[r][4 * g]) = vb;
    }
    __syncthreads();
    load(i0 + 64);  // unconditional (rows clamp), so nothing waits for it before the products
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    // 8 rows of LDS reads at a time ahead of their 32 products (row order kept)
#pragma unroll 2
    for (int rb = 0; rb < 64; rb += 8) {
      float va[8];
      float4 vb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        va[u] = xa[rb + u][ta];
        vb[u] = *reinterpret_cast<const float4*>(&xb[rb + u][tb]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        part[0] = __builtin_fmaf(va[u], vb[u].x, part[0]);
        part[1] = __builtin_fmaf(va[u], vb[u].y, part[1]);
        part[2] = __builtin_fmaf(va[u], vb[u].z, part[2]);
        part[3] = __builtin_fmaf(va[u], vb[u].w, part[3]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += (double)part[j];
    __syncthreads();
  }
  double* G = Gp + (int64_t)blockIdx.y * L * L;
#pragma unroll
  for (int j = 0; j < 4; ++j) G[(a0 + ta) * L + b0 + tb + j] = acc[j];
}

// G[a][b] = sum over the splits of Gp[z][a][b], read from the tile on or above the
// diagonal (so G is exactly symmetric).  Block: 64 entries x 4 groups of splits; group g
// takes splits g, g + 4, ... into four chains in a fixed order, then the four group sums
// are added in order, so the result does not depend on timing.
constexpr int kGramSumGroups = kBlock / 64;
__global__ __launch_bounds__(kBlock) void gram_sum_kernel(const double* __restrict__ Gp, int splits,
                                                          int L, double* __restrict__ G) {
  __shared__ double red[kGramSumGroups][64];
  const int t = threadIdx.x, eo = t & 63, g = t >> 6;
  const int64_t count = (int64_t)L * L;
  const int64_t e = (int64_t)blockIdx.x * 64 + eo;
  double v = 0.0;
  int64_t src = 0;
  if (e < count) {
    const int a = (int)(e / L), b = (int)(e % L);
    src = (a >> 5) <= (b >> 5) ? e : (int64_t)b * L + a;
    // four chains over the group's splits z = g + G (4 c + j), their loads issued
    // together; then added in a fixed order
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    int z = g;
    for (; z + 3 * kGramSumGroups < splits; z += 4 * kGramSumGroups) {
      double v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] = Gp[(int64_t)(z + j * kGramSumGroups) * count + src];
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] += v4[j];
    }
    for (int j = 0; z < splits; z += kGramSumGroups, ++j) s[j] += Gp[(int64_t)z * count + src];
    v = (s[0] + s[1]) + (s[2] + s[3]);
  }
  red[g][eo] = v;
  __syncthreads();
  if (g == 0 && e < count) {
    double s = red[0][eo];
    for (int k = 1; k < kGramSumGroups; ++k) s += red[k][eo];
    G[e] = s;
  }
}

// ------------------------------------------------------- symmetric eigen --

constexpr int kMaxWidth = 512;
constexpr int kLdsWidth = 96;  // widths up to this keep their two fp64 matrices in LDS
constexpr int kGrid = 32;                    // 32 x 32 threads own a small matrix
constexpr int kSmallBlocks = kLdsWidth / kGrid;  // entries per thread and side, at most
constexpr int kSyevThreads = kGrid * kGrid;
constexpr int kSyevWaves = kSyevThreads / kWave;

// Lane permutations of fp64 values by DPP (two 32-bit moves): quad_perm [1,0,3,2] and
// [2,3,0,1], row_half_mirror, row_mirror.
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// Sums over the 16 lanes of each DPP row, the 32 lanes of each half-wave and the 64
// lanes of the wave (every lane gets the sum, bit-identical): pairs combined by DPP
// within rows of 16, then across rows.
__device__ __forceinline__ double sum16_f64(double v) {
  v += dpp64<0xB1>(v);
  v += dpp64<0x4E>(v);
  v += dpp64<0x141>(v);
  return v + dpp64<0x140>(v);
}
__device__ __forceinline__ double sum32_f64(double v) {
  v = sum16_f64(v);
  return v + __shfl_xor(v, 16, kWave);
}
// Sum over the kGrid lanes sharing a row of the thread grid.
__device__ __forceinline__ double sumrow_f64(double v) {
  if constexpr (kGrid == 16) return sum16_f64(v);
  else return sum32_f64(v);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = sum32_f64(v);
  return v + __shfl_xor(v, 32, kWave);
}
// 1 / q from the hardware estimate and one Newton step.
__device__ __forceinline__ double recip(double q) {
  const double r = __builtin_amdgcn_rcp(q);
  return __builtin_fma(__builtin_fma(-q, r, 1.0), r, r);
}

// Eigendecomposition of the symmetric L x L matrix S (fp64), one block, in four phases:
//  1. Householder reduction to tridiagonal form T = H^T S H (H = H_0 ... H_{L-3}): step k
//     reflects row k right of the diagonal, x, onto alpha e_1 with v = x - alpha e_1,
//     alpha = -sign(x_0) |x|, tau = 2 / v^T v, and updates the trailing block by
//     S <- S - v w^T - w v^T, p = tau S v, w = p - (tau / 2)(p^T v) v (Golub and Van Loan,
//     Matrix Computations, section 8.3.1); row k keeps v (its first entry apart).
//  2. The nev largest eigenvalues of T by bisection on Sturm counts (the number of
//     negative pivots of T - x I, each pivot's reciprocal from the hardware estimate and
//     one Newton step), G-way multisection per eigenvalue by G lanes, to 2^-32 |T|.
//  3. Their eigenvectors by inverse iteration (three solves with the LU factors of
//     T - lambda I, pivots below eps |T| raised to eps |T|), one lane per eigenvalue;
//     eigenvalues closer than 1e-7 |T| to their predecessor form clusters whose members
//     are computed one level at a time and orthogonalized against the earlier ones.
//     Each eigenvalue is then the Rayleigh quotient of its unit eigenvector.
//  4. Back-transformation of the eigenvectors by the reflectors, last to first.
// On exit columns L - nev .. L - 1 of V (L x L) hold the eigenvectors (the other columns
// zero), evals the eigenvalues in increasing order (zero below L - nev), order the
// indices by decreasing eigenvalue.  LOCAL (L <= kLdsWidth):
// in phase 1 the 32 x 32 threads hold rows ti + 32 a and columns tj + 32 b of S in
// registers, step k publishing row k (which then keeps v) and its norm in LDS, then
// exchanging p and the row groups' parts of v^T S v through LDS, row sums being lane
// sums (DPP within 16 lanes, one shuffle across); in phase 4 they hold rows tj + 32 b and
// columns ti + 32 a of the eigenvectors, so the column sums v^T X are lane sums and a
// step needs no barrier.  Otherwise S
// and the eigenvectors live in the global buffers Sg and Vg, waves running over rows and
// lanes along them.  ug: L x L fp64 scratch (the LU pivots of each lane's solves).
template <bool LOCAL>
__global__ __launch_bounds__(kSyevThreads) void syev_kernel(double* __restrict__ Sg, int L, int nev,
                                                            double* __restrict__ Vg,
                                                            double* __restrict__ ug,
                                                            double* __restrict__ evals,
                                                            int* __restrict__ order) {
  constexpr int W = LOCAL ? kLdsWidth : kMaxWidth;
  constexpr int NC = (W + kWave - 1) / kWave;  // 64-lane chunks of a row
  __shared__ double Al[LOCAL ? kLdsWidth * kLdsWidth : 1], Xl[LOCAL ? kLdsWidth * kLdsWidth : 1];
  __shared__ double dd[W], ee[W], tau[W], vz[W], lam[W];
  __shared__ double part[LOCAL ? 1 : kSyevWaves][W];  // partial sums (LOCAL: p)
  __shared__ int pos[W];
  __shared__ double sh_lo, sh_hi, sh_tn, sh_pivmin, s2buf[2], kpart[kGrid];
  __shared__ int sh_maxpos;
  double* A = LOCAL ? Al : Sg;
  double* X = LOCAL ? Xl : Vg;
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const int ti = t / kGrid, tj = t % kGrid, nb = L / kGrid;

  // ---- 1. tridiagonalization
  if constexpr (LOCAL) {
    double a[kSmallBlocks][kSmallBlocks];
#pragma unroll
    for (int p = 0; p < kSmallBlocks; ++p)
#pragma unroll
      for (int q = 0; q < kSmallBlocks; ++q)
        a[p][q] = (p < nb && q < nb) ? Sg[(ti + kGrid * p) * L + tj + kGrid * q] : 0.0;
    // row k of the registers into LDS row k, and the squared norm of its entries past
    // column k + 1 into s2buf[k & 1]
    auto publish = [&](int k) {
      if (ti == k % kGrid) {
        double s2 = 0.0;
#pragma unroll
        for (int q = 0; q < kSmallBlocks; ++q) {
          double v = a[0][q];
#pragma unroll
          for (int p = 1; p < kSmallBlocks; ++p)
            if (p == k / kGrid) v = a[p][q];
          const int j = tj + kGrid * q;
          if (q < nb) A[k * L + j] = v;
          if (q < nb && j > k + 1) s2 += v * v;
        }
        s2 = sumrow_f64(s2);
        if (tj == 0) s2buf[k & 1] = s2;
      }
    };
    // step k, instantiated per block KP = k / 32 of row k and block KB = (k + 1) / 32 where
    // the reflector starts, so that the tests i, j >= k + 1 are compile-time outside the
    // block that straddles k + 1.  The owners of row k publish it; the one holding entry
    // k + 1 computes the reflector (alpha, v0, tau) once and stores v0 in its place.
    auto hstep = [&](auto kp_const, auto kb_const, int k) {
      constexpr int KP = decltype(kp_const)::value, KB = decltype(kb_const)::value;
      const int b = k + 1, kr = k - KP * kGrid, br = b - KB * kGrid;
      if (ti == kr) {
        double s2 = 0.0;
#pragma unroll
        for (int q = 0; q < kSmallBlocks; ++q) {
          if (q >= nb) continue;
          const double v = a[KP][q];
          const int j = tj + kGrid * q;
          A[k * L + j] = v;
          if (j > b) s2 += v * v;
        }
        s2 = sumrow_f64(s2);
        if (tj == kr) dd[k] = a[KP][KP];
        if (tj == br) {  // entry b = tj + 32 KB
          const double x0 = a[KP][KB];
          double tk = 0.0, v0 = x0, al = x0;
          if (s2 > 0.0) {
            const double mu = __builtin_sqrt(x0 * x0 + s2);
            al = x0 > 0.0 ? -mu : mu;
            v0 = x0 - al;
            tk = 2.0 / (v0 * v0 + s2);
          }
          A[k * L + b] = v0;
          ee[k] = al;
          tau[k] = tk;
          vz[k] = v0;
        }
      }
      __syncthreads();
      const double tk = tau[k];
      if (tk == 0.0) return;  // uniform
      const double* R = A + k * L;  // v: R[i] for i >= b, 0 before
      double vi[kSmallBlocks], vj[kSmallBlocks], ps[kSmallBlocks];
#pragma unroll
      for (int p = 0; p < kSmallBlocks; ++p) {
        vi[p] = vj[p] = 0.0;
        if (p < KB || p >= nb) continue;
        const double ri = R[ti + kGrid * p], rj = R[tj + kGrid * p];
        vi[p] = (p > KB || ti >= br) ? ri : 0.0;
        vj[p] = (p > KB || tj >= br) ? rj : 0.0;
      }
#pragma unroll
      for (int p = 0; p < kSmallBlocks; ++p) {
        ps[p] = 0.0;
        if (p < KB || p >= nb) continue;
        double acc = 0.0;
#pragma unroll
        for (int q = KB; q < kSmallBlocks; ++q)
          if (q < nb) acc += a[p][q] * vj[q];
        ps[p] = sumrow_f64(acc);
      }
      if (tj == 0) {  // p_i for the row group's rows, and its part of v^T S' v
        double vsv = 0.0;
#pragma unroll
        for (int p = KB; p < kSmallBlocks; ++p) {
          if (p >= nb) continue;
          part[0][ti + kGrid * p] = tk * ps[p];
          vsv += ps[p] * vi[p];
        }
        kpart[ti] = vsv;
      }
      __syncthreads();
      // K = (tau / 2) p^T v = (tau^2 / 2) v^T S' v
      const double K = 0.5 * tk * tk * sumrow_f64(kpart[tj]);
      double wi[kSmallBlocks], wj[kSmallBlocks];
#pragma unroll
      for (int p = 0; p < kSmallBlocks; ++p) {
        wi[p] = wj[p] = 0.0;
        if (p < KB || p >= nb) continue;
        wi[p] = part[0][ti + kGrid * p] - K * vi[p];
        wj[p] = part[0][tj + kGrid * p] - K * vj[p];
      }
#pragma unroll
      for (int p = KB; p < kSmallBlocks; ++p) {
        if (p >= nb) continue;
#pragma unroll
        for (int q = KB; q < kSmallBlocks; ++q) {
          if (q >= nb) continue;
          const double d = vi[p] * wj[q] + wi[p] * vj[q];
          if (p == KB || q == KB) {  // the straddling block: only entries i, j >= b
            const bool in = (p > KB || ti >= br) && (q > KB || tj >= br);
            a[p][q] = in ? a[p][q] - d : a[p][q];
          } else {
            a[p][q] -= d;
          }
        }
      }
    };
    static_assert(kSmallBlocks == 3, "one instantiation per pair of blocks");
    for (int k = 0; k < L - 2; ++k) {
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      if (k < kGrid - 1) hstep(I0{}, I0{}, k);
      else if (k == kGrid - 1) hstep(I0{}, I1{}, k);
      else if (k < 2 * kGrid - 1) hstep(I1{}, I1{}, k);
      else if (k == 2 * kGrid - 1) hstep(I1{}, I2{}, k);
      else hstep(I2{}, I2{}, k);
    }
    publish(L - 2);
    publish(L - 1);
    __syncthreads();
  } else {
  for (int k = 0; k < L - 2; ++k) {
    const int b = k + 1, n1 = L - b;
    double vv[NC];  // v_i for i = lane + 64 c (0 past the end)
    double s2 = 0.0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = lane + kWave * c;
      vv[c] = i < n1 ? A[k * L + b + i] : 0.0;
      if (i >= 1) s2 += vv[c] * vv[c];
    }
    s2 = wave_sum_f64(s2);  // the same in every wave
    const double x0 = A[k * L + b];
    double tk = 0.0, v0 = x0, al = x0;
    if (s2 > 0.0) {
      const double mu = __builtin_sqrt(x0 * x0 + s2);
      al = x0 > 0.0 ? -mu : mu;
      v0 = x0 - al;
      tk = 2.0 / (v0 * v0 + s2);
    }
    if (lane == 0) vv[0] = v0;
    if (t == 0) {
      dd[k] = A[k * L + k];
      ee[k] = al;
      tau[k] = tk;
      vz[k] = v0;
    }
    if (tk != 0.0) {  // uniform
      // part[w][i] = sum over the rows j of wave w's slice of S'[j][i] v_j
      const int j0 = (wv * n1) / kSyevWaves, j1 = ((wv + 1) * n1) / kSyevWaves;
      double acc[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = 0.0;
      for (int j = j0; j < j1; ++j) {
        const double vj = j == 0 ? v0 : A[k * L + b + j];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int i = lane + kWave * c;
          if (i < n1) acc[c] += A[(b + j) * L + b + i] * vj;
        }
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int i = lane + kWave * c;
        if (i < n1) part[wv][i] = acc[c];
      }
      __syncthreads();
      double ww[NC], kd = 0.0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int i = lane + kWave * c;
        double p = 0.0;
        if (i < n1) {
          for (int w = 0; w < kSyevWaves; ++w) p += part[w][i];
          p *= tk;
        }
        ww[c] = p;
        kd += p * vv[c];
      }
      const double K = 0.5 * tk * wave_sum_f64(kd);
#pragma unroll
      for (int c = 0; c < NC; ++c) ww[c] -= K * vv[c];
      for (int i = wv; i < n1; i += kSyevWaves) {  // S' -= v w^T + w v^T, row i
        double vsel = vv[0], wsel = ww[0];
#pragma unroll
        for (int c = 1; c < NC; ++c)
          if ((i >> 6) == c) {
            vsel = vv[c];
            wsel = ww[c];
          }
        const double vi = __shfl(vsel, i & (kWave - 1), kWave);
        const double wi = __shfl(wsel, i & (kWave - 1), kWave);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int j = lane + kWave * c;
          if (j < n1) A[(b + i) * L + b + j] -= vi * ww[c] + wi * vv[c];
        }
      }
    }
    __syncthreads();
  }
  }
  if (t == 0) {
    dd[L - 2] = A[(L - 2) * L + L - 2];
    dd[L - 1] = A[(L - 1) * L + L - 1];
    ee[L - 2] = A[(L - 2) * L + L - 1];
    ee[L - 1] = 0.0;
    tau[L - 2] = tau[L - 1] = 0.0;
    double lo = 0.0, hi = 0.0, e2max = 0.0;  // Gershgorin interval of T
    for (int i = 0; i < L; ++i) {
      const double r = (i > 0 ? __builtin_fabs(ee[i - 1]) : 0.0) + __builtin_fabs(ee[i]);
      const double l = dd[i] - r, h = dd[i] + r;
      lo = i == 0 || l < lo ? l : lo;
      hi = i == 0 || h > hi ? h : hi;
      e2max = ee[i] * ee[i] > e2max ? ee[i] * ee[i] : e2max;
    }
    const double tn = __builtin_fmax(__builtin_fabs(lo), __builtin_fabs(hi));
    const double pivmin = __DBL_MIN__ * (e2max > 1.0 ? e2max : 1.0);
    sh_lo = lo - (2.0 * __DBL_EPSILON__ * tn + pivmin);
    sh_hi = hi + (2.0 * __DBL_EPSILON__ * tn + pivmin);
    sh_tn = tn;
    sh_pivmin = pivmin;
  }
  __syncthreads();

  // ---- 2. eigenvalues L - nev .. L - 1 (ascending): lanes g G .. g G + G - 1 bracket the
  // (L - nev + g)-th smallest to 2^-32 |T|
  const double tn = sh_tn, pivmin = sh_pivmin;
  const int first = L - nev;
  {
    int G = 1;
    while (G < 8 && 2 * G * nev <= kSyevThreads) G *= 2;
    const int m = t % G, gbase = lane & ~(G - 1);
    const double tol = 0x1p-32 * tn + pivmin;
    for (int g = t / G; g < nev; g += kSyevThreads / G) {
      const int gi = first + g;
      double lo = sh_lo, hi = sh_hi;
      for (int it = 0; it < 200; ++it) {
        const double wdt = hi - lo;
        if (!(wdt > tol)) break;
        const double x = lo + (double)(m + 1) * wdt / (double)(G + 1);
        double q = dd[0] - x;
        if (__builtin_fabs(q) < pivmin) q = -pivmin;
        int cnt = q < 0.0 ? 1 : 0;
        for (int i = 1; i < L; ++i) {
          const double e = ee[i - 1];
          q = __builtin_fma(-(e * e), recip(q), dd[i] - x);
          if (__builtin_fabs(q) < pivmin) q = -pivmin;
          cnt += q < 0.0 ? 1 : 0;
        }
        double nlo = lo, nhi = hi;
        for (int mm = 0; mm < G; ++mm) {  // largest point with count <= gi, smallest with > gi
          const int cm = __shfl(cnt, gbase + mm, kWave);
          const double xm = lo + (double)(mm + 1) * wdt / (double)(G + 1);
          if (cm <= gi) nlo = xm;
        }
        for (int mm = G - 1; mm >= 0; --mm) {
          const int cm = __shfl(cnt, gbase + mm, kWave);
          const double xm = lo + (double)(mm + 1) * wdt / (double)(G + 1);
          if (cm > gi) nhi = xm;
        }
        lo = nlo;
        hi = nhi;
      }
      if (m == 0) lam[gi] = 0.5 * (lo + hi);
    }
  }
  for (int e = t; e < L * first; e += kSyevThreads) X[(e / first) * L + e % first] = 0.0;
  __syncthreads();

  // ---- 3. eigenvectors of T, cluster level by cluster level; each eigenvalue is then
  // refined to the Rayleigh quotient x^T T x of its unit eigenvector
  const double tnz = tn > 0.0 ? tn : 1.0;
  if (t == 0) {
    int mp = 0;
    pos[first] = 0;
    for (int i = first + 1; i < L; ++i) {
      pos[i] = lam[i] - lam[i - 1] <= 1e-7 * tnz ? pos[i - 1] + 1 : 0;
      mp = pos[i] > mp ? pos[i] : mp;
    }
    sh_maxpos = mp;
  }
  __syncthreads();
  {
    const double tiny = __DBL_EPSILON__ * tnz;
    const int maxpos = sh_maxpos;
    for (int lev = 0; lev <= maxpos; ++lev) {
      for (int i = first + t; i < L; i += kSyevThreads) {
        if (pos[i] != lev) continue;
        const double li = lam[i];
        for (int r = 0; r < L; ++r) X[r * L + i] = 1.0 + (double)((r * 40503 + i * 34283) & 1023) / 4096.0;
        for (int it = 0; it < 3; ++it) {
          // T - li I = L U: forward elimination fused with L y = x (y over x); ug keeps
          // the pivots' reciprocals
          double up = dd[0] - li;
          if (__builtin_fabs(up) < tiny) up = tiny;
          double rup = recip(up);
          ug[i] = rup;
          double y = X[i];
          for (int j = 1; j < L; ++j) {
            const double mlt = ee[j - 1] * rup;
            up = dd[j] - li - mlt * ee[j - 1];
            if (__builtin_fabs(up) < tiny) up = tiny;
            rup = recip(up);
            ug[j * L + i] = rup;
            y = X[j * L + i] - mlt * y;
            X[j * L + i] = y;
          }
          // U x = y
          double xn = y * rup, nrm = xn * xn;
          X[(L - 1) * L + i] = xn;
          for (int j0 = L - 2; j0 >= 0; j0 -= 8) {  // pivots of 8 rows loaded ahead
            double uu[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) uu[q] = j0 - q >= 0 ? ug[(j0 - q) * L + i] : 1.0;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const int j = j0 - q;
              if (j >= 0) {
                xn = (X[j * L + i] - ee[j] * xn) * uu[q];
                X[j * L + i] = xn;
                nrm += xn * xn;
              }
            }
          }
          if (!(nrm > 0.0 && nrm < __DBL_MAX__)) {  // no usable solve: start from e_i
            for (int r = 0; r < L; ++r) X[r * L + i] = r == i ? 1.0 : 0.0;
            nrm = 1.0;
          }
          double sc = 1.0 / __builtin_sqrt(nrm);
          for (int r = 0; r < L; ++r) X[r * L + i] *= sc;
          if (lev > 0) {  // orthogonalize against the cluster's earlier members
            for (int jj = i - lev; jj < i; ++jj) {
              double dot = 0.0;
              for (int r = 0; r < L; ++r) dot += X[r * L + jj] * X[r * L + i];
              for (int r = 0; r < L; ++r) X[r * L + i] -= dot * X[r * L + jj];
            }
            nrm = 0.0;
            for (int r = 0; r < L; ++r) nrm += X[r * L + i] * X[r * L + i];
            sc = nrm > 0.0 ? 1.0 / __builtin_sqrt(nrm) : 0.0;
            for (int r = 0; r < L; ++r) X[r * L + i] *= sc;
          }
        }
        double rq = 0.0, xp = X[i];
        for (int r = 0; r < L; ++r) {
          const double xr = xp;
          xp = r + 1 < L ? X[(r + 1) * L + i] : 0.0;
          rq += xr * (dd[r] * xr + 2.0 * ee[r] * xp);
        }
        lam[i] = rq;
      }
      __syncthreads();
    }
  }

  // ---- 4. back-transformation X <- H_k X, k = L - 3 .. 0
  if constexpr (LOCAL) {
    double x[kSmallBlocks][kSmallBlocks];  // x[q][p] = X[tj + 32 q][ti + 32 p]
#pragma unroll
    for (int q = 0; q < kSmallBlocks; ++q)
#pragma unroll
      for (int p = 0; p < kSmallBlocks; ++p)
        x[q][p] = (p < nb && q < nb) ? X[(tj + kGrid * q) * L + ti + kGrid * p] : 0.0;
    for (int k = L - 3; k >= 0; --k) {
      const double tk = tau[k];
      if (tk == 0.0) continue;
      const int b = k + 1;
      double vr[kSmallBlocks];
#pragma unroll
      for (int q = 0; q < kSmallBlocks; ++q) {
        const int r = tj + kGrid * q;
        vr[q] = (q < nb && r >= b) ? (r == b ? vz[k] : A[k * L + r]) : 0.0;
      }
#pragma unroll
      for (int p = 0; p < kSmallBlocks; ++p) {
        double y = 0.0;
#pragma unroll
        for (int q = 0; q < kSmallBlocks; ++q) y += vr[q] * x[q][p];
        y = tk * sumrow_f64(y);
#pragma unroll
        for (int q = 0; q < kSmallBlocks; ++q) x[q][p] -= vr[q] * y;
      }
    }
#pragma unroll
    for (int q = 0; q < kSmallBlocks; ++q)
#pragma unroll
      for (int p = 0; p < kSmallBlocks; ++p)
        if (p < nb && q < nb) Vg[(tj + kGrid * q) * L + ti + kGrid * p] = x[q][p];
  } else {
  for (int k = L - 3; k >= 0; --k) {
    const double tk = tau[k];
    if (tk == 0.0) continue;  // uniform
    const int b = k + 1, n1 = L - b;
    const int i0 = (wv * n1) / kSyevWaves, i1 = ((wv + 1) * n1) / kSyevWaves;
    double acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.0;
    for (int i = i0; i < i1; ++i) {
      const double vi = i == 0 ? vz[k] : A[k * L + b + i];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int col = lane + kWave * c;
        if (col < L) acc[c] += vi * X[(b + i) * L + col];
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = lane + kWave * c;
      if (col < L) part[wv][col] = acc[c];
    }
    __syncthreads();
    double yc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = lane + kWave * c;
      double y = 0.0;
      if (col < L)
        for (int w = 0; w < kSyevWaves; ++w) y += part[w][col];
      yc[c] = tk * y;
    }
    for (int i = wv; i < n1; i += kSyevWaves) {
      const double vi = i == 0 ? vz[k] : A[k * L + b + i];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int col = lane + kWave * c;
        if (col < L) X[(b + i) * L + col] -= vi * yc[c];
      }
    }
    __syncthreads();
  }
  }
  for (int i = t; i < L; i += kSyevThreads) {
    evals[i] = i >= first ? lam[i] : 0.0;
    order[i] = L - 1 - i;
  }
}

constexpr int kCholThreads = 1024;
constexpr int kCholWaves = kCholThreads / kWave;

// Cholesky QR with dropped pivots: G = U^T D U (U unit upper triangular, D diagonal) by
// right-looking elimination in the upper triangle, a pivot d_k <= 2^-16 g_kk (the column's
// squared distance from the span of the earlier ones below 2^-16 of its squared norm, or
// no larger than the error of the Gram matrix's fp32 sums, whose entries are within
// 2^-18 sqrt(g_aa g_bb)) drops column k; T = U^-1 D^-1/2 (L x L fp32, upper triangular)
// with zero row and column for dropped indices, so that the columns of Y T are the
// Gram-Schmidt vectors of Y's columns: orthonormal up to the Gram matrix's error relative
// to the pivots, zero where dropped.  Applied twice (the second time to Y T), the basis
// is orthonormal to about 2^-18.
//
// Widths up to kLdsWidth (chol_inverse_small_kernel): the matrix lives in registers, the
// 32 x 32 threads owning rows ti + 32 a and columns tj + 32 b (a, b < L / 32); step k
// broadcasts row k through LDS (one barrier) and every thread updates its entries.  The
// same eliminations applied to the identity, kept below the diagonal, leave L^-1 there
// (G = L D L^T, U = L^T), so no back substitution is needed.  Wider
// (chol_inverse_kernel): the matrices live in global memory (Ag, the Gram matrix,
// overwritten, and Xg, scratch), waves run over rows and lanes along them.  One block.
__global__ __launch_bounds__(kGrid * kGrid) void chol_inverse_small_kernel(const double* __restrict__ Ag,
                                                                          int L,
                                                                          float* __restrict__ T) {
  // R row k: the matrix's row k when step k starts, with 1 (the identity's entry) in
  // place of the pivot d_k; rinv[k] = 1 / d_k, 0 for a dropped column
  __shared__ double R[kLdsWidth * kLdsWidth];
  __shared__ double rinv[kLdsWidth];
  const int t = threadIdx.x, ti = t / kGrid, tj = t % kGrid;
  const int nb = L / kGrid;  // entries per thread along rows and columns
  // m[i][j]: on and above the diagonal the matrix being eliminated (rows of D U once
  // final); below it the eliminations applied to the identity, i.e. L^-1 (unit diagonal
  // implied) for G = L D L^T
  double a[kSmallBlocks][kSmallBlocks];
  double thr[kSmallBlocks];  // threads with ti = tj: 2^-16 g_ii of their diagonal entries
#pragma unroll
  for (int p = 0; p < kSmallBlocks; ++p) {
#pragma unroll
    for (int q = 0; q < kSmallBlocks; ++q) {
      const int i = ti + kGrid * p, j = tj + kGrid * q;
      a[p][q] = (p < nb && q < nb && j >= i) ? Ag[i * L + j] : 0.0;
    }
    thr[p] = 0x1p-16 * a[p][p];
  }
  // step k: rows i > k lose l_ik times row k, l_ik = m_ki / d_k, in the upper part (j >= i)
  // the elimination, in the lower part (j < k) and at j = k (the identity's 1) the same
  // operation on the identity.  Entry (i, k) is assigned -l_ik rather than updated, and
  // lower entries k < j < i take meaningless updates until step j assigns them: row k of
  // the identity's image is zero there, so nothing read later depends on them.  Finished
  // entries (rows <= k) are never read again, so blocks of rows all <= k skip the step and
  // rows <= k inside a live block take l = 0.
  // The step body is instantiated per block KB = k / 32 so that the selects for row and
  // column k (i > k, j = k) appear only in the block row and column that hold them.
  int k = 0;
  auto step = [&](auto kb_const) {
    constexpr int KB = decltype(kb_const)::value;
    const int kr = k - KB * kGrid;
    if (ti == kr) {  // owners of row k publish it
#pragma unroll
      for (int q = 0; q < kSmallBlocks; ++q)
        if (q < nb) {
          double v = a[KB][q];
          if (q == KB && tj == kr) {  // the pivot (ti = tj here)
            rinv[k] = v > thr[KB] ? recip(v) : 0.0;
            v = 1.0;
          }
          R[k * L + tj + kGrid * q] = v;
        }
    }
    __syncthreads();
    // every read of the step at once (k L + 95 stays inside R for L <= kLdsWidth)
    const double inv = rinv[k];
    double rj[kSmallBlocks], rk[kSmallBlocks];
#pragma unroll
    for (int q = 0; q < kSmallBlocks; ++q) {
      rj[q] = R[k * L + tj + kGrid * q];
      rk[q] = R[k * L + ti + kGrid * q];
    }
#pragma unroll
    for (int p = KB; p < kSmallBlocks; ++p) {  // blocks p < KB hold rows <= k only
      if (p >= nb) continue;
      double f = rk[p] * inv;
      if (p == KB) f = ti > kr ? f : 0.0;
#pragma unroll
      for (int q = 0; q < kSmallBlocks; ++q) {
        if (q >= nb) continue;
        double base = a[p][q];
        if (q == KB) base = tj == kr ? 0.0 : base;
        a[p][q] = __builtin_fma(-f, rj[q], base);
      }
    }
  };
  static_assert(kSmallBlocks == 3, "one instantiation per block of rows");
  for (; k < L; ++k) {
    if (k < kGrid)
      step(std::integral_constant<int, 0>{});
    else if (k < 2 * kGrid)
      step(std::integral_constant<int, 1>{});
    else
      step(std::integral_constant<int, 2>{});
  }
  // T = U^-1 D^-1/2 = (L^-1)^T D^-1/2: T[c][r] = m[r][c] / sqrt(d_r) for c < r, 1 / sqrt(d_r)
  // at c = r, zero for dropped rows and columns (the thread owning m[r][c] writes it)
#pragma unroll
  for (int p = 0; p < kSmallBlocks; ++p)
#pragma unroll
    for (int q = 0; q < kSmallBlocks; ++q) {
      const int r = ti + kGrid * p, c = tj + kGrid * q;
      if (p < nb && q < nb) {
        const bool keep = rinv[r] != 0.0 && rinv[c] != 0.0 && c <= r;
        const double x = c == r ? 1.0 : a[p][q];
        T[c * L + r] = keep ? (float)(x * __builtin_sqrt(rinv[r])) : 0.f;
      }
    }
}

__global__ __launch_bounds__(kCholThreads) void chol_inverse_kernel(double* __restrict__ A,
                                                                   double* __restrict__ X, int L,
                                                                   float* __restrict__ T) {
  __shared__ double piv[kMaxWidth];  // 1 / d_k, 0 for a dropped column
  constexpr int NC = kMaxWidth / kWave;  // 64-lane chunks of a row
  constexpr int PB = 2;                  // rows whose accesses are batched
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  for (int k = t; k < L; k += kCholThreads) piv[k] = A[k * L + k];  // g_kk, kept until step k
  for (int i = wv; i < L; i += kCholWaves)
    for (int j = lane; j < L; j += kWave) X[i * L + j] = i == j ? 1.0 : 0.0;
  __syncthreads();
  // step k: a_ij -= a_ki a_kj / d_k for k < i, k < j (a_k. is row k of D U, unscaled; the
  // entries below the diagonal are updated too and never read)
  for (int k = 0; k < L - 1; ++k) {
    const double d = A[k * L + k];
    const double inv = d > 0x1p-16 * piv[k] ? 1.0 / d : 0.0;
    if (inv != 0.0) {
      double rk[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int j = lane + kWave * c;
        rk[c] = (j > k && j < L) ? A[k * L + j] * inv : 0.0;
      }
      for (int i0 = k + 1 + wv; i0 < L; i0 += PB * kCholWaves) {
        double f[PB], a[PB][NC];
#pragma unroll
        for (int u = 0; u < PB; ++u) {
          const int i = i0 + u * kCholWaves;
          f[u] = i < L ? A[k * L + i] : 0.0;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int j = lane + kWave * c;
            if (i < L && j > k && j < L) a[u][c] = A[i * L + j];
          }
        }
#pragma unroll
        for (int u = 0; u < PB; ++u) {
          const int i = i0 + u * kCholWaves;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int j = lane + kWave * c;
            if (i < L && j > k && j < L) A[i * L + j] = a[u][c] - f[u] * rk[c];
          }
        }
      }
    }
    __syncthreads();
  }
  for (int k = t; k < L; k += kCholThreads) {
    const double d = A[k * L + k];
    piv[k] = d > 0x1p-16 * piv[k] ? 1.0 / d : 0.0;
  }
  __syncthreads();
  // X = U^-1 by back substitution on U X = I (u_ik = a_ik / d_i), one row finished per step
  for (int k = L - 1; k > 0; --k) {
    double xk[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int j = lane + kWave * c;
      xk[c] = (j >= k && j < L) ? X[k * L + j] : 0.0;
    }
    for (int i0 = wv; i0 < k; i0 += PB * kCholWaves) {  // columns k .. L - 1 of rows < k
      double uu[PB], x[PB][NC];
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int i = i0 + u * kCholWaves;
        uu[u] = i < k ? A[i * L + k] * piv[i] : 0.0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int j = lane + kWave * c;
          if (i < k && j >= k && j < L) x[u][c] = X[i * L + j];
        }
      }
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int i = i0 + u * kCholWaves;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int j = lane + kWave * c;
          if (i < k && j >= k && j < L) X[i * L + j] = x[u][c] - uu[u] * xk[c];
        }
      }
    }
    __syncthreads();
  }
  // T = X D^-1/2, column j scaled by 1 / sqrt(d_j), zero for dropped rows and columns
  for (int i = wv; i < L; i += kCholWaves)
    for (int j = lane; j < L; j += kWave)
      T[i * L + j] = (piv[i] != 0.0 && piv[j] != 0.0) ? (float)(X[i * L + j] * __builtin_sqrt(piv[j]))
                                                      : 0.f;
}

// T[b][c] = V[b][order[c]] * f(order[c]) for c < C (L x C fp32), where f is
// mode 1: sqrt(lambda) (sigma); mode 2: 1/sqrt(lambda), 0 for lambda <= 1e-12 lambda_max.
// sigma (may be null): sqrt(lambda) of the first C eigenvalues in decreasing order.
__global__ __launch_bounds__(kBlock) void transform_kernel(const double* __restrict__ V,
                                                           const double* __restrict__ evals,
                                                           const int* __restrict__ order, int L,
                                                           int C, int mode, float* __restrict__ T,
                                                           float* __restrict__ sigma) {
  const double lmax = evals[order[0]];
  for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < (int64_t)L * C;
       e += (int64_t)gridDim.x * kBlock) {
    const int b = (int)(e / C), c = (int)(e % C);
    const int k = order[c];
    const double lam = evals[k];
    double f;
    if (mode == 1) f = lam > 0.0 ? __builtin_sqrt(lam) : 0.0;
    else f = (lam > 1e-12 * lmax && lam > 0.0) ? 1.0 / __builtin_sqrt(lam) : 0.0;
    T[e] = (float)(V[(int64_t)b * L + k] * f);
    if (sigma && b == 0) sigma[c] = (float)(lam > 0.0 ? __builtin_sqrt(lam) : 0.0);
  }
}

// Out = X T for X (M x L fp32, row-major, M a multiple of 8) and T (L x C fp32): block of
// 64 rows x 32 columns; T's 32 columns and 64 x 32 tiles of X (coalesced row segments)
// staged in LDS; thread t: column c0 + t % 32, rows 8 (t / 32) .. + 8.  Outputs (each
// may be null): row-major fp32 (M x C), transposed fp32 (C x M) and transposed binary16
// (C x M, 16-byte aligned), the transposed ones stored 8 rows at a time as vectors (the
// fp32 one when its buffer is 16-byte aligned).
__global__ __launch_bounds__(kBlock) void apply_kernel(const float* __restrict__ X, int64_t M, int L,
                                                       const float* __restrict__ T, int C,
                                                       float* __restrict__ out_rm,
                                                       float* __restrict__ out_t32,
                                                       uint16_t* __restrict__ out_t16) {
  extern __shared__ float ts[];  // L x 33: T's 32 columns (dynamic, L * 33 floats)
  __shared__ float xs[64][33];
  const int t = threadIdx.x;
  const int c0 = blockIdx.y * 32;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  for (int e = t; e < L * 32; e += kBlock) {
    const int b = e >> 5, c = e & 31;
    ts[b * 33 + c] = c0 + c < C ? T[(int64_t)b * C + c0 + c] : 0.f;
  }
  const int c = t & 31, rb = (t >> 5) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int b0 = 0; b0 < L; b0 += 32) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // rows i0 .. + 64, columns b0 .. + 32 of X
      const int e = t + u * kBlock;
      const int r = e >> 5, col = e & 31;
      const int64_t i = i0 + r;
      xs[r][col] = i < M ? X[i * L + b0 + col] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int b = 0; b < 32; ++b) {
      const float tv = ts[(b0 + b) * 33 + c];
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = __builtin_fmaf(xs[rb + r][b], tv, acc[r]);
    }
    __syncthreads();
  }
  if (c0 + c >= C) return;
  const int64_t ib = i0 + rb;  // a multiple of 8; all 8 rows valid when ib < M
  if (ib >= M) return;
  if (out_rm) {
#pragma unroll
    for (int r = 0; r < 8; ++r) out_rm[(ib + r) * C + c0 + c] = acc[r];
  }
  if (out_t32) {
    float* o = out_t32 + (int64_t)(c0 + c) * M + ib;
    if ((reinterpret_cast<uintptr_t>(out_t32) & 15) == 0) {  // the caller's buffer may be 4-aligned
      reinterpret_cast<float4*>(o)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      reinterpret_cast<float4*>(o)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) o[r] = acc[r];
    }
  }
  if (out_t16) {
    uint4 h;
    h.x = f2h(acc[0]) | (f2h(acc[1]) << 16);
    h.y = f2h(acc[2]) | (f2h(acc[3]) << 16);
    h.z = f2h(acc[4]) | (f2h(acc[5]) << 16);
    h.w = f2h(acc[6]) | (f2h(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out_t16 + (int64_t)(c0 + c) * M + ib) = h;
  }
}

// apply_kernel for L = 32 LB <= 96: the block's 64 rows of X (all L columns) and T's 32
// columns come in with one round of 16-byte loads, all issued before any is stored to
// LDS (one global latency per block instead of one per 32 columns).  Same outputs.
template <int LB>
__global__ __launch_bounds__(kBlock) void apply_small_kernel(const float* __restrict__ X, int64_t M,
                                                             const float* __restrict__ T, int C,
                                                             float* __restrict__ out_rm,
                                                             float* __restrict__ out_t32,
                                                             uint16_t* __restrict__ out_t16) {
  constexpr int L = 32 * LB, XR = L + 1;  // X rows in LDS: odd stride
  constexpr int NX = 64 * L / 4 / kBlock, NT = L * 32 / 4 / kBlock;  // 16-byte loads per thread
  __shared__ float xs[64 * XR], ts[L * 33];
  const int t = threadIdx.x;
  const int c0 = blockIdx.y * 32;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  float4 xv[NX], tv4[NT];
#pragma unroll
  for (int u = 0; u < NX; ++u) {
    const int e = t + u * kBlock, r = e / (L / 4), g = e % (L / 4);
    const int64_t i = i0 + r < M ? i0 + r : M - 1;  // rows past M: unused
    xv[u] = reinterpret_cast<const float4*>(X + i * L)[g];
  }
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int e = t + u * kBlock, b = e >> 3, g = e & 7;
    tv4[u] = c0 + 4 * g < C ? reinterpret_cast<const float4*>(T + (int64_t)b * C + c0)[g]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int u = 0; u < NX; ++u) {
    const int e = t + u * kBlock, r = e / (L / 4), g = e % (L / 4);
    float* d = xs + r * XR + 4 * g;
    d[0] = xv[u].x; d[1] = xv[u].y; d[2] = xv[u].z; d[3] = xv[u].w;
  }
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int e = t + u * kBlock, b = e >> 3, g = e & 7;
    float* d = ts + b * 33 + 4 * g;
    d[0] = tv4[u].x; d[1] = tv4[u].y; d[2] = tv4[u].z; d[3] = tv4[u].w;
  }
  __syncthreads();
  const int c = t & 31, rb = (t >> 5) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int b = 0; b < L; ++b) {
    const float tv = ts[b * 33 + c];
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = __builtin_fmaf(xs[(rb + r) * XR + b], tv, acc[r]);
  }
  if (c0 + c >= C) return;
  const int64_t ib = i0 + rb;  // a multiple of 8; all 8 rows valid when ib < M
  if (ib >= M) return;
  if (out_rm) {
#pragma unroll
    for (int r = 0; r < 8; ++r) out_rm[(ib + r) * C + c0 + c] = acc[r];
  }
  if (out_t32) {
    float* o = out_t32 + (int64_t)(c0 + c) * M + ib;
    if ((reinterpret_cast<uintptr_t>(out_t32) & 15) == 0) {  // the caller's buffer may be 4-aligned
      reinterpret_cast<float4*>(o)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      reinterpret_cast<float4*>(o)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) o[r] = acc[r];
    }
  }
  if (out_t16) {
    uint4 h;
    h.x = f2h(acc[0]) | (f2h(acc[1]) << 16);
    h.y = f2h(acc[2]) | (f2h(acc[3]) << 16);
    h.z = f2h(acc[4]) | (f2h(acc[5]) << 16);
    h.w = f2h(acc[6]) | (f2h(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out_t16 + (int64_t)(c0 + c) * M + ib) = h;
  }
}

// ------------------------------------------------------------------ driver --

struct Carve {
  char* p;
  template <typename T>
  T* take(int64_t count) {
    T* r = reinterpret_cast<T*>(p);
    p += (count * (int64_t)sizeof(T) + 255) & ~(int64_t)255;
    return r;
  }
};

constexpr int64_t kPartialBudget = 64ll << 20;  // bytes of split-K partials at most
constexpr int64_t kGramBudget = 16ll << 20;     // bytes of partial Gram matrices at most

// Row splits of a Gram computation over M rows: enough blocks to fill the chip.
int gram_splits(int64_t M, int L) {
  const int64_t nt = L / 32, tiles = nt * (nt + 1) / 2;  // tiles on and above the diagonal
  int64_t s = (256 + tiles - 1) / tiles;
  if (s > (M + 63) / 64) s = (M + 63) / 64;
  const int64_t cap = kGramBudget / ((int64_t)L * L * 8);
  if (s > cap) s = cap;
  return s < 1 ? 1 : (int)s;
}

int gemm_splits(int64_t M, int64_t K, int L) {
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((L + kBN - 1) / kBN);
  int64_t s = (512 + tiles - 1) / tiles;
  if (s > 8) s = 8;
  if (s > K / kBK) s = K / kBK;
  const int64_t cap = kPartialBudget / (M * L * 4);
  if (s > cap) s = cap;
  return s < 1 ? 1 : (int)s;
}

}  // namespace

int64_t lowrank_workspace_bytes(int64_t m, int64_t n, int width) {
  const int64_t L = width, mx = m > n ? m : n;
  auto al = [](int64_t b) { return (b + 255) & ~(int64_t)255; };
  const int64_t sm = gemm_splits(m, n, width), sn = gemm_splits(n, m, width);
  const int64_t part = (sm * m > sn * n ? sm * m : sn * n) * L * 4;
  return al(m * n * 2) * 2 + al(mx * L * 4) + al(part) + al(L * mx * 2) + al(mx * L * 4) +
         al(L * L * 8) * 2 + al(L * 8) + al(L * 4) + al(L * L * 4) +
         al((int64_t)gram_splits(mx, width) * L * L * 8);  // gram_splits grows with M
}

hipError_t launch_residual(const uint16_t* W, const uint8_t* packed, const uint16_t* scale16,
                           const uint16_t* zero16, int64_t m, int64_t n, int nbits, int group_size,
                           uint16_t* dW, uint16_t* dWT, hipStream_t st) {
  const int gshift = group_size == 16 ? 4 : group_size == 32 ? 5 : group_size == 64 ? 6 : 7;
  const dim3 grid((unsigned)(n / kTile), (unsigned)(m / kTile));
  switch (nbits) {
    case 2: hipLaunchKernelGGL(residual_kernel<2>, grid, dim3(kBlock), 0, st, W, packed, scale16, zero16, m, n, gshift, dW, dWT); break;
    case 3: hipLaunchKernelGGL(residual_kernel<3>, grid, dim3(kBlock), 0, st, W, packed, scale16, zero16, m, n, gshift, dW, dWT); break;
    case 4: hipLaunchKernelGGL(residual_kernel<4>, grid, dim3(kBlock), 0, st, W, packed, scale16, zero16, m, n, gshift, dW, dWT); break;
    case 8: hipLaunchKernelGGL(residual_kernel<8>, grid, dim3(kBlock), 0, st, W, packed, scale16, zero16, m, n, gshift, dW, dWT); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lowrank(const LowrankParams& P, int cus, hipStream_t st) {
  const int L = P.width;
  const int64_t m = P.m, n = P.n, mx = m > n ? m : n;
  Carve cv{static_cast<char*>(P.workspace)};
  uint16_t* dW = cv.take<uint16_t>(m * n);
  uint16_t* dWT = cv.take<uint16_t>(m * n);
  float* Y = cv.take<float>(mx * L);
  const int64_t sm = gemm_splits(m, n, L), sn = gemm_splits(n, m, L);
  float* part = cv.take<float>((sm * m > sn * n ? sm * m : sn * n) * L);
  uint16_t* Q16 = cv.take<uint16_t>((int64_t)L * mx);
  float* Q32 = cv.take<float>(mx * L);
  double* G = cv.take<double>((int64_t)L * L);
  double* V = cv.take<double>((int64_t)L * L);
  double* ev = cv.take<double>(L);
  int* ord = cv.take<int>(L);
  float* T = cv.take<float>((int64_t)L * L);
  double* Gp = cv.take<double>((int64_t)gram_splits(mx, L) * L * L);
  hipError_t err;
  const int64_t grid_cap = (int64_t)cus * 8;
  const size_t apply_lds = (size_t)L * 33 * sizeof(float);  // apply_kernel's T slab

  // Out (M x L fp32) = A (M x K) B^T for B (L x K)
  auto gemm = [&](const uint16_t* A, int64_t M, int64_t K, const uint16_t* B, float* out) -> hipError_t {
    const int s = gemm_splits(M, K, L);
    const int64_t steps = K / kBK;
    const int64_t kslice = ((steps + s - 1) / s) * kBK;
    const dim3 grid((unsigned)((M + kBM - 1) / kBM), (unsigned)((L + kBN - 1) / kBN), (unsigned)s);
    hipLaunchKernelGGL(gemm16_kernel, grid, dim3(kBlock), 0, st, A, B, M, K, L, kslice, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t count = M * L;
    int64_t blocks = (count + kBlock - 1) / kBlock;
    if (blocks > grid_cap) blocks = grid_cap;
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, part, s, count, out);
    return hipGetLastError();
  };
  // G (L x L fp64) = X^T X for X (M x L fp32)
  auto gram = [&](const float* X, int64_t M) -> hipError_t {
    const int gs = gram_splits(M, L);
    const int64_t rs = (((M + gs - 1) / gs + 63) / 64) * 64;
    const int nt = L / 32;
    hipLaunchKernelGGL(gram_kernel, dim3(nt * (nt + 1) / 2, gs), dim3(kBlock), 0, st, X, M, L, rs, Gp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t count = (int64_t)L * L;
    hipLaunchKernelGGL(gram_sum_kernel, dim3((unsigned)((count + 63) / 64)), dim3(kBlock), 0, st, Gp, gs,
                       L, G);
    return hipGetLastError();
  };
  // X (M x L fp32) times T (L x C): apply_small_kernel where L <= 96 and C % 4 == 0 (its
  // 16-byte loads of T stay aligned), else apply_kernel
  auto apply = [&](const float* X, int64_t M, int C, float* o_rm, float* o_t32, uint16_t* o_t16) -> hipError_t {
    const dim3 grid((unsigned)((M + 63) / 64), (unsigned)((C + 31) / 32));
    if (C % 4 == 0 && L <= kLdsWidth) {
      switch (L / kGrid) {
        case 1: hipLaunchKernelGGL(apply_small_kernel<1>, grid, dim3(kBlock), 0, st, X, M, T, C, o_rm, o_t32, o_t16); break;
        case 2: hipLaunchKernelGGL(apply_small_kernel<2>, grid, dim3(kBlock), 0, st, X, M, T, C, o_rm, o_t32, o_t16); break;
        default: hipLaunchKernelGGL(apply_small_kernel<3>, grid, dim3(kBlock), 0, st, X, M, T, C, o_rm, o_t32, o_t16); break;
      }
    } else {
      hipLaunchKernelGGL(apply_kernel, grid, dim3(kBlock), apply_lds, st, X, M, L, T, C, o_rm, o_t32, o_t16);
    }
    return hipGetLastError();
  };
  // out32 (M x L fp32, may be null) and out16 (L x M binary16, transposed, may be null) =
  // X T with T from the Cholesky QR of X (M x L fp32): the Gram-Schmidt basis of X
  auto cholqr = [&](const float* X, int64_t M, float* out32, uint16_t* out16) -> hipError_t {
    hipError_t e = gram(X, M);
    if (e != hipSuccess) return e;
    if (L <= kLdsWidth)
      hipLaunchKernelGGL(chol_inverse_small_kernel, dim3(1), dim3(kGrid * kGrid), 0, st, G, L, T);
    else
      hipLaunchKernelGGL(chol_inverse_kernel, dim3(1), dim3(kCholThreads), 0, st, G, V, L, T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return apply(X, M, L, out32, (float*)nullptr, out16);
  };

  if ((err = launch_residual(P.W, P.packed, P.scale16, P.zero16, m, n, P.nbits, P.group_size, dW,
                             dWT, st)) != hipSuccess)
    return err;
  if ((err = gemm(dW, m, n, P.omega, Y)) != hipSuccess) return err;  // Y = dW Omega
  for (int it = 0; it < P.power_iters; ++it) {
    if ((err = cholqr(Y, m, nullptr, Q16)) != hipSuccess) return err;  // Q16 = basis(Y)^T
    if ((err = gemm(dWT, n, m, Q16, Y)) != hipSuccess) return err;     // Y = dW^T Q  (n x L)
    if ((err = cholqr(Y, n, nullptr, Q16)) != hipSuccess) return err;  // Q16 = basis(Y)^T
    if ((err = gemm(dW, m, n, Q16, Y)) != hipSuccess) return err;      // Y = dW Q    (m x L)
  }
  // Q = orth(Y) by two passes of Cholesky QR: Q1 -> Q32, Q -> Y (fp32) and Q16
  if ((err = cholqr(Y, m, Q32, nullptr)) != hipSuccess) return err;
  if ((err = cholqr(Q32, m, Y, Q16)) != hipSuccess) return err;
  if ((err = gemm(dWT, n, m, Q16, Q32)) != hipSuccess) return err;     // Z = dW^T Q = B_m^T (n x L)
  if ((err = gram(Q32, n)) != hipSuccess) return err;                  // B_m B_m^T = U~ Lambda U~^T
  if (L <= kLdsWidth)
    hipLaunchKernelGGL(syev_kernel<true>, dim3(1), dim3(kSyevThreads), 0, st, G, L, P.rank, V, Gp, ev, ord);
  else
    hipLaunchKernelGGL(syev_kernel<false>, dim3(1), dim3(kSyevThreads), 0, st, G, L, P.rank, V, Gp, ev, ord);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int r = P.rank;
  // B = Q U~_r Sigma_r (m x r);  A = Sigma_r^-1 U~_r^T B_m = (Z U~_r Sigma_r^-1)^T (r x n)
  hipLaunchKernelGGL(transform_kernel, dim3((unsigned)((L * r + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                     V, ev, ord, L, r, 1, T, P.sigma);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = apply(Y, m, r, P.B, (float*)nullptr, (uint16_t*)nullptr)) != hipSuccess) return err;
  hipLaunchKernelGGL(transform_kernel, dim3((unsigned)((L * r + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                     V, ev, ord, L, r, 2, T, (float*)nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return apply(Q32, n, r, (float*)nullptr, P.A, (uint16_t*)nullptr);
}

}  // namespace hqq
