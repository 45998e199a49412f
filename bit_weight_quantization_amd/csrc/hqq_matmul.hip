// hqq_matmul.hip -- gfx950 kernels of the product with a quantized weight,
// Y = X Q^-1(W_q)^T, where Q^-1(W_q) = s (W_q - z) is the inverse quantizer of section 2
// of "Half-Quadratic Quantization of Large Machine Learning Models" (Dropbox tech blog)
// applied to the codes and binary16 s and z that hqq_quantize stores.  The weight is
// N x K (row n holds output n, grouped along the input dimension K); X is M x K
// binary16; accumulation is fp32.
//
// Two kinds of kernel:
//   * few rows of X (decode, M <= 8): per 16 codes (always inside one group) a lane adds
//     s (sum x q - z sum x): the group's scale and zero are applied once per 16 codes and
//     the codes enter as exact small integers.  For 2-, 4- and 8-bit codes the sum x q is
//     taken on packed binary16 pairs with v_dot2_f32_f16 (one to four weight rows per
//     wavefront); 3-bit codes (which straddle bytes) use a wavefront per row and fp32
//     arithmetic.  Bound by HBM reads of the codes.
//   * 9 to 64 rows: a block of eight wavefronts per 16 or 32 weight rows splits K;
//     each lane decodes its codes straight into the B operand of v_mfma_f32_16x16x32_f16
//     (no LDS staging), so every weight is read and dequantized once per call.
//   * more rows (prefill): 128 x 128 output tiles per block of four wavefronts (64 x 64
//     each, 2 x 2 tiles of v_mfma_f32_32x32x16_f16); per 64-wide step of K the block
//     stages the X tile in LDS and dequantizes the weight tile once into LDS as binary16
//     (fp32 s*q - s*z, one rounding, then to binary16), double-buffered, then every
//     wavefront runs its MFMAs from LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "hqq_internal.h"
#include "hqq_matmul.h"

namespace hqq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float h2f(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Code j (0-based, compile-time after unrolling) of an LSB-first string held in words w.
template <int NB, int NW>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[NW], int j) {
  const int bit = NB * j;
  const int wi = bit >> 5, sh = bit & 31;
  constexpr uint32_t mask = (1u << NB) - 1u;
  if (sh + NB <= 32) return (w[wi] >> sh) & mask;
  return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
}

// The 32 codes (32*NB bits, NB words) starting at p (4*NB-byte aligned).
template <int NB>
__device__ __forceinline__ void load_codes32(const uint8_t* p, uint32_t (&w)[NB]) {
  if constexpr (NB == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (NB == 3) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    w[0] = q[0]; w[1] = q[1]; w[2] = q[2];
  } else if constexpr (NB == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0];
    const uint4 b = reinterpret_cast<const uint4*>(p)[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
}

// ------------------------------------------------------------------- GEMV --

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// One wavefront per weight row n (grid-stride over the rows); lane l takes the 32-code
// chunks l, l + 64, ... of the row.  MB >= M rows of X are handled together.
template <int NB, int MB>
__global__ __launch_bounds__(kBlock) void hqq_gemv_kernel(const MatmulParams P) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (kBlock / kWave);
  const int64_t chunks = P.K >> 5;
  const int64_t row_bytes = (P.K >> 3) * NB;
  const int64_t gpr = P.K / P.group_size;
  const int M = (int)P.M;
  for (int64_t n = wave; n < P.N; n += nwaves) {
    float acc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = 0.f;
    const uint8_t* row = P.packed + n * row_bytes;
    for (int64_t c = lane; c < chunks; c += kWave) {
      uint32_t w[NB];
      load_codes32<NB>(row + c * (4 * NB), w);
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // 16 codes lie inside one group (g >= 16)
        const int64_t k0 = c * 32 + 16 * h;
        const int64_t gi = n * gpr + k0 / P.group_size;
        const float s = h2f(P.scale16[gi]);
        const float z = h2f(P.zero16[gi]);
        float q[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) q[j] = (float)code_at<NB>(w, 16 * h + j);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m < M) {
            const uint4* xp = reinterpret_cast<const uint4*>(P.X + m * P.K + k0);
            const uint4 a = xp[0], b = xp[1];
            const uint32_t xw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            float p = 0.f, sx = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const float x = h2f((j & 1) ? (xw[j >> 1] >> 16) : (xw[j >> 1] & 0xffffu));
              p = __builtin_fmaf(x, q[j], p);
              sx += x;
            }
            acc[m] = __builtin_fmaf(s, __builtin_fmaf(-z, sx, p), acc[m]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = wave_sum(acc[m]);
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < M) {
          if (P.out_f32) static_cast<float*>(P.Y)[m * P.N + n] = acc[m];
          else static_cast<_Float16*>(P.Y)[m * P.N + n] = (_Float16)acc[m];
        }
      }
    }
  }
}

// Packed-binary16 form of the codes for the dot products: every 32-bit word is a
// pair of consecutive codes as exact binary16 integers.  A byte of codes is placed
// beside the binary16 exponent byte 0x64 (1024 + mantissa) with one byte permute, the
// other code fields of the byte are masked off, and one packed FMA scales and shifts
// each half to the code itself (1024 + 16 c -> c: exact in binary16).
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

template <int NB>
struct CodePairs {  // the 16 codes of one 16-code block as 8 pairs
  static constexpr int kWords = 16 * NB / 32;
  half2_t q[8];
  __device__ __forceinline__ void from(const uint32_t (&w)[kWords]) {
    constexpr uint32_t kMagic = 0x64646464u;
    if constexpr (NB == 8) {  // one code per byte: bytes 2i, 2i+1
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sel = 0x04000400u | (uint32_t)((2 * i) & 3) | ((uint32_t)((2 * i + 1) & 3) << 16);
        const uint32_t t = __builtin_amdgcn_perm(kMagic, w[i / 2], sel);
        q[i] = as_h2(t) - (half2_t){(_Float16)1024.f, (_Float16)1024.f};
      }
    } else if constexpr (NB == 4) {  // two codes per byte
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t b = (uint32_t)(i & 3);
        const uint32_t t = __builtin_amdgcn_perm(kMagic, w[i / 4], 0x04000400u | b | (b << 16)) &
                           0xFFF0FF0Fu;
        q[i] = __builtin_elementwise_fma(as_h2(t), (half2_t){(_Float16)1.f, (_Float16)0.0625f},
                                         (half2_t){(_Float16)-1024.f, (_Float16)-64.f});
      }
    } else {  // NB == 2: four codes per byte
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t b = (uint32_t)i;
        const uint32_t t = __builtin_amdgcn_perm(kMagic, w[0], 0x04000400u | b | (b << 16));
        q[2 * i] = __builtin_elementwise_fma(as_h2(t & 0xFF0CFF03u),
                                             (half2_t){(_Float16)1.f, (_Float16)0.25f},
                                             (half2_t){(_Float16)-1024.f, (_Float16)-256.f});
        q[2 * i + 1] = __builtin_elementwise_fma(as_h2(t & 0xFFC0FF30u),
                                                 (half2_t){(_Float16)0.0625f, (_Float16)0.015625f},
                                                 (half2_t){(_Float16)-64.f, (_Float16)-16.f});
      }
    }
  }
};

// One wavefront per group of R weight rows.  Lane l takes the 32-code chunks l, l + 64,
// ... of the rows: per chunk it reads 4 NB bytes of codes in each of the R rows and the
// chunk of X once for all R rows; a step covers U chunks per lane (2 for M <= 2, 1 for
// more activation rows, whose X chunks fill the registers), all loaded before any is
// computed.
// Per 16 codes (one group when g = 16, half of one otherwise): p = sum of x*q (packed
// dot products, exact products, fp32 sums) and s (p - z sum x).  The lanes' partial sums
// are added by a butterfly in fixed order.
template <int NB>
__device__ __forceinline__ void load_chunk_codes(const uint8_t* cp, uint32_t (&w)[NB]) {
  static_assert(NB == 2 || NB == 4 || NB == 8, "byte-aligned codes only");
  if constexpr (NB == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(cp);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (NB == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(cp);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    const uint4 v0 = reinterpret_cast<const uint4*>(cp)[0];
    const uint4 v1 = reinterpret_cast<const uint4*>(cp)[1];
    w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
    w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
  }
}

// Everything one chunk step of the GEMV reads: the codes of the chunk in each of the R
// rows, the chunk of each row of X, and the binary16 s and z of the chunk's groups (two
// when g = 16, G16; one otherwise).
template <int NB, int MB, int R, bool G16>
struct GemvStage {
  static constexpr int kGroups = G16 ? 2 : 1;
  uint32_t w[R][NB];
  uint4 x[MB][4];
  uint32_t s[R][kGroups], z[R][kGroups];
};

template <int NB, int MB, int R, bool G16>
__global__ __launch_bounds__(kBlock) void hqq_gemv_packed_kernel(const MatmulParams P) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  const int64_t n0 = wave * R;
  if (n0 >= P.N) return;  // wave-uniform; the kernel has no block-wide barrier
  const int64_t nchunk = P.K >> 5;  // 32-code chunks per row
  if (nchunk == 0) {
    // K = 0: the product is zero
    if (lane == 0) {
      const int nr0 = P.N - n0 < R ? (int)(P.N - n0) : R;
      for (int r = 0; r < nr0; ++r)
        for (int m = 0; m < (int)P.M; ++m) {
          if (P.out_f32) static_cast<float*>(P.Y)[m * P.N + n0 + r] = 0.f;
          else static_cast<_Float16*>(P.Y)[m * P.N + n0 + r] = (_Float16)0.f;
        }
    }
    return;
  }
  const int64_t row_bytes = (P.K >> 3) * NB;
  const int64_t gpr = P.K >> P.group_shift;
  const int M = (int)P.M;
  const int nr = P.N - n0 < R ? (int)(P.N - n0) : R;
  const half2_t kOnes = {(_Float16)1.f, (_Float16)1.f};
  // rows past the end of the weight (or of X) re-read the last valid one; results unused
  const uint8_t* rowp[R];
  const uint16_t* sp[R];
  const uint16_t* zp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t n = n0 + (r < nr ? r : nr - 1);
    rowp[r] = P.packed + n * row_bytes;
    sp[r] = P.scale16 + n * gpr;
    zp[r] = P.zero16 + n * gpr;
  }
  const uint16_t* xrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) xrow[m] = P.X + (int64_t)(m < M ? m : M - 1) * P.K;

  // chunk c's loads (c < nchunk)
  using Stage = GemvStage<NB, MB, R, G16>;
  auto load = [&](Stage& st, int64_t c) {
    const int64_t k0 = c << 5;
#pragma unroll
    for (int r = 0; r < R; ++r) load_chunk_codes<NB>(rowp[r] + c * (4 * NB), st.w[r]);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const uint4* xp = reinterpret_cast<const uint4*>(xrow[m] + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.x[m][i] = xp[i];
    }
    const int64_t g0 = k0 >> P.group_shift;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int g = 0; g < Stage::kGroups; ++g) {
        st.s[r][g] = sp[r][g0 + g];
        st.z[r][g] = zp[r][g0 + g];
      }
    }
  };

  float acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[r][m] = 0.f;

  auto compute = [&](const Stage& cur, bool valid) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // 16-code halves
      uint32_t xw[MB][8];
      float sx[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const uint4 a = cur.x[m][2 * h], b = cur.x[m][2 * h + 1];
        xw[m][0] = a.x; xw[m][1] = a.y; xw[m][2] = a.z; xw[m][3] = a.w;
        xw[m][4] = b.x; xw[m][5] = b.y; xw[m][6] = b.z; xw[m][7] = b.w;
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) t = __builtin_amdgcn_fdot2(as_h2(xw[m][j]), kOnes, t, false);
        sx[m] = t;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t hw[CodePairs<NB>::kWords];
#pragma unroll
        for (int i = 0; i < CodePairs<NB>::kWords; ++i) hw[i] = cur.w[r][h * CodePairs<NB>::kWords + i];
        CodePairs<NB> cq;
        cq.from(hw);
        const int g = G16 ? h : 0;
        const float sv = h2f(cur.s[r][g]);
        const float zv = h2f(cur.z[r][g]);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          float p = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) p = __builtin_amdgcn_fdot2(as_h2(xw[m][j]), cq.q[j], p, false);
          const float v = __builtin_fmaf(sv, __builtin_fmaf(-zv, sx[m], p), acc[r][m]);
          acc[r][m] = valid ? v : acc[r][m];
        }
      }
    }
  };

  // Wave-uniform steps of U x 64 chunks: every load of a step (all its chunks) is issued
  // before any of its arithmetic, behind a scheduling barrier, so a step costs one memory
  // round trip for U chunks per lane.  Loads and arithmetic are
  // unconditional (no divergent branch, so the compiler's waits stay per load): a lane
  // whose chunk is past the end reads the last chunk (all such lanes the same address)
  // and keeps its sums.
  constexpr int U = MB <= 2 ? 2 : 1;
  const int64_t last = nchunk - 1;
  for (int64_t c0 = 0; c0 < nchunk; c0 += U * kWave) {
    Stage st[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kWave + lane;
      load(st[u], c < last ? c : last);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) compute(st[u], c0 + u * kWave + lane < nchunk);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float v = wave_sum(acc[r][m]);
      if (lane == 0 && r < nr && m < M) {
        const int64_t n = n0 + r;
        if (P.out_f32) static_cast<float*>(P.Y)[m * P.N + n] = v;
        else static_cast<_Float16*>(P.Y)[m * P.N + n] = (_Float16)v;
      }
    }
  }
}

template <int NB, int R, bool G16>
void launch_gemv_packed_g(const MatmulParams& P, hipStream_t st) {
  constexpr int kRowsPerBlock = R * (kBlock / kWave);
  const dim3 grid((unsigned)((P.N + kRowsPerBlock - 1) / kRowsPerBlock)), block(kBlock);
  if (P.M <= 1) hipLaunchKernelGGL((hqq_gemv_packed_kernel<NB, 1, R, G16>), grid, block, 0, st, P);
  else if (P.M <= 2) hipLaunchKernelGGL((hqq_gemv_packed_kernel<NB, 2, R, G16>), grid, block, 0, st, P);
  else if (P.M <= 4) hipLaunchKernelGGL((hqq_gemv_packed_kernel<NB, 4, R, G16>), grid, block, 0, st, P);
  else hipLaunchKernelGGL((hqq_gemv_packed_kernel<NB, 8, R, G16>), grid, block, 0, st, P);
}

template <int NB, int R>
hipError_t launch_gemv_packed(const MatmulParams& P, hipStream_t st) {
  if (P.group_size == 16) launch_gemv_packed_g<NB, R, true>(P, st);
  else launch_gemv_packed_g<NB, R, false>(P, st);
  return hipGetLastError();
}

// Block barrier that orders LDS accesses only: __syncthreads() also makes every wavefront
// wait for its outstanding global loads (vmcnt(0)), which would end each prefetch at
// the barrier.  The workgroup fences here are restricted to the LDS address space.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------------- GEMM --

constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 8;  // binary16 per LDS row: 144 bytes (16-byte aligned, rows 4 banks apart)

typedef float float2_t __attribute__((ext_vector_type(2)));

// Dequantize 32 codes of one weight row to binary16: w = s*q - s*z in fp32 (s*z exact,
// one rounding) rounded to binary16 (v_cvt_pk_f16_f32, nearest even).  s0, sz0 for
// codes 0..15 and s1, sz1 for 16..31 (different groups only when g = 16).
template <int NB>
__device__ __forceinline__ void dequant32(const uint32_t (&w)[NB], float s0, float sz0, float s1,
                                          float sz1, uint4 (&out)[4]) {
  uint32_t h[16];
  if constexpr (NB == 3) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float s = j < 8 ? s0 : s1;
      const float sz = j < 8 ? sz0 : sz1;
      const float w0 = __builtin_fmaf(s, (float)code_at<NB>(w, 2 * j), -sz);
      const float w1 = __builtin_fmaf(s, (float)code_at<NB>(w, 2 * j + 1), -sz);
      h[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){w0, w1}, half2_t));
    }
  } else {  // the codes as exact binary16 pairs, converted inside the fp32 FMA (v_fma_mix_f32)
    constexpr int HW = NB / 2;  // words per 16 codes
    CodePairs<NB> cp[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint32_t ws[HW];
#pragma unroll
      for (int i = 0; i < HW; ++i) ws[i] = w[hh * HW + i];
      cp[hh].from(ws);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float s = j < 8 ? s0 : s1;
      const float sz = j < 8 ? sz0 : sz1;
      const half2_t qq = cp[j >> 3].q[j & 7];
      const float w0 = __builtin_fmaf(s, (float)qq[0], -sz);
      const float w1 = __builtin_fmaf(s, (float)qq[1], -sz);
      h[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){w0, w1}, half2_t));
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = make_uint4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);
}

// The 16 codes (16*NB bits) starting at p (2*NB-byte aligned), LSB first in words.
template <int NB>
struct Codes16 {
  static constexpr int kWords = (16 * NB + 31) / 32;
};
template <int NB>
__device__ __forceinline__ void load_codes16(const uint8_t* p, uint32_t (&w)[Codes16<NB>::kWords]) {
  if constexpr (NB == 2) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NB == 3) {  // 6 bytes, 2-byte aligned
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    w[0] = (uint32_t)q[0] | ((uint32_t)q[1] << 16);
    w[1] = q[2];
  } else if constexpr (NB == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
}

// Dequantize 16 codes of one group to binary16, as dequant32 (w = s*q - s*z in fp32, one
// rounding, then binary16).
template <int NB>
__device__ __forceinline__ void dequant16(const uint32_t (&w)[Codes16<NB>::kWords], float s, float sz,
                                          uint4 (&out)[2]) {
  uint32_t h[8];
  if constexpr (NB == 3) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w0 = __builtin_fmaf(s, (float)code_at<NB>(w, 2 * j), -sz);
      const float w1 = __builtin_fmaf(s, (float)code_at<NB>(w, 2 * j + 1), -sz);
      h[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){w0, w1}, half2_t));
    }
  } else {
    CodePairs<NB> cp;
    cp.from(w);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w0 = __builtin_fmaf(s, (float)cp.q[j][0], -sz);
      const float w1 = __builtin_fmaf(s, (float)cp.q[j][1], -sz);
      h[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){w0, w1}, half2_t));
    }
  }
  out[0] = make_uint4(h[0], h[1], h[2], h[3]);
  out[1] = make_uint4(h[4], h[5], h[6], h[7]);
}

// (32 TI WM) x (64 TJ) output tile per block of WM x 2 wavefronts, each (32 TI) x (32 TJ):
// TI x TJ tiles of v_mfma_f32_32x32x16_f16.  K advances in steps of 64: thread t stages
// rows (t + T r) / 2 of both tiles, elements 32 (t % 2) .. + 32 of the step (the X values
// as they are, the weight dequantized to binary16).  LDS is double-buffered: the next
// step's global loads are issued before this step's MFMAs and written to the other buffer
// after them, with one barrier per step.  Larger TI, TJ read fewer LDS operands per MFMA;
// a larger WM dequantizes each weight tile for more rows of X.
template <int NB, int WM, int TI, int TJ>
__global__ __launch_bounds__(2 * WM * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void hqq_gemm_kernel(const MatmulParams P) {
  constexpr int T = 2 * WM * kWave;                 // threads: WM x 2 wavefronts
  constexpr int BM = 32 * TI * WM, BN = 64 * TJ;    // the block's tile
  static_assert(2 * BM == T, "one 32-value item of X per thread and step");
  constexpr int CB = 64 * BN / T;                   // codes per thread and step
  static_assert(CB == 16 || CB == 32, "16 or 32 codes of the weight per thread and step");
  constexpr int BP = 64 / CB;                       // threads per weight row
  constexpr int CW = CB == 32 ? NB : Codes16<NB>::kWords;
  __shared__ __align__(16) _Float16 As[2][BM][kLdsRow];
  __shared__ __align__(16) _Float16 Bs[2][BN][kLdsRow];
  const int tid = threadIdx.x;
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  const int wm = wid >> 1, wn = wid & 1;  // the wavefront's part of the tile
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t row_bytes = (P.K >> 3) * NB;
  const int64_t gpr = P.K >> P.group_shift;
  const int g2 = P.group_size == 16 ? 1 : 0;
  // this thread's items of a step: X row tid / 2, values 32 (tid % 2) ..; weight row
  // tid / BP, codes CB (tid % BP) .. (rows past M or N read the last valid row; values
  // outside the matrices become zeros in LDS)
  const int xr = tid >> 1, xh = tid & 1;
  const int br = tid / BP, bp = tid % BP;
  const uint16_t* xrow = P.X + (m0 + xr < P.M ? m0 + xr : P.M - 1) * P.K;
  const int64_t wrow_n = n0 + br < P.N ? n0 + br : P.N - 1;
  const uint8_t* wrow = P.packed + wrow_n * row_bytes;
  const uint16_t* srow = P.scale16 + wrow_n * gpr;
  const uint16_t* zrow = P.zero16 + wrow_n * gpr;

  // the loader's registers, two steps deep: stage S holds the loads of steps S, S + 2, ..
  uint4 ar[2][4];
  uint32_t cw[2][CW];
  uint32_t s16[2][2], z16[2][2];
  auto load_global = [&](auto st_const, int64_t k0) {
    constexpr int S = decltype(st_const)::value;
    const int64_t ea = k0 + 32 * xh;
    const uint4* xp = reinterpret_cast<const uint4*>(xrow + (ea < P.K ? ea : 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[S][i] = xp[i];
    const int64_t eb0 = k0 + CB * bp;
    const int64_t eb = eb0 < P.K ? eb0 : 0;  // K % 64 == 32: the last step's upper half
    if constexpr (CB == 32) {
      load_codes32<NB>(wrow + (eb >> 5) * (4 * NB), cw[S]);
    } else {
      load_codes16<NB>(wrow + (eb >> 4) * (2 * NB), cw[S]);
    }
    const int64_t g0 = eb >> P.group_shift;
    s16[S][0] = srow[g0];
    z16[S][0] = zrow[g0];
    if constexpr (CB == 32) {
      s16[S][1] = srow[g0 + g2];
      z16[S][1] = zrow[g0 + g2];
    }
  };
  // the weight of step k0 (stage S) as binary16, zeros outside the matrix (s = 0)
  auto dequant_b = [&](auto st_const, int64_t k0, uint4 (&bv)[CB / 8]) {
    constexpr int S = decltype(st_const)::value;
    const bool ok = n0 + br < P.N && k0 + CB * bp < P.K;
    const float s0 = ok ? h2f(s16[S][0]) : 0.f;
    const float sz0 = ok ? s0 * h2f(z16[S][0]) : 0.f;  // s*z exact
    if constexpr (CB == 32) {
      const float s1 = ok ? h2f(s16[S][1]) : 0.f;
      const float sz1 = ok ? s1 * h2f(z16[S][1]) : 0.f;
      dequant32<NB>(cw[S], s0, sz0, s1, sz1, bv);
    } else {
      dequant16<NB>(cw[S], s0, sz0, bv);
    }
  };
  auto write_lds = [&](auto st_const, int buf, int64_t k0, const uint4 (&bv)[CB / 8]) {
    constexpr int S = decltype(st_const)::value;
    const bool ok = k0 + 32 * xh < P.K && m0 + xr < P.M;
    uint4* ad = reinterpret_cast<uint4*>(&As[buf][xr][32 * xh]);
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = ok ? ar[S][i] : make_uint4(0u, 0u, 0u, 0u);
    uint4* bd = reinterpret_cast<uint4*>(&Bs[buf][br][CB * bp]);
#pragma unroll
    for (int i = 0; i < CB / 8; ++i) bd[i] = bv[i];
  };

  float16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto mfma_step = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kk = ks * 16 + (lane >> 5) * 8;
      half8_t af[TI], bf[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(&As[buf][wm * (32 * TI) + i * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(&Bs[buf][wn * (BN / 2) + j * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  // step k0 (LDS buffer S, stage S): prefetch step k0 + 128 into stage S (its step k0 went
  // to LDS one step ago; past the end it re-reads step 0, unused), dequantize step k0 + 64
  // from stage S ^ 1 (loaded one step ago) in the same basic block as this step's MFMAs,
  // so the compiler can interleave them, write it to buffer S ^ 1, barrier
  auto step = [&](auto st_const, int64_t k0) {
    constexpr int S = decltype(st_const)::value;
    constexpr std::integral_constant<int, S ^ 1> other{};
    load_global(st_const, k0 + 2 * kBK < P.K ? k0 + 2 * kBK : 0);
    uint4 bv[CB / 8];
    dequant_b(other, k0 + kBK, bv);
    mfma_step(S);
    write_lds(other, S ^ 1, k0 + kBK, bv);  // (after the last step: unused; unconditional, so
    lds_barrier();                           // the dequantization is not sunk past the MFMAs;
  };                                         // the loads of step k0 + 128 stay in flight)

  if (P.K > 0) {
    constexpr std::integral_constant<int, 0> s0{};
    constexpr std::integral_constant<int, 1> s1{};
    load_global(s0, 0);
    load_global(s1, kBK < P.K ? kBK : 0);
    uint4 bv[CB / 8];
    dequant_b(s0, 0, bv);
    write_lds(s0, 0, 0, bv);
  }
  lds_barrier();
  for (int64_t k0 = 0; k0 < P.K; k0 += 2 * kBK) {
    step(std::integral_constant<int, 0>{}, k0);
    if (k0 + kBK >= P.K) break;
    step(std::integral_constant<int, 1>{}, k0 + kBK);
  }

  // C tile (i, j): lane l, element v holds row 8 (v / 4) + 4 (l / 32) + v % 4, col l % 32
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t n = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * (32 * TI) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < P.M && n < P.N) {
          if (P.out_f32) static_cast<float*>(P.Y)[m * P.N + n] = acc[i][j][v];
          else static_cast<_Float16*>(P.Y)[m * P.N + n] = (_Float16)acc[i][j][v];
        }
      }
    }
  }
}

// ----------------------------------------------------------- skinny GEMM --

typedef float float4_t __attribute__((ext_vector_type(4)));
constexpr int kSkinnyWaves = 8;  // wavefronts per block, splitting K

// Few rows of X (8 < M <= 16 MT), any K (a multiple of 32), any width and group size
// (hqq_skinny_kernel below covers the common aligned cases with fewer memory accesses):
// a block of kSkinnyWaves wavefronts over 16 NW weight
// rows; the wavefronts take consecutive shares of the 256-wide blocks of K and their
// partial tiles are added in LDS in a fixed order.  Lane l = j + 16 kq (j < 16, kq < 4)
// holds, per block at k0, the 64 codes k0 + 64 kq .. + 64 of weight rows n0 + 16 w + j
// (the four lanes of a row read one contiguous 128-byte line at 4 bits) and the same 64
// elements of X rows 16 t + j; the next block's codes, s and z are loaded before this
// block's arithmetic.  MFMA step (h, s) (v_mfma_f32_16x16x32_f16) takes elements
// 32 h + 8 s .. + 8 of every lane's slice: the instruction's k index 8 kq + e stands for
// the real k0 + 64 kq + 32 h + 8 s + e on both operands, so the product is the same sum
// in another order.  The weight enters as binary16 exactly as in the large-M kernel
// (s*q - s*z in fp32, one rounding, then to binary16).  C: lane j + 16 (i / 4), element
// i % 4 holds row i (of the 16 X rows), column j.
template <int NB, int MT, int NW>
__global__ __launch_bounds__(kSkinnyWaves * kWave) void hqq_skinny_general_kernel(const MatmulParams P) {
  __shared__ float red[kSkinnyWaves][MT][NW][4][kWave];
  const int wid = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int j = lane & 15, kq = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * NW;
  const int64_t row_bytes = (P.K >> 3) * NB;
  const int64_t gpr = P.K >> P.group_shift;
  const int g2 = P.group_size == 16 ? 1 : 0;
  const int64_t nblk = (P.K + 255) >> 8;
  const int64_t c0 = wid * nblk / kSkinnyWaves, c1 = (wid + 1) * nblk / kSkinnyWaves;
  float4_t acc[MT][NW];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int w = 0; w < NW; ++w) acc[t][w] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // the weight side of block c: per 32-code half h of the lane's slice, the codes and
  // the raw binary16 s, z of both 16-code halves (s = 0 where nothing is loaded)
  struct Wt {
    uint32_t cw[2][NW][NB];
    uint16_t s16[2][NW][2], z16[2][NW][2];
  };
  auto load_weights = [&](int64_t c, Wt& o) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t kl = (c << 8) + 64 * kq + 32 * h;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int64_t n = n0 + 16 * w + j;
        const bool ok = kl < P.K && n < P.N;
        const int64_t nn = ok ? n : 0, kk = ok ? kl : 0;  // a valid address when unused
        load_codes32<NB>(P.packed + nn * row_bytes + (kk >> 5) * (4 * NB), o.cw[h][w]);
        const int64_t gi = nn * gpr + (kk >> P.group_shift);
        o.s16[h][w][0] = ok ? P.scale16[gi] : (uint16_t)0;
        o.z16[h][w][0] = P.zero16[gi];
        o.s16[h][w][1] = ok ? P.scale16[gi + g2] : (uint16_t)0;
        o.z16[h][w][1] = P.zero16[gi + g2];
      }
    }
  };
  Wt cur, nxt;
  if (c0 < c1) load_weights(c0, nxt);
  for (int64_t c = c0; c < c1; ++c) {
    cur = nxt;
    if (c + 1 < c1) load_weights(c + 1, nxt);  // in flight during this block's arithmetic
    // X rows 16 t + j at the lane's 64 elements (both halves loaded together up to 32
    // rows; 64 rows load each half before its use, registers allowing)
    constexpr int XH = MT <= 2 ? 2 : 1;
    uint4 xa[XH][MT][4];
    auto load_x = [&](int h, uint4 (&xr)[MT][4]) {
      const int64_t kl = (c << 8) + 64 * kq + 32 * h;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int64_t m = 16 * t + j;
        if (kl < P.K && m < P.M) {
          const uint4* xp = reinterpret_cast<const uint4*>(P.X + m * P.K + kl);
#pragma unroll
          for (int i = 0; i < 4; ++i) xr[t][i] = xp[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) xr[t][i] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    };
    if constexpr (XH == 2) {
      load_x(0, xa[0]);
      load_x(1, xa[XH - 1]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float sc[NW][2], sz[NW][2];
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float sv = h2f(cur.s16[h][w][q]);
          sc[w][q] = sv;
          sz[w][q] = sv * h2f(cur.z16[h][w][q]);  // exact
        }
      if constexpr (XH == 1) load_x(h, xa[0]);
      const uint4 (&xr)[MT][4] = xa[XH == 2 ? h : 0];
      // the 32 codes of each row as exact binary16 pairs (byte-aligned widths); 3-bit
      // codes are extracted one by one
      constexpr int HW = NB == 3 ? 1 : NB / 2;  // words per 16 codes
      CodePairs<NB == 3 ? 2 : NB> cpa[NW][2];
      if constexpr (NB != 3) {
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            uint32_t ws[HW];
#pragma unroll
            for (int i = 0; i < HW; ++i) ws[i] = cur.cw[h][w][hh * HW + i];
            cpa[w][hh].from(ws);
          }
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        half8_t bf[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int q = st >> 1;  // codes 16 .. 31 of the half: second group when g = 16
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float c0, c1;
            if constexpr (NB == 3) {
              c0 = (float)code_at<NB>(cur.cw[h][w], 8 * st + e);
              c1 = (float)code_at<NB>(cur.cw[h][w], 8 * st + e + 1);
            } else {
              const half2_t qq = cpa[w][q].q[((8 * st + e) & 15) >> 1];
              c0 = (float)qq[0];
              c1 = (float)qq[1];
            }
            const float w0 = __builtin_fmaf(sc[w][q], c0, -sz[w][q]);
            const float w1 = __builtin_fmaf(sc[w][q], c1, -sz[w][q]);
            const half2_t hv = __builtin_convertvector((float2_t){w0, w1}, half2_t);
            bf[w][e] = hv[0];
            bf[w][e + 1] = hv[1];
          }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const half8_t af = __builtin_bit_cast(half8_t, xr[t][st]);
#pragma unroll
          for (int w = 0; w < NW; ++w)
            acc[t][w] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[w], acc[t][w], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wid][t][w][v][lane] = acc[t][w][v];
  __syncthreads();
  // wavefront wid writes the tiles (t, w) with (t NW + w) % kSkinnyWaves == wid, adding
  // the wavefronts' parts in order
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if ((t * NW + w) % kSkinnyWaves != wid) continue;
      const int64_t n = n0 + 16 * w + j;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float y = red[0][t][w][v][lane];
#pragma unroll
        for (int u = 1; u < kSkinnyWaves; ++u) y += red[u][t][w][v][lane];
        const int64_t m = 16 * t + 4 * kq + v;
        if (m < P.M && n < P.N) {
          if (P.out_f32) static_cast<float*>(P.Y)[m * P.N + n] = y;
          else static_cast<_Float16*>(P.Y)[m * P.N + n] = (_Float16)y;
        }
      }
    }
}

// Few rows of X (8 < M <= 16 MT) for 2-, 4- and 8-bit codes, groups of GS = 5, 6, 7
// (32, 64, 128 weights), K a multiple of 256 and 16-byte aligned s and z: a block of
// kSkinnyWaves2 wavefronts over 16 NW weight rows; the wavefronts take consecutive shares of
// the 256-wide blocks of K and their partial tiles are added in LDS in a fixed order.
// Per block of K (k0) the MFMA steps i = 0..7 (v_mfma_f32_16x16x32_f16) take k0 + 32 i +
// 8 kq .. + 8 in lane j + 16 kq on both operands, the instruction's own k order, so that
// each X load of a step covers 64 contiguous bytes of 16 rows.  The codes of a step are
// NB bytes per lane at a stride of 4 NB; a lane instead loads 8 NB contiguous bytes of its
// row (the codes of steps 2 kq and 2 kq + 1 of all four lanes) and the wavefront
// transposes them through its own LDS buffer (8-bit pieces are loaded in place).  s and
// z of the block's groups come in one load per row.  The next block's codes, s and z are
// loaded before this block's arithmetic; the weight enters the MFMA as in the other
// kernels (s*q - s*z in fp32, one rounding, binary16).  C: lane j + 16 kq, element v
// holds X row 16 t + 4 kq + v, weight row n0 + 16 w + j.
// LDS staging types of the skinny kernel: its buffers are written and read with
// different widths, so every access goes through may_alias types (no type-based alias
// assumption can reorder a read of a staged value before its write)
typedef uint16_t __attribute__((may_alias)) lds_u16;
typedef uint32_t __attribute__((may_alias)) lds_u32;
typedef unsigned int lds_u32x4 __attribute__((ext_vector_type(4), may_alias));

constexpr int kSkinnyWaves2 = 4;  // wavefronts per block of hqq_skinny_kernel, splitting K

template <int NB, int MT, int NW, int GS>
__global__ __launch_bounds__(kSkinnyWaves2 * kWave) void hqq_skinny_kernel(const MatmulParams P) {
  static_assert(NB == 2 || NB == 4 || NB == 8, "byte-aligned widths");
  static_assert(GS >= 5 && GS <= 7, "groups of 32, 64 or 128");
  constexpr bool kStage = NB != 8;        // pieces of NB bytes transposed through LDS
  constexpr int kRowBytes = 32 * NB + 16;  // a row's 4 x 8 pieces, 16 bytes of padding
  constexpr int kStageBytes = kStage ? kSkinnyWaves2 * NW * 16 * kRowBytes : 0;
  // X through LDS (up to 32 rows): per wavefront one block of X, MT tiles of two halves
  // (steps 0-3, 4-7) of 4 slabs, a slab 4 rows x 256 bytes (+16 bytes of padding)
  constexpr bool XS = MT <= 2;
  constexpr int kSlab = 4 * 256 + 16;
  constexpr int kXBytes = XS ? kSkinnyWaves2 * 2 * MT * 4 * kSlab : 0;
  constexpr int kRedBytes = kSkinnyWaves2 * MT * NW * 4 * kWave * 4;
  // the code staging and the X buffers; the reduction at the end reuses the second
  constexpr int kLds1 = kStageBytes > 16 ? kStageBytes : 16;
  constexpr int kLds2 = kXBytes > kRedBytes ? kXBytes : kRedBytes;
  constexpr int kSW = 256 >> GS < 2 ? 1 : (256 >> GS) / 2;  // 32-bit words of s (and z) per block
  constexpr int XD = 4;                                      // steps of X held at once (not XS)
  __shared__ __align__(16) unsigned char lds[kLds1];
  __shared__ __align__(16) unsigned char lds2[kLds2];
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x & (kWave - 1);
  const int j = lane & 15, kq = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * NW;
  const int64_t row_bytes = (P.K >> 3) * NB;
  const int64_t gpr = P.K >> GS;
  const int64_t nblk = P.K >> 8;
  const int64_t c0 = wid * nblk / kSkinnyWaves2, c1 = (wid + 1) * nblk / kSkinnyWaves2;
  // rows past N (or past M for X) read the last valid one; their results are not stored
  int64_t wrow[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int64_t n = n0 + 16 * w + j;
    wrow[w] = n < P.N ? n : P.N - 1;
  }
  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = 16 * t + j;
    xrow[t] = P.X + (m < P.M ? m : P.M - 1) * P.K + 8 * kq;
  }
  float4_t acc[MT][NW];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int w = 0; w < NW; ++w) acc[t][w] = (float4_t){0.f, 0.f, 0.f, 0.f};

  struct Wt {
    uint32_t cw[NW][2 * NB];       // staged: 8 NB bytes of the row from 8 NB kq; else piece i at 2i
    uint32_t sw[NW][kSW], zw[NW][kSW];  // binary16 s, z of the block's groups
  };
  auto load_wt = [&](int64_t c, Wt& o) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint8_t* cp = P.packed + wrow[w] * row_bytes + c * (32 * NB);
      if constexpr (kStage) {
        const uint4* p4 = reinterpret_cast<const uint4*>(cp + 8 * NB * kq);
#pragma unroll
        for (int h = 0; h < NB / 2; ++h) {
          const uint4 v = p4[h];
          o.cw[w][4 * h] = v.x; o.cw[w][4 * h + 1] = v.y; o.cw[w][4 * h + 2] = v.z; o.cw[w][4 * h + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint2 v = *reinterpret_cast<const uint2*>(cp + 32 * i + 8 * kq);
          o.cw[w][2 * i] = v.x; o.cw[w][2 * i + 1] = v.y;
        }
      }
      const int64_t g0 = wrow[w] * gpr + ((c << 8) >> GS);
      const uint16_t* sp = P.scale16 + g0;
      const uint16_t* zp = P.zero16 + g0;
      if constexpr (kSW == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(sp), b = *reinterpret_cast<const uint4*>(zp);
        o.sw[w][0] = a.x; o.sw[w][1] = a.y; o.sw[w][2] = a.z; o.sw[w][3] = a.w;
        o.zw[w][0] = b.x; o.zw[w][1] = b.y; o.zw[w][2] = b.z; o.zw[w][3] = b.w;
      } else if constexpr (kSW == 2) {
        const uint2 a = *reinterpret_cast<const uint2*>(sp), b = *reinterpret_cast<const uint2*>(zp);
        o.sw[w][0] = a.x; o.sw[w][1] = a.y;
        o.zw[w][0] = b.x; o.zw[w][1] = b.y;
      } else {
        o.sw[w][0] = *reinterpret_cast<const uint32_t*>(sp);
        o.zw[w][0] = *reinterpret_cast<const uint32_t*>(zp);
      }
    }
  };
  // the wavefront's LDS rows: [w][row j][kq][step] pieces of NB bytes
  unsigned char* stage = lds + wid * (NW * 16 * kRowBytes);
  // XS: the wavefront's X buffer [half][t][slab]; a slab is 4 rows of X (16 t + 4 n ..)
  // x 256 contiguous bytes (16 granules of 16 bytes) of one half-block, loaded by one
  // instruction: lane 16 r + q takes row r, granule (q + 4 r) % 16, so the 16 lanes of a
  // row read two whole 128-byte lines, and writes it to LDS at 16 (16 r + q); the step
  // reads below (row j, granule 4 s + kq) then fall on 16 different 4-bank groups
  unsigned char* xbuf = lds2 + wid * (2 * MT * 4 * kSlab);
  const int xr = lane >> 4, xg = ((lane & 15) + 4 * xr) & 15;
  lds_u32x4 xs[XS ? MT : 1][8];  // [t][4 half + slab]
  auto load_xs = [&](int64_t c) {
#pragma unroll
    for (int t = 0; t < (XS ? MT : 0); ++t)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int64_t m = 16 * t + 4 * n + xr;
        const uint16_t* g = P.X + (m < P.M ? m : P.M - 1) * P.K + (c << 8) + 8 * xg;
        xs[t][n] = *reinterpret_cast<const lds_u32x4*>(g);
        xs[t][4 + n] = *reinterpret_cast<const lds_u32x4*>(g + 128);
      }
  };
  auto write_xs = [&]() {
#pragma unroll
    for (int t = 0; t < (XS ? MT : 0); ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          *reinterpret_cast<lds_u32x4*>(xbuf + ((h * MT + t) * 4 + n) * kSlab + 16 * lane) = xs[t][4 * h + n];
  };
  auto read_x = [&](int i, int t) -> half8_t {
    const int h = i >> 2, st = i & 3, r = j & 3;
    const int off = ((h * MT + t) * 4 + (j >> 2)) * kSlab + 256 * r + 16 * ((4 * st + kq - 4 * r) & 15);
    return __builtin_bit_cast(half8_t, *reinterpret_cast<const lds_u32x4*>(xbuf + off));
  };

  // one block of K: cur holds its weights, nxt receives the next block's (with X through
  // LDS two Wt sets alternate, so no prefetched register is copied: a copy would wait for
  // the prefetch)
  auto block = [&](int64_t c, const Wt& cur, Wt& nxt) {
    const int64_t k0 = c << 8;
    const int64_t cn = c + 1 < c1 ? c + 1 : c;  // the next block (the last re-reads itself)
    uint4 xa[XD][MT];
    auto load_x = [&](int i) {
#pragma unroll
      for (int t = 0; t < MT; ++t) xa[i % XD][t] = *reinterpret_cast<const uint4*>(xrow[t] + k0 + 32 * i);
    };
    if constexpr (!XS) {
#pragma unroll
      for (int i = 0; i < XD - 1; ++i) load_x(i);
    } else {
      load_xs(cn);  // the next block's X, before its weights: written after this block
      __builtin_amdgcn_sched_barrier(0);  // (the write then waits for these loads only)
    }
    // the next block's weights (unconditional: no branch, so the waits for this block's
    // loads count exactly)
    load_wt(cn, nxt);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t cr[NW][2 * NB];  // piece i of the lane's codes: bytes NB i .. of its 8 NB
    if constexpr (kStage) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        unsigned char* rowp = stage + (w * 16 + j) * kRowBytes;
        // loaded piece (b, q) = bytes (4 b + q) NB of the lane's 8 NB: step 2 kq + b of lane q
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            unsigned char* dst = rowp + q * (8 * NB) + (2 * kq + b) * NB;
            const int e = (4 * b + q) * NB;  // byte offset in cur.cw[w]
            if constexpr (NB == 2)
              *reinterpret_cast<lds_u16*>(dst) = (uint16_t)(cur.cw[w][e >> 2] >> (8 * (e & 3)));
            else
              *reinterpret_cast<lds_u32*>(dst) = cur.cw[w][e >> 2];
          }
      }
      __builtin_amdgcn_wave_barrier();  // LDS accesses of a wavefront execute in order
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const lds_u32x4* src = reinterpret_cast<const lds_u32x4*>(stage + (w * 16 + j) * kRowBytes + kq * (8 * NB));
#pragma unroll
        for (int h = 0; h < NB / 2; ++h) {
          const lds_u32x4 v = src[h];
          cr[w][4 * h] = v.x; cr[w][4 * h + 1] = v.y; cr[w][4 * h + 2] = v.z; cr[w][4 * h + 3] = v.w;
        }
      }
      __builtin_amdgcn_wave_barrier();
    } else {
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int i = 0; i < 2 * NB; ++i) cr[w][i] = cur.cw[w][i];
    }
#pragma unroll
    for (int ip = 0; ip < 4; ++ip) {  // steps 2 ip, 2 ip + 1: 16 codes per row
      half8_t bf[2][NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        CodePairs<NB> cp;
        uint32_t ws[CodePairs<NB>::kWords];
#pragma unroll
        for (int u = 0; u < CodePairs<NB>::kWords; ++u) ws[u] = cr[w][ip * CodePairs<NB>::kWords + u];
        cp.from(ws);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int i = 2 * ip + b;
          const int g = (32 * i) >> GS;  // the step's group within the block
          const float sv = h2f((cur.sw[w][g >> 1] >> (16 * (g & 1))) & 0xffffu);
          const float sz = sv * h2f((cur.zw[w][g >> 1] >> (16 * (g & 1))) & 0xffffu);  // exact
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const half2_t qq = cp.q[4 * b + e];
            const float w0 = __builtin_fmaf(sv, (float)qq[0], -sz);
            const float w1 = __builtin_fmaf(sv, (float)qq[1], -sz);
            const half2_t hv = __builtin_convertvector((float2_t){w0, w1}, half2_t);
            bf[b][w][2 * e] = hv[0];
            bf[b][w][2 * e + 1] = hv[1];
          }
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int i = 2 * ip + b;
        if constexpr (!XS) {
          if (i + XD - 1 < 8) load_x(i + XD - 1);  // XD - 1 steps ahead
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          half8_t af;
          if constexpr (XS) af = read_x(i, t);
          else af = __builtin_bit_cast(half8_t, xa[i % XD][t]);
#pragma unroll
          for (int w = 0; w < NW; ++w)
            acc[t][w] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[b][w], acc[t][w], 0, 0, 0);
        }
      }
    }
    if constexpr (XS) write_xs();  // this block's reads are done (LDS accesses run in order)
  };
  if constexpr (XS) {
    Wt wa, wb;
    if (c0 < c1) {
      load_xs(c0);
      load_wt(c0, wa);
      write_xs();
    }
    for (int64_t c = c0; c < c1; c += 2) {
      block(c, wa, wb);
      if (c + 1 >= c1) break;
      block(c + 1, wb, wa);
    }
  } else {  // 64 rows: the registers allow one copy of the block body only
    Wt cur, nxt;
    if (c0 < c1) load_wt(c0, nxt);
    for (int64_t c = c0; c < c1; ++c) {
      cur = nxt;
      block(c, cur, nxt);
    }
  }
  __syncthreads();  // the X buffers become the reduction buffer
  float* red = reinterpret_cast<float*>(lds2);  // [wave][t][w][v][lane]
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(((wid * MT + t) * NW + w) * 4 + v) * kWave + lane] = acc[t][w][v];
  __syncthreads();
  // wavefront wid writes the tiles (t, w) with (t NW + w) % kSkinnyWaves2 == wid, adding
  // the wavefronts' parts in order
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if ((t * NW + w) % kSkinnyWaves2 != wid) continue;
      const int64_t n = n0 + 16 * w + j;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float y = red[((t * NW + w) * 4 + v) * kWave + lane];
#pragma unroll
        for (int u = 1; u < kSkinnyWaves2; ++u) y += red[(((u * MT + t) * NW + w) * 4 + v) * kWave + lane];
        const int64_t m = 16 * t + 4 * kq + v;
        if (m < P.M && n < P.N) {
          if (P.out_f32) static_cast<float*>(P.Y)[m * P.N + n] = y;
          else static_cast<_Float16*>(P.Y)[m * P.N + n] = (_Float16)y;
        }
      }
    }
}

// ------------------------------------------------------------- split-K GEMM --

// 17 to 64 rows of X (M <= 16 MT) for 2-, 4- and 8-bit codes, groups of GS = 5, 6, 7, K a
// multiple of 256 and 16-byte aligned s and z, with the rows of X shared by the block:
// a block of split_waves<NB>() wavefronts covers 16 NW weight rows per wavefront and one
// contiguous share (split blockIdx.y of `ksplit`) of the 256-wide blocks of K.  Per block
// of K the block loads the block's tile of X (16 MT rows x 256, 16-byte loads, two whole
// 128-byte lines per wavefront and instruction) into LDS once for all its wavefronts, so
// the block's weight rows share one read of X instead of one per wavefront's 16 NW rows
// (measured at M = 64: 2x faster than a kernel whose wavefronts each read their own
// X straight from global memory, whose address unit then stalled).  For 2- and 4-bit
// codes a block is 8 wavefronts of 16 rows (4-8% faster at M = 32-64 than 4 wavefronts of
// 32 rows, same sums); a launch has about 256 blocks, one per CU, so each wavefront may
// use up to 256 registers (two per SIMD); 8-bit codes need more registers for the
// weights and keep 4 wavefronts of 16 NW rows (NW = 2 from 4096 weight rows).
// Double-buffered with one LDS-only barrier per block of K (the weight loads stay in
// flight across it); the next block's X is held in registers during this block's
// arithmetic, and the X fragments of each pair of MFMA steps are read from LDS one pair
// ahead (M = 64 layer 0.264 -> 0.239 ms b2, same sums).  Blocks of 7 wavefronts for the
// 28672-row matrices (256 blocks instead of 224 of 8) were measured no faster: the time
// follows each wavefront's own chain of decode, loads and MFMAs, not the CU count.  Lane j + 16 kq
// takes the 64 consecutive
// codes k0 + 64 kq .. + 64 of each of its weight rows in one load, and MFMA step i
// (v_mfma_f32_16x16x32_f16) gives the instruction's k index 8 kq + e the real
// k0 + 64 kq + 8 i + e on both operands (X read from LDS at that column), so the
// product is the same sum in another order.  The weight enters as in the other kernels
// (s*q - s*z in fp32, one rounding, binary16).  With ksplit = 1 the block writes Y; else
// its fp32 partial tile goes to part[split][m][n] (slabs of `slab` floats) and
// hqq_splitk_reduce_kernel adds the splits in order.  C: lane j + 16 kq, element v holds
// X row 16 t + 4 kq + v, weight row n0 + 16 w + j.
template <int NB>
constexpr int split_waves() { return NB == 8 ? 4 : 8; }  // wavefronts per block, each its own weight rows
// Register sets of X and weights per wavefront: the block of K it works on and the next
// one in flight.  (Deeper rings, 3-5 sets with the loads issued 2-4 blocks ahead, were
// measured no faster at M = 32 and 64: the loop is not waiting on HBM.)
template <int NB>
constexpr int split_prefetch() { return 2; }

// f(integral_constant<int, i>) for i = 0 .. N - 1, unrolled at compile time.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}
constexpr int kXRowBytes = 512 + 16;       // a row of X per block of K in LDS (+16: rows 4 banks apart)

template <int NB, int MT, int NW, int GS, int PD>
__global__ __launch_bounds__(split_waves<NB>() * kWave, NB == 8 ? 1 : 2) void hqq_splitk_kernel(const MatmulParams P) {
  static_assert(NB == 2 || NB == 4 || NB == 8, "byte-aligned widths");
  static_assert(GS >= 5 && GS <= 7, "groups of 32, 64 or 128");
  constexpr int kSplitWaves = split_waves<NB>();
  constexpr int XR = 16 * MT;                    // rows of X
  constexpr int kXRows = kSplitWaves * kWave / 32;  // rows of X per round of 16-byte loads
  constexpr int kRounds = XR / kXRows;           // 16-byte loads per thread per block of K
  constexpr int kCW = 2 * NB;                    // code words per lane and weight row (64 codes)
  constexpr int kSZ = GS == 5 ? 2 : 1;           // groups per lane and weight row
  __shared__ __align__(16) unsigned char xs[2][XR * kXRowBytes];
  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid & (kWave - 1);
  const int j = lane & 15, kq = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * (kSplitWaves * 16 * NW) + wid * (16 * NW);
  const int ksplit = P.ksplit;
  const int64_t nkb = P.K >> 8;
  const int64_t kb0 = blockIdx.y * nkb / ksplit, kb1 = (blockIdx.y + 1) * nkb / ksplit;
  const int64_t row_bytes = (P.K >> 3) * NB;
  const int64_t gpr = P.K >> GS;
  // weight rows past N read the last one; their results are not stored
  const uint8_t* cbase[NW];
  const uint16_t* sbase[NW];
  const uint16_t* zbase[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int64_t n = n0 + 16 * w + j;
    const int64_t nn = n < P.N ? n : P.N - 1;
    cbase[w] = P.packed + nn * row_bytes + kq * (8 * NB);
    sbase[w] = P.scale16 + nn * gpr + ((64 * kq) >> GS);
    zbase[w] = P.zero16 + nn * gpr + ((64 * kq) >> GS);
  }
  // the thread's share of a block's X tile: rows kXRows r + tid / 32, 16-byte granule
  // tid % 32.  In LDS a row holds its four 128-byte quarters (the columns of kq = 0..3) in
  // the order 0, 2, 1, 3: a 16-byte LDS read serves its lanes in pairs of 8-lane groups,
  // {0-7, 24-31}, {8-15, 16-23} and the same in the upper half (measured on gfx950 with a
  // bank probe), and in natural order lanes j and j + 8 of the next kq land on the same
  // banks of the 64; in this order every pair covers all 64 banks once (no conflicts,
  // against 2-way before: 0.270 -> 0.266 ms per layer at M = 64, b2)
  const int xrow0 = tid >> 5, xg = tid & 31;
  const int xpos = (((xg >> 3) & 1) << 4) | ((xg >> 4) << 3) | (xg & 7);  // quarter order 0, 2, 1, 3
  const int kqp = ((kq & 1) << 1) | (kq >> 1);
  const uint16_t* xsrc[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t m = kXRows * r + xrow0;
    xsrc[r] = P.X + (m < P.M ? m : P.M - 1) * P.K + 8 * xg;
  }
  float4_t acc[MT][NW];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int w = 0; w < NW; ++w) acc[t][w] = (float4_t){0.f, 0.f, 0.f, 0.f};

  struct Wt {
    uint32_t cw[NW][kCW];                  // the lane's 64 codes of each weight row
    uint32_t sz[NW];                       // binary16 s (GS = 5: two, one per group)
    uint32_t zz[NW];                       // binary16 z
  };
  auto load_wt = [&](int64_t c, Wt& o) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint4* cp = reinterpret_cast<const uint4*>(cbase[w] + c * (32 * NB));
#pragma unroll
      for (int h = 0; h < kCW / 4; ++h) {
        const uint4 v = cp[h];
        o.cw[w][4 * h] = v.x; o.cw[w][4 * h + 1] = v.y; o.cw[w][4 * h + 2] = v.z; o.cw[w][4 * h + 3] = v.w;
      }
      const int64_t g = (c << 8) >> GS;  // first group of the block of K in the row
      if constexpr (kSZ == 2) {
        o.sz[w] = *reinterpret_cast<const uint32_t*>(sbase[w] + g);
        o.zz[w] = *reinterpret_cast<const uint32_t*>(zbase[w] + g);
      } else {
        o.sz[w] = sbase[w][g];
        o.zz[w] = zbase[w][g];
      }
    }
  };
  // X and weights of PD - 1 blocks of K in flight, in register rings of PD sets (slot =
  // block index within the split mod PD); X goes to LDS one block ahead
  lds_u32x4 xr[PD][kRounds];
  Wt wr[PD];
  auto load_x = [&](int64_t c, lds_u32x4 (&o)[kRounds]) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) o[r] = *reinterpret_cast<const lds_u32x4*>(xsrc[r] + (c << 8));
  };
  auto write_x = [&](int buf, const lds_u32x4 (&o)[kRounds]) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r)
      *reinterpret_cast<lds_u32x4*>(&xs[buf][(kXRows * r + xrow0) * kXRowBytes + 16 * xpos]) = o[r];
  };

  // block c of the split (slot I = its index mod PD, LDS buffer B = its index mod 2):
  // first the loads of block c + PD - 1 into slot (I + PD - 1) mod PD (its previous
  // block was read by block c - 1; LOAD = 0: none, 1: always, 2: if inside the split),
  // then the arithmetic of block c from LDS and slot I, then X of block c + 1 into the
  // other LDS buffer (every wavefront finished reading it before the last barrier)
  auto block = [&](auto i_const, auto load_const, int64_t c) {
    constexpr int I = decltype(i_const)::value % PD;
    constexpr int buf = decltype(i_const)::value & 1;
    constexpr int LOAD = decltype(load_const)::value;
    constexpr int IN = (I + PD - 1) % PD;
    if constexpr (LOAD == 1) {
      load_x(c + PD - 1, xr[IN]);
      load_wt(c + PD - 1, wr[IN]);
    } else if constexpr (LOAD == 2) {
      if (c + PD - 1 < kb1) {
        load_x(c + PD - 1, xr[IN]);
        load_wt(c + PD - 1, wr[IN]);
      }
    }
    const Wt& cur = wr[I];
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char* xb = xs[buf] + j * kXRowBytes + 128 * kqp;
    auto read_af = [&](int i, int t) -> half8_t {
      return __builtin_bit_cast(half8_t, *reinterpret_cast<const lds_u32x4*>(xb + (16 * t) * kXRowBytes + 16 * i));
    };
    // the X fragments of the step pair ip + 1 are read while ip's codes are decoded and
    // multiplied (each MFMA otherwise waited on the LDS read issued just before it)
    half8_t afs[2][2][MT];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < MT; ++t) afs[0][b][t] = read_af(b, t);
#pragma unroll
    for (int ip = 0; ip < 4; ++ip) {  // steps 2 ip, 2 ip + 1: 16 codes per row
      if (ip + 1 < 4) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int t = 0; t < MT; ++t) afs[(ip + 1) & 1][b][t] = read_af(2 * (ip + 1) + b, t);
      }
      half8_t bf[2][NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        CodePairs<NB> cp;
        uint32_t ws[CodePairs<NB>::kWords];
#pragma unroll
        for (int u = 0; u < CodePairs<NB>::kWords; ++u) ws[u] = cur.cw[w][ip * CodePairs<NB>::kWords + u];
        cp.from(ws);
        // codes 16 ip .. + 16 of the lane's 64: one group (GS = 5: group ip / 2)
        const int hs = kSZ == 2 ? 16 * (ip >> 1) : 0;
        const float sv = h2f((cur.sz[w] >> hs) & 0xffffu);
        const float sz = sv * h2f((cur.zz[w] >> hs) & 0xffffu);  // exact
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const half2_t qq = cp.q[4 * b + e];
            const float w0 = __builtin_fmaf(sv, (float)qq[0], -sz);
            const float w1 = __builtin_fmaf(sv, (float)qq[1], -sz);
            const half2_t hv = __builtin_convertvector((float2_t){w0, w1}, half2_t);
            bf[b][w][2 * e] = hv[0];
            bf[b][w][2 * e + 1] = hv[1];
          }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const half8_t af = afs[ip & 1][b][t];
#pragma unroll
          for (int w = 0; w < NW; ++w)
            acc[t][w] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[b][w], acc[t][w], 0, 0, 0);
        }
      }
    }
    if (LOAD == 1 || c + 1 < kb1) {
      write_x(buf ^ 1, xr[(I + 1) % PD]);
      lds_barrier();
    }
  };
  // U = lcm(PD, 2) blocks per round of the loop, whose loads all lie inside the split
  // (unconditional: their waits count exactly); the last up to U + PD - 2 blocks after it
  constexpr int U = PD % 2 == 0 ? PD : 2 * PD;
  if (kb0 < kb1) {
#pragma unroll
    for (int p = 0; p + 1 < PD; ++p) {
      if (kb0 + p < kb1) {
        load_x(kb0 + p, xr[p]);
        load_wt(kb0 + p, wr[p]);
      }
    }
    write_x(0, xr[0]);
    lds_barrier();
    int64_t c = kb0;
    for (; c + U + PD - 2 < kb1; c += U) {
      static_for<U>([&](auto i) { block(i, std::integral_constant<int, 1>{}, c + i); });
    }
    static_for<U + PD - 2>([&](auto i) {
      if (c + i < kb1) block(i, std::integral_constant<int, 2>{}, c + i);
    });
  }
  // the wavefront's tile: Y directly (one split) or the split's partial slab
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int64_t n = n0 + 16 * w + j;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = 16 * t + 4 * kq + v;
        if (m < P.M && n < P.N) {
          const float y = acc[t][w][v];
          if (ksplit > 1) P.part[blockIdx.y * P.slab + m * P.N + n] = y;
          else if (P.out_f32) static_cast<float*>(P.Y)[m * P.N + n] = y;
          else static_cast<_Float16*>(P.Y)[m * P.N + n] = (_Float16)y;
        }
      }
    }
}

// Y = the sum of the ksplit partial slabs in split order (fp32), 4 elements per thread;
// binary16 output is the nearest-even rounding of that sum.
__global__ __launch_bounds__(kBlock) void hqq_splitk_reduce_kernel(const MatmulParams P) {
  const int64_t mn = P.M * P.N;
  const int64_t stride = (int64_t)gridDim.x * kBlock * 4;
  for (int64_t i = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4; i < mn; i += stride) {
    const float* src = P.part + i;
    float4_t y = *reinterpret_cast<const float4_t*>(src);
    int k = 1;
    for (; k + 8 <= P.ksplit; k += 8) {  // eight loads in flight, added in split order
      float4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4_t*>(src + (k + u) * P.slab);
#pragma unroll
      for (int u = 0; u < 8; ++u) y += v[u];
    }
    for (; k < P.ksplit; ++k) y += *reinterpret_cast<const float4_t*>(src + k * P.slab);
    const int n = mn - i < 4 ? (int)(mn - i) : 4;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v < n) {
        if (P.out_f32) static_cast<float*>(P.Y)[i + v] = y[v];
        else static_cast<_Float16*>(P.Y)[i + v] = (_Float16)y[v];
      }
    }
  }
}

// The aligned skinny kernel applies: byte-aligned codes, groups of 32-128, K a multiple
// of 256, 16-byte aligned s and z.
bool skinny_aligned(const MatmulParams& P) {
  const bool aligned16 = ((reinterpret_cast<uintptr_t>(P.scale16) | reinterpret_cast<uintptr_t>(P.zero16)) & 15) == 0;
  return P.nbits != 3 && P.K % 256 == 0 && aligned16 && P.group_shift >= 5 && P.group_shift <= 7;
}

// Split-K geometry of the aligned skinny path, from the shapes and the code width alone
// (results do not depend on the device): 16 NW weight rows per wavefront (NW = 2 only for
// 8-bit codes from 4096 rows), and K split so that a launch has about kSplitTargetWaves
// wavefronts where K allows (two per SIMD; with 8-wavefront blocks, 4096 split the
// 28672-row matrices in two and were 1-4% slower at M = 32-64 than no split there).
constexpr int kSplitTargetWaves = 2048;
struct SplitGeom {
  int waves, nw, ksplit;
  int64_t row_blocks;
};
SplitGeom split_geometry(int64_t N, int64_t K, int nbits) {
  SplitGeom g;
  g.waves = nbits == 8 ? split_waves<8>() : split_waves<2>();
  g.nw = nbits == 8 && N >= 4096 ? 2 : 1;
  const int64_t rows = (int64_t)g.waves * 16 * g.nw;
  g.row_blocks = (N + rows - 1) / rows;
  const int64_t target = kSplitTargetWaves / g.waves;  // blocks
  int64_t ks = (target + g.row_blocks / 2) / g.row_blocks;
  const int64_t nkb = K >> 8;
  if (ks > nkb) ks = nkb;
  g.ksplit = ks < 1 ? 1 : (int)ks;
  return g;
}

// The split-K path applies (s and z alignment aside, checked at the call): 17 to 64 rows
// of X (up to 16 the aligned skinny kernel, which needs no workspace, is as fast).
bool splitk_shapes(int64_t M, int64_t K, int nbits, int group_size) {
  return nbits != 3 && K % 256 == 0 && group_size >= 32 && group_size <= 128 &&
         M > kSplitMinRows && M <= kSkinnyMaxRows;
}

template <int NB, int MT, int NW>
void launch_splitk_nw(const MatmulParams& P, dim3 grid, hipStream_t st) {
  const dim3 block(split_waves<NB>() * kWave);
  constexpr int PD = split_prefetch<NB>();
  switch (P.group_shift) {
    case 5: hipLaunchKernelGGL((hqq_splitk_kernel<NB, MT, NW, 5, PD>), grid, block, 0, st, P); return;
    case 6: hipLaunchKernelGGL((hqq_splitk_kernel<NB, MT, NW, 6, PD>), grid, block, 0, st, P); return;
    default: hipLaunchKernelGGL((hqq_splitk_kernel<NB, MT, NW, 7, PD>), grid, block, 0, st, P); return;
  }
}

template <int NB, int MT>
void launch_splitk(MatmulParams P, hipStream_t st) {
  const SplitGeom g = split_geometry(P.N, P.K, NB);
  P.ksplit = g.ksplit;
  P.slab = (P.M * P.N + 3) & ~(int64_t)3;
  const dim3 grid((unsigned)g.row_blocks, (unsigned)g.ksplit);
  if constexpr (NB == 8) {
    if (g.nw == 2) {
      launch_splitk_nw<NB, MT, 2>(P, grid, st);
    } else {
      launch_splitk_nw<NB, MT, 1>(P, grid, st);
    }
  } else {
    launch_splitk_nw<NB, MT, 1>(P, grid, st);
  }
  if (g.ksplit > 1) {
    int64_t blocks = (P.M * P.N + 4 * kBlock - 1) / (4 * kBlock);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(hqq_splitk_reduce_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, P);
  }
}

template <int NB, int MT, int NW>
void launch_skinny_nw(const MatmulParams& P, dim3 grid, hipStream_t st) {
  const dim3 block(kSkinnyWaves * kWave), block2(kSkinnyWaves2 * kWave);
  if constexpr (NB != 3) {
    if (skinny_aligned(P)) {
      switch (P.group_shift) {
        case 5: hipLaunchKernelGGL((hqq_skinny_kernel<NB, MT, NW, 5>), grid, block2, 0, st, P); return;
        case 6: hipLaunchKernelGGL((hqq_skinny_kernel<NB, MT, NW, 6>), grid, block2, 0, st, P); return;
        default: hipLaunchKernelGGL((hqq_skinny_kernel<NB, MT, NW, 7>), grid, block2, 0, st, P); return;
      }
    }
  }
  hipLaunchKernelGGL((hqq_skinny_general_kernel<NB, MT, NW>), grid, block, 0, st, P);
}

template <int NB, int MT>
void launch_skinny(const MatmulParams& P, hipStream_t st) {
  if (P.N >= 4096)  // 32 weight rows per block where there are enough rows
    launch_skinny_nw<NB, MT, 2>(P, dim3((unsigned)((P.N + 31) / 32)), st);
  else
    launch_skinny_nw<NB, MT, 1>(P, dim3((unsigned)((P.N + 15) / 16)), st);
}

template <int NB>
hipError_t launch_nb(const MatmulParams& P, int cus, hipStream_t st) {
  // the aligned skinny kernel costs about the same for 3-16 rows as the per-row one for 3
  const int64_t gemv_max = skinny_aligned(P) ? kGemvAlignedMaxRows : kGemvMaxRows;
  if constexpr (NB != 3) {  // packed binary16 codes (3-bit codes straddle bytes)
    if (P.M <= gemv_max) {
      // rows per wavefront: enough wavefronts to fill the chip (>= 2048) with as many
      // rows sharing each chunk of X as that allows
      if (P.N >= 8192) return launch_gemv_packed<NB, 4>(P, st);
      if (P.N >= 4096) return launch_gemv_packed<NB, 2>(P, st);
      return launch_gemv_packed<NB, 1>(P, st);
    }
  }
  if constexpr (NB != 3) {
    if (skinny_aligned(P) && splitk_shapes(P.M, P.K, NB, P.group_size)) {
      if (P.M <= 32) launch_splitk<NB, 2>(P, st);
      else launch_splitk<NB, 4>(P, st);
      return hipGetLastError();
    }
  }
  if (P.M > gemv_max && P.M <= kSkinnyMaxRows) {
    if (P.M <= 16) launch_skinny<NB, 1>(P, st);
    else if (P.M <= 32) launch_skinny<NB, 2>(P, st);
    else launch_skinny<NB, 4>(P, st);
    return hipGetLastError();
  }
  if (P.M <= kGemvMaxRows) {
    int64_t blocks = (P.N + kBlock / kWave - 1) / (kBlock / kWave);  // a wavefront per row
    const int64_t cap = (int64_t)cus * 32;
    if (blocks > cap) blocks = cap;
    const dim3 grid((unsigned)blocks), block(kBlock);
    if (P.M <= 1) hipLaunchKernelGGL((hqq_gemv_kernel<NB, 1>), grid, block, 0, st, P);
    else if (P.M <= 2) hipLaunchKernelGGL((hqq_gemv_kernel<NB, 2>), grid, block, 0, st, P);
    else if (P.M <= 4) hipLaunchKernelGGL((hqq_gemv_kernel<NB, 4>), grid, block, 0, st, P);
    else hipLaunchKernelGGL((hqq_gemv_kernel<NB, 8>), grid, block, 0, st, P);
  } else {
    // 256 x 128 tiles of 8 wavefronts from 512 rows (each weight tile is dequantized once
    // per 256 rows of X: half the decode per MFMA of 128 x 128 tiles), else 128 x 128 (4
    // wavefronts: twice the blocks for a few hundred rows); both 64 x 64 per wavefront, 2
    // wavefronts per SIMD
    if (P.M >= 512) {
      const dim3 grid((unsigned)((P.N + 127) / 128), (unsigned)((P.M + 255) / 256));
      hipLaunchKernelGGL((hqq_gemm_kernel<NB, 4, 2, 2>), grid, dim3(8 * kWave), 0, st, P);
    } else {
      const dim3 grid((unsigned)((P.N + 127) / 128), (unsigned)((P.M + 127) / 128));
      hipLaunchKernelGGL((hqq_gemm_kernel<NB, 2, 2, 2>), grid, dim3(4 * kWave), 0, st, P);
    }
  }
  return hipGetLastError();
}

}  // namespace

int64_t matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, int nbits, int group_size) {
  if (!splitk_shapes(M, K, nbits, group_size) || N <= 0) return 0;
  const SplitGeom g = split_geometry(N, K, nbits);
  if (g.ksplit <= 1) return 0;
  return (int64_t)g.ksplit * ((M * N + 3) & ~(int64_t)3) * (int64_t)sizeof(float);
}

hipError_t launch_matmul(MatmulParams prm, int cus, hipStream_t stream) {
  prm.ksplit = 1;
  prm.slab = 0;
  switch (prm.nbits) {
    case 2: return launch_nb<2>(prm, cus, stream);
    case 3: return launch_nb<3>(prm, cus, stream);
    case 4: return launch_nb<4>(prm, cus, stream);
    case 8: return launch_nb<8>(prm, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hqq
