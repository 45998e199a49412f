// hqq_meta.hip -- gfx950 kernels of the 8-bit meta quantization of the per-group s
// and z arrays.
//
// Method: "Half-Quadratic Quantization of Large Machine Learning Models" (Dropbox
// tech blog), section 4.1: the zero-points are stored in 8 bits without grouping or
// optimization; the note under its Llama-2 table also quantizes the scales to 8 bits
// in groups of 128.  Here: affine min-max round-to-nearest over the stored binary16
// values (no solver), groups of M consecutive values (M = 0: one group of all n
// values; the last group may be shorter):
//   mn, mx over the group; d = mx - mn;
//   code = clamp(rint(binary32(((v - mn) * 255) / d)), 0, 255)  (fp64 quotient,
//          rounded once to binary32, then half-even: the weight codes' precision);
//   meta scale = binary16(d / 255) (RNE from fp64), meta offset = mn (a zero minimum
//   as +0); a constant group has codes 0 and meta scale 1.
// The quotient is computed in fp64 exactly as defined (v - mn and the product are
// exact, the division is IEEE), so codes are bit-identical to that definition.
//
// Layout: values, codes, scales and offsets are flat arrays; lanes read and write
// consecutive elements (2-byte loads, 1-byte stores, coalesced per wavefront).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqq_internal.h"

namespace hqq {
namespace {

constexpr int kMetaBlock = 256;

__device__ __forceinline__ uint32_t uniform32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64m(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double half_to_double(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}

// Order-preserving 32-bit key of a finite binary16 (NaN excluded): negative values
// map below 0x8000 in reverse order, non-negative ones to 0x8000 + bits.
__device__ __forceinline__ uint32_t key_of(uint16_t h) {
  return (h & 0x8000u) ? (~(uint32_t)h & 0xffffu) : ((uint32_t)h | 0x8000u);
}
__device__ __forceinline__ uint16_t half_of_key(uint32_t k) {
  return (k & 0x8000u) ? (uint16_t)(k & 0x7fffu) : (uint16_t)(~k & 0xffffu);
}

// binary16 nearest-even of an fp64 value in the binary16 normal range: round to
// binary32 with round-to-odd (truncate toward zero, set the last bit if inexact),
// then round that to binary16 (24 >= 11 + 2 bits make the two steps one rounding).
__device__ __forceinline__ uint16_t f64_to_f16(double x) {
  float f = (float)x;
  const double back = (double)f;
  if (back != x) {
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    if (__builtin_fabs(back) > __builtin_fabs(x)) b -= 1u;  // toward zero
    b |= 1u;
    f = __builtin_bit_cast(float, b);
  }
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ uint8_t meta_code(uint16_t h, double mn, double d) {
  if (!(d > 0.0)) return 0;
  const double u = ((half_to_double(h) - mn) * 255.0) / d;
  const float q = __builtin_amdgcn_fmed3f(__builtin_rintf((float)u), 0.f, 255.f);
  return (uint8_t)q;
}

// Wave-wide min and max of the keys (every lane ends with the result).
__device__ __forceinline__ void wave_minmax(uint32_t& kmin, uint32_t& kmax) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t a = (uint32_t)__shfl_xor((int)kmin, off, 64);
    const uint32_t b = (uint32_t)__shfl_xor((int)kmax, off, 64);
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
}

// Meta scale and offset of a group from its min and max keys.
__device__ __forceinline__ void meta_params(uint32_t kmin, uint32_t kmax, double& mn, double& d,
                                            uint16_t& scale16, uint16_t& offset16) {
  uint16_t hmn = half_of_key(kmin);
  if ((hmn & 0x7fffu) == 0) hmn = 0;  // a zero minimum is stored as +0
  mn = half_to_double(hmn);
  d = half_to_double(half_of_key(kmax)) - mn;  // exact in fp64
  scale16 = f64_to_f16(d > 0.0 ? d / 255.0 : 1.0);
  offset16 = hmn;
}

// One wavefront per group of M values.
__global__ __launch_bounds__(kMetaBlock) void meta_grouped_kernel(const uint16_t* __restrict__ v,
                                                                  int64_t n, int64_t M,
                                                                  int64_t ngroups,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint16_t* __restrict__ mscale,
                                                                  uint16_t* __restrict__ moffset) {
  const int lane = threadIdx.x & 63;
  const int64_t grp = uniform64m(((int64_t)blockIdx.x * kMetaBlock + threadIdx.x) / 64);
  if (grp >= ngroups) return;
  const int64_t g0 = grp * M;
  const int64_t g1 = g0 + M < n ? g0 + M : n;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int64_t i = g0 + lane; i < g1; i += 64) {
    const uint32_t k = key_of(v[i]);
    kmin = k < kmin ? k : kmin;
    kmax = k > kmax ? k : kmax;
  }
  wave_minmax(kmin, kmax);
  double mn, d;
  uint16_t s16, o16;
  meta_params(uniform32(kmin), uniform32(kmax), mn, d, s16, o16);
  for (int64_t i = g0 + lane; i < g1; i += 64) codes[i] = meta_code(v[i], mn, d);
  if (lane == 0) {
    mscale[grp] = s16;
    moffset[grp] = o16;
  }
}

// Whole array: the workspace holds the min and max keys.
__global__ void meta_init_kernel(uint32_t* ws) {
  if (threadIdx.x == 0) {
    ws[0] = 0xffffffffu;
    ws[1] = 0u;
  }
}

__global__ __launch_bounds__(kMetaBlock) void meta_reduce_kernel(const uint16_t* __restrict__ v,
                                                                 int64_t n, uint32_t* ws) {
  const int64_t stride = (int64_t)gridDim.x * kMetaBlock;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int64_t i = (int64_t)blockIdx.x * kMetaBlock + threadIdx.x; i < n; i += stride) {
    const uint32_t k = key_of(v[i]);
    kmin = k < kmin ? k : kmin;
    kmax = k > kmax ? k : kmax;
  }
  wave_minmax(kmin, kmax);
  if ((threadIdx.x & 63) == 0) {
    atomicMin(&ws[0], kmin);
    atomicMax(&ws[1], kmax);
  }
}

__global__ __launch_bounds__(kMetaBlock) void meta_quant_all_kernel(
    const uint16_t* __restrict__ v, int64_t n, const uint32_t* ws, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ mscale, uint16_t* __restrict__ moffset) {
  double mn, d;
  uint16_t s16, o16;
  meta_params(ws[0], ws[1], mn, d, s16, o16);
  const int64_t stride = (int64_t)gridDim.x * kMetaBlock;
  for (int64_t i = (int64_t)blockIdx.x * kMetaBlock + threadIdx.x; i < n; i += stride)
    codes[i] = meta_code(v[i], mn, d);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    mscale[0] = s16;
    moffset[0] = o16;
  }
}

// offset + scale * code rounded once to binary16: s * c is exact in fp32 (11 x 8 bits);
// TwoSum gives the exact sum as hi + lo; round-to-odd on hi makes the final
// fp32 -> fp16 conversion a single rounding of the exact value.
__device__ __forceinline__ uint16_t meta_value(float s, float o, uint32_t c) {
  const float a = s * (float)c;
  const float hi = a + o;
  const float bb = hi - a;
  const float lo = (a - (hi - bb)) + (o - bb);
  uint32_t bits = __builtin_bit_cast(uint32_t, hi);
  if (lo != 0.f) {
    if ((lo > 0.f) != (hi > 0.f)) bits -= 1u;
    bits |= 1u;
  }
  return __builtin_bit_cast(uint16_t, (_Float16)__builtin_bit_cast(float, bits));
}

__global__ __launch_bounds__(kMetaBlock) void meta_dequant_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ mscale,
    const uint16_t* __restrict__ moffset, int64_t n, int64_t M, uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kMetaBlock;
  for (int64_t i = (int64_t)blockIdx.x * kMetaBlock + threadIdx.x; i < n; i += stride) {
    const int64_t g = M == 0 ? 0 : i / M;
    const float s = (float)__builtin_bit_cast(_Float16, mscale[g]);
    const float o = (float)__builtin_bit_cast(_Float16, moffset[g]);
    out[i] = meta_value(s, o, codes[i]);
  }
}

int64_t grid_for(int64_t n, int cus) {
  int64_t blocks = (n + kMetaBlock - 1) / kMetaBlock;
  const int64_t cap = (int64_t)cus * 16;
  return blocks < cap ? blocks : cap;
}

}  // namespace

hipError_t launch_meta_quantize(const uint16_t* values, int64_t n, int64_t M, uint8_t* codes,
                                uint16_t* mscale, uint16_t* moffset, uint32_t* workspace,
                                int cus, hipStream_t st) {
  if (M == 0) {
    const int64_t blocks = grid_for(n, cus);
    hipLaunchKernelGGL(meta_init_kernel, dim3(1), dim3(64), 0, st, workspace);
    hipLaunchKernelGGL(meta_reduce_kernel, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st, values,
                       n, workspace);
    hipLaunchKernelGGL(meta_quant_all_kernel, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st,
                       values, n, workspace, codes, mscale, moffset);
    return hipGetLastError();
  }
  const int64_t ngroups = (n + M - 1) / M;
  const int64_t blocks = (ngroups + kMetaBlock / 64 - 1) / (kMetaBlock / 64);
  hipLaunchKernelGGL(meta_grouped_kernel, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st, values,
                     n, M, ngroups, codes, mscale, moffset);
  return hipGetLastError();
}

hipError_t launch_meta_dequantize(const uint8_t* codes, const uint16_t* mscale,
                                  const uint16_t* moffset, int64_t n, int64_t M, uint16_t* out,
                                  int cus, hipStream_t st) {
  const int64_t blocks = grid_for(n, cus);
  hipLaunchKernelGGL(meta_dequant_kernel, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st, codes,
                     mscale, moffset, n, M, out);
  return hipGetLastError();
}

}  // namespace hqq
