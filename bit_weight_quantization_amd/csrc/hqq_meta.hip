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
//   code = the integer nearest the exact ratio (v - mn) * 255 / d, half to even;
//   meta scale = binary16(d / 255) (RNE from fp64), meta offset = mn (a zero minimum
//   as +0); a constant group has codes 0 and meta scale 1.
// Codes are bit-identical to that definition: an fp32 estimate decides them where it
// is provably on the same side of every rounding boundary, and an exact fp64
// comparison of the ratio with the half-integer decides the rest.
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

// The code is decided in fp32 without a division per value: x - min is rounded once
// (binary16 values are exact in fp32) and c = fl32(255 / d) once per group, so
// (x - min) c is within 3 2^-24 relative, i.e. 2^-14.4 absolute (u <= 255), of the
// ratio u = (x - min) 255 / d.  Unless the estimate lies within 2^-12 of a
// half-integer, u is on the same side of that half-integer and the code is the
// estimate's nearest integer.  Near a half-integer (about 0.1% of random values, and
// the exact binary16 ties) the candidates are fl and fl + 1 and the ratio is compared
// with fl + 1/2 exactly: 2 (x - min) 255 against (2 fl + 1) d, where x - min, d and
// both products are multiples of 2^-24 below 2^51 units, so every term is an exact
// fp64 value and an exact midpoint goes to the even code.
__device__ __forceinline__ uint8_t meta_code(uint16_t h, double mn, double d, float mn32, float c32) {
  if (!(d > 0.0)) return 0;
  const float ua = ((float)__builtin_bit_cast(_Float16, h) - mn32) * c32;
  const float fl = __builtin_floorf(ua);
  const float fr = ua - fl;  // exact
  float q;
  if (__builtin_fabsf(fr - 0.5f) > 0x1p-12f) {
    q = fr > 0.5f ? fl + 1.f : fl;
  } else {
    const double num2 = 2.0 * ((half_to_double(h) - mn) * 255.0);
    const double mid = (2.0 * (double)fl + 1.0) * d;
    const bool odd = ((int)fl & 1) != 0;
    q = (num2 > mid || (num2 == mid && odd)) ? fl + 1.f : fl;
  }
  return (uint8_t)__builtin_amdgcn_fmed3f(q, 0.f, 255.f);
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
                                            float& mn32, float& c32, uint16_t& scale16,
                                            uint16_t& offset16) {
  uint16_t hmn = half_of_key(kmin);
  if ((hmn & 0x7fffu) == 0) hmn = 0;  // a zero minimum is stored as +0
  mn = half_to_double(hmn);
  d = half_to_double(half_of_key(kmax)) - mn;  // exact in fp64
  mn32 = (float)mn;                        // exact (a binary16 value)
  c32 = d > 0.0 ? (float)(255.0 / d) : 0.f;  // relative 2^-24
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
  float mn32, c32;
  uint16_t s16, o16;
  meta_params(uniform32(kmin), uniform32(kmax), mn, d, mn32, c32, s16, o16);
  for (int64_t i = g0 + lane; i < g1; i += 64) codes[i] = meta_code(v[i], mn, d, mn32, c32);
  if (lane == 0) {
    mscale[grp] = s16;
    moffset[grp] = o16;
  }
}

// Whole array, two passes without atomics: each reduce block writes the min and max
// keys of its grid-stride share to workspace[2b], workspace[2b + 1]; every quantize
// block reduces those partials itself (at most kMetaPartials of them, L2-resident).
__device__ __forceinline__ void block_minmax(uint32_t& kmin, uint32_t& kmax) {
  __shared__ uint32_t smin[kMetaBlock / 64], smax[kMetaBlock / 64];
  wave_minmax(kmin, kmax);
  const int w = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) {
    smin[w] = kmin;
    smax[w] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMetaBlock / 64; ++i) {
    kmin = smin[i] < kmin ? smin[i] : kmin;
    kmax = smax[i] > kmax ? smax[i] : kmax;
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
  block_minmax(kmin, kmax);
  if (threadIdx.x == 0) {
    ws[2 * blockIdx.x] = kmin;
    ws[2 * blockIdx.x + 1] = kmax;
  }
}

__global__ __launch_bounds__(kMetaBlock) void meta_quant_all_kernel(
    const uint16_t* __restrict__ v, int64_t n, const uint32_t* __restrict__ ws, int partials,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ mscale, uint16_t* __restrict__ moffset) {
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int p = threadIdx.x; p < partials; p += kMetaBlock) {
    const uint32_t a = ws[2 * p], b = ws[2 * p + 1];
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  block_minmax(kmin, kmax);
  double mn, d;
  float mn32, c32;
  uint16_t s16, o16;
  meta_params(kmin, kmax, mn, d, mn32, c32, s16, o16);
  const int64_t stride = (int64_t)gridDim.x * kMetaBlock;
  for (int64_t i = (int64_t)blockIdx.x * kMetaBlock + threadIdx.x; i < n; i += stride)
    codes[i] = meta_code(v[i], mn, d, mn32, c32);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    mscale[0] = s16;
    moffset[0] = o16;
  }
}

// ---- vectorized forms: 8 values per lane (one 16-byte load, one 8-byte store) ------
// Used when values are 16-byte aligned, codes 8-byte aligned and n % 8 == 0.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_key(uint32_t v) {
  // quad_perm / row_half_mirror / row_mirror read lanes of the same row: never out of
  // bounds, so bound_ctrl only spares the compiler an initialisation.
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Min and max over an aligned segment of L lanes (L <= 16: DPP inside a row).
template <int L>
__device__ __forceinline__ void seg_minmax(uint32_t& kmin, uint32_t& kmax) {
  auto step = [&](uint32_t a, uint32_t b) {
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  };
  if constexpr (L >= 2) step(dpp_key<0xB1>(kmin), dpp_key<0xB1>(kmax));    // lane ^ 1
  if constexpr (L >= 4) step(dpp_key<0x4E>(kmin), dpp_key<0x4E>(kmax));    // lane ^ 2
  if constexpr (L >= 8) step(dpp_key<0x141>(kmin), dpp_key<0x141>(kmax));  // mirror in 8
  if constexpr (L >= 16) step(dpp_key<0x140>(kmin), dpp_key<0x140>(kmax)); // mirror in 16
}

__device__ __forceinline__ void chunk_keys(const uint4& raw, uint32_t& kmin, uint32_t& kmax) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t a = key_of((uint16_t)(w[j] & 0xffffu)), b = key_of((uint16_t)(w[j] >> 16));
    kmin = a < kmin ? a : kmin;
    kmin = b < kmin ? b : kmin;
    kmax = a > kmax ? a : kmax;
    kmax = b > kmax ? b : kmax;
  }
}

__device__ __forceinline__ uint2 chunk_codes(const uint4& raw, double mn, double d, float mn32,
                                             float c32) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[2 * j] = meta_code((uint16_t)(w[j] & 0xffffu), mn, d, mn32, c32);
    c[2 * j + 1] = meta_code((uint16_t)(w[j] >> 16), mn, d, mn32, c32);
  }
  return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                    c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
}

// Groups of M = 8 L values: a segment of L lanes per group, grid-stride over waves of
// 64 chunks (512 values; M divides 512, so segments never straddle a wave).
template <int L>
__global__ __launch_bounds__(kMetaBlock) void meta_grouped_vec_kernel(
    const uint4* __restrict__ v, int64_t nchunks, uint2* __restrict__ codes,
    uint16_t* __restrict__ mscale, uint16_t* __restrict__ moffset) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (kMetaBlock / 64);
  const int64_t w0 = uniform64m(((int64_t)blockIdx.x * kMetaBlock + threadIdx.x) / 64);
  // the next iteration's chunk is loaded before this one's arithmetic (from a clamped
  // index, so the load is unconditional and nothing waits for it early)
  auto fetch = [&](int64_t w) { const int64_t c = w * 64 + lane; return v[c < nchunks ? c : nchunks - 1]; };
  uint4 nxt = w0 * 64 < nchunks ? fetch(w0) : make_uint4(0u, 0u, 0u, 0u);
  for (int64_t w = w0; w * 64 < nchunks; w += nwaves) {
    const int64_t c = w * 64 + lane;
    const bool in = c < nchunks;
    const uint4 cur = nxt;
    nxt = fetch(w + nwaves);
    const uint4 raw = in ? cur : make_uint4(0u, 0u, 0u, 0u);
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    if (in) chunk_keys(raw, kmin, kmax);
    seg_minmax<L>(kmin, kmax);  // lanes past the end contribute neutral keys
    double mn, d;
    float mn32, c32;
    uint16_t s16, o16;
    meta_params(kmin, kmax, mn, d, mn32, c32, s16, o16);
    if (in) {
      codes[c] = chunk_codes(raw, mn, d, mn32, c32);
      if ((lane & (L - 1)) == 0) {
        mscale[c / L] = s16;
        moffset[c / L] = o16;
      }
    }
  }
}

__global__ __launch_bounds__(kMetaBlock) void meta_reduce_vec_kernel(const uint4* __restrict__ v,
                                                                     int64_t nchunks,
                                                                     uint32_t* ws) {
  const int64_t stride = (int64_t)gridDim.x * kMetaBlock;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int64_t c = (int64_t)blockIdx.x * kMetaBlock + threadIdx.x; c < nchunks; c += stride)
    chunk_keys(v[c], kmin, kmax);
  block_minmax(kmin, kmax);
  if (threadIdx.x == 0) {
    ws[2 * blockIdx.x] = kmin;
    ws[2 * blockIdx.x + 1] = kmax;
  }
}

__global__ __launch_bounds__(kMetaBlock) void meta_quant_all_vec_kernel(
    const uint4* __restrict__ v, int64_t nchunks, const uint32_t* __restrict__ ws, int partials,
    uint2* __restrict__ codes, uint16_t* __restrict__ mscale, uint16_t* __restrict__ moffset) {
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int p = threadIdx.x; p < partials; p += kMetaBlock) {
    const uint32_t a = ws[2 * p], b = ws[2 * p + 1];
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  block_minmax(kmin, kmax);
  double mn, d;
  float mn32, c32;
  uint16_t s16, o16;
  meta_params(kmin, kmax, mn, d, mn32, c32, s16, o16);
  const int64_t stride = (int64_t)gridDim.x * kMetaBlock;
  for (int64_t c = (int64_t)blockIdx.x * kMetaBlock + threadIdx.x; c < nchunks; c += stride)
    codes[c] = chunk_codes(v[c], mn, d, mn32, c32);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    mscale[0] = s16;
    moffset[0] = o16;
  }
}

// ---- one group per entry of a batched arena (hqq_meta_quantize_batch, meta_group 0) ---
// Block b covers values [b V, (b + 1) V) of the arena; it walks the entries that
// overlap its range (first group of entry e = firsts[e], the last entry ends at n),
// and per entry reduces its share and merges it into workspace[2e], [2e + 1] with one
// atomic min and max per block (a few dozen contenders per address at most).
constexpr int64_t kSegValues = 65536;

__device__ __forceinline__ int seg_entry_of(const BatchEntry* E, int count, int64_t g) {
  int lo = 0, hi = count - 1;  // last entry whose first group is <= g
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (E[mid].first_group <= g) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ void meta_seg_init_kernel(uint32_t* ws, int count) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < count; e += gridDim.x * blockDim.x) {
    ws[2 * e] = 0xffffffffu;
    ws[2 * e + 1] = 0u;
  }
}

// VEC: every entry starts at a multiple of 8 values and the arrays are aligned, so the
// sub-ranges are walked in 8-value chunks (16-byte loads, 8-byte code stores).
template <bool QUANT, bool VEC>
__global__ __launch_bounds__(kMetaBlock) void meta_seg_kernel(
    const uint16_t* __restrict__ v, int64_t n, const BatchEntry* __restrict__ E, int count,
    uint32_t* ws, uint8_t* __restrict__ codes, uint16_t* __restrict__ mscale,
    uint16_t* __restrict__ moffset) {
  const int64_t b0 = (int64_t)blockIdx.x * kSegValues;
  const int64_t b1 = b0 + kSegValues < n ? b0 + kSegValues : n;
  int e = (int)uniform32((uint32_t)seg_entry_of(E, count, b0));
  for (int64_t lo = b0; lo < b1; ++e) {
    const int64_t e_end = uniform64m(e + 1 < count ? E[e + 1].first_group : n);
    if (e_end <= lo) continue;  // an empty entry
    const int64_t hi = e_end < b1 ? e_end : b1;
    if constexpr (!QUANT) {
      uint32_t kmin = 0xffffffffu, kmax = 0u;
      if constexpr (VEC) {
        const uint4* vv = reinterpret_cast<const uint4*>(v);
        for (int64_t c = lo / 8 + threadIdx.x; c < hi / 8; c += kMetaBlock)
          chunk_keys(vv[c], kmin, kmax);
      } else {
        for (int64_t i = lo + threadIdx.x; i < hi; i += kMetaBlock) {
          const uint32_t k = key_of(v[i]);
          kmin = k < kmin ? k : kmin;
          kmax = k > kmax ? k : kmax;
        }
      }
      block_minmax(kmin, kmax);
      if (threadIdx.x == 0) {
        atomicMin(&ws[2 * e], kmin);
        atomicMax(&ws[2 * e + 1], kmax);
      }
      __syncthreads();  // block_minmax's LDS is reused for the next entry
    } else {
      double mn, d;
      float mn32, c32;
      uint16_t s16, o16;
      meta_params(ws[2 * e], ws[2 * e + 1], mn, d, mn32, c32, s16, o16);
      if constexpr (VEC) {
        const uint4* vv = reinterpret_cast<const uint4*>(v);
        uint2* cc = reinterpret_cast<uint2*>(codes);
        for (int64_t c = lo / 8 + threadIdx.x; c < hi / 8; c += kMetaBlock)
          cc[c] = chunk_codes(vv[c], mn, d, mn32, c32);
      } else {
        for (int64_t i = lo + threadIdx.x; i < hi; i += kMetaBlock)
          codes[i] = meta_code(v[i], mn, d, mn32, c32);
      }
      if (threadIdx.x == 0 && lo == E[e].first_group) {  // the block holding the entry's start
        mscale[e] = s16;
        moffset[e] = o16;
      }
    }
    lo = hi;
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
  const bool vec = n % 8 == 0 && (reinterpret_cast<uintptr_t>(values) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(codes) & 7) == 0;
  const int64_t nchunks = n / 8;
  if (vec && M == 0) {
    int64_t partials = (nchunks + kMetaBlock * 4 - 1) / (kMetaBlock * 4);
    if (partials > kMetaPartials) partials = kMetaPartials;
    hipLaunchKernelGGL(meta_reduce_vec_kernel, dim3((unsigned)partials), dim3(kMetaBlock), 0, st,
                       reinterpret_cast<const uint4*>(values), nchunks, workspace);
    const int64_t blocks = grid_for(nchunks, cus);
    hipLaunchKernelGGL(meta_quant_all_vec_kernel, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st,
                       reinterpret_cast<const uint4*>(values), nchunks, workspace, (int)partials,
                       reinterpret_cast<uint2*>(codes), mscale, moffset);
    return hipGetLastError();
  }
  if (vec && (M == 16 || M == 32 || M == 64 || M == 128)) {
    const int64_t waves = (nchunks + 63) / 64;
    int64_t blocks = (waves + kMetaBlock / 64 - 1) / (kMetaBlock / 64);
    const int64_t cap = (int64_t)cus * 16;
    if (blocks > cap) blocks = cap;
    const uint4* vv = reinterpret_cast<const uint4*>(values);
    uint2* cc = reinterpret_cast<uint2*>(codes);
    switch (M) {
      case 16: hipLaunchKernelGGL(meta_grouped_vec_kernel<2>, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st, vv, nchunks, cc, mscale, moffset); break;
      case 32: hipLaunchKernelGGL(meta_grouped_vec_kernel<4>, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st, vv, nchunks, cc, mscale, moffset); break;
      case 64: hipLaunchKernelGGL(meta_grouped_vec_kernel<8>, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st, vv, nchunks, cc, mscale, moffset); break;
      default: hipLaunchKernelGGL(meta_grouped_vec_kernel<16>, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st, vv, nchunks, cc, mscale, moffset); break;
    }
    return hipGetLastError();
  }
  if (M == 0) {
    // reduce: at most kMetaPartials blocks of >= 16 values per thread
    int64_t partials = (n + kMetaBlock * 16 - 1) / (kMetaBlock * 16);
    if (partials > kMetaPartials) partials = kMetaPartials;
    hipLaunchKernelGGL(meta_reduce_kernel, dim3((unsigned)partials), dim3(kMetaBlock), 0, st,
                       values, n, workspace);
    const int64_t blocks = grid_for(n, cus);
    hipLaunchKernelGGL(meta_quant_all_kernel, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st,
                       values, n, workspace, (int)partials, codes, mscale, moffset);
    return hipGetLastError();
  }
  const int64_t ngroups = (n + M - 1) / M;
  const int64_t blocks = (ngroups + kMetaBlock / 64 - 1) / (kMetaBlock / 64);
  hipLaunchKernelGGL(meta_grouped_kernel, dim3((unsigned)blocks), dim3(kMetaBlock), 0, st, values,
                     n, M, ngroups, codes, mscale, moffset);
  return hipGetLastError();
}

hipError_t launch_meta_quantize_segments(const uint16_t* values, int64_t n,
                                         const BatchEntry* entries, int count, bool starts_mod8,
                                         uint8_t* codes, uint16_t* mscale, uint16_t* moffset,
                                         uint32_t* workspace, hipStream_t st) {
  const int64_t blocks = (n + kSegValues - 1) / kSegValues;
  int init_blocks = (count + kMetaBlock - 1) / kMetaBlock;
  const bool vec = starts_mod8 && n % 8 == 0 && (reinterpret_cast<uintptr_t>(values) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(codes) & 7) == 0;
  hipLaunchKernelGGL(meta_seg_init_kernel, dim3((unsigned)init_blocks), dim3(kMetaBlock), 0, st,
                     workspace, count);
  if (vec) {
    hipLaunchKernelGGL((meta_seg_kernel<false, true>), dim3((unsigned)blocks), dim3(kMetaBlock), 0,
                       st, values, n, entries, count, workspace, codes, mscale, moffset);
    hipLaunchKernelGGL((meta_seg_kernel<true, true>), dim3((unsigned)blocks), dim3(kMetaBlock), 0,
                       st, values, n, entries, count, workspace, codes, mscale, moffset);
  } else {
    hipLaunchKernelGGL((meta_seg_kernel<false, false>), dim3((unsigned)blocks), dim3(kMetaBlock), 0,
                       st, values, n, entries, count, workspace, codes, mscale, moffset);
    hipLaunchKernelGGL((meta_seg_kernel<true, false>), dim3((unsigned)blocks), dim3(kMetaBlock), 0,
                       st, values, n, entries, count, workspace, codes, mscale, moffset);
  }
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
