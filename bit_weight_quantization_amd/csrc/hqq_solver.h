// hqq_solver.h -- device building blocks of the gfx950 HQQ solver, shared by the
// per-group kernel (hqq_kernels.hip) and the whole-tensor stop (hqq_tensor_stop.hip):
// lane-permute reductions over a group's segment, the group's load in code units, one
// solver step (evaluation, stop test, shrink, z mean) and the packed output of a group,
// plus the host-side dispatch over group size, stop metric and power mode.  The method
// and the code-unit formulation are described at the top of hqq_kernels.hip.
// Internal: included by the kernel sources only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqq_internal.h"

namespace hqq {
namespace {

// ---------------------------------------------------------------- helpers --

// DPP lane-permute controls (gfx9 encoding).
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141; // lane i of 8 reads lane 7-i
constexpr int kDppRowMirror = 0x140;     // lane i of 16 reads lane 15-i

// Every control used here reads a lane of the same row, so no source is out of
// bounds and bound_ctrl only spares the compiler an initialisation of the old value.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
}

// Butterfly sum over an aligned segment of L lanes; commutativity of IEEE
// addition gives every lane of the segment the same bits.
template <int L>
__device__ __forceinline__ float seg_sum(float v) {
  if constexpr (L >= 2) v += dpp<kDppQuadSwap1>(v);
  if constexpr (L >= 4) v += dpp<kDppQuadSwap2>(v);
  if constexpr (L >= 8) v += dpp<kDppRowHalfMirror>(v);
  if constexpr (L >= 16) v += dpp<kDppRowMirror>(v);
  return v;
}

// Sum of v[K0 .. K0 + N) as a balanced binary tree (N a power of two): fp32 rounding
// error grows with the tree's depth, log2 N, not with N.
template <int K0, int N>
__device__ __forceinline__ float tree_sum(const float (&v)[kLaneElems]) {
  if constexpr (N == 1) return v[K0];
  else return tree_sum<K0, N / 2>(v) + tree_sum<K0 + N / 2, N / 2>(v);
}

__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }   // v_log_f32
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32

__device__ __forceinline__ uint64_t ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Packed binary16 min/max on two halves at once (v_pk_min_f16 / v_pk_max_f16).
// Written as instructions because the compiler would otherwise quiet every
// operand first; inputs are finite weights, so quieting is not needed.
__device__ __forceinline__ uint32_t pk_min_f16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t pk_max_f16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Low half: max(-a.lo, -b.lo); high half: max(a.hi, b.hi).
__device__ __forceinline__ uint32_t pk_max_neglo_f16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2 neg_lo:[1,1]" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// w - m in fp32 for the binary16 in the low (HI = false) or high half of `pair`:
// one fused operation w*1 + (-m) with a single rounding (v_fma_mix_f32).
template <bool HI>
__device__ __forceinline__ float half_minus(uint32_t pair, float m) {
  float r;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(m));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(m));
  return r;
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, round to nearest even
}

// The solver mode PM packs the power mode of the shrink (bits 0-1: kPowGeneral,
// kPowOne, kPowZero) and the early-stop error metric (bits 2-3: kErrP = the lp error
// with the solver's p, kErrL1, kErrL2).
constexpr int shrink_mode(int pm) { return pm & 3; }
constexpr int err_mode(int pm) { return pm >> 2; }

// Error term of one residual in code units for the stop test (|0|^p := 0).
template <int PM>
__device__ __forceinline__ float pow_p(float rc, float p) {
  constexpr int SM = shrink_mode(PM), EM = err_mode(PM);
  if constexpr (EM == kErrL1 || (EM == kErrP && SM == kPowOne)) {
    return __builtin_fabsf(rc);
  } else if constexpr (EM == kErrL2) {
    return rc * rc;
  } else if constexpr (SM == kPowZero) {
    return rc != 0.0f ? 1.0f : 0.0f;
  } else {
    // log2(0) = -inf, p*(-inf) = -inf, exp2(-inf) = 0 for 0 < p < 1.
    return exp2_hw(p * log2_hw(__builtin_fabsf(rc)));
  }
}

// |rc|^(p-1), used by the shrink only (+inf at rc = 0 for p < 1).
template <int PM>
__device__ __forceinline__ float pow_pm1(float a, float pm1) {
  if constexpr (shrink_mode(PM) == kPowOne) {
    return 1.0f;
  } else if constexpr (shrink_mode(PM) == kPowZero) {
    return __builtin_amdgcn_rcpf(a);
  } else {
    return exp2_hw(pm1 * log2_hw(a));
  }
}

// s^q for the error reported in weight units (q: the error metric's exponent).
template <int PM>
__device__ __forceinline__ float scalar_pow(float x, float p) {
  constexpr int SM = shrink_mode(PM), EM = err_mode(PM);
  if constexpr (EM == kErrL1 || (EM == kErrP && SM == kPowOne)) return x;
  else if constexpr (EM == kErrL2) return x * x;
  else if constexpr (SM == kPowZero) return 1.0f;
  else return exp2_hw(p * log2_hw(x));
}

// ------------------------------------------------------------------ solver --

// Group scalars fixed at load.
struct GroupInit {
  float s, inv_s, z0, usum;
  uint32_t nm_mx;   // the group's -min (low half) and max (high half) as binary16
  bool may_shrink;  // the shrink can be non-zero at some step (|r| <= max - min always)
};

// Values every lane of the wave computes identically, kept in scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Whether the device entry table of a batched launch is the one the host validated:
// every lane hashes entries lane, lane + 64, ... (their fields only; no weight is
// read), the wave adds the lane sums, and the total is compared with the host's hash.
// Wave-uniform.  Thread 0 of block 0 records the verdict in the status word.
__device__ __forceinline__ bool batch_table_matches(const SolveParams& P) {
  const int lane = threadIdx.x & 63;
  uint64_t h = 0;
  for (int i = lane; i < P.batch_count; i += 64) {
    const BatchEntry& e = P.batch[i];
    h += table_entry_hash((uint64_t)(uintptr_t)e.W, e.rows, e.cols, e.first_group, i);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)h, off, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(h >> 32), off, 64);
    h += ((uint64_t)hi << 32) | lo;
  }
  const bool ok = uniform64((int64_t)h) == (int64_t)P.batch_hash;
  if (blockIdx.x == 0 && threadIdx.x == 0) *P.batch_status = ok ? 0 : 5;  // HQQ_OK, HQQ_ERR_TABLE_MISMATCH
  return ok;
}

// The entry of a batched launch that holds the wave's next group: its index, its
// group range [first, end) and its weights.  Wave-uniform.
struct BatchCursor {
  int m;
  int64_t first, end;
  const uint4* W;
};

// The entry holding global group g (binary search for the last entry whose first
// group is <= g; empty entries share their successor's first group).
__device__ __forceinline__ BatchCursor batch_cursor(const SolveParams& P, int64_t g) {
  int lo = 0, hi = P.batch_count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (P.batch[mid].first_group <= g) lo = mid;
    else hi = mid - 1;
  }
  BatchCursor c;
  c.m = uniform(lo);
  c.first = uniform64(P.batch[c.m].first_group);
  c.end = uniform64(c.m + 1 < P.batch_count ? P.batch[c.m + 1].first_group : P.ngroups);
  c.W = reinterpret_cast<const uint4*>(uniform64(reinterpret_cast<int64_t>(P.batch[c.m].W)));
  return c;
}

// Moves the cursor forward to the entry holding group g (g < number of groups).
__device__ __forceinline__ void batch_advance(const SolveParams& P, BatchCursor& c, int64_t g) {
  while (g >= c.end) {
    c.m = uniform(c.m + 1);
    c.first = c.end;
    c.W = reinterpret_cast<const uint4*>(uniform64(reinterpret_cast<int64_t>(P.batch[c.m].W)));
    c.end = uniform64(c.m + 1 < P.batch_count ? P.batch[c.m + 1].first_group : P.ngroups);
  }
}

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// The lane's 16 binary16 weights: two consecutive 16-byte chunks.
struct LaneW {
  uint4 lo, hi;
};

// The lane's 32 bytes of group `gi`.  Past the end of the wave's queue the lane reads
// the queue's last group instead (a valid address; the value is unused), so the loads
// are unconditional and their registers need no other initialisation.  In a batched
// launch a prime batch never extends past the cursor's entry, so the weights come from
// that entry (past its end or the queue's, the lane reads the entry's first group, a
// valid address whose value is unused).
template <int L, bool BATCH>
__device__ __forceinline__ LaneW fetch_chunk(const SolveParams& P, const BatchCursor& c,
                                             int64_t gi, int64_t g_end, int sl) {
  const uint4* p;
  if constexpr (!BATCH) {
    p = P.W + 2 * ((gi < g_end ? gi : g_end - 1) * L + sl);
  } else {
    const int64_t limit = g_end < c.end ? g_end : c.end;
    const int64_t g = gi < limit ? gi : c.first;
    p = c.W + 2 * ((g - c.first) * L + sl);
  }
  return LaneW{p[0], p[1]};
}

// The first code decision is round(U) of the exact ratio U = (w - mn) qmax / d.  u is
// U rounded once to fp32, and rounding is monotonic while half-integers are exact fp32
// values, so rint(u) is round(U) unless u landed exactly on a half-integer that U is not
// on.  For every u of the lane that lies exactly on a half-integer, the side is decided
// exactly in fp64 -- (w - mn) qmax against u (mx - mn), both products of binary16
// differences and small integers, exact -- and u moves one ulp towards U, so that every
// later evaluation starts from a value on U's side of every half-integer.  A real tie
// stays exactly on the half-integer.  Returns whether some u of the lane moved.
// nm_mx: the group's -min (low half) and max (high half) as binary16.
__device__ __forceinline__ bool settle_ties(const LaneW& raw, uint32_t nm_mx, float qmax,
                                            float (&u)[kLaneElems]) {
  const uint32_t pair[8] = {raw.lo.x, raw.lo.y, raw.lo.z, raw.lo.w,
                            raw.hi.x, raw.hi.y, raw.hi.z, raw.hi.w};
  const double mn64 = -(double)(float)__builtin_bit_cast(_Float16, (uint16_t)(nm_mx & 0xffffu));
  const double d64 = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(nm_mx >> 16)) - mn64;
  bool moved = false;
#pragma unroll
  for (int k = 0; k < kLaneElems; ++k) {
    if (__builtin_amdgcn_fractf(u[k]) != 0.5f) continue;
    const uint16_t hw = (uint16_t)(pair[k / 2] >> (16 * (k & 1)));
    const double num = ((double)(float)__builtin_bit_cast(_Float16, hw) - mn64) * (double)qmax;
    const double mid = (double)u[k] * d64;
    if (num != mid) {
      u[k] = bitsf(fbits(u[k]) + (num > mid ? 1u : 0xffffffffu));  // one ulp
      moved = true;
    }
  }
  return moved;
}

// From the lane's 16 raw binary16 weights, compute its u values and the group scalars.
// Called by all L lanes of a segment together (segment-wide DPP reductions).  With
// SETTLE the exact side of half-integer u is decided here (settle_ties); without, the
// caller does it (the per-group kernel finds such u in its first evaluation) and must
// recompute usum if a u moves.
template <int L, bool SETTLE = true>
__device__ __forceinline__ GroupInit init_group(const SolveParams& P, const LaneW& raw,
                                                float (&u)[kLaneElems]) {
  const float qmax = P.qmax;
  // Group min and max on the binary16 values themselves (exact): pairwise packed
  // min/max over the 8 words, then one word (-min, max) reduced over the segment
  // with packed max.
  const uint32_t m = pk_min_f16(pk_min_f16(pk_min_f16(raw.lo.x, raw.lo.y), pk_min_f16(raw.lo.z, raw.lo.w)),
                                pk_min_f16(pk_min_f16(raw.hi.x, raw.hi.y), pk_min_f16(raw.hi.z, raw.hi.w)));
  const uint32_t M = pk_max_f16(pk_max_f16(pk_max_f16(raw.lo.x, raw.lo.y), pk_max_f16(raw.lo.z, raw.lo.w)),
                                pk_max_f16(pk_max_f16(raw.hi.x, raw.hi.y), pk_max_f16(raw.hi.z, raw.hi.w)));
  uint32_t v = pk_max_neglo_f16(__builtin_amdgcn_perm(M, m, 0x05040100u),   // (m.lo, M.lo)
                                __builtin_amdgcn_perm(M, m, 0x07060302u));  // (m.hi, M.hi)
  if constexpr (L >= 2) v = pk_max_f16(v, dpp_u32<kDppQuadSwap1>(v));
  if constexpr (L >= 4) v = pk_max_f16(v, dpp_u32<kDppQuadSwap2>(v));
  if constexpr (L >= 8) v = pk_max_f16(v, dpp_u32<kDppRowHalfMirror>(v));
  if constexpr (L >= 16) v = pk_max_f16(v, dpp_u32<kDppRowMirror>(v));
  const float mn = -(float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
  const float mx = (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
  const float d = mx - mn;
  GroupInit g;
  g.nm_mx = v;
  // s = d / qmax and 1/s = qmax / d, each correctly rounded: a reciprocal estimate,
  // then one exact FMA residual step (d, qmax and the residuals are exact in fp32).
  const float rcp_d = d > 0.f ? __builtin_amdgcn_rcpf(d) : 0.f;
  if (d > 0.f) {
    const float s0 = d * P.inv_qmax;
    g.s = __builtin_fmaf(__builtin_fmaf(-s0, qmax, d), P.inv_qmax, s0);
    const float i0 = qmax * rcp_d;
    g.inv_s = __builtin_fmaf(__builtin_fmaf(-i0, d, qmax), rcp_d, i0);
  } else {  // constant group: s = 1, every u is 0
    g.s = 1.f;
    g.inv_s = 1.f;
  }
  // u = (w - mn) * qmax / d rounded once.  a = w - mn is exact for the binary16
  // inputs of a group (barring extreme exponent spans).  qmax/d is carried as the
  // pair c_hi + c_lo (c_hi = 1/s correctly rounded; c_lo = the exact remainder
  // qmax - c_hi*d times 1/d), and u = fma(a, c_hi, a*c_lo) adds the small term to
  // the exact product a*c_hi: before its single rounding the sum is within 2^-46
  // relative of the exact quotient, so u is exact whenever the quotient is
  // representable (a rounding tie of the initial quantizer stays a tie) and
  // correctly rounded otherwise except within 2^-46 of a rounding midpoint.  A
  // constant group has a = 0, hence u = 0.
  const float c_lo = __builtin_fmaf(-g.inv_s, d, qmax) * rcp_d;
  const uint32_t pair[8] = {raw.lo.x, raw.lo.y, raw.lo.z, raw.lo.w,
                            raw.hi.x, raw.hi.y, raw.hi.z, raw.hi.w};
  bool half = false;  // some u of the lane is exactly a half-integer
#pragma unroll
  for (int k = 0; k < kLaneElems; ++k) {
    const float a = (k & 1) ? half_minus<true>(pair[k / 2], mn) : half_minus<false>(pair[k / 2], mn);
    u[k] = __builtin_fmaf(a, g.inv_s, a * c_lo);
    if constexpr (SETTLE) half |= __builtin_amdgcn_fractf(u[k]) == 0.5f;
  }
  if constexpr (SETTLE) {
    if (ballot(half) != 0) {
      if (half) settle_ties(raw, v, qmax, u);
    }
  }
  g.usum = seg_sum<L>(tree_sum<0, kLaneElems>(u));
  g.z0 = -(mn * g.inv_s);
  // Without shrink every code lies in [0, qmax], so |z - z0| <= qmax and every
  // |r| = s|x - W_q| <= s * max(0.5, qmax) = d: the shrink stays zero if d is below
  // the smallest threshold beta_t^(-1/(2-p)) of the run (1e-4 relative margin).
  g.may_shrink = d >= P.tau_min * (1.0f - 1e-4f);
  return g;
}


// Orders this wave's LDS accesses: lanes hand group state to other lanes of the same
// wavefront through LDS (the standby pool and the done ring below).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

constexpr int kWavesPerBlock = kBlock / kWave;

// The lane's 16 codes packed as the bitstream stores them (LSB first): 2 bits in w[0],
// 4 bits in w[0..1], 8 bits in w[0..3], 3 bits as two 24-bit fields in w[0..1].
// Sum_k q_k 2^(nbits k) over up to 24 bits is an exact fp32 integer, so the fields are
// assembled with FMAs and converted once.
struct PackedCodes {
  uint32_t w[4];
};

// The two words of 2-, 3- or 4-bit codes.
__device__ __forceinline__ uint2 pack_codes_narrow(int nbits, const float (&q)[kLaneElems]) {
  auto horner = [&](int k0, int n, float radix) {
    float acc = q[k0 + n - 1];
#pragma unroll
    for (int k = n - 2; k >= 0; --k) acc = __builtin_fmaf(acc, radix, q[k0 + k]);
    return (uint32_t)acc;
  };
  switch (nbits) {
    case 4:
      return make_uint2(horner(0, 4, 16.f) | (horner(4, 4, 16.f) << 16),
                        horner(8, 4, 16.f) | (horner(12, 4, 16.f) << 16));
    case 2:
      return make_uint2(horner(0, 8, 4.f) | (horner(8, 8, 4.f) << 16), 0u);
    default:  // 3 bits
      return make_uint2(horner(0, 8, 8.f), horner(8, 8, 8.f));
  }
}

__device__ __forceinline__ PackedCodes pack_codes(int nbits, const float (&q)[kLaneElems]) {
  PackedCodes c = {{0u, 0u, 0u, 0u}};
  if (nbits == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int w = 0; w < 4; ++w) c.w[w] = __builtin_amdgcn_cvt_pk_u8_f32(q[4 * w + k], (uint32_t)k, c.w[w]);
  } else {
    const uint2 n = pack_codes_narrow(nbits, q);
    c.w[0] = n.x;
    c.w[1] = n.y;
  }
  return c;
}

// Stores the lane's packed codes; chunk = index of the lane's 16 elements.
__device__ __forceinline__ void store_codes(const SolveParams& P, int64_t chunk, const PackedCodes& c) {
  switch (P.nbits) {
    case 4: {  // 16 codes = 8 bytes, as two 4-byte words (the stream is 4-byte aligned)
      uint32_t* dst = reinterpret_cast<uint32_t*>(P.packed) + 2 * chunk;
      dst[0] = c.w[0];
      dst[1] = c.w[1];
      break;
    }
    case 2:  // 4 bytes
      reinterpret_cast<uint32_t*>(P.packed)[chunk] = c.w[0];
      break;
    case 8: {  // 16 bytes, as four 4-byte words
      uint32_t* dst = reinterpret_cast<uint32_t*>(P.packed) + 4 * chunk;
#pragma unroll
      for (int w = 0; w < 4; ++w) dst[w] = c.w[w];
      break;
    }
    default: {  // 3 bits: 16 codes = 48 bits = 6 bytes, 2-byte aligned
      uint16_t* dst = reinterpret_cast<uint16_t*>(P.packed + chunk * 6);
      dst[0] = (uint16_t)c.w[0];
      dst[1] = (uint16_t)((c.w[0] >> 16) | (c.w[1] << 8));
      dst[2] = (uint16_t)(c.w[1] >> 8);
      break;
    }
  }
}

// One evaluation of the lane's 16 weights at x = u + delta: the segment's lp error
// (code units) and code sum.  CLAMP = false is the exact shortcut for |delta| < 1/2.
// PACK: also the codes packed as stored (2, 3 and 4 bits; nothing for 8).
template <int L, int PM, bool CLAMP, bool ZERO = false, bool PACK = false>
__device__ __forceinline__ void eval_group(const float (&u)[kLaneElems], float delta, float qmax,
                                           float p, float& e, float& sq, int nbits = 0,
                                           uint2* pk = nullptr) {
  float a[kLaneElems], q[kLaneElems];
#pragma unroll
  for (int k = 0; k < kLaneElems; ++k) {
    const float x = ZERO ? u[k] : u[k] + delta;  // ZERO: delta == 0 (x = u + 0 = u exactly)
    q[k] = __builtin_rintf(x);
    if constexpr (CLAMP) q[k] = __builtin_amdgcn_fmed3f(q[k], 0.f, qmax);
    a[k] = pow_p<PM>(x - q[k], p);
  }
  e = seg_sum<L>(tree_sum<0, kLaneElems>(a));
  sq = seg_sum<L>(tree_sum<0, kLaneElems>(q));  // exact: a sum of small integers
  if constexpr (PACK) {
    if (nbits != 8) *pk = pack_codes_narrow(nbits, q);
  }
}

// State of one group held by a segment (identical in all L lanes of the segment).
struct Slot {
  float u[kLaneElems];  // this lane's code-unit values
  float s, inv_s, z0, usum;
  float delta, best_delta, best_e, e0;
  int t, t_star;
  int64_t gidx;
  bool may_shrink;
  bool active;   // iterating
  bool pending;  // stopped, outputs not yet written or handed to the done ring
};

// Clamping is a no-op while |delta| < 1/2: u lies in [0, qmax], so x = u + delta
// stays inside (-1/2, qmax + 1/2) and rounds into [0, qmax].
__device__ __forceinline__ bool far_delta(float delta) { return !(__builtin_fabsf(delta) < 0.4999f); }
__device__ __forceinline__ bool needs_clamp(const Slot& q) { return q.active && far_delta(q.delta); }

// What a solver step does after its evaluation (error e, code sum sq): the early-stop
// test of section 4.1, and unless the group stops, the sp1 shrink (only where it can be
// non-zero) and the sp2 mean.
template <int L, int PM>
__device__ __forceinline__ void step_tail(const SolveParams& P, Slot& q, float e, float sq) {
  constexpr float kInvG = 1.0f / (float)(L * kLaneElems);
  const float qmax = P.qmax;
  if (P.err_init && q.t == 0) q.e0 = e;
  const bool accept = !P.early_stop || (e < q.best_e);
  if (accept) {
    q.best_e = e;
    q.best_delta = q.delta;
    q.t_star = q.t;
  }
  if (!accept || q.t == P.iters) {
    q.active = false;
    q.pending = true;
    return;
  }
  float num = sq - q.usum;
  if (ballot(q.may_shrink) != 0) {
    // beta_t^(-1/(2-p)) and 1/beta_t, from t
    const float tf = (float)q.t;
    const float tau = P.tau0 * exp2_hw(tf * P.log2_rho);
    const float bound = __builtin_fmaxf(0.5f, __builtin_fabsf(q.delta)) + 1e-5f * (qmax + 1.f);
    const bool need = q.may_shrink && bound >= tau * q.inv_s * (1.0f - 1e-4f);
    if (ballot(need) != 0) {
      if (need) {
        float cs;  // s^(p-2)
        if constexpr (shrink_mode(PM) == kPowGeneral) cs = exp2_hw(P.pm2 * log2_hw(q.s));
        else if constexpr (shrink_mode(PM) == kPowOne) cs = q.inv_s;
        else cs = q.inv_s * q.inv_s;
        const float inv_beta = P.inv_beta0 * exp2_hw(-tf * P.log2_kappa);
        const float ib = cs * inv_beta;  // s^(p-2) / beta_t
        float we[kLaneElems];  // W_e / s
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) {
          const float x = q.u[k] + q.delta;
          const float qc = __builtin_amdgcn_fmed3f(__builtin_rintf(x), 0.f, qmax);
          const float rc = x - qc;
          const float a = __builtin_fabsf(rc);
          float m = 0.f;
          if (a > 0.f) m = __builtin_fmaxf(__builtin_fmaf(-pow_pm1<PM>(a, P.pm1), ib, a), 0.f);
          we[k] = __builtin_copysignf(m, rc);
        }
        num += seg_sum<L>(tree_sum<0, kLaneElems>(we));
      }
    }
  }
  const float next = num * kInvG;
  // With the per-group stop, a z update that leaves delta bit for bit unchanged makes the
  // next evaluation repeat this one (same x, codes, error and order of sums), so that
  // step cannot improve and the group stops there with this step as its best: stop now,
  // with the state that evaluation would have left.
  if (P.early_stop && fbits(next) == fbits(q.delta)) {
    q.active = false;
    q.pending = true;
    return;
  }
  q.delta = next;
  ++q.t;
}

// One step of the solver for an active group: evaluation at the current z (codes,
// residual, lp error), then step_tail.  FIRST: the step at t = 0 (delta = 0, no clamp
// needed).  Returns the evaluated error (code units).
template <int L, int PM, bool FIRST = false>
__device__ __forceinline__ float solver_step(const SolveParams& P, Slot& q, bool clamp) {
  const float qmax = P.qmax;
  float e, sq;
  if constexpr (FIRST) {
    eval_group<L, PM, false, true>(q.u, 0.f, qmax, P.p, e, sq);
  } else if (clamp) {
    eval_group<L, PM, true>(q.u, q.delta, qmax, P.p, e, sq);
  } else {
    eval_group<L, PM, false>(q.u, q.delta, qmax, P.p, e, sq);
  }
  step_tail<L, PM>(P, q, e, sq);
  return e;
}

// The evaluation at t = 0 in the per-group kernel (delta = 0, x = u, no clamp): error and
// code sum as eval_group, the codes packed for storing (2, 3 and 4 bits; nothing for 8),
// and whether some u of the lane is exactly a half-integer (|u - rint(u)| = 1/2;
// u - rint(u) is exact), i.e. needs settle_ties.
template <int L, int PM>
__device__ __forceinline__ bool eval_first(const float (&u)[kLaneElems], int nbits, float p,
                                           float& e, float& sq, uint2& pk) {
  float a[kLaneElems], q[kLaneElems], r[kLaneElems];
#pragma unroll
  for (int k = 0; k < kLaneElems; ++k) {
    q[k] = __builtin_rintf(u[k]);
    r[k] = __builtin_fabsf(u[k] - q[k]);
    a[k] = pow_p<PM>(u[k] - q[k], p);
  }
  e = seg_sum<L>(tree_sum<0, kLaneElems>(a));
  sq = seg_sum<L>(tree_sum<0, kLaneElems>(q));
  if (nbits != 8) pk = pack_codes_narrow(nbits, q);
  // max |rc| over the 16 elements (three-operand max instructions)
  float m = __builtin_fmaxf(__builtin_fmaxf(r[0], r[1]), r[2]);
#pragma unroll
  for (int k = 3; k + 1 < kLaneElems; k += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, r[k]), r[k + 1]);
  m = __builtin_fmaxf(m, r[kLaneElems - 1]);
  return m == 0.5f;
}

// The group's binary16 s and z (plus the optional fp32, stop-step and error outputs),
// written by lane 0 of the segment (sl == 0).
template <int PM>
__device__ __forceinline__ void write_meta(const SolveParams& P, int64_t gi, float gs, float best_z,
                                           float e0, float best_e, int t_star) {
  P.scale16[gi] = float_to_half_bits(gs);
  P.zero16[gi] = float_to_half_bits(best_z);
  if (P.scale32) P.scale32[gi] = gs;
  if (P.zero32) P.zero32[gi] = best_z;
  if (P.stop_step) P.stop_step[gi] = (uint8_t)t_star;
  if (P.err_init || P.err_best) {
    const float sp = scalar_pow<PM>(gs, P.p);
    if (P.err_init) P.err_init[gi] = e0 * sp;
    if (P.err_best) P.err_best[gi] = best_e * sp;
  }
}

// Codes at the accepted z, packed into the LSB-first bitstream, and the group's
// binary16 s and z (plus the optional fp32 and error outputs).  Called by the L lanes
// of a segment; lane sl writes the codes of its 16 elements.  CLAMP = false is exact
// when |bd| < 1/2 (the argument of needs_clamp); ZERO: bd == 0 (codes rint(u)).
template <int L, int PM, bool CLAMP, bool ZERO = false>
__device__ __forceinline__ void write_group(const SolveParams& P, int sl,
                                            const float (&u)[kLaneElems], int64_t gi, float gs,
                                            float z0, float bd, float e0, float best_e,
                                            int t_star) {
  const float qmax = P.qmax;
  float q[kLaneElems];  // codes as fp32 integers in [0, qmax]
#pragma unroll
  for (int k = 0; k < kLaneElems; ++k) {
    q[k] = __builtin_rintf(ZERO ? u[k] : u[k] + bd);
    if (CLAMP) q[k] = __builtin_amdgcn_fmed3f(q[k], 0.f, qmax);
  }
  store_codes(P, gi * L + sl, pack_codes(P.nbits, q));
  if (sl == 0) write_meta<PM>(P, gi, gs, z0 + bd, e0, best_e, t_star);
}

// write_group with the clamp only where some written group of the wave needs it.
template <int L, int PM>
__device__ __forceinline__ void write_group_any(const SolveParams& P, bool write, int sl,
                                                const float (&u)[kLaneElems], int64_t gi, float gs,
                                                float z0, float bd, float e0, float best_e,
                                                int t_star) {
  if (ballot(write && far_delta(bd)) != 0) {
    if (write) write_group<L, PM, true>(P, sl, u, gi, gs, z0, bd, e0, best_e, t_star);
  } else {
    if (write) write_group<L, PM, false>(P, sl, u, gi, gs, z0, bd, e0, best_e, t_star);
  }
}

// Wavefronts that can be resident at once for `kernel` (LDS and VGPRs set the limit).
template <typename K>
hipError_t resident_waves(K kernel, int cus, int64_t& waves) {
  int per_cu = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  waves = (int64_t)cus * per_cu * kWavesPerBlock;
  return hipSuccess;
}

// Dispatch on the group size, the early-stop metric and the shrink's power mode;
// `X` is passed through to Launch<G, PM>::run (launch-specific buffers).
template <template <int, int> class Launch, int G, int EM, class Extra>
hipError_t dispatch_power(const SolveParams& prm, const Extra& X, int power_mode,
                          int cus, hipStream_t st) {
  switch (power_mode) {
    case kPowOne: return Launch<G, kPowOne | (EM << 2)>::run(prm, X, cus, st);
    case kPowZero: return Launch<G, kPowZero | (EM << 2)>::run(prm, X, cus, st);
    default: return Launch<G, kPowGeneral | (EM << 2)>::run(prm, X, cus, st);
  }
}

template <template <int, int> class Launch, int G, class Extra>
hipError_t dispatch_metric(const SolveParams& prm, const Extra& X, int power_mode,
                           int cus, hipStream_t st) {
  switch (prm.err_metric) {
    case kErrL1: return dispatch_power<Launch, G, kErrL1, Extra>(prm, X, power_mode, cus, st);
    case kErrL2: return dispatch_power<Launch, G, kErrL2, Extra>(prm, X, power_mode, cus, st);
    default: return dispatch_power<Launch, G, kErrP, Extra>(prm, X, power_mode, cus, st);
  }
}

template <template <int, int> class Launch, class Extra>
hipError_t dispatch_group(const SolveParams& prm, const Extra& X, int group_size,
                          int power_mode, int cus, hipStream_t st) {
  switch (group_size) {
    case 16: return dispatch_metric<Launch, 16, Extra>(prm, X, power_mode, cus, st);
    case 32: return dispatch_metric<Launch, 32, Extra>(prm, X, power_mode, cus, st);
    case 64: return dispatch_metric<Launch, 64, Extra>(prm, X, power_mode, cus, st);
    case 128: return dispatch_metric<Launch, 128, Extra>(prm, X, power_mode, cus, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace
}  // namespace hqq
