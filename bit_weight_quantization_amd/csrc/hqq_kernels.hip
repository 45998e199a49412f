// hqq_kernels.hip -- gfx950 kernels of the group-wise HQQ quantizer.
//
// Method: "Half-Quadratic Quantization of Large Machine Learning Models"
// (Dropbox tech blog).  Section 2 gives the quantizer Q(W) = round(W/s + z),
// its inverse s (W_q - z), the lp error of W - Q^-1(Q(W)) and the alternating
// half-quadratic updates with s fixed; section 2.1 the shrink
// sign(x) relu(|x| - |x|^(p-1)/beta); section 2.2 the z update as a group mean
// computed with 1/s; section 4.1 the early exit once the error stops improving.
//
// Solver kernel layout (one fused pass: load, init, iterate, pack, store):
//   * every lane holds 8 consecutive fp16 weights (one 16-byte load, fully
//     coalesced inside a wavefront) converted once to fp32 registers;
//   * a group of G weights lives in a segment of L = G/8 adjacent lanes; a
//     wavefront holds S = 64/L groups; group sums/min/max are DPP butterflies
//     inside the segment (quad_perm, row_half_mirror, row_mirror), so every
//     lane of a segment ends with the bit-identical total;
//   * the iteration runs in "code units".  At load each weight becomes
//     u = (w - min) * qmax / (max - min) = w/s + z_0, rounded once to fp32 (a
//     reciprocal product plus an exact FMA residual correction), so an exact tie
//     of the initial quantizer (e.g. the midpoint of min and max) stays exact.  With
//     z = z_0 + delta, the pre-round value is x = u + delta and rc = x - W_q;
//     the residual is r = s*rc, the error sum|r|^p is s^p * sum|rc|^p (the stop
//     test compares the code-unit sums, which differ by the constant factor s^p),
//     and the shrink of r at beta equals s times the shrink of rc at
//     beta*s^(2-p);
//   * the z update of section 2.2, mean(W_q - (W - W_e)/s), is
//     z_0 + (sum W_q - sum u + sum W_e/s)/G in these units.  sum W_q is an exact
//     integer and sum u a per-group constant, so without shrink the new z is a
//     function of the code sum alone: when the codes repeat, z and the error
//     repeat bit for bit and the strict-improvement test stops exactly where the
//     mathematics does;
//   * the shrink is exactly zero whenever every |r| <= beta_t^(-1/(2-p)); the
//     largest |rc| of a group is max(0.5, |delta|) (its min and max sit at u = 0
//     and u = qmax), so a per-group bound decides (with a 1e-4 relative margin
//     that keeps the result bit-identical to evaluating the shrink) whether the
//     wave evaluates it;
//   * groups stop at different steps.  A segment whose group has stopped writes
//     its outputs and becomes idle; once `refill_at` segments of the wave are
//     idle they take the next groups of the wave's contiguous queue, so a wave
//     does not wait for its slowest group.  Every group is computed by exactly
//     the same instruction sequence whatever its slot, so results do not depend
//     on the schedule.
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

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
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

template <int L>
__device__ __forceinline__ float seg_min(float v) {
  if constexpr (L >= 2) v = __builtin_fminf(v, dpp<kDppQuadSwap1>(v));
  if constexpr (L >= 4) v = __builtin_fminf(v, dpp<kDppQuadSwap2>(v));
  if constexpr (L >= 8) v = __builtin_fminf(v, dpp<kDppRowHalfMirror>(v));
  if constexpr (L >= 16) v = __builtin_fminf(v, dpp<kDppRowMirror>(v));
  return v;
}

template <int L>
__device__ __forceinline__ float seg_max(float v) {
  if constexpr (L >= 2) v = __builtin_fmaxf(v, dpp<kDppQuadSwap1>(v));
  if constexpr (L >= 4) v = __builtin_fmaxf(v, dpp<kDppQuadSwap2>(v));
  if constexpr (L >= 8) v = __builtin_fmaxf(v, dpp<kDppRowHalfMirror>(v));
  if constexpr (L >= 16) v = __builtin_fmaxf(v, dpp<kDppRowMirror>(v));
  return v;
}

__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }   // v_log_f32
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32

__device__ __forceinline__ uint64_t ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Unpack the 8 fp16 weights of one 16-byte chunk into fp32.
__device__ __forceinline__ void load8(const uint4& v, float (&w)[kLaneElems]) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(u[i] & 0xffffu));
    _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(u[i] >> 16));
    w[2 * i] = (float)lo;
    w[2 * i + 1] = (float)hi;
  }
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, round to nearest even
}

// |rc|^p for the error sum (|0|^p := 0).
template <int PM>
__device__ __forceinline__ float pow_p(float rc, float p) {
  if constexpr (PM == kPowOne) {
    return __builtin_fabsf(rc);
  } else if constexpr (PM == kPowZero) {
    return rc != 0.0f ? 1.0f : 0.0f;
  } else {
    // log2(0) = -inf, p*(-inf) = -inf, exp2(-inf) = 0 for 0 < p < 1.
    return exp2_hw(p * log2_hw(__builtin_fabsf(rc)));
  }
}

// |rc|^(p-1), used by the shrink only (+inf at rc = 0 for p < 1).
template <int PM>
__device__ __forceinline__ float pow_pm1(float a, float pm1) {
  if constexpr (PM == kPowOne) {
    return 1.0f;
  } else if constexpr (PM == kPowZero) {
    return __builtin_amdgcn_rcpf(a);
  } else {
    return exp2_hw(pm1 * log2_hw(a));
  }
}

// x^p for a positive per-group scalar (error reporting and shrink scaling).
template <int PM>
__device__ __forceinline__ float scalar_pow(float x, float p) {
  if constexpr (PM == kPowOne) return x;
  else if constexpr (PM == kPowZero) return 1.0f;
  else return exp2_hw(p * log2_hw(x));
}

// ------------------------------------------------------------------ solver --

template <int G, int PM>
__global__ __launch_bounds__(kBlock) void hqq_solve_kernel(const SolveParams P) {
  constexpr int L = G / kLaneElems;  // lanes per group
  constexpr int S = kWave / L;       // groups per wavefront
  constexpr float kInvG = 1.0f / (float)G;

  const int lane = threadIdx.x & (kWave - 1);
  const int sl = lane & (L - 1);
  const int64_t wave = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  const int64_t g_begin = wave * P.groups_per_wave;
  const int64_t g_end = g_begin + P.groups_per_wave < P.ngroups ? g_begin + P.groups_per_wave
                                                                : P.ngroups;
  if (g_begin >= g_end) return;  // wave-uniform

  const float qmax = P.qmax;

  // Per-lane copy of the state of the lane's group (identical across the segment).
  float u[kLaneElems];  // w/s + z_0, correctly rounded
  float s = 1.f, inv_s = 1.f;
  float z0 = 0.f, usum = 0.f;            // initial zero point, sum of u over the group
  float delta = 0.f, best_delta = 0.f, best_e = 0.f, e0 = 0.f;
  float inv_beta = 0.f, tau = 0.f;
  int t = 0, t_star = 0;
  int64_t gidx = 0;
  bool active = false;
#pragma unroll
  for (int k = 0; k < kLaneElems; ++k) u[k] = 0.f;

  int64_t next = g_begin;  // wave-uniform: next unassigned group of this wave

  // Hand the next groups of the queue to the idle segments, in lane order.
  auto refill = [&]() {
    const uint64_t idle = ballot(!active);
    const int rank = lanes_below(idle) / L;  // idle segments below this one
    const int nidle = __builtin_popcountll(idle) / L;
    if (!active) {
      const int64_t gi = next + rank;
      if (gi < g_end) {
        gidx = gi;
        float w[kLaneElems];
        load8(P.W[gi * L + sl], w);
        float lmn = w[0], lmx = w[0];
#pragma unroll
        for (int k = 1; k < kLaneElems; ++k) {
          lmn = __builtin_fminf(lmn, w[k]);
          lmx = __builtin_fmaxf(lmx, w[k]);
        }
        const float mn = seg_min<L>(lmn);
        const float mx = seg_max<L>(lmx);
        const float d = mx - mn;
        // s = d / qmax and 1/s = qmax / d, each correctly rounded: a reciprocal
        // estimate, then one exact FMA residual step (d, qmax and the residuals
        // are exact in fp32).
        const float rcp_d = d > 0.f ? __builtin_amdgcn_rcpf(d) : 0.f;
        if (d > 0.f) {
          const float s0 = d * P.inv_qmax;
          s = __builtin_fmaf(__builtin_fmaf(-s0, qmax, d), P.inv_qmax, s0);
          const float i0 = qmax * rcp_d;
          inv_s = __builtin_fmaf(__builtin_fmaf(-i0, d, qmax), rcp_d, i0);
        } else {  // constant group: s = 1, every u is 0
          s = 1.f;
          inv_s = 1.f;
        }
        // u = (w - mn) * qmax / d rounded once: a = w - mn is exact for the
        // binary16 inputs of a group (barring extreme exponent spans); a*qmax is
        // carried exactly as p + e; r = a*qmax - q0*d is the exact residual of the
        // first quotient q0 = a * (qmax/d), and q0 + r/d is the correctly rounded
        // quotient.  A constant group has a = 0 and rcp_d = 0, hence u = 0.
        float lsum = 0.f;
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) {
          const float a = w[k] - mn;
          const float q0 = a * inv_s;
          const float p = a * qmax;
          const float e = __builtin_fmaf(a, qmax, -p);
          const float r = __builtin_fmaf(-q0, d, p) + e;
          u[k] = __builtin_fmaf(r, rcp_d, q0);
          lsum += u[k];
        }
        usum = seg_sum<L>(lsum);
        z0 = -(mn * inv_s);
        delta = 0.f;
        best_delta = 0.f;
        best_e = __builtin_inff();
        t = 0;
        t_star = 0;
        inv_beta = P.inv_beta0;
        tau = P.tau0;
        active = true;
      }
    }
    next += nidle;
  };

  refill();

  while (true) {
    const uint64_t act = ballot(active);
    if (act == 0) break;  // queue drained and every group written
    bool done = false;
    if (active) {
      // ---- evaluation at the current z: codes, residual, lp error --------
      float e, sq;
#pragma unroll
      for (int k = 0; k < kLaneElems; ++k) {
        const float x = u[k] + delta;
        const float q = __builtin_amdgcn_fmed3f(__builtin_rintf(x), 0.f, qmax);
        const float rc = x - q;
        const float a = pow_p<PM>(rc, P.p);
        e = k == 0 ? a : e + a;
        sq = k == 0 ? q : sq + q;
      }
      e = seg_sum<L>(e);
      sq = seg_sum<L>(sq);  // exact: a sum of small integers
      if (t == 0) e0 = e;
      const bool accept = !P.early_stop || (e < best_e);
      if (accept) {
        best_e = e;
        best_delta = delta;
        t_star = t;
      }
      done = !accept || t == P.iters;
      if (!done) {
        // ---- sp1 shrink (only where it can be non-zero) + sp2 mean ---------
        float num = sq - usum;
        const float bound = __builtin_fmaxf(0.5f, __builtin_fabsf(delta)) + 1e-5f * (qmax + 1.f);
        const bool need = bound >= tau * inv_s * (1.0f - 1e-4f);
        if (ballot(need) != 0) {
          if (need) {
            float cs;  // s^(p-2)
            if constexpr (PM == kPowGeneral) cs = exp2_hw(P.pm2 * log2_hw(s));
            else if constexpr (PM == kPowOne) cs = inv_s;
            else cs = inv_s * inv_s;
            const float ib = cs * inv_beta;  // s^(p-2) / beta_t
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < kLaneElems; ++k) {
              const float x = u[k] + delta;
              const float q = __builtin_amdgcn_fmed3f(__builtin_rintf(x), 0.f, qmax);
              const float rc = x - q;
              const float a = __builtin_fabsf(rc);
              float m = 0.f;
              if (a > 0.f) m = __builtin_fmaxf(__builtin_fmaf(-pow_pm1<PM>(a, P.pm1), ib, a), 0.f);
              acc += __builtin_copysignf(m, rc);  // W_e / s
            }
            num += seg_sum<L>(acc);
          }
        }
        delta = num * kInvG;
        inv_beta *= P.inv_kappa;
        tau *= P.rho;
        ++t;
      }
    }

    // ---- groups that stopped: final codes, packing, meta ---------------------
    if (ballot(active && done) != 0) {
      if (active && done) {
        uint32_t c[kLaneElems];
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) {
          const float x = u[k] + best_delta;
          c[k] = (uint32_t)__builtin_amdgcn_fmed3f(__builtin_rintf(x), 0.f, qmax);
        }
        const int64_t chunk = gidx * L + sl;  // index of this lane's 8 elements
        switch (P.nbits) {
          case 4: {
            uint32_t v = 0;
#pragma unroll
            for (int k = 0; k < kLaneElems; ++k) v |= c[k] << (4 * k);
            reinterpret_cast<uint32_t*>(P.packed)[chunk] = v;
            break;
          }
          case 2: {
            uint32_t v = 0;
#pragma unroll
            for (int k = 0; k < kLaneElems; ++k) v |= c[k] << (2 * k);
            reinterpret_cast<uint16_t*>(P.packed)[chunk] = (uint16_t)v;
            break;
          }
          case 8: {
            uint2 v;
            v.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
            v.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
            reinterpret_cast<uint2*>(P.packed)[chunk] = v;
            break;
          }
          default: {  // 3 bits: 8 codes = 24 bits = 3 bytes
            uint32_t v = 0;
#pragma unroll
            for (int k = 0; k < kLaneElems; ++k) v |= c[k] << (3 * k);
            uint8_t* dst = P.packed + chunk * 3;
            dst[0] = (uint8_t)v;
            dst[1] = (uint8_t)(v >> 8);
            dst[2] = (uint8_t)(v >> 16);
            break;
          }
        }
        if (sl == 0) {
          const float best_z = z0 + best_delta;
          P.scale16[gidx] = float_to_half_bits(s);
          P.zero16[gidx] = float_to_half_bits(best_z);
          if (P.scale32) P.scale32[gidx] = s;
          if (P.zero32) P.zero32[gidx] = best_z;
          if (P.stop_step) P.stop_step[gidx] = (uint8_t)t_star;
          if (P.err_init || P.err_best) {
            const float sp = scalar_pow<PM>(s, P.p);
            if (P.err_init) P.err_init[gidx] = e0 * sp;
            if (P.err_best) P.err_best[gidx] = best_e * sp;
          }
        }
        active = false;
      }
    }

    // ---- refill idle slots from the wave's queue -----------------------------
    if (next < g_end) {
      const int nidle = S - __builtin_popcountll(ballot(active)) / L;
      if (nidle >= P.refill_at) refill();
    }
  }
}

// ---------------------------------------------------------------- dequant --

// s*(q - z) for binary16 s, z and an integer code q < 256, rounded once to
// binary16.  s*q and s*z are exact in fp32 (11x8 and 11x11 significant bits);
// TwoSum gives the exact difference as hi + lo; forcing the last bit of hi to
// odd when lo != 0 (round-to-odd) makes the final fp32 -> fp16 rounding equal to
// a single rounding of the exact value (24 >= 11 + 2 bits).
__device__ __forceinline__ uint16_t dequant_one(float s, float sz, uint32_t q) {
  const float a = s * (float)q;
  const float b = -sz;
  const float hi = a + b;
  const float bb = hi - a;
  const float lo = (a - (hi - bb)) + (b - bb);
  uint32_t bits = __builtin_bit_cast(uint32_t, hi);
  if (lo != 0.f) {
    if ((lo > 0.f) != (hi > 0.f)) bits -= 1u;  // |exact| < |hi|: truncate toward zero
    bits |= 1u;
  }
  return float_to_half_bits(__builtin_bit_cast(float, bits));
}

__global__ __launch_bounds__(kBlock) void hqq_dequant_kernel(const DequantParams P) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t chunk = (int64_t)blockIdx.x * kBlock + threadIdx.x; chunk < P.nchunks;
       chunk += stride) {
    const int64_t g = chunk / P.chunks_per_group;
    const float s = (float)__builtin_bit_cast(_Float16, P.scale16[g]);
    const float z = (float)__builtin_bit_cast(_Float16, P.zero16[g]);
    const float sz = s * z;
    uint32_t c[kLaneElems];
    switch (P.nbits) {
      case 4: {
        const uint32_t v = reinterpret_cast<const uint32_t*>(P.packed)[chunk];
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) c[k] = (v >> (4 * k)) & 15u;
        break;
      }
      case 2: {
        const uint32_t v = reinterpret_cast<const uint16_t*>(P.packed)[chunk];
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) c[k] = (v >> (2 * k)) & 3u;
        break;
      }
      case 8: {
        const uint2 v = reinterpret_cast<const uint2*>(P.packed)[chunk];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          c[k] = (v.x >> (8 * k)) & 255u;
          c[k + 4] = (v.y >> (8 * k)) & 255u;
        }
        break;
      }
      default: {
        const uint8_t* src = P.packed + chunk * 3;
        const uint32_t v = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16);
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) c[k] = (v >> (3 * k)) & 7u;
        break;
      }
    }
    uint16_t h[kLaneElems];
#pragma unroll
    for (int k = 0; k < kLaneElems; ++k) h[k] = dequant_one(s, sz, c[k]);
    uint4 o;
    o.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    o.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    o.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
    o.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
    P.out[chunk] = o;
  }
}

template <int G>
hipError_t launch_solve_g(const SolveParams& prm, int power_mode, int blocks, hipStream_t st) {
  switch (power_mode) {
    case kPowOne:
      hipLaunchKernelGGL((hqq_solve_kernel<G, kPowOne>), dim3(blocks), dim3(kBlock), 0, st, prm);
      break;
    case kPowZero:
      hipLaunchKernelGGL((hqq_solve_kernel<G, kPowZero>), dim3(blocks), dim3(kBlock), 0, st, prm);
      break;
    default:
      hipLaunchKernelGGL((hqq_solve_kernel<G, kPowGeneral>), dim3(blocks), dim3(kBlock), 0, st,
                         prm);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_solve(const SolveParams& prm, int group_size, int power_mode, int blocks,
                        hipStream_t stream) {
  switch (group_size) {
    case 16: return launch_solve_g<16>(prm, power_mode, blocks, stream);
    case 32: return launch_solve_g<32>(prm, power_mode, blocks, stream);
    case 64: return launch_solve_g<64>(prm, power_mode, blocks, stream);
    case 128: return launch_solve_g<128>(prm, power_mode, blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequant(const DequantParams& prm, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(hqq_dequant_kernel, dim3(blocks), dim3(kBlock), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace hqq
