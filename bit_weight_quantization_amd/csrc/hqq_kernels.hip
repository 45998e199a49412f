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
//     coalesced inside a wavefront); group min/max run on the binary16 pairs;
//   * a group of G weights lives in a segment of L = G/8 adjacent lanes; a
//     wavefront holds S = 64/L groups; group sums/min/max are DPP butterflies
//     inside the segment (quad_perm, row_half_mirror, row_mirror), so every
//     lane of a segment ends with the bit-identical total;
//   * the iteration runs in "code units".  At load each weight becomes
//     u = (w - min) * qmax / (max - min) = w/s + z_0, rounded once to fp32 (an
//     FMA of the exact product with a double-float qmax/(max - min)), so an exact
//     tie of the initial quantizer (e.g. the midpoint of min and max) stays exact.  With
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
//   * groups stop at different steps, but every group takes at least two
//     evaluations (t = 0 is always accepted).  So a wavefront runs init and the
//     first two solver steps densely for S fresh groups at a time ("prime"
//     batches) and writes the groups that stopped at once (about 60% of them on
//     heavy-tailed weights).  The others wait in an LDS standby pool; each segment
//     of the wave iterates one of them, and a segment whose group stopped copies
//     its u values and header into an LDS done ring and takes a standby group in
//     the same pass.  Done groups are packed and written in dense batches of S.
//     Every group runs exactly the same instruction sequence whatever its batch or
//     slot, so results do not depend on the schedule.
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
  bool may_shrink;  // the shrink can be non-zero at some step (|r| <= max - min always)
};

// Values every lane of the wave computes identically, kept in scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
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

// The lane's 16-byte chunk of group `gi`.  Past the end of the wave's queue the
// lane reads the queue's last group instead (a valid address; the value is unused),
// so the load is unconditional and its registers need no other initialisation.  In a
// batched launch a prime batch never extends past the cursor's entry, so the chunk
// comes from that entry (past its end or the queue's, the lane reads the entry's
// first group, a valid address whose value is unused).
template <int L, bool BATCH>
__device__ __forceinline__ uint4 fetch_chunk(const SolveParams& P, const BatchCursor& c,
                                             int64_t gi, int64_t g_end, int sl) {
  if constexpr (!BATCH) {
    return P.W[(gi < g_end ? gi : g_end - 1) * L + sl];
  } else {
    const int64_t limit = g_end < c.end ? g_end : c.end;
    const int64_t g = gi < limit ? gi : c.first;
    return c.W[(g - c.first) * L + sl];
  }
}

// From the lane's 8 raw binary16 weights, compute its u values and the group scalars.
// Called by all L lanes of a segment together (segment-wide DPP reductions).
template <int L>
__device__ __forceinline__ GroupInit init_group(const SolveParams& P, const uint4& raw,
                                                float (&u)[kLaneElems]) {
  const float qmax = P.qmax;
  // Group min and max on the binary16 values themselves (exact): pairwise packed
  // min/max over the 4 words, then one word (-min, max) reduced over the segment
  // with packed max.
  const uint32_t m = pk_min_f16(pk_min_f16(raw.x, raw.y), pk_min_f16(raw.z, raw.w));
  const uint32_t M = pk_max_f16(pk_max_f16(raw.x, raw.y), pk_max_f16(raw.z, raw.w));
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
  const uint32_t pair[4] = {raw.x, raw.y, raw.z, raw.w};
  float lsum;
#pragma unroll
  for (int k = 0; k < kLaneElems; ++k) {
    const float a = (k & 1) ? half_minus<true>(pair[k / 2], mn) : half_minus<false>(pair[k / 2], mn);
    u[k] = __builtin_fmaf(a, g.inv_s, a * c_lo);
    lsum = k == 0 ? u[0] : lsum + u[k];
  }
  g.usum = seg_sum<L>(lsum);
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

// Per-wavefront LDS: u slots [0, kStandby) are the standby pool (groups past their
// first two evaluations, waiting for a free segment), u slots [kStandby, kStandby + S)
// the done ring (stopped groups waiting to be written).  A slot holds the G
// code-unit values u of a group; standby slots have a 12-word header (the full solver
// state), done slots an 8-word one.
template <int G>
struct SolveLds {
  static constexpr int S = kWave * kLaneElems / G;
  // Wavefronts per SIMD the kernel is compiled for (VGPR budget): seven at G = 32,
  // where the extra wavefront outweighs the smaller pool, six otherwise (measured).
  static constexpr int kWavesPerSimd = G == 32 ? 7 : 6;
  // A prime batch adds up to S groups to the pool, a hand-over up to S to the ring.
  // The pool holds 1.5 S groups, so it is restocked before it runs dry, where the LDS
  // of kWavesPerSimd wavefronts allows (G = 64, 128); S otherwise.
  static constexpr int kStandby = (G == 16 || G == 32) ? S : S + S / 2;
  static constexpr int kDone = S;
  float u[kWavesPerBlock][kStandby + kDone][G];
  uint4 standby_hdr[kWavesPerBlock][kStandby][3];
  uint4 done_hdr[kWavesPerBlock][kDone][2];
};

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

template <int G>
__device__ __forceinline__ void store_u(float* slot_u, int sl, const float (&u)[kLaneElems]) {
  float4* dst = reinterpret_cast<float4*>(slot_u + sl * kLaneElems);
  dst[0] = make_float4(u[0], u[1], u[2], u[3]);
  dst[1] = make_float4(u[4], u[5], u[6], u[7]);
}

template <int G>
__device__ __forceinline__ void load_u(const float* slot_u, int sl, float (&u)[kLaneElems]) {
  const float4* src = reinterpret_cast<const float4*>(slot_u + sl * kLaneElems);
  const float4 a = src[0], b = src[1];
  u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w;
  u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
}

// One evaluation of the lane's 8 weights at x = u + delta: the segment's lp error
// (code units) and code sum.  CLAMP = false is the exact shortcut for |delta| < 1/2.
template <int L, int PM, bool CLAMP, bool ZERO = false>
__device__ __forceinline__ void eval_group(const float (&u)[kLaneElems], float delta, float qmax,
                                           float p, float& e, float& sq) {
#pragma unroll
  for (int k = 0; k < kLaneElems; ++k) {
    const float x = ZERO ? u[k] : u[k] + delta;  // ZERO: delta == 0 (x = u + 0 = u exactly)
    float q = __builtin_rintf(x);
    if constexpr (CLAMP) q = __builtin_amdgcn_fmed3f(q, 0.f, qmax);
    const float rc = x - q;
    const float a = pow_p<PM>(rc, p);
    e = k == 0 ? a : e + a;
    sq = k == 0 ? q : sq + q;
  }
  e = seg_sum<L>(e);
  sq = seg_sum<L>(sq);  // exact: a sum of small integers
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

// One step of the solver for an active group: evaluation at the current z (codes,
// residual, lp error), the early-stop test of section 4.1, and unless the group
// stops, the sp1 shrink (only where it can be non-zero) and the sp2 mean.
// FIRST: the step at t = 0 (delta = 0, no clamp needed).  Returns the evaluated
// error (code units).
template <int L, int PM, bool FIRST = false>
__device__ __forceinline__ float solver_step(const SolveParams& P, Slot& q, bool clamp) {
  constexpr float kInvG = 1.0f / (float)(L * kLaneElems);
  const float qmax = P.qmax;
  float e, sq;
  if constexpr (FIRST) {
    eval_group<L, PM, false, true>(q.u, 0.f, qmax, P.p, e, sq);
  } else if (clamp) {
    eval_group<L, PM, true>(q.u, q.delta, qmax, P.p, e, sq);
  } else {
    eval_group<L, PM, false>(q.u, q.delta, qmax, P.p, e, sq);
  }
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
    return e;
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
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < kLaneElems; ++k) {
          const float x = q.u[k] + q.delta;
          const float qc = __builtin_amdgcn_fmed3f(__builtin_rintf(x), 0.f, qmax);
          const float rc = x - qc;
          const float a = __builtin_fabsf(rc);
          float m = 0.f;
          if (a > 0.f) m = __builtin_fmaxf(__builtin_fmaf(-pow_pm1<PM>(a, P.pm1), ib, a), 0.f);
          acc += __builtin_copysignf(m, rc);  // W_e / s
        }
        num += seg_sum<L>(acc);
      }
    }
  }
  q.delta = num * kInvG;
  ++q.t;
  return e;
}

// Codes at the accepted z, packed into the LSB-first bitstream, and the group's
// binary16 s and z (plus the optional fp32 and error outputs).  Called by the L lanes
// of a segment; lane sl writes the codes of its 8 elements.  CLAMP = false is exact
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
  // Packing: sum_k q_k 2^(nbits k) over up to 24 bits is an exact fp32 integer, so the
  // fields are assembled with FMAs and converted once.
  auto horner = [&](int k0, int n, float radix) {
    float acc = q[k0 + n - 1];
#pragma unroll
    for (int k = n - 2; k >= 0; --k) acc = __builtin_fmaf(acc, radix, q[k0 + k]);
    return (uint32_t)acc;
  };
  const int64_t chunk = gi * L + sl;  // index of this lane's 8 elements
  switch (P.nbits) {
    case 4: {
      const uint32_t v = horner(0, 4, 16.f) | (horner(4, 4, 16.f) << 16);
      reinterpret_cast<uint32_t*>(P.packed)[chunk] = v;
      break;
    }
    case 2: {
      reinterpret_cast<uint16_t*>(P.packed)[chunk] = (uint16_t)horner(0, 8, 4.f);
      break;
    }
    case 8: {
      uint2 v = make_uint2(0u, 0u);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v.x = __builtin_amdgcn_cvt_pk_u8_f32(q[k], (uint32_t)k, v.x);
        v.y = __builtin_amdgcn_cvt_pk_u8_f32(q[k + 4], (uint32_t)k, v.y);
      }
      reinterpret_cast<uint2*>(P.packed)[chunk] = v;
      break;
    }
    default: {  // 3 bits: 8 codes = 24 bits = 3 bytes
      const uint32_t v = horner(0, 8, 8.f);
      uint8_t* dst = P.packed + chunk * 3;
      dst[0] = (uint8_t)v;
      dst[1] = (uint8_t)(v >> 8);
      dst[2] = (uint8_t)(v >> 16);
      break;
    }
  }
  if (sl == 0) {
    const float best_z = z0 + bd;
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
}

// write_group with the clamp only where some written group of the wave needs it;
// TRY_ZERO adds the shortcut for bd == 0 in every written group.
template <int L, int PM, bool TRY_ZERO = false>
__device__ __forceinline__ void write_group_any(const SolveParams& P, bool write, int sl,
                                                const float (&u)[kLaneElems], int64_t gi, float gs,
                                                float z0, float bd, float e0, float best_e,
                                                int t_star) {
  if (TRY_ZERO && ballot(write && bd != 0.f) == 0) {
    if (write) write_group<L, PM, false, true>(P, sl, u, gi, gs, z0, 0.f, e0, best_e, t_star);
  } else if (ballot(write && far_delta(bd)) != 0) {
    if (write) write_group<L, PM, true>(P, sl, u, gi, gs, z0, bd, e0, best_e, t_star);
  } else {
    if (write) write_group<L, PM, false>(P, sl, u, gi, gs, z0, bd, e0, best_e, t_star);
  }
}

// Every group takes at least two evaluations (t = 0 is always accepted), so a wave
// runs them densely for S fresh groups at a time ("prime" batches): init and two
// solver steps in every segment.  Groups that stopped are written at once; the
// others wait in the standby pool for a segment of the iterating set.  Iterating
// segments whose group stops hand it to the done ring and take a standby group in
// the same pass; done groups are written in dense batches of S.  Every group runs
// exactly the same instruction sequence whatever its batch or slot, so results do
// not depend on the schedule.
template <int G, int PM, bool BATCH>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(SolveLds<G>::kWavesPerSimd))) void hqq_solve_kernel(const SolveParams P) {
  constexpr int L = G / kLaneElems;  // lanes per group
  constexpr int S = kWave / L;       // segments per wavefront
  constexpr int kStandby = SolveLds<G>::kStandby;  // standby-pool capacity
  constexpr int kDone = SolveLds<G>::kDone;        // done-ring capacity
  __shared__ SolveLds<G> lds;

  const int wid = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int seg = lane / L;
  const int sl = lane & (L - 1);
  // The wave's queue: chunks wave, wave + nwaves, wave + 2 nwaves, ... of C groups
  // (C a multiple of S), so all wavefronts sweep the weights together through a
  // window of nwaves * C groups (page and TLB locality) and finish within a chunk
  // of each other.
  const int64_t wave = uniform64(((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t C = P.chunk_groups;
  int64_t chunk = wave;
  if (chunk * C >= P.ngroups) return;  // wave-uniform; the kernel has no block-wide barrier
  int64_t next = chunk * C;            // next group of the wave's queue
  int64_t q_end = next + C < P.ngroups ? next + C : P.ngroups;  // end of the current chunk

  float (*U)[G] = lds.u[wid];
  uint4 (*H)[3] = lds.standby_hdr[wid];
  uint4 (*D)[2] = lds.done_hdr[wid];  // done slot j has u slot kStandby + j

  Slot sg;  // the group this segment iterates
#pragma unroll
  for (int k = 0; k < kLaneElems; ++k) sg.u[k] = 0.f;
  sg.s = sg.inv_s = 1.f;
  sg.z0 = sg.usum = sg.delta = sg.best_delta = sg.best_e = sg.e0 = 0.f;
  sg.t = sg.t_star = 0;
  sg.gidx = 0;
  sg.may_shrink = sg.active = sg.pending = false;

  // Wave-uniform bookkeeping.  The queue is exhausted when next == q_end == ngroups.
  int n_standby = 0;       // standby slots [0, n_standby) hold groups
  int done_head = 0, done_count = 0;

  // The weights of the next prime batch are fetched one batch ahead, so the HBM
  // latency overlaps the work in between.
  BatchCursor cursor = {0, 0, P.ngroups, P.W};
  if constexpr (BATCH) cursor = batch_cursor(P, next);
  uint4 prefetch = fetch_chunk<L, BATCH>(P, cursor, next + seg, q_end, sl);

  // Dense batch: segment j initializes group next + j and runs its first two steps.
  auto prime = [&]() {
    // In a batched launch the batch stops at the end of the cursor's entry.
    const int64_t avail = (BATCH && cursor.end < q_end ? cursor.end : q_end) - next;
    const int n = avail < S ? (int)avail : S;
    Slot a;
    a.active = a.pending = false;
    if (seg < n) {
      a.gidx = next + seg;
      const GroupInit gq = init_group<L>(P, prefetch, a.u);
      a.s = gq.s;
      a.inv_s = gq.inv_s;
      a.z0 = gq.z0;
      a.usum = gq.usum;
      a.may_shrink = gq.may_shrink;
      a.delta = a.best_delta = a.e0 = 0.f;
      a.best_e = __builtin_inff();
      a.t = a.t_star = 0;
      a.active = true;
    }
    next = uniform64(next + n);
    if (next >= q_end) {  // next chunk of the queue
      chunk += nwaves;
      next = chunk * C < P.ngroups ? chunk * C : P.ngroups;
      q_end = next + C < P.ngroups ? next + C : P.ngroups;
    }
    if constexpr (BATCH) {
      if (next < q_end) batch_advance(P, cursor, next);
    }
    prefetch = fetch_chunk<L, BATCH>(P, cursor, next + seg, q_end, sl);
    // t = 0: delta = 0, no clamp needed.
    if (a.active) solver_step<L, PM, true>(P, a, false);
    if (ballot(a.active) != 0) {
      const bool clamp = ballot(needs_clamp(a)) != 0;
      if (a.active) solver_step<L, PM>(P, a, clamp);
    }
    // Groups stopping here have t* = 0 (they stopped at t = 1) unless iters == 1.
    write_group_any<L, PM, true>(P, a.pending, sl, a.u, a.gidx, a.s, a.z0, a.best_delta, a.e0,
                                 a.best_e, a.t_star);
    const uint64_t m = ballot(a.active);
    if (a.active) {
      const int slot = n_standby + lanes_below(m) / L;  // n_standby <= kStandby - S
      store_u<G>(U[slot], sl, a.u);
      if (sl == 0) {
        H[slot][0] = make_uint4((uint32_t)a.gidx, (uint32_t)(a.gidx >> 32), fbits(a.s), fbits(a.inv_s));
        H[slot][1] = make_uint4(fbits(a.z0), fbits(a.usum), fbits(a.delta), fbits(a.best_delta));
        H[slot][2] = make_uint4(fbits(a.best_e), fbits(a.e0),
                                (uint32_t)a.t | ((uint32_t)a.t_star << 8) |
                                    (a.may_shrink ? 0x10000u : 0u),
                                0u);
      }
    }
    n_standby = uniform(n_standby + __builtin_popcountll(m) / L);
    wave_lds_sync();
  };

  // Segments with `want` set take standby groups (highest standby slot first).
  auto take_standby = [&](bool want) {
    const uint64_t m = ballot(want);
    const int rank = lanes_below(m) / L;
    if (want && rank < n_standby) {
      const int slot = n_standby - 1 - rank;
      load_u<G>(U[slot], sl, sg.u);
      const uint4 h0 = H[slot][0], h1 = H[slot][1], h2 = H[slot][2];
      sg.gidx = (int64_t)(((uint64_t)h0.y << 32) | h0.x);
      sg.s = bitsf(h0.z);
      sg.inv_s = bitsf(h0.w);
      sg.z0 = bitsf(h1.x);
      sg.usum = bitsf(h1.y);
      sg.delta = bitsf(h1.z);
      sg.best_delta = bitsf(h1.w);
      sg.best_e = bitsf(h2.x);
      sg.e0 = bitsf(h2.y);
      sg.t = (int)(h2.z & 0xffu);
      sg.t_star = (int)((h2.z >> 8) & 0xffu);
      sg.may_shrink = (h2.z & 0x10000u) != 0u;
      sg.active = true;
    }
    const int taken = __builtin_popcountll(m) / L;
    n_standby = uniform(n_standby - (taken < n_standby ? taken : n_standby));
    wave_lds_sync();
  };

  // Dense batch: segment j writes the codes and meta of done slot head + j.
  auto finalize = [&](int n) {
    const bool write = seg < n;
    const int slot = kStandby + (int)((unsigned)(done_head + (write ? seg : 0)) % (unsigned)kDone);
    float uu[kLaneElems];
    load_u<G>(U[slot], sl, uu);
    const uint4 h0 = D[slot - kStandby][0], h1 = D[slot - kStandby][1];
    write_group_any<L, PM>(P, write, sl, uu, (int64_t)(((uint64_t)h0.y << 32) | h0.x),
                           bitsf(h0.z), bitsf(h0.w), bitsf(h1.x), bitsf(h1.y), bitsf(h1.z),
                           (int)h1.w);
    done_head = uniform((int)((unsigned)(done_head + n) % (unsigned)kDone));
    done_count = uniform(done_count - n);
    wave_lds_sync();
  };

  // One pass per solver step of the iterating set.  A pass hands stopped groups to
  // the done ring, writes full done batches, primes a batch when segments are idle
  // and the pool is empty, and gives idle segments standby groups.
  while (true) {
    const bool any_active = ballot(sg.active) != 0;
    if (!any_active && n_standby == 0 && next >= q_end) break;
    if (any_active) {
      const bool clamp = ballot(needs_clamp(sg)) != 0;
      if (sg.active) solver_step<L, PM>(P, sg, clamp);
    }

    // ---- stopped groups: hand them to the done ring ---------------------------
    const uint64_t pm = ballot(sg.pending);
    const int npend = __builtin_popcountll(pm) / L;
    if (npend > 0 && (npend >= P.refill_at || ballot(sg.active) == 0)) {
      if (done_count + npend > kDone) finalize(done_count);  // rare: make room first
      if (sg.pending) {
        const int rank = lanes_below(pm) / L;
        const int slot = kStandby + (int)((unsigned)(done_head + done_count + rank) % (unsigned)kDone);
        store_u<G>(U[slot], sl, sg.u);
        if (sl == 0) {
          D[slot - kStandby][0] = make_uint4((uint32_t)sg.gidx, (uint32_t)(sg.gidx >> 32), fbits(sg.s),
                                      fbits(sg.z0));
          D[slot - kStandby][1] = make_uint4(fbits(sg.best_delta), fbits(sg.e0), fbits(sg.best_e),
                                      (uint32_t)sg.t_star);
        }
      }
      done_count = uniform(done_count + npend);
      sg.pending = false;
      wave_lds_sync();
      if (done_count >= S) finalize(S);
    }

    // ---- keep the pool stocked (a batch adds at most S), feed idle segments ------
    if (n_standby <= kStandby - S && next < q_end) prime();
    const bool idle = !sg.active && !sg.pending;
    if (n_standby > 0 && ballot(idle) != 0) take_standby(idle);
  }
  while (done_count > 0) finalize(done_count < S ? done_count : S);
}

// ------------------------------------------------------- whole-tensor stop --
//
// The early exit of section 4.1 read at the scope of the whole tensor: the error
// that must keep improving is E_t = sum over all groups of e_t (weight units), and
// every group returns the z of the same step t*, the end of the strictly decreasing
// run E_0 > E_1 > ... > E_t*.  Without a per-group stop every group takes the same
// steps, so a wavefront iterates S groups in lockstep and no standby pool is needed:
//   pass 1 (ACC): every group runs steps 0 .. iters; each wavefront adds its groups'
//     step errors into fp64 totals (two lanes per step, each over half of the
//     wavefront's groups) and writes them to its columns of the partial totals;
//   decision: one block adds the partials in a fixed order and finds t*;
//   pass 2 (OUT): every group runs t* updates and writes its outputs, which is the
//     per-group solver with the stop switched off and iters = t*, step for step.

// Partial totals of pass 1, laid out [step][2 * wave + half].
constexpr int kTensorStopMaxWaves = 8192;
constexpr int kMaxSteps = 256;  // iters <= 255
constexpr int kStepRows = 32;   // steps buffered in LDS between folds

template <int G, int PM, bool OUT>
__global__ __launch_bounds__(kBlock) void hqq_lockstep_kernel(const SolveParams P,
                                                              const TensorStopParams X) {
  constexpr int L = G / kLaneElems;
  constexpr int S = kWave / L;
  constexpr int kHalf = S / 2;       // groups folded by one lane
  constexpr int kRow = S + 4;        // floats per LDS row: 16-byte aligned, rows 4 banks apart
  constexpr int kAcc = kMaxSteps / kStepRows;
  __shared__ __align__(16) float ebuf[kWavesPerBlock][OUT ? 1 : kStepRows][OUT ? 4 : kRow];

  const int wid = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int seg = lane / L;
  const int sl = lane & (L - 1);
  const int64_t wave = uniform64(((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t nbatches = (P.ngroups + S - 1) / S;
  SolveParams Q = P;
  Q.early_stop = 0;
  if constexpr (OUT) Q.iters = uniform(*X.t_star);
  const int T = Q.iters;

  // Lane l folds half l / kStepRows of row l % kStepRows: acc[k] is its share of the
  // wavefront's total of step kStepRows * k + l % kStepRows.
  const int fold_row = lane & (kStepRows - 1);
  const int fold_half = lane / kStepRows;
  double acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = 0.0;

  for (int64_t b = wave; b < nbatches; b += nwaves) {
    const int64_t g0 = b * S;
    const int64_t left = P.ngroups - g0;
    const int n = left < S ? (int)left : S;
    // Every lane loads (a segment past the end reads the batch's first group).
    const uint4 raw = P.W[(seg < n ? g0 + seg : g0) * L + sl];
    Slot a;
    a.active = a.pending = false;
    a.gidx = g0 + seg;
    float sp = 0.f;  // s^q: code-unit error -> weight units
    if (seg < n) {
      const GroupInit gq = init_group<L>(P, raw, a.u);
      a.s = gq.s;
      a.inv_s = gq.inv_s;
      a.z0 = gq.z0;
      a.usum = gq.usum;
      a.may_shrink = gq.may_shrink;
      a.delta = a.best_delta = a.e0 = 0.f;
      a.best_e = __builtin_inff();
      a.t = a.t_star = 0;
      a.active = true;
      if constexpr (!OUT) sp = scalar_pow<PM>(a.s, P.p);
    }
    for (int t = 0; t <= T; ++t) {
      float e = 0.f;
      if (t == 0) {
        if (a.active) e = solver_step<L, PM, true>(Q, a, false);
      } else {
        const bool clamp = ballot(needs_clamp(a)) != 0;
        if (a.active) e = solver_step<L, PM>(Q, a, clamp);
      }
      if constexpr (!OUT) {
        const int r = t & (kStepRows - 1);
        if (sl == 0) ebuf[wid][r][seg] = e * sp;  // 0 for a segment without a group
        if (r == kStepRows - 1 || t == T) {  // fold rows 0 .. r into the fp64 totals
          wave_lds_sync();
          if (fold_row <= r) {
            const float* row = ebuf[wid][fold_row] + fold_half * kHalf;
            double sum = 0.0;
            if constexpr (kHalf % 4 == 0) {
#pragma unroll
              for (int j = 0; j < kHalf; j += 4) {
                const float4 v = *reinterpret_cast<const float4*>(row + j);
                sum += (double)v.x;
                sum += (double)v.y;
                sum += (double)v.z;
                sum += (double)v.w;
              }
            } else {
#pragma unroll
              for (int j = 0; j < kHalf; j += 2) {
                const float2 v = *reinterpret_cast<const float2*>(row + j);
                sum += (double)v.x;
                sum += (double)v.y;
              }
            }
            const int k = t / kStepRows;
#pragma unroll
            for (int kk = 0; kk < kAcc; ++kk)
              if (kk == k) acc[kk] += sum;
          }
          wave_lds_sync();
        }
      }
    }
    if constexpr (OUT) {
      write_group_any<L, PM>(Q, a.pending, sl, a.u, a.gidx, a.s, a.z0, a.best_delta, a.e0,
                             a.best_e, a.t_star);
    }
  }
  if constexpr (!OUT) {
    const int64_t stride = 2 * X.nwaves;  // row length of the partials
#pragma unroll
    for (int k = 0; k < kAcc; ++k) {
      const int t = k * kStepRows + fold_row;
      if (t <= T) X.partials[(int64_t)t * stride + 2 * wave + fold_half] = acc[k];
    }
  }
}

// E_t = sum of the partial totals of step t over the wavefronts (per-thread strided
// sums, then a tree in LDS: a fixed order for a given grid), and t*.
__global__ __launch_bounds__(kBlock) void hqq_tensor_decide_kernel(const TensorStopParams X,
                                                                   int T) {
  __shared__ double red[kBlock];
  __shared__ double total[kMaxSteps];
  const int tid = threadIdx.x;
  const int64_t n = 2 * X.nwaves;  // partials per step
  for (int t = 0; t <= T; ++t) {
    const double* row = X.partials + (int64_t)t * n;
    double s = 0.0;
    for (int64_t w = tid; w < n; w += kBlock) s += row[w];
    red[tid] = s;
    __syncthreads();
    for (int h = kBlock / 2; h > 0; h >>= 1) {
      if (tid < h) red[tid] += red[tid + h];
      __syncthreads();
    }
    if (tid == 0) total[t] = red[0];
    __syncthreads();
  }
  if (X.totals) {
    for (int t = tid; t <= T; t += kBlock) X.totals[t] = total[t];
  }
  if (tid == 0) {
    int ts = 0;
    while (ts < T && total[ts + 1] < total[ts]) ++ts;
    *X.t_star = ts;
    if (X.t_star_out) *X.t_star_out = ts;
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

// Persistent grid: as many blocks as can be resident at once (LDS and VGPRs set the
// limit), or fewer for small inputs; the wavefronts deal the chunks round robin.
constexpr int kChunkBatches = 4;  // chunk = 4 prime batches

template <typename K>
hipError_t resident_waves(K kernel, int cus, int64_t& waves) {
  int per_cu = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  waves = (int64_t)cus * per_cu * kWavesPerBlock;
  return hipSuccess;
}

template <int G, int PM>
struct SolveLaunch {
  static hipError_t run(SolveParams prm, const TensorStopParams&, int cus, hipStream_t st) {
    auto kernel = hqq_solve_kernel<G, PM, false>;
    if constexpr (err_mode(PM) == kErrP) {  // batched launches always use the lp error
      if (prm.batch) kernel = hqq_solve_kernel<G, PM, true>;
    }
    int64_t resident = 0;
    hipError_t err = resident_waves(kernel, cus, resident);
    if (err != hipSuccess) return err;
    constexpr int S = kWave * kLaneElems / G;
    prm.chunk_groups = kChunkBatches * S;
    const int64_t nchunks = (prm.ngroups + prm.chunk_groups - 1) / prm.chunk_groups;
    const int64_t nwaves = nchunks < resident ? nchunks : resident;
    const int64_t blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, prm);
    return hipGetLastError();
  }
};

// Pass 1, the decision and pass 2 of the whole-tensor stop, in stream order.
template <int G, int PM>
struct TensorStopLaunch {
  static hipError_t run(const SolveParams& prm, TensorStopParams X, int cus, hipStream_t st) {
    constexpr int S = kWave * kLaneElems / G;
    const int64_t nbatches = (prm.ngroups + S - 1) / S;
    auto acc_kernel = hqq_lockstep_kernel<G, PM, false>;
    auto out_kernel = hqq_lockstep_kernel<G, PM, true>;
    int64_t resident = 0;
    hipError_t err = resident_waves(acc_kernel, cus, resident);
    if (err != hipSuccess) return err;
    int64_t nwaves = nbatches < resident ? nbatches : resident;
    if (nwaves > kTensorStopMaxWaves) nwaves = kTensorStopMaxWaves;
    int64_t blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    X.nwaves = blocks * kWavesPerBlock;  // <= kTensorStopMaxWaves (a multiple of 4)
    hipLaunchKernelGGL(acc_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, prm, X);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(hqq_tensor_decide_kernel, dim3(1), dim3(kBlock), 0, st, X, prm.iters);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    err = resident_waves(out_kernel, cus, resident);
    if (err != hipSuccess) return err;
    nwaves = nbatches < resident ? nbatches : resident;
    blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(out_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, prm, X);
    return hipGetLastError();
  }
};

// Dispatch on the group size, the early-stop metric and the shrink's power mode.
template <template <int, int> class Launch, int G, int EM>
hipError_t dispatch_power(const SolveParams& prm, const TensorStopParams& X, int power_mode,
                          int cus, hipStream_t st) {
  switch (power_mode) {
    case kPowOne: return Launch<G, kPowOne | (EM << 2)>::run(prm, X, cus, st);
    case kPowZero: return Launch<G, kPowZero | (EM << 2)>::run(prm, X, cus, st);
    default: return Launch<G, kPowGeneral | (EM << 2)>::run(prm, X, cus, st);
  }
}

template <template <int, int> class Launch, int G>
hipError_t dispatch_metric(const SolveParams& prm, const TensorStopParams& X, int power_mode,
                           int cus, hipStream_t st) {
  switch (prm.err_metric) {
    case kErrL1: return dispatch_power<Launch, G, kErrL1>(prm, X, power_mode, cus, st);
    case kErrL2: return dispatch_power<Launch, G, kErrL2>(prm, X, power_mode, cus, st);
    default: return dispatch_power<Launch, G, kErrP>(prm, X, power_mode, cus, st);
  }
}

template <template <int, int> class Launch>
hipError_t dispatch_group(const SolveParams& prm, const TensorStopParams& X, int group_size,
                          int power_mode, int cus, hipStream_t st) {
  switch (group_size) {
    case 16: return dispatch_metric<Launch, 16>(prm, X, power_mode, cus, st);
    case 32: return dispatch_metric<Launch, 32>(prm, X, power_mode, cus, st);
    case 64: return dispatch_metric<Launch, 64>(prm, X, power_mode, cus, st);
    case 128: return dispatch_metric<Launch, 128>(prm, X, power_mode, cus, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_solve(const SolveParams& prm, int group_size, int power_mode, int cus,
                        hipStream_t stream) {
  return dispatch_group<SolveLaunch>(prm, TensorStopParams{}, group_size, power_mode, cus, stream);
}

hipError_t launch_tensor_stop(const SolveParams& prm, const TensorStopParams& X, int group_size,
                              int power_mode, int cus, hipStream_t stream) {
  return dispatch_group<TensorStopLaunch>(prm, X, group_size, power_mode, cus, stream);
}

int64_t tensor_stop_workspace_bytes(int iters) {
  return kTensorStopHeader + (int64_t)sizeof(double) * (iters + 1) * 2 * kTensorStopMaxWaves;
}

hipError_t launch_dequant(const DequantParams& prm, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(hqq_dequant_kernel, dim3(blocks), dim3(kBlock), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace hqq
