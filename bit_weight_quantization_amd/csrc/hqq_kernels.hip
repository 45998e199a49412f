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
//   * every lane holds 16 consecutive fp16 weights (two 16-byte loads; a
//     wavefront reads 2 KB contiguous); group min/max run on the binary16 pairs.
//     The per-lane control of the solver (ballots, scalar state, group sums) is
//     spread over 16 weights;
//   * a group of G weights lives in a segment of L = G/16 adjacent lanes; a
//     wavefront holds S = 64/L groups; a lane sums its 16 terms as a binary
//     tree, and group sums/min/max are DPP butterflies inside the segment
//     (quad_perm, row_half_mirror), so every lane of a segment ends with the
//     bit-identical total;
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
//     its u values and header into an LDS done ring and takes a standby group.
//     Done groups are packed and written in dense batches.  A pass of the
//     iterating set runs once every segment holds a group (or nothing is left to
//     feed), so passes run on full wavefronts;
//   * a z update that leaves delta bit for bit unchanged would make the next
//     evaluation repeat the last one, which cannot improve: the group stops there
//     without evaluating it (same outputs);
//   * every group runs exactly the same instruction sequence whatever its batch or
//     slot, so results do not depend on the schedule.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqq_solver.h"

namespace hqq {
namespace {

// Per-wavefront LDS: u slots [0, kStandby) are the standby pool (groups past their
// first two evaluations, waiting for a free segment), u slots [kStandby, kStandby + S)
// the done ring (stopped groups waiting to be written).  A slot holds the G
// code-unit values u of a group; standby slots have a 12-word header (the full solver
// state), done slots an 8-word one.  The u values are stored as four planes of 16-byte
// chunks: chunk i of lane sl of a slot sits at plane i, position slot * L + sl.  A
// wavefront's accesses go to consecutive slots in lane order (pool, ring and take
// ranks, finalize segments), so consecutive lanes touch consecutive 16-byte chunks and
// each 16-byte access instruction is free of bank conflicts.
template <int G>
struct SolveLds {
  static constexpr int S = kWave * kLaneElems / G;
  static constexpr int L = G / kLaneElems;
  // Wavefronts per SIMD the kernel is compiled for (the VGPR budget: 128 registers).
  // A wavefront holds 1024 weights; its LDS share is the pool (S slots, 12-word header)
  // and the done ring (kDone slots, 8-word header) of G code-unit values each.  With a
  // ring of S slots at G = 16 and 32 only three blocks of four wavefronts would fit in a
  // CU's 160 KB, so there the ring has S/2 slots (40 KB per block at G = 16, 32 KB at
  // G = 32; 37 KB at G = 64, 35 KB at G = 128 with S slots): four blocks per CU at every
  // group size (measured: the fourth wavefront per SIMD is worth more than a deeper pool
  // or ring).  A hand-over larger than the ring is written straight from registers.
  static constexpr int kWavesPerSimd = 4;
  // A prime batch adds up to S groups to the pool, a hand-over up to S to the ring.
  static constexpr int kStandby = S;
  static constexpr int kDone = G <= 32 ? S / 2 : S;
  static constexpr int kSlots = kStandby + kDone;
  float4 u[kWavesPerBlock][kLaneElems / 4][kSlots * L];
  uint4 standby_hdr[kWavesPerBlock][kStandby][3];
  uint4 done_hdr[kWavesPerBlock][kDone][2];
};

// The wavefront's u planes: plane i, position slot * L + sl.
template <int G>
using UPlanes = float4 (*)[SolveLds<G>::kSlots * SolveLds<G>::L];

template <int G>
__device__ __forceinline__ void store_u(UPlanes<G> U, int slot, int sl, const float (&u)[kLaneElems]) {
  constexpr int L = G / kLaneElems;
#pragma unroll
  for (int i = 0; i < kLaneElems / 4; ++i)
    U[i][slot * L + sl] = make_float4(u[4 * i], u[4 * i + 1], u[4 * i + 2], u[4 * i + 3]);
}

template <int G>
__device__ __forceinline__ void load_u(UPlanes<G> U, int slot, int sl, float (&u)[kLaneElems]) {
  constexpr int L = G / kLaneElems;
#pragma unroll
  for (int i = 0; i < kLaneElems / 4; ++i) {
    const float4 a = U[i][slot * L + sl];
    u[4 * i] = a.x; u[4 * i + 1] = a.y; u[4 * i + 2] = a.z; u[4 * i + 3] = a.w;
  }
}

// Every group takes at least two evaluations (t = 0 is always accepted), so a wave
// runs them densely for S fresh groups at a time ("prime" batches): init and two
// solver steps in every segment.  Groups that stopped are written at once; the
// others wait in the standby pool for a segment of the iterating set.  Iterating
// segments whose group stops hand it to the done ring and take a standby group;
// done groups are written in dense batches.  Every group runs exactly the same
// instruction sequence whatever its batch or slot, so results do not depend on the
// schedule.
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
  // A batched launch reads weights through the device entry table only once that table
  // is shown to be the validated one (else nothing is written).  Wave-uniform returns:
  // the kernel has no block-wide barrier.
  if constexpr (BATCH) {
    if (!batch_table_matches(P)) return;
  }
  if (chunk * C >= P.ngroups) return;
  int64_t next = chunk * C;            // next group of the wave's queue
  int64_t q_end = next + C < P.ngroups ? next + C : P.ngroups;  // end of the current chunk

  UPlanes<G> U = lds.u[wid];
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
  LaneW prefetch = fetch_chunk<L, BATCH>(P, cursor, next + seg, q_end, sl);

  // Dense batch: segment j initializes group next + j and runs its first two steps.
  auto prime = [&]() {
    // In a batched launch the batch stops at the end of the cursor's entry.
    const int64_t avail = (BATCH && cursor.end < q_end ? cursor.end : q_end) - next;
    const int n = avail < S ? (int)avail : S;
    Slot a;
    a.active = a.pending = false;
    uint32_t nm_mx = 0u;
    const BatchCursor entry = cursor;  // the entry holding this batch (wave-uniform)
    if (seg < n) {
      a.gidx = next + seg;
      const GroupInit gq = init_group<L, false>(P, prefetch, a.u);
      a.s = gq.s;
      a.inv_s = gq.inv_s;
      a.z0 = gq.z0;
      a.usum = gq.usum;
      a.may_shrink = gq.may_shrink;
      a.delta = a.best_delta = a.e0 = 0.f;
      a.best_e = __builtin_inff();
      a.t = a.t_star = 0;
      a.active = true;
      nm_mx = gq.nm_mx;
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
    // t = 0: delta = 0, no clamp needed.  The evaluation also packs the codes rint(u)
    // (the output of every group that stops at t = 1) and finds u lying exactly on a
    // half-integer; those are settled from the raw weights (read again: the lane's two
    // chunks, from the batch's entry), and if one moved the wave recomputes the sums and
    // the evaluation.
    float e = 0.f, sq = 0.f;
    uint2 pk0 = make_uint2(0u, 0u);
    bool tie = false;
    if (a.active) tie = eval_first<L, PM>(a.u, P.nbits, P.p, e, sq, pk0);
    if (ballot(tie) != 0) {
      bool moved = false;
      if (tie) {
        const uint4* wp = BATCH ? entry.W + 2 * ((a.gidx - entry.first) * L + sl)
                                : P.W + 2 * (a.gidx * L + sl);
        moved = settle_ties(LaneW{wp[0], wp[1]}, nm_mx, P.qmax, a.u);
      }
      if (ballot(moved) != 0) {
        if (a.active) {
          a.usum = seg_sum<L>(tree_sum<0, kLaneElems>(a.u));
          eval_first<L, PM>(a.u, P.nbits, P.p, e, sq, pk0);
        }
      }
    }
    if (a.active) step_tail<L, PM>(P, a, e, sq);
    // t = 1, with the codes packed as well
    uint2 pk1 = make_uint2(0u, 0u);
    if (ballot(a.active) != 0) {
      if (ballot(needs_clamp(a)) != 0) {
        if (a.active) eval_group<L, PM, true, false, true>(a.u, a.delta, P.qmax, P.p, e, sq, P.nbits, &pk1);
      } else {
        if (a.active) eval_group<L, PM, false, false, true>(a.u, a.delta, P.qmax, P.p, e, sq, P.nbits, &pk1);
      }
      if (a.active) step_tail<L, PM>(P, a, e, sq);
    }
    // Groups stopping here have t* = 0 or 1: their codes are those of the first or the
    // second evaluation, already packed (8-bit codes are rounded again).  The clamp the
    // second evaluation applied or skipped gives the codes write_group gives at that z
    // (skipping it is exact for |delta| < 1/2).
    if (P.nbits != 8) {
      if (a.pending) {
        const uint2 pk = a.t_star == 0 ? pk0 : pk1;
        store_codes(P, a.gidx * L + sl, PackedCodes{{pk.x, pk.y, 0u, 0u}});
        if (sl == 0) write_meta<PM>(P, a.gidx, a.s, a.z0 + a.best_delta, a.e0, a.best_e, a.t_star);
      }
    } else {
      write_group_any<L, PM>(P, a.pending, sl, a.u, a.gidx, a.s, a.z0, a.best_delta, a.e0,
                             a.best_e, a.t_star);
    }
    const uint64_t m = ballot(a.active);
    if (a.active) {
      const int slot = n_standby + lanes_below(m) / L;  // n_standby <= kStandby - S
      store_u<G>(U, slot, sl, a.u);
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
      load_u<G>(U, slot, sl, sg.u);
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
    load_u<G>(U, slot, sl, uu);
    const uint4 h0 = D[slot - kStandby][0], h1 = D[slot - kStandby][1];
    write_group_any<L, PM>(P, write, sl, uu, (int64_t)(((uint64_t)h0.y << 32) | h0.x),
                           bitsf(h0.z), bitsf(h0.w), bitsf(h1.x), bitsf(h1.y), bitsf(h1.z),
                           (int)h1.w);
    done_head = uniform((int)((unsigned)(done_head + n) % (unsigned)kDone));
    done_count = uniform(done_count - n);
    wave_lds_sync();
  };

  // Each round of the loop runs one pass of the iterating set (a solver step of every
  // segment's group) once every segment holds a group, or when nothing is left to feed
  // the idle ones; otherwise it primes a batch (the pool is empty) and gives idle
  // segments standby groups first, so that passes run on full wavefronts.  A pass hands
  // stopped groups to the done ring and writes full done batches.  Every round makes
  // progress: it runs a pass, or primes (the queue advances), or hands out standby groups.
  while (true) {
    const bool any_active = ballot(sg.active) != 0;
    const bool feed = n_standby > 0 || next < q_end;  // groups left for idle segments
    if (!any_active && !feed) break;
    const bool full = __builtin_popcountll(ballot(sg.active || sg.pending)) == kWave;
    if (any_active && (full || !feed)) {
      const bool clamp = ballot(needs_clamp(sg)) != 0;
      if (sg.active) solver_step<L, PM>(P, sg, clamp);
    }

    // ---- stopped groups: hand them to the done ring ---------------------------
    const uint64_t pm = ballot(sg.pending);
    const int npend = __builtin_popcountll(pm) / L;
    if (npend > 0 && (npend >= P.refill_at || ballot(sg.active) == 0)) {
      if (done_count + npend > kDone) finalize(done_count);  // rare: make room first
      if (npend > kDone) {  // more than the ring holds: written straight from registers
        write_group_any<L, PM>(P, sg.pending, sl, sg.u, sg.gidx, sg.s, sg.z0, sg.best_delta, sg.e0,
                               sg.best_e, sg.t_star);
      } else if (sg.pending) {
        const int rank = lanes_below(pm) / L;
        const int slot = kStandby + (int)((unsigned)(done_head + done_count + rank) % (unsigned)kDone);
        store_u<G>(U, slot, sl, sg.u);
        if (sl == 0) {
          D[slot - kStandby][0] = make_uint4((uint32_t)sg.gidx, (uint32_t)(sg.gidx >> 32), fbits(sg.s),
                                      fbits(sg.z0));
          D[slot - kStandby][1] = make_uint4(fbits(sg.best_delta), fbits(sg.e0), fbits(sg.best_e),
                                      (uint32_t)sg.t_star);
        }
      }
      if (npend <= kDone) done_count = uniform(done_count + npend);
      sg.pending = false;
      wave_lds_sync();
      if (done_count >= kDone) finalize(kDone);
    }

    // ---- keep the pool stocked (a batch adds at most S), feed idle segments ------
    if (n_standby <= kStandby - S && next < q_end) prime();
    const bool idle = !sg.active && !sg.pending;
    if (n_standby > 0 && ballot(idle) != 0) take_standby(idle);
  }
  while (done_count > 0) finalize(done_count < kDone ? done_count : kDone);
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
    uint32_t c[kDequantElems];
    switch (P.nbits) {
      case 4: {
        const uint32_t v = reinterpret_cast<const uint32_t*>(P.packed)[chunk];
#pragma unroll
        for (int k = 0; k < kDequantElems; ++k) c[k] = (v >> (4 * k)) & 15u;
        break;
      }
      case 2: {
        const uint32_t v = reinterpret_cast<const uint16_t*>(P.packed)[chunk];
#pragma unroll
        for (int k = 0; k < kDequantElems; ++k) c[k] = (v >> (2 * k)) & 3u;
        break;
      }
      case 8: {  // two 4-byte words (the stream is 4-byte aligned)
        const uint32_t* src = reinterpret_cast<const uint32_t*>(P.packed) + 2 * chunk;
        const uint32_t v0 = src[0], v1 = src[1];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          c[k] = (v0 >> (8 * k)) & 255u;
          c[k + 4] = (v1 >> (8 * k)) & 255u;
        }
        break;
      }
      default: {
        const uint8_t* src = P.packed + chunk * 3;
        const uint32_t v = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16);
#pragma unroll
        for (int k = 0; k < kDequantElems; ++k) c[k] = (v >> (3 * k)) & 7u;
        break;
      }
    }
    uint16_t h[kDequantElems];
#pragma unroll
    for (int k = 0; k < kDequantElems; ++k) h[k] = dequant_one(s, sz, c[k]);
    uint4 o;
    o.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    o.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    o.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
    o.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
    P.out[chunk] = o;
  }
}

// Persistent grid: as many blocks as can be resident at once (LDS and VGPRs set the
// limit), or fewer for small inputs; the wavefronts deal the chunks round robin.  A chunk
// is 4 consecutive prime batches (measured faster than single batches once there are
// about 3 chunks per wavefront), or one when 4 would give fewer than 2 chunks per
// wavefront, so that a small input spreads over more wavefronts.
constexpr int kChunkBatches = 4;

template <int G, int PM>
struct SolveLaunch {
  static hipError_t run(SolveParams prm, const int&, int cus, hipStream_t st) {
    auto kernel = hqq_solve_kernel<G, PM, false>;
    if constexpr (err_mode(PM) == kErrP) {  // batched launches always use the lp error
      if (prm.batch) kernel = hqq_solve_kernel<G, PM, true>;
    }
    int64_t resident = 0;
    hipError_t err = resident_waves(kernel, cus, resident);
    if (err != hipSuccess) return err;
    constexpr int S = kWave * kLaneElems / G;
    prm.chunk_groups = kChunkBatches * S;
    int64_t nchunks = (prm.ngroups + prm.chunk_groups - 1) / prm.chunk_groups;
    if (nchunks < 2 * resident) {  // one prime batch per chunk: wider spread, finer balance
      prm.chunk_groups = S;
      nchunks = (prm.ngroups + S - 1) / S;
    }
    const int64_t nwaves = nchunks < resident ? nchunks : resident;
    const int64_t blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, prm);
    return hipGetLastError();
  }
};
}  // namespace

hipError_t launch_solve(const SolveParams& prm, int group_size, int power_mode, int cus,
                        hipStream_t stream) {
  return dispatch_group<SolveLaunch>(prm, 0, group_size, power_mode, cus, stream);
}

hipError_t launch_dequant(const DequantParams& prm, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(hqq_dequant_kernel, dim3(blocks), dim3(kBlock), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace hqq
