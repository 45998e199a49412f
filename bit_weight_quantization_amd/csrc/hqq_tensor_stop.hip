// hqq_tensor_stop.hip -- gfx950 kernels of the whole-tensor early stop: the early exit
// of section 4.1 of "Half-Quadratic Quantization of Large Machine Learning Models"
// (Dropbox tech blog) read with the error of the whole matrix.  The solver step itself
// is the one of the per-group kernel (hqq_solver.h).
//
// The error that must keep improving is E_t = sum over all groups of e_t (weight
// units), and every group returns the z of the same step t*, the end of the strictly
// decreasing run E_0 > E_1 > ... > E_t*.  Without a per-group stop every group takes
// the same steps, so a wavefront iterates S groups in lockstep and no standby pool is
// needed:
//   pass 1 (ACC): every group runs steps 0 .. iters; each wavefront adds its groups'
//     step errors into fp64 totals (two lanes per step, each over half of the
//     wavefront's groups), and each block writes its total of every step;
//   totals: one block per step adds the block partials in a fixed order;
//   pass 2 (OUT): every wavefront derives t* from the totals, and every group runs t*
//     updates and writes its outputs: the per-group solver with the stop switched off
//     and iters = t*, step for step.
// A group that cannot shrink (its range is below every threshold of the run) and whose
// update left z bit-for-bit unchanged has reached a fixed point: its codes, error and z
// repeat at every later step.  Once every group of a wavefront is there, the wavefront
// stops iterating; pass 1 repeats each group's last error for the remaining steps and
// pass 2 takes the last z, which is what the remaining steps would give.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqq_solver.h"
#include "hqq_tensor_stop.h"

namespace hqq {
namespace {

constexpr int kStepRows = 32;  // step errors buffered in LDS between folds

template <int G, int PM, bool OUT>
__global__ __launch_bounds__(kBlock) void hqq_lockstep_kernel(const SolveParams P,
                                                              const TensorStopParams X) {
  constexpr int L = G / kLaneElems;
  constexpr int S = kWave / L;
  constexpr int kHalf = S / 2;  // groups folded by one lane
  constexpr int kRow = S + 4;   // floats per LDS row: 16-byte aligned, rows 4 banks apart
  constexpr int kAcc = kTensorStopMaxSteps / kStepRows;
  __shared__ __align__(16) float ebuf[kWavesPerBlock][OUT ? 1 : kStepRows][OUT ? 4 : kRow];
  __shared__ double red[kWavesPerBlock][OUT ? 1 : kWave];

  const int wid = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int seg = lane / L;
  const int sl = lane & (L - 1);
  const int64_t wave = uniform64(((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t nbatches = (P.ngroups + S - 1) / S;
  SolveParams Q = P;
  Q.early_stop = 0;
  if constexpr (OUT) {
    // t*: the end of the strictly decreasing run of the totals (every wavefront reads
    // the same values and reaches the same t*)
    int ts = 0;
    while (ts < P.iters && X.totals_ws[ts + 1] < X.totals_ws[ts]) ++ts;
    Q.iters = uniform(ts);
    if (X.t_star_out && blockIdx.x == 0 && threadIdx.x == 0) *X.t_star_out = Q.iters;
  }
  const int T = Q.iters;

  // Lane l folds half l / kStepRows of row l % kStepRows: acc[k] is its share of the
  // wavefront's total of step kStepRows * k + l % kStepRows.
  const int fold_row = lane & (kStepRows - 1);
  const int fold_half = lane / kStepRows;
  double acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = 0.0;

  // Pass 1: the segment's weighted error of step t into LDS row t % kStepRows; full
  // windows (and the last step) are folded into the fp64 totals.
  auto record = [&](int t, float ew) {
    const int r = t & (kStepRows - 1);
    if (sl == 0) ebuf[wid][r][seg] = ew;
    if (r == kStepRows - 1 || t == T) {
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
  };

  for (int64_t b = wave; b < nbatches; b += nwaves) {
    const int64_t g0 = b * S;
    const int64_t left = P.ngroups - g0;
    const int n = left < S ? (int)left : S;
    // Every lane loads (a segment past the end reads the batch's first group).
    const uint4* wp = P.W + 2 * ((seg < n ? g0 + seg : g0) * L + sl);
    const LaneW raw = {wp[0], wp[1]};
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
      const uint32_t before = fbits(a.delta);
      float e = 0.f;
      if (t == 0) {
        if (a.active) e = solver_step<L, PM, true>(Q, a, false);
      } else {
        const bool clamp = ballot(needs_clamp(a)) != 0;
        if (a.active) e = solver_step<L, PM>(Q, a, clamp);
      }
      if constexpr (!OUT) record(t, e * sp);  // 0 for a segment without a group
      const bool moving = a.active && (a.may_shrink || fbits(a.delta) != before);
      if (t < T && ballot(moving) == 0) {  // every group at a fixed point after step t
        if constexpr (OUT) {
          if (a.active) {  // the state the remaining accepted steps would leave
            a.best_e = e;
            a.best_delta = a.delta;
            a.t = a.t_star = T;
            a.active = false;
            a.pending = true;
          }
        } else {
          for (int t2 = t + 1; t2 <= T; ++t2) record(t2, e * sp);
        }
        break;
      }
    }
    if constexpr (OUT) {
      write_group_any<L, PM>(Q, a.pending, sl, a.u, a.gidx, a.s, a.z0, a.best_delta, a.e0,
                             a.best_e, a.t_star);
    }
  }
  if constexpr (!OUT) {
    // The block's total of every step, in a fixed order (per wavefront the two halves,
    // then the wavefronts in order), into the partials.  T is uniform over the grid, so
    // every wavefront reaches every barrier.
#pragma unroll
    for (int k = 0; k < kAcc; ++k) {
      if (k * kStepRows > T) break;
      red[wid][lane] = acc[k];
      __syncthreads();
      const int t = k * kStepRows + lane;
      if (wid == 0 && lane < kStepRows && t <= T) {
        double s = 0.0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) s += red[w][lane] + red[w][lane + kStepRows];
        X.partials[(int64_t)t * X.nblocks + blockIdx.x] = s;
      }
      __syncthreads();
    }
  }
}

// E_t for t = blockIdx.x: the block partials of step t added in a fixed order (four
// strided per-thread sums, then a tree in LDS).
__global__ __launch_bounds__(kBlock) void hqq_tensor_total_kernel(const TensorStopParams X) {
  __shared__ double red[kBlock];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const double* row = X.partials + (int64_t)t * X.nblocks;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int64_t b = tid;
  for (; b + 3 * kBlock < X.nblocks; b += 4 * kBlock) {
    s0 += row[b];
    s1 += row[b + kBlock];
    s2 += row[b + 2 * kBlock];
    s3 += row[b + 3 * kBlock];
  }
  for (; b < X.nblocks; b += kBlock) s0 += row[b];
  red[tid] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  for (int h = kBlock / 2; h > 0; h >>= 1) {
    if (tid < h) red[tid] += red[tid + h];
    __syncthreads();
  }
  if (tid == 0) {
    X.totals_ws[t] = red[0];
    if (X.totals) X.totals[t] = red[0];
  }
}

// Pass 1, the totals and pass 2 of the whole-tensor stop, in stream order.
template <int G, int PM>
struct TensorStopLaunch {
  static hipError_t run(const SolveParams& prm, TensorStopParams X, int cus, hipStream_t st) {
    constexpr int S = kWave * kLaneElems / G;
    const int64_t nbatches = (prm.ngroups + S - 1) / S;
    const int64_t batch_blocks = (nbatches + kWavesPerBlock - 1) / kWavesPerBlock;
    auto acc_kernel = hqq_lockstep_kernel<G, PM, false>;
    auto out_kernel = hqq_lockstep_kernel<G, PM, true>;
    int64_t resident = 0;
    hipError_t err = resident_waves(acc_kernel, cus, resident);
    if (err != hipSuccess) return err;
    int64_t blocks = resident / kWavesPerBlock;
    if (blocks > batch_blocks) blocks = batch_blocks;
    if (blocks > kTensorStopMaxBlocks) blocks = kTensorStopMaxBlocks;
    X.nblocks = blocks;
    hipLaunchKernelGGL(acc_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, prm, X);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(hqq_tensor_total_kernel, dim3(prm.iters + 1), dim3(kBlock), 0, st, X);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    err = resident_waves(out_kernel, cus, resident);
    if (err != hipSuccess) return err;
    blocks = resident / kWavesPerBlock;
    if (blocks > batch_blocks) blocks = batch_blocks;
    hipLaunchKernelGGL(out_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, prm, X);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_tensor_stop(const SolveParams& prm, const TensorStopParams& X, int group_size,
                              int power_mode, int cus, hipStream_t stream) {
  return dispatch_group<TensorStopLaunch>(prm, X, group_size, power_mode, cus, stream);
}

int64_t tensor_stop_workspace_bytes(int iters) {
  return kTensorStopHeader + (int64_t)sizeof(double) * (iters + 1) * kTensorStopMaxBlocks;
}

}  // namespace hqq
