// hqq_tensor_stop.hip -- gfx950 kernels of the whole-tensor early stop: the early exit
// of section 4.1 of "Half-Quadratic Quantization of Large Machine Learning Models"
// (Dropbox tech blog) read with the error of the whole matrix.  The solver step itself
// is the one of the per-group kernel (hqq_solver.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqq_solver.h"

namespace hqq {
namespace {

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
}  // namespace

hipError_t launch_tensor_stop(const SolveParams& prm, const TensorStopParams& X, int group_size,
                              int power_mode, int cus, hipStream_t stream) {
  return dispatch_group<TensorStopLaunch>(prm, X, group_size, power_mode, cus, stream);
}

int64_t tensor_stop_workspace_bytes(int iters) {
  return kTensorStopHeader + (int64_t)sizeof(double) * (iters + 1) * 2 * kTensorStopMaxWaves;
}

}  // namespace hqq
