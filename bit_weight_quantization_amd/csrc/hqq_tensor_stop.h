// hqq_tensor_stop.h -- launch interface of the whole-tensor early stop
// (hqq_tensor_stop.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqq_internal.h"

namespace hqq {

// Workspace of the whole-tensor stop (owned by the caller): the totals E_0 .. E_iters in
// its first kTensorStopHeader bytes, then the per-block partial totals of pass 1.
constexpr int kTensorStopMaxSteps = 256;  // iters <= 255
constexpr int64_t kTensorStopHeader = kTensorStopMaxSteps * (int64_t)sizeof(double);
constexpr int kTensorStopMaxBlocks = 2048;  // blocks of pass 1 at most

struct TensorStopParams {
  double* partials;        // [iters + 1][nblocks] fp64 partial totals of pass 1
  int64_t nblocks;         // blocks of pass 1 (set by the launcher)
  double* totals_ws;       // E_0 .. E_iters in the workspace (written by the decision)
  double* totals;          // optional copy of E_0 .. E_iters for the caller
  int* t_star_out;         // optional t*
};

// Pass 1, the totals and pass 2 on `stream`.
hipError_t launch_tensor_stop(const SolveParams& prm, const TensorStopParams& X, int group_size,
                              int power_mode, int cus, hipStream_t stream);
int64_t tensor_stop_workspace_bytes(int iters);

}  // namespace hqq
