// hqq_lowrank.h -- launch interface of the low-rank compensation of the quantization
// error (hqq_lowrank.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hqq {

struct LowrankParams {
  // the weight and its stored quantization
  const uint16_t* W;        // m x n binary16
  const uint8_t* packed;
  const uint16_t* scale16;
  const uint16_t* zero16;
  int64_t m, n;             // multiples of 64
  int nbits, group_size, group_shift;
  // the randomized truncated SVD
  int rank;                 // r
  int width;                // l = r + oversample, a multiple of 32
  int power_iters;          // q
  const uint16_t* omega;    // l x n binary16 Gaussian test matrix (row-major)
  // outputs
  float* B;                 // m x r, row-major: U_r Sigma_r
  float* A;                 // r x n, row-major: V_r^T
  float* sigma;             // r singular values, decreasing
  void* workspace;          // lowrank_workspace_bytes(m, n, l) bytes
};

int64_t lowrank_workspace_bytes(int64_t m, int64_t n, int width);
hipError_t launch_lowrank(const LowrankParams& prm, int cus, hipStream_t stream);

// Delta W = W - s (W_q - z) as binary16, row-major (m x n) and transposed (n x m).
hipError_t launch_residual(const uint16_t* W, const uint8_t* packed, const uint16_t* scale16,
                           const uint16_t* zero16, int64_t m, int64_t n, int nbits, int group_size,
                           uint16_t* dW, uint16_t* dWT, hipStream_t stream);

}  // namespace hqq
