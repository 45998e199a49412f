// hqq_matmul.h -- launch interface of the product with a quantized weight
// (hqq_matmul.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hqq {

struct MatmulParams {
  const uint16_t* X;        // M x K binary16 activations, row-major
  const uint8_t* packed;    // N x K codes, LSB-first bitstream over row-major elements
  const uint16_t* scale16;  // N x K/g binary16 s
  const uint16_t* zero16;   // N x K/g binary16 z
  void* Y;                  // M x N, binary16 or fp32
  int64_t M, N, K;
  int nbits, group_size;
  int group_shift;          // log2(group_size)
  int out_f32;
  float* part;              // split-K partial slabs (caller's workspace), or null
  int64_t slab;             // floats per partial slab: M*N rounded up to a multiple of 4
  int ksplit;               // splits of K (1: no partials)
};

// Rows of X up to which the wavefront-per-row kernel is used (kGemvAlignedMaxRows where
// the aligned skinny kernel applies: 2-, 4-, 8-bit codes, groups of 32-128, K a multiple
// of 256, 16-byte aligned s and z), and up to which a skinny matrix-core kernel is used
// above that (then the tiled matrix-core kernel).
constexpr int kGemvMaxRows = 8;
constexpr int kGemvAlignedMaxRows = 2;
constexpr int kSkinnyMaxRows = 64;
constexpr int kSplitMinRows = 16;  // above this (and up to kSkinnyMaxRows) K is split

// Bytes of workspace the product needs for these shapes (the split-K partial slabs of
// the skinny path; 0 when the path writes Y directly).  Depends on the shapes only.
int64_t matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, int nbits, int group_size);

// `prm.part` must hold matmul_workspace_bytes(...) bytes where that is not 0.
hipError_t launch_matmul(MatmulParams prm, int cus, hipStream_t stream);

}  // namespace hqq
