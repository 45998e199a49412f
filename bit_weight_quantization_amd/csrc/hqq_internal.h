// hqq_internal.h -- launch parameters shared by the host entry points and the
// gfx950 kernels of the HQQ quantizer.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hqq {

// How the lp power |x|^p is evaluated: general 0 < p < 1 through log2/exp2,
// or the two exact special cases p = 1 and p = 0.
enum PowerMode : int { kPowGeneral = 0, kPowOne = 1, kPowZero = 2 };
// Error metric of the early stop: the lp error with the solver's p, l1 or l2.
enum ErrMetric : int { kErrP = 0, kErrL1 = 1, kErrL2 = 2 };

// Device view of one hqq_batch_entry_t (same 32-byte layout).
struct BatchEntry {
  const uint4* W;          // fp16 weights viewed as 16-byte chunks of 8 halves
  int64_t rows, cols;
  int64_t first_group;     // global index of the matrix's first group
};

// Hash of a batch entry table, computed identically on the host (over the validated
// table) and on the device (over the copy the kernel reads): the sum over entries i of
// mix(mix(mix(mix(W + i) ^ rows) ^ cols) ^ first_group), with mix the SplitMix64
// finalizer (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
// 2014).  The entry index enters every term, so a reordered table changes the sum too.
__host__ __device__ inline uint64_t table_mix(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}
__host__ __device__ inline uint64_t table_entry_hash(uint64_t w, int64_t rows, int64_t cols,
                                                     int64_t first_group, int i) {
  uint64_t h = table_mix(w + (uint64_t)i);
  h = table_mix(h ^ (uint64_t)rows);
  h = table_mix(h ^ (uint64_t)cols);
  return table_mix(h ^ (uint64_t)first_group);
}

struct SolveParams {
  const uint4* W;          // fp16 weights viewed as 16-byte chunks of 8 halves (single matrix)
  const BatchEntry* batch; // device entry table (batched launch), else null
  int batch_count;
  uint64_t batch_hash;     // hash of the validated host table (batched launch)
  int32_t* batch_status;   // written by the batched launch: HQQ_OK or a table mismatch
  uint8_t* packed;         // packed code stream
  uint16_t* scale16;       // binary16 s per group
  uint16_t* zero16;        // binary16 z per group
  float* scale32;          // optional outputs (may be null)
  float* zero32;
  uint8_t* stop_step;
  float* err_init;
  float* err_best;
  int64_t ngroups;
  int64_t chunk_groups;    // groups per queue chunk, a multiple of S (set by the launcher)
  float qmax;
  float inv_qmax;          // 1/qmax rounded to fp32
  float p;                 // lp exponent
  float pm1;               // p - 1
  float pm2;               // p - 2
  float inv_beta0;         // 1 / beta_0
  float tau0;              // beta_0^(-1/(2-p)): the shrink is zero for |r| <= tau
  float log2_rho;          // log2 kappa^(-1/(2-p)): tau_t = tau0 * 2^(t log2_rho)
  float log2_kappa;        // 1/beta_t = (1/beta_0) * 2^(-t log2_kappa)
  float tau_min;           // smallest tau_t over the run
  int iters;
  int early_stop;
  int nbits;
  int refill_at;           // hand stopped groups over once this many segments are stopped
  int err_metric;          // ErrMetric of the early stop
};

struct DequantParams {
  const uint8_t* packed;
  const uint16_t* scale16;
  const uint16_t* zero16;
  uint4* out;              // fp16 output as 16-byte chunks of 8
  int64_t nchunks;         // elements / kDequantElems
  int chunks_per_group;    // group_size / kDequantElems
  int nbits;
};

// Launchers (return a hipError_t of the launch).
hipError_t launch_solve(const SolveParams& prm, int group_size, int power_mode, int cus,
                        hipStream_t stream);  // batched when prm.batch != nullptr
hipError_t launch_dequant(const DequantParams& prm, int blocks, hipStream_t stream);
// Meta quantization (M = 0: one group of all n values, using the workspace of
// 2 * kMetaPartials words for per-block partial minima and maxima).
constexpr int kMetaPartials = 1024;
hipError_t launch_meta_quantize(const uint16_t* values, int64_t n, int64_t M, uint8_t* codes,
                                uint16_t* mscale, uint16_t* moffset, uint32_t* workspace,
                                int cus, hipStream_t stream);
// One group per entry of a batched arena (n values, entry e starting at first_group).
hipError_t launch_meta_quantize_segments(const uint16_t* values, int64_t n,
                                         const BatchEntry* entries, int count, bool starts_mod8,
                                         uint8_t* codes, uint16_t* mscale, uint16_t* moffset,
                                         uint32_t* workspace, hipStream_t stream);
hipError_t launch_meta_dequantize(const uint8_t* codes, const uint16_t* mscale,
                                  const uint16_t* moffset, int64_t n, int64_t M, uint16_t* out,
                                  int cus, hipStream_t stream);

// Segment geometry shared with the host grid sizing: each solver lane holds 16 weights
// (two consecutive 16-byte chunks); the dequantization kernel handles 8 per lane.
constexpr int kLaneElems = 16;
constexpr int kDequantElems = 8;
constexpr int kWave = 64;
constexpr int kBlock = 256;

}  // namespace hqq
