// hqq_valu_probe.hip -- issue-rate probe of the gfx950 VALU instruction classes the
// quantizer's solver spends its time in (plain fp32 add / mul / fma, round-to-even,
// median-of-three, conversions, compares, selects, lane permutes, and the
// transcendental v_exp_f32 / v_log_f32 / v_rcp_f32), alone and in mixes (the
// instruction mix of one solver evaluation among them).
//
// Measurement library, separate from the quantizer (libhqq_valu_probe.so): the
// benchmark uses it to state the per-class peaks its VALU roofline is priced against.
// Every thread runs 8 independent chains of one instruction (inline assembly, so the
// compiler can neither fold nor pack them), 64 instructions per loop trip; a launch
// of many wavefronts per SIMD hides the instruction latency, so the launch time over
// the number of wave-instructions issued gives the SIMD cycles per wave-instruction.
// Only single-lane fp32 forms are issued (no packed fp32).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

enum Kind : int {
  kAdd = 0, kMul, kFma, kRndne, kMed3, kExp, kLog, kRcp,
  kMax, kFract, kCndmask, kCmp, kCvtF16, kFmaMix, kAddU32, kBfi, kPerm, kDppMov, kPkMaxF16,
  kCndmaskSgpr,
  // mixes over the 8 chains of a round (instruction of chain 0, 1, ..., 7):
  kMixRndneAdd,    // rndne, add, rndne, add, ...: half-rate with simple ops 1:1
  kMixExpAdd,      // exp, add, exp, add, ...: quarter-rate with simple ops 1:1
  kMixExpAdd3,     // exp, add, add, add, exp, add, add, add
  kMixEval,        // log, add, add, exp, add, rndne, add, mul: one solver evaluation's mix
  kKinds
};

template <int KIND>
__device__ __forceinline__ void op(float& a, float c, float d) {
  if constexpr (KIND == kAdd) asm volatile("v_add_f32 %0, %0, %1" : "+v"(a) : "v"(c));
  else if constexpr (KIND == kMul) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(a) : "v"(c));
  else if constexpr (KIND == kFma) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a) : "v"(c), "v"(d));
  else if constexpr (KIND == kRndne) asm volatile("v_rndne_f32 %0, %0" : "+v"(a));
  else if constexpr (KIND == kMed3) asm volatile("v_med3_f32 %0, %0, %1, %2" : "+v"(a) : "v"(c), "v"(d));
  else if constexpr (KIND == kExp) asm volatile("v_exp_f32 %0, %0" : "+v"(a));
  else if constexpr (KIND == kLog) asm volatile("v_log_f32 %0, %0" : "+v"(a));
  else if constexpr (KIND == kRcp) asm volatile("v_rcp_f32 %0, %0" : "+v"(a));
  else if constexpr (KIND == kMax) asm volatile("v_max_f32 %0, %0, %1" : "+v"(a) : "v"(c));
  else if constexpr (KIND == kFract) asm volatile("v_fract_f32 %0, %0" : "+v"(a));
  // the mask is all lanes false (vcc cleared once per chain op): a plain select
  else if constexpr (KIND == kCndmask) asm volatile("v_cndmask_b32 %0, %0, %1, vcc" : "+v"(a) : "v"(c));
  else if constexpr (KIND == kCmp) asm volatile("v_cmp_lt_f32 vcc, %0, %1" : : "v"(a), "v"(c) : "vcc");
  else if constexpr (KIND == kCvtF16) asm volatile("v_cvt_f32_f16 %0, %0" : "+v"(a));
  else if constexpr (KIND == kFmaMix) asm volatile("v_fma_mix_f32 %0, %0, %1, %2 op_sel_hi:[1,0,0]" : "+v"(a) : "v"(c), "v"(d));
  else if constexpr (KIND == kAddU32) asm volatile("v_add_u32 %0, %0, %1" : "+v"(a) : "v"(c));
  else if constexpr (KIND == kBfi) asm volatile("v_bfi_b32 %0, %0, %1, %2" : "+v"(a) : "v"(c), "v"(d));
  else if constexpr (KIND == kPerm) asm volatile("v_perm_b32 %0, %0, %1, %2" : "+v"(a) : "v"(c), "v"(d));
  else if constexpr (KIND == kDppMov) asm volatile("v_mov_b32_dpp %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "+v"(a));
  else if constexpr (KIND == kPkMaxF16) asm volatile("v_pk_max_f16 %0, %0, %1" : "+v"(a) : "v"(c));
  else asm volatile("v_cndmask_b32_e64 %0, %0, %1, s[40:41]" : "+v"(a) : "v"(c) : "s40", "s41");
}

// The instruction of chain J in a mixed kind (or the kind itself).
template <int KIND, int J>
constexpr int chain_kind() {
  if constexpr (KIND == kMixRndneAdd) return J % 2 == 0 ? kRndne : kAdd;
  else if constexpr (KIND == kMixExpAdd) return J % 2 == 0 ? kExp : kAdd;
  else if constexpr (KIND == kMixExpAdd3) return J % 4 == 0 ? kExp : kAdd;
  else if constexpr (KIND == kMixEval) {
    constexpr int k[8] = {kLog, kAdd, kAdd, kExp, kAdd, kRndne, kAdd, kMul};
    return k[J];
  } else return KIND;
}

// 64 instructions per trip: 8 rounds over 8 independent chains.
template <int KIND>
__global__ __launch_bounds__(256) void valu_probe_kernel(float* __restrict__ out, int trips,
                                                         float seed) {
  const float c = seed * 0.5f, d = seed + 1.0f;
  if constexpr (KIND == kCndmask) asm volatile("s_mov_b64 vcc, 0" : : : "vcc");
  if constexpr (KIND == kCndmaskSgpr) asm volatile("s_mov_b64 s[40:41], 0" : : : "s40", "s41");
  float a0 = seed + 1e-7f * (float)threadIdx.x, a1 = a0 + 0.125f, a2 = a0 + 0.25f,
        a3 = a0 + 0.375f, a4 = a0 + 0.5f, a5 = a0 + 0.625f, a6 = a0 + 0.75f, a7 = a0 + 0.875f;
  for (int i = 0; i < trips; ++i) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      op<chain_kind<KIND, 0>()>(a0, c, d);
      op<chain_kind<KIND, 1>()>(a1, c, d);
      op<chain_kind<KIND, 2>()>(a2, c, d);
      op<chain_kind<KIND, 3>()>(a3, c, d);
      op<chain_kind<KIND, 4>()>(a4, c, d);
      op<chain_kind<KIND, 5>()>(a5, c, d);
      op<chain_kind<KIND, 6>()>(a6, c, d);
      op<chain_kind<KIND, 7>()>(a7, c, d);
    }
  }
  // one store per thread keeps every chain live
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = ((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7));
}

template <int KIND>
hipError_t launch(int blocks, int trips, float* out, hipStream_t st) {
  hipLaunchKernelGGL(valu_probe_kernel<KIND>, dim3(blocks), dim3(256), 0, st, out, trips, 0.75f);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Number of instruction kinds; kind k's name is hqq_probe_kind_name(k).
int hqq_probe_kinds(void) { return kKinds; }

const char* hqq_probe_kind_name(int kind) {
  static const char* names[kKinds] = {"v_add_f32", "v_mul_f32", "v_fma_f32", "v_rndne_f32",
                                      "v_med3_f32", "v_exp_f32", "v_log_f32", "v_rcp_f32",
                                      "v_max_f32", "v_fract_f32", "v_cndmask_b32",
                                      "v_cmp_lt_f32", "v_cvt_f32_f16", "v_fma_mix_f32",
                                      "v_add_u32", "v_bfi_b32", "v_perm_b32", "v_mov_b32_dpp",
                                      "v_pk_max_f16", "v_cndmask_b32_e64 (sgpr mask)",
                                      "mix rndne:add 1:1", "mix exp:add 1:1", "mix exp:add 1:3",
                                      "mix of one evaluation (log, exp, rndne, mul, 4 add)"};
  return kind >= 0 && kind < kKinds ? names[kind] : "";
}

// Instructions of the probed kind issued per wavefront per loop trip.
int hqq_probe_instr_per_trip(void) { return 64; }

// Launches `blocks` blocks of 256 threads (4 wavefronts), each thread running `trips`
// loop trips of instruction `kind`; `out` receives blocks * 256 floats (device memory).
// Returns 0, 1 for invalid arguments, 4 if the launch failed.  Asynchronous on `stream`.
int hqq_probe_valu(int kind, int blocks, int trips, float* out, void* stream) {
  if (kind < 0 || kind >= kKinds || blocks <= 0 || trips <= 0 || !out) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (kind) {
    case kAdd: e = launch<kAdd>(blocks, trips, out, st); break;
    case kMul: e = launch<kMul>(blocks, trips, out, st); break;
    case kFma: e = launch<kFma>(blocks, trips, out, st); break;
    case kRndne: e = launch<kRndne>(blocks, trips, out, st); break;
    case kMed3: e = launch<kMed3>(blocks, trips, out, st); break;
    case kExp: e = launch<kExp>(blocks, trips, out, st); break;
    case kLog: e = launch<kLog>(blocks, trips, out, st); break;
    case kRcp: e = launch<kRcp>(blocks, trips, out, st); break;
    case kMax: e = launch<kMax>(blocks, trips, out, st); break;
    case kFract: e = launch<kFract>(blocks, trips, out, st); break;
    case kCndmask: e = launch<kCndmask>(blocks, trips, out, st); break;
    case kCmp: e = launch<kCmp>(blocks, trips, out, st); break;
    case kCvtF16: e = launch<kCvtF16>(blocks, trips, out, st); break;
    case kFmaMix: e = launch<kFmaMix>(blocks, trips, out, st); break;
    case kAddU32: e = launch<kAddU32>(blocks, trips, out, st); break;
    case kBfi: e = launch<kBfi>(blocks, trips, out, st); break;
    case kPerm: e = launch<kPerm>(blocks, trips, out, st); break;
    case kDppMov: e = launch<kDppMov>(blocks, trips, out, st); break;
    case kPkMaxF16: e = launch<kPkMaxF16>(blocks, trips, out, st); break;
    case kCndmaskSgpr: e = launch<kCndmaskSgpr>(blocks, trips, out, st); break;
    case kMixRndneAdd: e = launch<kMixRndneAdd>(blocks, trips, out, st); break;
    case kMixExpAdd: e = launch<kMixExpAdd>(blocks, trips, out, st); break;
    case kMixExpAdd3: e = launch<kMixExpAdd3>(blocks, trips, out, st); break;
    default: e = launch<kMixEval>(blocks, trips, out, st); break;
  }
  return e == hipSuccess ? 0 : 4;
}

}  // extern "C"
