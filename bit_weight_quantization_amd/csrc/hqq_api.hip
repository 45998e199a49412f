// hqq_api.hip -- extern "C" entry points of the HQQ quantizer (see include/hqq.h):
// argument validation, grid sizing and the launch on the caller's stream.
// No allocation, no synchronization.  The only global state is the device-resident
// scratch of hqq_quantize_tensor_stop_noalloc and its per-device address, looked up once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/hqq.h"
#include "hqq_internal.h"
#include "hqq_lowrank.h"
#include "hqq_matmul.h"
#include "hqq_tensor_stop.h"

namespace {

constexpr int kMaxIters = 255;
constexpr int64_t kMaxMetaGroup = 1 << 20;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool supported_nbits(int nbits) { return nbits == 2 || nbits == 3 || nbits == 4 || nbits == 8; }

bool supported_group(int g) { return g == 16 || g == 32 || g == 64 || g == 128; }

// rows*cols without overflow (both >= 0); -1 on overflow.
int64_t checked_elems(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return -1;
  if (rows != 0 && cols > INT64_MAX / 8 / rows) return -1;  // keep *nbits and *2 bytes in range
  return rows * cols;
}

int compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

int validate_common(int64_t rows, int64_t cols, int nbits, int group_size) {
  if (checked_elems(rows, cols) < 0) return HQQ_ERR_INVALID_ARG;
  if (!supported_nbits(nbits) || !supported_group(group_size)) return HQQ_ERR_UNSUPPORTED;
  if (cols % group_size != 0) return HQQ_ERR_INVALID_ARG;
  return HQQ_OK;
}

int validate_solver(float p, float beta, float kappa, int iters) {
  if (!(p >= 0.0f && p <= 1.0f)) return HQQ_ERR_INVALID_ARG;
  if (!(beta > 0.0f) || !isfinite(beta)) return HQQ_ERR_INVALID_ARG;
  if (!(kappa > 0.0f) || !isfinite(kappa)) return HQQ_ERR_INVALID_ARG;
  if (iters < 0 || iters > kMaxIters) return HQQ_ERR_INVALID_ARG;
  return HQQ_OK;
}

// Solver constants shared by the single-matrix and batched entry points.
void set_solver_params(hqq::SolveParams& prm, int nbits, int group_size, float p, float beta,
                       float kappa, int iters, int early_stop, int refill_threshold,
                       int err_metric) {
  const int slots = hqq::kWave * hqq::kLaneElems / group_size;  // groups resident in a wavefront
  prm.qmax = (float)((1 << nbits) - 1);
  prm.inv_qmax = (float)(1.0 / (double)((1 << nbits) - 1));
  prm.p = p;
  prm.pm1 = p - 1.0f;
  prm.pm2 = p - 2.0f;
  prm.inv_beta0 = (float)(1.0 / (double)beta);
  // The shrink of section 2.1 vanishes for |x|^(2-p) <= 1/beta, i.e. |x| <= beta^(-1/(2-p)).
  const double tau0 = pow((double)beta, -1.0 / (2.0 - (double)p));
  const double log2_rho = -log2((double)kappa) / (2.0 - (double)p);
  prm.tau0 = (float)tau0;
  prm.log2_rho = (float)log2_rho;
  prm.log2_kappa = (float)log2((double)kappa);
  prm.tau_min = (float)(log2_rho < 0.0 ? tau0 * exp2(log2_rho * iters) : tau0);
  prm.iters = iters;
  prm.early_stop = early_stop;
  prm.nbits = nbits;
  const int refill = refill_threshold > 0 ? refill_threshold : 1;
  prm.refill_at = refill > slots ? slots : refill;
  prm.err_metric = err_metric;
}

int power_mode_of(float p) {
  return p == 1.0f ? hqq::kPowOne : (p == 0.0f ? hqq::kPowZero : hqq::kPowGeneral);
}

// hqq_options_t with its defaults filled in (opt may be NULL), validated.
int read_options(const hqq_options_t* opt, hqq_options_t& o) {
  o = {1, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};
  if (!opt) return HQQ_OK;
  o = *opt;
  if (o.early_stop != 0 && o.early_stop != 1) return HQQ_ERR_INVALID_ARG;
  if (o.refill_threshold < 0) return HQQ_ERR_INVALID_ARG;
  if (o.err_metric < 0 || o.err_metric > 2) return HQQ_ERR_INVALID_ARG;
  if ((o.scale_f32 && !aligned(o.scale_f32, 4)) || (o.zero_f32 && !aligned(o.zero_f32, 4)) ||
      (o.err_init && !aligned(o.err_init, 4)) || (o.err_best && !aligned(o.err_best, 4)))
    return HQQ_ERR_ALIGNMENT;
  return HQQ_OK;
}

// Launch parameters of one matrix with the outputs of `o`.
hqq::SolveParams single_matrix_params(const void* W_f16, int64_t n, int nbits, int group_size,
                                      float p, float beta, float kappa, int iters,
                                      void* packed_codes, void* scale_f16, void* zero_f16,
                                      const hqq_options_t& o) {
  hqq::SolveParams prm = {};
  prm.W = static_cast<const uint4*>(W_f16);
  prm.batch = nullptr;
  prm.batch_count = 0;
  prm.packed = static_cast<uint8_t*>(packed_codes);
  prm.scale16 = static_cast<uint16_t*>(scale_f16);
  prm.zero16 = static_cast<uint16_t*>(zero_f16);
  prm.scale32 = o.scale_f32;
  prm.zero32 = o.zero_f32;
  prm.stop_step = o.stop_step;
  prm.err_init = o.err_init;
  prm.err_best = o.err_best;
  prm.ngroups = n / group_size;
  set_solver_params(prm, nbits, group_size, p, beta, kappa, iters, o.early_stop,
                    o.refill_threshold, o.err_metric);
  return prm;
}

// Checks shared by the single-matrix solver entry points; `n` receives rows * cols.
int validate_single(const void* W_f16, int64_t rows, int64_t cols, int nbits, int group_size,
                    float p, float beta, float kappa, int iters, const void* packed_codes,
                    const void* scale_f16, const void* zero_f16, int64_t& n) {
  int st = validate_common(rows, cols, nbits, group_size);
  if (st != HQQ_OK) return st;
  st = validate_solver(p, beta, kappa, iters);
  if (st != HQQ_OK) return st;
  n = rows * cols;
  if (n == 0) return HQQ_OK;
  if (!W_f16 || !packed_codes || !scale_f16 || !zero_f16) return HQQ_ERR_INVALID_ARG;
  if (!aligned(W_f16, 16) || !aligned(packed_codes, 4) || !aligned(scale_f16, 2) ||
      !aligned(zero_f16, 2))
    return HQQ_ERR_ALIGNMENT;
  return HQQ_OK;
}

}  // namespace

extern "C" {

const char* hqq_status_string(int status) {
  switch (status) {
    case HQQ_OK: return "ok";
    case HQQ_ERR_INVALID_ARG: return "invalid argument";
    case HQQ_ERR_UNSUPPORTED: return "unsupported nbits or group_size";
    case HQQ_ERR_ALIGNMENT: return "misaligned pointer";
    case HQQ_ERR_LAUNCH: return "kernel launch failed";
    case HQQ_ERR_TABLE_MISMATCH: return "device entry table differs from the host table";
    default: return "unknown status";
  }
}

int64_t hqq_packed_bytes(int64_t rows, int64_t cols, int nbits) {
  const int64_t n = checked_elems(rows, cols);
  if (n < 0 || !supported_nbits(nbits)) return -1;
  return (n * nbits + 7) / 8;
}

int64_t hqq_num_groups(int64_t rows, int64_t cols, int group_size) {
  const int64_t n = checked_elems(rows, cols);
  if (n < 0 || !supported_group(group_size) || cols % group_size != 0) return -1;
  return n / group_size;
}

int hqq_quantize_ex(const void* W_f16, int64_t rows, int64_t cols, int nbits, int group_size,
                    float p, float beta, float kappa, int iters, void* packed_codes,
                    void* scale_f16, void* zero_f16, const hqq_options_t* opt, void* stream) {
  int64_t n = 0;
  int st = validate_single(W_f16, rows, cols, nbits, group_size, p, beta, kappa, iters,
                           packed_codes, scale_f16, zero_f16, n);
  if (st != HQQ_OK || n == 0) return st;
  hqq_options_t o;
  st = read_options(opt, o);
  if (st != HQQ_OK) return st;
  const hqq::SolveParams prm = single_matrix_params(W_f16, n, nbits, group_size, p, beta, kappa,
                                                    iters, packed_codes, scale_f16, zero_f16, o);
  int cus = compute_units();
  if (cus <= 0) return HQQ_ERR_LAUNCH;
  hipError_t err = hqq::launch_solve(prm, group_size, power_mode_of(p), cus,
                                     static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

int64_t hqq_tensor_stop_workspace_bytes(int iters) {
  if (iters < 0 || iters > kMaxIters) return -1;
  return hqq::tensor_stop_workspace_bytes(iters);
}

int hqq_quantize_tensor_stop(const void* W_f16, int64_t rows, int64_t cols, int nbits,
                             int group_size, float p, float beta, float kappa, int iters,
                             void* packed_codes, void* scale_f16, void* zero_f16,
                             const hqq_options_t* opt, void* totals_f64, void* t_star_i32,
                             void* workspace, void* stream) {
  int64_t n = 0;
  int st = validate_single(W_f16, rows, cols, nbits, group_size, p, beta, kappa, iters,
                           packed_codes, scale_f16, zero_f16, n);
  if (st != HQQ_OK || n == 0) return st;
  hqq_options_t o;
  st = read_options(opt, o);
  if (st != HQQ_OK) return st;
  if (!workspace) return HQQ_ERR_INVALID_ARG;
  if (!aligned(workspace, 8) || (totals_f64 && !aligned(totals_f64, 8)) ||
      (t_star_i32 && !aligned(t_star_i32, 4)))
    return HQQ_ERR_ALIGNMENT;
  o.early_stop = 0;  // pass 2 runs the t* updates without a stop
  o.refill_threshold = 0;
  const hqq::SolveParams prm = single_matrix_params(W_f16, n, nbits, group_size, p, beta, kappa,
                                                    iters, packed_codes, scale_f16, zero_f16, o);
  hqq::TensorStopParams X = {};
  X.totals_ws = static_cast<double*>(workspace);
  X.partials = reinterpret_cast<double*>(static_cast<char*>(workspace) + hqq::kTensorStopHeader);
  X.totals = static_cast<double*>(totals_f64);
  X.t_star_out = static_cast<int*>(t_star_i32);
  int cus = compute_units();
  if (cus <= 0) return HQQ_ERR_LAUNCH;
  hipError_t err = hqq::launch_tensor_stop(prm, X, group_size, power_mode_of(p), cus,
                                           static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

}  // extern "C"

// ---- hqq_quantize_tensor_stop_noalloc: the tensor stop's scratch as a static device array --
//
// The whole-tensor stop needs per-block partial totals and the totals themselves between
// its kernels (hqq_tensor_stop_workspace_bytes(iters) bytes, 4 MiB at iters = 255).  For
// callers that cannot allocate, that scratch is a file-scope device array, one copy per
// GPU, sized for the largest iters.  In host code the array's name is only a stand-in,
// so its device address is looked up once per device with hipGetSymbolAddress (on the
// first call on that device, with that device current) and every launch uses that
// address.  Calls on one GPU share the array: calls that may overlap on one GPU race.
// Every byte the kernels read is written earlier in the same call, so nothing has to be
// cleared between calls.
namespace {

constexpr int64_t kNoallocScratchBytes = (int64_t)hqq::kTensorStopHeader +
                                         (int64_t)sizeof(double) * (kMaxIters + 1) *
                                             hqq::kTensorStopMaxBlocks;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// The calling thread's current device's copy of `scratch` (null if the lookup failed).
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(scratch_once[dev], [dev]() {
    void* ptr = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int64_t hqq_tensor_stop_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

int hqq_quantize_tensor_stop_noalloc(const void* W_f16, int64_t rows, int64_t cols, int nbits,
                                     int group_size, float p, float beta, float kappa, int iters,
                                     void* packed_codes, void* scale_f16, void* zero_f16,
                                     const hqq_options_t* opt, void* totals_f64, void* t_star_i32,
                                     void* stream) {
  int64_t n = 0;
  int st = validate_single(W_f16, rows, cols, nbits, group_size, p, beta, kappa, iters,
                           packed_codes, scale_f16, zero_f16, n);
  if (st != HQQ_OK || n == 0) return st;
  hqq_options_t o;  // everything hqq_quantize_tensor_stop checks, before the scratch is touched
  st = read_options(opt, o);
  if (st != HQQ_OK) return st;
  if ((totals_f64 && !aligned(totals_f64, 8)) || (t_star_i32 && !aligned(t_star_i32, 4)))
    return HQQ_ERR_ALIGNMENT;
  if (hqq::tensor_stop_workspace_bytes(iters) > kNoallocScratchBytes) return HQQ_ERR_INVALID_ARG;
  void* ws = scratch_of_current_device();
  if (!ws) return HQQ_ERR_LAUNCH;
  return hqq_quantize_tensor_stop(W_f16, rows, cols, nbits, group_size, p, beta, kappa, iters,
                                  packed_codes, scale_f16, zero_f16, opt, totals_f64, t_star_i32,
                                  ws, stream);
}

int hqq_quantize_batch(const hqq_batch_entry_t* entries, const hqq_batch_entry_t* entries_device,
                       int count, int nbits, int group_size, float p, float beta, float kappa,
                       int iters, void* packed_codes, void* scale_f16, void* zero_f16,
                       int32_t* status_device, void* stream) {
  static_assert(sizeof(hqq_batch_entry_t) == sizeof(hqq::BatchEntry), "entry layout");
  static_assert(offsetof(hqq_batch_entry_t, first_group) == offsetof(hqq::BatchEntry, first_group),
                "entry layout");
  if (count < 0) return HQQ_ERR_INVALID_ARG;
  if (!supported_nbits(nbits) || !supported_group(group_size)) return HQQ_ERR_UNSUPPORTED;
  int st = validate_solver(p, beta, kappa, iters);
  if (st != HQQ_OK) return st;
  if (count == 0) return HQQ_OK;
  if (!entries || !entries_device) return HQQ_ERR_INVALID_ARG;
  if (!aligned(entries_device, 8)) return HQQ_ERR_ALIGNMENT;
  int64_t total = 0;  // groups of the entries so far
  for (int i = 0; i < count; ++i) {
    const hqq_batch_entry_t& e = entries[i];
    st = validate_common(e.rows, e.cols, nbits, group_size);
    if (st != HQQ_OK) return st;
    if (e.first_group != total) return HQQ_ERR_INVALID_ARG;
    const int64_t n = e.rows * e.cols;
    if (n > 0) {
      if (!e.W_f16) return HQQ_ERR_INVALID_ARG;
      if (!aligned(e.W_f16, 16)) return HQQ_ERR_ALIGNMENT;
    }
    const int64_t groups = n / group_size;
    if (groups > INT64_MAX / 8 / group_size - total) return HQQ_ERR_INVALID_ARG;  // size overflow
    total += groups;
  }
  if (total == 0) return HQQ_OK;
  if (!packed_codes || !scale_f16 || !zero_f16 || !status_device) return HQQ_ERR_INVALID_ARG;
  if (!aligned(packed_codes, 4) || !aligned(scale_f16, 2) || !aligned(zero_f16, 2) ||
      !aligned(status_device, 4))
    return HQQ_ERR_ALIGNMENT;

  uint64_t hash = 0;  // of the table just validated; the kernel checks its copy against it
  for (int i = 0; i < count; ++i)
    hash += hqq::table_entry_hash((uint64_t)(uintptr_t)entries[i].W_f16, entries[i].rows,
                                  entries[i].cols, entries[i].first_group, i);
  hqq::SolveParams prm = {};
  prm.W = nullptr;
  prm.batch = reinterpret_cast<const hqq::BatchEntry*>(entries_device);
  prm.batch_count = count;
  prm.batch_hash = hash;
  prm.batch_status = status_device;
  prm.packed = static_cast<uint8_t*>(packed_codes);
  prm.scale16 = static_cast<uint16_t*>(scale_f16);
  prm.zero16 = static_cast<uint16_t*>(zero_f16);
  prm.ngroups = total;
  set_solver_params(prm, nbits, group_size, p, beta, kappa, iters, 1, 0, hqq::kErrP);
  int cus = compute_units();
  if (cus <= 0) return HQQ_ERR_LAUNCH;
  hipError_t err = hqq::launch_solve(prm, group_size, power_mode_of(p), cus,
                                     static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

int hqq_quantize(const void* W_f16, int64_t rows, int64_t cols, int nbits, int group_size, float p,
                 float beta, float kappa, int iters, void* packed_codes, void* scale_f16,
                 void* zero_f16, void* stream) {
  return hqq_quantize_ex(W_f16, rows, cols, nbits, group_size, p, beta, kappa, iters, packed_codes,
                         scale_f16, zero_f16, nullptr, stream);
}

int hqq_dequantize(const void* packed_codes, const void* scale_f16, const void* zero_f16,
                   int64_t rows, int64_t cols, int nbits, int group_size, void* W_out_f16,
                   void* stream) {
  int st = validate_common(rows, cols, nbits, group_size);
  if (st != HQQ_OK) return st;
  const int64_t n = rows * cols;
  if (n == 0) return HQQ_OK;
  if (!packed_codes || !scale_f16 || !zero_f16 || !W_out_f16) return HQQ_ERR_INVALID_ARG;
  if (!aligned(packed_codes, 4) || !aligned(scale_f16, 2) || !aligned(zero_f16, 2) ||
      !aligned(W_out_f16, 16))
    return HQQ_ERR_ALIGNMENT;
  hqq::DequantParams prm;
  prm.packed = static_cast<const uint8_t*>(packed_codes);
  prm.scale16 = static_cast<const uint16_t*>(scale_f16);
  prm.zero16 = static_cast<const uint16_t*>(zero_f16);
  prm.out = static_cast<uint4*>(W_out_f16);
  prm.nchunks = n / hqq::kDequantElems;
  prm.chunks_per_group = group_size / hqq::kDequantElems;
  prm.nbits = nbits;
  int cus = compute_units();
  if (cus <= 0) return HQQ_ERR_LAUNCH;
  int64_t blocks = (prm.nchunks + hqq::kBlock - 1) / hqq::kBlock;
  const int64_t cap = (int64_t)cus * 16;
  if (blocks > cap) blocks = cap;
  hipError_t err = hqq::launch_dequant(prm, (int)blocks, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

int64_t hqq_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, int nbits,
                                   int group_size) {
  if (checked_elems(M, K) < 0 || checked_elems(N, K) < 0 || checked_elems(M, N) < 0) return -1;
  if (!supported_nbits(nbits) || !supported_group(group_size)) return -1;
  return hqq::matmul_workspace_bytes(M, N, K, nbits, group_size);
}

int hqq_matmul(const void* X_f16, int64_t M, int64_t K, const void* packed_codes,
               const void* scale_f16, const void* zero_f16, int64_t N, int nbits,
               int group_size, void* Y, int out_f32, void* workspace, void* stream) {
  if (checked_elems(M, K) < 0 || checked_elems(N, K) < 0 || checked_elems(M, N) < 0)
    return HQQ_ERR_INVALID_ARG;
  if (!supported_nbits(nbits) || !supported_group(group_size)) return HQQ_ERR_UNSUPPORTED;
  if (K % group_size != 0) return HQQ_ERR_INVALID_ARG;
  if (K % 32 != 0) return HQQ_ERR_UNSUPPORTED;
  if (out_f32 != 0 && out_f32 != 1) return HQQ_ERR_INVALID_ARG;
  if (M > (int64_t)65535 * 128) return HQQ_ERR_INVALID_ARG;  // grid size
  if (M == 0 || N == 0) return HQQ_OK;
  if (!Y) return HQQ_ERR_INVALID_ARG;
  if (K > 0 && (!X_f16 || !packed_codes || !scale_f16 || !zero_f16)) return HQQ_ERR_INVALID_ARG;
  if (!aligned(Y, out_f32 ? 4 : 2)) return HQQ_ERR_ALIGNMENT;
  if (K > 0 && (!aligned(X_f16, 16) || !aligned(packed_codes, 16) || !aligned(scale_f16, 2) ||
                !aligned(zero_f16, 2)))
    return HQQ_ERR_ALIGNMENT;
  if (hqq::matmul_workspace_bytes(M, N, K, nbits, group_size) > 0) {
    if (!workspace) return HQQ_ERR_INVALID_ARG;
    if (!aligned(workspace, 16)) return HQQ_ERR_ALIGNMENT;
  }
  hqq::MatmulParams prm;
  prm.part = static_cast<float*>(workspace);
  prm.X = static_cast<const uint16_t*>(X_f16);
  prm.packed = static_cast<const uint8_t*>(packed_codes);
  prm.scale16 = static_cast<const uint16_t*>(scale_f16);
  prm.zero16 = static_cast<const uint16_t*>(zero_f16);
  prm.Y = Y;
  prm.M = M;
  prm.N = N;
  prm.K = K;
  prm.nbits = nbits;
  prm.group_size = group_size;
  prm.group_shift = group_size == 16 ? 4 : group_size == 32 ? 5 : group_size == 64 ? 6 : 7;
  prm.out_f32 = out_f32;
  int cus = compute_units();
  if (cus <= 0) return HQQ_ERR_LAUNCH;
  hipError_t err = hqq::launch_matmul(prm, cus, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

// Shapes of the residual and low-rank entry points: rows and cols multiples of 64,
// cols a multiple of the group size.
int validate_lowrank_shape(int64_t rows, int64_t cols, int nbits, int group_size) {
  int st = validate_common(rows, cols, nbits, group_size);
  if (st != HQQ_OK) return st;
  if (rows % 64 != 0 || cols % 64 != 0) return HQQ_ERR_UNSUPPORTED;
  return HQQ_OK;
}

int hqq_residual(const void* W_f16, const void* packed_codes, const void* scale_f16,
                 const void* zero_f16, int64_t rows, int64_t cols, int nbits, int group_size,
                 void* dW_f16, void* dWT_f16, void* stream) {
  int st = validate_lowrank_shape(rows, cols, nbits, group_size);
  if (st != HQQ_OK) return st;
  if (rows * cols == 0) return HQQ_OK;
  if (!W_f16 || !packed_codes || !scale_f16 || !zero_f16 || !dW_f16) return HQQ_ERR_INVALID_ARG;
  if (!aligned(W_f16, 16) || !aligned(packed_codes, 16) || !aligned(scale_f16, 2) ||
      !aligned(zero_f16, 2) || !aligned(dW_f16, 16) || (dWT_f16 && !aligned(dWT_f16, 16)))
    return HQQ_ERR_ALIGNMENT;
  hipError_t err = hqq::launch_residual(
      static_cast<const uint16_t*>(W_f16), static_cast<const uint8_t*>(packed_codes),
      static_cast<const uint16_t*>(scale_f16), static_cast<const uint16_t*>(zero_f16), rows, cols,
      nbits, group_size, static_cast<uint16_t*>(dW_f16), static_cast<uint16_t*>(dWT_f16),
      static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

int64_t hqq_lowrank_workspace_bytes(int64_t rows, int64_t cols, int rank, int oversample) {
  if (rows <= 0 || cols <= 0 || rows % 64 != 0 || cols % 64 != 0) return -1;
  if (checked_elems(rows, cols) < 0) return -1;
  if (rank < 1 || oversample < 0) return -1;
  const int64_t width = (int64_t)rank + oversample;
  if (width % 32 != 0 || width > 512 || width > rows || width > cols) return -1;
  return hqq::lowrank_workspace_bytes(rows, cols, (int)width);
}

int hqq_lowrank(const void* W_f16, const void* packed_codes, const void* scale_f16,
                const void* zero_f16, int64_t rows, int64_t cols, int nbits, int group_size,
                int rank, int oversample, int power_iters, const void* omega_f16, void* B_f32,
                void* A_f32, void* sigma_f32, void* workspace, void* stream) {
  int st = validate_lowrank_shape(rows, cols, nbits, group_size);
  if (st != HQQ_OK) return st;
  if (rows == 0 || cols == 0) return HQQ_ERR_INVALID_ARG;
  if (hqq_lowrank_workspace_bytes(rows, cols, rank, oversample) < 0) return HQQ_ERR_INVALID_ARG;
  if (power_iters < 0 || power_iters > 16) return HQQ_ERR_INVALID_ARG;
  if (!W_f16 || !packed_codes || !scale_f16 || !zero_f16 || !omega_f16 || !B_f32 || !A_f32 ||
      !sigma_f32 || !workspace)
    return HQQ_ERR_INVALID_ARG;
  if (!aligned(W_f16, 16) || !aligned(packed_codes, 16) || !aligned(scale_f16, 2) ||
      !aligned(zero_f16, 2) || !aligned(omega_f16, 16) || !aligned(B_f32, 4) ||
      !aligned(A_f32, 4) || !aligned(sigma_f32, 4) || !aligned(workspace, 256))
    return HQQ_ERR_ALIGNMENT;
  hqq::LowrankParams prm;
  prm.W = static_cast<const uint16_t*>(W_f16);
  prm.packed = static_cast<const uint8_t*>(packed_codes);
  prm.scale16 = static_cast<const uint16_t*>(scale_f16);
  prm.zero16 = static_cast<const uint16_t*>(zero_f16);
  prm.m = rows;
  prm.n = cols;
  prm.nbits = nbits;
  prm.group_size = group_size;
  prm.group_shift = group_size == 16 ? 4 : group_size == 32 ? 5 : group_size == 64 ? 6 : 7;
  prm.rank = rank;
  prm.width = rank + oversample;
  prm.power_iters = power_iters;
  prm.omega = static_cast<const uint16_t*>(omega_f16);
  prm.B = static_cast<float*>(B_f32);
  prm.A = static_cast<float*>(A_f32);
  prm.sigma = static_cast<float*>(sigma_f32);
  prm.workspace = workspace;
  int cus = compute_units();
  if (cus <= 0) return HQQ_ERR_LAUNCH;
  hipError_t err = hqq::launch_lowrank(prm, cus, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

int64_t hqq_meta_groups(int64_t n, int64_t meta_group) {
  if (n < 0 || meta_group < 0 || meta_group > kMaxMetaGroup) return -1;
  if (n == 0) return 0;
  return meta_group == 0 ? 1 : (n + meta_group - 1) / meta_group;
}

int64_t hqq_meta_workspace_bytes(void) { return 2 * hqq::kMetaPartials * (int64_t)sizeof(uint32_t); }

int hqq_meta_quantize(const void* values_f16, int64_t n, int64_t meta_group, void* codes_u8,
                      void* mscale_f16, void* moffset_f16, void* workspace, void* stream) {
  const int64_t ng = hqq_meta_groups(n, meta_group);
  if (ng < 0) return HQQ_ERR_INVALID_ARG;
  if (ng > (int64_t)INT32_MAX) return HQQ_ERR_INVALID_ARG;  // grid size
  if (n == 0) return HQQ_OK;
  if (!values_f16 || !codes_u8 || !mscale_f16 || !moffset_f16) return HQQ_ERR_INVALID_ARG;
  if (meta_group == 0 && !workspace) return HQQ_ERR_INVALID_ARG;
  if (!aligned(values_f16, 2) || !aligned(mscale_f16, 2) || !aligned(moffset_f16, 2))
    return HQQ_ERR_ALIGNMENT;
  if (meta_group == 0 && !aligned(workspace, 4)) return HQQ_ERR_ALIGNMENT;
  int cus = compute_units();
  if (cus <= 0) return HQQ_ERR_LAUNCH;
  hipError_t err = hqq::launch_meta_quantize(
      static_cast<const uint16_t*>(values_f16), n, meta_group, static_cast<uint8_t*>(codes_u8),
      static_cast<uint16_t*>(mscale_f16), static_cast<uint16_t*>(moffset_f16),
      static_cast<uint32_t*>(workspace), cus, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

int hqq_meta_quantize_batch(const hqq_batch_entry_t* entries,
                            const hqq_batch_entry_t* entries_device, int count, int group_size,
                            const void* values_f16, int64_t meta_group, void* codes_u8,
                            void* mscale_f16, void* moffset_f16, void* workspace, void* stream) {
  if (count < 0 || meta_group < 0 || meta_group > kMaxMetaGroup) return HQQ_ERR_INVALID_ARG;
  if (!supported_group(group_size)) return HQQ_ERR_UNSUPPORTED;
  if (count == 0) return HQQ_OK;
  if (!entries) return HQQ_ERR_INVALID_ARG;
  int64_t total = 0;
  bool starts_mod8 = true;  // every entry starts at a multiple of 8 values
  for (int i = 0; i < count; ++i) {
    const hqq_batch_entry_t& e = entries[i];
    if (checked_elems(e.rows, e.cols) < 0 || e.cols % group_size != 0) return HQQ_ERR_INVALID_ARG;
    if (e.first_group != total) return HQQ_ERR_INVALID_ARG;
    const int64_t groups = e.rows * e.cols / group_size;
    if (meta_group > 0 && groups % meta_group != 0) return HQQ_ERR_INVALID_ARG;
    if (groups % 8 != 0) starts_mod8 = false;
    total += groups;
  }
  if (total == 0) return HQQ_OK;
  if (meta_group > 0)  // entry-local groups coincide with groups of the whole arena
    return hqq_meta_quantize(values_f16, total, meta_group, codes_u8, mscale_f16, moffset_f16,
                             nullptr, stream);
  if (!entries_device || !values_f16 || !codes_u8 || !mscale_f16 || !moffset_f16 || !workspace)
    return HQQ_ERR_INVALID_ARG;
  if (!aligned(entries_device, 8) || !aligned(values_f16, 2) || !aligned(mscale_f16, 2) ||
      !aligned(moffset_f16, 2) || !aligned(workspace, 4))
    return HQQ_ERR_ALIGNMENT;
  if ((total + (1 << 16) - 1) >> 16 > (int64_t)INT32_MAX) return HQQ_ERR_INVALID_ARG;
  hipError_t err = hqq::launch_meta_quantize_segments(
      static_cast<const uint16_t*>(values_f16), total,
      reinterpret_cast<const hqq::BatchEntry*>(entries_device), count, starts_mod8,
      static_cast<uint8_t*>(codes_u8), static_cast<uint16_t*>(mscale_f16),
      static_cast<uint16_t*>(moffset_f16), static_cast<uint32_t*>(workspace),
      static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

int hqq_meta_dequantize(const void* codes_u8, const void* mscale_f16, const void* moffset_f16,
                        int64_t n, int64_t meta_group, void* values_f16, void* stream) {
  const int64_t ng = hqq_meta_groups(n, meta_group);
  if (ng < 0) return HQQ_ERR_INVALID_ARG;
  if (n == 0) return HQQ_OK;
  if (!codes_u8 || !mscale_f16 || !moffset_f16 || !values_f16) return HQQ_ERR_INVALID_ARG;
  if (!aligned(values_f16, 2) || !aligned(mscale_f16, 2) || !aligned(moffset_f16, 2))
    return HQQ_ERR_ALIGNMENT;
  int cus = compute_units();
  if (cus <= 0) return HQQ_ERR_LAUNCH;
  hipError_t err = hqq::launch_meta_dequantize(
      static_cast<const uint8_t*>(codes_u8), static_cast<const uint16_t*>(mscale_f16),
      static_cast<const uint16_t*>(moffset_f16), n, meta_group, static_cast<uint16_t*>(values_f16),
      cus, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? HQQ_OK : HQQ_ERR_LAUNCH;
}

}  // extern "C"
