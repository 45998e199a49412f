/*
 * hqq.h -- C ABI of the MI355X (gfx950) group-wise HQQ weight quantizer.
 *
 * The method is the one on the page "Half-Quadratic Quantization of Large
 * Machine Learning Models" (Dropbox tech blog):
 *   section 2    affine quantizer Q(W) = round(W/s + z) = W_q and its inverse
 *                Q^-1(W_q) = s (W_q - z); the error phi(W - Q^-1(Q(W))) with a
 *                sparsity-promoting lp norm; a half-quadratic split with the
 *                scale s fixed so that only z is optimized; alternating updates
 *                sp1 (W_e), sp2 (z) and beta <- kappa * beta;
 *   section 2.1  sp1 is the generalized soft-threshold
 *                shrink(x, beta) = sign(x) relu(|x| - |x|^(p-1) / beta);
 *   section 2.2  sp2 is the mean over the group of W_q - (W - W_e)/s, computed
 *                with the inverse scale 1/s;
 *   section 4.1  p = 0.7, beta = 1, kappa = 1.01, 20 iterations, early exit once
 *                the error stops improving, group-wise quantized buffers.
 * Readings of points the page leaves open (min-max initialisation, rounding
 * half to even, clamping to [0, 2^nbits - 1], the per-group lp error
 * sum |W - Q^-1(Q(W))|^p as the early-stop criterion with strict improvement,
 * LSB-first bit packing) are stated with each entry point below.
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers (HBM of the current HIP device),
 *     allocated and owned by the caller.  The library never allocates, frees
 *     or synchronizes.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL means the default stream).  The status is returned
 *     synchronously; faults inside a kernel surface at the caller's next
 *     synchronization, as usual in HIP.
 *   - All arguments are validated before anything is enqueued: on any error
 *     nothing is launched and no output byte is written.
 *   - Inputs are read-only; outputs are fully overwritten.  Inputs and outputs
 *     must not overlap.  Calls are reentrant: the library holds no mutable
 *     global state.
 *   - Matrices are row-major rows x cols.  Groups are group_size consecutive
 *     elements of a row (the input dimension); cols must be a multiple of
 *     group_size, so group j of row i has flat index i*(cols/group_size) + j and
 *     covers elements [j*group_size, (j+1)*group_size) of that row.
 */
#ifndef HQQ_MI355X_H
#define HQQ_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  HQQ_OK = 0,
  HQQ_ERR_INVALID_ARG = 1, /* null pointer, negative size, parameter out of range,
                              cols not a multiple of group_size, size overflow */
  HQQ_ERR_UNSUPPORTED = 2, /* nbits or group_size outside the supported sets */
  HQQ_ERR_ALIGNMENT = 3,   /* a pointer misses its documented alignment */
  HQQ_ERR_LAUNCH = 4,      /* the HIP runtime refused the launch (e.g. no device) */
  HQQ_ERR_TABLE_MISMATCH = 5 /* written by hqq_quantize_batch's kernel to its status word:
                                the device entry table differs from the validated host one */
};

/* Optional outputs and switches of hqq_quantize_ex.  Every pointer may be NULL.
 * Per-group arrays have hqq_num_groups(rows, cols, group_size) elements in the
 * row-major group order described above. */
typedef struct {
  int early_stop;      /* 1: per-group early exit (section 4.1, the default of
                          hqq_quantize).  0: every iteration is accepted and the
                          z after `iters` updates is returned. */
  float* scale_f32;    /* s as computed in fp32, before the binary16 cast */
  float* zero_f32;     /* returned z in fp32, before the binary16 cast */
  uint8_t* stop_step;  /* t*: index of the accepted evaluation whose z is
                          returned (0 = the min-max initialisation) */
  float* err_init;     /* e_0 = sum |W - Q^-1(Q(W))|^p at the initial z */
  float* err_best;     /* e_{t*}, the error at the returned z */
  int refill_threshold; /* performance knob, no effect on any output: a wavefront
                           iterates 64*16/group_size groups at a time and hands stopped
                           groups over (replacing them from its standby pool) once this
                           many have stopped.  0 = default (1); values above the slot
                           count are clamped; < 0 invalid. */
  int err_metric;      /* the error of the early-stop test (and of err_init/err_best):
                          0 = sum |r|^p with the solver's p (the default reading of
                          section 4.1's "error"); 1 = sum |r| (l1); 2 = sum r^2 (l2).
                          The shrink and z update are unchanged.  Other values invalid. */
} hqq_options_t;

/*
 * hqq_quantize -- group-wise asymmetric quantization with the HQQ zero-point
 * solver (sections 2, 2.1, 2.2 and 4.1 of the page above).
 *
 * For every group of group_size weights w_k:
 *   init  s = (max - min) / qmax, 1/s = qmax / (max - min), z = -min / s
 *         (qmax = 2^nbits - 1; a constant group takes s = 1);
 *   for t = 0 .. iters:
 *         W_q = clamp(round_half_even(w / s + z), 0, qmax)
 *         r   = w - s (W_q - z)                       residual
 *         e_t = sum_k |r_k|^p   (|0|^p := 0)          lp error of section 2
 *         stop unless e_t < best error so far; otherwise accept z;
 *         if t == iters stop;
 *         W_e = sign(r) relu(|r| - |r|^(p-1) / beta_t) (0 where r = 0)   sp1
 *         z   = mean_k (W_q - (w - W_e) / s)                             sp2
 *         beta_{t+1} = kappa * beta_t
 *   outputs: the codes W_q at the accepted z, s and z (binary16, RNE).
 * Arithmetic is fp32 on the device (the page's half-precision pipeline is not
 * reproduced); the codes are those of the fp32 solver.
 *
 * W_f16        rows x cols binary16 weights; 16-byte aligned.
 * rows, cols   >= 0; rows*cols == 0 is a valid no-op.  cols % group_size == 0.
 * nbits        2, 3, 4 or 8.
 * group_size   16, 32, 64 or 128.
 * p            lp exponent, 0 <= p <= 1 (section 2.1 allows this range).
 * beta         initial beta > 0, finite.      kappa  > 0, finite.
 * iters        0 .. 255 (0 gives plain min-max round-to-nearest).
 * packed_codes hqq_packed_bytes(rows, cols, nbits) bytes: an LSB-first
 *              little-endian bitstream over the row-major elements (element n
 *              occupies bits [n*nbits, (n+1)*nbits); bit i of a byte is 2^i).
 *              nbits = 4: byte k = code[2k] | code[2k+1] << 4.  4-byte aligned.
 * scale_f16    hqq_num_groups(...) binary16 values of s.  2-byte aligned.
 * zero_f16     hqq_num_groups(...) binary16 values of z, in code units
 *              (real-valued, not rounded to an integer).  2-byte aligned.
 * stream       hipStream_t or NULL.
 * Returns HQQ_OK or an error code; see the conventions above.
 */
int hqq_quantize(const void* W_f16, int64_t rows, int64_t cols, int nbits, int group_size,
                 float p, float beta, float kappa, int iters, void* packed_codes,
                 void* scale_f16, void* zero_f16, void* stream);

/* hqq_quantize with the optional outputs and switches of hqq_options_t
 * (opt == NULL behaves exactly like hqq_quantize).  Optional float outputs
 * must be 4-byte aligned. */
int hqq_quantize_ex(const void* W_f16, int64_t rows, int64_t cols, int nbits, int group_size,
                    float p, float beta, float kappa, int iters, void* packed_codes,
                    void* scale_f16, void* zero_f16, const hqq_options_t* opt, void* stream);

/*
 * hqq_quantize_tensor_stop -- hqq_quantize_ex with the early exit of section 4.1
 * taken at the scope of the whole matrix instead of each group (the page does not
 * say over what the error is measured; this is the reading where it is the error of
 * the whole tensor):
 *   E_t  = sum over all groups of e_t, the group error of hqq_quantize in weight
 *          units (with opt->err_metric), for t = 0 .. iters, every group iterating
 *          without a stop;
 *   t*   = the end of the strictly decreasing run E_0 > E_1 > ... > E_t*;
 *   outputs: exactly those of hqq_quantize_ex with early_stop = 0 and iters = t*
 *          (every group returns the z after t* updates; stop_step = t* everywhere).
 * E_t is accumulated in fp64 from the fp32 group errors in an order fixed for a
 * given device, so repeated calls give the same E_t and t*.
 *
 * opt          NULL or the optional outputs and err_metric of hqq_quantize_ex;
 *              early_stop and refill_threshold are not used.
 * totals_f64   NULL or iters + 1 doubles (device, 8-byte aligned): E_0 .. E_iters.
 * t_star_i32   NULL or one int32 (device, 4-byte aligned): t*.
 * workspace    hqq_tensor_stop_workspace_bytes(iters) bytes of device memory,
 *              8-byte aligned, owned by the caller: per-block partial totals and the
 *              totals, written and read on `stream` (no allocation, no memset); it
 *              must not be shared by calls that may run at the same time.
 * Three kernels run in stream order: every group through steps 0 .. iters
 * (accumulating the totals), one block per step adding them up, and every group
 * through t* updates writing the outputs (t* found on the device: no host
 * synchronization).  rows*cols == 0 is a no-op (nothing is written).
 * Other arguments, conventions and errors as for hqq_quantize_ex.
 */
int hqq_quantize_tensor_stop(const void* W_f16, int64_t rows, int64_t cols, int nbits,
                             int group_size, float p, float beta, float kappa, int iters,
                             void* packed_codes, void* scale_f16, void* zero_f16,
                             const hqq_options_t* opt, void* totals_f64, void* t_star_i32,
                             void* workspace, void* stream);

/* Bytes of the workspace of hqq_quantize_tensor_stop for `iters` (2048 + 16384 *
 * (iters + 1)); -1 for iters outside 0 .. 255. */
int64_t hqq_tensor_stop_workspace_bytes(int iters);

/*
 * hqq_quantize_tensor_stop_noalloc -- hqq_quantize_tensor_stop without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The scratch the
 * whole-tensor stop needs between its kernels lives in a device array inside the library
 * (hqq_tensor_stop_noalloc_max_bytes() bytes, enough for every iters up to 255; one copy
 * per GPU, held until the process ends); the first call on a device looks up that
 * device's copy.  The call allocates, frees and synchronizes nothing.  Calls on one GPU
 * share the array, so calls that may run at the same time on one GPU (other streams,
 * other threads) race and must be serialized by the caller; each call writes every
 * scratch byte it reads, so no clearing is needed between calls.  Arguments, results and
 * errors as for hqq_quantize_tensor_stop (bit-identical outputs); HQQ_ERR_INVALID_ARG if
 * the scratch would exceed the array, HQQ_ERR_LAUNCH if the array's address cannot be
 * obtained.
 */
int hqq_quantize_tensor_stop_noalloc(const void* W_f16, int64_t rows, int64_t cols, int nbits,
                                     int group_size, float p, float beta, float kappa, int iters,
                                     void* packed_codes, void* scale_f16, void* zero_f16,
                                     const hqq_options_t* opt, void* totals_f64, void* t_star_i32,
                                     void* stream);

/* Size of the device array behind hqq_quantize_tensor_stop_noalloc, in bytes. */
int64_t hqq_tensor_stop_noalloc_max_bytes(void);

/* One input matrix of hqq_quantize_batch (32 bytes; the same layout is read on
 * the host and on the device). */
typedef struct {
  const void* W_f16;   /* rows x cols binary16 weights, row-major; 16-byte aligned */
  int64_t rows;        /* >= 0 */
  int64_t cols;        /* >= 0, a multiple of group_size */
  int64_t first_group; /* index of the matrix's first group in the output arrays:
                          the sum of hqq_num_groups(...) over the entries before it */
} hqq_batch_entry_t;

/*
 * hqq_quantize_batch -- hqq_quantize (sections 2, 2.1, 2.2 and 4.1 of the page
 * above, same readings) applied to `count` matrices that share nbits, group_size
 * and the solver parameters, in one kernel launch.  The inputs are separate
 * allocations; the outputs of all matrices go to one set of arrays (an arena) in
 * entry order: the groups of entry i occupy group indices
 * [first_group_i, first_group_i + hqq_num_groups(rows_i, cols_i, group_size)).
 * Every output element equals, bit for bit, what hqq_quantize writes for that
 * matrix alone into arrays that start at its first group.
 *
 * entries         host array of `count` entries; read during the call only, for
 *                 validation.  first_group must be the running sum described above.
 * entries_device  device copy of the same `count` entries (8-byte aligned), made by
 *                 the caller; the kernel reads W_f16 and first_group from it, so it
 *                 must hold exactly what `entries` holds and stay unchanged until the
 *                 launch has completed.  The library hashes the validated host table
 *                 and passes the hash to the kernel by value; every wavefront hashes
 *                 the device copy before it reads any weight and, if the two differ,
 *                 writes nothing at all (see status_device).
 * count           >= 0; 0 (or no group at all) is a valid no-op.
 * packed_codes    total_groups * group_size * nbits / 8 bytes, 4-byte aligned; the
 *                 codes of group k start at byte k * group_size * nbits / 8 (the
 *                 LSB-first bitstream of hqq_quantize, matrix after matrix).
 * scale_f16, zero_f16  total_groups binary16 values each, 2-byte aligned.
 * status_device   one int32 of device memory (4-byte aligned, required when there is
 *                 a group to quantize).  The launch writes HQQ_OK there when the
 *                 device table matched, HQQ_ERR_TABLE_MISMATCH when it did not (then
 *                 no output byte is written).  A call with no group launches nothing
 *                 and leaves it untouched.  Read it after the stream has completed.
 * Other arguments, conventions and errors as for hqq_quantize; every entry is
 * validated before anything is enqueued.
 */
int hqq_quantize_batch(const hqq_batch_entry_t* entries, const hqq_batch_entry_t* entries_device,
                       int count, int nbits, int group_size, float p, float beta, float kappa,
                       int iters, void* packed_codes, void* scale_f16, void* zero_f16,
                       int32_t* status_device, void* stream);

/*
 * hqq_dequantize -- the inverse quantizer Q^-1(W_q) = s (W_q - z) of section 2,
 * evaluated from the stored binary16 s and z and rounded once (RNE) to binary16.
 * The result equals the exact value s*(W_q - z) rounded to binary16.
 * Layouts and alignment as for hqq_quantize; W_out_f16 (rows x cols) must be
 * 16-byte aligned.
 */
int hqq_dequantize(const void* packed_codes, const void* scale_f16, const void* zero_f16,
                   int64_t rows, int64_t cols, int nbits, int group_size, void* W_out_f16,
                   void* stream);

/*
 * hqq_meta_quantize -- 8-bit quantization of a per-group meta array: section 4.1
 * of the page stores the zero-points in 8 bits without grouping or optimization,
 * and the note under its Llama-2 table quantizes the scales to 8 bits in groups of
 * 128.  Reading: affine min-max round-to-nearest (no solver) over the binary16
 * values, in groups of meta_group consecutive values; per group, with mn and mx its
 * minimum and maximum and d = mx - mn:
 *   code  = the integer nearest the exact ratio (v - mn) * 255 / d, half to even
 *           (decided exactly, without rounding the ratio first),
 *   scale = binary16(d / 255) (nearest even), offset = mn (+0 for a zero minimum);
 * a constant group has codes 0 and scale 1.  The value is recovered as
 * offset + scale * code (hqq_meta_dequantize).
 *
 * values_f16   n binary16 values, e.g. the zero_f16 (meta_group 0) or scale_f16
 *              (meta_group 128) output of hqq_quantize; 2-byte aligned.
 * n            >= 0; 0 is a valid no-op.
 * meta_group   0: one group of all n values; otherwise 1 .. 2^20 consecutive values
 *              per group (the last group may be shorter).
 * codes_u8     n bytes.
 * mscale_f16, moffset_f16  hqq_meta_groups(n, meta_group) binary16 values each,
 *              2-byte aligned.
 * workspace    meta_group 0 only (ignored otherwise, may be NULL):
 *              hqq_meta_workspace_bytes() bytes of device memory, 4-byte aligned,
 *              owned by the caller; the call writes partial minima and maxima there
 *              and reads them back on `stream` (no allocation, no memset); it must
 *              not be shared by calls that may run at the same time.
 * Conventions and errors as for hqq_quantize.
 */
int hqq_meta_quantize(const void* values_f16, int64_t n, int64_t meta_group, void* codes_u8,
                      void* mscale_f16, void* moffset_f16, void* workspace, void* stream);

/* hqq_meta_dequantize -- offset + scale * code of hqq_meta_quantize's output,
 * rounded once to binary16 (the exact value is representable in fp64 and the
 * result equals its nearest-even binary16).  values_f16: n binary16 outputs,
 * 2-byte aligned; other arguments as above. */
int hqq_meta_dequantize(const void* codes_u8, const void* mscale_f16, const void* moffset_f16,
                        int64_t n, int64_t meta_group, void* values_f16, void* stream);

/* Number of meta groups: 0 for n == 0, 1 for meta_group == 0, else
 * ceil(n / meta_group).  -1 for invalid arguments. */
int64_t hqq_meta_groups(int64_t n, int64_t meta_group);

/* Bytes of the workspace hqq_meta_quantize needs with meta_group 0 (8192). */
int64_t hqq_meta_workspace_bytes(void);

/*
 * hqq_meta_quantize_batch -- hqq_meta_quantize applied to every entry of a
 * hqq_quantize_batch output arena in one launch sequence: `values_f16` is the
 * arena's zero_f16 or scale_f16 array (total groups of the entries, in entry
 * order); groups never span two entries.
 *   meta_group 0: one group per entry (the zero-points); mscale_f16 and moffset_f16
 *     hold `count` values (entry order; empty entries get none written and keep
 *     their slot); workspace: 8 * count bytes of device memory, 4-byte aligned,
 *     used for per-entry minima and maxima (initialized on `stream`).
 *   meta_group M > 0: groups of M inside each entry; every entry's group count must
 *     be a multiple of M, so this equals hqq_meta_quantize over the whole arena
 *     (total / M meta groups); entries_device and workspace are not used.
 * entries / entries_device: as for hqq_quantize_batch (W_f16 is not read).
 * codes_u8: total bytes.  Results equal hqq_meta_quantize on each entry's slice.
 */
int hqq_meta_quantize_batch(const hqq_batch_entry_t* entries,
                            const hqq_batch_entry_t* entries_device, int count, int group_size,
                            const void* values_f16, int64_t meta_group, void* codes_u8,
                            void* mscale_f16, void* moffset_f16, void* workspace, void* stream);

/*
 * hqq_matmul -- Y = X Q^-1(W_q)^T: the product of activations X with a weight stored
 * by hqq_quantize, through the inverse quantizer Q^-1(W_q) = s (W_q - z) of section 2
 * of the page above (the consumer of the stored format; the page reports the runtime
 * memory of models stored this way, section 4.1).  The weight is N x K: row n holds
 * the K inputs of output n, grouped along K, exactly as hqq_quantize(rows = N,
 * cols = K) writes packed_codes, scale_f16 and zero_f16.
 *   Y[m][n] = sum over k of X[m][k] * s[n][k/g] * (q[n][k] - z[n][k/g])
 * with the stored binary16 s and z.  Arithmetic: fp32 accumulation in an order that
 * depends on the path (not bit-reproducible against another order).  M <= 2 (M <= 8
 * for 3-bit codes, groups of 16, K not a multiple of 256 or s, z not 16-byte aligned):
 * per 16 codes, s * (sum x q - z sum x) in fp32 (the codes enter exactly).  More rows:
 * the weight is dequantized to binary16 (s*q - s*z in fp32, one rounding, then to
 * binary16) and multiplied on the matrix cores with fp32 accumulation.
 *
 * X_f16        M x K binary16, row-major, 16-byte aligned.
 * M, N, K      >= 0; K a multiple of group_size and of 32 (else HQQ_ERR_UNSUPPORTED);
 *              M <= 8388480.  M == 0 or N == 0 is a no-op; K == 0 writes zeros.
 * packed_codes, scale_f16, zero_f16  the N x K weight as hqq_quantize stores it;
 *              packed_codes 16-byte aligned.
 * nbits, group_size  as quantized (2, 3, 4, 8 and 16, 32, 64, 128).
 * Y            M x N row-major: binary16 (out_f32 = 0, RNE of the fp32 sum; 2-byte
 *              aligned) or fp32 (out_f32 = 1; 4-byte aligned).
 * workspace    hqq_matmul_workspace_bytes(M, N, K, nbits, group_size) bytes of device
 *              memory, 16-byte aligned, or NULL where that is 0.  For 17 to 64 rows of X
 *              with 2-, 4- or 8-bit codes, groups of 32-128 and K a multiple of 256, K is
 *              split over several blocks whose fp32 partial products go to the workspace
 *              and are added in a fixed order (results do not depend on the device or the
 *              run); the split depends on the shapes and nbits only.  Written and read on
 *              `stream`, no state between calls: calls that share a workspace must be
 *              ordered.
 *              NULL where it is needed: HQQ_ERR_INVALID_ARG.
 * Conventions and errors as for hqq_quantize.
 */
int hqq_matmul(const void* X_f16, int64_t M, int64_t K, const void* packed_codes,
               const void* scale_f16, const void* zero_f16, int64_t N, int nbits,
               int group_size, void* Y, int out_f32, void* workspace, void* stream);

/* Bytes of the workspace of hqq_matmul for these shapes (0: none needed); -1 for invalid
 * shapes, widths or group sizes. */
int64_t hqq_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, int nbits, int group_size);

/*
 * hqq_residual -- the quantization error Delta W = W - Q^-1(W_q) of a weight quantized
 * by hqq_quantize (Q^-1(W_q) = s (W_q - z), section 2 of the page above), as binary16:
 * w - (s q - s z) in fp32 (s z exact) rounded to binary16.
 * W_f16, packed_codes, scale_f16, zero_f16  the rows x cols weight and its stored
 *              quantization (W 16-byte, packed_codes 16-byte, s and z 2-byte aligned).
 * rows, cols   multiples of 64 (else HQQ_ERR_UNSUPPORTED); cols % group_size == 0.
 * dW_f16       rows x cols binary16, row-major, 16-byte aligned.
 * dWT_f16      NULL, or its transpose (cols x rows, row-major), 16-byte aligned.
 * Conventions and errors as for hqq_quantize.
 */
int hqq_residual(const void* W_f16, const void* packed_codes, const void* scale_f16,
                 const void* zero_f16, int64_t rows, int64_t cols, int nbits, int group_size,
                 void* dW_f16, void* dWT_f16, void* stream);

/*
 * hqq_lowrank -- data-free low-rank compensation of the quantization error: the plain
 * SVD compensation described on the page "Boost 2-bit LLM accuracy with EoRA" (section
 * on finding adapters in the eigenspace): with Delta W = W - Q^-1(W_q) = U Sigma V^T, the
 * LoRA factors B = U_r Sigma_r and A = V_r^T, so W_hat + B A corrects the quantized
 * weight.  Reading: the truncated SVD is computed by randomized subspace iteration with
 * a caller-supplied Gaussian test matrix Omega (width l = rank + oversample columns):
 * Y = Delta W Omega; power_iters times Y <- Delta W basis(Delta W^T basis(Y)), where
 * basis() is the Gram-Schmidt basis of the column space (Cholesky QR of the Gram matrix,
 * nearly dependent columns dropped); then
 * Q = orth(Y) with orthonormal columns, and the SVD of Q^T Delta W gives U = Q U~, Sigma,
 * V.  The accuracy against the exact SVD is set by oversample and power_iters (the
 * quantization error has a flat spectrum, so the exact rank-r subspace is itself nearly
 * degenerate).  Delta W is used in binary16 (as hqq_residual computes it), products
 * accumulate in fp32 on the matrix cores, the small l x l eigenproblems and Cholesky
 * factorizations are solved in fp64.
 *
 * W_f16, packed_codes, scale_f16, zero_f16, rows, cols, nbits, group_size  as for
 *              hqq_residual; rows, cols > 0.
 * rank         r >= 1; rank + oversample (>= 0) a multiple of 32, at most 512 and at most
 *              min(rows, cols).
 * power_iters  0 .. 16.
 * omega_f16    (rank + oversample) x cols binary16 test matrix (row-major, 16-byte aligned),
 *              e.g. standard normal samples; the caller's random numbers.
 * B_f32        rows x rank fp32 (row-major): U_r Sigma_r.
 * A_f32        rank x cols fp32 (row-major): V_r^T (orthonormal rows).
 * sigma_f32    rank fp32: the singular values, in decreasing order.  Each singular pair is
 *              determined up to a common sign of its column of B and row of A.
 * workspace    hqq_lowrank_workspace_bytes(rows, cols, rank, oversample) bytes of device
 *              memory, 256-byte aligned, owned by the caller, not shared by calls that may
 *              run at the same time (it holds Delta W in both layouts and the iterates).
 * All outputs are alignment 4.  Work is enqueued on `stream` (no allocation, no
 * synchronization); conventions and errors as for hqq_quantize.  The library keeps no
 * state between calls, so calls on different streams with workspaces of their own may
 * run at the same time (one matrix's one-block factorizations then overlap another's
 * products), with results bit-identical to the same calls made one after another.
 */
int hqq_lowrank(const void* W_f16, const void* packed_codes, const void* scale_f16,
                const void* zero_f16, int64_t rows, int64_t cols, int nbits, int group_size,
                int rank, int oversample, int power_iters, const void* omega_f16, void* B_f32,
                void* A_f32, void* sigma_f32, void* workspace, void* stream);

/* Bytes of the workspace of hqq_lowrank; -1 for invalid shapes or widths. */
int64_t hqq_lowrank_workspace_bytes(int64_t rows, int64_t cols, int rank, int oversample);

/* Bytes of the packed code stream: rows*cols*nbits/8 (exact for supported
 * shapes).  Returns -1 for invalid arguments or overflow. */
int64_t hqq_packed_bytes(int64_t rows, int64_t cols, int nbits);

/* Number of groups: rows*cols/group_size.  -1 for invalid arguments. */
int64_t hqq_num_groups(int64_t rows, int64_t cols, int group_size);

/* Static, never-NULL description of a status code. */
const char* hqq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* HQQ_MI355X_H */
