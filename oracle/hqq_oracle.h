/*
 * hqq_oracle.h -- declarations of the fp64 CPU oracle (test infrastructure only).
 * See hqq_oracle.c for the passages of "Half-Quadratic Quantization of Large
 * Machine Learning Models" that each function follows.
 */
#ifndef HQQ_ORACLE_H
#define HQQ_ORACLE_H
#include <stdint.h>

#define ORACLE_MAX_GROUP 1024

typedef struct {
  double scale;     /* s */
  double inv_scale; /* 1/s as used by the solver */
  double zero;      /* best (last accepted) z */
  int stop_step;    /* t*: iteration index of the accepted evaluation */
  double err_init;  /* e_0 */
  double err_best;  /* e_{t*} */
  int n_eval;       /* evaluations performed */
} oracle_group_result_t;

double oracle_f16_to_f64(uint16_t h);
uint16_t oracle_f64_to_f16(double v);
void oracle_f16_to_f64_array(const uint16_t* h, int64_t n, double* out);
void oracle_f64_to_f16_array(const double* v, int64_t n, uint16_t* out);

double oracle_shrink_lp(double x, double beta, double p);
double oracle_quantize_value(double w, double inv_s, double z, int qmax);
double oracle_round_ratio(double num, double den);
double oracle_quantize_init_value(double w, double mn, double mx, int qmax);
void oracle_minmax_init(const double* w, int g, int qmax, double* s, double* inv_s, double* z);
double oracle_group_error(const double* r, int g, double err_pow);
double oracle_z_update(const double* q, const double* w, const double* we, double inv_s, int g);

int oracle_hqq_group(const double* w, int g, int nbits, double p, double beta0, double kappa,
                     int iters, int early_stop, double err_pow, uint8_t* codes_out,
                     oracle_group_result_t* res, double* trace, int* n_trace);

int oracle_hqq_group_replay(const double* w, int g, int nbits, double p, double beta0,
                            double kappa, int iters, int early_stop, double err_pow,
                            uint8_t* codes_out, oracle_group_result_t* res, double* trace,
                            double* z_trace, int* n_trace, int n_flip, const int* flip_eval,
                            const int* flip_elem, int n_invert, const int* invert_eval);

int64_t oracle_packed_bytes(int64_t n, int nbits);
void oracle_pack_codes(const uint8_t* codes, int64_t n, int nbits, uint8_t* out);
void oracle_unpack_codes(const uint8_t* packed, int64_t n, int nbits, uint8_t* codes);

int oracle_hqq_quantize(const uint16_t* W_f16, int64_t rows, int64_t cols, int nbits,
                        int group_size, double p, double beta, double kappa, int iters,
                        int early_stop, double err_pow, uint8_t* packed, uint16_t* scale_f16,
                        uint16_t* zero_f16, double* scale_f64, double* zero_f64,
                        uint8_t* stop_step, double* err_init, double* err_best,
                        uint8_t* codes_out);

int oracle_hqq_dequantize(const uint8_t* packed, const uint16_t* scale_f16,
                          const uint16_t* zero_f16, int64_t rows, int64_t cols, int nbits,
                          int group_size, uint16_t* W_out_f16);

int oracle_hqq_quantize_tensor_stop(const uint16_t* W_f16, int64_t rows, int64_t cols, int nbits,
                                    int group_size, double p, double beta, double kappa,
                                    int iters, double err_pow, double* E, uint8_t* packed,
                                    uint16_t* scale_f16, uint16_t* zero_f16, double* scale_f64,
                                    double* zero_f64, uint8_t* stop_step, double* err_init,
                                    double* err_best, uint8_t* codes_out);

int64_t oracle_meta_quantize(const uint16_t* values, int64_t n, int64_t group, uint8_t* codes,
                             uint16_t* scale16, uint16_t* offset16);
int oracle_meta_dequantize(const uint8_t* codes, const uint16_t* scale16,
                           const uint16_t* offset16, int64_t n, int64_t group, uint16_t* out16);
int oracle_hqq_matmul(const uint16_t* X_f16, int64_t M, int64_t K, const uint8_t* packed,
                      const uint16_t* scale_f16, const uint16_t* zero_f16, int64_t N, int nbits,
                      int group_size, double* Y);
int oracle_hqq_residual(const uint16_t* W_f16, const uint8_t* packed, const uint16_t* scale_f16,
                        const uint16_t* zero_f16, int64_t rows, int64_t cols, int nbits,
                        int group_size, double* dW);
#endif
