/*
 * HQQ oracle: plain, single-threaded fp64 reference of the quantizer, the
 * bit-packing, the dequantisation and the dequantised GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  The product path (the HIP
 * library) shares no code with it.
 *
 * Source: the page "HQQ 算法解读：不用校准数据，怎样把大模型权重压到 4 bit"
 * (ludovicoyin.github.io), sections "量化公式" (the affine map and its inverse),
 * "为什么一定要分组" (groups, bit-packing, 4.5 bpw), "第一拍" (min-max start),
 * "第二拍" (the proximal loop), "为什么 zero 是这个均值" (the zero update),
 * "shrink 不是删除极值" (the shrink), "axis 不是一个无关紧要的开关" (grouping by
 * axis) and "从压缩文件到一次前向" (dequantise then x @ W_hat^T).
 *
 * Conventions: W is row-major [rows, cols], N = rows*cols, g = group size,
 * G = N/g groups.  axis=1: group j holds flat elements j*g + i.  axis=0: group
 * j holds flat elements i*(N/g) + j.  i = 0..g-1 is the in-group order of
 * every sum.  s is "codes per unit" (q = W*s + z), delta = 1/s is the stored
 * step, z is the zero point in code units.  Codes are one byte per weight in
 * flat row-major order.  Every sum (group sums, the whole-tensor MAE) is the balanced
 * pairwise sum in index order, zero-padded to a power of two (hqq_oracle_sum).
 *
 * Pins (tests/oracle_pins.py, each a fact fixed by the page or by the mathematics):
 * the worked example [-0.8, 0.7] (s0 = 10, z0 = 8, codes 0/8/15) through init, the
 * rounds and the solver; min-max RTN at iters = 0 with the Delta/2 error bound; ties to
 * even; degenerate groups; the zero update as the least-squares minimiser (brute force);
 * L2 monotonicity without the shrink; pack/unpack exhaustively and the 4.5 bpw size;
 * dequantisation and the GEMV through one-hot and linearity checks; the input
 * gradient through the adjoint identity with the forward product and one-hot rows; the stop
 * rule's alternative readings on hand-built MAE sequences and against the per-group steps run
 * for the kept number of rounds; binary16 conversions exhaustively against numpy.  Parity unpinned (readings, no value on the
 * page to check against): the shrink formula itself, the stop rule's rollback target
 * and tie handling, the summation order, and the solver's values on the full-size
 * synthetic tensors.
 */
#ifndef HQQ_ORACLE_H
#define HQQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double hqq_oracle_half_to_double(uint16_t h);
uint16_t hqq_oracle_double_to_half(double x);
void hqq_oracle_doubles_to_halves(const double* x, int64_t n, uint16_t* out);

double hqq_oracle_sum(const double* v, int64_t n);

int64_t hqq_oracle_group_elem(int64_t rows, int64_t cols, int g, int axis, int64_t j, int i);

void hqq_oracle_init_group(const double* w, int g, int nbits, double tiny, double* s, double* delta,
                           double* z0);
double hqq_oracle_shrink(double r, double beta, double p);
void hqq_oracle_round_group(const double* w, int g, int nbits, double s, double delta, double z, double beta,
                            double p, double* err_sum, double* z_next, double* q_out, double* e_out);
int hqq_oracle_stop_check(int k, double mae_k, double best);
int hqq_oracle_stop_iter(const double* mae, int n, int iters, int* rounds_out);
/* Stop rule: 0 keep z_(k-1) on a stop at round k (the page's rollback), 1 keep z_k, 2 keep
 * z_(k+1); flag 4 keeps z_(iters-1) instead of z_iters when the loop never stops. */
int hqq_oracle_stop_iter_rule(const double* mae, int n, int iters, int rule, int* rounds_out);

int hqq_oracle_quantize(const double* W, int64_t rows, int64_t cols, int nbits, int g, int axis, int iters,
                        double p, double beta0, double kappa, double tiny, uint8_t* codes, double* s_out,
                        double* delta_out, double* z_out, double* mae_out, int* rounds_out, int* kout_out);
int hqq_oracle_quantize_rule(const double* W, int64_t rows, int64_t cols, int nbits, int g, int axis, int iters,
                             double p, double beta0, double kappa, double tiny, int stop_rule, uint8_t* codes,
                             double* s_out, double* delta_out, double* z_out, double* mae_out, int* rounds_out,
                             int* kout_out);
/* Scale search per group over a grid of multipliers of the min-max scale (reading in
 * hqq_oracle.c, parity unpinned as to the reference project).  choice_out (may be NULL): the
 * index of the chosen multiplier per group. */
int hqq_oracle_quantize_v2(const double* W, int64_t rows, int64_t cols, int nbits, int g, int axis, int iters,
                           double p, double beta0, double kappa, double tiny, const double* grid, int ncand,
                           uint8_t* codes, double* s_out, double* delta_out, double* z_out, uint8_t* choice_out);
int hqq_oracle_quantize_groups(const double* Wg, int64_t n, int g, int nbits, int kout, double p, double beta0,
                               double kappa, double tiny, uint8_t* codes, double* s_out, double* delta_out,
                               double* z_out, double* z_traj, double* err_traj);

int64_t hqq_oracle_packed_bytes(int64_t N, int nbits);
int hqq_oracle_pack(const uint8_t* codes, int64_t N, int nbits, uint8_t* out);
int hqq_oracle_unpack(const uint8_t* packed, int64_t N, int nbits, uint8_t* codes);

int hqq_oracle_dequant(const uint8_t* packed, const double* delta, const double* zero, int64_t rows, int64_t cols,
                       int nbits, int g, int axis, double* out_f64, uint16_t* out_f16);
int hqq_oracle_gemv(const uint8_t* packed, const double* delta, const double* zero, int64_t N, int64_t K, int g,
                    const double* x, int64_t batch, const int64_t* rows_sel, int64_t n_sel, double* y);
int hqq_oracle_gemv_fmt(const uint8_t* packed, const double* delta, const double* zero, int64_t N, int64_t K,
                        int nbits, int g, int axis, const double* x, int64_t batch, const int64_t* rows_sel,
                        int64_t n_sel, double* y);
/* O9: dX [batch][n_sel] = dY [batch][N] @ W_hat [N][K] for the selected columns (the input
 * gradient of the forward product). */
int hqq_oracle_gemv_t(const uint8_t* packed, const double* delta, const double* zero, int64_t N, int64_t K,
                      int nbits, int g, int axis, const double* dy, int64_t batch, const int64_t* cols_sel,
                      int64_t n_sel, double* dx);

#ifdef __cplusplus
}
#endif
#endif
