/*
 * CPU oracle for the Gated DeltaNet prefill forward -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * may load this library. It shares no code, header or constant with the HIP
 * library it checks.
 *
 * What it computes is the token-by-token recurrence, which the chunkwise method
 * reproduces exactly up to rounding order:
 *   S_t = S_{t-1} * alpha_t * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T   (dv x dk)
 *   o_t = S_t q_t                        (read after the write)
 * with k, q L2-normalised, alpha_t = exp(-exp(A_log) softplus(a_t + dt_bias)),
 * beta_t = sigmoid(b_t).
 * Sources: "Simple math to speed up GDN prefill" (veitner), section Reminder,
 * state-transition equation; awehrs.io "NRM training kernels", General
 * implementation item 4 (a token sees its own write); pymllm gdn_chunkwise page,
 * Module Contents (gate parameters, q not pre-normalised, shapes).
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* in_dtype: 0 = fp32 values, 1 = bf16 bit patterns (uint16).
 * q, k: [N][H][dk]; v: [N][HV][dv]; a, b: [N][HV]; A_log, dt_bias: [HV].
 * heads[0..n_heads): the value heads to compute. Rows [row_lo, row_hi) of the state
 * (the dv index) are computed; rows evolve independently under the recurrence.
 * S: in/out, [batch][n_heads][row_hi-row_lo][dk] in fp64.
 * out: [N][n_heads][row_hi-row_lo] fp64 (rows of o for the selected heads).
 * eps: added to the squared norm before the inverse square root.
 * fp32_arith: 0 = fp64 arithmetic, 1 = the same loop in fp32 arithmetic.
 * Returns 0, or -1 on an invalid argument. */
int gdn_oracle_recurrence(int in_dtype, const void* q, const void* k, const void* v,
                          const float* a, const float* b, const float* A_log,
                          const float* dt_bias, const int64_t* cu_seqlens, int64_t batch,
                          int H, int HV, int dk, int dv, const int32_t* heads, int n_heads,
                          int row_lo, int row_hi, double* S, double* out, double eps,
                          int fp32_arith, int nthreads);

/* Gates for one (token, head): writes alpha, beta and g = log(alpha). */
void gdn_oracle_gates(double a, double b, double A_log, double dt_bias, double* alpha,
                      double* beta, double* g);

#ifdef __cplusplus
}
#endif
#endif
