/*
 * adaln_sched.h -- host-side batch scheduling for mixed-length diffusion
 * training, from the AdaptiveLoad technical summary (gist.science, paper
 * 2605.17923), section 2.A "Equilibrio de Carga Adaptativo de Doble
 * Restricción", and its load-balance measure in section 4.
 *
 * Groups of equal-length sequences get the largest batch B that meets both a
 * linear memory bound and a polynomial compute bound (attention grows like
 * S^2 per sequence), instead of an "equal tokens" batch B*S = const:
 *
 *     B*S <= M_mem,   B*S^p <= M_comp,
 *     B_shape(S) = max(1, min(floor(M_mem/S), floor(M_comp/S^p)))
 *
 * and p (from which M_comp follows for a step-time budget) is calibrated by
 * timing synthetic shapes and fitting, by nonlinear regression,
 *
 *     step_time ~= a + b * B * S^p.
 *
 * These functions run on the host only: no device memory, no HIP calls, no
 * allocation visible to the caller; they are reentrant and thread-safe.
 * Every pointer is caller-owned host memory.  Status codes are those of
 * adaln.h.
 */
#ifndef ADALN_SCHED_H_
#define ADALN_SCHED_H_

#include <stdint.h>

#include "adaln.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * adaln_sched_batch_size -- B_shape(S) for sequence length S >= 1, memory
 * budget m_mem >= 0 (tokens), compute budget m_comp >= 0 (units of S^p) and
 * exponent p > 0 (finite).  For integral p the compute bound is floored in
 * exact integer arithmetic (S^p beyond int64 means the bound is 0); otherwise
 * it is floor(m_comp / pow(S, p)) in IEEE double.  Returns B_shape >= 1, or
 * -1 for invalid arguments.
 */
int64_t adaln_sched_batch_size(int64_t S, int64_t m_mem, int64_t m_comp, double p);

/*
 * adaln_sched_plan -- cut n samples of the given sequence lengths into
 * groups: the samples of one length are taken in input order, B_shape(S) at a
 * time, the last group of a length holding the remainder.  Groups are
 * numbered 0, 1, ... by ascending length, then input order.
 *
 *   lengths  [n] int64, every entry >= 1
 *   group_of [n] int64, output: group index of each sample
 *   n_groups      int64*, output: number of groups
 *
 * n == 0 gives *n_groups = 0.  ADALN_ERR_INVALID_ARG for null pointers
 * (lengths and group_of may be null when n == 0), n < 0, a length < 1 or
 * invalid budgets / exponent (as in adaln_sched_batch_size); outputs are then
 * untouched.
 */
adaln_status_t adaln_sched_plan(const int64_t* lengths, int64_t n, int64_t m_mem, int64_t m_comp,
                                double p, int64_t* group_of, int64_t* n_groups);

/*
 * adaln_cost_fit -- least-squares fit of step_time = a + b * B * S^p to n
 * timings t[i] measured at batch B[i] > 0 and sequence length S[i] > 0, with
 * p searched in [p_lo, p_hi] (0 < p_lo < p_hi <= 16).  For fixed p the model
 * is linear in (a, b), which are then solved in closed form; p minimises the
 * remaining sum of squares (a grid of 256 points, then golden-section
 * refinement around the best one).  Outputs a, b, p and the residual sum of
 * squares rss.  ADALN_ERR_INVALID_ARG for n < 3, null pointers, non-finite or
 * non-positive B or S, non-finite t, a bad interval, or shapes whose B*S^p
 * are all equal (no slope to fit).
 */
adaln_status_t adaln_cost_fit(const double* B, const double* S, const double* t, int64_t n,
                              double p_lo, double p_hi, double* a, double* b, double* p,
                              double* rss);

/*
 * adaln_load_cv -- coefficient of variation of n >= 1 per-worker loads:
 * population standard deviation over the mean.  Returns NaN for n < 1, a null
 * pointer or a zero mean.
 */
double adaln_load_cv(const double* load, int64_t n);

#ifdef __cplusplus
}
#endif

#endif /* ADALN_SCHED_H_ */
