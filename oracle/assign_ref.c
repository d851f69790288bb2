/*
 * Oracle (test infrastructure only): nearest-centroid search by the plain
 * definition, in fp64, with plain loops.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this file's library.  The GPU path never links or calls it, and it
 * shares no code with the GPU path.
 *
 * What it computes (Flash-KMeans paper summary, "Method": the assignment
 * stage computes the squared distances to every centroid and takes the
 * row-wise arg-min; paper digest, "K-Means聚类算法": the objective is the sum
 * over points of ||x_i - c_{a_i}||^2):
 *
 *   d_ik = sum_j (x_ij - c_kj)^2          (fp64, j ascending)
 *   a_i  = the lowest k with d_ik == min_k d_ik   (strict '<' while k ascends)
 *   d1_i = d_{i,a_i}
 *   d2_i = min over k != a_i of d_ik      (+inf when K == 1)
 *
 * The pages do not state a tie rule; the lowest index is the reading taken.
 * d2 feeds the near-tie test of the parity checks (gap d2 - d1 against d1).
 */
#include <math.h>
#include <stdint.h>

void oracle_assign(const double *x, const double *c, int64_t n, int64_t k, int64_t d,
                   int64_t *a, double *d1, double *d2)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 64)
    for (i = 0; i < n; ++i) {
        const double *xi = x + i * d;
        double best = INFINITY, second = INFINITY;
        int64_t arg = 0;
        for (int64_t kk = 0; kk < k; ++kk) {
            const double *ck = c + kk * d;
            double s = 0.0;
            for (int64_t j = 0; j < d; ++j) {
                double t = xi[j] - ck[j];
                s += t * t;
            }
            if (s < best) {
                second = best;
                best = s;
                arg = kk;
            } else if (s < second) {
                second = s;
            }
        }
        a[i] = arg;
        d1[i] = best;
        d2[i] = second;
    }
}

/* Distances of points to one chosen centroid each: out_i = sum_j (x_ij - c_{sel_i, j})^2. */
void oracle_dist_to(const double *x, const double *c, const int64_t *sel, int64_t n, int64_t d,
                    double *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        const double *xi = x + i * d;
        const double *ck = c + sel[i] * d;
        double s = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            double t = xi[j] - ck[j];
            s += t * t;
        }
        out[i] = s;
    }
}

/* Number of OpenMP threads the loops above use. */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
#else
int oracle_threads(void) { return 1; }
#endif
