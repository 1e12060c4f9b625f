/*
 * Oracle for the gated, grouped, depthwise causal FIR convolution
 *     y = q (.) (h * (k (.) v))
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes, written out as the plain definition (no blocking, no
 * Toeplitz split, no reordering beyond the sum's natural index order):
 *
 *   Page "04. hardware-aware convolution kernels" (StripedHyena 2 explainer),
 *   section 1, first equation: a causal FIR filter h of length l_h applied to
 *   an input x of length l gives  y_t = sum_{j=0..t} h_{t-j} x_j,  with
 *   h_i = 0 for i < 0 or i >= l_h.
 *
 *   Same page, section 4 (Algorithm 1): the output chunk is gated by q after
 *   the convolution, and k is loaded beside v; the convolution input is read
 *   here as x = k (.) v, the reading under which the loaded k has a role.
 *
 *   Same page, section 4, first bullet list: all channels of a group share
 *   one filter; channel d uses filter floor(d / group_size).
 *
 * Arithmetic is fp64 on the exact values the caller passes (bf16 or fp32
 * inputs are widened to fp64 by the caller, which is lossless).  Each batch
 * row starts with zero history (x_t = 0 for t < 0).
 *
 * Layout: q, k, v, y are [B, L, D] row-major (D contiguous); h is
 * [D / group_size, l_h] row-major (taps contiguous).
 */
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Return codes: 0 ok, -1 null pointer, -2 bad shape, -3 bad group size,
 * -4 bad filter length. */
int hyena_ref_fwd_f64(const double *q, const double *k, const double *v,
                      const double *h, int64_t B, int64_t L, int64_t D,
                      int64_t group_size, int64_t l_h, double *y)
{
    if (!q || !k || !v || !h || !y)
        return -1;
    if (B < 0 || L < 0 || D < 0)
        return -2;
    if (group_size < 1 || (D % group_size) != 0)
        return -3;
    if (l_h < 1)
        return -4;
    if (B == 0 || L == 0 || D == 0)
        return 0;

    const int64_t rows = B * L;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        const int64_t b = row / L;
        const int64_t t = row % L;
        const size_t batch0 = (size_t)b * (size_t)L * (size_t)D;
        for (int64_t d = 0; d < D; ++d) {
            const double *hg = h + (size_t)(d / group_size) * (size_t)l_h;
            /* only j with 0 <= t - j < l_h contribute */
            int64_t j0 = t - (l_h - 1);
            if (j0 < 0)
                j0 = 0;
            double z = 0.0;
            for (int64_t j = j0; j <= t; ++j) {
                const size_t o = batch0 + (size_t)j * (size_t)D + (size_t)d;
                const double x = k[o] * v[o];
                z += hg[t - j] * x;
            }
            const size_t oy = batch0 + (size_t)t * (size_t)D + (size_t)d;
            y[oy] = q[oy] * z;
        }
    }
    return 0;
}

/* Number of OpenMP threads a call above uses (1 without OpenMP). */
int hyena_ref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the OpenMP threads later calls use (n >= 1); for timing the oracle
 * on one core beside all of them.  No effect without OpenMP. */
void hyena_ref_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Backward of the same operator: given dy = dLoss/dy, the gradients of
 *     y[b,t,d] = q[b,t,d] * z[b,t,d],   z[b,t,d] = sum_{s<l_h, s<=t} h[g,s] x[b,t-s,d],
 *     x = k (.) v,   g = d / group_size,
 * written out by the chain rule, term by term, in fp64:
 *     dq[b,t,d] = dy[b,t,d] * z[b,t,d]
 *     dz[b,t,d] = dy[b,t,d] * q[b,t,d]
 *     dx[b,j,d] = sum_{s<l_h, j+s<L} h[g,s] dz[b,j+s,d]      (x[b,j,d] enters z at t = j+s)
 *     dk = dx (.) v,   dv = dx (.) k
 *     dh[g,s]   = sum_{b, d in g, t>=s} dz[b,t,d] x[b,t-s,d]
 * The page "04. hardware-aware convolution kernels", section 7, states that
 * the filter gradient is a global accumulation over every position; here it
 * is that sum, in one fp64 accumulator per (g, s).  dh is [G, l_h]; every
 * other array is [B, L, D].  Any of dq, dk, dv, dh may be NULL (skipped).
 * Return codes as hyena_ref_fwd_f64.
 */
int hyena_ref_bwd_f64(const double *q, const double *k, const double *v,
                      const double *h, const double *dy, int64_t B, int64_t L,
                      int64_t D, int64_t group_size, int64_t l_h, double *dq,
                      double *dk, double *dv, double *dh)
{
    if (!q || !k || !v || !h || !dy)
        return -1;
    if (B < 0 || L < 0 || D < 0)
        return -2;
    if (group_size < 1 || (D % group_size) != 0)
        return -3;
    if (l_h < 1)
        return -4;
    const int64_t G = D / group_size;
    if (dh) {
        for (int64_t i = 0; i < G * l_h; ++i)
            dh[i] = 0.0;
    }
    if (B == 0 || L == 0 || D == 0)
        return 0;
    const int64_t rows = B * L;

    if (dq) {
#pragma omp parallel for schedule(static)
        for (int64_t row = 0; row < rows; ++row) {
            const int64_t b = row / L, t = row % L;
            const size_t batch0 = (size_t)b * (size_t)L * (size_t)D;
            for (int64_t d = 0; d < D; ++d) {
                const double *hg = h + (size_t)(d / group_size) * (size_t)l_h;
                int64_t j0 = t - (l_h - 1);
                if (j0 < 0)
                    j0 = 0;
                double z = 0.0;
                for (int64_t j = j0; j <= t; ++j) {
                    const size_t o = batch0 + (size_t)j * (size_t)D + (size_t)d;
                    z += hg[t - j] * (k[o] * v[o]);
                }
                const size_t oy = batch0 + (size_t)t * (size_t)D + (size_t)d;
                dq[oy] = dy[oy] * z;
            }
        }
    }
    if (dk || dv) {
#pragma omp parallel for schedule(static)
        for (int64_t row = 0; row < rows; ++row) {
            const int64_t b = row / L, j = row % L;
            const size_t batch0 = (size_t)b * (size_t)L * (size_t)D;
            for (int64_t d = 0; d < D; ++d) {
                const double *hg = h + (size_t)(d / group_size) * (size_t)l_h;
                double dx = 0.0;
                for (int64_t s = 0; s < l_h && j + s < L; ++s) {
                    const size_t o = batch0 + (size_t)(j + s) * (size_t)D + (size_t)d;
                    dx += hg[s] * (dy[o] * q[o]);
                }
                const size_t ox = batch0 + (size_t)j * (size_t)D + (size_t)d;
                if (dk)
                    dk[ox] = dx * v[ox];
                if (dv)
                    dv[ox] = dx * k[ox];
            }
        }
    }
    if (dh) {
        const int64_t pairs = G * l_h;
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t gs_ = 0; gs_ < pairs; ++gs_) {
            const int64_t g = gs_ / l_h, s = gs_ % l_h;
            double acc = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                const size_t batch0 = (size_t)b * (size_t)L * (size_t)D;
                for (int64_t t = s; t < L; ++t) {
                    const size_t rt = batch0 + (size_t)t * (size_t)D;
                    const size_t rx = batch0 + (size_t)(t - s) * (size_t)D;
                    for (int64_t d = g * group_size; d < (g + 1) * group_size; ++d)
                        acc += (dy[rt + d] * q[rt + d]) * (k[rx + d] * v[rx + d]);
                }
            }
            dh[gs_] = acc;
        }
    }
    return 0;
}
