/*
 * Plain CPU oracle for exact causal long convolution and for the autoregressive
 * mixer stack built from it.  TEST INFRASTRUCTURE ONLY: the product path never
 * links, loads or calls this file; only tests, the smoke check and the bench's
 * CPU-baseline leg do.
 *
 * Everything here is the definition written out, with no blocking, tiling or
 * reordering (the method is exact, so its result is the definition's result):
 *
 *   Flash Inference (arXiv 2410.12982), summary page, "Aufgabendefinition" and
 *   "LCSM-spezifische Definition": per layer and channel the mixer output at
 *   position t is  z_t = sum_{i=1..t} y_i * rho_{t-i}  (1-based positions).
 *   Storage here is 0-based: out[t] = sum_{s=0..t} h[t-s] * in[s].
 *
 *   Same page, "LCSM-Inferenz-Algorithmus" (Algorithm 2): at each position the
 *   layers run in order, layer l's input at that position is the block map of
 *   layer l-1's mixer output at that position, and the next model input is the
 *   sampler applied to the last layer's activation.  In the synthetic mixer
 *   stacks the block map and the sampler are elementwise tanh, so every
 *   (batch, channel) chain through all layers is independent of the others.
 *
 * Arithmetic: inputs and filters arrive as fp32; every product, sum and tanh
 * is evaluated in fp64, and activations are kept in fp64.  A second variant
 * with fp32 accumulation and fp32 activations (same loop order) exists only to
 * measure how fast rounding differences grow in feedback mode.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* out[t] = sum_{s<=t} h[t-s]*x[s] for t in [0, L) ; fp64 accumulation. */
static void conv_row_f64(const float *h, const float *x, int64_t L, double *out) {
    for (int64_t t = 0; t < L; ++t) {
        double acc = 0.0;
        for (int64_t s = 0; s <= t; ++s) acc += (double)h[t - s] * (double)x[s];
        out[t] = acc;
    }
}

/* Row-batched causal convolution: row r convolves h[r*h_ld ...] with
 * x[r*x_ld ...] over L positions into out[r*L ...].  Rows run in parallel. */
void orc_conv_rows(const float *h, int64_t h_ld, const float *x, int64_t x_ld,
                   int64_t rows, int64_t L, double *out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r)
        conv_row_f64(h + r * h_ld, x + r * x_ld, L, out + r * L);
}

/* Selected outputs only: out[k] = sum_{s<=ts[k]} h[ts[k]-s]*x[s].  Lets a
 * full-length row be checked at sampled positions in O(t) each. */
void orc_conv_points(const float *h, const float *x, const int64_t *ts, int64_t nt,
                     double *out) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t k = 0; k < nt; ++k) {
        const int64_t t = ts[k];
        double acc = 0.0;
        for (int64_t s = 0; s <= t; ++s) acc += (double)h[t - s] * (double)x[s];
        out[k] = acc;
    }
}

/*
 * Autoregressive mixer stack, one independent chain per entry of chan[].
 *
 *   filters : [M][D][L] fp32, layer-major, channel rows of L taps.
 *   chan    : channel index c of each chain (the batch index only selects the
 *             input values, the filter is shared over the batch).
 *   x_first : [nch] input of layer 0 at the first position.
 *   x_given : [nch][steps] layer-0 inputs for every position (teacher forcing),
 *             or NULL for feedback mode.
 *   map_tanh: 1 -> layer l+1 input = tanh(layer l output); 0 -> identity.
 *   fb_tanh : feedback (x_given == NULL): next layer-0 input = tanh(last output)
 *             if 1, else the last output itself.
 *   ys, xs  : [nch][M][steps] fp64 outputs: mixer output y and layer input x
 *             of every layer at every position.
 *
 * For position n (0-based) and layer l:
 *   y^l_n = sum_{s<=n} h^l[c][n-s] * x^l_s
 *   x^{l+1}_n = map(y^l_n)
 * then x^0_{n+1} = given value or feedback(y^{M-1}_n).
 */
void orc_stack(int M, int D, int64_t L, const float *filters, int nch, const int *chan,
               const float *x_first, const float *x_given, int map_tanh, int fb_tanh,
               int64_t steps, double *ys, double *xs) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int k = 0; k < nch; ++k) {
        const int c = chan[k];
        double *yk = ys + (int64_t)k * M * steps;
        double *xk = xs + (int64_t)k * M * steps;
        double x_next = (double)x_first[k];
        for (int64_t n = 0; n < steps; ++n) {
            double xin = (x_given != NULL) ? (double)x_given[(int64_t)k * steps + n] : x_next;
            for (int l = 0; l < M; ++l) {
                const float *h = filters + ((int64_t)l * D + c) * L;
                double *xl = xk + (int64_t)l * steps;
                xl[n] = xin;
                double acc = 0.0;
                for (int64_t s = 0; s <= n; ++s) acc += (double)h[n - s] * xl[s];
                yk[(int64_t)l * steps + n] = acc;
                xin = map_tanh ? tanh(acc) : acc;
            }
            const double ylast = yk[(int64_t)(M - 1) * steps + n];
            x_next = fb_tanh ? tanh(ylast) : ylast;
        }
        (void)D;
        (void)L;
    }
}

/* The same definition evaluated entirely in fp32 (storage, products, sums,
 * tanh).  Used only to measure the divergence horizon of feedback runs. */
void orc_stack_f32(int M, int D, int64_t L, const float *filters, int nch, const int *chan,
                   const float *x_first, int map_tanh, int fb_tanh, int64_t steps,
                   float *ys, float *xs) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int k = 0; k < nch; ++k) {
        const int c = chan[k];
        float *yk = ys + (int64_t)k * M * steps;
        float *xk = xs + (int64_t)k * M * steps;
        float x_next = x_first[k];
        for (int64_t n = 0; n < steps; ++n) {
            float xin = x_next;
            for (int l = 0; l < M; ++l) {
                const float *h = filters + ((int64_t)l * D + c) * L;
                float *xl = xk + (int64_t)l * steps;
                xl[n] = xin;
                float acc = 0.0f;
                for (int64_t s = 0; s <= n; ++s) acc += h[n - s] * xl[s];
                yk[(int64_t)l * steps + n] = acc;
                xin = map_tanh ? tanhf(acc) : acc;
            }
            const float ylast = yk[(int64_t)(M - 1) * steps + n];
            x_next = fb_tanh ? tanhf(ylast) : ylast;
        }
        (void)D;
        (void)L;
    }
}
