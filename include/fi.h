/*
 * fi.h -- C-ABI of the MI355X exact autoregressive long-convolution library.
 *
 * What it computes.  Flash Inference (arXiv 2410.12982), summary page,
 * "Aufgabendefinition" and "LCSM-spezifische Definition": for every layer l,
 * batch row b and channel c, the mixer output at position n (1-based) is
 *
 *     y^l_n[b,c] = sum_{s=1..n} h^l[c][n-s] * x^l_s[b,c]
 *
 * where x^l_s is the layer's input at position s, which only becomes known
 * after position s-1 has been produced ("unlock y_{i+1}" in Algorithm 1).
 * The filters h^l are data independent and known ahead.
 *
 * How.  "Kachelung-Strategie (Algorithmus 1)" and "Schicht-uebergreifende
 * Parallelisierung (Algorithmus 3)": after position n the library adds the
 * contribution of inputs [n-U+1, n] to outputs [n+1, n+U], U = largest power
 * of two dividing n ("gray block"), for all layers in one batched launch; the
 * own-position term h^l[c][0] * x^l_n ("red cell") is added when position n is
 * produced.  A gray block is computed either directly or through an FFT of
 * length 2U against a cached filter spectrum ("Technische Innovationen",
 * "FFT-Vorberechnung" and "Zirkulaere Faltungs-Trick"), chosen per block size
 * ("Hybrid" in "Vergleichsmethoden"; selection by profiling per shape and
 * block size, rebuttal page).
 *
 * Conventions shared by every call.
 *  - Positions are 1-based; the context starts at position 0 (nothing
 *    produced).  L, the maximum number of positions, must be a power of two
 *    (so no gray block runs past L).
 *  - All device buffers are caller-owned plain device pointers (for example
 *    torch tensors' data pointers), fp32, row-major, densely packed.
 *  - All calls are ordered on the stream bound at fi_init and return without
 *    waiting for the device unless stated; outputs are valid once that stream
 *    has been synchronised.
 *  - Any HIP error poisons the context: that call and every later call except
 *    fi_destroy/fi_last_error/fi_position return FI_ESTATE (the failing call
 *    itself returns FI_EDEVICE).  fi_last_error() describes the first failure.
 *  - A context is not thread safe; use one context per stream.
 */
#ifndef FI_H
#define FI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fi_ctx fi_ctx; /* opaque, owned by the library */

typedef enum fi_status {
    FI_OK = 0,
    FI_EINVAL = -1,  /* bad argument (shape, null pointer, L not a power of two) */
    FI_ENOMEM = -2,  /* device memory could not be allocated / workspace too small */
    FI_EDEVICE = -3, /* a HIP call failed (the context is now poisoned) */
    FI_ERANGE = -4,  /* stepping past position L */
    FI_ESTATE = -5   /* context poisoned, or call not valid in the current mode */
} fi_status;

/* Map between layers: x^{l+1}_n = map(y^l_n).  Feedback: x^0_{n+1} = fb(y^{M-1}_n).
 * (The pages' synthetic model puts a block after each mixer and a sampler at
 * the end, "LCSM-Inferenz-Algorithmus"; the elementwise tanh stands in for both.)
 * FI_MAP_EXTERNAL: the caller runs its own block between layers with
 * fi_layer_red() / fi_tiles().
 * FI_MAP_HYENA: the library runs a Hyena-style block after every mixer
 * ("Modellarchitektur": a^l = block^l(mixer^l(a^{l-1}))), weights given by
 * fi_set_block_weights: [u|v|w] = x W, the mixer convolves q = u*w, its output
 * c gates m = v*c, z = GELU(m W1) W2 (exact-erf GELU, no biases),
 * a = z / sqrt(mean(z^2) + 1e-6), next layer input a, next position's layer-0
 * input fb(a^{M-1}).  Needs D % 8 == 0, D <= 768 and B <= 8.  Here "y" of fi_step /
 * fi_generate is a^{M-1}_n, the value the feedback is applied to. */
enum { FI_MAP_TANH = 0, FI_MAP_IDENTITY = 1, FI_MAP_EXTERNAL = 2, FI_MAP_HYENA = 3 };
enum { FI_FEEDBACK_TANH = 0, FI_FEEDBACK_IDENTITY = 1 };

/* How gray blocks are computed. AUTO: per block size, the faster path as timed
 * on the device at fi_init; DIRECT/FFT force one path where it exists (direct
 * blocks exist for U <= 128, FFT blocks for U >= 4). */
enum { FI_TAU_AUTO = 0, FI_TAU_DIRECT = 1, FI_TAU_FFT = 2 };
enum { FI_PATH_NONE = 0, FI_PATH_DIRECT = 1, FI_PATH_FFT = 2 };

typedef struct fi_options {
    int map;               /* FI_MAP_*; default FI_MAP_TANH */
    int feedback;          /* FI_FEEDBACK_*; default FI_FEEDBACK_TANH */
    int tau_mode;          /* FI_TAU_*; default FI_TAU_AUTO */
    int tau_split;         /* -1: per-class choice (AUTO calibrates); q >= 0: classes
                              with U = 2^q' >= 2^q use FFT, smaller ones DIRECT */
    int record;            /* 1: keep every layer's input and mixer output (tests) */
    int use_graphs;        /* 1 (default): fi_generate replays captured hipGraphs */
    int block_graph_log2;  /* k: a block graph replays the 2^k - 1 positions between
                              multiples of 2^k (default 6; 0 disables) */
    int filters_on_device; /* 1: the filters pointer given to fi_init is device memory */
    int fft_max_log2;      /* widest gray block done as one workgroup transform, as
                              log2(U) in [12, 14] (default 14: 128 KB of LDS); the
                              next class runs as two halves of that width in one
                              workgroup, wider blocks are split into sub-blocks of
                              that width */
    int time_blocks;       /* 1: fi_generate brackets every FFT gray-block launch with
                              HIP events stamped by the launches themselves (read with
                              fi_block_times); those positions then bypass graphs */
    int defer_wide;        /* 1: a split gray block at position n computes only its
                              first output sub-block (V positions) before position
                              n+1; the others run on a second stream of the context,
                              overlapping positions n+1 .. n+V-1, and the context
                              stream waits for them before position n+V.  Cuts the
                              latency of that position; results are bit for bit
                              those without it.  2: the same, and the two-half
                              class (twice fft_max_log2) is deferred too, run as 4
                              sub-blocks of half the one-workgroup width (V =
                              2^(fft_max_log2-1)); its results then differ from the
                              two-half kernel's by rounding.  Level 2 needs
                              fft_max_log2 >= 13, adds the offset spectra of that
                              width to the workspace (7 * V/2 float4 per (l, c)),
                              and where no two-half class exists acts as 1.
                              Default 0 */
    int chunk_direct;      /* 1 (default): for maps that act channel by channel
                              (FI_MAP_TANH, FI_MAP_IDENTITY), fi_generate and
                              fi_prefill run the G = 2^q positions between two
                              FFT positions (q: the first FFT class) as one
                              launch, each workgroup owning whole chains.  The
                              direct gray blocks of a chunk then sum, target by
                              target, the same pairs the tiling assigns them
                              (summary page, "Kachelung-Strategie"; the blocks
                              below G never leave a chunk).  0: one launch (or
                              graph node) per position */
    int eager_prefill;     /* 1 (default): fi_prefill at position 0 computes the
                              prompt layer by layer with all of a layer's
                              positions at once (direct sums inside blocks of G,
                              FFT blocks above), when the map acts channel by
                              channel, P is a multiple of G, P <= L/2, and every
                              gray block after n <= P wider than one workgroup
                              transform either starts at n = P or (the two-half
                              class) ends inside the prompt -- e.g. at
                              L = 2^17, P = 16384, 32768, 65536 -- otherwise, or
                              with 0, P teacher-forced positions */
    int reserved[3];       /* must be zero */
} fi_options;

/* Fill *opt with the defaults listed above. */
void fi_default_options(fi_options *opt);

/* Library version string, e.g. "fi 0.1 gfx950". */
const char *fi_version(void);

/* Device bytes fi_init needs for this shape and options (0 on bad arguments).
 * The workspace holds the filters, the per-layer activation rows (inputs for
 * positions <= n, pending sums for positions > n: the pages' activation reuse,
 * "Speicheroptimierung"), the cached filter spectra and scratch. */
size_t fi_workspace_bytes(int layers, int batch, int channels, int64_t L,
                          const fi_options *opt);

/* Create a context.
 *   layers M >= 1, batch B >= 1, channels D >= 1, L = 2^P with 1 <= L <= 2^24.
 *   filters: fp32 [M][D][L] (layer-major, channel rows of L taps h[0..L-1]),
 *            host memory unless opt->filters_on_device; copied, the caller keeps
 *            ownership and may free it when fi_init returns.
 *   opt:     NULL for defaults.
 *   workspace: device buffer of at least fi_workspace_bytes() bytes, 256-byte
 *            aligned, owned by the caller and untouched by it while the context
 *            lives; or NULL to let the library allocate (and free) its own.
 *   stream:  hipStream_t the context runs on (NULL = default stream).
 * Computes the filter spectra and, for FI_TAU_AUTO, times the block paths on
 * the device: with chunked positions (fi_options.chunk_direct and a map that
 * acts channel by channel), one chunk plus its FFT block per candidate split
 * (fi_chunk_table); otherwise both paths per block size (fi_tau_table).
 * Synchronises the stream before returning.
 * Returns FI_EINVAL / FI_ENOMEM / FI_EDEVICE on failure (*out is then NULL). */
fi_status fi_init(fi_ctx **out, int layers, int batch, int channels, int64_t L,
                  const float *filters, const fi_options *opt, void *workspace,
                  void *stream);

/* Release the context (and its own allocations).  Safe on NULL. */
fi_status fi_destroy(fi_ctx *ctx);

/* Back to position 0 with all activations cleared; filters, spectra and the
 * block-path table are kept. */
fi_status fi_reset(fi_ctx *ctx);

/* Set fi_options.defer_wide (0, 1 or 2) for the following positions.
 * Large-block latency (Flash Inference summary page, "Hauptergebnisse": the
 * per-token time spikes at the positions of the widest blocks): with it on, a
 * split gray block (level 2: also a two-half block) puts its later output
 * sub-blocks on the context's second stream.  Any deferred work still running
 * is joined into the context stream first.  FI_EINVAL for other values;
 * FI_ESTATE for 2 when the context has a two-half class that fi_init did not
 * prepare (fi_options.defer_wide was not 2 there). */
fi_status fi_set_defer_wide(fi_ctx *ctx, int on);

/* Produce the next position n = fi_position()+1 (Algorithm 2 for one i).
 *   x_t: device fp32 [B][D], the layer-0 input x^0_n; NULL = feedback
 *        (x^0_n = fb(y^{M-1}_{n-1}); at n = 1 the value given by fi_set_input).
 *   y_t: device fp32 [B][D] receiving the last layer's mixer output
 *        y^{M-1}_n (before the map), or NULL.
 * Runs the red cells of all layers in order, then the gray blocks of all
 * layers after n.  FI_ERANGE when the position is already L.
 * Not valid in FI_MAP_EXTERNAL mode (FI_ESTATE). */
fi_status fi_step(fi_ctx *ctx, const float *x_t, float *y_t);

/* Set the layer-0 input used by the next feedback step when no previous
 * output exists (position 0), device fp32 [B][D]. */
fi_status fi_set_input(fi_ctx *ctx, const float *x0);

/* Teacher-forced prompt (Flash Inference rebuttal page, reply on prefill: the
 * prompt is given at once, so its contributions to all later outputs can be
 * pushed eagerly; summary page, "Einschraenkungen": prefill dominates the
 * cost for long prompts): equivalent to P calls fi_step(x + (i-1)*B*D, y ...)
 * for i = 1..P (the invariant the tests check).
 *   x: device fp32 [P][B][D]; y: device fp32 [P][B][D] or NULL.
 * The prompt's positions are processed in place (position advances by P). */
fi_status fi_prefill(fi_ctx *ctx, const float *x, int64_t P, float *y);

/* Free-running generation of `steps` positions with internal feedback (summary
 * page, "LCSM-Inferenz-Algorithmus", Algorithm 2: per position the layers' red
 * cells in order, the next input from the last layer's output, then every
 * layer's gray block; "Schicht-uebergreifende Parallelisierung", Algorithm 3:
 * the gray blocks of all layers in one launch), with one hipGraph per
 * block-size class plus block graphs (use_graphs = 1) or chunk launches.
 *   y: device fp32 [steps][B][D] receiving y^{M-1}_n for each position, or NULL.
 * FI_ERANGE if position + steps > L (nothing is run). */
fi_status fi_generate(fi_ctx *ctx, int64_t steps, float *y);

/* Positions produced so far (0..L). */
int64_t fi_position(const fi_ctx *ctx);

/* Human-readable description of the first failure, or "" . */
const char *fi_last_error(const fi_ctx *ctx);

/* Schedule of step n (1 <= n <= L): *q = log2 of the gray-block edge after n
 * (or -1 for n = L, which has no gray block); *path = FI_PATH_* used for it. */
fi_status fi_debug_schedule(const fi_ctx *ctx, int64_t n, int *q, int *path);

/* Block-path table: for q = 0..P-1 writes path[q] (FI_PATH_*) and, when
 * calibration ran, the measured microseconds per launch of the direct and FFT
 * paths (negative where a path does not exist or was not timed).  Arrays hold
 * at least P entries; any pointer may be NULL. */
fi_status fi_tau_table(const fi_ctx *ctx, int *path, double *us_direct, double *us_fft);

/* Chunk-path calibration (FI_TAU_AUTO with chunked positions): for each
 * candidate first FFT class g (chunks of 2^g positions carry every block below
 * 2^g), us_chunk[g] = measured microseconds of one chunk and the class-g FFT
 * gray blocks after it, us_run[g] = the modeled microseconds of the classes
 * the choice affects over a whole run ((L / 2^g) chunks plus the FFT blocks of
 * classes g .. 8); the split used is the shortest chunk whose us_run is within
 * 1.5% of the least (closer than the timing repeats), so repeated
 * calibrations agree.  -1 where not timed.  Arrays hold at least P + 1 entries; either may be NULL. */
fi_status fi_chunk_table(const fi_ctx *ctx, double *us_chunk, double *us_run);

/* Copy positions first..first+count-1 (first >= 1) of one layer into dst
 * (device fp32, [count][B][D]):
 * what = 0: the layer's convolution inputs x^l_s, what = 1: its mixer outputs
 * y^l_s, what = 2 (FI_MAP_HYENA only): its block outputs a^l_s (valid for
 * s <= position).  Needs record = 1 (FI_ESTATE otherwise). */
fi_status fi_history(const fi_ctx *ctx, int layer, int what, int64_t first, int64_t count, float *dst);

/* Block weights for FI_MAP_HYENA, as bf16 bit patterns in row-major x*W
 * layout: W [M][D][3D], W1 [M][D][4D], W2 [M][4D][D]; host memory unless
 * on_device.  Copied (stored transposed); the caller keeps ownership.
 * Synchronises the stream.  Must precede any step in that mode (FI_ESTATE). */
fi_status fi_set_block_weights(fi_ctx *ctx, const uint16_t *W, const uint16_t *W1, const uint16_t *W2,
                               int on_device);

/* fi_set_block_weights for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same upload and the same result, but the staging buffer the
 * weights pass through on their way to the transposed layout is a fixed
 * device array of the library (4.5 MiB per device, its address looked up at
 * the first call on a device) instead of an allocation; no hipMalloc, hipFree
 * or other allocating call is made.  Limit: 4*D*D 16-bit values must fit the
 * array, i.e. D <= 768, the widest block FI_MAP_HYENA takes (FI_EINVAL with a
 * message otherwise).  Every call on one device shares that device's array
 * and leaves its contents there: calls that overlap on one device (other
 * streams or threads) race.  Synchronises the stream, like
 * fi_set_block_weights. */
fi_status fi_set_block_weights_static(fi_ctx *ctx, const uint16_t *W, const uint16_t *W1, const uint16_t *W2,
                                      int on_device);

/* Device wall-clock stamps (100 MHz counter ticks) written when each position
 * finished: dst (host int64 [count]) receives the stamps of positions
 * first..first+count-1.  Synchronises the stream. */
fi_status fi_stamps(fi_ctx *ctx, int64_t first, int64_t count, int64_t *dst);

/* External-block mode (FI_MAP_EXTERNAL).  For the current position
 * n = fi_position()+1 the caller, for l = 0..M-1 in order, supplies the
 * layer's mixer input q (device [B][D]) and receives its mixer output
 *     y^l_n = (pending sum at n) + h^l[c][0] * q
 * (the red cell of Algorithm 2), then calls fi_tiles() to run all layers'
 * gray blocks after n and advance to n.  y may alias nothing else. */
fi_status fi_layer_red(fi_ctx *ctx, int layer, const float *q, float *y);
fi_status fi_tiles(fi_ctx *ctx);

/* GPU Lazy baseline ("Vergleichsmethoden", Lazy: each position computes its
 * full sum on demand, O(n) per position, all layers' sums in parallel):
 * same semantics as fi_step / fi_generate (internal feedback) on a context
 * that has not run any tiled step since fi_init/fi_reset (FI_ESTATE
 * otherwise; likewise tiled calls after Lazy calls until fi_reset). */
fi_status fi_lazy_step(fi_ctx *ctx, const float *x_t, float *y_t);
fi_status fi_lazy_generate(fi_ctx *ctx, int64_t steps, float *y);

/* The pages' baselines and their ablations ("Vergleichsmethoden": Lazy,
 * Eager, Lazy NP, Eager NP; "Ablationsstudien", cross-layer parallelism):
 *   FI_BASE_LAZY      position n computes its full O(n) sum, all layers in
 *                     one launch, then the red cells (= fi_lazy_step);
 *   FI_BASE_EAGER     the red cells of n, then x_n is pushed into the pending
 *                     sums of every later position (O(L - n)), all layers in
 *                     one launch;
 *   FI_BASE_LAZY_NP,
 *   FI_BASE_EAGER_NP  the same with the per-row work launched layer by layer
 *                     (no cross-layer parallelism).
 * fi_baseline_step / fi_baseline_generate have the semantics of fi_step /
 * fi_generate (x_t device [B][D] or NULL for internal feedback; y_t device
 * [B][D] or NULL; y device [steps][B][D] or NULL).  A context steps one
 * family at a time: Lazy kinds and Eager kinds, and either with tiled calls,
 * cannot be mixed without fi_reset (FI_ESTATE).  kind outside the list:
 * FI_EINVAL; external-block and Hyena-style maps: FI_ESTATE. */
enum { FI_BASE_LAZY = 0, FI_BASE_EAGER = 1, FI_BASE_LAZY_NP = 2, FI_BASE_EAGER_NP = 3 };
fi_status fi_baseline_step(fi_ctx *ctx, int kind, const float *x_t, float *y_t);
fi_status fi_baseline_generate(fi_ctx *ctx, int kind, int64_t steps, float *y);

/* Benchmark support for the baselines: the mean device time in microseconds
 * of one baseline position n of the given kind (its sums or pushes plus the
 * red cells), over `reps` launches timed with HIP events, without advancing.
 * Overwrites activation rows: fi_reset is required before further stepping
 * (FI_ESTATE otherwise). */
fi_status fi_baseline_time(fi_ctx *ctx, int kind, int64_t n, int reps, double *us);

/* Per-class FFT gray-block timing (needs time_blocks = 1): for q = 0..P-1,
 * ms[q] = summed event-measured milliseconds of the FFT gray-block kernels of
 * class q launched by fi_generate, count[q] = number of such launches.
 * Synchronises the stream.  clear = 1 zeroes the sums afterwards.  Arrays hold
 * at least P entries; either may be NULL. */
fi_status fi_block_times(fi_ctx *ctx, int clear, double *ms, int64_t *count);

/* Chunk-kernel timing (needs time_blocks = 1): *ms = summed event-measured
 * milliseconds of the chunk kernels fi_generate / fi_step launched (each runs
 * the red cells and direct gray blocks of 2^k consecutive positions, see
 * fi_options.chunk_direct), *count = their number.  Synchronises the stream;
 * clear = 1 zeroes both afterwards.  Either pointer may be NULL. */
fi_status fi_chunk_times(fi_ctx *ctx, int clear, double *ms, int64_t *count);

/* Per-size runtime of one gray-block path (the pages' runtime-per-tile-size
 * comparison, "Pareto-Optimalitaetskurve"): the mean device time in
 * microseconds of the gray-block kernels of class q (U = 2^q) over `reps`
 * launches at position n = 2^q, timed with HIP events, without advancing.
 * path = FI_PATH_DIRECT (the direct kernel, red cells included) or
 * FI_PATH_FFT (the FFT kernels alone).  FI_EINVAL where the path does not
 * exist for q.  Overwrites activation rows: fi_reset is required before any
 * further stepping (FI_ESTATE otherwise). */
fi_status fi_time_block(fi_ctx *ctx, int q, int path, int reps, double *us);

/* Benchmark support for the time split between mixer and block (summary page,
 * "Zeit-Zerlegung (Abbildung 2a)"): the mean device time in microseconds of
 * one position's block kernels in FI_MAP_HYENA mode -- every layer's
 * projection (with its red cell), GELU up-projection and down-projection, then
 * the RMSNorm'd output and feedback -- without the gray blocks, over `reps`
 * launches timed with HIP events, without advancing.  Needs the block weights
 * (FI_ESTATE otherwise).  The activation rows are overwritten: fi_reset is
 * required before any further stepping (FI_ESTATE otherwise). */
fi_status fi_time_hyena_block(fi_ctx *ctx, int reps, double *us);

/* Benchmark support for the Lazy baseline: the mean device time in
 * microseconds of the Lazy work of position n (every layer's full O(n) sum
 * plus the red cells), over `reps` launches timed with HIP events, without
 * advancing.  The activation rows are overwritten: the context must be reset
 * (fi_reset) before any further stepping (FI_ESTATE otherwise). */
fi_status fi_lazy_time(fi_ctx *ctx, int64_t n, int reps, double *us);

/* ------------------------------------------------------------------------
 * Data-dependent filters.  Flash Inference, summary page, "Datenabhaengige
 * Filter-Erweiterung (Appendix B)": with a filter that depends on the data, a
 * modified tiling (Algorithm 5) keeps the method exact at twice the work; the
 * rebuttal page adds that each block then takes two same-size transforms
 * instead of one.  The pages give nothing more.  Reading used here: both
 * sequences arrive online, per batch row b and channel c the input x_t and the
 * filter tap h_t at position t (0-based, t = 0 .. L-1), and
 *
 *     y_t[b,c] = sum_{i+j=t} x_i[b,c] * h_j[b,c]
 *
 * (one layer; taps per (b, c), since a data-dependent filter differs per
 * sequence).  Tiling, p a power of two: red cell y_t = pend_t + x_t h_0 +
 * x_0 h_t; at t = 2p-1 the square x[p, 2p) * h[p, 2p); at t = (m+1)p-1,
 * m >= 2, the two band products x[t+1-p, t] * h[p, 2p) and h[t+1-p, t] *
 * x[p, 2p).  Each adds into the pending sums of positions t+1 .. t+2p-1.
 * Products of p >= 2^fft_min_log2 run as 2p-point FFTs against the cached
 * spectrum of the fixed block, smaller ones directly.
 *
 * One context per stream; calls are stream-ordered on the bound stream and
 * not thread-safe.  All pointers are caller-owned device memory, fp32,
 * [B][D] per position (row r = b*D + c), densely packed.
 * ------------------------------------------------------------------------ */
typedef struct fi_dd fi_dd; /* opaque, owned by the library */

/* Device bytes the workspace of a data-dependent context needs: three
 * [B*D][L] fp32 arrays (inputs, taps, pending sums) plus the fixed-block
 * spectra (16 L bytes per row), twiddles and one [B*D] array (the layer
 * inputs of a position, used by stacks).  0 if the shape is unsupported:
 * B, D >= 1, B*D <= 2^24, L a power of two up to 32768 (the widest product,
 * L/2 points, must fit one workgroup's transform); fft_min_log2 in [2, 15], or
 * -1 for the default 8.  Products of p < 2^fft_min_log2 run directly: up to
 * p = 128 inside the position's first launch (one thread per target), wider
 * ones one thread per row; the rest as FFTs. */
size_t fi_dd_workspace_bytes(int batch, int channels, int64_t L, int fft_min_log2);

/* Create a context at position 0 over the caller's workspace (device, at
 * least fi_dd_workspace_bytes, 256-byte aligned; the context keeps using it
 * until fi_dd_destroy).  stream: the hipStream_t every call of the context is
 * ordered on (NULL = default stream).  Synchronises the stream.  FI_EINVAL for a null
 * pointer or an unsupported shape, FI_EDEVICE if a HIP call fails. */
fi_status fi_dd_init(fi_dd **out, int batch, int channels, int64_t L, int fft_min_log2, void *workspace,
                     void *stream);

/* A stack of `layers` data-dependent layers in one context (the summary page's
 * layer stacks, "Schicht-uebergreifende Parallelisierung (Algorithmus 3)",
 * with the filters of "Datenabhaengige Filter-Erweiterung (Appendix B)"):
 * at each position layer l's taps h^l_t arrive with the data, layer 0's input
 * x^0_t too, and layer l+1's input is tanh(y^l_t).  The red cells run layer
 * after layer (one thread per (b, c) chain); every product of the position
 * then runs once for the rows of all layers.  Sizes and limits as
 * fi_dd_workspace_bytes, with 1 <= layers <= 64 and layers * batch * channels
 * rows; 0 for an unsupported shape. */
size_t fi_dd_stack_workspace_bytes(int layers, int batch, int channels, int64_t L, int fft_min_log2);

/* Create a stack context (as fi_dd_init; layers = 1 is the single layer). */
fi_status fi_dd_stack_init(fi_dd **out, int layers, int batch, int channels, int64_t L, int fft_min_log2,
                           void *workspace, void *stream);

/* One position: x_t ([B][D], device: layer 0's input) and h_t ([M][B][D],
 * device: every layer's tap, M the context's layers, 1 for fi_dd_init) arrive,
 * y_t ([M][B][D], device: every layer's output) is written.  FI_ERANGE after
 * L positions, FI_EINVAL for null pointers, FI_ESTATE after a device failure. */
fi_status fi_dd_step(fi_dd *ctx, const float *x_t, const float *h_t, float *y_t);

/* `steps` positions in a row: x is [steps][B][D], h and y [steps][M][B][D]
 * (device). */
fi_status fi_dd_run(fi_dd *ctx, const float *x, const float *h, int64_t steps, float *y);

/* Back to position 0 (inputs, taps and pending sums cleared). */
fi_status fi_dd_reset(fi_dd *ctx);

/* Positions produced so far (-1 for a null context). */
int64_t fi_dd_position(const fi_dd *ctx);

/* Message of the last failed call. */
const char *fi_dd_last_error(const fi_dd *ctx);

/* Synchronise the stream and free the context (not the workspace); FI_OK
 * for a null context, FI_EDEVICE if the synchronisation fails. */
fi_status fi_dd_destroy(fi_dd *ctx);

#ifdef __cplusplus
}
#endif

#endif /* FI_H */
