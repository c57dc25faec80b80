/*
 * conv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The fp64 reference ("oracle") for the forward convolution layer.  Only the
 * tests, the smoke check and the bench's CPU-baseline leg load this library;
 * the product (libconv and its Python binding) never does, and the two share
 * no source, header, table or helper.
 *
 * What it computes (definition, written out):
 *   The direct convolution compute shader of the page "PP-OCR on Vulkan
 *   compute shaders" (lpnh.cn/news/2745477), section 2.2: every output element
 *   is a gather -- start from the output coordinate, derive the input
 *   coordinate  in = out*stride - pad + k  for each kernel tap k, skip taps that
 *   fall outside the input (zero padding), multiply by the weight at
 *   ((oc*inC + ic)*kH + ky)*kW + kx, sum over input channels and taps, and add
 *   the bias of the output channel.  No kernel flip (cross-correlation).
 *   The same section notes that gathering from the output side is race free.
 *   The activation is applied to (sum + bias); section 4.4 of that page fuses
 *   ReLU into the write-back of the convolution.
 *   The 3-D form (one more spatial axis, frames) is the Convolution3D layer of
 *   the page "SeedVR2 NCNN Vulkan" (Tencent/ncnn discussion 7001), section 3.2;
 *   it adds the frame axis with the same gather rule.
 *   Layouts: x [N][C][T][H][W], w [CO][C][KT][KH][KW], b [CO], y [N][CO][OT][OH][OW]
 *   (2-D is T = KT = 1, pad_t = 0, stride_t = 1).
 *
 * Alongside each output it returns S = |b| + sum over in-bounds taps of
 * |x*w|, the denominator of the relative error bound used by the tests.
 *
 * Arithmetic: IEEE fp64 throughout, one output element at a time, in the plain
 * loop order ci, kt, kh, kw.  OpenMP distributes output elements over threads;
 * every element is computed by exactly one thread, so the result does not
 * depend on the thread count.
 *
 * Pins: tests/test_oracle.py (closed form for all-ones inputs, delta kernels,
 * linearity, brute-force im2col x matmul, torch's fp64 CPU convolution, the
 * stride and 3-D/2-D identities, the hand-computed fixture in tests/golden/;
 * for time padding on one side: the all-ones closed form, torch's conv3d of
 * the explicitly zero-padded input, and causal = symmetric then cropped).
 */
#include <math.h>
#include <stdint.h>
#include <omp.h>

/* Geometry of one call.  Index order of dims[]: D_PT is the time padding
 * before the first frame, D_PTB the time padding after the last one (equal
 * for the symmetric padding of the conv shader; the causal padding of the
 * spatio-temporal VAE in "SeedVR2 NCNN Vulkan", section 7.2, pads only before
 * the first frame). */
enum { D_N, D_C, D_T, D_H, D_W, D_CO, D_KT, D_KH, D_KW,
       D_PT, D_PH, D_PW, D_ST, D_SH, D_SW, D_PTB, D_COUNT };

typedef struct {
  long N, C, T, H, W, CO, KT, KH, KW, pt, ph, pw, st, sh, sw, ptb;
  long OT, OH, OW;
} geom_t;

/*
 * Number of output positions along one axis: the window of k taps starting at
 * o*stride - pad must end inside the padded input [-pad, in - 1 + pad].
 * Counted by walking o upwards -- the plain reading of "slide the window until
 * it no longer fits".
 */
long oracle_out_extent(long in, long k, long pad, long stride)
{
  if (in < 1 || k < 1 || pad < 0 || stride < 1) return -1;
  long count = 0;
  for (long o = 0; o * stride - pad + (k - 1) <= in - 1 + pad; ++o) ++count;
  return count;
}

/*
 * The same count with different padding before (pad_lo) and after (pad_hi)
 * the input: the window must end inside [-pad_lo, in - 1 + pad_hi].
 */
long oracle_out_extent2(long in, long k, long pad_lo, long pad_hi, long stride)
{
  if (in < 1 || k < 1 || pad_lo < 0 || pad_hi < 0 || stride < 1) return -1;
  long count = 0;
  for (long o = 0; o * stride - pad_lo + (k - 1) <= in - 1 + pad_hi; ++o) ++count;
  return count;
}

static int make_geom(const long* d, geom_t* g)
{
  g->N = d[D_N];  g->C = d[D_C];  g->T = d[D_T];  g->H = d[D_H];  g->W = d[D_W];
  g->CO = d[D_CO]; g->KT = d[D_KT]; g->KH = d[D_KH]; g->KW = d[D_KW];
  g->pt = d[D_PT]; g->ph = d[D_PH]; g->pw = d[D_PW];
  g->st = d[D_ST]; g->sh = d[D_SH]; g->sw = d[D_SW];
  g->ptb = d[D_PTB];
  if (g->N < 1 || g->C < 1 || g->CO < 1) return -1;
  g->OT = oracle_out_extent2(g->T, g->KT, g->pt, g->ptb, g->st);
  g->OH = oracle_out_extent(g->H, g->KH, g->ph, g->sh);
  g->OW = oracle_out_extent(g->W, g->KW, g->pw, g->sw);
  if (g->OT < 0 || g->OH < 0 || g->OW < 0) return -1;
  return 0;
}

/* One output element y[n][co][ot][oh][ow] and its S. */
static void conv_point(const double* x, const double* w, const double* b,
                       const geom_t* g, int relu,
                       long n, long co, long ot, long oh, long ow,
                       double* y_out, double* s_out)
{
  double acc = 0.0, mag = 0.0;
  if (b) { acc = b[co]; mag = fabs(b[co]); }
  for (long ci = 0; ci < g->C; ++ci) {
    for (long kt = 0; kt < g->KT; ++kt) {
      long it = ot * g->st - g->pt + kt;
      if (it < 0 || it >= g->T) continue;          /* zero padding in time */
      for (long kh = 0; kh < g->KH; ++kh) {
        long ih = oh * g->sh - g->ph + kh;
        if (ih < 0 || ih >= g->H) continue;        /* zero padding in height */
        for (long kw = 0; kw < g->KW; ++kw) {
          long iw = ow * g->sw - g->pw + kw;
          if (iw < 0 || iw >= g->W) continue;      /* zero padding in width */
          double xv = x[(((n * g->C + ci) * g->T + it) * g->H + ih) * g->W + iw];
          double wv = w[(((co * g->C + ci) * g->KT + kt) * g->KH + kh) * g->KW + kw];
          double p = xv * wv;
          acc += p;
          mag += fabs(p);
        }
      }
    }
  }
  if (relu && !(acc > 0.0)) acc = 0.0;
  *y_out = acc;
  *s_out = mag;
}

static void set_threads(int threads)
{
  if (threads > 0) omp_set_num_threads(threads);
}

/* Threads the next parallel region will use. */
int oracle_threads(int threads)
{
  set_threads(threads);
  return omp_get_max_threads();
}

/*
 * Full convolution.  dims[] as in the enum above; b may be NULL (no bias);
 * relu is 0 or 1.  y and s hold N*CO*OT*OH*OW doubles each.  threads <= 0
 * keeps OpenMP's default.  Returns 0, or -1 on bad geometry.
 */
int oracle_conv(const double* x, const double* w, const double* b,
                double* y, double* s, const long* dims, int relu, int threads)
{
  geom_t g;
  if (make_geom(dims, &g) != 0) return -1;
  long total = g.N * g.CO * g.OT * g.OH * g.OW;
  set_threads(threads);
  #pragma omp parallel for schedule(dynamic, 256)
  for (long idx = 0; idx < total; ++idx) {
    long r = idx;
    long ow = r % g.OW; r /= g.OW;
    long oh = r % g.OH; r /= g.OH;
    long ot = r % g.OT; r /= g.OT;
    long co = r % g.CO; r /= g.CO;
    long n = r;
    conv_point(x, w, b, &g, relu, n, co, ot, oh, ow, &y[idx], &s[idx]);
  }
  return 0;
}

/*
 * Selected outputs only: idx[i] is a flat index into y [N][CO][OT][OH][OW].
 * Returns 0, -1 on bad geometry, -2 on an index out of range.
 */
int oracle_conv_points(const double* x, const double* w, const double* b,
                       const int64_t* idx, long npts, double* y, double* s,
                       const long* dims, int relu, int threads)
{
  geom_t g;
  if (make_geom(dims, &g) != 0) return -1;
  long total = g.N * g.CO * g.OT * g.OH * g.OW;
  for (long i = 0; i < npts; ++i)
    if (idx[i] < 0 || idx[i] >= total) return -2;
  set_threads(threads);
  #pragma omp parallel for schedule(dynamic, 16)
  for (long i = 0; i < npts; ++i) {
    long r = (long)idx[i];
    long ow = r % g.OW; r /= g.OW;
    long oh = r % g.OH; r /= g.OH;
    long ot = r % g.OT; r /= g.OT;
    long co = r % g.CO; r /= g.CO;
    long n = r;
    conv_point(x, w, b, &g, relu, n, co, ot, oh, ow, &y[i], &s[i]);
  }
  return 0;
}
