/*
 * synth.c -- seeded synthetic input images for connected-component labelling.
 *
 * These generators draw pictures; they hold none of the labelling arithmetic
 * and are shared by the tests, the benchmark and the smoke check (both the
 * oracle and the HIP path receive the same bytes).
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based hash of
 * (seed, stream, index); a uniform double is the top 53 bits times 2^-53.  No
 * library distributions are used, so the bytes depend only on the seed.
 *
 * Colours of 32-bit pictures are packed 0x00RRGGBB.
 *
 * Every generator returns 0 on success and a negative value on bad arguments
 * or allocation failure.  OpenMP parallel loops write disjoint pixels or rows,
 * and every parallel reduction is order-independent, so the output does not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ RNG */

static inline uint64_t mix64(uint64_t x)
{
    x += 0x9E3779B97F4A7C15ULL;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ULL;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBULL;
    return x ^ (x >> 31);
}

static inline uint64_t rng_u64(uint64_t seed, uint64_t stream, uint64_t idx)
{
    return mix64(mix64(seed ^ mix64(stream * 0xD1B54A32D192ED03ULL + 1)) + idx);
}

static inline double rng_unif(uint64_t seed, uint64_t stream, uint64_t idx)
{
    return (double)(rng_u64(seed, stream, idx) >> 11) * (1.0 / 9007199254740992.0);
}

/* A sequential stream: successive draws from (seed, stream). */
typedef struct { uint64_t seed, stream, i; } rng_t;
static inline double draw(rng_t *r) { return rng_unif(r->seed, r->stream, r->i++); }
static inline int64_t draw_int(rng_t *r, int64_t lo, int64_t hi) /* [lo, hi] */
{
    int64_t v = lo + (int64_t)(draw(r) * (double)(hi - lo + 1));
    return v > hi ? hi : v;
}

/* ------------------------------------------------------------ geometry */

static inline double clampd(double v, double lo, double hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

/* distance from point (px,py) to segment (ax,ay)-(bx,by) */
static inline double seg_dist(double px, double py, double ax, double ay,
                              double bx, double by)
{
    const double vx = bx - ax, vy = by - ay;
    const double l2 = vx * vx + vy * vy;
    double t = l2 > 0 ? ((px - ax) * vx + (py - ay) * vy) / l2 : 0.0;
    t = clampd(t, 0.0, 1.0);
    const double dx = px - (ax + t * vx), dy = py - (ay + t * vy);
    return sqrt(dx * dx + dy * dy);
}

/* stroke coverage of a pixel whose centre is d away from the centre line */
static inline double coverage(double width, double d)
{
    return clampd(width * 0.5 + 0.5 - d, 0.0, 1.0);
}

static inline uint32_t rgb(int r, int g, int b)
{
    return ((uint32_t)r << 16) | ((uint32_t)g << 8) | (uint32_t)b;
}

/* "over" compositing of one stroke colour with coverage cov, per channel */
static inline uint32_t over(uint32_t under, uint32_t stroke, double cov)
{
    uint32_t out = 0;
    for (int sh = 0; sh <= 16; sh += 8) {
        const double u = (double)((under >> sh) & 0xFF);
        const double s = (double)((stroke >> sh) & 0xFF);
        int v = (int)floor(cov * s + (1.0 - cov) * u + 0.5);
        v = v < 0 ? 0 : (v > 255 ? 255 : v);
        out |= (uint32_t)v << sh;
    }
    return out;
}

/* ==================================================================
 * Config 1: small drawing.  White background, 40 random line segments of
 * width 1-4 px in black whose partly covered edge pixels take one of 8 grey
 * shades (shade k = ceil(8*coverage), grey = round(255*(1-k/9)); overlaps keep
 * the darker value), then 10 opaque rectangles of 8-64 px sides in colours
 * from a fixed 16-entry palette.
 * ================================================================== */

static const uint32_t PALETTE16[16] = {
    0xE6194B, 0x3CB44B, 0xFFE119, 0x4363D8, 0xF58231, 0x911EB4, 0x46F0F0, 0xF032E6,
    0xBCF60C, 0xFABEBE, 0x008080, 0xE6BEFF, 0x9A6324, 0xFFFAC8, 0x800000, 0xAAFFC3};

int synth_lines(uint32_t *out, int64_t H, int64_t W, uint64_t seed, int nlines, int nrects)
{
    if (!out || H < 0 || W < 0 || nlines < 0 || nrects < 0) return -1;
    const int64_t n = H * W;
    for (int64_t i = 0; i < n; ++i) out[i] = 0xFFFFFF;
    rng_t r = {seed, 1, 0};
    for (int s = 0; s < nlines; ++s) {
        const double ax = draw(&r) * W, ay = draw(&r) * H;
        const double bx = draw(&r) * W, by = draw(&r) * H;
        const double w = (double)draw_int(&r, 1, 4);
        const double R = w * 0.5 + 0.5;
        const int64_t x0 = (int64_t)floor(fmin(ax, bx) - R) - 1, x1 = (int64_t)ceil(fmax(ax, bx) + R) + 1;
        const int64_t y0 = (int64_t)floor(fmin(ay, by) - R) - 1, y1 = (int64_t)ceil(fmax(ay, by) + R) + 1;
        for (int64_t y = y0 < 0 ? 0 : y0; y <= y1 && y < H; ++y)
            for (int64_t x = x0 < 0 ? 0 : x0; x <= x1 && x < W; ++x) {
                const double cov = coverage(w, seg_dist(x + 0.5, y + 0.5, ax, ay, bx, by));
                if (cov <= 0.0) continue;
                uint32_t c;
                if (cov >= 1.0) {
                    c = 0x000000;
                } else {
                    const int k = (int)ceil(8.0 * cov);
                    const int g = (int)floor(255.0 * (1.0 - k / 9.0) + 0.5);
                    c = rgb(g, g, g);
                }
                /* keep the darker of the two greys (all values here are grey) */
                if ((c & 0xFF) < (out[y * W + x] & 0xFF) || out[y * W + x] == 0xFFFFFF)
                    out[y * W + x] = c;
            }
    }
    for (int k = 0; k < nrects; ++k) {
        const int64_t x0 = draw_int(&r, 0, W > 0 ? W - 1 : 0), y0 = draw_int(&r, 0, H > 0 ? H - 1 : 0);
        const int64_t w = draw_int(&r, 8, 64), h = draw_int(&r, 8, 64);
        const uint32_t c = PALETTE16[draw_int(&r, 0, 15)];
        for (int64_t y = y0; y < y0 + h && y < H; ++y)
            for (int64_t x = x0; x < x0 + w && x < W; ++x) out[y * W + x] = c;
    }
    return 0;
}

/* ==================================================================
 * Config 2: batch of binary noise.  Image b is 1 where a uniform draw is
 * below p_b, with p_b evenly spaced from p_lo to p_hi over the batch.
 * ================================================================== */

int synth_bernoulli(uint8_t *out, int64_t B, int64_t H, int64_t W, uint64_t seed,
                    double p_lo, double p_hi)
{
    if (!out || B < 0 || H < 0 || W < 0) return -1;
    const int64_t n = H * W;
    for (int64_t b = 0; b < B; ++b) {
        const double p = B > 1 ? p_lo + (p_hi - p_lo) * (double)b / (double)(B - 1) : p_lo;
        uint8_t *o = out + b * n;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            o[i] = rng_unif(seed, 100 + (uint64_t)b, (uint64_t)i) < p ? 1 : 0;
    }
    return 0;
}

/* ==================================================================
 * Config 3: two interleaved square spirals.  Arm A (offset 0) and arm B
 * (offset 2) are 1-px paths; loop j of an arm with offset o draws, with
 * t = l = o+4j, b = H-1-o-4j, r = W-1-o-4j: the top row t from column o
 * (j = 0) or l-4 (j > 0) to r, the right column r (rows t..b), the bottom
 * row b (columns l..r) and the left column l (rows t+4..b).  Each arm is one
 * long winding region.  Every other pixel is background colour C with
 * probability 1/2, else one of two fringe shades of A or of B (1/8 each).
 * ================================================================== */

#define SPIRAL_A 0xC81E1Eu
#define SPIRAL_B 0x1E1EC8u
#define SPIRAL_C 0xF0F0F0u
static const uint32_t SPIRAL_FRINGE[4] = {0xE08C8C, 0xF0C8C8, 0x8C8CE0, 0xC8C8F0};

static void spiral_arm(uint32_t *out, int64_t H, int64_t W, int64_t o, uint32_t colour)
{
    for (int64_t j = 0;; ++j) {
        const int64_t t = o + 4 * j, l = o + 4 * j;
        const int64_t b = H - 1 - o - 4 * j, r = W - 1 - o - 4 * j;
        const int64_t start = j == 0 ? o : l - 4;
        if (r - start < 1 || b - t < 1) break;
        for (int64_t x = start; x <= r; ++x) out[t * W + x] = colour;        /* top    */
        for (int64_t y = t; y <= b; ++y) out[y * W + r] = colour;            /* right  */
        for (int64_t x = l; x <= r; ++x) out[b * W + x] = colour;            /* bottom */
        if (b >= t + 4)
            for (int64_t y = t + 4; y <= b; ++y) out[y * W + l] = colour;    /* left   */
    }
}

int synth_spiral(uint32_t *out, int64_t H, int64_t W, uint64_t seed)
{
    if (!out || H < 0 || W < 0) return -1;
    const int64_t n = H * W;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const uint64_t h = rng_u64(seed, 200, (uint64_t)i);
        const unsigned k = (unsigned)(h >> 61);        /* 3 bits: 8 equal parts */
        out[i] = k < 4 ? SPIRAL_C : SPIRAL_FRINGE[(k - 4) & 3];
    }
    spiral_arm(out, H, W, 0, SPIRAL_A);
    spiral_arm(out, H, W, 2, SPIRAL_B);
    return 0;
}

/* ==================================================================
 * Config 4: tissue-scan-like binary image.  Uniform white noise (float32),
 * separable Gaussian blur (sigma, radius = ceil(4*sigma), taps applied in a
 * fixed order, mirror boundary d c b a | a b c d), thresholded at the value of
 * rank floor(q*N) in ascending order: output 1 where the blurred value is
 * above it (about 1-q of the pixels), 0 elsewhere.
 * ================================================================== */

static inline int64_t mirror(int64_t i, int64_t n)
{
    while (i < 0 || i >= n) {
        if (i < 0) i = -i - 1;
        if (i >= n) i = 2 * n - i - 1;
    }
    return i;
}

/* exact k-th smallest of non-negative floats by two 16-bit histogram passes
 * over their bit patterns (which order like the values) */
static float kth_smallest_nonneg(const float *v, int64_t n, int64_t k)
{
    uint64_t *hist = (uint64_t *)calloc(65536, sizeof(uint64_t));
    if (!hist) return NAN;
    const uint32_t *u = (const uint32_t *)v;
#pragma omp parallel
    {
        uint64_t *loc = (uint64_t *)calloc(65536, sizeof(uint64_t));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i) loc[u[i] >> 16]++;
#pragma omp critical
        for (int j = 0; j < 65536; ++j) hist[j] += loc[j];
        free(loc);
    }
    int64_t acc = 0;
    uint32_t hi = 0;
    for (uint32_t j = 0; j < 65536; ++j) {
        if (acc + (int64_t)hist[j] > k) { hi = j; break; }
        acc += (int64_t)hist[j];
    }
    const int64_t k2 = k - acc;
    memset(hist, 0, 65536 * sizeof(uint64_t));
#pragma omp parallel
    {
        uint64_t *loc = (uint64_t *)calloc(65536, sizeof(uint64_t));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            if ((u[i] >> 16) == hi) loc[u[i] & 0xFFFF]++;
#pragma omp critical
        for (int j = 0; j < 65536; ++j) hist[j] += loc[j];
        free(loc);
    }
    acc = 0;
    uint32_t lo = 0;
    for (uint32_t j = 0; j < 65536; ++j) {
        if (acc + (int64_t)hist[j] > k2) { lo = j; break; }
        acc += (int64_t)hist[j];
    }
    free(hist);
    const uint32_t bits = (hi << 16) | lo;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

int synth_tissue(uint8_t *out, int64_t H, int64_t W, uint64_t seed, double sigma, double q)
{
    if (!out || H < 0 || W < 0 || sigma <= 0 || q < 0 || q >= 1) return -1;
    const int64_t n = H * W;
    if (n == 0) return 0;
    const int R = (int)ceil(4.0 * sigma);
    float *taps = (float *)malloc((size_t)(2 * R + 1) * sizeof(float));
    float *a = (float *)malloc((size_t)n * sizeof(float));
    float *b = (float *)malloc((size_t)n * sizeof(float));
    if (!taps || !a || !b) { free(taps); free(a); free(b); return -2; }
    double tsum = 0;
    for (int k = -R; k <= R; ++k) tsum += exp(-0.5 * (k * k) / (sigma * sigma));
    for (int k = -R; k <= R; ++k) taps[k + R] = (float)(exp(-0.5 * (k * k) / (sigma * sigma)) / tsum);

#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        a[i] = (float)(rng_u64(seed, 300, (uint64_t)i) >> 40) * (1.0f / 16777216.0f);

    /* horizontal pass a -> b */
#pragma omp parallel for schedule(static)
    for (int64_t y = 0; y < H; ++y) {
        const float *row = a + y * W;
        float *o = b + y * W;
        for (int64_t x = 0; x < W; ++x) {
            float s = 0.0f;
            if (x >= R && x + R < W) {
                for (int k = 0; k <= 2 * R; ++k) s += taps[k] * row[x - R + k];
            } else {
                for (int k = 0; k <= 2 * R; ++k) s += taps[k] * row[mirror(x - R + k, W)];
            }
            o[x] = s;
        }
    }
    /* vertical pass b -> a, in column blocks for locality */
    const int64_t CB = 256;
#pragma omp parallel for schedule(static)
    for (int64_t xb = 0; xb < W; xb += CB) {
        const int64_t xe = xb + CB < W ? xb + CB : W;
        for (int64_t y = 0; y < H; ++y) {
            float *o = a + y * W;
            for (int64_t x = xb; x < xe; ++x) o[x] = 0.0f;
            for (int k = 0; k <= 2 * R; ++k) {
                const float t = taps[k];
                const float *src = b + mirror(y - R + k, H) * W;
                for (int64_t x = xb; x < xe; ++x) o[x] += t * src[x];
            }
        }
    }
    const float thr = kth_smallest_nonneg(a, n, (int64_t)floor(q * (double)n));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = a[i] > thr ? 1 : 0;
    free(taps); free(a); free(b);
    return 0;
}

/* ==================================================================
 * Config 5: synthetic construction sheet.  White paper; primitives in this
 * order, composited "over" with 8-bit rounding per channel:
 *   walls     2-8 px wide, 40% at 0 deg, 40% at 90 deg, 10% at 45 deg, 10% at a
 *             random angle, 500-12000 px long;
 *   hatching  fields of 45-degree lines 1-2 px wide, spacing 16-32 px, clipped
 *             to rectangles with 600-3000 px sides;
 *   bubbles   circles of radius 40-120 px, stroke 2-4 px;
 *   glyphs    20-40 px cells of 3-6 short strokes each, set in rows of text.
 * Strokes are black; each primitive is one of 12 hues with probability 1%.
 * Counts are given per 806.4 Mpx and scale with the sheet's area.
 * ================================================================== */

typedef struct {
    float ax, ay, bx, by;  /* segment, or centre (ax, ay) and radius bx for rings */
    float w;               /* stroke width */
    float cx0, cy0, cx1, cy1; /* clip rectangle (inclusive-exclusive), or none */
    uint32_t colour;
    int ring;
} prim_t;

static const uint32_t HUES12[12] = {
    0xD62728, 0x1F77B4, 0x2CA02C, 0xFF7F0E, 0x9467BD, 0x8C564B,
    0xE377C2, 0x17BECF, 0xBCBD22, 0x7F7F7F, 0x393B79, 0x637939};

typedef struct { prim_t *p; int64_t n, cap; } plist_t;

static int push(plist_t *l, prim_t p)
{
    if (l->n == l->cap) {
        int64_t nc = l->cap ? l->cap * 2 : 4096;
        prim_t *q = (prim_t *)realloc(l->p, (size_t)nc * sizeof(prim_t));
        if (!q) return -1;
        l->p = q; l->cap = nc;
    }
    l->p[l->n++] = p;
    return 0;
}

static void prim_bbox(const prim_t *p, double *x0, double *y0, double *x1, double *y1)
{
    const double R = p->w * 0.5 + 1.0;
    if (p->ring) {
        *x0 = p->ax - p->bx - R; *x1 = p->ax + p->bx + R;
        *y0 = p->ay - p->bx - R; *y1 = p->ay + p->bx + R;
    } else {
        *x0 = fmin(p->ax, p->bx) - R; *x1 = fmax(p->ax, p->bx) + R;
        *y0 = fmin(p->ay, p->by) - R; *y1 = fmax(p->ay, p->by) + R;
    }
    if (p->cx1 > p->cx0) {
        *x0 = fmax(*x0, p->cx0); *x1 = fmin(*x1, p->cx1);
        *y0 = fmax(*y0, p->cy0); *y1 = fmin(*y1, p->cy1);
    }
}

static uint32_t stroke_colour(rng_t *r)
{
    const double u = draw(r);
    const int64_t h = draw_int(r, 0, 11);
    return u < 0.01 ? HUES12[h] : 0x000000;
}

static void raster_rows(uint32_t *img, int64_t W, int64_t ylo, int64_t yhi, const prim_t *p)
{
    double bx0, by0, bx1, by1;
    prim_bbox(p, &bx0, &by0, &bx1, &by1);
    int64_t y0 = (int64_t)floor(by0), y1 = (int64_t)ceil(by1);
    if (y0 < ylo) y0 = ylo;
    if (y1 >= yhi) y1 = yhi - 1;
    const double R = p->w * 0.5 + 0.5;
    for (int64_t y = y0; y <= y1; ++y) {
        const double py = y + 0.5;
        double xa, xb;
        if (p->ring) {
            xa = p->ax - p->bx - R - 1; xb = p->ax + p->bx + R + 1;
        } else {
            /* x-extent of the part of the segment within R+1 rows of py */
            const double dy = p->by - p->ay;
            double t0 = 0, t1 = 1;
            if (fabs(dy) > 1e-9) {
                double ta = (py - R - 1 - p->ay) / dy, tb = (py + R + 1 - p->ay) / dy;
                if (ta > tb) { double s = ta; ta = tb; tb = s; }
                t0 = fmax(0, ta); t1 = fmin(1, tb);
                if (t0 > t1) continue;
            }
            const double xs = p->ax + t0 * (p->bx - p->ax), xe = p->ax + t1 * (p->bx - p->ax);
            xa = fmin(xs, xe) - R - 1; xb = fmax(xs, xe) + R + 1;
        }
        xa = fmax(xa, bx0); xb = fmin(xb, bx1);
        int64_t x0 = (int64_t)floor(xa), x1 = (int64_t)ceil(xb);
        if (x0 < 0) x0 = 0;
        if (x1 >= W) x1 = W - 1;
        uint32_t *row = img + y * W;
        for (int64_t x = x0; x <= x1; ++x) {
            const double px = x + 0.5;
            if (p->cx1 > p->cx0 && (px < p->cx0 || px >= p->cx1 || py < p->cy0 || py >= p->cy1))
                continue;
            double d;
            if (p->ring) {
                const double dx = px - p->ax, dyy = py - p->ay;
                d = fabs(sqrt(dx * dx + dyy * dyy) - p->bx);
            } else {
                d = seg_dist(px, py, p->ax, p->ay, p->bx, p->by);
            }
            const double cov = coverage(p->w, d);
            if (cov <= 0.0) continue;
            row[x] = cov >= 1.0 ? p->colour : over(row[x], p->colour, cov);
        }
    }
}

int synth_sheet(uint32_t *out, int64_t H, int64_t W, uint64_t seed, double density)
{
    if (!out || H < 0 || W < 0 || density < 0) return -1;
    const int64_t n = H * W;
    if (n == 0) return 0;
    const double area = (double)n / (24000.0 * 33600.0);
    const double scale = sqrt(area);         /* lengths scale with the side */
    plist_t L = {0};
    rng_t r = {seed, 500, 0};
    int err = 0;

    const int nwalls = (int)floor(400 * area * density + 0.5);
    for (int k = 0; k < nwalls && !err; ++k) {
        prim_t p = {0};
        const double u = draw(&r);
        const double ang = u < 0.4 ? 0.0 : u < 0.8 ? M_PI / 2 : u < 0.9 ? M_PI / 4 : draw(&r) * M_PI;
        const double len = (500 + draw(&r) * 11500) * scale;
        p.ax = (float)(draw(&r) * W); p.ay = (float)(draw(&r) * H);
        p.bx = (float)(p.ax + len * cos(ang)); p.by = (float)(p.ay + len * sin(ang));
        p.w = (float)draw_int(&r, 2, 8);
        p.colour = stroke_colour(&r);
        err |= push(&L, p);
    }
    const int nhatch = (int)floor(80 * area * density + 0.5);
    for (int k = 0; k < nhatch && !err; ++k) {
        const double fw = (600 + draw(&r) * 2400) * scale, fh = (600 + draw(&r) * 2400) * scale;
        const double fx = draw(&r) * W, fy = draw(&r) * H;
        const double sp = (double)draw_int(&r, 16, 32);
        const double w = (double)draw_int(&r, 1, 2);
        const uint32_t c = stroke_colour(&r);
        /* lines x - y = const, spaced sp apart horizontally, spanning the field */
        for (double off = -fh; off < fw && !err; off += sp) {
            prim_t p = {0};
            p.ax = (float)(fx + off); p.ay = (float)fy;
            p.bx = (float)(fx + off + fh); p.by = (float)(fy + fh);
            p.w = (float)w; p.colour = c;
            p.cx0 = (float)fx; p.cy0 = (float)fy; p.cx1 = (float)(fx + fw); p.cy1 = (float)(fy + fh);
            err |= push(&L, p);
        }
    }
    const int ncirc = (int)floor(300 * area * density + 0.5);
    for (int k = 0; k < ncirc && !err; ++k) {
        prim_t p = {0};
        p.ring = 1;
        p.ax = (float)(draw(&r) * W); p.ay = (float)(draw(&r) * H);
        p.bx = (float)(40 + draw(&r) * 80);
        p.w = (float)draw_int(&r, 2, 4);
        p.colour = stroke_colour(&r);
        err |= push(&L, p);
    }
    /* glyphs: text blocks of rows of cells until the glyph budget is used */
    const int64_t nglyph = (int64_t)floor(200000 * area * density + 0.5);
    int64_t placed = 0;
    while (placed < nglyph && !err) {
        const double size = 20 + draw(&r) * 20;
        const int64_t rows = draw_int(&r, 1, 6), cols = draw_int(&r, 4, 40);
        const double bx = draw(&r) * W, by = draw(&r) * H;
        const uint32_t c = stroke_colour(&r);
        for (int64_t rr = 0; rr < rows && placed < nglyph && !err; ++rr)
            for (int64_t cc = 0; cc < cols && placed < nglyph && !err; ++cc) {
                const double gx = bx + cc * size * 0.85, gy = by + rr * size * 1.6;
                const int64_t ns = draw_int(&r, 3, 6);
                const double sw = (double)draw_int(&r, 2, 3);
                for (int64_t s = 0; s < ns && !err; ++s) {
                    prim_t p = {0};
                    p.ax = (float)(gx + draw(&r) * size * 0.7); p.ay = (float)(gy + draw(&r) * size);
                    p.bx = (float)(gx + draw(&r) * size * 0.7); p.by = (float)(gy + draw(&r) * size);
                    p.w = (float)sw; p.colour = c;
                    err |= push(&L, p);
                }
                ++placed;
            }
    }
    if (err) { free(L.p); return -2; }

    /* bin primitives by bands of rows, keeping primitive order within a band */
    const int64_t BAND = 64;
    const int64_t nb = (H + BAND - 1) / BAND;
    int64_t *cnt = (int64_t *)calloc((size_t)nb + 1, sizeof(int64_t));
    if (!cnt) { free(L.p); return -2; }
    for (int64_t i = 0; i < L.n; ++i) {
        double x0, y0, x1, y1;
        prim_bbox(&L.p[i], &x0, &y0, &x1, &y1);
        int64_t b0 = (int64_t)floor(y0) / BAND, b1 = (int64_t)ceil(y1) / BAND;
        if (y1 < 0 || y0 >= H || x1 < 0 || x0 >= W) continue;
        if (b0 < 0) b0 = 0;
        if (b1 >= nb) b1 = nb - 1;
        for (int64_t b = b0; b <= b1; ++b) cnt[b + 1]++;
    }
    for (int64_t b = 0; b < nb; ++b) cnt[b + 1] += cnt[b];
    int64_t *idx = (int64_t *)malloc((size_t)(cnt[nb] > 0 ? cnt[nb] : 1) * sizeof(int64_t));
    int64_t *fill = (int64_t *)calloc((size_t)nb, sizeof(int64_t));
    if (!idx || !fill) { free(L.p); free(cnt); free(idx); free(fill); return -2; }
    for (int64_t i = 0; i < L.n; ++i) {
        double x0, y0, x1, y1;
        prim_bbox(&L.p[i], &x0, &y0, &x1, &y1);
        if (y1 < 0 || y0 >= H || x1 < 0 || x0 >= W) continue;
        int64_t b0 = (int64_t)floor(y0) / BAND, b1 = (int64_t)ceil(y1) / BAND;
        if (b0 < 0) b0 = 0;
        if (b1 >= nb) b1 = nb - 1;
        for (int64_t b = b0; b <= b1; ++b) idx[cnt[b] + fill[b]++] = i;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t ylo = b * BAND, yhi = ylo + BAND < H ? ylo + BAND : H;
        for (int64_t i = ylo * W; i < yhi * W; ++i) out[i] = 0xFFFFFF;
        for (int64_t j = cnt[b]; j < cnt[b + 1]; ++j)
            raster_rows(out, W, ylo, yhi, &L.p[idx[j]]);
    }
    free(L.p); free(cnt); free(idx); free(fill);
    return 0;
}
