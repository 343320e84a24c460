/*
 * ccl_oracle.c -- plain, sequential CPU oracle for connected-component labelling.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes (per image of a batch, each image on its own):
 *   leader(p) = the smallest reading-order index q (q = row*W + col inside the
 *               image) such that p and q are joined by a chain of neighbours of
 *               identical colour value.  Neighbours are the 8 (or 4) pixels
 *               around p inside the H x W rectangle; rows do not wrap and images
 *               never touch each other.
 *   label(p)  = 1 + the number of leaders r with r < leader(p).
 *   count     = the number of leaders.
 *
 * Sources (titles of the pages the method is taken from):
 *   "Accountable AI starts at the pixel" (every-colour blog), ch.01-02: a region
 *     is touching pixels of exactly one colour, corners count (8 neighbours).
 *   same page, ch.04 "Point at a leader": one parent per pixel; joining two
 *     groups re-points the leader with the larger position at the smaller, so a
 *     region's leader is its first pixel in reading order; the pixel scan looks
 *     at up-left, up, up-right, then left.
 *   same page, ch.05 "Start, Connect, Collapse, Number": the four stages.
 *   same page, ch.08 idea 3 "Shorten arrows while walking": path halving; it
 *     only moves arrows closer to the leader and never changes which pixel is
 *     the leader, so it is used here for speed only.
 *   same page, ch.08 idea 5: a leader's number is 1 + the leaders before it.
 *   same page, ch.08 idea 4 "Ignore the paper": a caller may name one colour
 *     to ignore; its pixels get label 0 in Start and take part in nothing
 *     after (no joins, not counted, not numbered).  Leader images mark them
 *     with -1 (label 0 in the "leader + 1" form that the TorchCC page uses,
 *     where 0 is kept for background); numbers give them 0.
 *   "About Connected Components Labeling on GPU" (TorchCC blog), "The basic
 *     approach: Union-Find" and "Application in CCL": Find / Union / Compress,
 *     the raster two-pass scan over already-visited neighbours, 4- and
 *     8-connectivity; its introduction names the uses of a labelling, such as
 *     a region's bounding box.
 *   "Accountable AI starts at the pixel", ch.11 "How we know it is right":
 *     images of more than 2^31 pixels were not run; their leaders need
 *     64-bit indices (oracle_label64, oracle_number64).  The union-find below
 *     works on 64-bit parents for every entry point; the 32-bit ones narrow
 *     the result.
 *   The tissue-scan segmentation article, sections 1.1 and 2.3: each region's
 *     area and position are summed over its pixels once it is numbered.
 *     oracle_region_stats computes, per region, its area, bounding box and the
 *     sums of its pixels' row and column indices (the position is sum / area).
 *
 * The BFS labeller below is an independent second algorithm (graph traversal,
 * the alternative that page names in "The basic approach") used to pin the
 * union-find oracle; it is not used by the union-find code.
 *
 * dtype: 1 = one byte per pixel, 4 = one 32-bit word per pixel, 3 = three
 * bytes per pixel (an RGB picture as it is stored, "Accountable AI starts at
 * the pixel", ch.08 "Tried and dropped" and ch.09: the labeller reads the RGB
 * picture without packing it); colours are compared as whole stored values,
 * all three bytes of an RGB pixel.  An RGB pixel's colour value, as an ignored
 * colour is named, is b0 | b1 << 8 | b2 << 16 with b0 its first byte.
 *
 * Building with -DORACLE_MUTANT=k plants a deliberate mistake (k = 1..14) so the
 * pin tests can show that they catch it.  The default build plants nothing.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

enum { ORACLE_OK = 0, ORACLE_ERR_ARG = -1, ORACLE_ERR_NOMEM = -2 };

/* Colour of pixel i of one image (whole stored value). */
static inline uint32_t colour_at(const void *img, int dtype, int64_t i)
{
    if (dtype == 1)
        return ((const uint8_t *)img)[i];
    if (dtype == 3) {
        const uint8_t *p = (const uint8_t *)img + 3 * i;
#if ORACLE_MUTANT == 11
        return (uint32_t)p[0] | ((uint32_t)p[1] << 8);   /* mutant: third byte not compared */
#else
        return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
#endif
    }
#if ORACLE_MUTANT == 7
    return ((const uint32_t *)img)[i] & 0xFFu; /* mutant: low byte only */
#else
    return ((const uint32_t *)img)[i];
#endif
}

/* Find: walk parent arrows to the pixel that points at itself, halving the
 * path on the way (each visited pixel is pointed at its grandparent). */
static int64_t find_leader(int64_t *P, int64_t x)
{
    while (P[x] != x) {
        P[x] = P[P[x]];
        x = P[x];
    }
    return x;
}

/* Union: find both leaders and re-point the larger at the smaller. */
static void join(int64_t *P, int64_t p, int64_t q)
{
    int64_t a = find_leader(P, p);
    int64_t b = find_leader(P, q);
    if (a == b)
        return;
#if ORACLE_MUTANT == 3
    if (a < b) P[q] = a; else P[p] = b;   /* mutant: re-point the node, not its leader */
#elif ORACLE_MUTANT == 4
    if (a < b) P[a] = b; else P[b] = a;   /* mutant: larger leader wins */
#else
    if (a < b) P[b] = a; else P[a] = b;
#endif
}

/* Stages Start and Connect for one image: P[i] = i, then the reading-order
 * scan joining each pixel with its earlier same-colour neighbours in the
 * order up-left, up, up-right, left (4-connectivity: up, left).  With
 * ign != 0, pixels of colour `ignv` are marked -1 in Start and skipped by
 * Connect, as the pixel itself and as a neighbour. */
static void start_connect(const void *img, int dtype, int64_t H, int64_t W,
                          int conn, int ign, uint32_t ignv, int64_t *P)
{
    const int64_t n = H * W;
    for (int64_t i = 0; i < n; ++i)                          /* Start */
#if ORACLE_MUTANT == 10
        P[i] = i;                       /* mutant: the ignored colour is labelled */
#else
        P[i] = (ign && colour_at(img, dtype, i) == ignv) ? -1 : i;
#endif

    for (int64_t r = 0; r < H; ++r) {
        for (int64_t c = 0; c < W; ++c) {
            const int64_t p = r * W + c;
#if ORACLE_MUTANT != 10
            if (P[p] < 0) continue;                          /* ignored: no joins */
#endif
            const uint32_t v = colour_at(img, dtype, p);
            /* candidate earlier neighbours as (row offset, col offset) */
            int64_t dr[4], dc[4];
            int k = 0;
            if (conn == 8) {
#if ORACLE_MUTANT != 6
                dr[k] = -1; dc[k] = -1; ++k;                 /* up-left  */
#endif
                dr[k] = -1; dc[k] = 0; ++k;                  /* up       */
#if ORACLE_MUTANT != 1
                dr[k] = -1; dc[k] = +1; ++k;                 /* up-right */
#endif
                dr[k] = 0; dc[k] = -1; ++k;                  /* left     */
            } else {
                dr[k] = -1; dc[k] = 0; ++k;                  /* up       */
#if ORACLE_MUTANT == 8
                dr[k] = -1; dc[k] = +1; ++k;   /* mutant: a diagonal in 4-connectivity */
#endif
                dr[k] = 0; dc[k] = -1; ++k;                  /* left     */
            }
            for (int j = 0; j < k; ++j) {
                const int64_t rr = r + dr[j], cc = c + dc[j];
#if ORACLE_MUTANT == 2
                /* mutant: neighbours taken in the flat index, so row ends wrap */
                const int64_t q = p + dr[j] * W + dc[j];
                if (q < 0 || q >= n) continue;
#else
                if (rr < 0 || cc < 0 || cc >= W) continue;   /* inside H x W only */
                const int64_t q = rr * W + cc;
#endif
                if (P[q] >= 0 && colour_at(img, dtype, q) == v)
                    join(P, p, q);
            }
        }
    }
}

/* Stage Collapse: every pixel points straight at its leader.  P[i] <= i holds
 * for every pixel, so an ascending pass sees each parent's leader first.
 * Ignored pixels (-1) stay -1. */
static void collapse(int64_t *P, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (P[i] >= 0)
            P[i] = (P[i] == i) ? i : P[P[i]];
}

static int check_args(const void *img, int dtype, int64_t B, int64_t H,
                      int64_t W, int conn, const void *out, int64_t max_pixels)
{
    if (B < 0 || H < 0 || W < 0) return ORACLE_ERR_ARG;
    if (dtype != 1 && dtype != 3 && dtype != 4) return ORACLE_ERR_ARG;
    if (conn != 4 && conn != 8) return ORACLE_ERR_ARG;
    if (W > 0 && H > max_pixels / W) return ORACLE_ERR_ARG;
    if (B * H * W > 0 && (img == NULL || out == NULL)) return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/* Per-image scratch of 64-bit parents for the entry points with 32-bit
 * results; the arithmetic is the same for both widths. */
static int64_t *scratch64(int64_t n)
{
    return (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
}

static void narrow(const int64_t *a, int64_t n, int32_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (int32_t)a[i];
}

/* Parent array after the Connect stage (no Collapse) -- exposed so tests can
 * check the stage semantics against the worked examples on the pages. */
int oracle_connect(const void *img, int dtype, int64_t B, int64_t H, int64_t W,
                   int conn, int32_t *parents)
{
    int rc = check_args(img, dtype, B, H, W, conn, parents, 2147483647LL);
    if (rc) return rc;
    const int64_t n = H * W;
    int64_t *P = scratch64(n);
    if (!P) return ORACLE_ERR_NOMEM;
    for (int64_t b = 0; b < B; ++b) {
        start_connect((const char *)img + b * n * dtype, dtype, H, W, conn, 0, 0u, P);
        narrow(P, n, parents + b * n);
    }
    free(P);
    return ORACLE_OK;
}

/* Start, Connect and Collapse of each image into 64-bit leaders (leaders64),
 * or through a scratch array into 32-bit ones (leaders32). */
static int label_images(const void *img, int dtype, int64_t B, int64_t H, int64_t W,
                        int conn, int ign, uint32_t ignv, int32_t *leaders32,
                        int64_t *leaders64)
{
    const int64_t n = H * W;
    int64_t *tmp = NULL;
    if (leaders32 && !(tmp = scratch64(n))) return ORACLE_ERR_NOMEM;
    for (int64_t b = 0; b < B; ++b) {
        int64_t *P = leaders32 ? tmp : leaders64 + b * n;
        start_connect((const char *)img + b * n * dtype, dtype, H, W, conn, ign, ignv, P);
        collapse(P, n);
        if (leaders32) narrow(P, n, leaders32 + b * n);
    }
    free(tmp);
    return ORACLE_OK;
}

/* Leaders: Start, Connect, Collapse, per image.  Indices are per image. */
int oracle_label(const void *img, int dtype, int64_t B, int64_t H, int64_t W,
                 int conn, int32_t *leaders)
{
    int rc = check_args(img, dtype, B, H, W, conn, leaders, 2147483647LL);
    if (rc) return rc;
    return label_images(img, dtype, B, H, W, conn, 0, 0u, leaders, NULL);
}

/* Leaders with one colour ignored ("Accountable AI starts at the pixel",
 * ch.08 idea 4): pixels of colour `ignore` (compared as the whole stored
 * value; a CCL_U8-style byte image has no colour above 255, so such a value
 * ignores nothing) get -1 and join nothing; every other pixel gets its
 * region's leader. */
int oracle_label_ignore(const void *img, int dtype, int64_t B, int64_t H, int64_t W,
                        int conn, uint32_t ignore, int32_t *leaders)
{
    int rc = check_args(img, dtype, B, H, W, conn, leaders, 2147483647LL);
    if (rc) return rc;
    return label_images(img, dtype, B, H, W, conn, 1, ignore, leaders, NULL);
}

/* 64-bit leaders, for images of any size: a picture of more than 2^31 pixels
 * has reading-order indices beyond int32 ("Accountable AI starts at the
 * pixel", ch.11 "How we know it is right", lists such images as not yet run;
 * ch.10 shows what a size wrapped to 32 bits does).  ign != 0 ignores colour
 * `ignore`, as oracle_label_ignore does. */
int oracle_label64(const void *img, int dtype, int64_t B, int64_t H, int64_t W,
                   int conn, int ign, uint32_t ignore, int64_t *leaders)
{
    int rc = check_args(img, dtype, B, H, W, conn, leaders, INT64_MAX / 8);
    if (rc) return rc;
#if ORACLE_MUTANT == 14
    ign = 0;                                  /* mutant: the ignored colour dropped */
#endif
    return label_images(img, dtype, B, H, W, conn, ign != 0, ignore, NULL, leaders);
}

/* Stage Number for one image: leaders become 1, 2, 3, ... in reading order
 * and every pixel takes its leader's number.  Requires a valid leader image
 * (leader[p] <= p, leader[leader[p]] == leader[p]): a leader comes no later
 * than its pixels, so its number is already written when a later pixel copies
 * it.  A pixel whose leader is negative (an ignored pixel) gets 0 and is not
 * counted.  Returns the count. */
static int64_t number_image(const int64_t *L, int64_t n, int64_t *out)
{
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (L[i] < 0) {
#if ORACLE_MUTANT == 9
            k += 1;                               /* mutant: ignored pixels counted */
#endif
            out[i] = 0;
        } else if (L[i] == i) {
#if ORACLE_MUTANT == 5
            out[i] = k;                           /* mutant: numbers start at 0 */
            k += 1;
#else
            k += 1;
            out[i] = k;
#endif
        } else {
            out[i] = out[L[i]];
        }
    }
    return k;
}

/* Number, 32-bit leaders and labels (through 64-bit scratch); counts may be
 * NULL. */
int oracle_number(const int32_t *leaders, int64_t B, int64_t H, int64_t W,
                  int32_t *labels, int32_t *counts)
{
    if (B < 0 || H < 0 || W < 0) return ORACLE_ERR_ARG;
    const int64_t n = H * W;
    if (B * n > 0 && (leaders == NULL || labels == NULL)) return ORACLE_ERR_ARG;
    int64_t *L = scratch64(n), *out = scratch64(n);
    if (!L || !out) {
        free(L);
        free(out);
        return ORACLE_ERR_NOMEM;
    }
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < n; ++i) L[i] = leaders[b * n + i];
        const int64_t k = number_image(L, n, out);
        narrow(out, n, labels + b * n);
        if (counts) counts[b] = (int32_t)k;
    }
    free(L);
    free(out);
    return ORACLE_OK;
}

/* Number, 64-bit leaders, labels and counts; counts may be NULL. */
int oracle_number64(const int64_t *leaders, int64_t B, int64_t H, int64_t W,
                    int64_t *labels, int64_t *counts)
{
    if (B < 0 || H < 0 || W < 0) return ORACLE_ERR_ARG;
    const int64_t n = H * W;
    if (B * n > 0 && (leaders == NULL || labels == NULL)) return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t k = number_image(leaders + b * n, n, labels + b * n);
        if (counts) counts[b] = k;
    }
    return ORACLE_OK;
}

/* Count: number of leaders (pixels with leader[p] == p) per image. */
int oracle_count(const int32_t *leaders, int64_t B, int64_t H, int64_t W,
                 int32_t *counts)
{
    if (B < 0 || H < 0 || W < 0 || counts == NULL) return ORACLE_ERR_ARG;
    const int64_t n = H * W;
    if (B * n > 0 && leaders == NULL) return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < B; ++b) {
        const int32_t *L = leaders + b * n;
        int32_t k = 0;
        for (int64_t i = 0; i < n; ++i)
            k += (L[i] == i);
        counts[b] = k;
    }
    return ORACLE_OK;
}

/* Independent second labeller: breadth-first flood fill.  Seeds are taken in
 * reading order, so each seed is the smallest index of its region (every
 * smaller pixel was reached from an earlier seed), and every pixel of the
 * region gets the seed's index.  Used only to pin the union-find above. */
int oracle_bfs_label(const void *img, int dtype, int64_t B, int64_t H, int64_t W,
                     int conn, int32_t *leaders)
{
    int rc = check_args(img, dtype, B, H, W, conn, leaders, 2147483647LL);
    if (rc) return rc;
    const int64_t n = H * W;
    int32_t *queue = (int32_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
    if (!queue) return ORACLE_ERR_NOMEM;
    static const int dr8[8] = {-1, -1, -1, 0, 0, 1, 1, 1};
    static const int dc8[8] = {-1, 0, 1, -1, 1, -1, 0, 1};
    static const int dr4[4] = {-1, 0, 0, 1};
    static const int dc4[4] = {0, -1, 1, 0};
    const int *dr = conn == 8 ? dr8 : dr4;
    const int *dc = conn == 8 ? dc8 : dc4;
    const int nn = conn;
    for (int64_t b = 0; b < B; ++b) {
        const void *im = (const char *)img + b * n * dtype;
        int32_t *L = leaders + b * n;
        for (int64_t i = 0; i < n; ++i) L[i] = -1;
        for (int64_t s = 0; s < n; ++s) {
            if (L[s] >= 0) continue;
            const uint32_t v = colour_at(im, dtype, s);
            int64_t head = 0, tail = 0;
            queue[tail++] = (int32_t)s;
            L[s] = (int32_t)s;
            while (head < tail) {
                const int64_t p = queue[head++];
                const int64_t r = p / W, c = p % W;
                for (int j = 0; j < nn; ++j) {
                    const int64_t rr = r + dr[j], cc = c + dc[j];
                    if (rr < 0 || rr >= H || cc < 0 || cc >= W) continue;
                    const int64_t q = rr * W + cc;
                    if (L[q] < 0 && colour_at(im, dtype, q) == v) {
                        L[q] = (int32_t)s;
                        queue[tail++] = (int32_t)q;
                    }
                }
            }
        }
    }
    free(queue);
    return ORACLE_OK;
}

/* Per-region statistics of a numbered label image (labels 1..counts[b] per
 * image b, 0 for pixels of no region).  Region k of image b is entry
 * i = off[b] + k - 1, off[b] = counts[0] + ... + counts[b-1]:
 *   area[i]          number of its pixels
 *   bbox[4i .. 4i+3] smallest row, smallest column, largest row, largest
 *                    column of its pixels
 *   sum_y[i], sum_x[i]  sums of its pixels' row and column indices
 * Entries of regions without pixels keep area 0, bbox (INT32_MAX, INT32_MAX,
 * -1, -1) and sums 0.  A label outside [0, counts[b]] is an error. */
int oracle_region_stats(const int32_t *labels, int64_t B, int64_t H, int64_t W,
                        const int32_t *counts, int32_t *area, int32_t *bbox,
                        int64_t *sum_y, int64_t *sum_x)
{
    if (B < 0 || H < 0 || W < 0 || counts == NULL) return ORACLE_ERR_ARG;
    int64_t total = 0;
    for (int64_t b = 0; b < B; ++b) {
        if (counts[b] < 0) return ORACLE_ERR_ARG;
        total += counts[b];
    }
    if (total > 0 && (area == NULL || bbox == NULL || sum_y == NULL || sum_x == NULL))
        return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < total; ++i) {
        area[i] = 0;
        bbox[4 * i] = bbox[4 * i + 1] = 2147483647;
        bbox[4 * i + 2] = bbox[4 * i + 3] = -1;
        sum_y[i] = sum_x[i] = 0;
    }
    const int64_t n = H * W;
    int64_t off = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int32_t *L = labels + b * n;
        for (int64_t r = 0; r < H; ++r) {
            for (int64_t c = 0; c < W; ++c) {
                const int32_t k = L[r * W + c];
                if (k == 0) continue;
                if (k < 0 || k > counts[b]) return ORACLE_ERR_ARG;
                const int64_t i = off + k - 1;
                area[i] += 1;
                if (r < bbox[4 * i]) bbox[4 * i] = (int32_t)r;
                if (c < bbox[4 * i + 1]) bbox[4 * i + 1] = (int32_t)c;
#if ORACLE_MUTANT == 12
                if (r >= bbox[4 * i + 2]) bbox[4 * i + 2] = (int32_t)r + 1;  /* mutant: exclusive bottom */
#else
                if (r > bbox[4 * i + 2]) bbox[4 * i + 2] = (int32_t)r;
#endif
                if (c > bbox[4 * i + 3]) bbox[4 * i + 3] = (int32_t)c;
                sum_y[i] += r;
#if ORACLE_MUTANT == 13
                sum_x[i] += r;                        /* mutant: row summed as column */
#else
                sum_x[i] += c;
#endif
            }
        }
        off += counts[b];
    }
    return ORACLE_OK;
}
