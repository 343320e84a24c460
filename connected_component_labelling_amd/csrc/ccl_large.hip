// ccl_large.hip -- labelling of images of any size, beyond 2^31 pixels, with
// 64-bit leaders and numbers.
//
// "Accountable AI starts at the pixel" lists images of more than 2^31 pixels
// as not run (ch.11 "How we know it is right"), and shows in ch.10 what a size
// wrapped to 32 bits does.  Here such an image is cut into bands of whole tile
// rows, each small enough for the 32-bit tile pipeline; the bands number
// their own regions, with no 32-bit array over the picture, and the regions
// that continue across a band seam are joined by (band, number):
//   1. every band goes through the whole tile pipeline in number mode (its
//      own numbers 1..n_b and count) and keeps its tile records; for leaders
//      each seam node's record also points at its root, whose key is the
//      region's band-local leader;
//   2. the band-local numbers of the rows either side of each seam are
//      written out (the final write of those tile rows), and for leaders
//      their band-local leaders too;
//   3. each seam region (band, number) gets one entry of a hash table; its
//      canonical node is its first seam pixel, equal-colour neighbours across
//      the seams are joined over canonical nodes keyed by (band, number),
//      which orders regions as their leaders do, so each set's root is its
//      region's leading part (a join points the larger key at the smaller, as
//      the tile pipeline does inside a band: same page, ch.04 "Point at a
//      leader");
//   4. every other part is merged: bit n of its band's mask; each band's
//      merged numbers are prefix-counted, the bands' own numbers give each
//      band's first number G_b and the picture's count (ch.08 idea 5 "Number
//      without a giant list"); each root's number is G_b + n - (merged numbers
//      below n), or its leader the band's first pixel plus its band-local
//      leader, and each merged number takes its root's, stored at its rank
//      among its band's merged numbers;
//   5. each band's final write maps its numbers through that (Map64) and
//      writes the 64-bit labels straight from its tile records: a merged
//      number's entry, else the band's own number or leader moved to the
//      picture's.
//
// The seams between bands are the same seams a band per GPU would have: this
// is the one-GPU form of labelling one picture across several GPUs.
#include "ccl.h"
#include "ccl_internal.h"

#include <limits.h>

namespace ccl {
namespace large {

constexpr int LB = 256;                // threads per workgroup
constexpr int SEAM_BUDGET = 1 << 20;   // bound on one union's find/link steps
constexpr int64_t AUTO_BAND_PX = int64_t(1) << 30;

// Geometry of one image cut into bands.
struct Bands {
    int64_t H, W, HW;
    int64_t hb;        // rows per band (a multiple of 64 when there are several)
    int64_t band_px;   // hb * W
    int64_t nb;        // bands
    int64_t nseam;     // seam pixels: (nb - 1) * 2W
};

// Node ids of seam pixels: seam s (between bands s and s+1) owns ids
// [s*2W, (s+1)*2W): s*2W + c is column c of band s's last row, s*2W + W + c
// column c of band s+1's first row.

__device__ __forceinline__ uint32_t seam_colour(const uint8_t *img, int dtype, int64_t i)
{
    if (dtype == CCL_U8) return img[i];
    if (dtype == CCL_U32) return ((const uint32_t *)img)[i];
    const uint8_t *p = img + 3 * i;
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
}

__device__ __forceinline__ int32_t ld_parent(const int32_t *P, int64_t x)
{
    return __hip_atomic_load(P + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ int32_t seam_find(int32_t *P, int32_t x, int &budget)
{
    while (budget-- > 0) {
        const int32_t p = ld_parent(P, x);
        if (p == x) return x;
        const int32_t gp = ld_parent(P, p);
        if (gp == p) return p;
        atomicCAS(&P[x], p, gp);  // path halving: x moves to an ancestor
        x = gp;
    }
    return x;
}

// Links always go from a root to a root of smaller key, so the sets stay
// trees and a set's root is the node of its smallest key.
__device__ void seam_unite(int32_t *P, const int64_t *K, int32_t a, int32_t b, uint32_t *err)
{
    int budget = SEAM_BUDGET;
    while (budget > 0) {
        a = seam_find(P, a, budget);
        b = seam_find(P, b, budget);
        if (budget <= 0) break;
        if (a == b) return;
        if (K[a] < K[b]) {
            const int32_t t = a;
            a = b;
            b = t;
        }
        if (atomicCAS(&P[a], a, b) == a) return;  // a was still a root: linked
        --budget;
    }
    atomicOr(err, ERR_LOOP);
}

// Step 3: joins across each seam: column c of band s+1's first row with the
// columns c-1, c, c+1 (8 neighbours) or c (4 neighbours) of band s's last row.
__global__ __launch_bounds__(LB) void seam_union_kernel(Bands g, const uint8_t *img, int dtype,
                                                        int conn, const int32_t *C, int32_t *P,
                                                        const int64_t *K, uint32_t *err)
{
    const int64_t i = (int64_t)blockIdx.x * LB + threadIdx.x;  // (seam, column)
    if (i >= (g.nb - 1) * g.W) return;
    const int64_t s = i / g.W;
    const int64_t c = i - s * g.W;
    const int32_t *Cu = C + s * 2 * g.W;  // band s's last row
    const int32_t *Cl = Cu + g.W;         // band s+1's first row
    const int32_t a = Cl[c];
    if (a < 0) return;
    const int64_t row1 = (s + 1) * g.hb;  // band s+1's first row
    const uint32_t v = seam_colour(img, dtype, row1 * g.W + c);
    // Pairs of nodes equal to a pair of the column before are skipped (same
    // nodes, so same colours: the same join): straight up when both nodes
    // repeat, up-left when the lower node repeats (it is column c-1's straight
    // pair), up-right when the upper node repeats (it is this column's).
    const int lo = conn == 8 ? -1 : 0, hi = conn == 8 ? 1 : 0;
    for (int d = lo; d <= hi; ++d) {
        const int64_t cc = c + d;
        if (cc < 0 || cc >= g.W) continue;
        const int32_t b = Cu[cc];
        if (b < 0) continue;
        if (d == 0 && c > 0 && Cl[c - 1] == a && Cu[c - 1] == b) continue;
        if (d < 0 && Cl[c - 1] == a) continue;
        if (d > 0 && Cu[c] == b) continue;
        if (seam_colour(img, dtype, (row1 - 1) * g.W + cc) != v) continue;
        seam_unite(P, K, a, b, err);
    }
}

// ---------------------------------------------------------------- seam regions

// seam pixel `node`: its band and its entry in the seam rows (its band-local
// number, or leader)
__device__ __forceinline__ int32_t seam_entry(const Bands &g, int64_t node, const int32_t *rows,
                                              int64_t &band)
{
    const int64_t s = node / (2 * g.W);
    const int64_t rem = node - s * 2 * g.W;
    // seam s: TH rows of band s's last tile row, then TH rows of band s+1's first
    const int32_t *top = rows + s * 2 * TH * g.W, *bot = top + TH * g.W;
    if (rem < g.W) {
        band = s;
        return top[(TH - 1) * g.W + rem];
    }
    band = s + 1;
    return bot[rem - g.W];
}

__device__ __forceinline__ void seam_number(const Bands &g, int64_t node, const int32_t *rows,
                                            int64_t &band, uint32_t &n)
{
    n = (uint32_t)seam_entry(g, node, rows, band);
}

__global__ __launch_bounds__(LB) void nm_clear_kernel(int64_t *hkey, int32_t *hnode, int64_t cap)
{
    for (int64_t i = (int64_t)blockIdx.x * LB + threadIdx.x; i < cap; i += (int64_t)gridDim.x * LB) {
        hkey[i] = -1;
        hnode[i] = INT32_MAX;
    }
}

// the words of each band's merge mask that its numbers use (bit n, n <= n_b)
constexpr int MCB = 16;  // workgroups per band
__global__ __launch_bounds__(LB) void nm_mclear_kernel(const int32_t *bandcnt, int64_t wpb,
                                                       uint64_t *M)
{
    const int64_t k = blockIdx.x / MCB;
    const int64_t nw = ((int64_t)bandcnt[k] >> 6) + 1;
    for (int64_t i = (int64_t)(blockIdx.x % MCB) * LB + threadIdx.x; i < nw; i += (int64_t)MCB * LB)
        M[k * wpb + i] = 0ull;
}

// the table slot of key (inserted if new); -1 if the table is full (it holds
// twice the seam pixels, so it never is)
__device__ int64_t nm_insert(int64_t *hkey, uint32_t hmask, int64_t key)
{
    uint32_t h = seam_hash(key, hmask);
    for (uint32_t i = 0; i <= hmask; ++i, h = (h + 1u) & hmask) {
        const int64_t k = hkey[h];
        if (k == key) return h;
        if (k == -1) {
            const unsigned long long old = atomicCAS((unsigned long long *)&hkey[h],
                                                     (unsigned long long)-1ll,
                                                     (unsigned long long)key);
            if ((int64_t)old == -1 || (int64_t)old == key) return h;
        }
    }
    return -1;
}

// the first pixel of each stretch of one number along a seam row enters the
// number into the table (the others find it there next), so that a region
// along the whole row makes one entry, not one per pixel
__global__ __launch_bounds__(LB) void nm_insert_kernel(Bands g, const int32_t *rows, int64_t *hkey,
                                                       int32_t *hnode, uint32_t hmask, int32_t *S,
                                                       uint32_t *err)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam) return;
    int64_t band;
    uint32_t n;
    seam_number(g, node, rows, band, n);
    int32_t slot = -1;
    if (n != 0u) {  // (0: an ignored pixel)
        int64_t bl;
        uint32_t nl = 0;
        if (node % g.W != 0) seam_number(g, node - 1, rows, bl, nl);
        if (nl == n) {
            slot = -2;  // looked up next
        } else {
            const int64_t h = nm_insert(hkey, hmask, (band << 32) | n);
            if (h < 0) {
                atomicOr(err, ERR_LOOP);
            } else {
                slot = (int32_t)h;
                atomicMin(&hnode[h], (int32_t)node);
            }
        }
    }
    S[node] = slot;
}

// canonical node of each seam pixel (its region's first seam pixel); those
// take their region's key
__global__ __launch_bounds__(LB) void nm_canon_kernel(Bands g, const int32_t *rows, int32_t *S,
                                                      const int64_t *hkey, uint32_t hmask,
                                                      const int32_t *hnode, int32_t *C, int32_t *P,
                                                      int64_t *K, uint32_t *err)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam) return;
    P[node] = (int32_t)node;
    int32_t slot = S[node];
    if (slot == -2) {  // its stretch's first pixel entered the number
        int64_t band;
        uint32_t n;
        seam_number(g, node, rows, band, n);
        const int64_t key = (band << 32) | n;
        uint32_t h = seam_hash(key, hmask);
        slot = -1;
        for (uint32_t i = 0; i <= hmask; ++i, h = (h + 1u) & hmask)
            if (hkey[h] == key) {
                slot = (int32_t)h;
                break;
            }
        if (slot < 0) atomicOr(err, ERR_LOOP);
        S[node] = slot;
    }
    if (slot < 0) {
        C[node] = -1;
        return;
    }
    const int32_t c = hnode[slot];
    C[node] = c;
    if (c == node) {
        int64_t band;
        uint32_t n;
        seam_number(g, node, rows, band, n);
        K[node] = (band << 32) | n;
    }
}

// each canonical node's root; a part that is not its region's root is merged
__global__ __launch_bounds__(LB) void nm_mark_kernel(Bands g, const int32_t *rows, const int32_t *C,
                                                     int32_t *P, int32_t *R, int64_t wpb,
                                                     uint64_t *M, uint32_t *err)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam || C[node] != node) return;
    int budget = SEAM_BUDGET;
    const int32_t r = seam_find(P, (int32_t)node, budget);
    if (budget <= 0) atomicOr(err, ERR_LOOP);
    R[node] = r;
    if (r != node) {
        int64_t band;
        uint32_t n;
        seam_number(g, node, rows, band, n);
        atomicOr((unsigned long long *)&M[band * wpb + (n >> 6)], 1ull << (n & 63u));
    }
}

// per band (one workgroup each): merged numbers before each mask word, and in all
constexpr int MS_T = 1024;
__global__ __launch_bounds__(MS_T) void nm_mscan_kernel(const int32_t *bandcnt, int64_t wpb,
                                                        const uint64_t *M, uint32_t *Mpre,
                                                        int32_t *mcnt)
{
    __shared__ uint32_t sWave[MS_T / 64];
    const int64_t k = blockIdx.x;
    const int64_t nw = ((int64_t)bandcnt[k] >> 6) + 1;
    const uint64_t *Mk = M + k * wpb;
    uint32_t *Pk = Mpre + k * wpb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t carry = 0;
    for (int64_t base = 0; base < nw; base += MS_T) {
        const int64_t i = base + threadIdx.x;
        const uint32_t c = i < nw ? (uint32_t)__popcll(Mk[i]) : 0u;
        uint32_t x = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t y = __shfl_up(x, d);
            if (lane >= d) x += y;
        }
        if (lane == 63) sWave[wave] = x;
        __syncthreads();
        uint32_t off = 0, tot = 0;
        for (int j = 0; j < MS_T / 64; ++j) {
            const uint32_t v = sWave[j];
            off += j < wave ? v : 0u;
            tot += v;
        }
        if (i < nw) Pk[i] = carry + off + x - c;
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) mcnt[k] = (int32_t)carry;
}

// each band's first number (its regions that are not merged follow the
// earlier bands'), and the picture's count
__global__ void nm_gnum_kernel(const int32_t *bandcnt, const int32_t *mcnt, int64_t nb, int64_t *G,
                               int64_t *count)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int64_t run = 0;
    for (int64_t k = 0; k < nb; ++k) {
        G[k] = run;
        run += (int64_t)bandcnt[k] - mcnt[k];
    }
    if (count) *count = run;
}

// the number of each seam region: at its root, G + n - (merged numbers below
// n), or (leaders: rowsL holds the seam rows' band-local leaders) the band's
// first pixel plus the root's band-local leader; then the merged parts take
// their root's
__global__ __launch_bounds__(LB) void nm_rootval_kernel(Bands g, const int32_t *rows,
                                                        const int32_t *rowsL, const int32_t *C,
                                                        const int32_t *R, const int32_t *S,
                                                        int64_t wpb, const uint64_t *M,
                                                        const uint32_t *Mpre, const int64_t *G,
                                                        int64_t *hval)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam || C[node] != node || R[node] != node) return;
    int64_t band;
    if (rowsL) {
        const int32_t l = seam_entry(g, node, rowsL, band);
        hval[S[node]] = band * g.band_px + (int64_t)l;
        return;
    }
    uint32_t n;
    seam_number(g, node, rows, band, n);
    const int64_t wi = band * wpb + (n >> 6);
    const uint64_t below = M[wi] & ((1ull << (n & 63u)) - 1ull);
    hval[S[node]] = G[band] + (int64_t)n - (int64_t)(Mpre[wi] + (uint32_t)__popcll(below));
}

// each merged number's picture number (or leader), at its rank among its
// band's merged numbers (a band has at most 2W: each has a seam pixel there)
__global__ __launch_bounds__(LB) void nm_mergedval_kernel(Bands g, const int32_t *rows,
                                                          const int32_t *C, const int32_t *R,
                                                          const int32_t *S, int64_t wpb,
                                                          const uint64_t *M, const uint32_t *Mpre,
                                                          const int64_t *hval, int64_t *MV)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam || C[node] != node || R[node] == node) return;
    int64_t band;
    uint32_t n;
    seam_number(g, node, rows, band, n);
    const int64_t wi = band * wpb + (n >> 6);
    const uint32_t r = Mpre[wi] + (uint32_t)__popcll(M[wi] & ((1ull << (n & 63u)) - 1ull));
    MV[band * 2 * g.W + r] = hval[S[R[node]]];
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of one image: every band's tile workspace (bands keep their
// records until their final write), the seam rows (numbers, and leaders), the
// seam-region table and the merge masks.
struct LargeLayout {
    Bands g;
    Layout band;     // tile-pipeline layout of the tallest band
    size_t band_ws;  // bytes of one full band's workspace (band k's starts at k * band_ws)
    int64_t wpb;     // merge-mask words per band (bit n for numbers 0..band_px)
    int64_t cap;     // seam-region table entries (a power of two)
    size_t off_bands, off_bandcnt, off_mcnt, off_G, off_rows, off_rowsL, off_S, off_C, off_P,
        off_R, off_K, off_hkey, off_hnode, off_hval, off_M, off_Mpre, off_MV, total;
};

// Fills `L` for one image of the batch; returns a ccl_status.
static int make_large_layout(int64_t H, int64_t W, int64_t band_rows, LargeLayout *L)
{
    Bands &g = L->g;
    int64_t hb;
    if (band_rows == 0) {
        // about 2^30 pixels, and within the tile pipeline's tile limit
        hb = AUTO_BAND_PX / W;
        const int64_t tile_rows = MAX_TILES / ((W + TW - 1) / TW) * TH;
        if (hb > tile_rows) hb = tile_rows;
        hb = hb / 64 * 64;
        if (hb < 64) hb = 64;
    } else {
        if (band_rows < 0 || band_rows % 64 != 0) return CCL_ERR_BAND;
        hb = band_rows;
    }
    // one band is the whole image (its height need not be a multiple of 64);
    // the band's pixels must be indexable by the tile pipeline
    if (hb >= H) hb = H;
    if (hb > INT32_MAX / W) return band_rows ? CCL_ERR_BAND : CCL_ERR_TOO_LARGE;
    g.H = H;
    g.W = W;
    g.HW = H * W;
    g.hb = hb;
    g.band_px = hb * W;
    g.nb = (H + hb - 1) / hb;
    g.nseam = (g.nb - 1) * 2 * W;
    if (g.nseam > INT32_MAX - 2) return CCL_ERR_TOO_LARGE;  // seam node ids are int32
    if (!make_layout(1, hb, W, &L->band)) return CCL_ERR_TOO_LARGE;

    L->band_ws = align256(L->band.total);
    L->wpb = g.band_px / 64 + 1;
    int64_t cap = 1024;
    while (cap < 2 * g.nseam) cap *= 2;
    L->cap = cap;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t nb = (size_t)g.nb, ns = (size_t)g.nseam;
    const size_t seam_rows = (nb - 1) * 2 * TH * (size_t)g.W * sizeof(int32_t);
    // band 0's workspace comes first, so its error word is the workspace's;
    // the last band may be shorter
    Layout last;
    make_layout(1, g.H - (g.nb - 1) * g.hb, g.W, &last);  // fits: no taller than a full band
    L->off_bands = take((nb - 1) * L->band_ws + last.total);
    L->off_bandcnt = take(nb * sizeof(int32_t));
    L->off_mcnt = take(nb * sizeof(int32_t));
    L->off_G = take(nb * sizeof(int64_t));
    L->off_rows = take(seam_rows);
    L->off_rowsL = take(seam_rows);
    L->off_S = take(ns * sizeof(int32_t));
    L->off_C = take(ns * sizeof(int32_t));
    L->off_P = take(ns * sizeof(int32_t));
    L->off_R = take(ns * sizeof(int32_t));
    L->off_K = take(ns * sizeof(int64_t));
    L->off_hkey = take((size_t)cap * sizeof(int64_t));
    L->off_hnode = take((size_t)cap * sizeof(int32_t));
    L->off_hval = take((size_t)cap * sizeof(int64_t));
    L->off_M = take(nb * (size_t)L->wpb * sizeof(uint64_t));
    L->off_Mpre = take(nb * (size_t)L->wpb * sizeof(uint32_t));
    L->off_MV = take(nb * 2 * (size_t)g.W * sizeof(int64_t));
    L->total = off;
    return CCL_OK;
}

static unsigned grid_for(int64_t items, int64_t cap)
{
    int64_t b = (items + LB - 1) / LB;
    if (b < 1) b = 1;
    return (unsigned)(b < cap ? b : cap);
}

static int check_large_shape(int64_t B, int64_t H, int64_t W, bool *empty)
{
    if (B < 0 || H < 0 || W < 0) return CCL_ERR_SHAPE;
    *empty = (B == 0 || H == 0 || W == 0);
    if (*empty) return CCL_OK;
    const int64_t LIM = int64_t(1) << 46;  // 70 T pixels: every size below stays in int64
    if (H > LIM / W || B > LIM / (H * W)) return CCL_ERR_TOO_LARGE;
    return CCL_OK;
}

// ccl_label_large (the steps above); lead: leaders, else numbers
static int label_large_bands(const void *colours, int dtype, int64_t batch, int connectivity,
                             int ign, uint32_t ignore, int lead, const LargeLayout &N,
                             int64_t *out, int64_t *counts, char *ws, hipStream_t s)
{
    const Bands &g = N.g;
    int32_t *bandcnt = (int32_t *)(ws + N.off_bandcnt);
    int32_t *mcnt = (int32_t *)(ws + N.off_mcnt);
    int64_t *G = (int64_t *)(ws + N.off_G);
    int32_t *rows = (int32_t *)(ws + N.off_rows);
    int32_t *rowsL = (int32_t *)(ws + N.off_rowsL);
    int32_t *S = (int32_t *)(ws + N.off_S);
    int32_t *C = (int32_t *)(ws + N.off_C);
    int32_t *P = (int32_t *)(ws + N.off_P);
    int32_t *R = (int32_t *)(ws + N.off_R);
    int64_t *K = (int64_t *)(ws + N.off_K);
    int64_t *hkey = (int64_t *)(ws + N.off_hkey);
    int32_t *hnode = (int32_t *)(ws + N.off_hnode);
    int64_t *hval = (int64_t *)(ws + N.off_hval);
    uint64_t *M = (uint64_t *)(ws + N.off_M);
    uint32_t *Mpre = (uint32_t *)(ws + N.off_Mpre);
    int64_t *MV = (int64_t *)(ws + N.off_MV);
    uint32_t *err = (uint32_t *)ws;  // band 0's error word: the call's
    const size_t px_bytes = (size_t)dtype;
    const uint32_t hmask = (uint32_t)(N.cap - 1);
    const unsigned gs = grid_for(g.nseam, INT32_MAX);

    for (int64_t b = 0; b < batch; ++b) {
        const uint8_t *img = (const uint8_t *)colours + (size_t)(b * g.HW) * px_bytes;
        Layout Lb[2];  // the layouts of two bands at a time
        auto band_work = [&](int64_t k, Layout &Lk) -> Work {
            const int64_t r0 = k * g.hb;
            const int64_t rowsk = g.H - r0 < g.hb ? g.H - r0 : g.hb;
            make_layout(1, rowsk, g.W, &Lk);  // fits: no taller than the full band
            Work w = bind_work(Lk, ws + N.off_bands + (size_t)k * N.band_ws);
            w.err = err;  // every band reports into the call's error word
            return w;
        };
        // 1. every band through the tile pipeline in number mode (leaders:
        //    each seam node's record pointed at its root)
        for (int64_t k = 0; k < g.nb; ++k) {
            const Work w = band_work(k, Lb[0]);
            launch_tile(img + (size_t)(k * g.hb * g.W) * px_bytes, dtype, connectivity, ign,
                        ignore, Lb[0].g, w, b == 0 && k == 0, s);
            launch_seam(Lb[0].g, w, connectivity, s);
            launch_seam_roots(Lb[0].g, w, s);
            launch_scan(Lb[0].g, w, bandcnt + k, 1, 1, s);
            launch_resolve(Lb[0].g, w, lead ? 2 : 1, s);
        }
        if (g.nb > 1) {
            // 2. the band-local numbers (and leaders) of the tile rows either
            //    side of each seam: band s's last (whole: bands hold a
            //    multiple of 64 rows) and band s+1's first
            for (int64_t sm = 0; sm + 1 < g.nb; ++sm) {
                const int64_t so = sm * 2 * TH * g.W;
                const Work wa = band_work(sm, Lb[0]);
                const uint32_t lastrow = (uint32_t)(Lb[0].g.nty - 1) * (uint32_t)Lb[0].g.ntx;
                const int64_t up = (int64_t)(Lb[0].g.nty - 1) * TH * g.W;  // rows above it
                const Work wb = band_work(sm + 1, Lb[1]);
                for (int form = 1; form <= (lead ? 2 : 1); ++form) {
                    int32_t *top = (form == 1 ? rows : rowsL) + so, *bot = top + TH * g.W;
                    const uint32_t ignv = form == 1 ? 0u : 0xFFFFFFFFu;
                    launch_final(Lb[0].g, wa, top - up, form, ignv, s, lastrow,
                                 (uint32_t)Lb[0].g.ntx);
                    launch_final(Lb[1].g, wb, bot, form, ignv, s, 0u, (uint32_t)Lb[1].g.ntx);
                }
            }
            // 3. the seam regions and their joins
            hipLaunchKernelGGL(nm_clear_kernel, dim3(grid_for(N.cap, 4096)), dim3(LB), 0, s, hkey,
                               hnode, N.cap);
            hipLaunchKernelGGL(nm_insert_kernel, dim3(gs), dim3(LB), 0, s, g, rows, hkey, hnode,
                               hmask, S, err);
            hipLaunchKernelGGL(nm_canon_kernel, dim3(gs), dim3(LB), 0, s, g, rows, S, hkey, hmask,
                               hnode, C, P, K, err);
            hipLaunchKernelGGL(seam_union_kernel, dim3(grid_for((g.nb - 1) * g.W, INT32_MAX)),
                               dim3(LB), 0, s, g, img, dtype, connectivity, C, P, K, err);
        }
        // 4. merged parts, each band's first number, the seam regions' numbers
        //    (or leaders)
        hipLaunchKernelGGL(nm_mclear_kernel, dim3((unsigned)(g.nb * MCB)), dim3(LB), 0, s, bandcnt,
                           N.wpb, M);
        if (g.nb > 1)
            hipLaunchKernelGGL(nm_mark_kernel, dim3(gs), dim3(LB), 0, s, g, rows, C, P, R, N.wpb, M,
                               err);
        hipLaunchKernelGGL(nm_mscan_kernel, dim3((unsigned)g.nb), dim3(MS_T), 0, s, bandcnt, N.wpb,
                           M, Mpre, mcnt);
        hipLaunchKernelGGL(nm_gnum_kernel, dim3(1), dim3(64), 0, s, bandcnt, mcnt, g.nb, G,
                           counts ? counts + b : (int64_t *)nullptr);
        if (g.nb > 1) {
            hipLaunchKernelGGL(nm_rootval_kernel, dim3(gs), dim3(LB), 0, s, g, rows,
                               lead ? rowsL : (const int32_t *)nullptr, C, R, S, N.wpb, M, Mpre, G,
                               hval);
            hipLaunchKernelGGL(nm_mergedval_kernel, dim3(gs), dim3(LB), 0, s, g, rows, C, R, S,
                               N.wpb, M, Mpre, hval, MV);
        }
        // 5. 64-bit numbers (or leaders), band by band, from the bands' records
        for (int64_t k = 0; k < g.nb; ++k) {
            const Work w = band_work(k, Lb[0]);
            Map64 m;
            m.M = M + k * N.wpb;
            m.Mpre = Mpre + k * N.wpb;
            m.MV = MV + k * 2 * g.W;
            m.G = G;
            m.base = k * g.band_px;
            m.band = (uint32_t)k;
            m.merges = g.nb > 1;
            launch_final64(Lb[0].g, w, out + b * g.HW + k * g.band_px, m, lead, s);
        }
    }
    return hipGetLastError() == hipSuccess ? CCL_OK : CCL_ERR_HIP;
}

}  // namespace large
}  // namespace ccl

using namespace ccl;
using namespace ccl::large;

extern "C" {

size_t ccl_large_workspace_bytes(int64_t batch, int64_t height, int64_t width, int64_t band_rows)
{
    bool empty;
    if (check_large_shape(batch, height, width, &empty) != CCL_OK) return SIZE_MAX;
    if (empty) return 0;
    LargeLayout L;
    if (make_large_layout(height, width, band_rows, &L) != CCL_OK) return SIZE_MAX;
    return L.total;
}

int ccl_label_large(const void *colours, int dtype, int64_t batch, int64_t height, int64_t width,
                    int connectivity, int flags, uint32_t ignore, int64_t band_rows, int64_t *out,
                    int64_t *counts, void *workspace, size_t workspace_bytes, void *stream)
{
    if (flags & ~(CCL_NUMBER | CCL_IGNORE)) return CCL_ERR_FLAGS;
    bool empty;
    int rc = check_large_shape(batch, height, width, &empty);
    if (rc != CCL_OK) return rc;
    if (dtype != CCL_U8 && dtype != CCL_RGB24 && dtype != CCL_U32) return CCL_ERR_DTYPE;
    if (connectivity != 4 && connectivity != 8) return CCL_ERR_CONNECTIVITY;
    const int ign = (flags & CCL_IGNORE) != 0;
    if (ign && dtype != CCL_U32 && ignore >= (1u << (8 * dtype))) return CCL_ERR_IGNORE;
    if (band_rows < 0 || band_rows % 64 != 0) return CCL_ERR_BAND;
    hipStream_t s = (hipStream_t)stream;
    if (empty) {
        if (counts && batch > 0) {
            // counts are int64: zero them as 2*batch int32 words
            launch_zero_i32((int32_t *)counts, 2 * batch, s);
            return hipGetLastError() == hipSuccess ? CCL_OK : CCL_ERR_HIP;
        }
        return CCL_OK;
    }
    if (!colours || !out || !workspace) return CCL_ERR_NULL;
    LargeLayout L;
    rc = make_large_layout(height, width, band_rows, &L);
    if (rc != CCL_OK) return rc;
    if (workspace_bytes < L.total) return CCL_ERR_WORKSPACE;
    return label_large_bands(colours, dtype, batch, connectivity, ign, ignore,
                             (flags & CCL_NUMBER) ? 0 : 1, L, out, counts, (char *)workspace, s);
}

}  // extern "C"
