// ccl_large.hip -- labelling of images of any size, beyond 2^31 pixels, with
// 64-bit leaders and numbers.
//
// "Accountable AI starts at the pixel" lists images of more than 2^31 pixels
// as not run (ch.11 "How we know it is right"), and shows in ch.10 what a size
// wrapped to 32 bits does.  Here such an image is cut into bands of whole tile
// rows, each small enough for the 32-bit tile pipeline:
//
//   1. each band is labelled on its own (leaders relative to the band) into
//      one int32 array over the whole image;
//   2. the leaders of the pixels on the rows either side of each band seam are
//      tagged: each such leader's own entry is replaced by -(2 + node), node
//      one of its seam pixels (the largest), so every pixel can tell that its
//      leader is a seam node and which one;
//   3. equal-colour neighbours across each seam are joined in a union-find
//      over seam nodes whose keys are the leaders' 64-bit reading-order
//      indices; a join points the larger key at the smaller, as the tile
//      pipeline does inside a band (same page, ch.04 "Point at a leader"), so
//      each set's root is its region's first pixel;
//   4. (numbers or counts) a pass flags each image's leaders in one bit per
//      pixel, with per-word and per-block counts, and a scan turns the block
//      counts into 64-bit prefixes (ch.08 idea 5 "Number without a giant list");
//   5. a final pass writes each pixel's 64-bit leader or number.
//
// The seams between bands are the same seams a band per GPU would have: this
// is the one-GPU form of labelling one picture across several GPUs.
#include "ccl.h"
#include "ccl_internal.h"

#include <limits.h>

namespace ccl {
namespace large {

constexpr int LB = 256;            // threads per workgroup
constexpr int LWAVES = LB / 64;
constexpr int WPW = 16;            // 64-pixel words per wave in the flag pass
constexpr int BLK_WORDS = LWAVES * WPW;    // words per numbering block
constexpr int BLK_PX = BLK_WORDS * 64;     // 4096 pixels per numbering block
constexpr int BLK_SHIFT = 12;
static_assert(BLK_PX == (1 << BLK_SHIFT), "numbering blocks are 2^12 pixels");
constexpr int SEAM_BUDGET = 1 << 20;       // bound on one union's find/link steps
constexpr int64_t AUTO_BAND_PX = int64_t(1) << 30;

// Geometry of one image cut into bands.
struct Bands {
    int64_t H, W, HW;
    int64_t hb;        // rows per band (a multiple of 64 when there are several)
    int64_t band_px;   // hb * W
    int64_t nb;        // bands
    int64_t nseam;     // seam pixels: (nb - 1) * 2W
    int64_t nwords;    // 64-pixel words of the image
    int64_t nblk;      // numbering blocks of the image
};

// Node ids of seam pixels: seam s (between bands s and s+1) owns ids
// [s*2W, (s+1)*2W): s*2W + c is column c of band s's last row, s*2W + W + c
// column c of band s+1's first row.
__device__ __forceinline__ void seam_pixel(const Bands &g, int64_t node, int64_t &band,
                                           int64_t &local)
{
    const int64_t s = node / (2 * g.W);
    const int64_t rem = node - s * 2 * g.W;
    if (rem < g.W) {
        band = s;
        local = (g.hb - 1) * g.W + rem;
    } else {
        band = s + 1;
        local = rem - g.W;
    }
}

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

// Step 2: every seam pixel tags its band leader's own entry with the largest
// of the leader's seam nodes.  Ignored pixels (-1) take part in nothing.
__global__ __launch_bounds__(LB) void tag_kernel(Bands g, int32_t *lead)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam) return;
    int64_t band, local;
    seam_pixel(g, node, band, local);
    int32_t *L = lead + band * g.band_px;
    const int32_t l = L[local];
    if (l == -1) return;
    // l < -1: this pixel is a leader another seam pixel has tagged already
    const int64_t target = l < 0 ? local : (int64_t)l;
    atomicMin(&L[target], (int32_t)(-2 - node));
}

// Step 2b: each seam pixel records its canonical node (the tag of its leader);
// the canonical node of a leader takes the leader's 64-bit key.
__global__ __launch_bounds__(LB) void canon_kernel(Bands g, const int32_t *lead, int32_t *C,
                                                   int32_t *P, int64_t *K)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam) return;
    int64_t band, local;
    seam_pixel(g, node, band, local);
    const int32_t *L = lead + band * g.band_px;
    const int32_t l = L[local];
    P[node] = (int32_t)node;
    if (l == -1) {
        C[node] = -1;
        return;
    }
    const int64_t leader = l < 0 ? local : (int64_t)l;
    const int32_t t = l < 0 ? l : L[leader];
    const int32_t canon = -2 - t;
    C[node] = canon;
    if (canon == node) K[node] = band * g.band_px + leader;
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
    const int32_t a = C[s * 2 * g.W + g.W + c];
    if (a < 0) return;
    const int64_t row1 = (s + 1) * g.hb;  // band s+1's first row
    const uint32_t v = seam_colour(img, dtype, row1 * g.W + c);
    const int lo = conn == 8 ? -1 : 0, hi = conn == 8 ? 1 : 0;
    for (int d = lo; d <= hi; ++d) {
        const int64_t cc = c + d;
        if (cc < 0 || cc >= g.W) continue;
        const int32_t b = C[s * 2 * g.W + cc];
        if (b < 0) continue;
        if (seam_colour(img, dtype, (row1 - 1) * g.W + cc) != v) continue;
        seam_unite(P, K, a, b, err);
    }
}

// Step 3b: the key of each canonical node's root, i.e. its region's leader.
__global__ __launch_bounds__(LB) void seam_root_kernel(Bands g, const int32_t *C, int32_t *P,
                                                       const int64_t *K, int64_t *rootkey,
                                                       uint32_t *err)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam || C[node] != node) return;
    int budget = SEAM_BUDGET;
    const int32_t r = seam_find(P, (int32_t)node, budget);
    if (budget <= 0) atomicOr(err, ERR_LOOP);
    rootkey[node] = K[r];
}

// A pixel's 64-bit leader from its band-relative entry l (not -1).
__device__ __forceinline__ int64_t global_leader(const int32_t *lead, const int64_t *rootkey,
                                                 int64_t base, int32_t l)
{
    if (l <= -2) return rootkey[-2 - l];  // the pixel is a tagged seam leader
    const int32_t t = lead[base + l];
    return t <= -2 ? rootkey[-2 - t] : base + l;
}

// Step 4: leader bits, per-word prefixes inside each block, block counts.
__global__ __launch_bounds__(LB) void flag_kernel(Bands g, const int32_t *lead,
                                                  const int64_t *rootkey, uint64_t *mask,
                                                  uint16_t *wordin, uint32_t *blkcnt)
{
    __shared__ uint32_t wtot[LWAVES];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t k = blockIdx.x; k < g.nblk; k += gridDim.x) {
        uint32_t run = 0, mine = 0;
        const int64_t w0 = k * BLK_WORDS + wave * WPW;
        for (int j = 0; j < WPW; ++j) {
            const int64_t pw = (w0 + j) * 64;
            if (pw >= g.HW) break;
            const int64_t base = pw / g.band_px * g.band_px;
            const int64_t px = pw + lane;
            bool is_lead = false;
            if (px < g.HW) {
                const int32_t l = lead[px];
                is_lead = l == (int32_t)(px - base) || (l <= -2 && rootkey[-2 - l] == px);
            }
            const uint64_t m = __ballot(is_lead);
            if (lane == 0) mask[w0 + j] = m;
            if (lane == j) mine = run;
            run += (uint32_t)__popcll(m);
        }
        if (lane == 0) wtot[wave] = run;
        __syncthreads();
        uint32_t off = 0, tot = 0;
        for (int v = 0; v < LWAVES; ++v) {
            off += v < wave ? wtot[v] : 0u;
            tot += wtot[v];
        }
        if (lane < WPW && (w0 + lane) * 64 < g.HW) wordin[w0 + lane] = (uint16_t)(off + mine);
        if (threadIdx.x == 0) blkcnt[k] = tot;
        __syncthreads();
    }
}

// Step 4b: exclusive 64-bit prefix of the block counts (one workgroup of 1024
// threads, 16 blocks per thread per round); blkpre[nblk] and *count = total.
constexpr int SCAN_T = 1024;
constexpr int SCAN_PER = 16;
__global__ __launch_bounds__(SCAN_T) void block_scan_kernel(const uint32_t *blkcnt, int64_t nblk,
                                                            int64_t *blkpre, int64_t *count)
{
    __shared__ int64_t wsum[SCAN_T / 64];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int64_t carry = 0;
    for (int64_t base = 0; base < nblk; base += (int64_t)SCAN_T * SCAN_PER) {
        const int64_t i0 = base + (int64_t)t * SCAN_PER;
        uint32_t v[SCAN_PER];
        int64_t sum = 0;
        for (int j = 0; j < SCAN_PER; ++j) {
            v[j] = i0 + j < nblk ? blkcnt[i0 + j] : 0u;
            sum += v[j];
        }
        int64_t inc = sum;  // inclusive scan over the wave
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t o = __shfl_up(inc, d, 64);
            if (lane >= d) inc += o;
        }
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        int64_t woff = 0, total = 0;
        for (int v2 = 0; v2 < SCAN_T / 64; ++v2) {
            woff += v2 < wave ? wsum[v2] : 0;
            total += wsum[v2];
        }
        int64_t run = carry + woff + inc - sum;
        for (int j = 0; j < SCAN_PER; ++j) {
            if (i0 + j < nblk) blkpre[i0 + j] = run;
            run += v[j];
        }
        carry += total;
        __syncthreads();
    }
    if (t == 0) {
        blkpre[nblk] = carry;
        if (count) *count = carry;
    }
}

// Step 5: each pixel's 64-bit leader (number = 0) or number 1..n (number = 1);
// ignored pixels get -1 or 0.
__global__ __launch_bounds__(LB) void final_kernel(Bands g, const int32_t *lead,
                                                   const int64_t *rootkey, const uint64_t *mask,
                                                   const uint16_t *wordin, const int64_t *blkpre,
                                                   int number, int64_t *out)
{
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * LWAVES;
    for (int64_t w = (int64_t)blockIdx.x * LWAVES + (threadIdx.x >> 6); w < g.nwords;
         w += stride) {
        const int64_t pw = w * 64;
        const int64_t base = pw / g.band_px * g.band_px;
        const int64_t px = pw + lane;
        if (px >= g.HW) continue;
        const int32_t l = lead[px];
        int64_t v;
        if (l == -1) {
            v = number ? 0 : -1;
        } else {
            const int64_t G = global_leader(lead, rootkey, base, l);
            if (number) {
                const int64_t wd = G >> 6;
                const uint64_t below = mask[wd] & ((uint64_t(1) << (G & 63)) - 1);
                v = 1 + blkpre[G >> BLK_SHIFT] + wordin[wd] + __popcll(below);
            } else {
                v = G;
            }
        }
        __builtin_nontemporal_store(v, out + px);
    }
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct LargeLayout {
    Bands g;
    Layout band;      // tile-pipeline layout of the tallest band
    size_t off_lead, off_C, off_P, off_K, off_root, off_mask, off_wordin, off_blkcnt, off_blkpre,
        total;
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
        if (hb * W > INT32_MAX) return CCL_ERR_TOO_LARGE;  // a 64-row band is too wide
    } else {
        if (band_rows < 0 || band_rows % 64 != 0) return CCL_ERR_BAND;
        if (band_rows > INT32_MAX / W) return CCL_ERR_BAND;
        hb = band_rows;
    }
    if (hb >= H) hb = H;  // one band: the whole image
    g.H = H;
    g.W = W;
    g.HW = H * W;
    g.hb = hb;
    g.band_px = hb * W;
    g.nb = (H + hb - 1) / hb;
    g.nseam = (g.nb - 1) * 2 * W;
    if (g.nseam > INT32_MAX - 2) return CCL_ERR_TOO_LARGE;  // node tags are int32
    g.nwords = (g.HW + 63) / 64;
    g.nblk = (g.HW + BLK_PX - 1) / BLK_PX;
    if (!make_layout(1, hb, W, &L->band)) return CCL_ERR_TOO_LARGE;

    // the band workspace comes first, so its error word is the workspace's
    size_t off = align256(L->band.total);
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t ns = (size_t)g.nseam;
    L->off_lead = take((size_t)g.HW * sizeof(int32_t));
    L->off_C = take(ns * sizeof(int32_t));
    L->off_P = take(ns * sizeof(int32_t));
    L->off_K = take(ns * sizeof(int64_t));
    L->off_root = take(ns * sizeof(int64_t));
    L->off_mask = take((size_t)g.nwords * sizeof(uint64_t));
    L->off_wordin = take((size_t)g.nwords * sizeof(uint16_t));
    L->off_blkcnt = take((size_t)g.nblk * sizeof(uint32_t));
    L->off_blkpre = take((size_t)(g.nblk + 1) * sizeof(int64_t));
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
    const Bands &g = L.g;
    char *ws = (char *)workspace;
    int32_t *lead = (int32_t *)(ws + L.off_lead);
    int32_t *C = (int32_t *)(ws + L.off_C);
    int32_t *P = (int32_t *)(ws + L.off_P);
    int64_t *K = (int64_t *)(ws + L.off_K);
    int64_t *rootkey = (int64_t *)(ws + L.off_root);
    uint64_t *mask = (uint64_t *)(ws + L.off_mask);
    uint16_t *wordin = (uint16_t *)(ws + L.off_wordin);
    uint32_t *blkcnt = (uint32_t *)(ws + L.off_blkcnt);
    int64_t *blkpre = (int64_t *)(ws + L.off_blkpre);
    uint32_t *err = (uint32_t *)ws;  // the band workspace's error word
    const int number = (flags & CCL_NUMBER) != 0;
    const bool need_scan = number || counts != nullptr;
    const size_t px_bytes = (size_t)dtype;

    for (int64_t b = 0; b < batch; ++b) {
        const uint8_t *img = (const uint8_t *)colours + (size_t)(b * g.HW) * px_bytes;
        // 1. bands through the tile pipeline: band-relative leaders, -1 ignored
        for (int64_t k = 0; k < g.nb; ++k) {
            const int64_t r0 = k * g.hb;
            const int64_t rows = g.H - r0 < g.hb ? g.H - r0 : g.hb;
            Layout Lb;
            if (!make_layout(1, rows, g.W, &Lb)) return CCL_ERR_TOO_LARGE;
            const Work w = bind_work(Lb, workspace);
            launch_tile(img + (size_t)(r0 * g.W) * px_bytes, dtype, connectivity, ign, ignore,
                        Lb.g, w, s);
            launch_seam(Lb.g, w, connectivity, s);
            launch_resolve(Lb.g, w, 0, s);
            launch_final(Lb.g, w, lead + r0 * g.W, 0, 0xFFFFFFFFu, s);
        }
        // 2-3. joins across the band seams
        if (g.nb > 1) {
            const unsigned gs = grid_for(g.nseam, INT32_MAX);
            hipLaunchKernelGGL(tag_kernel, dim3(gs), dim3(LB), 0, s, g, lead);
            hipLaunchKernelGGL(canon_kernel, dim3(gs), dim3(LB), 0, s, g, lead, C, P, K);
            hipLaunchKernelGGL(seam_union_kernel, dim3(grid_for((g.nb - 1) * g.W, INT32_MAX)),
                               dim3(LB), 0, s, g, img, dtype, connectivity, C, P, K, err);
            hipLaunchKernelGGL(seam_root_kernel, dim3(gs), dim3(LB), 0, s, g, C, P, K, rootkey,
                               err);
        }
        // 4. leader bits and their prefixes
        if (need_scan) {
            const unsigned gf = (unsigned)(g.nblk < (1 << 20) ? g.nblk : (1 << 20));
            hipLaunchKernelGGL(flag_kernel, dim3(gf), dim3(LB), 0, s, g, lead, rootkey, mask,
                               wordin, blkcnt);
            hipLaunchKernelGGL(block_scan_kernel, dim3(1), dim3(SCAN_T), 0, s, blkcnt, g.nblk,
                               blkpre, counts ? counts + b : (int64_t *)nullptr);
        }
        // 5. 64-bit results
        const int64_t waves = g.nwords;
        const int64_t blocks = (waves + LWAVES - 1) / LWAVES;
        hipLaunchKernelGGL(final_kernel, dim3((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20))),
                           dim3(LB), 0, s, g, lead, rootkey, mask, wordin, blkpre, number,
                           out + b * g.HW);
    }
    return hipGetLastError() == hipSuccess ? CCL_OK : CCL_ERR_HIP;
}

}  // extern "C"
