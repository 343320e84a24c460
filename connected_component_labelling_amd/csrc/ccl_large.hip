// ccl_large.hip -- labelling of images of any size, beyond 2^31 pixels, with
// 64-bit leaders and numbers.
//
// "Accountable AI starts at the pixel" lists images of more than 2^31 pixels
// as not run (ch.11 "How we know it is right"), and shows in ch.10 what a size
// wrapped to 32 bits does.  Here such an image is cut into bands of whole tile
// rows, each small enough for the 32-bit tile pipeline.  Leaders:
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
//   4. (counts) a pass flags each image's leaders in one bit per pixel, with
//      per-word and per-block counts, and a scan turns the block counts into
//      64-bit prefixes (ch.08 idea 5 "Number without a giant list");
//   5. a final pass writes each pixel's 64-bit leader.
//
// Numbers take another route, with no 32-bit array over the picture (see
// "numbers" below): the bands number themselves and their seam regions are
// joined by (band, number).
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

// Step 2: the seam pixels tag their band leader's own entry with the largest
// of the leader's run-starting seam nodes.  Ignored pixels (-1) take part in
// nothing.
__global__ __launch_bounds__(LB) void tag_kernel(Bands g, int32_t *lead)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam) return;
    int64_t band, local;
    seam_pixel(g, node, band, local);
    int32_t *L = lead + band * g.band_px;
    const int32_t l = L[local];
    if (l == -1) return;
    // one atomic per run of one leader along the seam row: a pixel whose left
    // neighbour on the row has its leader leaves the tag to that run's first
    // pixel (the leader itself, if on the row, starts its run)
    const int64_t col = node % g.W;
    if (l >= 0 && col > 0 && L[local - 1] == l) return;
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

// Block of round `base` taken by workgroup bid: workgroups are dealt to the 8
// XCDs round-robin, so XCD j gets the j-th contiguous eighth of the round's
// blocks; the earlier rows that a pixel's leader lookups read were then mostly
// streamed through the same XCD's L2.
__device__ __forceinline__ int64_t xcd_block(int64_t base, int64_t nblk, uint32_t bid,
                                             uint32_t grid)
{
    const int64_t left = nblk - base;
    const uint32_t n = left < grid ? (uint32_t)left : grid;
    if (bid >= n) return -1;
    const uint32_t q = n >> 3, r = n & 7u;
    const uint32_t j = bid & 7u, i = bid >> 3;
    if (n < 8) return base + bid;
    return base + j * q + (j < r ? j : r) + i;
}

// The 16 consecutive words of one wave: their first pixel pw0 (wave-uniform)
// and, per word, the first pixel of its band.  Bands hold a multiple of 64
// pixels whenever there are several, so a word never straddles two; the band
// of the first word takes one division and later words step band by band.
struct WaveWords {
    int64_t pw0;
    int64_t base[WPW];
    int64_t band[WPW];
};

__device__ __forceinline__ void wave_words(const Bands &g, int64_t w0, WaveWords &ww)
{
    ww.pw0 = w0 * 64;
    if (g.nb == 1) {  // one band: the whole image
#pragma unroll
        for (int j = 0; j < WPW; ++j) {
            ww.base[j] = 0;
            ww.band[j] = 0;
        }
        return;
    }
    // words past the image keep the last band (their values are never used,
    // and every band index stays below nb)
    int64_t band = ww.pw0 / g.band_px;
    if (band > g.nb - 1) band = g.nb - 1;
    int64_t base = band * g.band_px;
    int64_t next = base + g.band_px;
#pragma unroll
    for (int j = 0; j < WPW; ++j) {
        const int64_t pw = ww.pw0 + 64 * j;
        while (pw >= next && next < g.HW) {
            base = next;
            next += g.band_px;
            ++band;
        }
        ww.base[j] = base;
        ww.band[j] = band;
    }
}

// Step 4: leader bits, per-word prefixes inside each block, block counts.
// Workgroup k takes block k (4096 pixels), wave v its words 16v..16v+15; every
// lane's 16 loads are issued before the first is used.
__global__ __launch_bounds__(LB) void flag_kernel(Bands g, const int32_t *lead,
                                                  const int64_t *rootkey, uint64_t *mask,
                                                  uint16_t *wordin, uint32_t *blkcnt)
{
    __shared__ uint32_t wtot[LWAVES];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t round = 0; round < g.nblk; round += gridDim.x) {
        const int64_t k = xcd_block(round, g.nblk, blockIdx.x, gridDim.x);
        if (k < 0) break;
        const int64_t w0 = k * BLK_WORDS + wave * WPW;
        WaveWords ww;
        wave_words(g, w0, ww);
        int32_t l[WPW];
#pragma unroll
        for (int j = 0; j < WPW; ++j) {
            const int64_t px = ww.pw0 + 64 * j + lane;
            l[j] = px < g.HW ? lead[px] : -1;
        }
        uint32_t run = 0, mine = 0;
        uint64_t mymask = 0;  // lane j keeps word j's bits
#pragma unroll
        for (int j = 0; j < WPW; ++j) {
            const int64_t px = ww.pw0 + 64 * j + lane;
            const bool is_lead = l[j] == (int32_t)(px - ww.base[j]) ||
                                 (l[j] <= -2 && rootkey[-2 - l[j]] == px);
            const uint64_t m = __ballot(is_lead);
            if (lane == j) {
                mine = run;
                mymask = m;
            }
            run += (uint32_t)__popcll(m);
        }
        if (lane == 0) wtot[wave] = run;
        __syncthreads();
        uint32_t off = 0, tot = 0;
        for (int v = 0; v < LWAVES; ++v) {
            off += v < wave ? wtot[v] : 0u;
            tot += wtot[v];
        }
        if (lane < WPW && (w0 + lane) * 64 < g.HW) {
            mask[w0 + lane] = mymask;
            wordin[w0 + lane] = (uint16_t)(off + mine);
        }
        if (threadIdx.x == 0) blkcnt[k] = tot;
        __syncthreads();
    }
}

// Step 4b: exclusive 64-bit prefix of the block counts in two levels: chunks
// of CHUNK blocks scanned by one workgroup each (prefix inside the chunk, and
// the chunk's total), the chunk totals by one workgroup, then each block adds
// its chunk's prefix.  blkpre[nblk] and *count = the image's total.
constexpr int SCAN_T = 1024;
constexpr int SCAN_PER = 16;
constexpr int64_t CHUNK = (int64_t)SCAN_T * SCAN_PER;

// Exclusive scan of n values (v loaded per thread, SCAN_PER consecutive each)
// across one workgroup of SCAN_T threads; returns this thread's first prefix
// and the total through `total`.
__device__ __forceinline__ int64_t wg_exclusive(int64_t sum, int64_t *wsum, int64_t &total)
{
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int64_t inc = sum;
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int64_t woff = 0;
    total = 0;
    for (int v = 0; v < SCAN_T / 64; ++v) {
        woff += v < wave ? wsum[v] : 0;
        total += wsum[v];
    }
    __syncthreads();
    return woff + inc - sum;
}

__global__ __launch_bounds__(SCAN_T) void chunk_scan_kernel(const uint32_t *blkcnt, int64_t nblk,
                                                            int64_t *blkpre, int64_t *chunktot)
{
    __shared__ int64_t wsum[SCAN_T / 64];
    const int64_t i0 = blockIdx.x * CHUNK + (int64_t)threadIdx.x * SCAN_PER;
    uint32_t v[SCAN_PER];
    int64_t sum = 0;
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) {
        v[j] = i0 + j < nblk ? blkcnt[i0 + j] : 0u;
        sum += v[j];
    }
    int64_t total;
    int64_t run = wg_exclusive(sum, wsum, total);
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) {
        if (i0 + j < nblk) blkpre[i0 + j] = run;
        run += v[j];
    }
    if (threadIdx.x == 0) chunktot[blockIdx.x] = total;
}

__global__ __launch_bounds__(SCAN_T) void chunk_total_scan_kernel(int64_t *chunktot,
                                                                  int64_t nchunk, int64_t *total_out,
                                                                  int64_t *count)
{
    __shared__ int64_t wsum[SCAN_T / 64];
    int64_t carry = 0;
    for (int64_t base = 0; base < nchunk; base += CHUNK) {
        const int64_t i0 = base + (int64_t)threadIdx.x * SCAN_PER;
        int64_t v[SCAN_PER];
        int64_t sum = 0;
        for (int j = 0; j < SCAN_PER; ++j) {
            v[j] = i0 + j < nchunk ? chunktot[i0 + j] : 0;
            sum += v[j];
        }
        int64_t total;
        int64_t run = carry + wg_exclusive(sum, wsum, total);
        for (int j = 0; j < SCAN_PER; ++j) {
            if (i0 + j < nchunk) chunktot[i0 + j] = run;  // in place: now the chunk's prefix
            run += v[j];
        }
        carry += total;
    }
    if (threadIdx.x == 0) {
        *total_out = carry;
        if (count) *count = carry;
    }
}

__global__ __launch_bounds__(LB) void chunk_add_kernel(int64_t *blkpre, int64_t nblk,
                                                       const int64_t *chunkpre)
{
    const int64_t i = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (i < nblk) blkpre[i] += chunkpre[i / CHUNK];
}

// Step 5 (leaders): each pixel's 64-bit leader; ignored pixels get -1.  A
// wave takes the same 16 words as in the flag pass, as 8 groups of 128 pixels
// with 2 consecutive pixels per lane (8-byte loads of the entries, 16-byte
// stores of the results: each store instruction covers 1 KB without gaps), in
// phases so that each phase's loads are in flight together: the pixels' own
// entries, then their leaders' entries.  A leader's entry holds what the pixel
// needs: a tag (a seam node: its root's key) or its own index.
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef long long v2i64 __attribute__((ext_vector_type(2)));
constexpr int FGRP = WPW / 2;  // groups of 128 pixels per wave

__device__ __forceinline__ int64_t out_leader(int32_t l, int32_t t, int64_t base,
                                              const int64_t *rootkey)
{
    if (l == -1) return -1;
    const int32_t tag = l <= -2 ? l : t;
    if (tag <= -2) return rootkey[-2 - tag];
    return base + l;
}

__global__ __launch_bounds__(LB) void final_kernel(Bands g, const int32_t *lead,
                                                   const int64_t *rootkey, int64_t *out, int out16)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 5;  // the lane's word inside a group of 2
    for (int64_t round = 0; round < g.nblk; round += gridDim.x) {
        const int64_t k = xcd_block(round, g.nblk, blockIdx.x, gridDim.x);
        if (k < 0) break;
        const int64_t w0 = k * BLK_WORDS + wave * WPW;
        WaveWords ww;
        wave_words(g, w0, ww);
        int64_t base[FGRP];
#pragma unroll
        for (int i = 0; i < FGRP; ++i) base[i] = q == 0 ? ww.base[2 * i] : ww.base[2 * i + 1];
        int32_t l[FGRP][2], t[FGRP][2];
#pragma unroll
        for (int i = 0; i < FGRP; ++i) {
            const int64_t px = ww.pw0 + 128 * i + 2 * lane;
            if (px + 1 < g.HW) {
                const v2i32 v = *(const v2i32 *)(lead + px);
                l[i][0] = v.x;
                l[i][1] = v.y;
            } else {
                l[i][0] = px < g.HW ? lead[px] : -1;
                l[i][1] = -1;
            }
        }
#pragma unroll
        for (int i = 0; i < FGRP; ++i)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                t[i][e] = l[i][e] >= 0 ? lead[base[i] + l[i][e]] : l[i][e];
#pragma unroll
        for (int i = 0; i < FGRP; ++i) {
            const int64_t px = ww.pw0 + 128 * i + 2 * lane;
            const int64_t v0 = out_leader(l[i][0], t[i][0], base[i], rootkey);
            const int64_t v1 = out_leader(l[i][1], t[i][1], base[i], rootkey);
            if (out16 && px + 1 < g.HW) {
                v2i64 a;
                a.x = v0;
                a.y = v1;
                __builtin_nontemporal_store(a, (v2i64 *)(out + px));
            } else {
                if (px < g.HW) __builtin_nontemporal_store(v0, out + px);
                if (px + 1 < g.HW) __builtin_nontemporal_store(v1, out + px + 1);
            }
        }
    }
}

// ---------------------------------------------------------------- numbers
// Numbers take another route, with no 32-bit intermediate over the picture:
//   1. every band goes through the whole tile pipeline in number mode (its
//      own numbers 1..n_b and count) and keeps its tile records;
//   2. the band-local numbers of the rows either side of each seam are
//      written out (the final write of those tile rows);
//   3. each seam region (band, number) gets one entry of a hash table; its
//      canonical node is its first seam pixel, equal-colour neighbours across
//      the seams are joined over canonical nodes keyed by (band, number),
//      which orders regions as their leaders do, so each set's root is its
//      region's leading part;
//   4. every other part is merged: bit n of its band's mask; each band's
//      merged numbers are prefix-counted, the bands' own numbers give each
//      band's first number G_b, each root's number is G_b + n - (merged
//      numbers below n), and each merged number takes its root's, stored at
//      its rank among its band's merged numbers;
//   5. each band's final write maps its numbers through that (Map64) and
//      writes the 64-bit labels straight from its tile records.

// seam pixel `node`: its band and band-local number (from the seam rows)
__device__ __forceinline__ void seam_number(const Bands &g, int64_t node, const int32_t *rows,
                                            int64_t &band, uint32_t &n)
{
    const int64_t s = node / (2 * g.W);
    const int64_t rem = node - s * 2 * g.W;
    // seam s: TH rows of band s's last tile row, then TH rows of band s+1's first
    const int32_t *top = rows + s * 2 * TH * g.W, *bot = top + TH * g.W;
    if (rem < g.W) {
        band = s;
        n = (uint32_t)top[(TH - 1) * g.W + rem];
    } else {
        band = s + 1;
        n = (uint32_t)bot[rem - g.W];
    }
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
// n); then the merged parts take their root's
__global__ __launch_bounds__(LB) void nm_rootval_kernel(Bands g, const int32_t *rows,
                                                        const int32_t *C, const int32_t *R,
                                                        const int32_t *S, int64_t wpb,
                                                        const uint64_t *M, const uint32_t *Mpre,
                                                        const int64_t *G, int64_t *hval)
{
    const int64_t node = (int64_t)blockIdx.x * LB + threadIdx.x;
    if (node >= g.nseam || C[node] != node || R[node] != node) return;
    int64_t band;
    uint32_t n;
    seam_number(g, node, rows, band, n);
    const int64_t wi = band * wpb + (n >> 6);
    const uint64_t below = M[wi] & ((1ull << (n & 63u)) - 1ull);
    hval[S[node]] = G[band] + (int64_t)n - (int64_t)(Mpre[wi] + (uint32_t)__popcll(below));
}

// each merged number's picture number, at its rank among its band's merged
// numbers (a band has at most 2W: each has a seam pixel there)
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

struct LargeLayout {
    Bands g;
    Layout band;      // tile-pipeline layout of the tallest band
    size_t off_lead, off_C, off_P, off_K, off_root, off_mask, off_wordin,
        off_blkcnt, off_blkpre, off_chunk, total;
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
    L->off_chunk = take((size_t)((g.nblk + CHUNK - 1) / CHUNK) * sizeof(int64_t));
    L->total = off;
    return CCL_OK;
}

// Numbers: every band's tile workspace (bands keep their records until their
// final write), the seam rows, the seam-region table and the merge masks.
struct NumLayout {
    Layout band;     // tile-pipeline layout of the tallest band
    size_t band_ws;  // bytes of one full band's workspace (band k's starts at k * band_ws)
    int64_t wpb;     // merge-mask words per band (bit n for numbers 0..band_px)
    int64_t cap;     // seam-region table entries (a power of two)
    size_t off_bands, off_bandcnt, off_mcnt, off_G, off_rows, off_S, off_C, off_P, off_R, off_K,
        off_hkey, off_hnode, off_hval, off_M, off_Mpre, off_MV, total;
};

static void make_num_layout(const Bands &g, const Layout &band, NumLayout *N)
{
    N->band = band;
    N->band_ws = align256(band.total);
    N->wpb = g.band_px / 64 + 1;
    int64_t cap = 1024;
    while (cap < 2 * g.nseam) cap *= 2;
    N->cap = cap;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t nb = (size_t)g.nb, ns = (size_t)g.nseam;
    // band 0's workspace comes first, so its error word is the workspace's;
    // the last band may be shorter
    Layout last;
    make_layout(1, g.H - (g.nb - 1) * g.hb, g.W, &last);  // fits: no taller than a full band
    N->off_bands = take((nb - 1) * N->band_ws + last.total);
    N->off_bandcnt = take(nb * sizeof(int32_t));
    N->off_mcnt = take(nb * sizeof(int32_t));
    N->off_G = take(nb * sizeof(int64_t));
    N->off_rows = take((nb - 1) * 2 * TH * (size_t)g.W * sizeof(int32_t));
    N->off_S = take(ns * sizeof(int32_t));
    N->off_C = take(ns * sizeof(int32_t));
    N->off_P = take(ns * sizeof(int32_t));
    N->off_R = take(ns * sizeof(int32_t));
    N->off_K = take(ns * sizeof(int64_t));
    N->off_hkey = take((size_t)cap * sizeof(int64_t));
    N->off_hnode = take((size_t)cap * sizeof(int32_t));
    N->off_hval = take((size_t)cap * sizeof(int64_t));
    N->off_M = take(nb * (size_t)N->wpb * sizeof(uint64_t));
    N->off_Mpre = take(nb * (size_t)N->wpb * sizeof(uint32_t));
    N->off_MV = take(nb * 2 * (size_t)g.W * sizeof(int64_t));
    N->total = off;
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

// ccl_label_large with CCL_NUMBER (see "numbers" above)
static int label_large_numbers(const void *colours, int dtype, int64_t batch, int connectivity,
                               int ign, uint32_t ignore, const Bands &g, const NumLayout &N,
                               int64_t *out, int64_t *counts, char *ws, hipStream_t s)
{
    int32_t *bandcnt = (int32_t *)(ws + N.off_bandcnt);
    int32_t *mcnt = (int32_t *)(ws + N.off_mcnt);
    int64_t *G = (int64_t *)(ws + N.off_G);
    int32_t *rows = (int32_t *)(ws + N.off_rows);
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
        // 1. every band through the tile pipeline in number mode
        for (int64_t k = 0; k < g.nb; ++k) {
            const Work w = band_work(k, Lb[0]);
            launch_tile(img + (size_t)(k * g.hb * g.W) * px_bytes, dtype, connectivity, ign,
                        ignore, Lb[0].g, w, b == 0 && k == 0, s);
            launch_seam(Lb[0].g, w, connectivity, s);
            launch_seam_roots(Lb[0].g, w, s);
            launch_scan(Lb[0].g, w, bandcnt + k, 1, 1, s);
            launch_resolve(Lb[0].g, w, 1, s);
        }
        if (g.nb > 1) {
            // 2. the band-local numbers of the tile rows either side of each
            //    seam: band s's last (whole: bands hold a multiple of 64 rows)
            //    and band s+1's first
            for (int64_t sm = 0; sm + 1 < g.nb; ++sm) {
                int32_t *top = rows + sm * 2 * TH * g.W, *bot = top + TH * g.W;
                const Work wa = band_work(sm, Lb[0]);
                const uint32_t lastrow = (uint32_t)(Lb[0].g.nty - 1) * (uint32_t)Lb[0].g.ntx;
                launch_final(Lb[0].g, wa, top - (int64_t)(Lb[0].g.nty - 1) * TH * g.W, 1, 0u, s,
                             lastrow, (uint32_t)Lb[0].g.ntx);
                const Work wb = band_work(sm + 1, Lb[1]);
                launch_final(Lb[1].g, wb, bot, 1, 0u, s, 0u, (uint32_t)Lb[1].g.ntx);
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
            hipLaunchKernelGGL(nm_rootval_kernel, dim3(gs), dim3(LB), 0, s, g, rows, C, R, S, N.wpb,
                               M, Mpre, G, hval);
            hipLaunchKernelGGL(nm_mergedval_kernel, dim3(gs), dim3(LB), 0, s, g, rows, C, R, S,
                               N.wpb, M, Mpre, hval, MV);
        }
        // 5. 64-bit numbers, band by band, from the bands' records
        for (int64_t k = 0; k < g.nb; ++k) {
            const Work w = band_work(k, Lb[0]);
            Map64 m;
            m.M = M + k * N.wpb;
            m.Mpre = Mpre + k * N.wpb;
            m.MV = MV + k * 2 * g.W;
            m.G = G;
            m.band = (uint32_t)k;
            m.merges = g.nb > 1;
            launch_final64(Lb[0].g, w, out + b * g.HW + k * g.band_px, m, s);
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
    NumLayout N;
    make_num_layout(L.g, L.band, &N);
    return L.total > N.total ? L.total : N.total;  // leaders or numbers
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
    NumLayout N;
    make_num_layout(L.g, L.band, &N);
    if (workspace_bytes < (L.total > N.total ? L.total : N.total)) return CCL_ERR_WORKSPACE;
    if (flags & CCL_NUMBER)
        return label_large_numbers(colours, dtype, batch, connectivity, ign, ignore, L.g, N, out,
                                   counts, (char *)workspace, (hipStream_t)stream);
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
    int64_t *chunk = (int64_t *)(ws + L.off_chunk);
    const int64_t nchunk = (g.nblk + CHUNK - 1) / CHUNK;
    uint32_t *err = (uint32_t *)ws;  // the band workspace's error word
    const bool need_scan = counts != nullptr;  // (leaders here: numbers went above)
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
            // the first band's tile pass clears the error word for the whole call
            launch_tile(img + (size_t)(r0 * g.W) * px_bytes, dtype, connectivity, ign, ignore,
                        Lb.g, w, b == 0 && k == 0, s);
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
        const unsigned gblk = (unsigned)(g.nblk < (1 << 22) ? g.nblk : (1 << 22));
        if (need_scan) {
            hipLaunchKernelGGL(flag_kernel, dim3(gblk), dim3(LB), 0, s, g, lead, rootkey, mask,
                               wordin, blkcnt);
            hipLaunchKernelGGL(chunk_scan_kernel, dim3((unsigned)nchunk), dim3(SCAN_T), 0, s,
                               blkcnt, g.nblk, blkpre, chunk);
            hipLaunchKernelGGL(chunk_total_scan_kernel, dim3(1), dim3(SCAN_T), 0, s, chunk, nchunk,
                               blkpre + g.nblk, counts ? counts + b : (int64_t *)nullptr);
            if (nchunk > 1)
                hipLaunchKernelGGL(chunk_add_kernel, dim3(grid_for(g.nblk, INT32_MAX)), dim3(LB),
                                   0, s, blkpre, g.nblk, chunk);
        }
        // 5. 64-bit leaders
        int64_t *o = out + b * g.HW;
        const int o16 = ((uintptr_t)o & 15u) == 0;  // 16-byte stores where aligned
        hipLaunchKernelGGL(final_kernel, dim3(gblk), dim3(LB), 0, s, g, lead, rootkey, o, o16);
    }
    return hipGetLastError() == hipSuccess ? CCL_OK : CCL_ERR_HIP;
}

}  // extern "C"
