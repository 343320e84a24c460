// ccl_kernels.hip -- gfx950 kernels of the tiled union-find labeller.
//
// The four stages of "Accountable AI starts at the pixel" (ch.05 "Start,
// Connect, Collapse, Number"), mapped onto 64x32 tiles:
//
//   tile_label_kernel     Start + Connect + Collapse inside one tile, in LDS.
//                         Start groups each tile row into runs of one colour by
//                         a wave64 ballot (ch.08 idea 1, "Let the warp find the
//                         runs"); Connect joins each run to the runs of the row
//                         above only where no other join already covers the
//                         pair (ch.08 idea 2, "Skip joins someone else makes"),
//                         row above first (ch.08 "the order of the joins"),
//                         with an atomic minimum that re-points the larger
//                         leader at the smaller and retries when it lost a race
//                         (ch.06 "Two workers, one leader"; the Union routine of
//                         "About Connected Components Labeling on GPU", section
//                         "Block-based Union-Find") and path halving (ch.08
//                         idea 3).  Regions that touch a tile edge get a seam
//                         node; the joins across the tile's top and left edges
//                         are written as requests.
//   seam_merge_kernel     the requests: global atomic-min unions of seam nodes,
//                         keyed by the reading-order index of each node's pixel.
//   seam_collapse_kernel  every seam node points straight at its leader (ch.05
//                         Collapse); surviving leaders are counted per row
//                         segment for Number.
//   scan_*_kernel         exclusive prefix of leaders per 64-px row segment in
//                         reading order, per image (the prefix sum in the
//                         middle of Number, ch.12 "The call").
//   final_write_kernel    each pixel gets its leader or 1 + the leaders before
//                         it (ch.08 idea 5), written once, coalesced.
//
// Standalone ccl_number / ccl_count use leader_flag_kernel (one wave64 ballot
// per row segment), the same scan, and leader_assign_kernel.
#include "ccl_internal.h"

namespace ccl {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint64_t mask_lt(int lane) { return (1ull << lane) - 1ull; }

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

// Map workgroup ids to tiles so that each XCD (workgroups are dealt to the 8
// XCDs round-robin) works on one contiguous range of tiles: neighbouring
// tiles then share that XCD's L2.
__device__ __forceinline__ int64_t remap_tile(int64_t bid, int64_t n)
{
    const int64_t q = n >> 3, r = n & 7;
    const int64_t j = bid & 7, i = bid >> 3;
    return j * q + (j < r ? j : r) + i;
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f)
{
    return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}

__device__ __forceinline__ void set_err(uint32_t *err, uint32_t bit)
{
    __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// exclusive prefix over the workgroup; `total` receives the sum of all values
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *sWave, uint32_t &total)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) sWave[wave] = x;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) {
        const uint32_t s = sWave[i];
        off += (i < wave) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

// ------------------------------------------------------- union-find in LDS
// Parents point only at smaller run ids; a root points at itself.

// Every find/union carries a step budget: a correct forest never comes near
// it (tile chains are shorter than a tile's runs, and halving keeps seam chains
// short); if it is ever exhausted the call stops early and flags ERR_LOOP in
// the workspace error word instead of spinning.
constexpr int LDS_BUDGET = 1 << 16;
constexpr int GLOBAL_BUDGET = 1 << 22;

__device__ __forceinline__ uint32_t lds_load(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ uint32_t lds_find(uint32_t *P, uint32_t x, int &budget)
{
    while (budget-- > 0) {
        const uint32_t p = lds_load(&P[x]);
        if (p == x) return x;
        const uint32_t g = lds_load(&P[p]);
        if (g == p) return p;
        atomicMin(&P[x], g);  // path halving: an arrow only moves closer to the root
        x = g;
    }
    return x;
}

__device__ void lds_unite(uint32_t *P, uint32_t a, uint32_t b, uint32_t *err)
{
    int budget = LDS_BUDGET;
    while (budget > 0) {
        a = lds_find(P, a, budget);
        b = lds_find(P, b, budget);
        if (budget <= 0) break;
        if (a == b) return;
        if (a > b) {
            const uint32_t t = a;
            a = b;
            b = t;
        }
        const uint32_t old = atomicMin(&P[b], a);  // re-point the larger root at the smaller
        if (old == b) return;                      // b was still a root: joined
        b = old;                                   // someone re-pointed b first: retry
        --budget;
    }
    set_err(err, ERR_LOOP);
}

__device__ uint32_t lds_root(uint32_t *P, uint32_t x, uint32_t *err)
{
    int budget = LDS_BUDGET;
    const uint32_t r = lds_find(P, x, budget);
    if (budget <= 0) set_err(err, ERR_LOOP);
    return r;
}

// --------------------------------------------------- union-find in global
// Seam node record: (reading-order key of the parent's pixel << 32) | parent
// node id.  A root's record holds its own key and id, and the 64-bit minimum
// orders records by key, so joins always keep the earlier pixel as leader.

__device__ __forceinline__ uint64_t g_load(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t g_min(uint64_t *p, uint64_t v)
{
    return __hip_atomic_fetch_min(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ uint32_t g_find(uint64_t *gp, uint32_t x, uint64_t &root_rec, int &budget)
{
    uint64_t rec = g_load(&gp[x]);
    while (budget-- > 0) {
        const uint32_t p = (uint32_t)rec;
        if (p == x) break;
        const uint64_t prec = g_load(&gp[p]);
        if ((uint32_t)prec == p) {
            x = p;
            rec = prec;
            break;
        }
        g_min(&gp[x], prec);  // path halving
        x = (uint32_t)prec;
        rec = g_load(&gp[x]);
    }
    root_rec = rec;
    return x;
}

__device__ void g_unite(uint64_t *gp, uint32_t a, uint32_t b, uint32_t *err)
{
    int budget = GLOBAL_BUDGET;
    while (budget > 0) {
        uint64_t ra_rec, rb_rec;
        const uint32_t ra = g_find(gp, a, ra_rec, budget);
        const uint32_t rb = g_find(gp, b, rb_rec, budget);
        if (budget <= 0) break;
        if (ra == rb) return;
        uint32_t lo = ra, hi = rb;
        uint64_t lo_rec = ra_rec, hi_rec = rb_rec;
        if (ra_rec > rb_rec) {
            lo = rb; hi = ra;
            lo_rec = rb_rec; hi_rec = ra_rec;
        }
        const uint64_t old = g_min(&gp[hi], lo_rec);
        if (old == hi_rec) return;  // hi was still a root: joined
        // hi had just been joined elsewhere (to old's node), and the minimum may
        // have moved it under lo: join lo with that node so neither join is lost
        a = lo;
        b = (uint32_t)old;
        --budget;
    }
    set_err(err, ERR_LOOP);
}

__device__ uint32_t g_root(uint64_t *gp, uint32_t x, uint64_t &root_rec, uint32_t *err)
{
    int budget = GLOBAL_BUDGET;
    const uint32_t r = g_find(gp, x, root_rec, budget);
    if (budget <= 0) set_err(err, ERR_LOOP);
    return r;
}

// ------------------------------------------------------------- tile pass

template <typename T, int CONN>
__global__ __launch_bounds__(BLOCK) void tile_label_kernel(const T *__restrict__ img, Geom g,
                                                           Work w)
{
    __shared__ uint32_t sP[TPX];          // run parents
    __shared__ uint32_t sStart[TPX];      // run start: row << 6 | col
    __shared__ uint16_t sNb[TPX + 1];     // final (non-border) roots before each run
    __shared__ uint8_t sFs[TPX];          // border flag, then seam slot (0xFF: none)
    __shared__ uint32_t sRowBase[TH + 1];
    __shared__ uint32_t sRowCnt[TH];
    __shared__ uint32_t sXcol[NWAVES][TW];   // colours of each wave's last row
    __shared__ uint32_t sXrid[NWAVES][TW];   // run ids of each wave's last row
    __shared__ uint32_t sColC[TH];           // colour at column 0 of each row
    __shared__ uint32_t sHalo[TH];           // colour left of column 0 of each row
    __shared__ uint32_t sWave[NWAVES];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int64_t t = remap_tile(blockIdx.x, g.ntiles);
    const int64_t b = t / g.tpi;
    const int64_t tt = t - b * g.tpi;
    const int ty = (int)(tt / g.ntx), tx = (int)(tt - (int64_t)ty * g.ntx);
    const int64_t y0 = (int64_t)ty * TH, x0 = (int64_t)tx * TW;
    const int vh = (int)(g.H - y0 < TH ? g.H - y0 : TH);
    const int vw = (int)(g.W - x0 < TW ? g.W - x0 : TW);
    const bool has_top = ty > 0, has_left = tx > 0;
    const bool has_bottom = y0 + TH < g.H, has_right = x0 + TW < g.W;
    const int64_t W = g.W;
    const T *im = img + b * g.HW;
    const bool lane_ok = lane < vw;
    const uint64_t lt = mask_lt(lane);

    // ---- load the tile (one coalesced row per wave instruction) and halos
    uint32_t c[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int y = wave * RPW + i;
        c[i] = (lane_ok && y < vh) ? (uint32_t)im[(y0 + y) * W + x0 + lane] : 0u;
    }
    uint32_t hrow = 0, hm1 = 0, hp1 = 0;  // row above: (y0-1, x0+lane), (y0-1, x0-1), (y0-1, x0+TW)
    if (wave == 0 && has_top) {
        const T *up = im + (y0 - 1) * W + x0;
        if (lane_ok) hrow = up[lane];
        if (lane == 0 && has_left) hm1 = up[-1];
        if (lane == TW - 1 && has_right) hp1 = up[TW];
    }
    if (wave == 1 && has_left && lane < vh) sHalo[lane] = im[(y0 + lane) * W + x0 - 1];

    // ---- Start: runs of one colour along each tile row, by ballot
    uint64_t m[RPW];
    uint32_t k[RPW];
    bool st[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int y = wave * RPW + i;
        const bool valid = lane_ok && y < vh;
        const uint32_t left = __shfl_up(c[i], 1);
        st[i] = valid && (lane == 0 || left != c[i]);
        m[i] = __ballot(st[i]);
        k[i] = popc64(m[i] & lt) + (st[i] ? 0u : 0xFFFFFFFFu);  // run index within the row
        if (lane == 0) {
            sRowCnt[y] = popc64(m[i]);
            sColC[y] = c[i];
            w.runmask[t * TH + y] = m[i];  // rows past the image edge store 0
        }
    }
    sXcol[wave][lane] = c[RPW - 1];
    __syncthreads();

    // row bases: exclusive prefix of the run counts (every wave computes it)
    uint32_t rc = lane < TH ? sRowCnt[lane] : 0u;
    const uint32_t own = rc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t v = __shfl_up(rc, d);
        if (lane >= d) rc += v;
    }
    const uint32_t R = __shfl(rc, TH - 1);
    const uint32_t rex = rc - own;
    if (wave == 0 && lane < TH) sRowBase[lane] = rex;
    if (wave == 0 && lane == 0) sRowBase[TH] = R;

    uint32_t rid[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        rid[i] = __shfl(rex, wave * RPW + i) + k[i];
        if (st[i]) {
            sP[rid[i]] = rid[i];
            sStart[rid[i]] = (uint32_t)((wave * RPW + i) << 6 | lane);
            sFs[rid[i]] = 0;
        }
    }
    sXrid[wave][lane] = rid[RPW - 1];
    __syncthreads();

    // ---- Connect inside the tile, row above first
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int y = wave * RPW + i;
        uint32_t ac = 0, ar = 0;
        if (i > 0) {
            ac = c[i - 1];
            ar = rid[i - 1];
        } else if (wave > 0) {
            ac = sXcol[wave - 1][lane];
            ar = sXrid[wave - 1][lane];
        }
        const uint32_t acm = __shfl_up(ac, 1), acp = __shfl_down(ac, 1);
        const uint32_t arm = __shfl_up(ar, 1), arp = __shfl_down(ar, 1);
        if (y >= 1 && y < vh && lane_ok) {
            const uint32_t cur = c[i];
            const bool um1 = lane >= 1 && acm == cur;
            const bool u0 = ac == cur;
            const bool up1 = lane + 1 < vw && acp == cur;
            if (CONN == 8) {
                if (up1 && !u0) lds_unite(sP, rid[i], arp, w.err);
                if (st[i]) {
                    if (um1) lds_unite(sP, rid[i], arm, w.err);
                    else if (u0) lds_unite(sP, rid[i], ar, w.err);
                }
            } else {
                if (u0 && (st[i] || !um1)) lds_unite(sP, rid[i], ar, w.err);
            }
        }
    }
    __syncthreads();

    // ---- Collapse inside the tile
    for (uint32_t r = tid; r < R; r += BLOCK) {
        const uint32_t root = lds_root(sP, r, w.err);
        atomicMin(&sP[r], root);
    }
    __syncthreads();

    // ---- roots of regions touching an edge that has a neighbour tile
    if (tid < TW) {
        const uint32_t r = sRowBase[0] + tid;
        if (has_top && r < sRowBase[1]) sFs[sP[r]] = 1;
    } else if (tid < 2 * TW) {
        const uint32_t r = sRowBase[TH - 1] + (tid - TW);
        if (has_bottom && r < sRowBase[TH]) sFs[sP[r]] = 1;
    } else if (tid < 2 * TW + TH) {
        const int y = tid - 2 * TW;
        if (has_left && y < vh) sFs[sP[sRowBase[y]]] = 1;
    } else if (tid < 2 * TW + 2 * TH) {
        const int y = tid - 2 * TW - TH;
        if (has_right && y < vh) sFs[sP[sRowBase[y + 1] - 1]] = 1;
    }
    __syncthreads();

    // ---- seam slots of border roots, ranks of the other roots (run order)
    {
        const uint32_t r0 = (uint32_t)tid * 8;
        uint32_t nb = 0, bd = 0, kinds = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t r = r0 + j;
            if (r < R && sP[r] == r) {
                if (sFs[r]) {
                    ++bd;
                    kinds |= 2u << (2 * j);
                } else {
                    ++nb;
                    kinds |= 1u << (2 * j);
                }
            }
        }
        uint32_t total;
        const uint32_t base = block_exclusive_scan((nb << 16) | bd, sWave, total);
        uint32_t run_nb = base >> 16, run_bd = base & 0xFFFFu;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t r = r0 + j;
            if (r < R) {
                sNb[r] = (uint16_t)run_nb;
                const uint32_t kd = (kinds >> (2 * j)) & 3u;
                if (kd == 2) {
                    sFs[r] = (uint8_t)(run_bd < KMAX ? run_bd : KMAX - 1);
                    ++run_bd;
                } else if (kd == 1) {
                    sFs[r] = 0xFF;
                    ++run_nb;
                }
            }
        }
        if (tid == 0) {
            sNb[R] = (uint16_t)(total >> 16);
            const uint32_t nnodes = total & 0xFFFFu;
            if (nnodes > KMAX) set_err(w.err, ERR_SLOTS);
            w.hdr[t].nruns = R;
            w.hdr[t].nnodes = nnodes < KMAX ? nnodes : KMAX;
        }
    }
    __syncthreads();

    // ---- per-run records, seam nodes, segment counts, edge slots
    uint32_t *rinfo = w.runinfo + t * TPX;
    for (uint32_t r = tid; r < R; r += BLOCK) {
        const uint32_t root = sP[r];
        const uint32_t s0 = sStart[root];
        const uint32_t fs = sFs[root];
        const uint32_t rank = (uint32_t)sNb[root] - (uint32_t)sNb[sRowBase[s0 >> 6]];
        rinfo[r] = fs != 0xFF ? (INFO_BORDER | fs) : ((rank << 11) | s0);
        if (root == r && fs != 0xFF) {
            const uint32_t node = (uint32_t)(t * KMAX) + fs;
            const uint64_t key = (uint64_t)((y0 + (s0 >> 6)) * W + x0 + (s0 & 63));
            w.gp[node] = (key << 32) | node;
            w.aux[node] = ((s0 >> 6) << 8) | rank;
        }
    }
    if (tid < vh)
        w.seg[(b * g.H + y0 + tid) * g.ntx + tx] =
            (uint32_t)sNb[sRowBase[tid + 1]] - (uint32_t)sNb[sRowBase[tid]];
    if (has_bottom && wave == NWAVES - 1 && lane_ok)
        w.bslot[t * TW + lane] = sFs[sP[rid[RPW - 1]]];
    if (has_right && tid >= TW && tid < TW + TH && tid - TW < vh)
        w.rslot[t * TH + (tid - TW)] = sFs[sP[sRowBase[tid - TW + 1] - 1]];

    // ---- seam requests across the top edge (wave 0: tile row 0 against the row above)
    if (wave == 0) {
        uint32_t ntop = 0;
        if (has_top) {
            const uint32_t cur = c[0];
            const uint32_t hl = __shfl_up(hrow, 1), hr = __shfl_down(hrow, 1);
            const bool vm1 = lane >= 1 || has_left;
            const uint32_t cm1 = lane >= 1 ? hl : hm1;
            const bool vp1 = lane < TW - 1 ? lane + 1 < vw : has_right;
            const uint32_t cp1 = lane < TW - 1 ? hr : hp1;
            const bool um1 = lane_ok && vm1 && cm1 == cur;
            const bool u0 = lane_ok && hrow == cur;
            const bool up1 = lane_ok && vp1 && cp1 == cur;
            bool ra = false, rb = false;
            int xb = lane;
            if (CONN == 8) {
                ra = up1 && !u0;
                if (st[0]) {
                    if (um1) {
                        rb = true;
                        xb = lane - 1;
                    } else if (u0) {
                        rb = true;
                    }
                }
            } else {
                rb = u0 && (st[0] || !um1);
            }
            const uint64_t ba = __ballot(ra), bb = __ballot(rb);
            const uint32_t pos = popc64(ba & lt) + popc64(bb & lt);
            if (ra || rb) {
                const uint32_t me = sFs[sP[rid[0]]];
                uint16_t *q = w.req + t * REQMAX;
                if (rb) q[pos] = (uint16_t)(me | ((uint32_t)(xb + 1) << 8));
                if (ra) q[pos + (rb ? 1 : 0)] = (uint16_t)(me | ((uint32_t)(lane + 2) << 8));
            }
            ntop = popc64(ba) + popc64(bb);
        }
        if (lane == 0) w.hdr[t].ntop = ntop;
    }

    // ---- seam requests across the left edge (wave 1: one lane per tile row)
    if (wave == 1) {
        uint32_t nleft = 0;
        if (has_left) {
            const int y = lane;
            const bool valid = y < vh;
            const uint32_t cur = valid ? sColC[y] : 0u;
            const uint32_t h = valid ? sHalo[y] : 0u;
            const bool ml = valid && h == cur;
            const bool up_ok = valid && y >= 1;
            const bool dn_ok = valid && y + 1 < vh;
            const uint32_t cu = up_ok ? sColC[y - 1] : 0u, hu = up_ok ? sHalo[y - 1] : 0u;
            const uint32_t cd = dn_ok ? sColC[y + 1] : 0u, hd = dn_ok ? sHalo[y + 1] : 0u;
            const bool up_same = up_ok && cu == cur;
            const bool rl = ml && !(up_same && hu == cur);
            bool rul = false, rdl = false;
            if (CONN == 8) {
                rul = up_ok && hu == cur && !up_same && !(ml && h == hu);
                rdl = dn_ok && hd == cur && cd != cur && !(ml && h == hd);
            }
            const uint64_t bu = __ballot(rul), bl = __ballot(rl), bdl = __ballot(rdl);
            uint32_t pos = popc64(bu & lt) + popc64(bl & lt) + popc64(bdl & lt);
            if (rul || rl || rdl) {
                const uint32_t me = sFs[sP[sRowBase[y]]];
                uint16_t *q = w.req + t * REQMAX + REQ_TOP;
                if (rul) q[pos++] = (uint16_t)(me | ((0x80u | (uint32_t)(y - 1)) << 8));
                if (rl) q[pos++] = (uint16_t)(me | ((0x80u | (uint32_t)y) << 8));
                if (rdl) q[pos++] = (uint16_t)(me | ((0x80u | (uint32_t)(y + 1)) << 8));
            }
            nleft = popc64(bu) + popc64(bl) + popc64(bdl);
        }
        if (lane == 0) w.hdr[t].nleft = nleft;
    }
}

// ------------------------------------------------------------ seam merge
// One wave per tile resolves its requests to seam nodes of the neighbour
// tiles and joins them; a request equal to the previous lane's is skipped.

__global__ __launch_bounds__(BLOCK) void seam_merge_kernel(Geom g, Work w)
{
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * NWAVES + (threadIdx.x >> 6);
    if (t >= g.ntiles) return;
    const TileHdr h = w.hdr[t];
    const uint16_t *q = w.req + t * REQMAX;
    const uint32_t mine = (uint32_t)(t * KMAX);
    for (uint32_t base = 0; base < h.ntop; base += 64) {
        const uint32_t i = base + lane;
        const bool active = i < h.ntop;
        uint32_t a = 0xFFFFFFFFu, bn = 0xFFFFFFFFu;
        if (active) {
            const uint32_t rq = q[i];
            const int xp = (int)(rq >> 8) - 1;
            int64_t tn;
            int col;
            if (xp < 0) {
                tn = t - g.ntx - 1;
                col = TW - 1;
            } else if (xp >= TW) {
                tn = t - g.ntx + 1;
                col = 0;
            } else {
                tn = t - g.ntx;
                col = xp;
            }
            a = mine + (rq & 0xFFu);
            bn = (uint32_t)(tn * KMAX) + w.bslot[tn * TW + col];
        }
        const uint32_t pa = __shfl_up(a, 1), pb = __shfl_up(bn, 1);
        const bool dup = lane > 0 && pa == a && pb == bn;
        if (active && !dup) g_unite(w.gp, a, bn, w.err);
    }
    for (uint32_t base = 0; base < h.nleft; base += 64) {
        const uint32_t i = base + lane;
        const bool active = i < h.nleft;
        uint32_t a = 0xFFFFFFFFu, bn = 0xFFFFFFFFu;
        if (active) {
            const uint32_t rq = q[REQ_TOP + i];
            const int64_t tn = t - 1;
            a = mine + (rq & 0xFFu);
            bn = (uint32_t)(tn * KMAX) + w.rslot[tn * TH + ((rq >> 8) & 0x7Fu)];
        }
        const uint32_t pa = __shfl_up(a, 1), pb = __shfl_up(bn, 1);
        const bool dup = lane > 0 && pa == a && pb == bn;
        if (active && !dup) g_unite(w.gp, a, bn, w.err);
    }
}

// ---------------------------------------------------------- seam collapse
// One wave per tile: each seam node points straight at its leader; a node that
// is its own leader is a leader of the whole image: it is counted in its row
// segment and gets its rank among that segment's leaders.

__global__ __launch_bounds__(BLOCK) void seam_collapse_kernel(Geom g, Work w, int count_survivors)
{
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * NWAVES + (threadIdx.x >> 6);
    if (t >= g.ntiles) return;
    const uint32_t k = w.hdr[t].nnodes;
    if (k == 0) return;
    const int64_t b = t / g.tpi;
    const int64_t tt = t - b * g.tpi;
    const int ty = (int)(tt / g.ntx), tx = (int)(tt - (int64_t)ty * g.ntx);
    const int64_t y0 = (int64_t)ty * TH;
    const uint64_t lt = mask_lt(lane);
    uint32_t carry_row = 0xFFFFFFFFu, carry_cnt = 0;
    for (uint32_t base = 0; base < k; base += 64) {
        const uint32_t s = base + lane;
        const bool active = s < k;
        const uint32_t n = (uint32_t)(t * KMAX) + s;
        bool surv = false;
        uint32_t row = 0xFFFFFFFEu, a = 0;
        if (active) {
            uint64_t rrec;
            const uint32_t root = g_root(w.gp, n, rrec, w.err);
            g_min(&w.gp[n], rrec);
            surv = root == n;
            a = w.aux[n];
            row = a >> 8;
        }
        if (!count_survivors) continue;
        // survivors before this lane in the same tile row (slots are in row order)
        const uint64_t sb = __ballot(active && surv);
        const uint32_t prow = __shfl_up(row, 1);
        const uint64_t nb = __ballot(active && (lane == 0 || prow != row));
        const uint64_t le = nb & (lt | (1ull << lane));
        const int rs = 63 - __clzll(le | 1ull);  // first lane of my row in this chunk
        uint32_t cnt = popc64(sb & lt & ~mask_lt(rs));
        if (rs == 0 && row == carry_row) cnt += carry_cnt;
        if (active && surv) {
            w.aux[n] = (a & 0xFFu) + cnt;
            atomicAdd(&w.seg[(b * g.H + y0 + row) * g.ntx + tx], 1u);
        }
        const int last = (int)(k - 1 - base < 63 ? k - 1 - base : 63);
        const uint32_t lrow = __shfl(row, last);
        const uint32_t lcnt = __shfl(cnt, last) + (__shfl(surv ? 1u : 0u, last));
        carry_row = lrow;
        carry_cnt = lcnt;
    }
}

// ------------------------------------------------------------------ scan
// seg[] holds, per image, the leaders of each 64-px row segment in reading
// order; it is replaced in place by the exclusive prefix, per image.

__global__ __launch_bounds__(BLOCK) void scan_reduce_kernel(Geom g, Work w)
{
    __shared__ uint32_t sWave[NWAVES];
    const int64_t c = blockIdx.x;
    const int64_t b = c / g.cpi, cc = c - b * g.cpi;
    const int64_t img_end = (b + 1) * g.H * g.ntx;
    const int64_t base = b * g.H * g.ntx + cc * SCAN_CHUNK + (int64_t)threadIdx.x * SCAN_PT;
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < SCAN_PT; ++j)
        if (base + j < img_end) sum += w.seg[base + j];
    uint32_t total;
    block_exclusive_scan(sum, sWave, total);
    if (threadIdx.x == 0) w.chunk[c] = total;
}

__global__ __launch_bounds__(BLOCK) void scan_chunks_kernel(Geom g, Work w, int32_t *counts)
{
    __shared__ uint32_t sWave[NWAVES];
    const int64_t b = blockIdx.x;
    uint32_t carry = 0;
    for (int64_t base = 0; base < g.cpi; base += BLOCK) {
        const int64_t i = base + threadIdx.x;
        const uint32_t v = i < g.cpi ? w.chunk[b * g.cpi + i] : 0u;
        uint32_t total;
        const uint32_t ex = block_exclusive_scan(v, sWave, total);
        if (i < g.cpi) w.chunk[b * g.cpi + i] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0 && counts) counts[b] = (int32_t)carry;
}

__global__ __launch_bounds__(BLOCK) void scan_apply_kernel(Geom g, Work w)
{
    __shared__ uint32_t sWave[NWAVES];
    const int64_t c = blockIdx.x;
    const int64_t b = c / g.cpi, cc = c - b * g.cpi;
    const int64_t img_end = (b + 1) * g.H * g.ntx;
    const int64_t base = b * g.H * g.ntx + cc * SCAN_CHUNK + (int64_t)threadIdx.x * SCAN_PT;
    uint32_t v[SCAN_PT];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < SCAN_PT; ++j) {
        v[j] = base + j < img_end ? w.seg[base + j] : 0u;
        sum += v[j];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan(sum, sWave, total) + w.chunk[c];
#pragma unroll
    for (int j = 0; j < SCAN_PT; ++j) {
        if (base + j < img_end) w.seg[base + j] = run;
        run += v[j];
    }
}

// ----------------------------------------------------------- final write

__global__ __launch_bounds__(BLOCK) void final_write_kernel(Geom g, Work w, int32_t *out,
                                                            int number)
{
    __shared__ uint32_t sLab[TPX];
    __shared__ uint32_t sSlotLab[KMAX];
    __shared__ uint64_t sSurv[TH];
    __shared__ uint32_t sPrefix[TH];

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int64_t t = remap_tile(blockIdx.x, g.ntiles);
    const int64_t b = t / g.tpi;
    const int64_t tt = t - b * g.tpi;
    const int ty = (int)(tt / g.ntx), tx = (int)(tt - (int64_t)ty * g.ntx);
    const int64_t y0 = (int64_t)ty * TH, x0 = (int64_t)tx * TW;
    const int vh = (int)(g.H - y0 < TH ? g.H - y0 : TH);
    const int vw = (int)(g.W - x0 < TW ? g.W - x0 : TW);
    const int64_t W = g.W;
    const TileHdr h = w.hdr[t];
    const uint32_t R = h.nruns, k = h.nnodes;

    // run starts of this wave's rows and their run bases
    const uint64_t mk = lane < TH ? w.runmask[t * TH + lane] : 0ull;
    const uint32_t cnt = popc64(mk);
    uint32_t inc = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t v = __shfl_up(inc, d);
        if (lane >= d) inc += v;
    }
    const uint32_t ex = inc - cnt;
    uint64_t rm[RPW];
    uint32_t rb[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        rm[i] = __shfl(mk, wave * RPW + i);
        rb[i] = __shfl(ex, wave * RPW + i);
    }
    if (tid < TH) {
        sSurv[tid] = 0;
        sPrefix[tid] = (number && tid < vh) ? w.seg[(b * g.H + y0 + tid) * g.ntx + tx] : 0u;
    }
    __syncthreads();
    if ((uint32_t)tid < k) {
        const uint32_t n = (uint32_t)(t * KMAX) + tid;
        const uint64_t rec = w.gp[n];
        const uint32_t L = (uint32_t)rec;
        const uint32_t key = (uint32_t)(rec >> 32);
        const uint32_t Y = fast_div(key, g.divW);
        const uint32_t X = key - Y * (uint32_t)W;
        if (L == n)
            atomicOr((unsigned long long *)&sSurv[Y - y0], 1ull << (X - x0));
        uint32_t lab = key;
        if (number)
            lab = 1u + w.seg[(b * g.H + Y) * g.ntx + (X >> 6)] + w.aux[L];
        sSlotLab[tid] = lab;
    }
    __syncthreads();
    const uint32_t *rinfo = w.runinfo + t * TPX;
    for (uint32_t r = tid; r < R; r += BLOCK) {
        const uint32_t info = rinfo[r];
        uint32_t lab;
        if (info & INFO_BORDER) {
            lab = sSlotLab[info & 0xFFu];
        } else {
            const uint32_t row = (info >> 6) & 31u, col = info & 63u;
            if (number)
                lab = 1u + sPrefix[row] + ((info >> 11) & 63u) +
                      popc64(sSurv[row] & mask_lt((int)col));
            else
                lab = (uint32_t)((y0 + row) * W + x0 + col);
        }
        sLab[r] = lab;
    }
    __syncthreads();
    int32_t *o = out + b * g.HW;
    const uint64_t lt = mask_lt(lane);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int y = wave * RPW + i;
        if (y < vh && lane < vw) {
            const uint32_t s = (uint32_t)(rm[i] >> lane) & 1u;
            const uint32_t run = rb[i] + popc64(rm[i] & lt) + s - 1u;
            o[(y0 + y) * W + x0 + lane] = (int32_t)sLab[run];
        }
    }
}

// ------------------------------------------------ standalone number/count
// Row segments of 64 pixels: one wave64 ballot of "leaders[p] == p" each.

__global__ __launch_bounds__(BLOCK) void leader_flag_kernel(const int32_t *leaders, Geom g,
                                                            Work w, int write_mask)
{
    const int lane = lane_id();
    const int64_t nw = (int64_t)gridDim.x * NWAVES;
    for (int64_t sgi = (int64_t)blockIdx.x * NWAVES + (threadIdx.x >> 6); sgi < g.nseg; sgi += nw) {
        const int64_t row = sgi / g.ntx;          // b*H + Y
        const int64_t sx = sgi - row * g.ntx;
        const int64_t Y = row % g.H;
        const int64_t x = sx * 64 + lane;
        bool root = false;
        if (x < g.W) root = (int64_t)leaders[row * g.W + x] == Y * g.W + x;
        const uint64_t m = __ballot(root);
        if (lane == 0) {
            w.seg[sgi] = popc64(m);
            if (write_mask) w.runmask[sgi] = m;
        }
    }
}

__global__ __launch_bounds__(BLOCK) void leader_assign_kernel(const int32_t *leaders,
                                                              int32_t *labels, Geom g, Work w)
{
    const int64_t nrows = g.B * g.H;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t b = row / g.H;
        const int64_t segbase = b * g.H * g.ntx;
        for (int64_t x = threadIdx.x; x < g.W; x += BLOCK) {
            const int64_t i = row * g.W + x;
            const int32_t v = leaders[i];
            int32_t lab = 0;
            if (v >= 0 && (int64_t)v < g.HW) {
                const uint32_t Y = fast_div((uint32_t)v, g.divW);
                const uint32_t X = (uint32_t)v - Y * (uint32_t)g.W;
                const int64_t sg = segbase + (int64_t)Y * g.ntx + (X >> 6);
                lab = (int32_t)(1u + w.seg[sg] + popc64(w.runmask[sg] & mask_lt((int)(X & 63u))));
            }
            labels[i] = lab;
        }
    }
}

__global__ void zero_i32_kernel(int32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// ------------------------------------------------------------- launchers

static inline unsigned grid_of(int64_t n, int64_t per)
{
    return (unsigned)((n + per - 1) / per);
}

void launch_tile(const void *img, int dtype_bytes, int conn, const Geom &g, const Work &w,
                 hipStream_t s)
{
    const dim3 grid((unsigned)g.ntiles), block(BLOCK);
    if (dtype_bytes == 1) {
        if (conn == 8)
            hipLaunchKernelGGL((tile_label_kernel<uint8_t, 8>), grid, block, 0, s,
                               (const uint8_t *)img, g, w);
        else
            hipLaunchKernelGGL((tile_label_kernel<uint8_t, 4>), grid, block, 0, s,
                               (const uint8_t *)img, g, w);
    } else {
        if (conn == 8)
            hipLaunchKernelGGL((tile_label_kernel<uint32_t, 8>), grid, block, 0, s,
                               (const uint32_t *)img, g, w);
        else
            hipLaunchKernelGGL((tile_label_kernel<uint32_t, 4>), grid, block, 0, s,
                               (const uint32_t *)img, g, w);
    }
}

void launch_seam(const Geom &g, const Work &w, hipStream_t s)
{
    hipLaunchKernelGGL(seam_merge_kernel, dim3(grid_of(g.ntiles, NWAVES)), dim3(BLOCK), 0, s, g, w);
}

void launch_seam_collapse(const Geom &g, const Work &w, int count_survivors, hipStream_t s)
{
    hipLaunchKernelGGL(seam_collapse_kernel, dim3(grid_of(g.ntiles, NWAVES)), dim3(BLOCK), 0, s,
                       g, w, count_survivors);
}

void launch_scan(const Geom &g, const Work &w, int32_t *counts, int apply, hipStream_t s)
{
    hipLaunchKernelGGL(scan_reduce_kernel, dim3((unsigned)g.nchunk), dim3(BLOCK), 0, s, g, w);
    hipLaunchKernelGGL(scan_chunks_kernel, dim3((unsigned)g.B), dim3(BLOCK), 0, s, g, w, counts);
    if (apply)
        hipLaunchKernelGGL(scan_apply_kernel, dim3((unsigned)g.nchunk), dim3(BLOCK), 0, s, g, w);
}

void launch_final(const Geom &g, const Work &w, int32_t *out, int number, hipStream_t s)
{
    hipLaunchKernelGGL(final_write_kernel, dim3((unsigned)g.ntiles), dim3(BLOCK), 0, s, g, w, out,
                       number);
}

void launch_leader_flags(const int32_t *leaders, const Geom &g, const Work &w, int write_mask,
                         hipStream_t s)
{
    int64_t blocks = grid_of(g.nseg, NWAVES);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(leader_flag_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, s, leaders, g,
                       w, write_mask);
}

void launch_leader_assign(const int32_t *leaders, int32_t *labels, const Geom &g, const Work &w,
                          hipStream_t s)
{
    int64_t blocks = g.B * g.H;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(leader_assign_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, s, leaders,
                       labels, g, w);
}

void launch_zero_i32(int32_t *p, int64_t n, hipStream_t s)
{
    int64_t blocks = grid_of(n, BLOCK);
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, s, p, n);
}

}  // namespace ccl
