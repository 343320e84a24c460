// ccl_kernels.hip -- gfx950 kernels of the tiled union-find labeller.
//
// The four stages of "Accountable AI starts at the pixel" (ch.05 "Start,
// Connect, Collapse, Number") mapped onto 64x32 tiles:
//
//   tile_label_kernel     Start + Connect + Collapse inside one tile, in LDS.
//                         Start groups each tile row into runs of one colour by
//                         a wave64 ballot (ch.08 idea 1, "Let the warp find the
//                         runs").  Connect joins each run once to every run of
//                         the row above that touches it and has its colour, so
//                         no join is made twice (ch.08 idea 2, "Skip joins
//                         someone else makes"), always against the row above
//                         (ch.08 "the order of the joins"), with an atomic
//                         minimum that re-points the larger leader at the
//                         smaller and retries when it lost a race (ch.06 "Two
//                         workers, one leader"; the Union routine of "About
//                         Connected Components Labeling on GPU", section
//                         "Block-based Union-Find") and path halving (ch.08
//                         idea 3).  Regions that touch an edge shared with
//                         another tile get a seam node; the joins across the
//                         tile's top and left edges are written as requests.
//   seam_merge_kernel     the requests: global atomic-min unions of seam nodes,
//                         ordered by the reading-order index of each node's pixel.
//   seam_roots_kernel     seam nodes that are still roots lead regions of the
//                         whole image: they are added to their row segment's
//                         leader mask and count.
//   scan_kernel           exclusive prefix of leaders per 64-px row segment in
//                         reading order, per image (the prefix sum in the middle
//                         of Number, ch.12 "The call"), one decoupled look-back
//                         pass over bands of tiles.
//   resolve_kernel        each seam node finds its leader (ch.05 Collapse) and
//                         gets the value of its pixels.
//   final_write_kernel    every pixel gets its leader or 1 + the leaders before
//                         it (ch.08 idea 5), written once, coalesced.
//
// Standalone ccl_number / ccl_count use leader_flag_kernel (one wave64 ballot
// per row segment), the same scan, and leader_assign_kernel.
#include "ccl_internal.h"

namespace ccl {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint64_t mask_lt(int lane) { return (1ull << lane) - 1ull; }

__device__ __forceinline__ uint64_t mask_le(int x) { return x >= 63 ? ~0ull : ((2ull << x) - 1ull); }

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

// value of lane-1 (lane 0 gets 0): one DPP move across the whole wave64.  A
// lane that is switched off at the call also reads as 0, so lane shifts are
// taken where every lane is active.
__device__ __forceinline__ uint32_t from_left_lane(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138 /* wave_shr:1 */, 0xF, 0xF, true);
}

// Map workgroup ids to work items so that each XCD (workgroups are dealt to the
// 8 XCDs round-robin) gets one contiguous range: neighbouring tiles then share
// that XCD's L2.  A bijection of 0..n-1.  Used where it measured faster: the
// final write and the seam passes, not the tile pass.  Never for the scan,
// whose bands wait for the bands before them and so must start in order.
__device__ __forceinline__ uint32_t remap_tile(uint32_t bid, uint32_t n)
{
    const uint32_t q = n >> 3, r = n & 7u;
    const uint32_t j = bid & 7u, i = bid >> 3;
    return j * q + (j < r ? j : r) + i;
}

// The tile pass's order: runs of TILE_RUN consecutive tiles dealt to the 8 XCDs
// in turn (workgroup ids reach the XCDs round-robin), so that the tiles of one
// stretch of the picture are spread over every XCD while three tiles in four
// find their left neighbour's pixels (their halo column) in their own L2.  A
// bijection of 0..n-1: the last n mod 8*TILE_RUN ids map to themselves.
constexpr uint32_t TILE_RUN = 4;
__device__ __forceinline__ uint32_t tile_order(uint32_t bid, uint32_t n)
{
    constexpr uint32_t G = 8 * TILE_RUN;
    if (bid >= n / G * G) return bid;
    const uint32_t i = bid >> 3;
    return i / TILE_RUN * G + (bid & 7u) * TILE_RUN + i % TILE_RUN;
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f)
{
    return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}

__device__ __forceinline__ void set_err(uint32_t *err, uint32_t bit)
{
    __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// clears the band status words before a scan (grid-stride over the threads
// of the calling kernel)
__device__ __forceinline__ void clear_bands(const Geom &g, const Work &w)
{
    const uint64_t n = (uint64_t)g.nbands;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        w.bandst[i] = 0ull;
}

// Positions inside one image are 32-bit: an image holds fewer than 2^31 pixels.
struct TilePos {
    uint32_t b, ty, tx;
    uint32_t y0, x0;  // first row and column
    int vh, vw;       // rows and columns inside the image
};

__device__ __forceinline__ TilePos tile_pos(uint32_t t, const Geom &g)
{
    TilePos p;
    p.b = fast_div(t, g.divTpi);
    const uint32_t tt = t - p.b * (uint32_t)g.tpi;
    p.ty = fast_div(tt, g.divNtx);
    p.tx = tt - p.ty * (uint32_t)g.ntx;
    p.y0 = p.ty * TH;
    p.x0 = p.tx * TW;
    const uint32_t rh = (uint32_t)g.H - p.y0, rw = (uint32_t)g.W - p.x0;
    p.vh = (int)(rh < (uint32_t)TH ? rh : (uint32_t)TH);
    p.vw = (int)(rw < (uint32_t)TW ? rw : (uint32_t)TW);
    return p;
}

// tile, row and column (inside the tile) of pixel `key` of image b
__device__ __forceinline__ void pixel_tile(uint32_t key, uint32_t b, const Geom &g, uint32_t &t,
                                           uint32_t &row, uint32_t &col)
{
    const uint32_t Y = fast_div(key, g.divW);
    const uint32_t X = key - Y * (uint32_t)g.W;
    t = b * (uint32_t)g.tpi + (Y / TH) * (uint32_t)g.ntx + X / TW;
    row = Y % TH;
    col = X % TW;
}

// ------------------------------------------------------- union-find in LDS
// Run slots are numbered y*64+k (k-th run of tile row y): reading order, so a
// smaller slot is an earlier run.  Parents only point at smaller slots; a root
// points at itself.  A root's word may also carry its seam slot in bits 16..23
// (stored as 255 - slot, so the smallest slot wins an atomic maximum).

constexpr uint32_t PMASK = 0xFFFFu;

// Loops here need no step budget: every arrow points at a smaller slot, and
// each loop below only moves to strictly smaller slots (a word that does not
// point lower counts as a root), so it ends after at most TPX steps even on a
// corrupted forest.

// SEAM: roots may carry seam bits (after Connect), so they are masked off
template <bool SEAM>
__device__ __forceinline__ uint32_t lds_parent(const uint32_t *P, uint32_t x)
{
    const uint32_t v = __hip_atomic_load(&P[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return SEAM ? v & PMASK : v;
}

// root of x, halving the path on the way (an arrow only moves closer to the root)
template <bool SEAM>
__device__ __forceinline__ uint32_t lds_find(uint32_t *P, uint32_t x)
{
    uint32_t p = lds_parent<SEAM>(P, x);
    while (p < x) {
        const uint32_t g = lds_parent<SEAM>(P, p);
        if (g < p) atomicMin(&P[x], g);
        x = p;
        p = g;
    }
    return x;
}

// join the trees of a and b (during Connect: no seam bits yet): the larger
// root is re-pointed at the smaller; if it stopped being a root meanwhile, join
// again from where it points now (the larger of the two roots strictly
// decreases each time)
__device__ __forceinline__ void lds_unite(uint32_t *P, uint32_t a, uint32_t b)
{
    for (;;) {
        a = lds_find<false>(P, a);
        b = lds_find<false>(P, b);
        if (a == b) return;
        const uint32_t lo = a < b ? a : b, hi = a ^ b ^ lo;
        const uint32_t old = atomicMin(&P[hi], lo);
        if (old >= hi) return;  // hi was still a root: joined
        a = lo;
        b = old;
    }
}

// --------------------------------------------------- union-find in global
// These loops carry a step budget: a correct forest never comes near it
// (halving keeps seam chains short); if it is ever exhausted the call stops
// early and flags ERR_LOOP in the workspace error word instead of spinning.
constexpr int GLOBAL_BUDGET = 1 << 22;

// Seam node record: (reading-order key of the parent's pixel << 32) | parent
// node id.  A root's record holds its own key and id, and the 64-bit minimum
// orders records by key, so joins always keep the earlier pixel as leader.

__device__ __forceinline__ uint64_t *node_rec(const Work &w, uint32_t node)
{
    const uint32_t t = node >> 8, slot = node & 0xFFu;
    return slot == UNI_SLOT ? &w.hdr[t].rec : w.gp + (size_t)t * KMAX + slot;
}

// A seam node's region lies in its tile alone when no union ever touched the
// node: it is still a root (its record names itself) and no other node has it
// as root (bit 63 of a root's record, set by those nodes in the resolve pass
// of the statistics; a key takes 31 bits).
constexpr uint64_t REC_SHARED = 1ull << 63;
__device__ __forceinline__ bool lone_node(uint64_t rec, uint32_t node)
{
    return (uint32_t)rec == node && !(rec & REC_SHARED);
}

__device__ __forceinline__ uint64_t g_min(uint64_t *p, uint64_t v)
{
    return __hip_atomic_fetch_min(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Finds read records with cacheable loads, which may be stale: a record only
// ever moves to a parent with a smaller key in the same region, so a stale
// record still names an ancestor, and a walk still ends (keys fall at every
// step) at a node of the same region.  During the merge such a node may have
// stopped being a root; the atomic minimum that links it returns its true
// record, and the union goes on from there (g_unite).  Once every union is
// done, roots no longer change and the walk ends at the root.
// HALVE = false walks without path halving (without re-pointing each node
// passed at its grandparent): once every union is done the walks are mostly
// a step or two long, and many of them pass the same few nodes (a block's
// root), whose records the halving's atomic minimums would then queue on.
// Measured on the 4096^2 spiral, whose two regions reach every tile, scan
// and resolve took 0.071 ms without halving against 0.085 ms with it from
// a walk's second step on, and halving only past the 2nd, 4th or 8th step
// gave 0.086-0.090 ms.
template <bool HALVE = true>
__device__ uint32_t g_find(const Work &w, uint32_t x, uint64_t &root_rec, int &budget)
{
    auto load = [&](uint32_t i) -> uint64_t { return *node_rec(w, i); };
    uint64_t rec = load(x);
    while (budget-- > 0) {
        const uint32_t p = (uint32_t)rec;
        if (p == x) break;
        const uint64_t prec = load(p);
        if ((uint32_t)prec == p) {
            x = p;
            rec = prec;
            break;
        }
        if (HALVE) g_min(node_rec(w, x), prec);  // path halving
        x = (uint32_t)prec;
        rec = load(x);
    }
    root_rec = rec;
    return x;
}

__device__ void g_unite(const Work &w, uint32_t a, uint32_t b)
{
    int budget = GLOBAL_BUDGET;
    while (budget > 0) {
        uint64_t ra_rec, rb_rec;
        const uint32_t ra = g_find(w, a, ra_rec, budget);
        const uint32_t rb = g_find(w, b, rb_rec, budget);
        if (budget <= 0) break;
        if (ra == rb) return;
        uint32_t lo = ra, hi = rb;
        uint64_t lo_rec = ra_rec, hi_rec = rb_rec;
        if (ra_rec > rb_rec) {
            lo = rb;
            hi = ra;
            lo_rec = rb_rec;
            hi_rec = ra_rec;
        }
        const uint64_t old = g_min(node_rec(w, hi), lo_rec);
        if (old == hi_rec) return;  // hi was still a root: joined
        // hi had just been joined elsewhere (to old's node), and the minimum may
        // have moved it under lo: join lo with that node so neither join is lost
        a = lo;
        b = (uint32_t)old;
        --budget;
    }
    set_err(w.err, ERR_LOOP);
}

// the root of x once every union is done
__device__ uint32_t g_root(const Work &w, uint32_t x, uint64_t &root_rec)
{
    int budget = GLOBAL_BUDGET;
    const uint32_t r = g_find<false>(w, x, root_rec, budget);
    if (budget <= 0) set_err(w.err, ERR_LOOP);
    return r;
}

// ------------------------------------------------------------- tile pass
// One workgroup per 64x32 tile; wave w holds tile rows 8w..8w+7, lane = column.
//   1 Start    a ballot per row marks run starts ("left neighbour differs");
//              start lanes initialise their run's parent and start column.  A
//              tile whose valid pixels all have one colour is finished on a
//              short path (one region, no run tables).
//   2 Connect  each run is joined once to every run of the row above that
//              touches it and has its colour.  The joins are found per pixel
//              from the row above (shifted one lane each way), so that exactly
//              one pixel of the run stands for each such pair; they are queued
//              per wave and united in LDS with every lane busy.
//   3 Collapse every run points at its tile root; a run on an edge shared with
//              another tile offers its edge position as the region's seam slot.
//   4 Write    per-run records, the leader mask and count of each row
//              segment, seam nodes, the slots of the bottom row and right
//              column, and the seam requests for the top and left edges (joins
//              with pixels of the tiles above and to the left, found from a
//              one-pixel halo).

// barrier for LDS traffic only (outstanding global stores are not waited for)
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// value of lane+1 (lane 63 gets 0)
__device__ __forceinline__ uint32_t from_right_lane(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x130 /* wave_shl:1 */, 0xF, 0xF, true);
}

// number of set bits of m below this lane
__device__ __forceinline__ uint32_t mbcnt(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// number of set bits of m below this lane, plus acc
__device__ __forceinline__ uint32_t mbcnt_acc(uint64_t m, uint32_t acc)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, acc));
}

// this lane's bit of the wave-uniform mask m (no vector instruction: the mask
// itself becomes the lane condition)
__device__ __forceinline__ bool lane_bit(uint64_t m) { return __builtin_amdgcn_inverse_ballot_w64(m); }

// a value that is the same in every lane, in scalar registers
__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
}

// v with lane i replaced by the wave-uniform value x: a plain select on the
// lane id, which the compiler sees whole (other lanes keep their values).
// Used for tile-header words built in straight-line code.
__device__ __forceinline__ uint32_t write_lane(uint32_t v, uint32_t x, int i)
{
    return lane_id() == i ? x : v;
}

constexpr int QCAP = 256;  // join queue of one wave (a ring; at most 63 + 128 pending)

// Run slots: wave w numbers the runs of its rows w*RPW*TW, w*RPW*TW + 1, ...
// in reading order, so slot order is reading order across the whole tile and
// the runs of one wave sit in consecutive LDS words.
constexpr uint32_t WAVE_SLOTS = RPW * TW;  // slots of one wave (a run per pixel at most)

template <bool IGN>
struct TileLds {
    // (each array has a tail of TW words past the run slots: lanes with
    // nothing to store write there, so the row loop stores without branching)
    uint32_t P[TPX + TW];          // parent of run slot; roots: + seam slot
    uint16_t RXY[TPX + TW];        // tile row << 8 | start column of run slot
    uint16_t RowBase[TH];          // slot of the first run of each tile row
    uint32_t WaveRuns[NWAVES];     // runs in each wave's rows
    uint32_t Q[NWAVES][QCAP];      // queued joins: slot | other slot << 16
    uint64_t Mask[TH];             // run starts of each tile row
    uint64_t Lead[TH];             // start columns of the final roots of each row
    uint32_t LastC[NWAVES - 1][TW]; // last row of waves 0..2 (the next wave's row above)
    uint32_t ColC[TH];             // colour at column 0 of each row
    uint64_t Used[KMAX / 64];
    uint64_t Uni[NWAVES];          // per wave: (one colour? << 32) | first colour
    uint64_t Ign[IGN ? TH : 1];    // with an ignored colour: its pixels in each tile row
};

// Seam requests across the top edge (wave 0, lane = column): tile row 0
// (colours cur, run starts st0, seam slot me of the lane's region) against the
// row above (hrow; hm1 / hp1 = the pixels diagonally beyond columns 0 and 63,
// held by lanes 0 and 63).  ok_m: lanes of the tile's columns.  The joins are
// found as in Connect, one request per pair of touching stretches.  Returns
// the number written.  Lanes outside keep_m (pixels of an ignored colour)
// make none.
template <int CONN>
__device__ __forceinline__ uint32_t top_requests(uint16_t *q, int lane, uint64_t ok_m, bool has_left,
                                                 bool has_right, uint32_t cur, uint64_t st0,
                                                 uint32_t me, uint32_t hrow, uint32_t hm1,
                                                 uint32_t hp1, uint64_t keep_m)
{
    const uint64_t u0 = __ballot(hrow == cur) & ok_m;
    uint64_t um1 = __ballot(from_left_lane(hrow) == cur) & ok_m & ~1ull;
    if (has_left) um1 |= __ballot(hm1 == cur) & 1ull;
    uint64_t ra = 0, rb, lu = 0;
    if (CONN == 8) {
        uint64_t up1 = __ballot(from_right_lane(hrow) == cur) & ok_m & (ok_m >> 1);
        if (has_right) up1 |= __ballot(hp1 == cur) & (1ull << 63);
        ra = up1 & ~u0;         // up-right starts a stretch of the run's colour
        rb = st0 & (um1 | u0);  // a run's first pixel also takes up-left or up
        lu = um1;
    } else {
        rb = u0 & (st0 | ~um1);
    }
    ra &= keep_m;  // lanes of an ignored colour make no requests
    rb &= keep_m;
    // requests in lane order, a lane's up-left/up one before its up-right one;
    // the byte above the slot is 1 + the column of the pixel above
    const uint32_t pos = mbcnt(ra) + mbcnt(rb);
    if (lane_bit(rb)) q[pos] = (uint16_t)(me | ((uint32_t)(lane + (lane_bit(lu) ? 0 : 1)) << 8));
    if (lane_bit(ra)) q[pos + (lane_bit(rb) ? 1u : 0u)] = (uint16_t)(me | ((uint32_t)(lane + 2) << 8));
    return popc64(ra) + popc64(rb);
}

// Seam requests across the left edge (wave 0, lane = tile row y): the pixel at
// column 0 (colour cur, seam slot me) against the halo column h (the pixel left
// of it); rows y-1 and y+1 are read from the neighbouring lanes.  vh_m: lanes
// of the tile's rows; lanes outside keep_m (an ignored colour) make none.
template <int CONN>
__device__ __forceinline__ uint32_t left_requests(uint16_t *q, int y, uint64_t vh_m, uint32_t me,
                                                  uint32_t cur, uint32_t h, uint64_t keep_m)
{
    const uint32_t hu = from_left_lane(h), hd = from_right_lane(h);
    const uint32_t cu = from_left_lane(cur), cd = from_right_lane(cur);
    const uint64_t up_ok = vh_m & ~1ull, dn_ok = vh_m & (vh_m >> 1);
    const uint64_t ml = __ballot(h == cur) & vh_m;
    const uint64_t up_same = __ballot(cu == cur) & up_ok;
    const uint64_t hu_cur = __ballot(hu == cur);
    // skip a join that the row above (or this row's left join) already makes
    const uint64_t rl = ml & ~(up_same & hu_cur) & keep_m;
    uint64_t rul = 0, rdl = 0;
    if (CONN == 8) {
        rul = up_ok & hu_cur & ~up_same & ~(ml & __ballot(h == hu)) & keep_m;
        rdl = dn_ok & __ballot(hd == cur) & ~__ballot(cd == cur) & ~(ml & __ballot(h == hd)) & keep_m;
    }
    uint32_t pos = mbcnt(rul) + mbcnt(rl) + mbcnt(rdl);
    if (lane_bit(rul)) q[pos++] = (uint16_t)(me | ((0x80u | (uint32_t)(y - 1)) << 8));
    if (lane_bit(rl)) q[pos++] = (uint16_t)(me | ((0x80u | (uint32_t)y) << 8));
    if (lane_bit(rdl)) q[pos] = (uint16_t)(me | ((0x80u | (uint32_t)(y + 1)) << 8));
    return popc64(rul) + popc64(rl) + popc64(rdl);
}

// A pixel of an RGB picture as it is stored: three bytes, any alignment.  Its
// colour value is b0 | b1 << 8 | b2 << 16 (b0 the first byte), so that pixels
// are equal exactly when all three bytes are.
struct Rgb24 {
    uint8_t b[3];
};
static_assert(sizeof(Rgb24) == 3, "three bytes per RGB pixel");

// colour value of a stored pixel
__device__ __forceinline__ uint32_t px(uint8_t v) { return v; }
__device__ __forceinline__ uint32_t px(uint32_t v) { return v; }
__device__ __forceinline__ uint32_t px(const Rgb24 &v)
{
    return (uint32_t)v.b[0] | ((uint32_t)v.b[1] << 8) | ((uint32_t)v.b[2] << 16);
}

// The pixels one wave reads for a tile: its 8 rows (lane = column) and, for
// wave 0, the halo: the row above the tile and the column to its left.
struct TileIn {
    uint32_t c[RPW];
    uint32_t hrow, hm1, hp1;  // wave 0: (y0-1, x0+lane), (y0-1, x0-1), (y0-1, x0+TW)
    uint32_t hleft;           // wave 0: (y0+lane, x0-1)
};

// Lane p's pixel of a whole tile row of an RGB picture (64 pixels, 192 bytes
// from `row`, any alignment): the lane loads the aligned dword holding its
// pixel's first byte and, when the three bytes cross into the next dword,
// that one too (else the same dword again), and takes its bytes from the pair.
// Every dword read holds a byte of the lane's pixel.
__device__ __forceinline__ uint32_t load_row_rgb(const Rgb24 *row, int lane)
{
    const uint32_t m = (uint32_t)(uintptr_t)row & 3u;
    // (pointer arithmetic, not integers, so the loads stay global ones)
    const uint32_t *base = (const uint32_t *)((const char *)row - m);
    const uint32_t o = m + 3u * (uint32_t)lane;  // byte of the lane's pixel from base
    const uint32_t d = o >> 2, k = o & 3u;
    const uint32_t lo = base[d];
    const uint32_t hi = base[k >= 2u ? d + 1u : d];
    return __builtin_amdgcn_alignbyte(hi, lo, k) & 0xFFFFFFu;
}

template <typename T, bool FULL>
__device__ __forceinline__ TileIn load_tile(const T *__restrict__ img, const Geom &g,
                                            const TilePos &tp, int wave, int lane)
{
    TileIn in;
    const uint32_t W = (uint32_t)g.W, y0 = tp.y0, x0 = tp.x0;
    const int vh = FULL ? TH : tp.vh, vw = FULL ? TW : tp.vw;
    const bool lane_ok = FULL || lane < vw;
    const T *im = img + (size_t)tp.b * (size_t)g.HW;
    const T *rows = im + ((y0 + (uint32_t)(wave * RPW)) * W + x0);
    constexpr bool RGB_ROWS = FULL && std::is_same<T, Rgb24>::value;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        if constexpr (RGB_ROWS)
            in.c[i] = load_row_rgb(rows + (uint32_t)i * W, lane);
        else if constexpr (FULL)  // a uniform base and a 32-bit byte offset per lane
            in.c[i] = px(*(const T *)((const char *)rows +
                                      (uint32_t)(((uint32_t)i * W + lane) * sizeof(T))));
        else
            in.c[i] = (lane_ok && wave * RPW + i < vh) ? px(rows[(uint32_t)i * W + lane]) : 0u;
    }
    in.hrow = in.hm1 = in.hp1 = in.hleft = 0;
    if (wave == 0 && tp.ty > 0) {
        const T *up = im + ((y0 - 1u) * W + x0);
        if constexpr (RGB_ROWS) in.hrow = load_row_rgb(up, lane);
        else if (lane_ok) in.hrow = px(up[lane]);
        if (lane == 0 && tp.tx > 0) in.hm1 = px(up[-1]);
        if (lane == TW - 1 && x0 + TW < W) in.hp1 = px(up[TW]);
    }
    if (wave == 0 && tp.tx > 0 && lane < vh) in.hleft = px(im[(y0 + (uint32_t)lane) * W + x0 - 1u]);
    return in;
}

// FULL: the tile lies wholly inside the image (every edge check folds away).
// IGN: pixels of colour ign take part in nothing: their runs join no run,
// reach no seam slot, lead no region and make no seam request; their run
// records say so (INFO_IGNORED), and a tile of that one colour only writes a
// header that says so (KIND_IGNORED).
template <int CONN, bool FULL, bool IGN>
__device__ __forceinline__ void label_tile(const Geom &g, const Work &w, TileLds<IGN> &s, uint32_t t,
                                           const TilePos &tp, const TileIn &in, uint32_t ign)
{
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // the same in the whole wave
    const uint32_t W = (uint32_t)g.W;
    const uint32_t y0 = tp.y0, x0 = tp.x0;
    const int vh = FULL ? TH : tp.vh, vw = FULL ? TW : tp.vw;
    const bool has_top = tp.ty > 0, has_left = tp.tx > 0;
    const bool has_bottom = y0 + TH < (uint32_t)g.H, has_right = x0 + TW < W;
    const bool lane_ok = lane < vw;
    uint32_t c[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) c[i] = in.c[i];
    const uint32_t hrow = in.hrow, hm1 = in.hm1, hp1 = in.hp1, hleft = in.hleft;

    // ---- a tile of one colour needs none of the run phases: is every valid
    //      pixel equal to the tile's first?
    const uint32_t c00 = __builtin_amdgcn_readfirstlane(c[0]);
    const bool full = FULL;
    if (full) {
        // every row is valid: fold the differences from c00 in each lane
        uint32_t d = 0;
#pragma unroll
        for (int i = 0; i < RPW; ++i) d |= c[i] ^ c00;
        const bool bad = __ballot(d != 0) != 0;
        if (lane == 0) s.Uni[wave] = bad ? 0ull : ((uint64_t)1u << 32) | c00;
    } else {
        uint64_t bad = 0;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const uint64_t diff = __ballot(c[i] != c00);
            if (wave * RPW + i < vh) bad |= diff;
        }
        bad &= __ballot(lane_ok);
        if (lane == 0)
            s.Uni[wave] = ((uint64_t)(wave * RPW >= vh ? 2u : (bad == 0 ? 1u : 0u)) << 32) | c00;
    }
    lds_barrier();
    // every wave reads the same words, so every wave takes the same branch:
    // one colour if every wave with rows saw only the colour of the first pixel
    bool uni;
    {
        const uint64_t u0 = s.Uni[0], u1 = s.Uni[1], u2 = s.Uni[2], u3 = s.Uni[3];
        if (full) {
            uni = (((u1 ^ u0) | (u2 ^ u0) | (u3 ^ u0)) == 0) && (u0 >> 32) == 1u;
        } else {
            auto same = [&](uint64_t u) { return u == u0 || (u >> 32) == 2u; };
            uni = (u0 >> 32) == 1u && same(u1) && same(u2) && same(u3);
        }
    }
    // the same for every thread: said so, the branch below stays uniform
    const bool uniform = __builtin_amdgcn_readfirstlane((int)uni) != 0;

    TileHdr &hdr = w.hdr[t];
    const size_t t32 = (size_t)t * TH;

    if (uniform) {
        // ---- one colour: a single region led by the tile's first pixel, with
        //      the seam slot of its first open edge (top row, bottom row, left
        //      column, right column), one run per row.  Wave 0 writes the
        //      header, which holds everything the later passes need, and the
        //      region's seam node; the other waves are done.
        if (wave != 0) return;
        const uint32_t C = c00;  // (wave 0) the colour of the tile's first pixel
        if (IGN && C == ign) {
            // the ignored colour: no region, no seam node, no requests
            uint32_t v = 0;
            v = write_lane(v, KIND_UNIFORM | KIND_IGNORED | (255u << 8), 0);
            v = write_lane(v, (uint32_t)vh, 2);
            if (lane < (int)(sizeof(TileHdr) / 4)) ((uint32_t *)&hdr)[lane] = v;
            return;
        }
        const uint32_t es = has_top ? 0u : has_bottom ? (uint32_t)TW
                          : has_left ? (uint32_t)(2 * TW) : has_right ? (uint32_t)(2 * TW + TH) : 255u;
        uint32_t kind = KIND_UNIFORM | (es << 8);
        uint64_t topmask = 0;
        uint32_t ntop = 0, nleft = 0, leftmask = 0;
        const uint64_t ok_m = FULL || vw >= TW ? ~0ull : (1ull << vw) - 1ull;
        if (has_top) {
            // tile row 0 is one run of colour C against the row above: lane
            // masks of the pixels up, up-left and up-right that have colour C
            // (lanes 0 and 63 look at the halo corners hm1 and hp1)
            const uint64_t u0 = __ballot(hrow == C) & ok_m;
            uint64_t um1 = __ballot(from_left_lane(hrow) == C) & ok_m & ~1ull;
            if (has_left) um1 |= __ballot(hm1 == C) & 1ull;
            if (CONN == 8) {
                uint64_t up1 = __ballot(from_right_lane(hrow) == C) & ok_m & (ok_m >> 1);
                if (has_right) up1 |= __ballot(hp1 == C) & (1ull << 63);
                topmask = up1 & ~u0;  // a stretch of the colour starts up-right
                if ((um1 | u0) & 1ull) {
                    kind |= KIND_TOP0 | ((um1 & 1ull) ? KIND_TOP0_UL : 0u);
                    ntop = 1;
                }
                ntop += popc64(topmask);
            } else {
                topmask = u0 & (~um1 | 1ull);  // a stretch starts up
                ntop = popc64(topmask);
            }
        }
        if (has_left) {
            // lane y: column 0 of row y (colour C) against the halo column;
            // the row above already joins unless its halo pixel differs
            const uint64_t ml = __ballot(hleft == C) & ((1ull << vh) - 1ull);
            const uint64_t hu = __ballot(from_left_lane(hleft) == C);
            leftmask = (uint32_t)(ml & (~hu | 1ull));
            nleft = (uint32_t)__popc(leftmask);
        }
        // the header: lane i holds word i
        uint32_t v = 0;
        v = write_lane(v, kind, 0);
        v = write_lane(v, (uint32_t)vh, 2);
        v = write_lane(v, ntop, 3);
        v = write_lane(v, nleft, 4);
        v = write_lane(v, leftmask, 5);
        if (es != 255u) {
            // its seam node's record: (key of its first pixel << 32) | node
            v = write_lane(v, (t << 8) | UNI_SLOT, 6);
            v = write_lane(v, y0 * W + x0, 7);
        } else {
            v = write_lane(v, 1u, 14);  // the whole image: its first pixel leads
        }
        v = write_lane(v, (uint32_t)topmask, 12);
        v = write_lane(v, (uint32_t)(topmask >> 32), 13);
        if (lane < (int)(sizeof(TileHdr) / 4)) ((uint32_t *)&hdr)[lane] = v;
        return;
    }

    // ---- 1 Start and 2 Connect, fused per row: a ballot marks the row's run
    //      starts ("left neighbour differs"), start lanes initialise their run,
    //      and the row is joined to the row above it.  The joins are found per
    //      pixel against the row above (shifted one lane each way), so that
    //      exactly one pixel stands for each pair of touching runs of one
    //      colour; they are queued per wave and united in LDS with every lane
    //      busy.  A wave's first row is joined to the last row of the wave
    //      above only after the barrier: until then every arrow stays inside
    //      the wave's own rows, which it has initialised itself.
    uint32_t *q = s.Q[wave];
    uint32_t head = 0, tail = 0;
    // lanes of the tile's columns
    const uint64_t ok_m = FULL || vw >= TW ? ~0ull : (1ull << vw) - 1ull;
    // unite queued joins, 64 at a time while 64 wait (all: until none wait);
    // join_rows calls it whenever it queues
    auto drain = [&](bool all) {
        while (tail - head >= 64u || (all && tail != head)) {
            const uint32_t n = tail - head;
            __syncwarp();
            if ((uint32_t)lane < n) {
                const uint32_t e = q[(head + (uint32_t)lane) & (QCAP - 1)];
                lds_unite(s.P, e & 0xFFFFu, e >> 16);
            }
            head += n < 64u ? n : 64u;
        }
    };
    // Rows are handled as lane masks: a ballot per comparison, the logic on
    // the masks in scalar registers.  me / mea: run slot of the lane's pixel in
    // row y / in the row above (bit 0 of a row's start mask is always set, so
    // the run of lane L is the row's first slot + the starts in lanes 1..L).
    // The joins of row y (colours cc, run starts st_m) with the row above it
    // (ca, sta_m).  direct: row y was initialised just now and nothing refers
    // to its runs yet, so the first join of each run is made at once by
    // pointing the run at the parent of the run it joins (which puts it in
    // that run's tree); only a run's further joins are queued as unions.
    auto join_rows = [&](uint32_t cc, uint64_t st_m, uint32_t me, uint32_t ca, uint64_t sta_m,
                         uint32_t mea, uint64_t ig_m, bool direct) {
        // lane shifts read other lanes, so they run with every lane active
        const uint32_t cl = from_left_lane(ca), cr = from_right_lane(ca);
        const uint64_t u0 = __ballot(ca == cc) & ok_m;
        const uint64_t um1 = __ballot(cl == cc) & ok_m & ~1ull;
        uint64_t ra = 0, rb, lu = 0;
        if (CONN == 8) {
            const uint64_t up1 = __ballot(cr == cc) & ok_m & (ok_m >> 1);
            ra = up1 & ~u0;          // a run of the colour starts up-right
            rb = st_m & (um1 | u0);  // the run's first pixel takes up-left or up
            lu = um1 & sta_m;        // ... up-left, where the run above starts at the lane
        } else {
            rb = u0 & (st_m | ~um1);
        }
        if (IGN) {  // a pixel of the ignored colour joins nothing
            ra &= ~ig_m;
            rb &= ~ig_m;
        }
        // run of the row above at column lane-1 (if taken) or lane; at lane+1
        const uint32_t ab = mea - (lane_bit(lu) ? 1u : 0u);
        const uint32_t ar = mea + (lane_bit(sta_m >> 1) ? 1u : 0u);
        if (direct) {
            // each run's first lane with a join (a lane's rb join before its
            // ra join): a 1 added at every run start carries through the
            // run's lanes that make no join and stops at the first that makes
            // one, or at the run's last lane (in E), which keeps the carry out
            // of the next run
            const uint64_t jm = ra | rb;
            const uint64_t em = (st_m >> 1) | (1ull << 63);
            const uint64_t first = (~(jm | em) + st_m) & jm;
            // every lane reads the parent of the run above that its join (rb
            // before ra) would take -- ab and ar are slots of the row above in
            // every lane -- and stores it: a run's first join into the run's
            // word, every other lane into the tail
            const uint32_t pv = lds_parent<false>(s.P, lane_bit(rb) ? ab : ar);
            __hip_atomic_store(&s.P[lane_bit(first) ? me : (uint32_t)(TPX + lane)], pv,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            // joins other than each run's first are left (a lane's ra join
            // stays when its rb join came first); most rows have none
            if (popc64(ra) + popc64(rb) == popc64(first)) return false;
            ra &= ~(first & ~rb);
            rb &= ~first;
        }
        if ((rb | ra) == 0ull) return false;
        // further joins (rare): queued as unions
        if (lane_bit(rb)) q[mbcnt_acc(rb, tail) & (QCAP - 1)] = me | (ab << 16);
        tail += popc64(rb);
        if (lane_bit(ra)) q[mbcnt_acc(ra, tail) & (QCAP - 1)] = me | (ar << 16);
        tail += popc64(ra);
        drain(false);
        return true;
    };
    const int nrows = vh - wave * RPW < 0 ? 0 : (vh - wave * RPW < RPW ? vh - wave * RPW : RPW);
    const uint32_t c0 = c[0];
    const uint32_t wbase = (uint32_t)wave * WAVE_SLOTS;  // the wave's first slot
    {
        uint32_t ca = 0, mea = 0;
        uint64_t sta = 0;
        uint32_t mlo = 0, mhi = 0;  // lane i collects row i's run starts
        uint32_t ilo = 0, ihi = 0;  // ... and its pixels of the ignored colour
        uint32_t rbase = 0;         // ... and its first slot
        uint32_t base = wbase;      // the slot of the row's first run
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if (i >= nrows) break;
            const int y = wave * RPW + i;
            const uint32_t cc = c[i];
            const uint64_t st_m = (__ballot(from_left_lane(cc) != cc) | 1ull) & ok_m;
            const uint32_t me = mbcnt_acc(st_m >> 1, base);
            uint64_t ig_m = 0;
            if (IGN) ig_m = __ballot(cc == ign) & ok_m;
            // the start lane of each run stores its row and column and its
            // parent; the other lanes store into the arrays' tails
            const uint32_t ws = lane_bit(st_m) ? me : (uint32_t)(TPX + lane);
            s.RXY[ws] = (uint16_t)((y << 8) | lane);
            s.P[ws] = me;
            // lane i keeps row i's masks.  A select, not a v_writelane: these
            // values live through the joins' divergent loops (gathered with an
            // inline-asm v_writelane, whose other lanes the compiler does not
            // know it keeps, they came out wrong in one instance of this pass
            // on MI355X)
            mlo = lane == i ? (uint32_t)st_m : mlo;
            mhi = lane == i ? (uint32_t)(st_m >> 32) : mhi;
            rbase = lane == i ? base : rbase;
            if (IGN) {
                ilo = lane == i ? (uint32_t)ig_m : ilo;
                ihi = lane == i ? (uint32_t)(ig_m >> 32) : ihi;
            }
            base += popc64(st_m);
            if (i > 0) join_rows(cc, st_m, me, ca, sta, mea, ig_m, true);
            ca = cc;
            sta = st_m;
            mea = me;
        }
        if (lane < RPW) {  // rows past the image edge store 0
            s.Mask[wave * RPW + lane] = ((uint64_t)mhi << 32) | mlo;
            s.RowBase[wave * RPW + lane] = (uint16_t)rbase;
        }
        if (IGN && lane < RPW) s.Ign[wave * RPW + lane] = ((uint64_t)ihi << 32) | ilo;
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < RPW; ++i) s.ColC[wave * RPW + i] = c[i];  // (0 past the image edge)
        }
        if (wave < NWAVES - 1) s.LastC[wave][lane] = ca;  // this wave's last row
        if (lane == 0) s.WaveRuns[wave] = base - wbase;
    }
    if (tid < KMAX / 64) s.Used[tid] = 0;
    if (tid < TH) s.Lead[tid] = 0;
    lds_barrier();
    if (tid < TH) w.runmask[t32 + tid] = s.Mask[tid];

    // runs of the tile; reading-order run r is slot r - off[w] + w*WAVE_SLOTS
    // of the wave w with off[w] <= r < off[w+1] (the waves' rows follow each
    // other)
    const uint32_t n0 = __builtin_amdgcn_readfirstlane(s.WaveRuns[0]),
                   n1 = __builtin_amdgcn_readfirstlane(s.WaveRuns[1]),
                   n2 = __builtin_amdgcn_readfirstlane(s.WaveRuns[2]),
                   n3 = __builtin_amdgcn_readfirstlane(s.WaveRuns[3]);
    const uint32_t off1 = n0, off2 = off1 + n1, off3 = off2 + n2, R = off3 + n3;
    // (three independent selects of wave-uniform offsets, not a chain of
    // branches)
    const uint32_t adj1 = 1u * WAVE_SLOTS - off1, adj2 = 2u * WAVE_SLOTS - off2,
                   adj3 = 3u * WAVE_SLOTS - off3;
    auto run_slot = [&](uint32_t r) -> uint32_t {
        uint32_t adj = r >= off1 ? adj1 : 0u;
        adj = r >= off2 ? adj2 : adj;
        adj = r >= off3 ? adj3 : adj;
        return r + adj;
    };

    // the wave's first row against the last row of the wave above (unions:
    // both rows' runs may already be joined to others); then every join still
    // queued (fewer than 64 from the wave's rows, and these) is united
    if (wave > 0 && nrows > 0) {
        const int y = wave * RPW;
        const uint64_t mi = uniform64(s.Mask[y]), ma = uniform64(s.Mask[y - 1]);
        const uint32_t ba = __builtin_amdgcn_readfirstlane((uint32_t)s.RowBase[y - 1]);
        join_rows(c0, mi, mbcnt_acc(mi >> 1, wbase), s.LastC[wave - 1][lane], ma,
                  mbcnt_acc(ma >> 1, ba), IGN ? uniform64(s.Ign[y]) : 0ull, false);
    }
    drain(true);
    lds_barrier();
    // the join queues are free now: wave 0 leaves the halo column there for
    // wave 1, which makes the left-edge seam requests
    uint32_t *const s_hleft = s.Q[0];
    if (wave == 0 && lane < TH) s_hleft[lane] = hleft;

    // ---- 3 Collapse, in two steps.  First the runs on an edge shared with
    //      another tile offer their edge position as their region's seam slot
    //      (the smallest wins): thread k < 64 takes the k-th run of the top
    //      row, 64 + k of the bottom row, 128 + y the first run of row y and
    //      160 + y its last run.
    if (tid < KMAX) {
        const int part = tid >> 5;  // 0, 1: top; 2, 3: bottom; 4: left; 5: right
        uint32_t slot = 0, es = 255;
        if (part < 2) {
            const uint64_t m0 = s.Mask[0];
            if (has_top && (uint32_t)tid < popc64(m0)) {
                slot = (uint32_t)tid;  // row 0 starts at slot 0
                es = (uint32_t)tid;
            }
        } else if (part < 4) {
            const uint32_t k = (uint32_t)tid - TW;
            if (has_bottom && k < popc64(s.Mask[TH - 1])) {
                slot = s.RowBase[TH - 1] + k;
                es = TW + k;
            }
        } else {
            const int y = tid & (TH - 1);
            if (y < vh && (part == 4 ? has_left : has_right)) {
                slot = s.RowBase[y] + (part == 4 ? 0u : popc64(s.Mask[y]) - 1u);
                es = (uint32_t)(2 * TW) + (part == 4 ? 0u : (uint32_t)TH) + (uint32_t)y;
            }
        }
        if (IGN && es != 255) {  // a run of the ignored colour offers nothing
            const uint32_t sxy = s.RXY[slot];
            if ((s.Ign[sxy >> 8] >> (sxy & 63u)) & 1ull) es = 255;
        }
        if (es != 255) {
            const uint32_t root = lds_find<true>(s.P, slot);
            atomicMax(&s.P[root], ((255u - es) << 16) | root);
        }
    }
    lds_barrier();

    // ---- 4 Write: one thread per run; records in reading order.  Each run
    //      finds its root (and points straight at it: the last steps read
    //      one arrow per run)
    uint16_t *rinfo = w.runinfo + (size_t)t * TPX;
    for (uint32_t r = tid; r < R; r += BLOCK) {
        const uint32_t slot = run_slot(r);
        if (IGN) {
            const uint32_t sxy = s.RXY[slot];
            if ((s.Ign[sxy >> 8] >> (sxy & 63u)) & 1ull) {
                rinfo[r] = (uint16_t)INFO_IGNORED;
                continue;
            }
        }
        const uint32_t root = lds_find<true>(s.P, slot);
        const uint32_t rv = s.P[root];
        // (a root keeps its word, seam slot included: it stores into the tail)
        atomicMin(&s.P[root == slot ? (uint32_t)(TPX + lane) : slot], root);
        const uint32_t es = 255u - (rv >> 16);
        const uint32_t rxy = s.RXY[root];
        const uint32_t rrow = rxy >> 8, rcol = rxy & 63u;
        rinfo[r] = (uint16_t)(es != 255u ? (INFO_BORDER | es) : ((rrow << 6) | rcol));
        if (root == slot) {
            if (es == 255u) {
                atomicOr((unsigned long long *)&s.Lead[rrow], 1ull << rcol);
            } else {
                const uint32_t node = (t << 8) | es;
                const uint32_t key = (y0 + rrow) * W + x0 + rcol;
                w.gp[(size_t)t * KMAX + es] = ((uint64_t)key << 32) | node;
                atomicOr((unsigned long long *)&s.Used[es >> 6], 1ull << (es & 63u));
            }
        }
    }
    lds_barrier();

    // seam slot of the region of run slot `run`
    auto seam_of = [&](uint32_t run) -> uint32_t {
        const uint32_t root = s.P[run] & PMASK;
        return 255u - (s.P[root] >> 16);
    };
    // the last steps, spread over the waves: 3 the bottom row's seam slots and
    // the header, 2 the right column's slots and the leader masks, 1 the
    // left-edge requests, 0 the top-edge requests
    if (wave == NWAVES - 1) {
        if (has_bottom && lane_ok) {
            const uint64_t mb = uniform64(s.Mask[TH - 1]);
            const uint32_t bb = __builtin_amdgcn_readfirstlane((uint32_t)s.RowBase[TH - 1]);
            w.bslot[(size_t)t * TW + lane] = (uint8_t)seam_of(mbcnt_acc(mb >> 1, bb));
        }
        // the header but its words 3 and 4 (the requests' counts, from waves 0
        // and 1; the one-colour fields stay 0); the first eight bytes also give
        // the final write the bounds of its reads
        const uint32_t nslots = s.Used[2] ? 128u + 64u - (uint32_t)__builtin_clzll(s.Used[2])
                              : s.Used[1] ? 64u + 64u - (uint32_t)__builtin_clzll(s.Used[1])
                              : s.Used[0] ? 64u - (uint32_t)__builtin_clzll(s.Used[0]) : 0u;
        uint32_t v = lane >= 6 && lane < 12 ? ((const uint32_t *)s.Used)[lane - 6] : 0u;
        v = write_lane(v, nslots << 8, 0);
        v = write_lane(v, R, 1);
        v = write_lane(v, R, 2);
        if (lane < (int)(sizeof(TileHdr) / 4) && lane != 3 && lane != 4) ((uint32_t *)&hdr)[lane] = v;
    }
    if (wave == 2) {
        if (has_right && lane < vh)
            w.rslot[t32 + lane] = (uint8_t)seam_of((uint32_t)s.RowBase[lane] + popc64(s.Mask[lane]) - 1u);
        if (lane < TH) {  // rows past the image edge store 0
            const uint64_t lead = s.Lead[lane];
            w.leadmask[t32 + lane] = lead;
            w.seg[t32 + lane] = popc64(lead);
        }
    }
    if (wave == 1) {
        uint32_t nleft = 0;
        if (has_left) {
            const bool valid = lane < vh;
            const uint32_t me = valid ? seam_of((uint32_t)s.RowBase[lane]) : 0u;
            const uint32_t cur = valid ? s.ColC[lane] : 0u;
            nleft = left_requests<CONN>(w.req + (size_t)t * REQMAX + REQ_TOP, lane,
                                        (1ull << vh) - 1ull, me, cur, lane < TH ? s_hleft[lane] : 0u,
                                        IGN ? ~__ballot(valid && cur == ign) : ~0ull);
        }
        if (lane == 4) ((uint32_t *)&hdr)[4] = nleft;  // the header's word 4
    }
    if (wave == 0) {
        uint32_t ntop = 0;
        if (has_top) {
            const uint64_t m0 = uniform64(s.Mask[0]);
            const uint32_t me = seam_of(mbcnt_acc(m0 >> 1, 0u));  // region of the lane's run
            ntop = top_requests<CONN>(w.req + (size_t)t * REQMAX, lane, ok_m, has_left, has_right,
                                      c[0], m0, me, hrow, hm1, hp1,
                                      IGN ? ~uniform64(s.Ign[0]) : ~0ull);
        }
        if (lane == 3) ((uint32_t *)&hdr)[3] = ntop;  // the header's word 3
    }
}

// One workgroup per tile: workgroup v labels tile t0 + tile_order(v), so that
// every stretch of the picture (and its tiles of several colours) is spread
// over all the XCDs, and the whole GPU reads one stretch at a time.
// (Contiguous tile ranges per XCD, as the final write takes them, made this
// pass 5 % slower on a drawing whose detail is unevenly spread.)  Tiles wholly
// inside the image are loaded without edge checks.
//
// The arguments come as one struct, read through the kernel-argument segment
// pointer at each use.  Arguments named as parameters are all loaded into scalar
// registers at kernel entry and stay live; this pass needs more scalar registers
// than are left after that, and the spills (to vector lanes) cost vector
// instructions in every tile, one-colour tiles included.
template <typename T>
struct TileArgs {
    const T *img;
    Geom g;
    Work w;
    uint32_t ign;        // the ignored colour (IGN instances only)
    uint32_t clear_err;  // workgroup 0 clears the error word (the call's first kernel)
    uint32_t t0;         // the first tile of the launch (workgroup v: tile t0 + tile_order(v))
};

template <typename T, int CONN, bool IGN>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(8))) void tile_label_kernel(TileArgs<T> args)
{
    (void)args;  // read below through the segment pointer
    const TileArgs<T> &a = *(const TileArgs<T> *)__builtin_amdgcn_kernarg_segment_ptr();
    const T *__restrict__ img = a.img;
    const Geom &g = a.g;
    const Work &w = a.w;
    __shared__ TileLds<IGN> s;
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // no kernel of this call has run before this one, and the later ones set
    // the word only after it has ended
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.clear_err) *w.err = 0u;
    const uint32_t t = a.t0 + tile_order(blockIdx.x, gridDim.x);
    const TilePos tp = tile_pos(t, g);
    if (tp.vh == TH && tp.vw == TW)
        label_tile<CONN, true, IGN>(g, w, s, t, tp, load_tile<T, true>(img, g, tp, wave, lane), a.ign);
    else
        label_tile<CONN, false, IGN>(g, w, s, t, tp, load_tile<T, false>(img, g, tp, wave, lane), a.ign);
}

// ------------------------------------------------------------- seam passes
// The seam passes give each workgroup a group of tiles and deal their items
// (requests or seam nodes) to its threads: the per-tile counts are
// prefix-summed and each thread takes every BLOCK-th item, so a tile with
// many items does not serialise on one lane.  The roots and resolve passes use
// few tiles per workgroup (most threads hold one item, so that many find
// chains are in flight at once).
constexpr int SEAM_TILES = 64;

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
        const uint32_t sv = sWave[i];
        off += i < wave ? sv : 0u;
        tot += sv;
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

// index j of the tile holding item i: the largest j with off[j] <= i
// (off[NT] is the total, so a tile found this way has items)
template <int NT>
__device__ __forceinline__ uint32_t item_tile(const uint32_t *off, uint32_t i)
{
    uint32_t lo = 0, hi = NT - 1;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (off[mid] <= i) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// the r-th set bit (from 0) of a 64-bit mask
__device__ __forceinline__ uint32_t select_bit64(uint64_t m, uint32_t r)
{
    uint32_t base = 0;
    const uint32_t lo = popc64(m & 0xFFFFFFFFull);
    if (r >= lo) {
        r -= lo;
        m >>= 32;
        base = 32;
    }
    uint32_t x = (uint32_t)m;
    for (; r > 0; --r) x &= x - 1u;  // drop the r lowest set bits
    return base + (uint32_t)__builtin_ctz(x);
}

// the r-th set bit (from 0) of the 192-bit mask u[0..2]
__device__ __forceinline__ uint32_t select_bit(const uint64_t (&u)[KMAX / 64], uint32_t r)
{
    uint32_t base = 0;
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word) {
        const uint32_t c = popc64(u[word]);
        if (r < c) {
            uint64_t m = u[word];
            uint32_t pos = 0;
#pragma unroll
            for (int half = 32; half >= 1; half >>= 1) {  // binary search on popcounts
                const uint64_t lowm = m & ((1ull << half) - 1ull);
                const uint32_t lc = popc64(lowm);
                if (r >= lc) {
                    r -= lc;
                    m >>= half;
                    pos += half;
                } else {
                    m = lowm;
                }
            }
            return base + pos;
        }
        r -= c;
        base += 64;
    }
    return 0;
}

// ------------------------------------------------------------ seam merge
// Two passes over blocks of MB x MB tiles of one image (thread j < BT of a
// workgroup holds tile (j / MB, j % MB) of its block; all threads share the
// block's nodes and requests).
//   block_merge_kernel  joins the seam requests whose two tiles both lie in the
//       block, with a union-find over the block's seam nodes in LDS (records
//       ordered by key as in global memory, so the smallest key leads), then
//       points every node's global record straight at its block root.  A block
//       with more than NODE_CAP nodes joins those requests with global unions
//       instead (one with more than REQ_CAP requests finds each request's tile
//       by a search over the tiles' offsets rather than from a list).
//   border_merge_kernel joins the requests that cross a block border, with
//       global unions, which now start from nearly flat trees.
// Within a block a long chain of joins (a row of blank tiles, each joined to
// the one before it) costs LDS steps, not global round trips.
constexpr int MB = 8;             // block side in tiles
constexpr int BT = MB * MB;       // tiles per block
// LDS tables of a block (21 KB in all, so 7 blocks fit a CU).  On the sheet the
// median block has 176 seam nodes and 5 % of blocks have more than 1536; those
// join their requests with global unions instead.  Tables of 3072 (40 KB, 4
// blocks per CU) made the merge 0.167 ms there, 1536 make it 0.153 ms.
constexpr int NODE_CAP = 1536;    // seam nodes of a block merged in LDS
constexpr int REQ_CAP = 1536;     // seam requests of a block joined in LDS
static_assert(BT <= BLOCK, "one thread per tile of a block");

// the workgroup's block: the tile number of its first tile, and how many of
// its tile rows / columns lie in the image
struct BlockBase {
    uint32_t t0;
    int rows, cols;
};

__device__ __forceinline__ BlockBase block_base(const Geom &g, uint32_t blk)
{
    const uint32_t nbx = ((uint32_t)g.ntx + MB - 1) / MB, nby = ((uint32_t)g.nty + MB - 1) / MB;
    const uint32_t per = nbx * nby;
    const uint32_t b = blk / per, r = blk - b * per, by = r / nbx, bx = r - by * nbx;
    BlockBase bb;
    bb.t0 = b * (uint32_t)g.tpi + by * MB * (uint32_t)g.ntx + bx * MB;
    bb.rows = min(MB, g.nty - (int)(by * MB));
    bb.cols = min(MB, g.ntx - (int)(bx * MB));
    return bb;
}

struct BlockTile {
    int ly, lx;   // place in the block
    bool valid;   // inside the image
    uint32_t t;   // tile number
};

__device__ __forceinline__ BlockTile block_tile(const Geom &g, const BlockBase &bb, int j)
{
    BlockTile p;
    p.ly = j / MB;
    p.lx = j % MB;
    p.valid = j < BT && p.ly < bb.rows && p.lx < bb.cols;
    p.t = bb.t0 + (uint32_t)p.ly * (uint32_t)g.ntx + (uint32_t)p.lx;
    return p;
}

// One seam request of a tile: its own seam slot, the neighbour tile's offset
// (dy = -1: a tile above; dx = -1, 0, +1) and the neighbour's pixel on its
// bottom row (column) or right column (row).
struct SeamReq {
    uint32_t me;
    int dy, dx;
    uint32_t pos;
};

// request r of tile t (the first ntop cross its top edge, the rest its left
// edge); a one-colour tile's requests come from its header masks
__device__ __forceinline__ SeamReq decode_req(const Work &w, uint32_t t, uint32_t r, uint32_t kind,
                                              uint32_t ntop, uint32_t leftmask, uint64_t topmask,
                                              int conn)
{
    SeamReq q;
    const bool uni = kind & KIND_UNIFORM;
    const uint16_t *rq = w.req + (size_t)t * REQMAX;
    if (r < ntop) {
        // across the top edge: the column of the pixel above (-1 and TW: the
        // tiles up-left and up-right)
        int xp;
        if (uni) {
            q.me = UNI_SLOT;
            const uint32_t r0 = (kind & KIND_TOP0) ? 1u : 0u;
            if (r < r0) {
                xp = (kind & KIND_TOP0_UL) ? -1 : 0;
            } else {
                const int x = (int)select_bit64(topmask, r - r0);
                xp = conn == 8 ? x + 1 : x;
            }
        } else {
            const uint32_t e = rq[r];
            q.me = e & 0xFFu;
            xp = (int)(e >> 8) - 1;
        }
        q.dy = -1;
        q.dx = xp < 0 ? -1 : (xp >= TW ? 1 : 0);
        q.pos = xp < 0 ? (uint32_t)(TW - 1) : (xp >= TW ? 0u : (uint32_t)xp);
    } else {
        // across the left edge: the tile row
        if (uni) {
            q.me = UNI_SLOT;
            q.pos = select_bit64((uint64_t)leftmask, r - ntop);
        } else {
            const uint32_t e = rq[REQ_TOP + r - ntop];
            q.me = e & 0xFFu;
            q.pos = (e >> 8) & 0x7Fu;
        }
        q.dy = 0;
        q.dx = -1;
    }
    return q;
}

// the neighbour's seam slot at the request's pixel (a one-colour tile has one)
__device__ __forceinline__ uint32_t nb_slot(const Work &w, uint32_t tn, uint32_t nkind,
                                            const SeamReq &q)
{
    if (nkind & KIND_UNIFORM) return UNI_SLOT;
    return q.dy < 0 ? w.bslot[(size_t)tn * TW + q.pos] : w.rslot[(size_t)tn * TH + q.pos];
}

// LDS union-find over block nodes: record = (key << 32) | parent index; the
// same rules as g_find / g_unite (every arrow points at a smaller key, so each
// loop ends)
__device__ __forceinline__ uint32_t l_find(uint64_t *R, uint32_t x, uint64_t &root_rec)
{
    auto load = [&](uint32_t i) {
        return __hip_atomic_load(&R[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    uint64_t rec = load(x);
    for (;;) {
        const uint32_t p = (uint32_t)rec;
        if (p == x) break;
        const uint64_t prec = load(p);
        if ((uint32_t)prec == p) {
            x = p;
            rec = prec;
            break;
        }
        atomicMin((unsigned long long *)&R[x], prec);  // path halving
        x = (uint32_t)prec;
        rec = load(x);
    }
    root_rec = rec;
    return x;
}

__device__ __forceinline__ void l_unite(uint64_t *R, uint32_t a, uint32_t b)
{
    for (;;) {
        uint64_t ra_rec, rb_rec;
        const uint32_t ra = l_find(R, a, ra_rec), rb = l_find(R, b, rb_rec);
        if (ra == rb) return;
        const bool a_lo = ra_rec < rb_rec;
        const uint32_t lo = a_lo ? ra : rb, hi = a_lo ? rb : ra;
        const uint64_t lo_rec = a_lo ? ra_rec : rb_rec, hi_rec = a_lo ? rb_rec : ra_rec;
        const uint64_t old = atomicMin((unsigned long long *)&R[hi], lo_rec);
        if (old == hi_rec) return;
        a = lo;
        b = (uint32_t)old;
    }
}

__global__ __launch_bounds__(BLOCK) void block_merge_kernel(Geom g, Work w, int conn, uint32_t slices)
{
    __shared__ uint64_t sRec[NODE_CAP];      // node records: (key << 32) | parent
    __shared__ uint16_t sNode[NODE_CAP];     // node -> (local tile << 8) | seam slot
    __shared__ uint16_t sReq[REQ_CAP];       // request -> (local tile << 8) | its index
    __shared__ uint64_t sUsed[BT][KMAX / 64];
    __shared__ uint64_t sTop[BT];
    __shared__ uint32_t sBase[BT], sOff[BT + 1];
    __shared__ uint32_t sKind[BT], sNtop[BT], sLeft[BT];
    __shared__ uint32_t sWave[NWAVES];
    const int j = threadIdx.x;
    // workgroup (block, slice): a block that joins its requests with global
    // unions deals them over its slices; one merged in LDS uses slice 0 alone.
    // Each XCD takes a contiguous range of blocks.
    const uint32_t wg = remap_tile(blockIdx.x, gridDim.x);
    const uint32_t blk = wg / slices, slice = wg - blk * slices;
    const BlockBase bb = block_base(g, blk);
    const BlockTile me = block_tile(g, bb, j);
    uint32_t nnodes = 0, nreq = 0, kind = 0;
    uint64_t u[KMAX / 64] = {0ull, 0ull, 0ull};
    {
        uint64_t topmask = 0;
        uint32_t ntop = 0, leftmask = 0;
        if (me.valid) {
            const TileHdr &h = w.hdr[me.t];
            kind = h.kind;
            ntop = h.ntop;
            nreq = ntop + h.nleft;
            if (kind & KIND_UNIFORM) {
                nnodes = ((kind >> 8) & 0xFFu) != 255u ? 1u : 0u;  // if it has an open edge
                topmask = h.topmask;
                leftmask = h.leftmask;
            } else {
#pragma unroll
                for (int word = 0; word < KMAX / 64; ++word) {
                    u[word] = h.used[word];
                    nnodes += popc64(u[word]);
                }
            }
        }
        if (j < BT) {
#pragma unroll
            for (int word = 0; word < KMAX / 64; ++word) sUsed[j][word] = u[word];
            sTop[j] = topmask;
            sKind[j] = kind;
            sNtop[j] = ntop;
            sLeft[j] = leftmask;
        }
    }
    uint32_t total_nodes, total_req;
    const uint32_t noff = block_exclusive_scan(nnodes, sWave, total_nodes);
    const uint32_t roff = block_exclusive_scan(nreq, sWave, total_req);
    const bool in_lds = total_nodes <= (uint32_t)NODE_CAP;  // the union-find fits in LDS
    const bool listed = total_req <= (uint32_t)REQ_CAP;     // so does the request list
    if (in_lds && slice != 0) return;
    if (j <= BT) sOff[j] = roff;  // entry BT: the total
    if (in_lds && j < BT) {
        // each tile lists its nodes (slots in order)
        sBase[j] = noff;
        if (kind & KIND_UNIFORM) {
            if (nnodes) sNode[noff] = (uint16_t)((j << 8) | UNI_SLOT);
        } else {
            uint32_t k = noff;
#pragma unroll
            for (int word = 0; word < KMAX / 64; ++word)
                for (uint64_t m = u[word]; m; m &= m - 1ull)
                    sNode[k++] = (uint16_t)((j << 8) | (uint32_t)(word * 64 + __builtin_ctzll(m)));
        }
    }
    if (listed && j < BT)  // ... and its requests
        for (uint32_t r = 0; r < nreq; ++r) sReq[roff + r] = (uint16_t)((j << 8) | r);
    __syncthreads();
    // local index of seam slot `slot` of local tile jj
    auto local_node = [&](int jj, uint32_t slot) -> uint32_t {
        if (slot == UNI_SLOT) return sBase[jj];
        const uint32_t word = slot >> 6;
        uint32_t below = popc64(sUsed[jj][word] & mask_lt((int)(slot & 63u)));
        if (word > 0) below += popc64(sUsed[jj][0]);
        if (word > 1) below += popc64(sUsed[jj][1]);
        // (a slot in use always lands inside the tile's nodes; the bound only
        // keeps a malformed request inside the table)
        return min(sBase[jj] + below, total_nodes - 1u);
    };
    if (in_lds) {
        // the nodes' own records, two per thread at a time (their loads overlap)
        for (uint32_t i0 = j; i0 < total_nodes; i0 += 2 * BLOCK) {
            const uint32_t i1 = i0 + BLOCK;
            const uint32_t n0 = sNode[i0], n1 = i1 < total_nodes ? sNode[i1] : n0;
            const uint64_t r0 = *node_rec(w, (block_tile(g, bb, (int)(n0 >> 8)).t << 8) | (n0 & 0xFFu));
            const uint64_t r1 = *node_rec(w, (block_tile(g, bb, (int)(n1 >> 8)).t << 8) | (n1 & 0xFFu));
            // before the merge every record is its node's own: (key << 32) | node
            sRec[i0] = (r0 & 0xFFFFFFFF00000000ull) | i0;
            if (i1 < total_nodes) sRec[i1] = (r1 & 0xFFFFFFFF00000000ull) | i1;
        }
        __syncthreads();
    }
    // the requests whose two tiles lie in the block
    const uint32_t step = in_lds ? (uint32_t)BLOCK : slices * (uint32_t)BLOCK;
    for (uint32_t i = (in_lds ? 0u : slice * (uint32_t)BLOCK) + (uint32_t)j; i < total_req; i += step) {
        uint32_t jj, r;
        if (listed) {
            const uint32_t e = sReq[i];
            jj = e >> 8;
            r = e & 0xFFu;
        } else {  // without the lists: the tile holding item i, by its offsets
            jj = item_tile<BT>(sOff, i);
            r = i - sOff[jj];
        }
        const BlockTile tt = block_tile(g, bb, (int)jj);
        const SeamReq q = decode_req(w, tt.t, r, sKind[jj], sNtop[jj], sLeft[jj], sTop[jj], conn);
        const int nly = tt.ly + q.dy, nlx = tt.lx + q.dx;
        if (nly < 0 || nlx < 0 || nlx >= MB) continue;  // crosses the block border
        const int jn = nly * MB + nlx;
        const uint32_t tn = block_tile(g, bb, jn).t;
        const uint32_t ns = nb_slot(w, tn, sKind[jn], q);
        if (in_lds)
            l_unite(sRec, local_node((int)jj, q.me), local_node(jn, ns));
        else
            g_unite(w, (tt.t << 8) | q.me, (tn << 8) | ns);
    }
    if (!in_lds) return;
    __syncthreads();
    // every node's record names its block root (roots keep their own)
    for (uint32_t i = j; i < total_nodes; i += BLOCK) {
        uint64_t rrec;
        const uint32_t r = l_find(sRec, i, rrec);
        if (r == i) continue;
        const uint32_t ni = sNode[i], nr = sNode[r];
        const uint32_t gi = (block_tile(g, bb, (int)(ni >> 8)).t << 8) | (ni & 0xFFu);
        const uint32_t gr = (block_tile(g, bb, (int)(nr >> 8)).t << 8) | (nr & 0xFFu);
        *node_rec(w, gi) = (rrec & 0xFFFFFFFF00000000ull) | gr;
    }
}

// The requests that cross a block border, from the tiles on the block's top
// row and its left and right columns.
__global__ __launch_bounds__(BLOCK) void border_merge_kernel(Geom g, Work w, int conn, uint32_t slices)
{
    __shared__ uint64_t sTop[BT];
    __shared__ uint32_t sOff[BT + 1];
    __shared__ uint32_t sKind[BT], sNtop[BT], sLeft[BT];
    __shared__ uint32_t sWave[NWAVES];
    const int j = threadIdx.x;
    // workgroup (block, slice): the slices of a block take its rounds in turn;
    // each XCD takes a contiguous range of blocks
    const uint32_t wg = remap_tile(blockIdx.x, gridDim.x);
    const uint32_t blk = wg / slices, slice = wg - blk * slices;
    const BlockBase bb = block_base(g, blk);
    const BlockTile me = block_tile(g, bb, j);
    const bool border = me.ly == 0 || me.lx == 0 || me.lx == MB - 1;
    uint32_t nreq = 0, kind = 0, ntop = 0, leftmask = 0;
    uint64_t topmask = 0;
    if (me.valid && border) {
        const TileHdr &h = w.hdr[me.t];
        kind = h.kind;
        ntop = h.ntop;
        nreq = ntop + h.nleft;
        topmask = h.topmask;
        leftmask = h.leftmask;
    }
    if (j < BT) {
        sTop[j] = topmask;
        sKind[j] = kind;
        sNtop[j] = ntop;
        sLeft[j] = leftmask;
    }
    uint32_t total;
    const uint32_t off = block_exclusive_scan(nreq, sWave, total);
    if (j <= BT) sOff[j] = off;  // entry BT: the total
    __syncthreads();
    const int lane = lane_id();
    const uint32_t rounds = (total + BLOCK - 1) / BLOCK;
    for (uint32_t k = slice; k < rounds; k += slices) {
        const uint32_t i = k * BLOCK + (uint32_t)j;
        uint32_t a = 0xFFFFFFFFu, bn = 0xFFFFFFFFu;
        if (i < total) {
            const uint32_t jj = item_tile<BT>(sOff, i);
            const BlockTile tt = block_tile(g, bb, (int)jj);
            const SeamReq q = decode_req(w, tt.t, i - sOff[jj], sKind[jj], sNtop[jj], sLeft[jj],
                                         sTop[jj], conn);
            const int nly = tt.ly + q.dy, nlx = tt.lx + q.dx;
            if (nly < 0 || nlx < 0 || nlx >= MB) {
                const uint32_t tn = tt.t - (q.dy < 0 ? (uint32_t)g.ntx : 0u) + (uint32_t)q.dx;
                a = (tt.t << 8) | q.me;
                bn = (tn << 8) | nb_slot(w, tn, w.hdr[tn].kind, q);
            }
        }
        // a request equal to the one before it (held by the previous lane) is skipped
        const uint32_t pa = __shfl_up(a, 1), pb = __shfl_up(bn, 1);
        if (a != 0xFFFFFFFFu && !(lane > 0 && pa == a && pb == bn)) g_unite(w, a, bn);
    }
}

// ------------------------------------------------------------- seam roots
// Seam nodes of tpw (<= SEAM_TILES) consecutive tiles, dealt round-robin to the
// workgroup's threads.  A node that is still a root after the merge leads a
// region of the whole image: it joins its row segment's leader mask and count
// (a one-colour tile's node sets the tile's leader bit).  This pass also
// clears the band status words of the scan that follows.

__global__ __launch_bounds__(BLOCK) void seam_roots_kernel(Geom g, Work w, uint32_t tpw)
{
    clear_bands(g, w);
    __shared__ uint32_t sOff[SEAM_TILES + 1];
    __shared__ uint64_t sUsed[SEAM_TILES][KMAX / 64];
    __shared__ uint8_t sUni[SEAM_TILES];
    __shared__ uint32_t sWave[NWAVES];
    // the workgroup's leaders, gathered per tile row before they join the row
    // segments' masks and counts (each tile belongs to this workgroup alone)
    __shared__ uint64_t sLead[SEAM_TILES * TH];
    __shared__ uint32_t sCnt[SEAM_TILES * TH];
    for (int i = threadIdx.x; i < SEAM_TILES * TH; i += BLOCK) {
        sLead[i] = 0ull;
        sCnt[i] = 0u;
    }
    // tiles t0 .. t0+tpw-1 (tpw <= SEAM_TILES); each XCD takes a contiguous range
    const uint32_t t0 = remap_tile(blockIdx.x, gridDim.x) * tpw;
    const uint32_t tme = t0 + threadIdx.x;
    const bool mine = threadIdx.x < tpw && tme < (uint32_t)g.ntiles;
    uint32_t n = 0;
    bool uni = false;
    if (mine) {
        const uint32_t kind = w.hdr[tme].kind;
        uni = (kind & KIND_UNIFORM) != 0;
        if (uni) n = ((kind >> 8) & 0xFFu) != 255u ? 1u : 0u;  // its node, if it has an open edge
    }
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word) {
        const uint64_t u = (mine && !uni) ? w.hdr[tme].used[word] : 0ull;
        if (threadIdx.x < SEAM_TILES) sUsed[threadIdx.x][word] = u;
        n += popc64(u);
    }
    if (threadIdx.x < SEAM_TILES) sUni[threadIdx.x] = uni ? 1 : 0;
    uint32_t total;
    const uint32_t off = block_exclusive_scan(n, sWave, total);
    if (threadIdx.x <= SEAM_TILES) sOff[threadIdx.x] = off;  // sOff[SEAM_TILES] = total
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < total; i += BLOCK) {
        const uint32_t j = item_tile<SEAM_TILES>(sOff, i);
        const uint32_t t = t0 + j;
        uint64_t u[KMAX / 64];
#pragma unroll
        for (int word = 0; word < KMAX / 64; ++word) u[word] = sUsed[j][word];
        const uint32_t node = (t << 8) | (sUni[j] ? UNI_SLOT : select_bit(u, i - sOff[j]));
        // every union is done: a node leads its region exactly when its record
        // still names itself
        const uint64_t rec = *node_rec(w, node);
        if ((uint32_t)rec != node) continue;
        if (sUni[j]) {
            w.hdr[t].lead = 1u;  // a one-colour tile's only node: its first pixel leads
        } else {
            const TilePos tp = tile_pos(t, g);
            const uint32_t key = (uint32_t)(rec >> 32);
            const uint32_t Y = fast_div(key, g.divW);
            const uint32_t row = Y - tp.y0, col = key - Y * (uint32_t)g.W - tp.x0;
            atomicOr((unsigned long long *)&sLead[j * TH + row], 1ull << col);
            atomicAdd(&sCnt[j * TH + row], 1u);
        }
    }
    __syncthreads();
    // the tile pass wrote these words (its own leaders); add the seam leaders
    // (each segment is this workgroup's alone: the atomics only spare the
    // workgroup a read before each write)
    for (int i = threadIdx.x; i < (int)tpw * TH; i += BLOCK) {
        const uint32_t cnt = sCnt[i];
        if (cnt == 0) continue;
        const size_t sg = (size_t)t0 * TH + i;
        __hip_atomic_fetch_or((unsigned long long *)&w.leadmask[sg], (unsigned long long)sLead[i],
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(&w.seg[sg], cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------------------ scan
// seg[] holds the leaders of each row segment (tile-major).  One workgroup per
// tile row of tiles ("band"), in one pass.  Thread (y, g) owns tile row y of
// a contiguous group g of the band's tiles (32 rows x 32 groups = 1024 threads;
// the 32 threads of a group read one tile's 32 counts, 128 contiguous bytes).
// It sums its counts; the sums give, for each row, the leaders of the earlier
// groups and of all earlier rows of the band; the leaders of all earlier
// bands of the image come from a decoupled look-back (each band publishes its
// own total at once and its inclusive prefix as soon as it knows it; one wave
// inspects 64 earlier bands per step).  Then every segment gets its
// exclusive prefix in reading order.

constexpr int SCAN_BLOCK = 1024;                // threads per band
constexpr int SCAN_GROUPS = SCAN_BLOCK / TH;    // tile groups per band

// Band status word: (value << 32) | state; state 1: value = the band's own
// leaders, state 2: value = the leaders of the band and all earlier bands of
// its image.  Cleared by the pass before the scan.
constexpr uint32_t BAND_TOTAL = 1u, BAND_PREFIX = 2u;
constexpr int LOOKBACK_BUDGET = 1 << 22;

__device__ __forceinline__ void band_publish(uint64_t *p, uint32_t state, uint32_t value)
{
    __hip_atomic_store(p, ((uint64_t)value << 32) | state, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Leaders of SCAN_U consecutive segments of tile row y (tiles t .. t+n-1, n <=
// SCAN_U), all loads issued before any is used: with headers (the labelling
// path), a one-colour tile counts the leader bit of its header in its row 0
// and 0 in its other rows (it never wrote row-segment counts, so the count
// read for it is not used); ccl_number / ccl_count have no headers.  uni[u]
// tells whether tile t+u is a one-colour tile.
constexpr int SCAN_U = 8;
__device__ __forceinline__ void scan_counts(const Work &w, size_t t, uint32_t n, int y, int use_hdr,
                                            uint32_t (&c)[SCAN_U], bool (&uni)[SCAN_U])
{
    uint32_t kind[SCAN_U], lead[SCAN_U];
#pragma unroll
    for (int u = 0; u < SCAN_U; ++u) {
        kind[u] = lead[u] = c[u] = 0;
        if ((uint32_t)u < n) {
            if (use_hdr) {
                kind[u] = w.hdr[t + u].kind;
                lead[u] = w.hdr[t + u].lead;
            }
            c[u] = w.seg[(t + u) * TH + (size_t)y];
        }
    }
#pragma unroll
    for (int u = 0; u < SCAN_U; ++u) {
        uni[u] = (kind[u] & KIND_UNIFORM) != 0;
        if (uni[u]) c[u] = y == 0 ? lead[u] : 0u;
    }
}

// apply = 0 only counts.
__global__ __launch_bounds__(SCAN_BLOCK) void scan_kernel(Geom g, Work w, int32_t *counts, int apply,
                                                     int use_hdr, uint32_t band0)
{
    __shared__ uint32_t sPart[TH][SCAN_GROUPS + 1];  // per row: each group's sum, then its prefix
    __shared__ uint32_t sRowPre[TH + 1];             // leaders of the earlier rows; [TH]: the band's
    __shared__ uint32_t sPre;                        // leaders of the earlier bands of the image
    const uint32_t band = band0 + blockIdx.x;  // b * nty + ty
    const uint32_t b = fast_div(band, g.divNty), ty = band - b * (uint32_t)g.nty;
    const size_t t0 = (size_t)b * g.tpi + (size_t)ty * g.ntx;
    const uint32_t ntx = (uint32_t)g.ntx;
    const int y = threadIdx.x & (TH - 1), grp = threadIdx.x / TH;
    const int lane = lane_id();
    const uint32_t G = (ntx + SCAN_GROUPS - 1) / SCAN_GROUPS;
    const uint32_t tx0 = min(ntx, (uint32_t)grp * G), tx1 = min(ntx, tx0 + G);

    uint32_t sum = 0;
    for (uint32_t tx = tx0; tx < tx1; tx += SCAN_U) {
        uint32_t c[SCAN_U];
        bool uni[SCAN_U];
        scan_counts(w, t0 + tx, tx1 - tx, y, use_hdr, c, uni);
#pragma unroll
        for (int u = 0; u < SCAN_U; ++u) sum += c[u];
    }
    sPart[y][grp] = sum;
    __syncthreads();
    if (threadIdx.x < 64) {
        // lane y < TH: the groups' prefixes in row y and the row's total, then
        // the exclusive prefix over the rows
        uint32_t tot = 0;
        if (lane < TH) {
#pragma unroll
            for (int k = 0; k < SCAN_GROUPS; ++k) {
                const uint32_t v = sPart[lane][k];
                sPart[lane][k] = tot;
                tot += v;
            }
        }
        uint32_t x = tot;
#pragma unroll
        for (int d = 1; d < TH; d <<= 1) {
            const uint32_t v = __shfl_up(x, d);
            if (lane >= d) x += v;
        }
        if (lane < TH) sRowPre[lane] = x - tot;
        if (lane == TH - 1) sRowPre[TH] = x;
        __syncwarp();
        const uint32_t total = __shfl(x, TH - 1);  // the band's leaders

        // look-back: every lane of wave 0 takes part
        uint32_t pre = 0;
        if (ty == 0) {
            if (lane == 0) band_publish(&w.bandst[band], BAND_PREFIX, total);
        } else {
            if (lane == 0) band_publish(&w.bandst[band], BAND_TOTAL, total);
            uint32_t hi = band - 1;  // nearest band not yet added
            uint32_t left = ty;      // earlier bands of the image not yet added: hi, hi-1, ...
            int budget = LOOKBACK_BUDGET;
            while (true) {
                // lane i looks at band hi - i, if that is still in the image
                const bool in = (uint32_t)lane < left;
                const uint64_t v = in ? __hip_atomic_load(&w.bandst[hi - (uint32_t)lane],
                                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                      : (uint64_t)BAND_PREFIX;  // before the image: prefix 0
                const uint32_t state = (uint32_t)v;
                const uint64_t pm = __ballot(state == BAND_PREFIX);
                const uint64_t zm = __ballot(state == 0u);
                const int near = pm ? (int)__builtin_ctzll(pm) : 63;  // last lane to add
                if (zm & mask_le(near)) {  // a band up to there has not reported yet
                    if (--budget <= 0) {   // never reported: flag it, do not wait
                        if (lane == 0) set_err(w.err, ERR_LOOP);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                uint32_t add = lane <= near ? (uint32_t)(v >> 32) : 0u;
#pragma unroll
                for (int d = 32; d >= 1; d >>= 1) add += __shfl_xor(add, d);
                pre += add;
                if (pm) break;
                hi -= 64u;  // no lane was past the image, so left >= 64
                left -= 64u;
            }
            if (lane == 0) band_publish(&w.bandst[band], BAND_PREFIX, pre + total);
        }
        if (lane == 0) {
            sPre = pre;
            if (counts && ty == (uint32_t)g.nty - 1) counts[b] = (int32_t)(pre + total);
        }
    }
    __syncthreads();
    if (!apply) return;
    // leaders before this thread's first segment, then along its tiles
    uint32_t run = sPre + sRowPre[y] + sPart[y][grp];
    for (uint32_t tx = tx0; tx < tx1; tx += SCAN_U) {
        uint32_t c[SCAN_U];
        bool uni[SCAN_U];
        const size_t t = t0 + tx;
        scan_counts(w, t, tx1 - tx, y, use_hdr, c, uni);
#pragma unroll
        for (int u = 0; u < SCAN_U; ++u) {
            if (tx + (uint32_t)u >= tx1) break;
            if (uni[u]) {
                if (y == 0) w.hdr[t + u].pre = run;  // leaders before the tile's first pixel
            } else {
                w.seg[(t + u) * TH + (size_t)y] = run;
            }
            run += c[u];
        }
    }
}

// ---------------------------------------------------------------- resolve
// After the scan, each seam node finds its leader (Collapse) and gets the value
// its pixels will carry: the leader's index, or 1 + the leaders before it.
// Nodes of tpw (<= SEAM_TILES) consecutive tiles are dealt round-robin to the
// workgroup's threads.  The records are only read here, so the walks may run
// side by side; the values go to nval (a one-colour tile: its header).

// Statistics outputs of the labelling call (rec == nullptr: none): records of
// the image's regions, image b's region k at off[b] + k - 1, only the first
// cap written.
struct StatsOut {
    RegionRec *rec;
    int64_t cap;
    const int64_t *off;  // [B] first record of each image
};

// an empty record: area 0, box (INT32_MAX, INT32_MAX, -1, -1), sums 0
__device__ __forceinline__ void stats_empty(RegionRec *r)
{
    uint64_t *q = (uint64_t *)r;
    q[0] = q[1] = 0ull;                                      // sums
    q[2] = (uint64_t)2147483647u << 32;                      // area 0, y0 INT32_MAX
    q[3] = 2147483647u | ((uint64_t)0xFFFFFFFFu << 32);      // x0 INT32_MAX, y1 -1
    q[4] = 0xFFFFFFFFu;                                      // x1 -1, pad 0
}

__global__ __launch_bounds__(BLOCK) void resolve_kernel(Geom g, Work w, int number, StatsOut so,
                                                       uint32_t tpw)
{
    __shared__ uint32_t sOff[SEAM_TILES + 1];
    __shared__ uint64_t sUsed[SEAM_TILES][KMAX / 64];
    __shared__ uint8_t sUni[SEAM_TILES];
    __shared__ uint32_t sWave[NWAVES];
    // tiles t0 .. t0+tpw-1 (tpw <= SEAM_TILES); each XCD takes a contiguous range
    const uint32_t t0 = remap_tile(blockIdx.x, gridDim.x) * tpw;
    const uint32_t tme = t0 + threadIdx.x;
    const bool mine = threadIdx.x < tpw && tme < (uint32_t)g.ntiles;
    uint32_t n = 0;
    bool uni = false;
    if (mine) {
        const uint32_t kind = w.hdr[tme].kind;
        uni = (kind & KIND_UNIFORM) != 0;
        if (uni) n = ((kind >> 8) & 0xFFu) != 255u ? 1u : 0u;  // its node, if it has an open edge
    }
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word) {
        const uint64_t u = (mine && !uni) ? w.hdr[tme].used[word] : 0ull;
        if (threadIdx.x < SEAM_TILES) sUsed[threadIdx.x][word] = u;
        n += popc64(u);
    }
    if (threadIdx.x < SEAM_TILES) sUni[threadIdx.x] = uni ? 1 : 0;
    uint32_t total;
    const uint32_t off = block_exclusive_scan(n, sWave, total);
    if (threadIdx.x <= SEAM_TILES) sOff[threadIdx.x] = off;  // sOff[SEAM_TILES] = total
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < total; i += BLOCK) {
        const uint32_t j = item_tile<SEAM_TILES>(sOff, i);
        const uint32_t t = t0 + j;
        uint64_t u[KMAX / 64];
#pragma unroll
        for (int word = 0; word < KMAX / 64; ++word) u[word] = sUsed[j][word];
        const uint32_t node = (t << 8) | (sUni[j] ? UNI_SLOT : select_bit(u, i - sOff[j]));
        uint64_t rrec;
        const uint32_t root = g_root(w, node, rrec);
        const uint32_t key = (uint32_t)(rrec >> 32) & 0x7FFFFFFFu;  // (without REC_SHARED)
        uint32_t val = key;
        if (number) {
            uint32_t tl, row, col;
            pixel_tile(key, fast_div(t, g.divTpi), g, tl, row, col);
            const uint32_t lkind = w.hdr[tl].kind;
            if (lkind & KIND_UNIFORM) {
                val = 1u + w.hdr[tl].pre;  // the leader is a one-colour tile's first pixel
            } else {
                const size_t sg = (size_t)tl * TH + row;
                val = 1u + w.seg[sg] + popc64(w.leadmask[sg] & mask_lt((int)col));
            }
        }
        if (sUni[j])
            w.hdr[t].value = val;  // a one-colour tile's only node
        else
            w.nval[(size_t)t * KMAX + (node & 0xFFu)] = val;
        // number == 2: the node's record also takes its root's (the key of the
        // region's leader), for leaders written from a numbered labelling
        if (number == 2 && root != node) g_min(node_rec(w, node), rrec);
        // statistics: each region with a seam node has one root node, which
        // opens its record (the tiles' parts are added later); the other nodes
        // mark the root's record as shared.  Every such store writes the same
        // value, and the walks of other nodes only read the root's id and key
        // from it, so they may run side by side.
        if (so.rec != nullptr) {
            if (root == node) {
                const int64_t idx = so.off[fast_div(t, g.divTpi)] + (int64_t)val - 1;
                if ((uint64_t)idx < (uint64_t)so.cap) stats_empty(&so.rec[idx]);
            } else if (!(rrec & REC_SHARED)) {
                *node_rec(w, root) = rrec | REC_SHARED;
            }
        }
    }
}

// ------------------------------------------- statistics in the final write
// With statistics (ccl_label_stats), the final write also gathers each
// region's area, bounding box and sums of row and column indices from the
// run records it expands (see the statistics section below for the steps).

constexpr int SR_CAP = 128;  // regions inside one tile gathered per pass over its runs

// a region's part in one tile, packed: area (11 bits: at most 2047 pixels in a
// tile of several colours), sums of local rows (15: at most 31744) and local
// columns (16: at most 64512), then rows y0, y1 (5 each), columns x0, x1 (6
// each).  The three sums alone (the low 42 bits) add without carries between
// them, so parts are gathered with one 64-bit add.
__device__ __forceinline__ uint64_t pack_part(uint64_t sums, uint32_t rows, uint64_t cols)
{
    const uint32_t y0 = (uint32_t)__builtin_ctz(rows), y1 = 31u - (uint32_t)__builtin_clz(rows);
    const uint32_t x0 = (uint32_t)__builtin_ctzll(cols), x1 = 63u - (uint32_t)__builtin_clzll(cols);
    return sums | ((uint64_t)y0 << 42) | ((uint64_t)y1 << 47) | ((uint64_t)x0 << 52) |
           ((uint64_t)x1 << 58);
}

// a one-colour tile's whole record (its region lies in this tile alone)
__device__ __forceinline__ void tile_record(RegionRec *r, const TilePos &tp)
{
    const int64_t vh = tp.vh, vw = tp.vw, y0 = tp.y0, x0 = tp.x0;
    uint64_t *q = (uint64_t *)r;
    q[0] = (uint64_t)(vw * (vh * y0 + vh * (vh - 1) / 2));
    q[1] = (uint64_t)(vh * (vw * x0 + vw * (vw - 1) / 2));
    q[2] = (uint64_t)(uint32_t)(vh * vw) | ((uint64_t)(uint32_t)y0 << 32);
    q[3] = (uint64_t)(uint32_t)x0 | ((uint64_t)(uint32_t)(y0 + vh - 1) << 32);
    q[4] = (uint64_t)(uint32_t)(x0 + vw - 1);
}

// the whole record of a region that lies in one tile, from its packed part
// (local sums and box) and the tile's position
__device__ __forceinline__ void part_record(RegionRec *r, uint64_t pk, const TilePos &tp)
{
    const uint64_t a = pk & 0x7FFu;
    uint64_t *q = (uint64_t *)r;
    q[0] = ((pk >> 11) & 0x7FFFu) + a * tp.y0;
    q[1] = ((pk >> 26) & 0xFFFFu) + a * tp.x0;
    q[2] = a | ((uint64_t)(tp.y0 + (uint32_t)((pk >> 42) & 31u)) << 32);
    q[3] = (uint64_t)(tp.x0 + (uint32_t)((pk >> 52) & 63u)) |
           ((uint64_t)(tp.y0 + (uint32_t)((pk >> 47) & 31u)) << 32);
    q[4] = (uint64_t)(tp.x0 + (uint32_t)(pk >> 58));
}

// the r-th set bit (from 0) of m, r < popcount(m): a binary search on
// popcounts, without branches
__device__ __forceinline__ uint32_t select_bit64_bs(uint64_t m, uint32_t r)
{
    const uint32_t lo = (uint32_t)m, c32 = (uint32_t)__builtin_popcount(lo);
    const bool up = r >= c32;
    uint32_t x = up ? (uint32_t)(m >> 32) : lo;
    uint32_t pos = up ? 32u : 0u;
    r -= up ? c32 : 0u;
#pragma unroll
    for (int half = 16; half >= 1; half >>= 1) {
        const uint32_t c = (uint32_t)__builtin_popcount(x & ((1u << half) - 1u));
        const bool hi = r >= c;
        x = hi ? x >> half : x;
        pos += hi ? (uint32_t)half : 0u;
        r -= hi ? c : 0u;
    }
    return pos;
}

// run r of a tile: its row, first and last column.  rex_y (wave-uniform) is
// the number of runs before row y; lane y of mlo / mhi / rexv holds row y's
// run starts and run count before it.
struct RunPos {
    uint32_t y, x, e;
};

__device__ __forceinline__ RunPos run_pos(uint32_t r, const uint32_t (&rex)[TH], int vh, int vw,
                                          uint32_t mlo, uint32_t mhi, uint32_t rexv)
{
    uint32_t cnt = 0;
#pragma unroll
    for (int y = 1; y < TH; ++y) cnt += (y < vh && rex[y] <= r) ? 1u : 0u;
    const int src = (int)cnt << 2;
    const uint64_t m = ((uint64_t)(uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)mhi) << 32) |
                       (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)mlo);
    const uint32_t k = r - (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)rexv);
    const uint32_t x = select_bit64_bs(m, k);
    const uint64_t above = (m >> x) >> 1;
    const uint32_t e = above ? x + (uint32_t)__builtin_ctzll(above) : (uint32_t)vw - 1u;
    return {cnt, x, e};
}
// one wave's statistics tables in the final write (they take the place of
// its label staging once the tile's rows are written)
struct FwTabs {
    union {
        // first pass: parts of the regions on the tile's edges, by seam slot
        struct {
            unsigned long long sum[KMAX], col[KMAX];
            uint32_t row[KMAX];
        } b;
        // then the regions inside the tile, by rank among the tile's inner
        // roots (reading order) minus the pass's first rank, and numbers
        struct {
            unsigned long long sum[SR_CAP], col[SR_CAP];
            uint32_t row[SR_CAP], num[SR_CAP];
        } in;
    } u;
    unsigned long long ir[TH];  // inner roots' start columns in each row
    uint32_t irpre[TH];         // inner roots in the rows before
};

// one wave's LDS in the final write
struct FwRows {  // while the rows are written: the labels of the first DLAB
                 // runs, the seam nodes' values (+ IGN_SLOT: the ignored value)
    uint32_t lab[DLAB];
    uint32_t node[KMAX + 1];
};
template <bool STATS> struct FwWave {
    union {
        FwRows rows;
        FwTabs tabs;  // then the statistics
    } u;
    uint64_t lead[TH];   // leaders of each row segment
    uint32_t pre[TH];    // leaders of the image before each row segment
    uint16_t pos[DLAB];  // start of each of the first DLAB runs: row << 6 | column
};
template <> struct FwWave<false> {
    union {
        FwRows rows;
    } u;
    uint64_t lead[TH];
    uint32_t pre[TH];
};

// a run's packed sums (as a part): area, sum of rows, sum of columns
__device__ __forceinline__ unsigned long long run_sums(uint32_t y, uint32_t x, uint32_t e)
{
    const uint32_t len = e - x + 1u;
    return (unsigned long long)len | ((unsigned long long)(len * y) << 11) |
           ((unsigned long long)(len * x + len * (len - 1u) / 2u) << 26);
}
// the columns x .. e of a row, as a mask
__device__ __forceinline__ unsigned long long run_cols(uint32_t x, uint32_t e)
{
    return (~0ull >> (63u - e)) & (~0ull << x);
}

// The statistics of a tile of several colours, once its labels are written:
// its run starts are in pos (the first DLAB runs), the words of its run
// records in info[] (two per word, as the final write loads them), the values
// and records of its seam nodes in nv[] and nrec[] (slot lane + 64k), the
// leaders of its row segments in lead[] / pre[].
//   First pass over the runs: each run of a region on the tile's edges adds
//   to its seam slot's part, and the inner roots (runs whose record names
//   themselves) are marked.  The parts then go to their seam nodes' record
//   slots (free once resolve has run) for the reduce pass, or, for a region
//   on the edges whose seam node no union touched, into its record, whole.
//   Then one pass per SR_CAP regions inside the tile: their records, whole.
__device__ __forceinline__ void fw_stats_mixed(const Geom &g, const Work &w, const StatsOut &so,
                                               uint32_t t, const TilePos &tp, uint32_t R,
                                               uint32_t mlo, uint32_t mhi, uint32_t rexv,
                                               const uint32_t (&info)[DLAB / 128],
                                               const uint32_t (&nv)[KMAX / 64],
                                               const uint64_t (&nrec)[KMAX / 64],
                                               const uint64_t *lead, const uint32_t *pre,
                                               const uint16_t *pos, FwTabs &L, int lane)
{
    const int vh = tp.vh, vw = tp.vw;
    const int64_t off = so.off[tp.b];
    const uint16_t *rinfo = w.runinfo + (size_t)t * TPX;
    for (int i = lane; i < KMAX; i += 64) {
        L.u.b.sum[i] = L.u.b.col[i] = 0ull;
        L.u.b.row[i] = 0u;
    }
    if (lane < TH) L.ir[lane] = 0ull;
    __syncwarp();
    // run base + lane (base a multiple of 64; every lane takes part): its
    // record, row, first and last column
    auto run_at = [&](uint32_t base, uint32_t &rec, uint32_t &y, uint32_t &x, uint32_t &e) {
        const uint32_t r = base + (uint32_t)lane;
        const uint32_t rc = r < R ? r : R - 1u;
        if (base < (uint32_t)DLAB) {
            const uint32_t b = base >> 6;  // wave-uniform
            const uint32_t word = b < 2 ? info[0] : b < 4 ? info[1] : b < 6 ? info[2] : info[3];
            const int src = (int)((((b & 1u) << 5) + ((uint32_t)lane >> 1)) << 2);
            const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)word);
            rec = (lane & 1) ? v >> 16 : v & 0xFFFFu;
            const uint32_t p = pos[rc];
            y = p >> 6;
            x = p & 63u;
            const int sy = (int)(y << 2);
            const uint64_t m = ((uint64_t)(uint32_t)__builtin_amdgcn_ds_bpermute(sy, (int)mhi) << 32) |
                               (uint32_t)__builtin_amdgcn_ds_bpermute(sy, (int)mlo);
            const uint64_t above = (m >> x) >> 1;
            e = above ? x + (uint32_t)__builtin_ctzll(above) : (uint32_t)vw - 1u;
        } else {
            // past the staged runs: decode here
            uint32_t rex[TH];
#pragma unroll
            for (int yy = 0; yy < TH; ++yy) rex[yy] = __builtin_amdgcn_readlane(rexv, yy);
            const RunPos p = run_pos(rc, rex, vh, vw, mlo, mhi, rexv);
            rec = rinfo[rc];
            y = p.y;
            x = p.x;
            e = p.e;
        }
    };
    static_assert(DLAB == 512, "four words of run records per lane");

    for (uint32_t base = 0; base < R; base += 64) {
        uint32_t rec, y, x, e;
        run_at(base, rec, y, x, e);
        if (base + (uint32_t)lane >= R || rec == INFO_IGNORED) continue;
        if (rec & INFO_BORDER) {
            const uint32_t sl_ = rec & 0xFFu;
            atomicAdd(&L.u.b.sum[sl_], run_sums(y, x, e));
            atomicOr(&L.u.b.row[sl_], 1u << y);
            atomicOr(&L.u.b.col[sl_], run_cols(x, e));
        } else if (rec == ((y << 6) | x)) {
            atomicOr(&L.ir[y], 1ull << x);
        }
    }
    __syncwarp();
#pragma unroll
    for (int k = 0; k < KMAX / 64; ++k) {
        const int i = lane + 64 * k;
        const unsigned long long sum = L.u.b.sum[i];
        if (sum == 0ull) continue;
        const uint64_t pk = pack_part(sum, L.u.b.row[i], L.u.b.col[i]);
        uint64_t *slot = w.gp + (size_t)t * KMAX + i;
        if (lone_node(nrec[k], (t << 8) | (uint32_t)i)) {
            const int64_t idx = off + (int64_t)nv[k] - 1;
            if ((uint64_t)idx < (uint64_t)so.cap) part_record(&so.rec[idx], pk, tp);
            *slot = 0ull;  // nothing left for the reduce pass
        } else {
            *slot = pk;
        }
    }
    // inner roots in the rows before each row
    const uint32_t nr = lane < TH ? popc64(L.ir[lane]) : 0u;
    uint32_t ninc = nr;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t v = __shfl_up(ninc, d);
        if (lane >= d) ninc += v;
    }
    if (lane < TH) L.irpre[lane] = ninc - nr;
    const uint32_t ni = __builtin_amdgcn_readlane(ninc, TH - 1);
    __syncwarp();  // (the edge tables are free: the inner tables take their place)

    for (uint32_t p0 = 0; p0 < ni; p0 += SR_CAP) {
        const uint32_t nin = ni - p0 < (uint32_t)SR_CAP ? ni - p0 : (uint32_t)SR_CAP;
        for (uint32_t i = lane; i < nin; i += 64) {
            L.u.in.sum[i] = L.u.in.col[i] = 0ull;
            L.u.in.row[i] = 0u;
        }
        __syncwarp();
        for (uint32_t base = 0; base < R; base += 64) {
            uint32_t rec, y, x, e;
            run_at(base, rec, y, x, e);
            if (base + (uint32_t)lane >= R || (rec & INFO_BORDER)) continue;  // (ignored too)
            const uint32_t ry = rec >> 6, rc = rec & 63u;
            const uint32_t rank = L.irpre[ry] + popc64(L.ir[ry] & mask_lt((int)rc));
            if (rank < p0 || rank >= p0 + nin) continue;
            const uint32_t k = rank - p0;
            if (ry == y && rc == x) L.u.in.num[k] = 1u + pre[ry] + popc64(lead[ry] & mask_lt((int)rc));
            atomicAdd(&L.u.in.sum[k], run_sums(y, x, e));
            atomicOr(&L.u.in.row[k], 1u << y);
            atomicOr(&L.u.in.col[k], run_cols(x, e));
        }
        __syncwarp();
        for (uint32_t i = lane; i < nin; i += 64) {
            const int64_t idx = off + (int64_t)L.u.in.num[i] - 1;
            if ((uint64_t)idx < (uint64_t)so.cap)
                part_record(&so.rec[idx], pack_part(L.u.in.sum[i], L.u.in.row[i], L.u.in.col[i]), tp);
        }
        __syncwarp();
    }
}

// ------------------------------------------------------------ final write
// One wave per tile: stage the tile's run labels in LDS (runs beyond DLAB are
// labelled from their records on the fly), then write the tile's rows, four
// pixels (16 bytes) per lane where rows are whole and 16-byte aligned.

// Label stores are streaming (non-temporal): the labels are not read again by
// this pass, so they should not take L2 space from the run records.
typedef int int4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_label4(int32_t *p, int4 v)
{
    const int4v vv = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(vv, (int4v *)p);
}
__device__ __forceinline__ void store_label(int32_t *p, int32_t v)
{
    __builtin_nontemporal_store(v, p);
}

// labels of the tile's rows y = lane/16, +4, ...: lane covers columns
// 4*(lane%16) .. +3.  rowmask/rowex: lane y holds row y's run starts and the
// runs before row y.
// With pos, the starts of the first DLAB runs (row << 6 | column) are written
// there too.
template <bool ALL_STAGED, typename L>
__device__ __forceinline__ void write_rows_x4(int32_t *o0, int64_t W, int vh, int lane,
                                              uint32_t mlo, uint32_t mhi, uint32_t rex,
                                              const uint32_t *lab, L run_label_slow,
                                              uint16_t *pos = nullptr)
{
    const int c4 = 4 * (lane & 15);
    for (int yb = 0; yb < vh; yb += 4) {  // the same trip count for every lane
        const int y = yb + (lane >> 4);
        const int ys = y < vh ? y : vh - 1;
        const uint64_t m = ((uint64_t)(uint32_t)__shfl((int)mhi, ys) << 32) | (uint32_t)__shfl((int)mlo, ys);
        const uint32_t rb = (uint32_t)__shfl((int)rex, ys);
        if (y >= vh) continue;
        const uint32_t bits = (uint32_t)(m >> c4) & 15u;
        const uint32_t r0 = rb + popc64(m & mask_le(c4)) - 1u;
        const uint32_t r1 = r0 + ((bits >> 1) & 1u), r2 = r1 + ((bits >> 2) & 1u), r3 = r2 + (bits >> 3);
        if (pos != nullptr) {
            const uint16_t p0 = (uint16_t)(((uint32_t)y << 6) | (uint32_t)c4);
            if ((bits & 1u) && r0 < (uint32_t)DLAB) pos[r0] = p0;
            if ((bits & 2u) && r1 < (uint32_t)DLAB) pos[r1] = (uint16_t)(p0 + 1);
            if ((bits & 4u) && r2 < (uint32_t)DLAB) pos[r2] = (uint16_t)(p0 + 2);
            if ((bits & 8u) && r3 < (uint32_t)DLAB) pos[r3] = (uint16_t)(p0 + 3);
        }
        int4 v;
        if (ALL_STAGED) {
            v = make_int4((int)lab[r0], (int)lab[r1], (int)lab[r2], (int)lab[r3]);
        } else {
            v = make_int4((int)(r0 < DLAB ? lab[r0] : run_label_slow(r0)),
                          (int)(r1 < DLAB ? lab[r1] : run_label_slow(r1)),
                          (int)(r2 < DLAB ? lab[r2] : run_label_slow(r2)),
                          (int)(r3 < DLAB ? lab[r3] : run_label_slow(r3)));
        }
        store_label4(o0 + y * W + c4, v);
    }
}

// STATS: also the statistics of ccl_label_stats (numbers only)
template <bool STATS>
__global__ __launch_bounds__(BLOCK) void final_write_kernel(Geom g, Work w, int32_t *out,
                                                            int number, uint32_t ignv,
                                                            uint32_t t0, uint32_t t1, StatsOut so)
{
    __shared__ FwWave<STATS> sW[NWAVES];

    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t t = t0 + remap_tile(blockIdx.x, gridDim.x) * NWAVES + wave;
    if (t >= t1) return;  // tiles t0 .. t1-1
    const TilePos tp = tile_pos(t, g);
    const int64_t y0 = tp.y0, x0 = tp.x0, W = g.W;
    const size_t t32 = (size_t)t * TH;
    const uint16_t *rinfo = w.runinfo + (size_t)t * TPX;
    int32_t *o0 = out + (int64_t)tp.b * g.HW + y0 * W + x0;
    const bool lane_ok = lane < tp.vw;
    // 16-byte stores: whole tile rows whose starts are 16-byte aligned
    const bool x4 = tp.vw == TW && (W & 3) == 0 && ((uintptr_t)out & 15u) == 0;
    const TileHdr &h = w.hdr[t];
    const uint2 uv = *(const uint2 *)&h;  // kind, value

    if (uv.x & KIND_UNIFORM) {
        // one colour: every pixel carries the region's value (its seam
        // node's, unless the tile is the whole image)
        const bool seam = tp.ty > 0 || tp.tx > 0 || y0 + TH < g.H || x0 + TW < W;
        uint32_t v = uv.y;
        if (!seam) v = number == 1 ? 1u + h.pre : (uint32_t)(y0 * W + x0);
        else if (number == 2) v = (uint32_t)(h.rec >> 32) & 0x7FFFFFFFu;  // its root's key
        if (uv.x & KIND_IGNORED) v = ignv;
        if (x4) {
            const int4 v4 = make_int4((int)v, (int)v, (int)v, (int)v);
            for (int y = lane >> 4; y < tp.vh; y += 4) store_label4(o0 + y * W + 4 * (lane & 15), v4);
        } else if (lane_ok) {
            for (int y = 0; y < tp.vh; ++y) store_label(o0 + y * W + lane, (int32_t)v);
        }
        if constexpr (STATS) {
            // the record of a region that is this tile alone: the whole image,
            // or a seam node no union touched
            if (lane == 0 && !(uv.x & KIND_IGNORED) &&
                (!seam || lone_node(h.rec, (t << 8) | UNI_SLOT))) {
                const int64_t idx = so.off[tp.b] + (int64_t)v - 1;
                if ((uint64_t)idx < (uint64_t)so.cap) tile_record(&so.rec[idx], tp);
            }
        }
        return;
    }

    const uint32_t R = uv.y;                 // a tile of several colours: its runs
    const uint32_t nslots = (uv.x >> 8) & 0xFFu;  // 1 + its highest seam slot in use
    FwWave<STATS> &lw = sW[wave];
    uint32_t *lab = lw.u.rows.lab;
    uint32_t *nodev = lw.u.rows.node;
    uint64_t *lead = lw.lead;
    uint32_t *pre = lw.pre;
    // every record of the tile is requested before any is used, so that their
    // latencies overlap
    const uint64_t mk = lane < TH ? w.runmask[t32 + lane] : 0ull;
    const uint64_t ld = (number == 1 && lane < TH) ? w.leadmask[t32 + lane] : 0ull;
    const uint32_t pr = (number == 1 && lane < TH) ? w.seg[t32 + lane] : 0u;
    uint64_t used[KMAX / 64];
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word) used[word] = h.used[word];
    // buffer loads bounded by the used seam slots and the run count (from the
    // header's first eight bytes): lanes past them read 0 without touching
    // memory, and no branch splits the loads
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(w.nval + (size_t)t * KMAX), (short)0, (int)(nslots * 4u), 0x00020000);
    uint32_t nv[KMAX / 64];
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word)
        nv[word] = __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(word * 64 + lane) * 4u, 0, 0);
    if (number == 2) {  // leaders: each seam node's value is its root's key
#pragma unroll
        for (int word = 0; word < KMAX / 64; ++word) {
            const uint32_t i = (uint32_t)(word * 64 + lane);
            nv[word] = i < nslots ? (uint32_t)(w.gp[(size_t)t * KMAX + i] >> 32) & 0x7FFFFFFFu : 0u;
        }
    }
    const uint32_t nl = R < DLAB ? R : DLAB;
    // two 16-bit records per dword: lane l of load j holds runs 2(l + 64j) and
    // 2(l + 64j) + 1 (the bound is rounded up to whole dwords; a run past nl is
    // never used)
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)rinfo, (short)0, (int)((nl * 2u + 3u) & ~3u), 0x00020000);
    uint32_t info[DLAB / 128];
#pragma unroll
    for (int j = 0; j < DLAB / 128; ++j)
        info[j] = __builtin_amdgcn_raw_buffer_load_b32(rr, ((uint32_t)lane + 64u * (uint32_t)j) * 4u, 0, 0);
    uint64_t nrec[KMAX / 64];  // with statistics: the seam nodes' records
#pragma unroll
    for (int k = 0; k < KMAX / 64; ++k) {
        const uint32_t i = (uint32_t)(lane + 64 * k);
        nrec[k] = (STATS && i < nslots) ? w.gp[(size_t)t * KMAX + i] : 0ull;
    }
    if (number && lane < TH) {
        lead[lane] = ld;
        pre[lane] = pr;
    }
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word)
        if ((used[word] >> lane) & 1ull) nodev[word * 64 + lane] = nv[word];
    if (lane == 0) nodev[IGN_SLOT] = ignv;  // runs of an ignored colour read it
    __syncwarp();
    auto run_label = [&](uint32_t info) -> uint32_t {
        if (info & INFO_BORDER) return nodev[info & 0xFFu];
        const uint32_t row = info >> 6, col = info & 63u;
        if (number == 1) return 1u + pre[row] + popc64(lead[row] & mask_lt((int)col));
        return (uint32_t)((y0 + row) * W + x0 + col);
    };
#pragma unroll
    for (int j = 0; j < DLAB / 128; ++j) {
        const uint32_t r = 2u * ((uint32_t)lane + 64u * (uint32_t)j);
        if (r < nl) lab[r] = run_label(info[j] & 0xFFFFu);
        if (r + 1u < nl) lab[r + 1u] = run_label(info[j] >> 16);
    }
    __syncwarp();

    // runs before each row (lane y holds row y's)
    const uint32_t cnt = popc64(mk);
    uint32_t inc = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t v = __shfl_up(inc, d);
        if (lane >= d) inc += v;
    }
    const uint32_t rex = inc - cnt;
    const uint32_t mlo = (uint32_t)mk, mhi = (uint32_t)(mk >> 32);
    auto slow = [&](uint32_t run) -> uint32_t { return run_label(rinfo[run]); };
    uint16_t *pos = nullptr;  // with statistics: the run starts
    if constexpr (STATS) pos = lw.pos;
    if (x4) {
        if (R <= DLAB)
            write_rows_x4<true>(o0, W, tp.vh, lane, mlo, mhi, rex, lab, slow, pos);
        else
            write_rows_x4<false>(o0, W, tp.vh, lane, mlo, mhi, rex, lab, slow, pos);
    } else {
        for (int y = 0; y < tp.vh; ++y) {
            const uint64_t m = ((uint64_t)__builtin_amdgcn_readlane(mhi, y) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane(mlo, y);
            const uint32_t rb = __builtin_amdgcn_readlane(rex, y);
            if (lane_ok) {
                const uint32_t start = (uint32_t)((m >> lane) & 1ull);
                const uint32_t run = rb + mbcnt(m) + start - 1u;
                store_label(o0 + y * W + lane, (int32_t)(run < DLAB ? lab[run] : run_label(rinfo[run])));
                if (STATS && start && run < (uint32_t)DLAB)
                    pos[run] = (uint16_t)(((uint32_t)y << 6) | (uint32_t)lane);
            }
        }
    }
    if constexpr (STATS) {
        __syncwarp();  // (the label staging is done with: the tables take its place)
        fw_stats_mixed(g, w, so, t, tp, R, mlo, mhi, rex, info, nv, nrec, lead, pre, pos, lw.u.tabs,
                       lane);
    }
}

// ------------------------------------------------ 64-bit final write
// The final write of one band of a picture cut into bands (ccl_label_large,
// numbers): as above, the tile's runs are labelled once (their band-local
// numbers, through Map64, to the picture's 64-bit numbers) and expanded into
// rows; 8-byte labels, two per 16-byte store where rows are whole and aligned,
// 32 lanes to a row so that each store instruction covers two whole rows (with
// four pixels per lane, each instruction leaves every other 16 bytes of its
// rows to the next, and the non-temporal stores ran at 1.9 TB/s instead of 4.8).

__device__ __forceinline__ void store2_i64(int64_t *p, int64_t a, int64_t b)
{
    const int4v vv = {(int)(uint32_t)a, (int)(a >> 32), (int)(uint32_t)b, (int)(b >> 32)};
    __builtin_nontemporal_store(vv, (int4v *)p);
}

template <bool LEAD>
__global__ __launch_bounds__(BLOCK) void final_write64_kernel(Geom g, Work w, int64_t *out, Map64 m)
{
    __shared__ int64_t sLab[NWAVES][DLAB];
    __shared__ uint32_t sNode[NWAVES][KMAX + 1];
    __shared__ uint32_t sKey[LEAD ? NWAVES : 1][KMAX + 1];  // leaders: each seam node's root key
    __shared__ uint64_t sLead[NWAVES][TH];
    __shared__ uint32_t sPre[NWAVES][TH];

    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t t = remap_tile(blockIdx.x, gridDim.x) * NWAVES + wave;
    if (t >= (uint32_t)g.ntiles) return;
    const TilePos tp = tile_pos(t, g);
    const int64_t y0 = tp.y0, x0 = tp.x0, W = g.W;
    const size_t t32 = (size_t)t * TH;
    const uint16_t *rinfo = w.runinfo + (size_t)t * TPX;
    int64_t *o0 = out + (int64_t)tp.b * g.HW + y0 * W + x0;
    const bool lane_ok = lane < tp.vw;
    // 16-byte stores (two labels): whole tile rows whose starts are 16-byte aligned
    const bool x4 = tp.vw == TW && (W & 1) == 0 && ((uintptr_t)out & 15u) == 0;
    const int64_t G = m.merges ? m.G[m.band] : 0;
    // band-local number n to the picture's number (0: an ignored pixel), in
    // two steps so that many can be in flight: the mask and prefix words of n,
    // then (merged numbers only) its entry
    // (leaders: the band-local leader key travels with n; an ignored pixel,
    // n = 0, is -1)
    struct Pend {
        uint64_t word;
        uint32_t pre, n, key;
    };
    auto map_load = [&](uint32_t n, uint32_t key) -> Pend {
        Pend q{0ull, 0u, n, key};
        if (n != 0u && m.merges) {
            q.word = m.M[n >> 6];
            q.pre = m.Mpre[n >> 6];
        }
        return q;
    };
    auto map_done = [&](const Pend &q) -> int64_t {
        if (q.n == 0u) return LEAD ? -1 : 0;
        if (!m.merges) return LEAD ? (int64_t)q.key : (int64_t)q.n;
        const uint32_t r = q.pre + popc64(q.word & mask_lt((int)(q.n & 63u)));
        if ((q.word >> (q.n & 63u)) & 1ull) return m.MV[r];
        return LEAD ? m.base + (int64_t)q.key : G + (int64_t)q.n - (int64_t)r;
    };
    auto map = [&](uint32_t n, uint32_t key) -> int64_t { return map_done(map_load(n, key)); };
    const TileHdr &h = w.hdr[t];
    const uint2 uv = *(const uint2 *)&h;  // kind, value

    if (uv.x & KIND_UNIFORM) {
        const bool seam = tp.ty > 0 || tp.tx > 0 || y0 + TH < g.H || x0 + TW < W;
        uint32_t v = uv.y;
        if (!seam) v = 1u + h.pre;
        if (uv.x & KIND_IGNORED) v = 0u;
        // (leaders: its root's key, or its first pixel if the tile is the band)
        const uint32_t key = seam ? (uint32_t)(h.rec >> 32) & 0x7FFFFFFFu : (uint32_t)(y0 * W + x0);
        const int64_t v64 = map(v, key);
        if (x4) {
            for (int y = lane >> 5; y < tp.vh; y += 2) store2_i64(o0 + y * W + 2 * (lane & 31), v64, v64);
        } else if (lane_ok) {
            for (int y = 0; y < tp.vh; ++y) __builtin_nontemporal_store(v64, o0 + y * W + lane);
        }
        return;
    }

    const uint32_t R = uv.y;
    const uint32_t nslots = (uv.x >> 8) & 0xFFu;
    int64_t *lab = sLab[wave];
    uint32_t *nodev = sNode[wave];
    uint64_t *lead = sLead[wave];
    uint32_t *pre = sPre[wave];
    const uint64_t mk = lane < TH ? w.runmask[t32 + lane] : 0ull;
    const uint64_t ld = lane < TH ? w.leadmask[t32 + lane] : 0ull;
    const uint32_t pr = lane < TH ? w.seg[t32 + lane] : 0u;
    uint64_t used[KMAX / 64];
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word) used[word] = h.used[word];
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(w.nval + (size_t)t * KMAX), (short)0, (int)(nslots * 4u), 0x00020000);
    uint32_t nv[KMAX / 64];
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word)
        nv[word] = __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(word * 64 + lane) * 4u, 0, 0);
    const uint32_t nl = R < DLAB ? R : DLAB;
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)rinfo, (short)0, (int)((nl * 2u + 3u) & ~3u), 0x00020000);
    uint32_t info[DLAB / 128];
#pragma unroll
    for (int j = 0; j < DLAB / 128; ++j)
        info[j] = __builtin_amdgcn_raw_buffer_load_b32(rr, ((uint32_t)lane + 64u * (uint32_t)j) * 4u, 0, 0);
    if (lane < TH) {
        lead[lane] = ld;
        pre[lane] = pr;
    }
    uint32_t nk[KMAX / 64] = {0u, 0u, 0u};
    if constexpr (LEAD) {
#pragma unroll
        for (int word = 0; word < KMAX / 64; ++word) {
            const uint32_t i = (uint32_t)(word * 64 + lane);
            nk[word] = i < nslots ? (uint32_t)(w.gp[(size_t)t * KMAX + i] >> 32) & 0x7FFFFFFFu : 0u;
        }
    }
    uint32_t *nodek = sKey[LEAD ? wave : 0];
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word)
        if ((used[word] >> lane) & 1ull) {
            nodev[word * 64 + lane] = nv[word];
            if (LEAD) nodek[word * 64 + lane] = nk[word];
        }
    if (lane == 0) nodev[IGN_SLOT] = 0u;  // runs of an ignored colour
    __syncwarp();
    auto run_number = [&](uint32_t inf) -> uint32_t {
        if (inf & INFO_BORDER) return nodev[inf & 0xFFu];
        const uint32_t row = inf >> 6, col = inf & 63u;
        return 1u + pre[row] + popc64(lead[row] & mask_lt((int)col));
    };
    // leaders: the band-local key of the run's leader (a run of an ignored
    // colour has none, and its number 0 decides)
    auto run_key = [&](uint32_t inf) -> uint32_t {
        if (!LEAD) return 0u;
        if (inf & INFO_BORDER) return (inf & 0xFFu) < IGN_SLOT ? nodek[inf & 0xFFu] : 0u;
        const uint32_t row = inf >> 6, col = inf & 63u;
        return (uint32_t)((y0 + row) * W + x0 + col);
    };
    Pend pq[DLAB / 64];  // the lane's staged runs, all requested before any is used
#pragma unroll
    for (int j = 0; j < DLAB / 128; ++j) {
        const uint32_t r = 2u * ((uint32_t)lane + 64u * (uint32_t)j);
        const uint32_t i0 = info[j] & 0xFFFFu, i1 = info[j] >> 16;
        pq[2 * j] = map_load(r < nl ? run_number(i0) : 0u, run_key(i0));
        pq[2 * j + 1] = map_load(r + 1u < nl ? run_number(i1) : 0u, run_key(i1));
    }
#pragma unroll
    for (int j = 0; j < DLAB / 128; ++j) {
        const uint32_t r = 2u * ((uint32_t)lane + 64u * (uint32_t)j);
        if (r < nl) lab[r] = map_done(pq[2 * j]);
        if (r + 1u < nl) lab[r + 1u] = map_done(pq[2 * j + 1]);
    }
    __syncwarp();

    const uint32_t cnt = popc64(mk);
    uint32_t inc = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t v = __shfl_up(inc, d);
        if (lane >= d) inc += v;
    }
    const uint32_t rex = inc - cnt;
    const uint32_t mlo = (uint32_t)mk, mhi = (uint32_t)(mk >> 32);
    auto label_of = [&](uint32_t run) -> int64_t {
        if (run < (uint32_t)DLAB) return lab[run];
        const uint32_t inf = rinfo[run];
        return map(run_number(inf), run_key(inf));
    };
    if (x4) {
        const int c2 = 2 * (lane & 31);
        for (int yb = 0; yb < tp.vh; yb += 2) {  // the same trip count for every lane
            const int y = yb + (lane >> 5);
            const int ys = y < tp.vh ? y : tp.vh - 1;
            const uint64_t mm = ((uint64_t)(uint32_t)__shfl((int)mhi, ys) << 32) | (uint32_t)__shfl((int)mlo, ys);
            const uint32_t rb = (uint32_t)__shfl((int)rex, ys);
            if (y >= tp.vh) continue;
            const uint32_t r0 = rb + popc64(mm & mask_le(c2)) - 1u;
            const uint32_t r1 = r0 + (uint32_t)((mm >> (c2 + 1)) & 1ull);
            store2_i64(o0 + y * W + c2, label_of(r0), label_of(r1));
        }
        return;
    }
    for (int y = 0; y < tp.vh; ++y) {
        const uint64_t mm = ((uint64_t)__builtin_amdgcn_readlane(mhi, y) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane(mlo, y);
        const uint32_t rb = __builtin_amdgcn_readlane(rex, y);
        if (lane_ok) {
            const uint32_t run = rb + mbcnt(mm) + (uint32_t)((mm >> lane) & 1ull) - 1u;
            __builtin_nontemporal_store(label_of(run), o0 + y * W + lane);
        }
    }
}

// ------------------------------------------------ standalone number/count
// A leader image has no tiles of its own; its row segments use the same
// tile-major layout so that the same scan numbers them.  One wave per row
// segment: a ballot of "leaders[p] == p".

// Each wave takes LF_U consecutive row segments of one tile at a time (the
// segment count per tile, 32, is a multiple of LF_U), all their loads issued
// before the first ballot.
constexpr int LF_U = 8;
static_assert(TH % LF_U == 0, "a wave's segments lie in one tile");

__global__ __launch_bounds__(BLOCK) void leader_flag_kernel(const int32_t *leaders, Geom g,
                                                            Work w, int write_mask, int clear_err)
{
    // the call's first kernel (of its first pass of images) clears the error word
    if (clear_err && blockIdx.x == 0 && threadIdx.x == 0) *w.err = 0u;
    clear_bands(g, w);
    const int lane = lane_id();
    const uint64_t nsegs = (uint64_t)g.ntiles * TH;
    const uint64_t nw = (uint64_t)gridDim.x * NWAVES;
    for (uint64_t sg0 = ((uint64_t)blockIdx.x * NWAVES + (threadIdx.x >> 6)) * LF_U; sg0 < nsegs;
         sg0 += nw * LF_U) {
        const uint32_t t = (uint32_t)(sg0 / TH), y0 = (uint32_t)(sg0 % TH);
        const TilePos tp = tile_pos(t, g);
        const int64_t X = tp.x0 + lane;
        const int32_t *base = leaders + (int64_t)tp.b * g.HW;
        int32_t v[LF_U];
#pragma unroll
        for (int u = 0; u < LF_U; ++u) {
            const int64_t Y = tp.y0 + y0 + u;
            v[u] = ((int)(y0 + u) < tp.vh && lane < tp.vw) ? base[Y * g.W + X] : -1;
        }
        uint32_t cnt = 0;
        uint64_t mask = 0;  // lane u keeps segment u's
#pragma unroll
        for (int u = 0; u < LF_U; ++u) {
            const int64_t Y = tp.y0 + y0 + u;
            const uint64_t m = __ballot(v[u] >= 0 && (int64_t)v[u] == Y * g.W + X);
            cnt = lane == u ? popc64(m) : cnt;
            mask = lane == u ? m : mask;
        }
        if (lane < LF_U) {
            w.seg[sg0 + lane] = cnt;
            if (write_mask) w.leadmask[sg0 + lane] = mask;
        }
    }
}

// One workgroup per image row at a time; each thread takes LA_U pixels of the
// row BLOCK apart, all their leaders' loads, then all their segment words'
// loads, issued before the first is used.  Where a wave's 64 pixels share one
// leader (the inside of a large region: on a drawing, most of the paper), the
// number is computed once, from segment words read through the scalar cache:
// every such wave of a region reads the same two words, which as vector loads
// all queue at one L2 channel.
constexpr int LA_U = 4;
typedef __attribute__((address_space(4))) const uint32_t const_u32;
typedef __attribute__((address_space(4))) const uint64_t const_u64;

__global__ __launch_bounds__(BLOCK) void leader_assign_kernel(const int32_t *leaders,
                                                              int32_t *labels, Geom g, Work w)
{
    const int64_t nrows = g.B * g.H;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const uint32_t b = (uint32_t)(row / g.H);
        for (int64_t x0 = threadIdx.x; x0 < g.W; x0 += (int64_t)BLOCK * LA_U) {
            int32_t v[LA_U];
#pragma unroll
            for (int u = 0; u < LA_U; ++u) {
                const int64_t x = x0 + (int64_t)u * BLOCK;
                v[u] = x < g.W ? leaders[row * g.W + x] : -1;
            }
            uint32_t sg[LA_U], col[LA_U];
            uint64_t lm[LA_U];
            bool ok[LA_U];
            int32_t one[LA_U];  // the wave's label where all its pixels share a leader
            uint64_t uni = 0;   // bit u: they do
#pragma unroll
            for (int u = 0; u < LA_U; ++u) {
                // a value outside the image (an ignored pixel's -1) is never
                // dereferenced and gets 0
                const int32_t v0 = __builtin_amdgcn_readfirstlane(v[u]);
                one[u] = 0;
                sg[u] = 0u;
                lm[u] = 0ull;
                col[u] = 0u;
                ok[u] = false;
                if (__ballot(v[u] != v0) == 0ull) {
                    uni |= 1ull << u;
                    if (v0 >= 0 && (int64_t)v0 < g.HW) {
                        uint32_t tl, r, c;
                        pixel_tile((uint32_t)v0, b, g, tl, r, c);
                        const size_t si = (size_t)tl * TH + r;
                        const uint32_t sgs = ((const const_u32 *)w.seg)[si];
                        const uint64_t lms = ((const const_u64 *)w.leadmask)[si];
                        one[u] = (int32_t)(1u + sgs + popc64(lms & mask_lt((int)c)));
                    }
                } else {
                    ok[u] = v[u] >= 0 && (int64_t)v[u] < g.HW;
                    uint32_t tl = 0, r = 0, c = 0;
                    if (ok[u]) pixel_tile((uint32_t)v[u], b, g, tl, r, c);
                    const size_t si = (size_t)tl * TH + r;
                    sg[u] = ok[u] ? w.seg[si] : 0u;
                    lm[u] = ok[u] ? w.leadmask[si] : 0ull;
                    col[u] = c;
                }
            }
#pragma unroll
            for (int u = 0; u < LA_U; ++u) {
                const int64_t x = x0 + (int64_t)u * BLOCK;
                if (x < g.W)
                    labels[row * g.W + x] =
                        ((uni >> u) & 1ull) ? one[u]
                        : ok[u] ? (int32_t)(1u + sg[u] + popc64(lm[u] & mask_lt((int)col[u])))
                                : 0;
            }
        }
    }
}

__global__ void zero_i32_kernel(int32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// ------------------------------------------------------ region statistics
// Per-region area, bounding box and sums of row and column indices of a
// numbered labelling.  One workgroup per area of ST_ROWS x ST_COLS pixels of
// one image, taken in chunks of ST_CHUNK rows: each wave takes 64-pixel row
// segments, finds their runs of one label with a ballot, and adds each run to
// its label's entry in a hash table in LDS (local coordinates: every sum fits
// 32 bits).  A segment that is one run adds to a wave-uniform sum for its
// label instead (paper, the inside of large regions: one table update per
// change of label, not per segment).  Entries leave the table at the end of
// the area, or after a chunk once the table is half full (anti-aliased glyph
// rows put up to 20,000 labels in one area of the sheet); then the entries of
// regions that reach the last row taken so far stay (they may go on below)
// and the others leave:
//   - a region that touches no side of the area shared with another area is
//     complete: its record is written with plain stores;
//   - a region on a shared side is added to the region's record with atomics,
//     so a region that covers the whole picture takes one set per area.
// A run whose label finds neither its entry nor a free slot within ST_PROBES
// goes to the region's statistics at once, and from then on every entry of the
// workgroup is added with atomics.

constexpr int ST_COLS = 512, ST_ROWS = 256, ST_CHUNK = 8;
constexpr int ST_CAP = 1024;                       // labels per area in LDS
constexpr int ST_PROBES = 16;                      // slots a label tries before it gives up
constexpr uint32_t ST_FLUSH_AT = ST_CAP / 2;       // entries that trigger a write-out
constexpr int ST_SEGS = ST_COLS / TW;              // row segments per area row
constexpr int ST_SPW = ST_CHUNK * ST_SEGS / NWAVES;  // segments of a chunk per wave
static_assert((ST_CAP & (ST_CAP - 1)) == 0, "the hash table size is a power of two");

struct StatsArgs {
    const int32_t *labels;
    const int32_t *counts;
    const int64_t *off;        // [B] first record of each image
    RegionRec *rec;
    int64_t B, H, W, HW;
    int64_t n_total;           // entries of the outputs
    uint32_t ay, ax;           // areas per image column / row
};

__device__ __forceinline__ void stats_global(const StatsArgs &a, int64_t i, uint32_t n, uint64_t sy,
                                             uint64_t sx, int32_t y0, int32_t x0, int32_t y1,
                                             int32_t x1)
{
    RegionRec &r = a.rec[i];
    atomicAdd(&r.sum_y, (unsigned long long)sy);
    atomicAdd(&r.sum_x, (unsigned long long)sx);
    atomicAdd(&r.area, (int32_t)n);
    atomicMin(&r.y0, y0);
    atomicMin(&r.x0, x0);
    atomicMax(&r.y1, y1);
    atomicMax(&r.x1, x1);
}

__global__ __launch_bounds__(BLOCK) void stats_kernel(StatsArgs a)
{
    __shared__ uint32_t sKey[ST_CAP];                    // label, 0: free
    __shared__ unsigned long long sNY[ST_CAP];           // area | (sum of local rows << 32)
    __shared__ uint32_t sSX[ST_CAP];                     // sum of local columns
    __shared__ uint32_t sY0[ST_CAP], sX0[ST_CAP], sY1[ST_CAP], sX1[ST_CAP];
    __shared__ uint32_t sUsed;                           // entries in use
    __shared__ uint32_t sSpill;                          // some run went to the global statistics
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const uint32_t per_img = a.ay * a.ax;
    const uint32_t b = blockIdx.x / per_img, rem = blockIdx.x - b * per_img;
    const uint32_t by = rem / a.ax, bx = rem - by * a.ax;
    const int32_t Y0 = (int32_t)(by * ST_ROWS), X0 = (int32_t)(bx * ST_COLS);
    const int32_t W = (int32_t)a.W, H = (int32_t)a.H;
    const int32_t nrows = min(ST_ROWS, H - Y0), ncols = min(ST_COLS, W - X0);
    const int32_t nmax = a.counts[b];
    const int64_t off = a.off[b] - 1;                    // entry of label k: off + k
    const int32_t *img = a.labels + (int64_t)b * a.HW;
    const bool up = Y0 > 0, down = Y0 + nrows < H, left = X0 > 0, right = X0 + ncols < W;

    auto clear = [&]() {
        for (int i = threadIdx.x; i < ST_CAP; i += BLOCK) {
            sKey[i] = 0u;
            sNY[i] = 0ull;
            sSX[i] = 0u;
            sY0[i] = sX0[i] = 0xFFFFFFFFu;
            sY1[i] = sX1[i] = 0u;
        }
        if (threadIdx.x == 0) sUsed = 0u;
    };
    clear();
    if (threadIdx.x == 0) sSpill = 0u;
    __syncthreads();

    // one run's contribution (local coordinates) to its label's entry, or to
    // the region's global statistics if the table has no room for the label
    auto add = [&](int32_t v, uint32_t n, uint32_t syl, uint32_t sxl, uint32_t y0, uint32_t x0,
                   uint32_t y1, uint32_t x1) {
        uint32_t h = ((uint32_t)v * 2654435761u) >> (32 - 10);
        static_assert(ST_CAP == 1024, "the hash takes 10 bits");
        int e = -1;
        for (int p = 0; p < ST_PROBES; ++p, h = (h + 1u) & (ST_CAP - 1)) {
            const uint32_t k = sKey[h];
            if (k == (uint32_t)v) { e = (int)h; break; }
            if (k == 0u) {
                const uint32_t old = atomicCAS(&sKey[h], 0u, (uint32_t)v);
                if (old == 0u) atomicAdd(&sUsed, 1u);
                if (old == 0u || old == (uint32_t)v) { e = (int)h; break; }
            }
        }
        if (e < 0) {
            sSpill = 1u;
            stats_global(a, off + v, n, (uint64_t)syl + (uint64_t)n * (uint64_t)Y0,
                         (uint64_t)sxl + (uint64_t)n * (uint64_t)X0, Y0 + (int32_t)y0,
                         X0 + (int32_t)x0, Y0 + (int32_t)y1, X0 + (int32_t)x1);
            return;
        }
        atomicAdd(&sNY[e], (unsigned long long)n | ((unsigned long long)syl << 32));
        atomicAdd(&sSX[e], sxl);
        atomicMin(&sY0[e], y0);
        atomicMin(&sX0[e], x0);
        atomicMax(&sY1[e], y1);
        atomicMax(&sX1[e], x1);
    };

    // write out the entries of regions that do not reach row `keep` (-1: all),
    // returning in kept[] the slots of those that do
    constexpr int SLOTS = ST_CAP / BLOCK;  // table slots per thread
    auto write_out = [&](int keep, bool (&kept)[SLOTS]) {
        const bool spill = sSpill != 0u;
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const int i = threadIdx.x + j * BLOCK;
            kept[j] = false;
            const uint32_t k = sKey[i];
            if (k == 0u) continue;
            if ((int)sY1[i] == keep) {
                kept[j] = true;
                continue;
            }
            const unsigned long long ny = sNY[i];
            const uint32_t n = (uint32_t)ny, syl = (uint32_t)(ny >> 32);
            const uint32_t y0 = sY0[i], x0 = sX0[i], y1 = sY1[i], x1 = sX1[i];
            const uint64_t sy = (uint64_t)syl + (uint64_t)n * (uint64_t)Y0;
            const uint64_t sx = (uint64_t)sSX[i] + (uint64_t)n * (uint64_t)X0;
            const int64_t e = off + (int64_t)k;
            const bool open = (up && y0 == 0u) || (down && y1 == (uint32_t)(nrows - 1)) ||
                              (left && x0 == 0u) || (right && x1 == (uint32_t)(ncols - 1));
            if (open || spill) {
                stats_global(a, e, n, sy, sx, Y0 + (int32_t)y0, X0 + (int32_t)x0,
                             Y0 + (int32_t)y1, X0 + (int32_t)x1);
            } else {  // the whole record, five 8-byte stores
                uint64_t *r = (uint64_t *)&a.rec[e];
                r[0] = sy;
                r[1] = sx;
                r[2] = (uint64_t)n | ((uint64_t)(uint32_t)(Y0 + (int32_t)y0) << 32);
                r[3] = (uint64_t)(uint32_t)(X0 + (int32_t)x0) | ((uint64_t)(uint32_t)(Y0 + (int32_t)y1) << 32);
                r[4] = (uint64_t)(uint32_t)(X0 + (int32_t)x1);
            }
        }
    };

    bool kept[SLOTS];
    for (int r0 = 0; r0 < nrows; r0 += ST_CHUNK) {
        const int r1 = min(nrows, r0 + ST_CHUNK);
        // the wave's open sum for one-run segments (label cv, 0: none)
        int32_t cv = 0;
        uint32_t cn = 0, csy = 0, csx = 0, cy0 = 0, cx0 = 0, cy1 = 0, cx1 = 0;
        // the wave's segments of the chunk: all their loads first, so that they
        // are in flight together (one at a time, the pass ran at 1.6 TB/s)
        int32_t vv[ST_SPW];
#pragma unroll
        for (int u = 0; u < ST_SPW; ++u) {
            const int sg = r0 * ST_SEGS + wave + u * NWAVES;
            const int ly = sg / ST_SEGS, lx = (sg - ly * ST_SEGS) * TW + lane;
            vv[u] = (ly < r1 && lx < ncols) ? img[(int64_t)(Y0 + ly) * W + X0 + lx] : 0;
        }
#pragma unroll
        for (int u = 0; u < ST_SPW; ++u) {
            const int sg = r0 * ST_SEGS + wave + u * NWAVES;
            const int ly = sg / ST_SEGS, lx0 = (sg - ly * ST_SEGS) * TW;  // local row, first column
            const int lx = lx0 + lane;
            const bool in = ly < r1 && lx < ncols;
            const int32_t v = vv[u];
            // runs of one label in the segment: lane L starts one where the
            // label differs from lane L-1's (lane 0 always, if it has a pixel)
            const uint64_t valid = __ballot(in);
            const uint64_t st = (__ballot(from_left_lane((uint32_t)v) != (uint32_t)v) | 1ull) & valid;
            if (st == 1ull) {  // one run: the whole segment (its valid part)
                const int32_t v0 = __builtin_amdgcn_readfirstlane(v);
                if (v0 <= 0 || v0 > nmax || off + v0 >= a.n_total) continue;
                if (v0 != cv) {
                    if (cv != 0 && lane == 0) add(cv, cn, csy, csx, cy0, cx0, cy1, cx1);
                    cv = v0;
                    cn = csy = csx = 0;
                    cy0 = cx0 = 0xFFFFFFFFu;
                    cy1 = cx1 = 0;
                }
                const uint32_t len = popc64(valid);
                cn += len;
                csy += len * (uint32_t)ly;
                csx += len * (uint32_t)lx0 + len * (len - 1u) / 2u;
                cy0 = min(cy0, (uint32_t)ly);
                cx0 = min(cx0, (uint32_t)lx0);
                cy1 = max(cy1, (uint32_t)ly);
                cx1 = max(cx1, (uint32_t)lx0 + len - 1u);
                continue;
            }
            if (!lane_bit(st) || v <= 0 || v > nmax || off + v >= a.n_total) continue;
            // the run ends before the next start (or at the last valid lane)
            const uint64_t after = st & ~mask_le(lane);
            const int end = after ? (int)__builtin_ctzll(after) - 1 : 63 - (int)__builtin_clzll(valid);
            const uint32_t len = (uint32_t)(end - lane + 1);
            add(v, len, len * (uint32_t)ly, len * (uint32_t)lx + len * (len - 1u) / 2u,
                (uint32_t)ly, (uint32_t)lx, (uint32_t)ly, (uint32_t)(lx0 + end));
        }
        if (cv != 0 && lane == 0) add(cv, cn, csy, csx, cy0, cx0, cy1, cx1);
        __syncthreads();
        if (r1 < nrows && sUsed > ST_FLUSH_AT) {  // the same for every thread
            write_out(r1 - 1, kept);
            // the entries that stay, out of the table and back into the cleared one
            uint32_t kk[SLOTS], ksx[SLOTS], ky0[SLOTS], kx0[SLOTS], ky1[SLOTS], kx1[SLOTS];
            unsigned long long kny[SLOTS];
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                const int i = threadIdx.x + j * BLOCK;
                kk[j] = kept[j] ? sKey[i] : 0u;
                kny[j] = sNY[i];
                ksx[j] = sSX[i];
                ky0[j] = sY0[i];
                kx0[j] = sX0[i];
                ky1[j] = sY1[i];
                kx1[j] = sX1[i];
            }
            __syncthreads();
            clear();
            __syncthreads();
#pragma unroll
            for (int j = 0; j < SLOTS; ++j)
                if (kk[j] != 0u)
                    add((int32_t)kk[j], (uint32_t)kny[j], (uint32_t)(kny[j] >> 32), ksx[j], ky0[j],
                        kx0[j], ky1[j], kx1[j]);
            __syncthreads();
        }
    }
    write_out(-1, kept);
}

// Entries of every region start empty (area 0, box (INT32_MAX, INT32_MAX, -1,
// -1), sums 0); block 0 also writes the first entry of each image.
// Records of the first n_init regions set empty, and the first record of each
// image of the pass: after *carry records (the regions of the batch's earlier
// passes; 0 for the first pass), and *carry advanced past this pass's.
__global__ __launch_bounds__(BLOCK) void stats_init_kernel(StatsArgs a, int64_t n_init,
                                                           int64_t *off, uint32_t *err,
                                                           int64_t *carry, int first)
{
    // the call's first kernel (of its first pass of images)
    if (first && blockIdx.x == 0 && threadIdx.x == 0) *err = 0u;
    for (int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x; i < n_init;
         i += (int64_t)gridDim.x * BLOCK) {
        uint64_t *r = (uint64_t *)&a.rec[i];
        r[0] = r[1] = 0ull;                                      // sums
        r[2] = (uint64_t)2147483647u << 32;                      // area 0, y0 INT32_MAX
        r[3] = 2147483647u | ((uint64_t)0xFFFFFFFFu << 32);      // x0 INT32_MAX, y1 -1
        r[4] = 0xFFFFFFFFu;                                      // x1 -1, pad 0
    }
    if (blockIdx.x != 0) return;
    // exclusive prefix of the counts: thread j sums its chunk, a workgroup scan
    // of the chunk sums, then each thread writes its chunk's prefixes
    __shared__ uint32_t sWave[NWAVES];
    const int64_t base = first ? 0 : *carry;  // (read before the scan's barriers)
    const int64_t B = a.B;
    const int64_t per = (B + BLOCK - 1) / BLOCK;
    const int64_t j0 = (int64_t)threadIdx.x * per, j1 = min(B, j0 + per);
    int64_t sum = 0;
    for (int64_t j = j0; j < j1; ++j) sum += a.counts[j];
    // (the counts of one pass add up to fewer than 2^32 regions: each needs a
    // pixel and a pass has fewer than 2^24 tiles of 2048 pixels)
    uint32_t total;
    const uint32_t ex = block_exclusive_scan((uint32_t)sum, sWave, total);
    int64_t run = base + ex;
    for (int64_t j = j0; j < j1; ++j) {
        off[j] = run;
        run += a.counts[j];
    }
    if (threadIdx.x == 0) *carry = base + total;
}

// ------------------------------------ statistics in the labelling call
// ccl_label_stats computes the records of ccl_region_stats inside the
// labelling call, from the run records the final write expands (row masks and
// per-run records, already in hand there), not from the labels.  Three steps:
//   - resolve opens the record of every region with a seam node (its root
//     node does, once), and marks each root that other nodes reach;
//   - the final write with statistics, per tile: a region inside a tile of
//     several colours is complete there and gets its record whole, and so
//     does a region on the tile's edges whose seam node no union touched (a
//     one-colour tile too); the part of any other region is packed into 64
//     bits in its seam node's record slot (free once resolve has run);
//   - stats_reduce_kernel, one workgroup per group of 16 x 16 tiles: the
//     parts of the group's seam nodes (and of its one-colour tiles, in closed
//     form) are gathered per region in an LDS table and added to the records
//     with global atomics, so a region covering the picture takes one set of
//     atomics per group.

// first record of each image: exclusive prefix of the per-image region counts
// the first record of each image of the pass (after *carry records of the
// batch's earlier passes; 0 for the first), and *carry advanced past this
// pass's regions
__global__ __launch_bounds__(BLOCK) void image_offsets_kernel(const int32_t *counts, int64_t B,
                                                             int64_t *off, int64_t *carry,
                                                             int first)
{
    __shared__ uint32_t sWave[NWAVES];
    const int64_t base = first ? 0 : *carry;  // (read before the scan's barriers)
    const int64_t per = (B + BLOCK - 1) / BLOCK;
    const int64_t j0 = (int64_t)threadIdx.x * per, j1 = min(B, j0 + per);
    int64_t sum = 0;
    for (int64_t j = j0; j < j1; ++j) sum += counts[j];
    // (a batch has fewer than 2^32 regions: each needs a pixel and a batch has
    // fewer than 2^24 tiles of 2048 pixels in a pass)
    uint32_t total;
    int64_t run = base + block_exclusive_scan((uint32_t)sum, sWave, total);
    for (int64_t j = j0; j < j1; ++j) {
        off[j] = run;
        run += counts[j];
    }
    if (threadIdx.x == 0) *carry = base + total;
}

constexpr int RD_CAP = 1024;   // regions of a block gathered in LDS
constexpr int RD_PROBES = 16;  // table slots a region tries before its part goes to the record

__device__ __forceinline__ void stats_add_global(RegionRec &r, uint32_t a, uint64_t sy, uint64_t sx,
                                                 int32_t y0, int32_t x0, int32_t y1, int32_t x1)
{
    atomicAdd(&r.sum_y, (unsigned long long)sy);
    atomicAdd(&r.sum_x, (unsigned long long)sx);
    atomicAdd(&r.area, (int32_t)a);
    atomicMin(&r.y0, y0);
    atomicMin(&r.x0, x0);
    atomicMax(&r.y1, y1);
    atomicMax(&r.x1, x1);
}

// groups of 16 x 16 tiles, one tile per thread: a region spread over the
// picture takes one set of global atomics per group
constexpr int RG = 16;
constexpr int RT = RG * RG;
static_assert(RT == BLOCK, "one thread per tile of a group");

__device__ __forceinline__ BlockTile group_tile(const Geom &g, uint32_t gb, int j)
{
    const uint32_t ngx = ((uint32_t)g.ntx + RG - 1) / RG, ngy = ((uint32_t)g.nty + RG - 1) / RG;
    const uint32_t per = ngx * ngy;
    const uint32_t b = gb / per, r = gb - b * per, gy = r / ngx, gx = r - gy * ngx;
    BlockTile p;
    p.ly = j / RG;
    p.lx = j % RG;
    const uint32_t ty = gy * RG + (uint32_t)p.ly, tx = gx * RG + (uint32_t)p.lx;
    p.valid = ty < (uint32_t)g.nty && tx < (uint32_t)g.ntx;
    p.t = b * (uint32_t)g.tpi + ty * (uint32_t)g.ntx + tx;
    return p;
}

__global__ __launch_bounds__(BLOCK) void stats_reduce_kernel(Geom g, Work w, StatsOut so)
{
    __shared__ uint32_t sKey[RD_CAP];  // region number, 0: free
    __shared__ unsigned long long sSY[RD_CAP], sSX[RD_CAP];
    __shared__ uint32_t sA[RD_CAP], sY0[RD_CAP], sX0[RD_CAP], sY1[RD_CAP], sX1[RD_CAP];
    __shared__ uint64_t sUsed[RT][KMAX / 64];
    __shared__ uint32_t sOff[RT];
    __shared__ uint8_t sUni[RT];
    __shared__ uint32_t sWave[NWAVES];
    const int j = threadIdx.x;
    const BlockTile me = group_tile(g, blockIdx.x, j);
    const int64_t off = so.off[fast_div(group_tile(g, blockIdx.x, 0).t, g.divTpi)];
    for (int i = j; i < RD_CAP; i += BLOCK) {
        sKey[i] = 0u;
        sSY[i] = sSX[i] = 0ull;
        sA[i] = sY1[i] = sX1[i] = 0u;
        sY0[i] = sX0[i] = 0x7FFFFFFFu;
    }
    // the block's seam nodes: a one-colour tile's (if it has an open edge and
    // is not of the ignored colour), or the used seam slots of a tile of
    // several colours
    uint32_t n = 0;
    bool uni = false;
    uint64_t u[KMAX / 64] = {0ull, 0ull, 0ull};
    if (me.valid) {
        const uint32_t kind = w.hdr[me.t].kind;
        uni = (kind & KIND_UNIFORM) != 0;
        if (uni) {
            n = (((kind >> 8) & 0xFFu) != 255u && !(kind & KIND_IGNORED)) ? 1u : 0u;
        } else {
#pragma unroll
            for (int word = 0; word < KMAX / 64; ++word) {
                u[word] = w.hdr[me.t].used[word];
                n += popc64(u[word]);
            }
        }
    }
#pragma unroll
    for (int word = 0; word < KMAX / 64; ++word) sUsed[j][word] = u[word];
    sUni[j] = uni ? 1 : 0;
    uint32_t total;
    sOff[j] = block_exclusive_scan(n, sWave, total);
    __syncthreads();
    for (uint32_t i = j; i < total; i += BLOCK) {
        const uint32_t jj = item_tile<RT>(sOff, i);
        const BlockTile bt = group_tile(g, blockIdx.x, (int)jj);
        const TilePos tp = tile_pos(bt.t, g);
        uint32_t number, a;
        uint64_t sy, sx;
        int32_t y0, x0, y1, x1;
        if (sUni[jj]) {
            if (lone_node(w.hdr[bt.t].rec, (bt.t << 8) | UNI_SLOT)) continue;  // done already
            number = w.hdr[bt.t].value;
            const int64_t vh = tp.vh, vw = tp.vw;
            a = (uint32_t)(vh * vw);
            sy = (uint64_t)(vw * (vh * (int64_t)tp.y0 + vh * (vh - 1) / 2));
            sx = (uint64_t)(vh * (vw * (int64_t)tp.x0 + vw * (vw - 1) / 2));
            y0 = (int32_t)tp.y0;
            x0 = (int32_t)tp.x0;
            y1 = (int32_t)(tp.y0 + vh - 1);
            x1 = (int32_t)(tp.x0 + vw - 1);
        } else {
            uint64_t uu[KMAX / 64];
#pragma unroll
            for (int word = 0; word < KMAX / 64; ++word) uu[word] = sUsed[jj][word];
            const uint32_t slot = select_bit(uu, i - sOff[jj]);
            number = w.nval[(size_t)bt.t * KMAX + slot];
            const uint64_t pk = w.gp[(size_t)bt.t * KMAX + slot];
            a = (uint32_t)(pk & 0x7FFu);
            if (a == 0u) continue;  // a region on this tile's edges alone: done already
            sy = ((pk >> 11) & 0x7FFFu) + (uint64_t)a * tp.y0;
            sx = ((pk >> 26) & 0xFFFFu) + (uint64_t)a * tp.x0;
            y0 = (int32_t)(tp.y0 + ((pk >> 42) & 31u));
            y1 = (int32_t)(tp.y0 + ((pk >> 47) & 31u));
            x0 = (int32_t)(tp.x0 + ((pk >> 52) & 63u));
            x1 = (int32_t)(tp.x0 + ((pk >> 58) & 63u));
        }
        // the region's entry in the table, or its record if none is free
        uint32_t hsh = (number * 2654435761u) >> (32 - 10);
        static_assert(RD_CAP == 1024, "the hash takes 10 bits");
        int e = -1;
        for (int p = 0; p < RD_PROBES; ++p, hsh = (hsh + 1u) & (RD_CAP - 1)) {
            const uint32_t k = sKey[hsh];
            if (k == number) { e = (int)hsh; break; }
            if (k == 0u) {
                const uint32_t old = atomicCAS(&sKey[hsh], 0u, number);
                if (old == 0u || old == number) { e = (int)hsh; break; }
            }
        }
        if (e < 0) {
            const int64_t idx = off + (int64_t)number - 1;
            if ((uint64_t)idx < (uint64_t)so.cap) stats_add_global(so.rec[idx], a, sy, sx, y0, x0, y1, x1);
            continue;
        }
        atomicAdd(&sSY[e], (unsigned long long)sy);
        atomicAdd(&sSX[e], (unsigned long long)sx);
        atomicAdd(&sA[e], a);
        atomicMin(&sY0[e], (uint32_t)y0);
        atomicMin(&sX0[e], (uint32_t)x0);
        atomicMax(&sY1[e], (uint32_t)y1);
        atomicMax(&sX1[e], (uint32_t)x1);
    }
    __syncthreads();
    for (int i = j; i < RD_CAP; i += BLOCK) {
        const uint32_t k = sKey[i];
        if (k == 0u) continue;
        const int64_t idx = off + (int64_t)k - 1;
        if ((uint64_t)idx >= (uint64_t)so.cap) continue;
        stats_add_global(so.rec[idx], sA[i], sSY[i], sSX[i], (int32_t)sY0[i], (int32_t)sX0[i],
                         (int32_t)sY1[i], (int32_t)sX1[i]);
    }
}

// ------------------------------------------------------------- launchers

static inline unsigned grid_of(int64_t n, int64_t per)
{
    return (unsigned)((n + per - 1) / per);
}

template <typename T, int CONN>
static void launch_tile_t(const void *img, int ignore, uint32_t ign, const Geom &g, const Work &w,
                          int clear_err, hipStream_t s, uint32_t t0, uint32_t nt)
{
    const dim3 grid(nt), block(BLOCK);
    const TileArgs<T> a{(const T *)img, g, w, ign, (uint32_t)(clear_err != 0), t0};
    if (ignore)
        hipLaunchKernelGGL((tile_label_kernel<T, CONN, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((tile_label_kernel<T, CONN, false>), grid, block, 0, s, a);
}

void launch_tile(const void *img, int dtype_bytes, int conn, int ignore, uint32_t ign,
                 const Geom &g, const Work &w, int clear_err, hipStream_t s, uint32_t t0,
                 uint32_t nt)
{
    const int c = clear_err;
    if (nt == 0) nt = (uint32_t)g.ntiles;
    if (dtype_bytes == 1) {
        if (conn == 8) launch_tile_t<uint8_t, 8>(img, ignore, ign, g, w, c, s, t0, nt);
        else launch_tile_t<uint8_t, 4>(img, ignore, ign, g, w, c, s, t0, nt);
    } else if (dtype_bytes == 3) {
        if (conn == 8) launch_tile_t<Rgb24, 8>(img, ignore, ign, g, w, c, s, t0, nt);
        else launch_tile_t<Rgb24, 4>(img, ignore, ign, g, w, c, s, t0, nt);
    } else {
        if (conn == 8) launch_tile_t<uint32_t, 8>(img, ignore, ign, g, w, c, s, t0, nt);
        else launch_tile_t<uint32_t, 4>(img, ignore, ign, g, w, c, s, t0, nt);
    }
}

void launch_seam(const Geom &g, const Work &w, int conn, hipStream_t s)
{
    const int64_t blocks = g.B * ((g.nty + MB - 1) / MB) * ((g.ntx + MB - 1) / MB);
    // few blocks (small images, small batches): each block's global unions are
    // dealt over up to 16 workgroups, so that about 2048 are in flight
    const int64_t want = (2048 + blocks - 1) / blocks;
    const uint32_t slices = (uint32_t)(want < 1 ? 1 : want > 16 ? 16 : want);
    const dim3 grid((unsigned)(blocks * slices));
    hipLaunchKernelGGL(block_merge_kernel, grid, dim3(BLOCK), 0, s, g, w, conn, slices);
    // images of one block each (at most 8 x 8 tiles) have no block borders
    if (g.ntx > MB || g.nty > MB)
        hipLaunchKernelGGL(border_merge_kernel, grid, dim3(BLOCK), 0, s, g, w, conn, slices);
}

// tiles per workgroup of the roots and resolve passes: SEAM_TILES, or fewer
// on small inputs, so that about 2048 workgroups walk their nodes at once
static uint32_t seam_tiles_per_wg(const Geom &g)
{
    const int64_t k = g.ntiles / 2048;
    return (uint32_t)(k < 1 ? 1 : k > SEAM_TILES ? SEAM_TILES : k);
}

void launch_seam_roots(const Geom &g, const Work &w, hipStream_t s)
{
    const uint32_t tpw = seam_tiles_per_wg(g);
    hipLaunchKernelGGL(seam_roots_kernel, dim3(grid_of(g.ntiles, tpw)), dim3(BLOCK), 0, s, g, w, tpw);
}

void launch_scan(const Geom &g, const Work &w, int32_t *counts, int apply, int use_hdr,
                 hipStream_t s)
{
    // launches of at most 2^21 bands (a launch stays below 2^32 threads); a
    // band's look-back finds the bands of earlier launches finished
    constexpr int64_t PER_LAUNCH = int64_t(1) << 21;
    for (int64_t b0 = 0; b0 < g.nbands; b0 += PER_LAUNCH) {
        const int64_t n = g.nbands - b0 < PER_LAUNCH ? g.nbands - b0 : PER_LAUNCH;
        hipLaunchKernelGGL(scan_kernel, dim3((unsigned)n), dim3(SCAN_BLOCK), 0, s, g, w, counts,
                           apply, use_hdr, (uint32_t)b0);
    }
}

void launch_resolve(const Geom &g, const Work &w, int number, hipStream_t s, RegionRec *rec,
                    int64_t cap)
{
    const StatsOut so{rec, cap, (const int64_t *)w.bandst};
    const uint32_t tpw = seam_tiles_per_wg(g);
    hipLaunchKernelGGL(resolve_kernel, dim3(grid_of(g.ntiles, tpw)), dim3(BLOCK), 0, s, g, w, number,
                       so, tpw);
}

void launch_final64(const Geom &g, const Work &w, int64_t *out, const Map64 &m, int lead,
                    hipStream_t s)
{
    if (lead)
        hipLaunchKernelGGL(final_write64_kernel<true>, dim3(grid_of(g.ntiles, NWAVES)), dim3(BLOCK),
                           0, s, g, w, out, m);
    else
        hipLaunchKernelGGL(final_write64_kernel<false>, dim3(grid_of(g.ntiles, NWAVES)),
                           dim3(BLOCK), 0, s, g, w, out, m);
}

void launch_final(const Geom &g, const Work &w, int32_t *out, int number, uint32_t ignv,
                  hipStream_t s, uint32_t t0, uint32_t nt)
{
    if (nt == 0) nt = (uint32_t)g.ntiles;
    const StatsOut none{nullptr, 0, nullptr};
    hipLaunchKernelGGL(final_write_kernel<false>, dim3(grid_of(nt, NWAVES)), dim3(BLOCK), 0, s, g,
                       w, out, number, ignv, t0, t0 + nt, none);
}

void launch_leader_flags(const int32_t *leaders, const Geom &g, const Work &w, int write_mask,
                         int clear_err, hipStream_t s)
{
    int64_t blocks = grid_of(g.ntiles * (TH / LF_U), NWAVES);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(leader_flag_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, s, leaders, g,
                       w, write_mask, clear_err);
}

void launch_leader_assign(const int32_t *leaders, int32_t *labels, const Geom &g, const Work &w,
                          hipStream_t s)
{
    int64_t blocks = g.B * g.H;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(leader_assign_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, s, leaders,
                       labels, g, w);
}

// the regions counted by the batch's passes so far, carried from pass to pass
// in the workspace's first 256 bytes (after the error word), which every
// pass's layout shares
static int64_t *pass_carry(const Work &w) { return (int64_t *)((char *)w.err + 8); }

void launch_region_stats(const int32_t *labels, const int32_t *counts, const Geom &g,
                         const Work &w, int64_t n_total, RegionRec *recs, int first, hipStream_t s)
{
    StatsArgs a;
    a.labels = labels;
    a.counts = counts;
    a.off = (const int64_t *)w.bandst;
    a.rec = recs;
    a.B = g.B;
    a.H = g.H;
    a.W = g.W;
    a.HW = g.HW;
    a.n_total = n_total;
    a.ay = (uint32_t)((g.H + ST_ROWS - 1) / ST_ROWS);
    a.ax = (uint32_t)((g.W + ST_COLS - 1) / ST_COLS);
    // the first pass sets every record empty
    const int64_t n_init = first ? n_total : 0;
    int64_t iblocks = grid_of(n_init, BLOCK);
    if (iblocks > 4096) iblocks = 4096;
    if (iblocks < 1) iblocks = 1;
    hipLaunchKernelGGL(stats_init_kernel, dim3((unsigned)iblocks), dim3(BLOCK), 0, s, a, n_init,
                       (int64_t *)w.bandst, w.err, pass_carry(w), first);
    const int64_t blocks = g.B * (int64_t)a.ay * (int64_t)a.ax;
    hipLaunchKernelGGL(stats_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, s, a);
}

void launch_label_stats(const Geom &g, const Work &w, const int32_t *counts, int32_t *out,
                        RegionRec *rec, int64_t cap, int stage, int first, hipStream_t s)
{
    const StatsOut so{rec, cap, (const int64_t *)w.bandst};
    if (stage == 0) {
        hipLaunchKernelGGL(image_offsets_kernel, dim3(1), dim3(BLOCK), 0, s, counts, g.B,
                           (int64_t *)w.bandst, pass_carry(w), first);
    } else if (stage == 1) {
        hipLaunchKernelGGL(final_write_kernel<true>, dim3(grid_of(g.ntiles, NWAVES)), dim3(BLOCK), 0,
                           s, g, w, out, 1, 0u, 0u, (uint32_t)g.ntiles, so);
    } else {
        const int64_t blocks = g.B * ((g.nty + RG - 1) / RG) * ((g.ntx + RG - 1) / RG);
        hipLaunchKernelGGL(stats_reduce_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, s, g, w, so);
    }
}

void launch_zero_i32(int32_t *p, int64_t n, hipStream_t s)
{
    int64_t blocks = grid_of(n, BLOCK);
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0, s, p, n);
}

}  // namespace ccl
