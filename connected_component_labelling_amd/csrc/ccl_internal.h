// ccl_internal.h -- tile geometry, workspace layout and kernel launchers shared
// by the C ABI (ccl_api.hip) and the kernels (ccl_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ccl {

// A tile is 64 columns (one wave64 lane per column) by 32 rows.  The tile pass
// runs one 256-thread workgroup per tile (wave w loads rows 8w..8w+7); the
// final write runs one wave per tile; the seam passes run one lane per tile.
constexpr int TW = 64;
constexpr int TH = 32;
constexpr int NWAVES = 4;
constexpr int BLOCK = 64 * NWAVES;
constexpr int RPW = TH / NWAVES;            // rows per wave
constexpr int TPX = TW * TH;                // pixels (and at most runs) per tile
// Seam-node slots of a tile, one per position a region can touch an open edge
// through: top-row run k (k), bottom-row run k (64+k), first run of row y
// (128+y), last run of row y (160+y).  A region's slot is the smallest of its.
constexpr int KMAX = 2 * TW + 2 * TH;
constexpr int REQ_TOP = 2 * TW;             // seam requests along the top edge
constexpr int REQ_LEFT = 3 * TH;            // seam requests along the left edge
constexpr int REQMAX = REQ_TOP + REQ_LEFT;
constexpr int DLAB = 512;                   // run labels a final-write wave stages in LDS

static_assert(KMAX <= 255, "seam slots are stored in one byte");

// Seam node ids are (tile << 8) | slot.  Slots below KMAX are the regions of a
// tile of several colours, whose records are gp[tile*KMAX + slot]; a one-colour
// tile has one node, slot UNI_SLOT, whose record sits in its header.
constexpr uint32_t UNI_SLOT = 255;
// tiles of one pass of the pipeline: node ids (tile << 8 | slot) are 32-bit,
// and a launch of one 256-thread workgroup per tile stays below 2^32 threads
constexpr int64_t MAX_TILES = (int64_t(1) << 24) - 1;
static_assert(TH == 32 && TW == 64, "row masks are one wave64 ballot, tile rows are lanes");

// Bit layout of a per-run record (16 bits) written by the tile pass.
//   bit 15 set:   the run's region has seam node <slot> = bits 0..7
//   bit 15 clear: the region lies inside the tile; bits 0..10 = row*64+col of
//                 its first pixel (its tile-local root)
constexpr uint32_t INFO_BORDER = 0x8000u;
// A run of an ignored colour: a border record whose slot is IGN_SLOT, one past
// the last seam slot, where the final write keeps the ignored pixels' value.
constexpr uint32_t IGN_SLOT = KMAX;
constexpr uint32_t INFO_IGNORED = INFO_BORDER | IGN_SLOT;
static_assert(IGN_SLOT < UNI_SLOT, "the ignored slot is no seam slot");

// error word bits (first word of the workspace)
constexpr uint32_t ERR_LOOP = 1u;      // a find/union loop hit its safety bound

// Per-tile header, 64 bytes, written by the tile pass in one store.  A tile
// whose valid pixels all have one colour ("one-colour tile") writes nothing
// else: its runs, masks, edge slots and seam requests follow from the fields
// marked "one-colour" below.
struct TileHdr {
    uint32_t kind;      // bit 0: one-colour tile.  One-colour: bits 8..15 the slot of
                        //   its first open edge (255: none, so no seam node; its node
                        //   is slot UNI_SLOT); bit 1: a top-edge request at column 0
                        //   (8 neighbours), bit 2: that request goes up-left, bit 3:
                        //   the ignored colour (no node, no requests, no leader).
                        //   Otherwise bits 8..15: 1 + the highest seam slot in use
                        //   (0: none)
    uint32_t value;     // one-colour tile with a seam node: its pixels' value
                        //   (written by the resolve pass); otherwise its runs
    uint32_t nruns;     // runs in the tile
    uint32_t ntop;      // seam requests along the top edge
    uint32_t nleft;     // seam requests along the left edge
    uint32_t leftmask;  // one-colour: rows with a left-edge request
    union {
        uint64_t used[3];   // seam slots in use (bit s of word s/64)
        uint64_t rec;       // one-colour: the record of its seam node
    };
    uint64_t topmask;   // one-colour: columns with a top-edge request to the pixel
                        //   up-right (8 neighbours) or up (4 neighbours)
    uint32_t lead;      // one-colour: 1 if its first pixel leads a region (collapse pass)
    uint32_t pre;       // one-colour: leaders before its first pixel in its image
                        //   (scan pass)
};
static_assert(sizeof(TileHdr) == 64, "one 64-byte store per tile");

constexpr uint32_t KIND_UNIFORM = 1u;
constexpr uint32_t KIND_TOP0 = 2u;      // one-colour: top request at column 0
constexpr uint32_t KIND_TOP0_UL = 4u;   // ... to the pixel up-left of column 0
constexpr uint32_t KIND_IGNORED = 8u;   // one-colour: the tile is of the ignored colour

// exact unsigned division of n < 2^31 by a fixed d >= 1: q = (n*m) >> s, with
// a 32-bit m (one 32x32 multiply and a shift)
struct FastDiv {
    uint32_t m;
    uint32_t s;
    uint32_t d;
    uint32_t pad;
};

struct Geom {
    int64_t B, H, W;
    int64_t HW;
    int32_t ntx, nty;           // tiles per row / per column of one image
    int64_t tpi;                // tiles per image
    int64_t ntiles;             // tiles in the batch
    int64_t nbands;             // B * nty
    FastDiv divW;               // by W
    FastDiv divTpi;             // by tiles per image
    FastDiv divNtx;             // by tiles per image row
    FastDiv divNty;             // by tile rows per image
};

// Per tile row ("row segment": 64 pixels of one image row), tile-major:
// entry t*TH + y is row y of tile t.
struct Work {
    uint32_t *err;      // [1]
    TileHdr *hdr;       // [ntiles]
    uint64_t *runmask;  // [ntiles*TH] run starts of each row segment
    uint64_t *leadmask; // [ntiles*TH] leaders of the image in each row segment
    uint16_t *runinfo;  // [ntiles*TPX] per-run records
    uint64_t *gp;       // [ntiles*KMAX] seam node records of tiles of several colours:
                        //   (key of parent << 32) | parent node
    uint32_t *nval;     // [ntiles*KMAX] the value of each such node's pixels (resolve)
    uint8_t *bslot;     // [ntiles*TW] seam slot of each bottom-row pixel
    uint8_t *rslot;     // [ntiles*TH] seam slot of each right-column pixel
    uint16_t *req;      // [ntiles*REQMAX] seam requests
    uint32_t *seg;      // [ntiles*TH] leaders per row segment, then their exclusive
                        //   prefix in reading order (per image)
    uint64_t *bandst;   // [B*nty] scan status of each band of tiles: (value << 32) | state
};

struct Layout {
    Geom g;
    size_t off_err, off_hdr, off_runmask, off_leadmask, off_runinfo, off_gp, off_nval, off_bslot,
        off_rslot, off_req, off_seg, off_bandst, total;
};

// Fills `L` for a batch shape; returns false if the shape is too large to
// index (caller maps that to CCL_ERR_TOO_LARGE).  Pure host arithmetic.
bool make_layout(int64_t B, int64_t H, int64_t W, Layout *L);
Work bind_work(const Layout &L, void *workspace);

// Launchers (enqueue only).  dtype_bytes is 1, 3 (RGB) or 4, conn is 4 or 8.
// ignore: pixels of colour ign take part in nothing (their regions are neither
// labelled nor counted).  clear_err: the tile pass clears the workspace's
// error word first (the first kernel of a call).
// t0, nt: the pass labels tiles t0 .. t0+nt-1 only (a band of whole tile rows
// whose pixels, and the row above them, are in place); nt = 0: every tile
void launch_tile(const void *img, int dtype_bytes, int conn, int ignore, uint32_t ign,
                 const Geom &g, const Work &w, int clear_err, hipStream_t s, uint32_t t0 = 0,
                 uint32_t nt = 0);
void launch_seam(const Geom &g, const Work &w, int conn, hipStream_t s);
void launch_seam_roots(const Geom &g, const Work &w, hipStream_t s);
void launch_scan(const Geom &g, const Work &w, int32_t *counts, int apply, int use_hdr,
                 hipStream_t s);
struct RegionRec;
// number: 0 leaders, 1 numbers, 2 numbers and each seam node's record pointed
// at its root (whose key is the region's leader).  rec: with numbers, each
// region that crosses a tile edge gets an empty record (statistics of the
// labelling call; the band-status words hold the first record of each image by
// then)
void launch_resolve(const Geom &g, const Work &w, int number, hipStream_t s,
                    RegionRec *rec = nullptr, int64_t cap = 0);
// number: 0 leaders, 1 numbers, 2 leaders of a workspace numbered with
// resolve's number == 2.  ignv: the value written for pixels of an ignored
// colour
void launch_final(const Geom &g, const Work &w, int32_t *out, int number, uint32_t ignv,
                  hipStream_t s, uint32_t t0 = 0, uint32_t nt = 0);

// Numbers of one band of a picture cut into bands, to the picture's numbers
// (ccl_label_large): band-local number n (1..) is merged into a region led
// elsewhere when bit n of M is set; with r the merged numbers below n, it then
// takes MV[r], else it becomes G + n - r.  For leaders, MV holds the picture's
// leader of each merged number, and an unmerged region's leader is base + its
// band-local leader.
struct Map64 {
    const uint64_t *M;     // bit n: number n merged (this band's words)
    const uint32_t *Mpre;  // merged numbers in the words before each word
    const int64_t *MV;     // the picture's number (or leader) of each merged number, by rank
    const int64_t *G;      // [band]: numbers of the picture before the band's own
    int64_t base;          // the picture index of the band's first pixel (leaders)
    uint32_t band;
    int merges;            // 0: one band, its numbers are the picture's
};

// a seam region's table slot to start probing at
__device__ __forceinline__ uint32_t seam_hash(int64_t key, uint32_t mask)
{
    const uint64_t k = (uint64_t)key * 0x9E3779B97F4A7C15ull;
    return (uint32_t)(k >> 40) & mask;
}

// the final write of one band with 64-bit numbers through the map (ignored
// pixels 0), or with leaders (lead: the band's workspace was numbered with
// keys, number == 2 in resolve; ignored pixels -1)
void launch_final64(const Geom &g, const Work &w, int64_t *out, const Map64 &m, int lead,
                    hipStream_t s);
void launch_leader_flags(const int32_t *leaders, const Geom &g, const Work &w, int write_mask,
                         int clear_err, hipStream_t s);
void launch_leader_assign(const int32_t *leaders, int32_t *labels, const Geom &g, const Work &w,
                          hipStream_t s);
// One region's statistics, laid out as ccl_region of the C ABI.
struct RegionRec {
    unsigned long long sum_y, sum_x;
    int32_t area, y0, x0, y1, x1, pad;
};
static_assert(sizeof(RegionRec) == 40, "40-byte region records");

// per-region statistics of a numbered labelling, one pass of images (first:
// the batch's first pass, which sets all n_total records empty); the
// workspace's band-status words hold the first record of each image of the
// pass (B int64 fit in its B*nty words), counted on from the earlier passes'
void launch_region_stats(const int32_t *labels, const int32_t *counts, const Geom &g,
                         const Work &w, int64_t n_total, RegionRec *recs, int first,
                         hipStream_t s);
// statistics of the labelling call: stage 0 the first record of each image
// (into the band-status words, after the scan; first: the batch's first pass
// of images), stage 1 the final write with statistics (numbers into out),
// stage 2 the reduce pass
void launch_label_stats(const Geom &g, const Work &w, const int32_t *counts, int32_t *out,
                        RegionRec *rec, int64_t cap, int stage, int first, hipStream_t s);
void launch_zero_i32(int32_t *p, int64_t n, hipStream_t s);

}  // namespace ccl
