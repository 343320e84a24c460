// ccl_api.hip -- the C ABI declared in include/ccl.h: argument checks, the
// workspace layout, and the launch sequence on the caller's stream.
#include "ccl.h"
#include "ccl_internal.h"

#include <limits.h>

#include <mutex>
#include <vector>

namespace ccl {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static FastDiv make_fastdiv(uint32_t d)
{
    // exact for every n < 2^31: with l = ceil(log2 d), s = 31 + l and
    // m = ceil(2^s / d), the error e = m*d - 2^s < d gives n*e < 2^31 * 2^l = 2^s,
    // so floor(n*m / 2^s) = floor(n / d); and 2^(l-1) < d (or d = 1) keeps
    // m < 2^32.
    FastDiv f;
    uint32_t l = 0;
    while (l < 32 && (1ull << l) < d) ++l;
    f.s = 31 + l;
    f.m = (uint32_t)(((1ull << f.s) + d - 1) / d);
    f.d = d;
    f.pad = 0;
    return f;
}

bool make_layout(int64_t B, int64_t H, int64_t W, Layout *L)
{
    Geom &g = L->g;
    g.B = B;
    g.H = H;
    g.W = W;
    g.HW = H * W;
    g.ntx = (int32_t)((W + TW - 1) / TW);
    g.nty = (int32_t)((H + TH - 1) / TH);
    g.tpi = (int64_t)g.ntx * g.nty;
    g.ntiles = B * g.tpi;
    if (g.ntiles > MAX_TILES) return false;  // seam node ids are 32-bit
    g.nbands = B * g.nty;
    g.divW = make_fastdiv(W > 0 ? (uint32_t)W : 1u);
    g.divTpi = make_fastdiv(g.tpi > 0 ? (uint32_t)g.tpi : 1u);
    g.divNtx = make_fastdiv(g.ntx > 0 ? (uint32_t)g.ntx : 1u);
    g.divNty = make_fastdiv(g.nty > 0 ? (uint32_t)g.nty : 1u);

    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t nt = (size_t)g.ntiles;
    L->off_err = take(256);
    L->off_hdr = take(nt * sizeof(TileHdr));
    L->off_runmask = take(nt * TH * sizeof(uint64_t));
    L->off_leadmask = take(nt * TH * sizeof(uint64_t));
    L->off_runinfo = take(nt * TPX * sizeof(uint16_t));
    L->off_gp = take(nt * KMAX * sizeof(uint64_t));
    L->off_nval = take(nt * KMAX * sizeof(uint32_t));
    L->off_bslot = take(nt * TW);
    L->off_rslot = take(nt * TH);
    L->off_req = take(nt * REQMAX * sizeof(uint16_t));
    L->off_seg = take(nt * TH * sizeof(uint32_t));
    L->off_bandst = take((size_t)g.nbands * sizeof(uint64_t));
    L->total = off;
    return true;
}

Work bind_work(const Layout &L, void *workspace)
{
    char *base = (char *)workspace;
    Work w;
    w.err = (uint32_t *)(base + L.off_err);
    w.hdr = (TileHdr *)(base + L.off_hdr);
    w.runmask = (uint64_t *)(base + L.off_runmask);
    w.leadmask = (uint64_t *)(base + L.off_leadmask);
    w.runinfo = (uint16_t *)(base + L.off_runinfo);
    w.gp = (uint64_t *)(base + L.off_gp);
    w.nval = (uint32_t *)(base + L.off_nval);
    w.bslot = (uint8_t *)(base + L.off_bslot);
    w.rslot = (uint8_t *)(base + L.off_rslot);
    w.req = (uint16_t *)(base + L.off_req);
    w.seg = (uint32_t *)(base + L.off_seg);
    w.bandst = (uint64_t *)(base + L.off_bandst);
    return w;
}

// Shape checks shared by every call.  On success `empty` tells whether the
// batch has no pixels.
static int check_shape(int64_t B, int64_t H, int64_t W, bool *empty)
{
    if (B < 0 || H < 0 || W < 0) return CCL_ERR_SHAPE;
    *empty = (B == 0 || H == 0 || W == 0);
    if (*empty) return CCL_OK;
    if (H > INT32_MAX / W) return CCL_ERR_TOO_LARGE;  // per-image indices are int32
    if (B > INT64_MAX / (H * W)) return CCL_ERR_TOO_LARGE;
    return CCL_OK;
}

// Images per pass: a batch with more tiles than seam node ids can name
// (MAX_TILES) is labelled in passes of whole images, one after another on the
// stream, all in one workspace sized for one pass.  0: one image alone has too
// many tiles.
static int64_t images_per_pass(int64_t B, int64_t H, int64_t W)
{
    const int64_t tpi = ((W + TW - 1) / TW) * ((H + TH - 1) / TH);
    const int64_t per = MAX_TILES / tpi;
    return per < B ? per : B;
}

static int finish_launches()
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? CCL_OK : CCL_ERR_HIP;
}

// Checks of ccl_label's arguments other than the buffers (host only).
static int check_label_args(int dtype, int64_t B, int64_t H, int64_t W, int conn, int flags,
                            uint32_t ignore, bool *empty)
{
    if (flags & ~(CCL_NUMBER | CCL_IGNORE)) return CCL_ERR_FLAGS;
    int rc = check_shape(B, H, W, empty);
    if (rc != CCL_OK) return rc;
    if (dtype != CCL_U8 && dtype != CCL_RGB24 && dtype != CCL_U32) return CCL_ERR_DTYPE;
    if (conn != 4 && conn != 8) return CCL_ERR_CONNECTIVITY;
    if ((flags & CCL_IGNORE) && dtype != CCL_U32 && ignore >= (1u << (8 * dtype)))
        return CCL_ERR_IGNORE;
    return CCL_OK;
}

static int label_impl(const void *colours, int dtype, int64_t B, int64_t H, int64_t W, int conn,
                      int flags, uint32_t ignore, int32_t *out, int32_t *counts, void *workspace,
                      size_t workspace_bytes, void *stream, void **events, int n_events)
{
    bool empty;
    int rc = check_label_args(dtype, B, H, W, conn, flags, ignore, &empty);
    if (rc != CCL_OK) return rc;
    if (events != nullptr && n_events < 6) return CCL_ERR_NULL;
    const int ign = (flags & CCL_IGNORE) != 0;
    hipStream_t s = (hipStream_t)stream;
    if (empty) {
        if (counts && B > 0) {
            launch_zero_i32(counts, B, s);
            return finish_launches();
        }
        return CCL_OK;
    }
    if (!colours || !out || !workspace) return CCL_ERR_NULL;
    const int64_t per = images_per_pass(B, H, W);
    Layout L;
    if (per < 1 || !make_layout(per, H, W, &L)) return CCL_ERR_TOO_LARGE;
    if (workspace_bytes < L.total) return CCL_ERR_WORKSPACE;
    const int number = (flags & CCL_NUMBER) != 0;
    const bool need_scan = number || counts != nullptr;
    const int64_t HW = H * W;

    // (with several passes the events are recorded again by each: they time
    // the last pass)
    auto mark = [&](int i) {
        if (events) (void)hipEventRecord((hipEvent_t)events[i], s);
    };
    for (int64_t b0 = 0; b0 < B; b0 += per) {
        Layout Lp = L;
        if (B - b0 < per) make_layout(B - b0, H, W, &Lp);  // fits: fewer images
        const Work w = bind_work(Lp, workspace);
        const void *cp = (const char *)colours + (size_t)(b0 * HW) * (size_t)dtype;
        int32_t *op = out + b0 * HW;
        int32_t *np = counts ? counts + b0 : nullptr;
        mark(0);
        // the first pass's tile pass clears the error word for the whole call
        launch_tile(cp, dtype, conn, ign, ignore, Lp.g, w, b0 == 0, s);
        mark(1);
        launch_seam(Lp.g, w, conn, s);
        mark(2);
        if (need_scan) launch_seam_roots(Lp.g, w, s);
        mark(3);
        if (need_scan) launch_scan(Lp.g, w, np, number, 1, s);
        launch_resolve(Lp.g, w, number, s);
        mark(4);
        // ignored pixels: number 0, or leader -1 (label 0 in the leader + 1 form)
        launch_final(Lp.g, w, op, number, number ? 0u : 0xFFFFFFFFu, s);
        mark(5);
    }
    return finish_launches();
}

// ---- the workspace of ccl_label_noalloc: one static device array per GPU.
// Host code never uses the array's name as an address (on the host it is only
// a stand-in for the symbol): its device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and kept here.
static __device__ __align__(256) unsigned char scratch[CCL_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 256;
static void *g_scratch_ptr[MAX_DEVICES];
static std::mutex g_scratch_mu;

static int scratch_address(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return CCL_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return CCL_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return CCL_OK;
}

}  // namespace ccl

using namespace ccl;

extern "C" {

size_t ccl_workspace_bytes(int64_t batch, int64_t height, int64_t width)
{
    bool empty;
    if (check_shape(batch, height, width, &empty) != CCL_OK) return SIZE_MAX;
    if (empty) return 0;
    // one pass of images (the whole batch unless it has 2^24 tiles or more)
    const int64_t per = images_per_pass(batch, height, width);
    Layout L;
    if (per < 1 || !make_layout(per, height, width, &L)) return SIZE_MAX;
    return L.total;
}

int ccl_label(const void *colours, int dtype, int64_t batch, int64_t height, int64_t width,
              int connectivity, int flags, uint32_t ignore, int32_t *out, int32_t *counts,
              void *workspace, size_t workspace_bytes, void *stream)
{
    return label_impl(colours, dtype, batch, height, width, connectivity, flags, ignore, out,
                      counts, workspace, workspace_bytes, stream, nullptr, 0);
}

int ccl_label_profiled(const void *colours, int dtype, int64_t batch, int64_t height,
                       int64_t width, int connectivity, int flags, uint32_t ignore, int32_t *out,
                       int32_t *counts, void *workspace, size_t workspace_bytes, void *stream,
                       void **events, int n_events)
{
    if (events == nullptr) return CCL_ERR_NULL;
    return label_impl(colours, dtype, batch, height, width, connectivity, flags, ignore, out,
                      counts, workspace, workspace_bytes, stream, events, n_events);
}

int ccl_label_noalloc(const void *colours, int dtype, int64_t batch, int64_t height,
                      int64_t width, int connectivity, int flags, uint32_t ignore, int32_t *out,
                      int32_t *counts, void *stream)
{
    // every check comes before any HIP call: a batch that does not fit is
    // rejected without touching a device
    bool empty;
    int rc = check_label_args(dtype, batch, height, width, connectivity, flags, ignore, &empty);
    if (rc != CCL_OK) return rc;
    void *ws = nullptr;
    if (!empty) {
        if (!colours || !out) return CCL_ERR_NULL;
        const int64_t per = images_per_pass(batch, height, width);
        Layout L;
        if (per < 1 || !make_layout(per, height, width, &L)) return CCL_ERR_TOO_LARGE;
        if (L.total > CCL_SCRATCH_BYTES) return CCL_ERR_SCRATCH;
        rc = scratch_address(&ws);
        if (rc != CCL_OK) return rc;
    }
    return label_impl(colours, dtype, batch, height, width, connectivity, flags, ignore, out,
                      counts, ws, CCL_SCRATCH_BYTES, stream, nullptr, 0);
}

int ccl_label_host(const void *host_colours, int dtype, int64_t batch, int64_t height,
                   int64_t width, int connectivity, int flags, uint32_t ignore, int32_t *host_out,
                   int32_t *counts, void *dev_colours, int32_t *dev_out, void *workspace,
                   size_t workspace_bytes, int64_t band_rows, void *stream, void *h2d_stream,
                   void *d2h_stream)
{
    bool empty;
    int rc = check_label_args(dtype, batch, height, width, connectivity, flags, ignore, &empty);
    if (rc != CCL_OK) return rc;
    if (band_rows < 0 || band_rows % TH != 0) return CCL_ERR_BAND;
    hipStream_t s = (hipStream_t)stream;
    if (empty) {
        if (counts && batch > 0) {
            launch_zero_i32(counts, batch, s);
            return finish_launches();
        }
        return CCL_OK;
    }
    if (!host_colours || !host_out || !dev_colours || !dev_out || !workspace) return CCL_ERR_NULL;
    if (h2d_stream == nullptr || d2h_stream == nullptr || h2d_stream == stream ||
        d2h_stream == stream || h2d_stream == d2h_stream)
        return CCL_ERR_STREAM;
    // the workspace of one pass of images, as for ccl_label: every group of
    // images below is labelled in it in turn, and a group never has more
    // tiles than a pass (a group of several images has fewer than 2^23)
    const int64_t per = images_per_pass(batch, height, width);
    Layout L;
    if (per < 1 || !make_layout(per, height, width, &L)) return CCL_ERR_TOO_LARGE;
    if (workspace_bytes < L.total) return CCL_ERR_WORKSPACE;
    hipStream_t sin = (hipStream_t)h2d_stream, sout = (hipStream_t)d2h_stream;
    const int ign = (flags & CCL_IGNORE) != 0;
    const int number = (flags & CCL_NUMBER) != 0;
    const bool need_scan = number || counts != nullptr;
    const size_t bpp = (size_t)dtype;  // bytes per pixel (CCL_U8 1, CCL_RGB24 3, CCL_U32 4)
    const int64_t HW = height * width;

    // Steps of the pipeline.  A large image is cut into bands of whole tile
    // rows (band_rows, or automatically an eighth of it but at least 2^22
    // pixels); small images are taken whole, in groups of at least 2^22
    // pixels.  Each group (an image with its bands, or a group of images) is
    // labelled as one batch; the steps of a group are its bands.
    constexpr int64_t STEP_PX = int64_t(1) << 22;
    int64_t brows = band_rows;
    if (brows == 0) {
        const int64_t eighth = (height + 8 * TH - 1) / (8 * TH) * TH;
        const int64_t least = ((STEP_PX + width - 1) / width + TH - 1) / TH * TH;
        brows = HW > 2 * STEP_PX ? (eighth > least ? eighth : least) : height;
    }
    if (brows > height) brows = (height + TH - 1) / TH * TH;
    const int64_t nband = (height + brows - 1) / brows;
    int64_t per_group = 1;  // images per group (bands of one image if there are several)
    if (nband == 1) {
        per_group = (STEP_PX + HW - 1) / HW;
        if (per_group > batch) per_group = batch;
    }
    const int64_t ngroup = (batch + per_group - 1) / per_group;
    const int64_t nstep = ngroup * nband;

    std::vector<hipEvent_t> ev(2 * (size_t)nstep + 2, nullptr);
    auto cleanup = [&]() {
        for (hipEvent_t e : ev)
            if (e) (void)hipEventDestroy(e);
    };
    for (hipEvent_t &e : ev)
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
            e = nullptr;
            cleanup();
            return CCL_ERR_HIP;
        }
    hipEvent_t *ein = ev.data(), *eout = ev.data() + nstep;
    hipEvent_t estart = ev[2 * nstep], edone = ev[2 * nstep + 1];
    bool ok = true;
    auto chk = [&](hipError_t e) { ok = ok && e == hipSuccess; };
    // pixels of step (group j, band k): first pixel and count (contiguous)
    auto step_px = [&](int64_t j, int64_t k, int64_t &first, int64_t &n) {
        const int64_t b0 = j * per_group, nb = batch - b0 < per_group ? batch - b0 : per_group;
        const int64_t r0 = k * brows, r1 = r0 + brows < height ? r0 + brows : height;
        first = b0 * HW + r0 * width;
        n = nband == 1 ? nb * HW : (r1 - r0) * width;
    };

    // the copy streams start after everything already on the caller's stream
    // (an earlier call may still read dev_colours or write dev_out there)
    chk(hipEventRecord(estart, s));
    chk(hipStreamWaitEvent(sin, estart, 0));
    chk(hipStreamWaitEvent(sout, estart, 0));
    // 1. every step's pixels in, in order, each followed by its event
    for (int64_t j = 0; j < ngroup && ok; ++j)
        for (int64_t k = 0; k < nband; ++k) {
            int64_t first, n;
            step_px(j, k, first, n);
            chk(hipMemcpyAsync((char *)dev_colours + (size_t)first * bpp,
                               (const char *)host_colours + (size_t)first * bpp, (size_t)n * bpp,
                               hipMemcpyHostToDevice, sin));
            chk(hipEventRecord(ein[j * nband + k], sin));
        }
    // 2. each group: its bands' tile passes, each once its pixels (and the
    //    row above them, in the band before) are in; the seam merge, seam
    //    roots, scan and resolve of the group; its bands' final writes, each
    //    followed by the copy of its labels out
    for (int64_t j = 0; j < ngroup && ok; ++j) {
        const int64_t b0 = j * per_group, nb = batch - b0 < per_group ? batch - b0 : per_group;
        Layout Lg;
        make_layout(nb, height, width, &Lg);  // fits: no more tiles than a pass
        const Geom &g = Lg.g;
        const Work w = bind_work(Lg, workspace);
        const char *img = (const char *)dev_colours + (size_t)(b0 * HW) * bpp;
        int32_t *o = dev_out + b0 * HW;
        const uint32_t band_tiles = (uint32_t)(brows / TH) * (uint32_t)g.ntx;
        auto tiles_of = [&](int64_t k, uint32_t &t0, uint32_t &nt) {
            t0 = nband == 1 ? 0u : (uint32_t)k * band_tiles;
            nt = nband == 1 ? (uint32_t)g.ntiles
                            : (t0 + band_tiles <= (uint32_t)g.ntiles ? band_tiles
                                                                     : (uint32_t)g.ntiles - t0);
        };
        for (int64_t k = 0; k < nband; ++k) {
            uint32_t t0, nt;
            tiles_of(k, t0, nt);
            chk(hipStreamWaitEvent(s, ein[j * nband + k], 0));
            launch_tile(img, dtype, connectivity, ign, ignore, g, w, j == 0 && k == 0, s, t0, nt);
        }
        launch_seam(g, w, connectivity, s);
        if (need_scan) launch_seam_roots(g, w, s);
        if (need_scan) launch_scan(g, w, counts ? counts + b0 : nullptr, number, 1, s);
        launch_resolve(g, w, number, s);
        for (int64_t k = 0; k < nband; ++k) {
            uint32_t t0, nt;
            tiles_of(k, t0, nt);
            launch_final(g, w, o, number, number ? 0u : 0xFFFFFFFFu, s, t0, nt);
            chk(hipEventRecord(eout[j * nband + k], s));
            chk(hipStreamWaitEvent(sout, eout[j * nband + k], 0));
            int64_t first, n;
            step_px(j, k, first, n);
            chk(hipMemcpyAsync(host_out + first, dev_out + first, (size_t)n * sizeof(int32_t),
                               hipMemcpyDeviceToHost, sout));
        }
    }
    // 3. the call ends on the caller's stream once the last labels are out
    chk(hipEventRecord(edone, sout));
    chk(hipStreamWaitEvent(s, edone, 0));
    cleanup();  // each event is released once the work it marks has run
    if (!ok) return CCL_ERR_HIP;
    return finish_launches();
}

int ccl_label_stats(const void *colours, int dtype, int64_t batch, int64_t height, int64_t width,
                    int connectivity, int flags, uint32_t ignore, int32_t *out, int32_t *counts,
                    ccl_region *stats, int64_t stats_capacity, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    bool empty;
    int rc = check_label_args(dtype, batch, height, width, connectivity, flags, ignore, &empty);
    if (rc != CCL_OK) return rc;
    if (!(flags & CCL_NUMBER)) return CCL_ERR_FLAGS;  // records are indexed by number
    if (stats_capacity < 0) return CCL_ERR_SHAPE;
    if (!counts || (stats_capacity > 0 && !stats)) return CCL_ERR_NULL;
    hipStream_t s = (hipStream_t)stream;
    if (empty) {
        if (batch > 0) {
            launch_zero_i32(counts, batch, s);
            return finish_launches();
        }
        return CCL_OK;
    }
    if (!colours || !out || !workspace) return CCL_ERR_NULL;
    const int64_t per = images_per_pass(batch, height, width);
    Layout L;
    if (per < 1 || !make_layout(per, height, width, &L)) return CCL_ERR_TOO_LARGE;
    if (workspace_bytes < L.total) return CCL_ERR_WORKSPACE;
    const int ign = (flags & CCL_IGNORE) != 0;
    static_assert(sizeof(ccl_region) == sizeof(RegionRec), "one record layout");
    RegionRec *rec = (RegionRec *)stats;
    const int64_t HW = height * width;
    for (int64_t b0 = 0; b0 < batch; b0 += per) {  // passes of whole images
        Layout Lp = L;
        if (batch - b0 < per) make_layout(batch - b0, height, width, &Lp);  // fits
        const Work w = bind_work(Lp, workspace);
        const void *cp = (const char *)colours + (size_t)(b0 * HW) * (size_t)dtype;
        int32_t *op = out + b0 * HW, *np = counts + b0;
        const int first = b0 == 0;
        launch_tile(cp, dtype, connectivity, ign, ignore, Lp.g, w, first, s);
        launch_seam(Lp.g, w, connectivity, s);
        launch_seam_roots(Lp.g, w, s);
        launch_scan(Lp.g, w, np, 1, 1, s);
        // the first record of each image (after the earlier passes' regions)
        launch_label_stats(Lp.g, w, np, op, rec, stats_capacity, 0, first, s);
        launch_resolve(Lp.g, w, 1, s, rec, stats_capacity);  // opens seam regions' records
        launch_label_stats(Lp.g, w, np, op, rec, stats_capacity, 1, first, s);  // numbers, parts
        launch_label_stats(Lp.g, w, np, op, rec, stats_capacity, 2, first, s);  // parts in
    }
    return finish_launches();
}

int ccl_number(const int32_t *leaders, int64_t batch, int64_t height, int64_t width,
               int32_t *labels, int32_t *counts, void *workspace, size_t workspace_bytes,
               void *stream)
{
    bool empty;
    int rc = check_shape(batch, height, width, &empty);
    if (rc != CCL_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (empty) {
        if (counts && batch > 0) {
            launch_zero_i32(counts, batch, s);
            return finish_launches();
        }
        return CCL_OK;
    }
    if (!leaders || !labels || !workspace) return CCL_ERR_NULL;
    const int64_t per = images_per_pass(batch, height, width);
    Layout L;
    if (per < 1 || !make_layout(per, height, width, &L)) return CCL_ERR_TOO_LARGE;
    if (workspace_bytes < L.total) return CCL_ERR_WORKSPACE;
    const int64_t HW = height * width;
    for (int64_t b0 = 0; b0 < batch; b0 += per) {  // passes of whole images
        Layout Lp = L;
        if (batch - b0 < per) make_layout(batch - b0, height, width, &Lp);  // fits
        const Work w = bind_work(Lp, workspace);
        launch_leader_flags(leaders + b0 * HW, Lp.g, w, 1, b0 == 0, s);
        launch_scan(Lp.g, w, counts ? counts + b0 : nullptr, 1, 0, s);
        launch_leader_assign(leaders + b0 * HW, labels + b0 * HW, Lp.g, w, s);
    }
    return finish_launches();
}

int ccl_count(const int32_t *leaders, int64_t batch, int64_t height, int64_t width,
              int32_t *counts, void *workspace, size_t workspace_bytes, void *stream)
{
    bool empty;
    int rc = check_shape(batch, height, width, &empty);
    if (rc != CCL_OK) return rc;
    if (!counts) return CCL_ERR_NULL;
    hipStream_t s = (hipStream_t)stream;
    if (empty) {
        if (batch > 0) {
            launch_zero_i32(counts, batch, s);
            return finish_launches();
        }
        return CCL_OK;
    }
    if (!leaders || !workspace) return CCL_ERR_NULL;
    const int64_t per = images_per_pass(batch, height, width);
    Layout L;
    if (per < 1 || !make_layout(per, height, width, &L)) return CCL_ERR_TOO_LARGE;
    if (workspace_bytes < L.total) return CCL_ERR_WORKSPACE;
    const int64_t HW = height * width;
    for (int64_t b0 = 0; b0 < batch; b0 += per) {  // passes of whole images
        Layout Lp = L;
        if (batch - b0 < per) make_layout(batch - b0, height, width, &Lp);  // fits
        const Work w = bind_work(Lp, workspace);
        launch_leader_flags(leaders + b0 * HW, Lp.g, w, 0, b0 == 0, s);
        launch_scan(Lp.g, w, counts + b0, 0, 0, s);
    }
    return finish_launches();
}

int ccl_region_stats(const int32_t *labels, int64_t batch, int64_t height, int64_t width,
                     const int32_t *counts, int64_t n_total, ccl_region *stats,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    bool empty;
    int rc = check_shape(batch, height, width, &empty);
    if (rc != CCL_OK) return rc;
    if (n_total < 0) return CCL_ERR_SHAPE;
    if (n_total > 0 && !stats) return CCL_ERR_NULL;
    if (empty || n_total == 0) return CCL_OK;  // no pixel, or no region: nothing to write
    if (!labels || !counts || !workspace) return CCL_ERR_NULL;
    const int64_t per = images_per_pass(batch, height, width);
    Layout L;
    if (per < 1 || !make_layout(per, height, width, &L)) return CCL_ERR_TOO_LARGE;
    if (workspace_bytes < L.total) return CCL_ERR_WORKSPACE;
    static_assert(sizeof(ccl_region) == sizeof(RegionRec), "one record layout");
    const int64_t HW = height * width;
    for (int64_t b0 = 0; b0 < batch; b0 += per) {  // passes of whole images
        Layout Lp = L;
        if (batch - b0 < per) make_layout(batch - b0, height, width, &Lp);  // fits
        const Work w = bind_work(Lp, workspace);
        launch_region_stats(labels + b0 * HW, counts + b0, Lp.g, w, n_total, (RegionRec *)stats,
                            b0 == 0, (hipStream_t)stream);
    }
    return finish_launches();
}

const char *ccl_status_string(int status)
{
    switch (status) {
    case CCL_OK: return "ok";
    case CCL_ERR_NULL: return "a required pointer is NULL";
    case CCL_ERR_SHAPE: return "batch, height or width is negative";
    case CCL_ERR_TOO_LARGE: return "image or batch too large to index";
    case CCL_ERR_CONNECTIVITY: return "connectivity must be 4 or 8";
    case CCL_ERR_DTYPE: return "dtype must be CCL_U8, CCL_RGB24 or CCL_U32";
    case CCL_ERR_WORKSPACE: return "workspace smaller than ccl_workspace_bytes()";
    case CCL_ERR_HIP: return "HIP rejected a kernel launch";
    case CCL_ERR_FLAGS: return "unknown flag bits";
    case CCL_ERR_IGNORE: return "ignored colour does not fit the dtype";
    case CCL_ERR_BAND:
        return "band_rows must be a non-negative multiple of 64 (ccl_label_large, with "
               "band_rows*width < 2^31) or of 32 (ccl_label_host)";
    case CCL_ERR_SCRATCH: return "batch needs more workspace than the static scratch array holds";
    case CCL_ERR_STREAM: return "the copy streams must be two streams other than the call's stream";
    default: return "unknown status";
    }
}

}  // extern "C"
