/*
 * ccl.h -- C ABI of the MI355X (gfx950) connected-component labeller.
 *
 * What is computed (per image of a batch, each image on its own):
 *   Two pixels belong to one region exactly when a chain of neighbours of
 *   identical colour value joins them.  Neighbours are the 8 pixels around a
 *   pixel (or the 4 sharing an edge) inside the H x W rectangle: rows do not
 *   wrap and images never touch ("Accountable AI starts at the pixel",
 *   ch.01 "The job" and ch.02 "Regions"; "About Connected Components Labeling
 *   on GPU", section "Connected Components Labeling" for 4 vs 8 neighbours).
 *   A region's leader is its smallest reading-order index (row * W + col,
 *   counted inside its image): joins always re-point the larger leader at the
 *   smaller ("Accountable AI starts at the pixel", ch.04 "Point at a leader").
 *   Its number is 1 + the count of leaders before it in reading order (same
 *   page, ch.08 idea 5 "Number without a giant list").  Colours are compared
 *   as whole stored values: all 32 bits of a CCL_U32 pixel, the byte of a
 *   CCL_U8 pixel.  Every value, 0 included, forms regions, unless the caller
 *   names one colour to ignore (CCL_IGNORE, same page, ch.08 idea 4 "Ignore the
 *   paper"): its pixels then belong to no region and are neither numbered nor
 *   counted.
 *
 * Memory.  Every pointer argument except the host-side ones named below is a
 * DEVICE pointer on the current HIP device.  Images are contiguous row-major
 * [batch, height, width]; labels are int32 [batch, height, width]; counts are
 * int32 [batch].  The caller owns every buffer, including the workspace; the
 * library allocates nothing and keeps no state between calls, so calls are
 * reentrant.  Two calls that run at the same time need distinct workspaces.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Calls only enqueue work on it and never synchronise; results are
 * ready when the stream reaches that point.  ccl_label, ccl_label_noalloc,
 * ccl_label_stats, ccl_number, ccl_count and ccl_region_stats enqueue kernel
 * launches only (no memory-set or copy: what must start empty is cleared by
 * the kernels), so they can be recorded into a HIP graph and replayed
 * (ccl_label_noalloc needs one call on the device before capture, which looks
 * up its scratch array).
 *
 * Errors.  Each call returns a ccl_status.  Arguments are checked on the host
 * before anything is enqueued; on a validation error nothing is enqueued and
 * the output buffers are untouched.  CCL_ERR_HIP reports a launch that HIP
 * rejected.  Faults inside kernels are asynchronous and surface at the
 * caller's next synchronisation, as for any HIP kernel.  A batch, height or
 * width of 0 is valid and does nothing except writing zeros to `counts`.
 */
#ifndef CCL_H
#define CCL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CCL_OK = 0,
    CCL_ERR_NULL = -1,          /* a required pointer is NULL                        */
    CCL_ERR_SHAPE = -2,         /* batch, height or width is negative                */
    CCL_ERR_TOO_LARGE = -3,     /* height*width > 2^31-1, or one image has 2^24
                                   tiles or more: each image is cut into 64 x 32
                                   tiles, a partial one at the right or bottom edge
                                   counting whole (2^24 full tiles: 34 Gpx).  A
                                   batch of more tiles is labelled in passes of
                                   whole images (ccl_label_host: in its groups of
                                   images, in the same workspace)                    */
    CCL_ERR_CONNECTIVITY = -4,  /* connectivity is not 4 or 8                        */
    CCL_ERR_DTYPE = -5,         /* dtype is not CCL_U8, CCL_RGB24 or CCL_U32         */
    CCL_ERR_WORKSPACE = -6,     /* workspace smaller than ccl_workspace_bytes()      */
    CCL_ERR_HIP = -7,           /* HIP rejected a kernel launch                      */
    CCL_ERR_FLAGS = -8,         /* unknown bits in flags                             */
    CCL_ERR_IGNORE = -9,        /* CCL_IGNORE with a value wider than the pixel:
                                   above 255 (CCL_U8) or 0xFFFFFF (CCL_RGB24)        */
    CCL_ERR_BAND = -10,         /* ccl_label_large: band_rows negative, not a
                                   multiple of 64, or band_rows*width > 2^31-1;
                                   ccl_label_host: band_rows negative or not a
                                   multiple of 32                                    */
    CCL_ERR_SCRATCH = -11,      /* ccl_label_noalloc: the batch needs more workspace
                                   than the static scratch array holds
                                   (ccl_workspace_bytes() > CCL_SCRATCH_BYTES)       */
    CCL_ERR_STREAM = -12        /* ccl_label_host: the two copy streams are NULL,
                                   the same stream, or the call's own stream         */
} ccl_status;

/* Colour element types; the value is the size of one pixel in bytes.
 *   CCL_U8     one byte per pixel
 *   CCL_RGB24  three bytes per pixel, an RGB picture as it is stored: all three
 *              bytes are compared, in place, with no packed copy ("Accountable
 *              AI starts at the pixel", ch.08 "Tried and dropped" and ch.09
 *              "Against NVIDIA's libraries").  Its colour value, where an
 *              ignored colour is named, is b0 | b1 << 8 | b2 << 16, b0 the
 *              pixel's first byte.
 *   CCL_U32    one 32-bit word per pixel */
enum { CCL_U8 = 1, CCL_RGB24 = 3, CCL_U32 = 4 };

/* ccl_label flags.
 *   CCL_NUMBER  write numbers 1..n instead of leaders.
 *   CCL_IGNORE  pixels whose colour equals `ignore` take part in nothing
 *               ("Accountable AI starts at the pixel", ch.08 idea 4): they join
 *               no neighbour, lead no region and are not counted.  They are
 *               written as 0 with CCL_NUMBER and as -1 without it (the label 0
 *               of the "leader + 1, 0 for background" form of "About Connected
 *               Components Labeling on GPU", "Application in CCL").  Every
 *               other pixel gets the leader it gets without the flag (regions
 *               never mix colours), and numbers count only such leaders. */
enum { CCL_NUMBER = 1, CCL_IGNORE = 2 };

/*
 * Bytes of device workspace any call below needs for a batch of this shape.
 * Pure host arithmetic (no HIP call).  Returns 0 for an empty batch and
 * SIZE_MAX for a negative shape or an image too large.  A batch of 2^24
 * tiles or more (see CCL_ERR_TOO_LARGE) is labelled in passes of as many whole
 * images as fit in 2^24 - 1 tiles, one after another on the stream in the same
 * workspace, so the size is that of one such pass.  The workspace must be
 * 256-byte aligned (any HIP allocation is); its contents need no
 * initialisation.
 *
 * Error word.  The workspace's first 4 bytes are an error word.  Every call
 * that takes a workspace clears it in its first kernel, and sets bit 0
 * (CCL_WS_ERR_LOOP) if a bounded loop gave up: the seam unions and walks
 * (2^22 steps each), the numbering scan's wait for an earlier band (2^22
 * polls) and, in ccl_label_large, a band-seam union (2^20 steps).  None of
 * these bounds is reached by a correct run; a call that reaches one still
 * returns CCL_OK (the return value only covers what the host can check before
 * enqueueing), and its labels must then be taken as wrong.  Read the word
 * after the stream has reached the end of the call (the Python binding's
 * check=True does that and raises).
 */
size_t ccl_workspace_bytes(int64_t batch, int64_t height, int64_t width);
enum { CCL_WS_ERR_LOOP = 1 };

/*
 * Label a batch of colour images: Start, Connect, Collapse and (with
 * CCL_NUMBER) Number, the four stages of "Accountable AI starts at the pixel",
 * ch.05.
 *   colours       device, [batch, height, width] of uint8 (dtype CCL_U8),
 *                 uint32 (CCL_U32) or three bytes (CCL_RGB24, any alignment)
 *   connectivity  8 (edges and corners) or 4 (edges only)
 *   flags         0: out[p] = leader of p (per-image reading-order index);
 *                 CCL_NUMBER: out[p] = number of p's region, 1..n per image;
 *                 | CCL_IGNORE: the colour `ignore` is ignored (see above)
 *   ignore        the ignored colour, used only with CCL_IGNORE (a whole stored
 *                 value; at most 255 for CCL_U8 and 0xFFFFFF for CCL_RGB24,
 *                 else CCL_ERR_IGNORE)
 *   out           device int32 [batch, height, width]; must not overlap colours
 *   counts        device int32 [batch] or NULL: number of regions per image
 *   workspace     device, at least ccl_workspace_bytes(batch, height, width)
 */
int ccl_label(const void *colours, int dtype, int64_t batch, int64_t height, int64_t width,
              int connectivity, int flags, uint32_t ignore, int32_t *out, int32_t *counts,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * ccl_label with stage timing: records `events[0]` before the first kernel
 * and `events[i]` after stage i, for the stages tile labelling, seam merge,
 * seam collapse, numbering scan and final write (n_events >= 6; the scan
 * event is recorded even when no scan runs).  `events` is a host array of
 * hipEvent_t created by the caller.  Same results as ccl_label.  A batch
 * labelled in several passes records the events again in each: they time the
 * last pass.
 */
int ccl_label_profiled(const void *colours, int dtype, int64_t batch, int64_t height,
                       int64_t width, int connectivity, int flags, uint32_t ignore,
                       int32_t *out, int32_t *counts, void *workspace, size_t workspace_bytes,
                       void *stream, void **events, int n_events);

/*
 * Number a leader image: labels[p] = 1 + (number of leaders r < leaders[p]) in
 * p's image ("Accountable AI starts at the pixel", ch.05 stage Number and
 * ch.08 idea 5).
 *   leaders  device int32 [batch, height, width]: a valid leader image, i.e.
 *            leaders[p] <= p and leaders[leaders[p]] == leaders[p] (as written
 *            by ccl_label).  Not checked; a value outside [0, height*width),
 *            such as the -1 of an ignored pixel, yields label 0 and is never
 *            dereferenced.
 *   labels   device int32 [batch, height, width]; may be the same buffer as
 *            leaders (in-place), must not otherwise overlap it
 *   counts   device int32 [batch] or NULL
 */
int ccl_number(const int32_t *leaders, int64_t batch, int64_t height, int64_t width,
               int32_t *labels, int32_t *counts, void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * Count the regions of a leader image: counts[b] = number of pixels p of image
 * b with leaders[p] == p, i.e. the leaders, one per region ("Accountable AI
 * starts at the pixel", ch.04 "Point at a leader": the pixel that points at
 * itself leads its group; ch.10 "What we saw in NPP" compares labellers by
 * this count of regions per image).
 *   leaders  device int32 [batch, height, width] (any int32 values)
 *   counts   device int32 [batch], required
 */
int ccl_count(const int32_t *leaders, int64_t batch, int64_t height, int64_t width,
              int32_t *counts, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Statistics of one region (40 bytes, 8-byte aligned): see ccl_region_stats.
 */
typedef struct {
    int64_t sum_y, sum_x;    /* sums of its pixels' row / column indices (exact) */
    int32_t area;            /* its pixels */
    int32_t y0, x0, y1, x1;  /* bounding box: smallest row, smallest column,
                                largest row, largest column (inclusive) */
    int32_t pad;             /* 0 */
} ccl_region;

/*
 * Per-region statistics of a numbered labelling (as written by ccl_label with
 * CCL_NUMBER, or by ccl_number): for each region, its area, its bounding box
 * and the sums of its pixels' row and column indices, from which its position
 * (centroid) is sum / area.  Computing such statistics over the regions is the
 * step after labelling ("About Connected Components Labeling on GPU",
 * introduction: bounding boxes; the tissue-scan segmentation article, section
 * 1.1: area and position of each numbered region, section 2.3: sums over a
 * region's pixels as a global reduction).
 *   labels   device int32 [batch, height, width]: region numbers 1..counts[b]
 *            in image b, 0 for a pixel of no region (an ignored colour).  Other
 *            values are skipped.
 *   counts   device int32 [batch]: regions per image (as ccl_label wrote them)
 *   n_total  host: counts[0] + ... + counts[batch-1], the number of records;
 *            records past it are never written
 *   stats    device ccl_region [n_total], 8-byte aligned: region k of image b
 *            is record counts[0] + ... + counts[b-1] + k - 1
 * Every record is written: a number with no pixel keeps area 0, box
 * (INT32_MAX, INT32_MAX, -1, -1) and sums 0.  The workspace is the one of
 * ccl_workspace_bytes(batch, height, width).
 */
int ccl_region_stats(const int32_t *labels, int64_t batch, int64_t height, int64_t width,
                     const int32_t *counts, int64_t n_total, ccl_region *stats,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * ccl_label for a picture in host memory, with the copies overlapped with the
 * labelling.  On a discrete GPU most of a call from host memory is the copy
 * of the picture in and of the labels out ("Accountable AI starts at the
 * pixel", ch.09 "Results", Fig. 20 "Where the time of one call goes"); here
 * the copies run on two streams of their own beside the kernels, in steps:
 *   - a large image is cut into bands of band_rows rows (automatic: an eighth
 *     of the image, but at least 2^22 pixels, for images above 2^23 pixels);
 *     smaller images are taken whole, in groups of at least 2^22 pixels;
 *   - every step's pixels are copied in, in order, on h2d_stream, and each
 *     band's tile pass starts as soon as its pixels are in (it reads the row
 *     above it from the band before);
 *   - the seam merge, seam roots, scan and resolve run once per image (or
 *     group of images), after its last band: a region at the bottom of a
 *     picture can change the labels at its top, so no label of an image
 *     leaves before the whole image is in;
 *   - each band's final write is followed by the copy of its labels out on
 *     d2h_stream, while the next band is written;
 *   - images are independent, so one group's pixels come in while the group
 *     before is labelled and its labels go out (both PCIe directions at once).
 * The call is complete, host_out included, when `stream` reaches its end.
 *   host_colours  host, [batch, height, width] as for ccl_label; page-locked
 *                 (hipHostMalloc, or torch's pin_memory()), else HIP copies
 *                 through staging buffers and the copies do not overlap
 *   host_out      host int32 [batch, height, width], page-locked: leaders or
 *                 numbers as ccl_label writes them
 *   counts        device int32 [batch] or NULL
 *   dev_colours   device, batch*height*width pixels: where the picture is
 *                 copied to (left holding it)
 *   dev_out       device int32 [batch, height, width]: the labels on the
 *                 device (left holding them)
 *   workspace     device, at least ccl_workspace_bytes(batch, height, width)
 *   band_rows     rows per band, a multiple of 32 (CCL_ERR_BAND otherwise); 0:
 *                 automatic; height or more: whole images
 *   stream, h2d_stream, d2h_stream  three distinct streams (CCL_ERR_STREAM
 *                 otherwise); the copy streams first wait for the work already
 *                 on `stream`, and `stream` ends by waiting for the last copy
 * Results do not depend on band_rows.  CCL_ERR_HIP: an event could not be
 * made, or a copy or launch was rejected (work enqueued before it stays
 * enqueued).  Other errors as for ccl_label.
 */
int ccl_label_host(const void *host_colours, int dtype, int64_t batch, int64_t height,
                   int64_t width, int connectivity, int flags, uint32_t ignore, int32_t *host_out,
                   int32_t *counts, void *dev_colours, int32_t *dev_out, void *workspace,
                   size_t workspace_bytes, int64_t band_rows, void *stream, void *h2d_stream,
                   void *d2h_stream);

/*
 * ccl_label with CCL_NUMBER that also computes the per-region statistics of
 * ccl_region_stats (area, bounding box, sums of row and column indices), in
 * the same call, from the run records the final write expands instead of
 * from the labels ("About Connected Components Labeling on GPU",
 * introduction: bounding boxes; the tissue-scan segmentation article, section
 * 1.1: area and position of each numbered region, section 6.1: sums gathered
 * per block before global atomics).  A region inside one 64 x 32 tile gets its
 * record there whole; a region crossing tile edges has its record opened by
 * its root seam node and its parts, gathered per block of 8 x 8 tiles, added
 * with atomics.
 *   flags           must contain CCL_NUMBER (CCL_ERR_FLAGS otherwise); may
 *                   contain CCL_IGNORE
 *   counts          device int32 [batch], required
 *   stats           device ccl_region [stats_capacity], 8-byte aligned: region
 *                   k of image b is record counts[0] + ... + counts[b-1] + k - 1
 *   stats_capacity  records the caller has room for (>= 0); records past it
 *                   are not written.  The number of records written is
 *                   min(capacity, counts[0] + ... + counts[batch-1]); the sum
 *                   of counts tells whether the capacity was enough.
 * Every record below the capacity and the regions' total is written, each
 * once, with the values ccl_region_stats gives for the same labels.  Other
 * arguments, memory, streams and errors as for ccl_label; the workspace is
 * the one of ccl_workspace_bytes(batch, height, width).
 */
int ccl_label_stats(const void *colours, int dtype, int64_t batch, int64_t height, int64_t width,
                    int connectivity, int flags, uint32_t ignore, int32_t *out, int32_t *counts,
                    ccl_region *stats, int64_t stats_capacity, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace ccl_label_large needs for a batch of this shape
 * and band height (256-byte aligned; its first 4 bytes are the error word, as
 * for ccl_workspace_bytes).  Pure host arithmetic.  Returns 0 for an empty
 * batch and SIZE_MAX for a shape or band height ccl_label_large rejects.
 * The same for leaders and numbers: the tile pipeline's workspace for every
 * band of one image (about 4 bytes per pixel), each seam's two tile rows of
 * numbers and of leaders, and tables of a few bytes per seam pixel.
 */
size_t ccl_large_workspace_bytes(int64_t batch, int64_t height, int64_t width, int64_t band_rows);

/*
 * ccl_label for images of any size, beyond 2^31 pixels ("Accountable AI starts
 * at the pixel", ch.11 "How we know it is right", names such images as not run;
 * ch.10 shows a size wrapped to 32 bits): the same leaders, numbers and
 * counts, as 64-bit values.
 *   colours, dtype, connectivity, flags, ignore   as for ccl_label
 *   band_rows  0: automatic (about 2^30 pixels per band); else the rows of each
 *              band, a multiple of 64 with band_rows*width <= 2^31-1
 *              (CCL_ERR_BAND otherwise).  Results do not depend on it.
 *   out        device int64 [batch, height, width]: leaders (per-image reading-
 *              order index, -1 for an ignored pixel) or, with CCL_NUMBER,
 *              numbers 1..n (0 for an ignored pixel)
 *   counts     device int64 [batch] or NULL: regions per image
 *   workspace  device, at least ccl_large_workspace_bytes(batch, height, width,
 *              band_rows)
 * The image is cut into bands of band_rows rows; each band numbers its own
 * regions with the pipeline of ccl_label, the regions that continue across a
 * seam are joined by (band, number), and each band's final write turns its
 * numbers, or its leaders, into the picture's as it writes them (no 32-bit
 * array over the picture).  Images of a batch are labelled one after another.
 * CCL_ERR_TOO_LARGE: height*width*batch > 2^46, a band of 64 rows is wider
 * than 2^31-1 pixels, or the seams hold more than 2^31-3 pixels (2*width per
 * seam: seam pixels have int32 ids).  Memory, streams and errors as for
 * ccl_label.
 */
int ccl_label_large(const void *colours, int dtype, int64_t batch, int64_t height, int64_t width,
                    int connectivity, int flags, uint32_t ignore, int64_t band_rows,
                    int64_t *out, int64_t *counts, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * ccl_label without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It calls no allocating routine; its workspace is a
 * static device array of CCL_SCRATCH_BYTES (64 MiB) that each GPU the library
 * runs on holds until the process ends (its address is looked up once per
 * device, on the first call there).
 *   arguments  as for ccl_label, less the workspace; the caller still passes
 *              the input, `out` and `counts`
 * CCL_ERR_SCRATCH: ccl_workspace_bytes(batch, height, width) exceeds
 * CCL_SCRATCH_BYTES (about 17 Mpx of 64 x 32 tiles: a batch of 64 images of
 * 512 x 512, or one 4096 x 4096 image, fits).  CCL_ERR_HIP: the array's
 * address could not be looked up, or a launch failed.
 * Every call on one GPU uses the same array, which keeps the last call's
 * contents (each call clears what must start empty, its error word included):
 * two calls on one GPU whose work overlaps in time, e.g. on two streams, race
 * and give wrong results; serialise them (one stream, or events).  The error
 * word of ccl_workspace_bytes is not reported by this entry point.
 * Same results as ccl_label.
 */
#define CCL_SCRATCH_BYTES ((size_t)64 << 20)
int ccl_label_noalloc(const void *colours, int dtype, int64_t batch, int64_t height,
                      int64_t width, int connectivity, int flags, uint32_t ignore, int32_t *out,
                      int32_t *counts, void *stream);

/* Static text for a status code (never NULL). */
const char *ccl_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CCL_H */
