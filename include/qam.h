/*
 * qam.h -- C ABI of libqam: mixed-depth reads of one stored int8 weight copy
 * on AMD Instinct MI355X (gfx950).
 *
 * One stored copy of int8 weights is kept as four residual 2-bit slices.
 * Each block of 64 output rows is read at its own depth from the ladder
 * ZERO < D2 < D4 < D6 < D8; a block read at d bits touches d/2 slices and a
 * ZERO block touches nothing.  The depth of every block comes from a level
 * map (one byte per block) built by the lens rules or set uniformly (the
 * top-4-bit pass and its 8-bit re-run).
 *
 * Sources (cited by page title and section):
 *   [FoQLens]  "FoQLens" (foqlens.sawking.tech), table "Progress" and section
 *              "FoQZones, the mechanism".
 *   [Lens]     "FoQLens" landing page (vovanda.github.io/FoQLens), section
 *              "The mechanism" and the field description.
 *   [PoD]      "Precision on Demand: Escalating Weight Bits at Uncertain
 *              Decoding Steps in a Small Local Model" (arXiv:2611.14418 v1),
 *              abstract.
 *
 * Conventions shared by every call:
 *   - Pointers marked (device) are HIP device pointers owned by the caller;
 *     pointers marked (host) are host memory owned by the caller and only
 *     read during the call.  The library never allocates or frees device
 *     memory; the one static device array it holds is the scratch of
 *     qam_qmatvec_noalloc.
 *   - Work is enqueued on the caller's stream `s` (0 = the null stream) and
 *     is asynchronous: outputs are ready once the stream has reached that
 *     point (calls whose description says they synchronise `s` return with
 *     their work done).  A kernel fault surfaces at the caller's next
 *     synchronisation.
 *   - Every argument check runs on the host before anything is enqueued.  On
 *     failure a negative QAM_ERR_* code is returned, nothing is enqueued and
 *     qam_last_error() describes the problem.  Nothing aborts or throws across
 *     the ABI, and no call falls back silently to another kernel variant:
 *     qam_last_variant() names the variant the last successful call ran.
 *   - Calls are reentrant: the library keeps no state but the thread-local
 *     error and variant strings (and, for qam_qmatvec_noalloc alone, one
 *     scratch array per GPU).  Launch plans are fixed per call (defaults)
 *     or per group at qam_group_init_tuned, never process-wide.
 *   - Device-side errors (a level map holding a rung that is not a depth of
 *     the product) do not fault: the kernel raises a bit in the status word
 *     of the call's workspace (qam_status reads and clears it) and writes NaN
 *     for the outputs it could not compute.  Nothing is read silently at
 *     another depth.
 */
#ifndef QAM_H
#define QAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- errors */
#define QAM_OK             0
#define QAM_ERR_NULL      -1   /* a required pointer is NULL                      */
#define QAM_ERR_SHAPE     -2   /* N or K not a multiple of 64, or out of range    */
#define QAM_ERR_ARG       -3   /* a scalar argument is out of range              */
#define QAM_ERR_LADDER    -4   /* ladder not accepted by this call                */
#define QAM_ERR_ALIGN     -5   /* a pointer is not aligned as required            */
#define QAM_ERR_HIP       -6   /* a HIP runtime call failed                       */
#define QAM_ERR_WORKSPACE -7   /* workspace missing or too small                  */
#define QAM_ERR_IO        -8   /* a stack file cannot be opened, read or written,
                                  or is not a well-formed stack file            */

#define QAM_ROWS_PER_BLOCK 64
#define QAM_MAX_K          65536      /* keeps every exact integer sum in range */
#define QAM_MAX_LENSES     64
#define QAM_MAX_RUNGS      16
#define QAM_MAX_BATCH      1          /* requests per call on the staged-limb route   */
#define QAM_MAX_BATCH_MFMA 32         /* requests per qam_qmatvec call (matrix cores) */
#define QAM_MAX_BLOCKS     65536      /* blocks per matrix (N <= 4,194,304)         */
#define QAM_MAX_FIELD_BLOCKS 262144   /* blocks of a field for qam_field_width       */
/* Every workspace (and a group's or a decoder's device memory) starts with a
 * counter region: per-block arrival counters, then the status word. */
#define QAM_WS_STATUS_OFFSET (QAM_MAX_BLOCKS * 4)
#define QAM_WS_COUNTER_BYTES (QAM_MAX_BLOCKS * 4 + 256)

/* Status bits (qam_status). */
#define QAM_STATUS_BAD_RUNG 1u        /* a level map held a rung above 4: the blocks
                                         concerned were not read and their outputs
                                         are NaN */

/* Size of the static scratch array of qam_qmatvec_noalloc (per GPU). */
#define QAM_SCRATCH_BYTES (32 * 1024 * 1024)

#define QAM_X_F32  0
#define QAM_X_BF16 1

/* ---------------------------------------------------------------- packed weights */
/*
 * Slice-major layout of one packed matrix W [N][K] (int8, row-major input):
 *
 *   bytes [0, N*K)            four planes of N*K/4 bytes each.  Plane p holds the
 *                             2-bit digit s = 3 - p of every code (p = 0 is the
 *                             top digit and carries the sign), so reading depth d
 *                             touches planes 0 .. d/2-1 only.
 *   bytes [N*K, N*K + 4N)     the per-row fp32 scales (copied at pack time).
 *
 * Inside a plane: block b (rows 64b .. 64b+63) owns 16*K contiguous bytes;
 * inside a block, tile t (columns 64t .. 64t+63) owns 1024 bytes; inside a
 * tile, lane L (0..63) owns 16 bytes = four 32-bit words j = 0..3.  Word j
 * holds the digits of row 16j + (L & 15), columns 16(L >> 4) + 4u + i
 * (u, i = 0..3), the digit for (u, i) at bit (8i + 2s - 2u) mod 32.  A group
 * of four digits therefore rotates into a byte-aligned int8x4 word with one
 * mask per slice and one rotation.
 */
typedef struct qam_packed {
    int64_t N;          /* output rows, multiple of 64            */
    int64_t K;          /* input columns, multiple of 64, <= QAM_MAX_K */
    int64_t n_blocks;   /* N / 64                                 */
    void*   planes;     /* (device) qam_packed_bytes(N, K) bytes, 256-B aligned */
    float*  scales;     /* (device) = (float*)((char*)planes + N*K)  */
} qam_packed;

/* Bytes of one packed matrix: N*K slice bytes + 4*N scale bytes. */
size_t qam_packed_bytes(int64_t N, int64_t K);

/*
 * qam_pack_slices -- split int8 codes into the four residual 2-bit slices.
 *   [FoQLens] "Progress": one stored stack, a base with refinements over it,
 *   any depth read from the same copy without repacking; [Lens] "The
 *   mechanism": one stored copy of residual slices read at 2, 4, 6 or 8 bits.
 *
 *   W        (device) int8 [N][K], row-major, any values (-128 allowed).
 *   scales   (device) fp32 [N] per-row scales.
 *   N, K     multiples of 64; K <= QAM_MAX_K.
 *   out      (device) qam_packed_bytes(N, K) bytes, 256-byte aligned; must
 *            not overlap W or scales.
 *   desc_out (host)   filled with N, K, n_blocks, planes = out, scales.
 * Packing happens once per matrix (offline); W and scales may be freed once
 * the stream has passed this call.
 */
int qam_pack_slices(const int8_t* W, const float* scales, int64_t N, int64_t K,
                    void* out, size_t out_bytes, qam_packed* desc_out, hipStream_t s);

/*
 * qam_describe_packed -- fill a descriptor for an already packed buffer.
 */
int qam_describe_packed(void* packed_buf, int64_t N, int64_t K, qam_packed* desc_out);

/*
 * qam_unpack_codes -- debug probe: the int8 codes the product kernels read.
 *   Writes codes_out[n][k] = the code of W[n][k] truncated to the depth of
 *   block n/64 in `level_map`, rebuilt from the slices by the same device
 *   routine the product kernels use.  ZERO blocks give 0.
 *   packed    (host)   descriptor from qam_pack_slices.
 *   level_map (device) uint8 [n_blocks], rung indices 0..4 of {0,2,4,6,8}.
 *   codes_out (device) int8 [N][K].
 */
int qam_unpack_codes(const qam_packed* packed, const uint8_t* level_map, int8_t* codes_out,
                     hipStream_t s);

/* ---------------------------------------------------------------- stored stack */
/*
 * One stored stack on disk ([FoQLens] "Progress": one stored copy, a base
 * with refinements over it, read at 2, 4, 6 or 8 bits without repacking).
 * The file holds the packed planes of many matrices, plane-major, so that a
 * read at depth d is the first d/2 plane sections of the file plus the
 * scales: one contiguous prefix and one tail, no repacking on load.
 *
 * Layout (all integers little-endian; every offset a multiple of 256):
 *   [0, 128)                   qam_stack_header
 *   [128, 128 + 64 n)          n qam_stack_entry, one per matrix, in order
 *   zero bytes up to data_offset = round_up(128 + 64 n, 4096)
 *   plane sections p = 0 .. 3, each plane_section_bytes long, starting at
 *                              data_offset + p * plane_section_bytes; inside
 *                              section p, matrix m's plane p (N K / 4 bytes,
 *                              the packed layout above) at entry.plane_offset
 *                              = sum of N K / 4 over the matrices before m
 *   scales section at scales_offset = data_offset + 4 plane_section_bytes:
 *                              matrix m's N fp32 scales at scales_offset +
 *                              entry.scales_offset, = sum of 4 N over the
 *                              matrices before m
 *   file_bytes = scales_offset + scales_bytes.
 */
#define QAM_STACK_VERSION       1
#define QAM_STACK_NAME_BYTES    32
#define QAM_STACK_MAX_MATRICES  65536
#define QAM_STACK_ALIGN         4096

typedef struct qam_stack_header {        /* 128 bytes */
    char     magic[8];                   /* "QAMSTACK" (no terminator)            */
    uint32_t version;                    /* QAM_STACK_VERSION                     */
    uint32_t n_matrices;                 /* 1 .. QAM_STACK_MAX_MATRICES           */
    uint32_t n_rungs;                    /* 5                                     */
    uint8_t  ladder_bits[16];            /* {0, 2, 4, 6, 8}, then zeros           */
    uint32_t rows_per_block;             /* 64                                    */
    uint64_t data_offset;                /* start of plane section 0              */
    uint64_t plane_section_bytes;        /* sum of N K / 4                        */
    uint64_t scales_offset;              /* start of the scales section           */
    uint64_t scales_bytes;               /* sum of 4 N                            */
    uint64_t file_bytes;                 /* total length                          */
    uint8_t  reserved[48];               /* zeros                                 */
} qam_stack_header;

typedef struct qam_stack_entry {         /* 64 bytes */
    int64_t  N, K;                       /* shape, as in qam_packed               */
    uint64_t plane_offset;               /* offset inside every plane section     */
    uint64_t scales_offset;              /* offset inside the scales section      */
    char     name[QAM_STACK_NAME_BYTES]; /* NUL-padded; may be all NUL            */
} qam_stack_entry;

/*
 * qam_stack_write -- write packed matrices to a stack file (created or
 *   truncated).  Synchronises `s` first (the planes must be complete), then
 *   copies the planes and scales out of device memory through pinned host
 *   staging buffers that the call allocates and frees.
 *   path       (host) file name.
 *   mats       (host) n_matrices descriptors from qam_pack_slices.
 *   names      (host) NULL, or n_matrices C strings (NULL entries allowed) of
 *              at most QAM_STACK_NAME_BYTES - 1 characters.
 *   Returns QAM_ERR_IO when the file cannot be written (a partial file may be
 *   left behind).
 */
int qam_stack_write(const char* path, const qam_packed* mats, const char* const* names, int n_matrices,
                    hipStream_t s);

/*
 * qam_stack_info -- read and check a stack file's header and table.
 *   hdr_out     (host) the header.
 *   entries_out (host, may be NULL) room for max_entries entries; the first
 *               min(n_matrices, max_entries) are written.
 *   Every field is checked against the layout above (magic, version, ladder,
 *   offsets, shapes, and the file's length); QAM_ERR_IO names the first
 *   mismatch.  Host only: no device call.
 */
int qam_stack_info(const char* path, qam_stack_header* hdr_out, qam_stack_entry* entries_out, int max_entries);

/*
 * qam_stack_read -- load matrices [first, first + count) of a stack file at
 *   depth 2 * slices bits into caller device buffers.
 *   slices      1 .. 4: planes 0 .. slices-1 are read; planes slices .. 3
 *               of each destination are zero-filled, so any deeper read of
 *               the loaded matrix returns the codes at depth 2 * slices.
 *   dst         (host) count descriptors (qam_describe_packed on caller
 *               buffers of qam_packed_bytes(N, K)), shapes equal to the
 *               file's entries.
 *   bytes_read  (host, may be NULL) bytes read from the file:
 *               slices * sum(N K / 4) + sum(4 N) over the matrices loaded.
 *   The file is read with large sequential reads into pinned host staging
 *   buffers (allocated and freed by the call), double-buffered against the
 *   host-to-device copies on `s`; returns after `s` has been synchronised.
 */
int qam_stack_read(const char* path, int slices, int first, int count, const qam_packed* dst, hipStream_t s,
                   uint64_t* bytes_read);

/* ---------------------------------------------------------------- level maps */
typedef struct qam_lens {
    double cx, cy;      /* centre on the 2-D block field */
    double r;           /* size r_i >= 0 (the radius is R_i = r_i f / (1 - f)) */
} qam_lens;

#define QAM_COMBINE_SUM 0
#define QAM_COMBINE_MAX 1
#define QAM_MAX_STOPS   (QAM_MAX_RUNGS - 1)

#define QAM_RADIUS_LENS 0   /* R_i = r_i f / (1 - f)     ([Lens] "The mechanism") */
#define QAM_RADIUS_ZONE 1   /* R = f D, D the field width ([FoQLens] "FoQZones, the
                               mechanism", rule 1: f = 0 the centre only, f = 1 the
                               whole network); every lens the same R, r_i unused */

typedef struct qam_lens_params {
    double f;           /* focus_area, in [0, 1]                        */
    double g;           /* focus_strength, in [0, 1]                    */
    int    combine;     /* QAM_COMBINE_SUM or QAM_COMBINE_MAX           */
    int    n_stops;     /* 0: default stops; else must equal kappa - glass */
    double stops[QAM_MAX_STOPS]; /* s_(glass+1) > s_(glass+2) > ... > s_kappa > 0, in radii */
    int    radius_mode; /* QAM_RADIUS_LENS (0) or QAM_RADIUS_ZONE       */
    int    reserved;
    double width;       /* zone mode: the field width D >= 0 (e.g. qam_field_width) */
} qam_lens_params;

/*
 * qam_build_level_map -- per-block rung index from the lens rules.
 *   [Lens] "The mechanism" rules 1-6 and [FoQLens] "FoQZones, the mechanism":
 *     R_i = r_i f / (1 - f); kappa = glass + floor(g (m - glass));
 *     rho_i(b) = d(b, c_i) / R_i; L_i(b) = max(0, 1 - rho_i(b) / s_last);
 *     L(b) = min(1, sum_i L_i) or max_i L_i; rho* = s_last (1 - L(b));
 *     level = the ring rho* falls into, the glass outside every lens.
 *   Readings: d is Euclidean on the block coordinates; s_last = s_(glass+1);
 *   default stops s_(glass+j) = (n - j + 1) / n with n = kappa - glass; rings
 *   are half-open (level = glass + #{j : rho* < s_(glass+j)}); f = 1 gives
 *   R = +inf; R = 0 lifts only a block at distance 0.
 *   One thread per block, fp64 throughout, no contraction into FMA, correctly
 *   rounded sqrt and division: the map is bit-identical to the same rules run
 *   in IEEE fp64 on a CPU.
 *
 *   With params->radius_mode == QAM_RADIUS_ZONE the radius is the zone
 *   rule R = f D of [FoQLens] "FoQZones, the mechanism" (rule 1), D =
 *   params->width, the same for every lens; the other rules are unchanged.
 *
 *   coords      (device) fp64 [n_blocks][2], finite.
 *   n_blocks    >= 0 (0 enqueues nothing).
 *   lenses      (host) [n_lenses], n_lenses in [0, QAM_MAX_LENSES]; r >= 0.
 *   params      (host) f, g in [0, 1]; explicit stops strictly decreasing, > 0;
 *               radius_mode and, for zones, a finite width >= 0.
 *   ladder_bits (host) [n_rungs]: the product ladder {0, 2, 4, 6, 8}
 *               (n_rungs = 5), so that a rung index is the number of slices
 *               qam_qmatvec reads; QAM_ERR_LADDER otherwise (the rules on
 *               other ladders: qam_build_rung_map).
 *   glass       rung index gamma in [0, n_rungs - 1].
 *   level_out   (device) uint8 [n_blocks].
 * A uniform map (every block at one rung, e.g. the all-D4 pass and its D8
 * re-run of [PoD]) is this call with n_lenses = 0 and glass = that rung.
 */
int qam_build_level_map(const double* coords, int64_t n_blocks,
                        const qam_lens* lenses, int n_lenses, const qam_lens_params* params,
                        const uint8_t* ladder_bits, int n_rungs, int glass,
                        uint8_t* level_out, hipStream_t s);

/*
 * qam_build_rung_map -- the same rules on any ladder ([FoQLens] "FoQZones,
 *   the mechanism": the ladder is set by the model and its storage, the rules
 *   are generic): ladder_bits[0] == 0, strictly increasing, 2 <= n_rungs <=
 *   QAM_MAX_RUNGS; only the rung count enters the rules.  rung_out holds rung
 *   indices of that ladder, which are not read depths of qam_qmatvec unless
 *   the ladder is {0, 2, 4, 6, 8}.  Other arguments as qam_build_level_map.
 */
int qam_build_rung_map(const double* coords, int64_t n_blocks,
                       const qam_lens* lenses, int n_lenses, const qam_lens_params* params,
                       const uint8_t* ladder_bits, int n_rungs, int glass,
                       uint8_t* rung_out, hipStream_t s);

/*
 * qam_field_width -- the width D of a block field for the zone radius: the
 *   largest Euclidean distance between two blocks (its diameter), so that at
 *   f = 1 a zone around any block reaches every block ([FoQLens] "FoQZones,
 *   the mechanism", rule 1: f = 1 takes the whole network).  The maximum of
 *   the squared distances dx*dx + dy*dy (fp64, no contraction) is exact in
 *   any order; D = sqrt of it, correctly rounded.
 *   coords     (device) fp64 [n_blocks][2], finite, 8-byte aligned.
 *   n_blocks   1 .. QAM_MAX_FIELD_BLOCKS (one block gives D = 0).
 *   workspace  (device) 256 bytes, 256-byte aligned.
 *   width_out  (host) D.
 *   Host-synchronous.
 */
int qam_field_width(const double* coords, int64_t n_blocks, void* workspace, size_t workspace_bytes,
                    double* width_out, hipStream_t s);

/*
 * qam_build_level_maps -- one level map per request, n_maps of them, each by
 *   the rules of qam_build_level_map with its own lenses and parameters (the
 *   per-request maps of a batch).  Maps are computed in launches of up to 8
 *   maps (fewer when the maps' lenses would exceed QAM_MAX_LENSES).
 *   lenses     (host) [n_maps][n_lenses], map k's lenses at k * n_lenses.
 *   params     (host) [n_maps].
 *   n_maps     1 .. QAM_MAX_BATCH_MFMA.
 *   level_out  (device) uint8 [n_maps][n_blocks].
 *   Other arguments (the product ladder) and the numerics as
 *   qam_build_level_map; each map is bit-identical to a qam_build_level_map
 *   call with its lenses and params.
 */
int qam_build_level_maps(const double* coords, int64_t n_blocks, const qam_lens* lenses, int n_lenses,
                         const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs,
                         int glass, int n_maps, uint8_t* level_out, hipStream_t s);

/*
 * qam_fit_focus_area -- the byte-budget regulator: the largest focus area f
 *   in [0, 1] whose lens map reads at most budget_bytes of weights
 *   ([Lens] "The mechanism": memory is what the lenses cost, rule 7 bytes
 *   sum_b w_b bits(b) / 8; focus_area widens every lens).  Bytes never
 *   decrease as f grows, so f is found by bisection: f = 1 if it fits, else
 *   f = 0 if even that does not fit (then *bytes_out > budget_bytes), else
 *   `iters` halvings of [0, 1] keeping the end that fits.  Each step builds
 *   the map on the device (the kernel of qam_build_level_map, so the maps
 *   are those of the rules) and sums its bytes exactly in int64; the host
 *   reads the sum (one synchronisation of `s` per step).  Every decision is
 *   an integer comparison: f is the same double as the same bisection
 *   evaluated on a CPU.
 *   coords, n_blocks, lenses, n_lenses, ladder_bits, n_rungs, glass
 *               as qam_build_level_map; params: g, combine and stops (its f
 *               is not read).
 *   block_weights (device) int64 [n_blocks], w_b >= 0 (64 K for a block of
 *               a K-column matrix); sum_b w_b bits(b) must fit in int64.
 *   iters       0 .. 60.
 *   level_out   (device) uint8 [n_blocks]: the map at the returned f.
 *   workspace   (device) 256 bytes, 256-byte aligned.
 *   f_out, bytes_out  (host) the focus area and its bytes.
 *   Host-synchronous; not for graph capture.
 */
int qam_fit_focus_area(const double* coords, int64_t n_blocks, const int64_t* block_weights,
                       const qam_lens* lenses, int n_lenses, const qam_lens_params* params,
                       const uint8_t* ladder_bits, int n_rungs, int glass, int64_t budget_bytes,
                       int iters, uint8_t* level_out, void* workspace, size_t workspace_bytes,
                       double* f_out, int64_t* bytes_out, hipStream_t s);

/*
 * qam_layer_levels -- level maps decided by the layer from its own read at
 *   the base depth ([FoQLens] "FoQZones, the mechanism", the variant in which
 *   the layer decides; scores and levels stay on the device).  Per request r
 *   and block c (64 output rows):
 *     s^ = ((|y_c|^2 Delta_c^2) Delta_c^2) / w_c   (the reduced draft score),
 *   y_c the block's 64 values of y_base, Delta_c^2 the mean over its rows of
 *   the squared row scale, w_c = 64 K; rows summed in order in fp64 (the
 *   oracle's sums, bit for bit).  kappa = glass + floor(g (m - glass)),
 *   m = n_rungs - 1.  Rung:
 *     QAM_LAYER_THRESHOLD: glass + #{j in 1 .. kappa - glass : s^ >= lambda 16^j}
 *       (lambda is left open by the page: the caller's; a NaN score stays
 *       at the glass);
 *     QAM_LAYER_SHARE: the floor(share n_blocks) blocks of largest s^ rise
 *       to kappa (equal scores in block order, NaN scores never), the rest
 *       stay at the glass.  Cost O(n_blocks^2) comparisons per request.
 *   y_base     (device) fp32 [B][N], 16-byte aligned: the product at the
 *              base depth (a uniform map at `glass`), as qam_qmatvec writes it.
 *   B          0 .. 65535 requests (0: nothing is launched).
 *   w          (host) the packed matrix; only N, K and its scales are read.
 *   rule       (host) mode, lambda (not NaN), share in [0, 1], g in [0, 1].
 *   shat_out   (device) fp64 [B][n_blocks]: the scores (written in both modes).
 *   level_out  (device) uint8 [B][n_blocks]: the maps, as qam_qmatvec takes
 *              per-request maps (row r is request r's map).
 *   Errors: QAM_ERR_NULL, QAM_ERR_SHAPE, QAM_ERR_ARG, QAM_ERR_LADDER (glass
 *   outside the ladder), QAM_ERR_ALIGN.  Asynchronous on `s`.
 */
#define QAM_LAYER_THRESHOLD 0
#define QAM_LAYER_SHARE     1
typedef struct qam_layer_rule {
    int    mode;        /* QAM_LAYER_THRESHOLD or QAM_LAYER_SHARE */
    int    reserved;
    double lambda;      /* threshold mode: the lambda of lambda 16^j */
    double share;       /* share mode: the share f of the blocks that rise */
    double g;           /* focus strength: the ceiling kappa */
} qam_layer_rule;

int qam_layer_levels(const float* y_base, int64_t B, const qam_packed* w, const qam_layer_rule* rule,
                     int n_rungs, int glass, double* shat_out, uint8_t* level_out, hipStream_t s);

/*
 * qam_layer_levels_group -- qam_layer_levels for up to QAM_LAYER_GROUP_MAX
 *   matrices of one layer in one launch (same rule, glass and batch B; the
 *   same scores and maps, bit for bit, as one qam_layer_levels call per
 *   item).  A workgroup per (item, request) scores the request's blocks
 *   and, in share mode, ranks them in LDS, so every item must have at most
 *   512 blocks (QAM_ERR_SHAPE otherwise; call qam_layer_levels for larger
 *   ones).
 *   items   (host) [n_items], 1 <= n_items <= QAM_LAYER_GROUP_MAX: each
 *           item's base outputs, packed matrix, scores and maps, laid out
 *           and aligned as in qam_layer_levels.
 *   Errors: as qam_layer_levels, naming the item.  Asynchronous on `s`.
 */
#define QAM_LAYER_GROUP_MAX 16
typedef struct qam_layer_item {
    const float* y_base;   /* (device) fp32 [B][N] */
    qam_packed   w;        /* N, K and the scales are read */
    double*      shat_out; /* (device) fp64 [B][n_blocks] */
    uint8_t*     level_out;/* (device) uint8 [B][n_blocks] */
} qam_layer_item;

int qam_layer_levels_group(const qam_layer_item* items, int n_items, int64_t B, const qam_layer_rule* rule,
                           int n_rungs, int glass, hipStream_t s);

/*
 * qam_map_weight_bytes -- rule 7 and the bytes-read cost for a map (host).
 *   [Lens] rule 7: bits = sum_b w_b bits(b) / sum_b w_b; [PoD]: cost counted
 *   in weight bytes read.  w_b = 64 * K for every block of one matrix.
 *   level (host) uint8 [n_blocks]; ladder_bits (host) [n_rungs].
 *   Outputs (host, may be NULL): mean bits, weight bytes sum_b w_b bits(b)/8.
 */
int qam_map_weight_bytes(const uint8_t* level, int64_t n_blocks, int64_t K,
                         const uint8_t* ladder_bits, int n_rungs,
                         double* mean_bits, int64_t* weight_bytes);

/* ---------------------------------------------------------------- qmatvec */
/*
 * qam_qmatvec -- y[r][n] = scale[n] * sum_k c[n][k] x[r][k] with c the code
 *   of W[n][k] read at the depth of block n/64 ([FoQLens] "Progress": every
 *   block of rows read at its own depth straight from the stored bytes inside
 *   the pass; [PoD]: cost counted in weight bytes read).  A ZERO block loads
 *   nothing and writes y = 0.
 *
 *   Arithmetic (exact integer products on a fixed-point x): x is taken in
 *   chunks of columns per request (sub-chunks of 1024 columns at B = 1, the
 *   column chunks of the pre-pass at B > 1).  With 2^(e-1) <= max|x| < 2^e
 *   over the chunk,
 *     q1 = round(x 2^(22-e)),  r1 = x - q1 2^(e-22),
 *     q2 = round(r1 2^(45-e)), r2 = r1 - q2 2^(e-45)       (r1, r2 exact),
 *   each q held as three signed int8 limbs; c . q1 and c . q2 are accumulated
 *   exactly in int32 (v_mfma_i32_16x16x64_i8) and scaled into an fp64 row
 *   sum.  |r2| <= 2^(e-46); an element with |r2| > 2^-15 |x| (possible only
 *   for |x| < 2^(e-31)) is "uncovered": on the pre-pass route (B > 1) its
 *   c * r2 is added exactly in fp64 afterwards; at B = 1 a sub-chunk holding
 *   one is computed instead in fp32 on the vector ALUs (each lane sums at
 *   most 256 products c x, one rounding per fused multiply-add, and the lane
 *   sums meet in fp64: relative error at most 2^-16 of that sub-chunk's
 *   sum |w||x|).  On the pre-pass route a (chunk, request) whose coarse split
 *   (q1, then one digit q2c = round(r1 2^(29-e)), r2c = r1 - q2c 2^(e-29),
 *   |r2c| <= 2^(e-30)) leaves at most 4 elements with |r2c| > 2^-15 |x|
 *   multiplies four limb columns instead of six, and those elements' c * r2c
 *   are added exactly instead.  Every element therefore enters the sum with
 *   relative error at most 2^-15, and for every finite x and every code
 *     |y - y_exact| <= 2^-15 sum_k |w_k||x_k| + 2^-24 |y_exact| (+ fp64 sums),
 *   inside 1e-4 sum|w||x|.  Chunks are summed in fp64 in a fixed order and
 *   y = fl32(scale * sum): results are bit-reproducible run to run (for one
 *   launch plan: x's split is per column chunk, so plans that chunk K
 *   differently can differ in the last bits).
 *   Integer-valued x with |x| < 2^22 and scale 1 gives exact integer
 *   outputs; a D8 map gives the untruncated int8 product.  A non-finite x
 *   makes that request's non-ZERO outputs NaN.
 *
 *   Routes.  B = 1, the staged-limb route: each wavefront stages its
 *   sub-chunk's limbs in LDS inside the product kernel and multiplies the
 *   rebuilt codes (four int8x4 words per 16-byte slice word, 16 rows x 64
 *   columns per lane group) by them, B-operand column l holding limb l.
 *   B = 2 .. 32, the pre-pass route: a pre-pass writes the limbs of x per
 *   column chunk as MFMA B operands (four or six columns per request, up to 16
 *   requests per set) and lists each chunk's uncovered elements, then the
 *   product kernel multiplies the codes by them.  With per-request maps a
 *   block is read once, to the deepest slice any request needs, and each
 *   request gets the codes at its own depth, built from the same words (the
 *   residual slices make the code at depth d the sum of the first d/2
 *   slices): the codes at each depth present are multiplied by the limbs of
 *   the requests at that depth.
 *
 *   x          (device) [B][K] row-major, fp32 (x_dtype QAM_X_F32) or bf16
 *              (QAM_X_BF16); 16-byte aligned.
 *   B          1 .. QAM_MAX_BATCH_MFMA requests.
 *   packed     (host) descriptor from qam_pack_slices.
 *   level_map  (device) uint8 rung indices of the ladder {0,2,4,6,8}
 *              (rung index = slices read): [n_blocks] shared by all requests
 *              (per_request_maps = 0) or [B][n_blocks], one map per request
 *              (per_request_maps = 1).  A rung above 4 raises
 *              QAM_STATUS_BAD_RUNG; its outputs are NaN.
 *   y          (device) fp32 [B][N], must not overlap x.
 *   workspace  (device) qam_qmatvec_workspace_bytes(N, K, B) bytes (at least
 *              QAM_WS_COUNTER_BYTES), 256-byte aligned.  Its first
 *              QAM_WS_COUNTER_BYTES hold per-block arrival counters and the
 *              status word: they must be zero before the first use; every
 *              call leaves the counters zero again, whatever the shape, so
 *              one buffer serves calls of any shape.  The rest holds fp64
 *              partial sums, limbs and lists that each call writes before it
 *              reads.  Calls that share a workspace must be ordered (same
 *              stream or synchronised).
 *   N          at most QAM_MAX_BLOCKS blocks of 64 rows (half that for
 *              B > 16 on the pre-pass route).
 */
size_t qam_qmatvec_workspace_bytes(int64_t N, int64_t K, int64_t B);

int qam_qmatvec(const void* x, int x_dtype, int64_t B, const qam_packed* packed,
                const uint8_t* level_map, int per_request_maps, float* y,
                void* workspace, size_t workspace_bytes, hipStream_t s);

/*
 * qam_status -- read the status word of a workspace (or of a group's or a
 *   decoder's device memory: the dev_mem given at init), optionally clearing
 *   it.  Bits QAM_STATUS_*; 0 when every launch since the last clear ran as
 *   documented.  Host-synchronous; a debugging aid, not needed for results.
 */
int qam_status(const void* workspace, int clear, uint32_t* status_out, hipStream_t s);

/*
 * qam_qmatvec_noalloc -- qam_qmatvec for callers that cannot allocate device
 *   memory (code under HIP graph capture, tight serving loops, harnesses that
 *   forbid hipMalloc).  Same arguments and the same result, bit for bit, as
 *   qam_qmatvec, with no workspace argument: the workspace is a static
 *   256-byte aligned device array of QAM_SCRATCH_BYTES bytes built into the
 *   library, one copy per GPU, held until the process ends.  The call never
 *   allocates or frees memory.
 *
 *   A shape whose qam_qmatvec_workspace_bytes(N, K, B) exceeds
 *   QAM_SCRATCH_BYTES is rejected with QAM_ERR_WORKSPACE before anything is
 *   enqueued (use qam_qmatvec with a workspace of that size).  The first
 *   call on a device also enqueues, on `s`, a clear of the array's counter
 *   region.  Every call on one GPU shares that GPU's array, which keeps the
 *   last call's contents: calls that overlap on one GPU (different streams
 *   without ordering, or different threads) race and give wrong results.
 *   The array's status word is not exposed; a rung above 4 still yields NaN
 *   outputs.  Errors as qam_qmatvec, plus QAM_ERR_HIP when the array's
 *   device address cannot be looked up.
 */
int qam_qmatvec_noalloc(const void* x, int x_dtype, int64_t B, const qam_packed* packed,
                        const uint8_t* level_map, int per_request_maps, float* y, hipStream_t s);

/* ---------------------------------------------------------------- fused epilogues */
/*
 * qam_qmatvec_ep -- qam_qmatvec with the glue of a decode step folded into
 *   the product's last stage, so a decoder layer is one launch per matrix.
 *   None of this is from the pages: it is the plainest stand-in for the
 *   normalisation and gated activation around the weight reads of the
 *   decoder-only model the [PoD] abstract decodes (Qwen3-0.6B), so that a
 *   decode step can be timed as tokens/s with no kernel other than the
 *   mixed-depth product.  One request (B = 1).
 *
 *   With v[r][n] = scale[n] * sum_k c[n][k] x'[r][k], where
 *     x' = x                                 (ep->rms_norm == 0)
 *     x' = x / sqrt(mean_k x[r][k]^2 + eps)   (ep->rms_norm == 1; the factor
 *          is applied to the exact row sum, computed in fp64 over all K),
 *   the output is
 *     QAM_OUT_STORE: y[r][n] = fl32(v)
 *     QAM_OUT_ADD:   y[r][n] = fl32(y[r][n] + v)        (residual; y is read)
 *     QAM_OUT_GLU:   block b's rows 64b..64b+31 are gate rows and rows
 *                    64b+32..64b+63 the up rows of features 32b..32b+31;
 *                    y[r][32b+i] = fl32(silu(v_gate) * v_up), silu(t) =
 *                    t / (1 + e^-t), in fp64; y is [B][N/2].
 *   A ZERO block reads nothing: v = 0 for its rows (QAM_OUT_ADD leaves y as
 *   it is, QAM_OUT_GLU writes 0).  Other arguments, the workspace and the
 *   error bound (on v) are those of qam_qmatvec's staged-limb route; y must
 *   not overlap x.  B = 1; ep == NULL is qam_qmatvec at B = 1.
 */
#define QAM_OUT_STORE 0
#define QAM_OUT_ADD   1
#define QAM_OUT_GLU   2

typedef struct qam_epilogue {
    int    rms_norm;   /* 0 or 1                                  */
    int    out_mode;   /* QAM_OUT_STORE, QAM_OUT_ADD, QAM_OUT_GLU */
    double eps;        /* >= 0, used when rms_norm == 1           */
} qam_epilogue;

int qam_qmatvec_ep(const void* x, int x_dtype, int64_t B, const qam_packed* packed,
                   const uint8_t* level_map, const qam_epilogue* ep, float* y,
                   void* workspace, size_t workspace_bytes, hipStream_t s);

/* ---------------------------------------------------------------- grouped qmatvec */
/*
 * A group runs qam_qmatvec over many matrices, each with its own x, y and
 * level map, in ONE launch ([FoQLens] "Progress": the whole pass reads every
 * block at its own depth).  Typical use: every matrix of a weight field, or
 * the matrices of one layer that take different inputs.  The pointers are
 * bound once by qam_group_init; qam_qmatvec_group then replays the product
 * on whatever the bound buffers hold (e.g. once per decode step).
 */
typedef struct qam_gemv_item {
    qam_packed     w;          /* descriptor from qam_pack_slices                    */
    const void*    x;          /* (device) [B][w.K], fp32 or bf16, 16-byte aligned   */
    float*         y;          /* (device) [B][w.N]                                  */
    const uint8_t* level_map;  /* (device) rungs of {0,2,4,6,8}: [w.n_blocks] shared by
                                  the B requests, or per request B rows of w.n_blocks */
    int64_t        level_stride; /* per-request maps: bytes from one request's row to the
                                  next (0: w.n_blocks), e.g. the block count of a whole
                                  field whose maps are stored [B][field blocks]        */
    const double*  coords;     /* (device) fp64 [w.n_blocks][2] block coordinates on the
                                  field, e.g. rows of the field's coordinate array; only
                                  qam_qmatvec_group_lens reads them (may be NULL)     */
} qam_gemv_item;

typedef struct qam_group {     /* filled by qam_group_init; treat as opaque          */
    void*   dev_mem;           /* (device) the dev_mem given at init (counters, status) */
    int     ksplit;            /* pre-pass route: waves per request set on a chunk    */
    int     n_items;
    int64_t B;
    int     x_dtype;
    int64_t n_workgroups;
    size_t  lds_bytes;
    void*   table;             /* (device) descriptor table inside dev_mem           */
    void*   wg_map;            /* (device) workgroup -> item map inside dev_mem      */
    int     route;             /* 0: staged-limb route, 1: pre-pass route            */
    int     per_request_maps;
    int64_t n_pre_workgroups;  /* pre-pass route: limb pre-pass workgroups           */
    void*   pre_map;           /* (device) pre-pass workgroup -> item map            */
    int     lens_ready;        /* 1: staged-limb route with every item's coords bound */
    int     sets;              /* pre-pass route: request sets per workgroup          */
    int     set_size;          /* pre-pass route: requests per set                    */
    int     col_groups;        /* pre-pass route: 16-column groups per set            */
} qam_group;

/* Device bytes qam_group_init needs (0 if the items are invalid).  The route
 * is chosen as by qam_qmatvec from B. */
size_t qam_group_bytes(const qam_gemv_item* items, int n_items, int64_t B, int per_request_maps);

/*
 * Launch-plan settings of a group: how the work is cut into workgroups, never
 * the results (every setting gives the same bits).  0 in a field takes the
 * library's default.
 */
typedef struct qam_tuning {
    int target_waves;      /* wavefronts aimed for per launch (64 .. 2^20)           */
    int max_chunk_tiles;   /* B = 1: longest column chunk, in 64-column tiles        */
    int tail_pct;          /* B = 1: share of the block tiles planned with short chunks
                              (-1: none)                                              */
    int tail_div;          /* B = 1: how much shorter (1 .. 64)                      */
    int ksplit;            /* B > 1: waves per request set splitting a chunk (1, 2, 4) */
    int set_max;           /* B > 1: most requests per set (8 .. 16)                 */
    int tiles_per_request; /* B > 1: shortest chunk, in tiles per request (1 .. 64)  */
} qam_tuning;

size_t qam_group_bytes_tuned(const qam_gemv_item* items, int n_items, int64_t B, int per_request_maps,
                             const qam_tuning* tuning);

/*
 * qam_group_init -- validate the items (as qam_qmatvec does for each), lay
 *   out and upload the descriptor table, and zero the counter region.
 *   items    (host) [n_items]; sum of blocks <= QAM_MAX_BLOCKS.
 *   dev_mem  (device) qam_group_bytes(...) bytes, 256-byte aligned, owned by
 *            the caller and kept alive as long as the group is used; it holds
 *            the counters, fp64 partials, the table and the workgroup map.
 *   Synchronises `s` before returning (one-time set-up, not for graph capture).
 */
int qam_group_init(const qam_gemv_item* items, int n_items, int64_t B, int x_dtype,
                   int per_request_maps, void* dev_mem, size_t dev_bytes, qam_group* group_out,
                   hipStream_t s);

/* qam_group_init with a launch plan of the caller's (tuning may be NULL:
 * defaults); the plan is stored in the group and used by every launch of it.
 * dev_bytes from qam_group_bytes_tuned with the same tuning. */
int qam_group_init_tuned(const qam_gemv_item* items, int n_items, int64_t B, int x_dtype,
                         int per_request_maps, const qam_tuning* tuning, void* dev_mem, size_t dev_bytes,
                         qam_group* group_out, hipStream_t s);

/*
 * qam_qmatvec_group -- one launch (two on the pre-pass route: the limb
 *   pre-pass, then the product) computing y_i = the mixed-depth product of
 *   every item i, with exactly the arithmetic of qam_qmatvec.  Enqueues
 *   kernels and nothing else (safe to capture in a HIP graph).  Calls on one
 *   group must be ordered.
 */
int qam_qmatvec_group(const qam_group* group, hipStream_t s);

/*
 * qam_qmatvec_group_refine -- the group's product from slice first_slice
 *   on, added to y: for every request and block whose depth d (in slices)
 *   exceeds first_slice, y += scale * (code at d - code at first_slice) . x,
 *   reading only slices first_slice .. d - 1; other blocks leave y as it is.
 *   With y holding the product at a uniform depth first_slice, y becomes the
 *   product at the group's maps ([FoQLens] "FoQZones, the mechanism": the
 *   layer read once, its lifted blocks read deeper after it decides).  The
 *   sum is formed in fp64 from the fp32 y and rounded once.
 *   group        initialised by qam_group_init on the pre-pass route (B >= 2).
 *   first_slice  1 .. 3.
 *   Errors: QAM_ERR_NULL (uninitialised group), QAM_ERR_ARG (another route,
 *   first_slice out of range).  Asynchronous on `s`.
 */
int qam_qmatvec_group_refine(const qam_group* group, int first_slice, hipStream_t s);

/*
 * qam_qmatvec_group_lens -- qam_qmatvec_group with the level maps built in
 *   the same launch: every item's map is computed from the lens rules of
 *   qam_build_level_map ([Lens] "The mechanism" rules 1-6, the same readings
 *   and numerics, hence bit-identical to qam_build_level_map over the item's
 *   coords), written to the item's level_map and used for its product.  Each
 *   wavefront computes the rung of its own block, one lane per lens, before
 *   reading the block's planes: the map costs no launch of its own and the
 *   planes read are those of the map.
 *   group      from qam_group_init with B = 1 (the staged-limb route),
 *              every item's coords bound (group->lens_ready); else
 *              QAM_ERR_ARG, nothing enqueued.
 *   lenses, n_lenses, params, glass   as qam_build_level_map; one map rule
 *              set for every item (the items are blocks of one field).
 *   ladder_bits/n_rungs  must be the product ladder {0, 2, 4, 6, 8}
 *              (QAM_ERR_LADDER otherwise).
 *   Outputs: every item's y, as qam_qmatvec_group with that map, and its
 *   level_map.  Enqueues one kernel and nothing else (safe to capture).
 */
int qam_qmatvec_group_lens(const qam_group* group, const qam_lens* lenses, int n_lenses,
                           const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs,
                           int glass, hipStream_t s);

/* ---------------------------------------------------------------- decode driver */
/*
 * A decode step of a decoder-only model in which every weight read is the
 * mixed-depth product at one uniform depth per step ([PoD] abstract: the
 * 8-bit weights are read with their top 4 bits, and a step whose output looks
 * uncertain is run again at 8 bits; the cost is weight bytes read per token).
 * The step is a chain of 4 n_layers + 1 qam_qmatvec_ep launches and nothing
 * else; per layer, with h the hidden state [hidden]:
 *   qkv = W_qkv rms(h)          QAM_OUT_STORE; rows: q_dim queries, then
 *                               kv_dim keys and kv_dim values
 *   h  += W_o qkv[0 : q_dim]    QAM_OUT_ADD; the query part stands in for the
 *                               attention output (weights are synthetic)
 *   m   = glu(W_gu rms(h))      QAM_OUT_GLU; W_gu rows interleaved per block:
 *                               32 gate rows, then the 32 matching up rows
 *   h  += W_down m              QAM_OUT_ADD
 * and finally logits = W_lm rms(h).  rms(v) = v / sqrt(mean(v^2) + eps).
 */
typedef struct qam_decoder_layer {
    qam_packed qkv;       /* [q_dim + 2 kv_dim][hidden] */
    qam_packed o;         /* [hidden][q_dim]            */
    qam_packed gate_up;   /* [2 ffn][hidden], interleaved per 64-row block */
    qam_packed down;      /* [hidden][ffn]              */
} qam_decoder_layer;

typedef struct qam_decoder_desc {
    int                      n_layers;
    int64_t                  hidden, q_dim, kv_dim, ffn, vocab;   /* multiples of 64 (ffn of 32) */
    const qam_decoder_layer* layers;        /* (host) [n_layers]; descriptors are copied */
    qam_packed               lm_head;       /* [vocab][hidden] */
    double                   eps;           /* RMS epsilon, >= 0 */
    int                      target_waves;  /* launch width goal per matrix (workgroups); 0 = 16 */
    int                      waves_per_block; /* 1, 2, 4 or 8 wavefronts split each block's chunk
                                               of columns inside a workgroup, for every
                                               product; 0 = per product: 8 for o, 1 for the
                                               head, 4 for the others */
    int                      max_chunk_tiles; /* longest column chunk of every product, in
                                               64-column tiles; 0 = per product: 32 for o,
                                               16 for the others */
} qam_decoder_desc;

typedef struct qam_decoder qam_decoder;     /* opaque host object */

/* Device bytes qam_decoder_create needs (0 if the description is invalid). */
size_t qam_decoder_bytes(const qam_decoder_desc* d);

/*
 * qam_decoder_create -- validate the shapes, lay out the step's buffers in
 *   dev_mem (caller-owned, qam_decoder_bytes bytes, 256-byte aligned, kept
 *   alive while the decoder lives): split-K workspace, h, qkv, m, logits and
 *   one uniform level map per rung.  Fills the maps and zeroes the counters
 *   on `s`, then synchronises `s`.  The packed weights must stay alive.
 */
int qam_decoder_create(const qam_decoder_desc* d, void* dev_mem, size_t dev_bytes,
                       qam_decoder** out, hipStream_t s);

/* (device) the step's buffers: QAM_DEC_H h [hidden] (the step reads its
 * input here and leaves the final h), QAM_DEC_QKV [q_dim + 2 kv_dim],
 * QAM_DEC_M [ffn], QAM_DEC_LOGITS [vocab]; NULL for an unknown id. */
#define QAM_DEC_H      0
#define QAM_DEC_QKV    1
#define QAM_DEC_M      2
#define QAM_DEC_LOGITS 3
float* qam_decoder_buffer(qam_decoder* dec, int which);

/* qam_decoder_step -- enqueue one step with every block read at `rung`
 *   (0..4 of {0,2,4,6,8}; 2 = D4, 4 = D8).  Kernels only: capturable. */
int qam_decoder_step(qam_decoder* dec, int rung, hipStream_t s);

/* qam_decoder_run -- enqueue products first .. first+count-1 of the step's
 *   chain (4 per layer in the order qkv, o, gate_up, down, then the head),
 *   exactly as qam_decoder_step launches them; for inspecting one product's
 *   inputs and outputs. */
int qam_decoder_run(qam_decoder* dec, int rung, int first, int count, hipStream_t s);

/* qam_decoder_capture -- capture qam_decoder_step(dec, rung) on `s` (not the
 *   null stream) as a HIP graph kept by the decoder (replaces any earlier
 *   graph of that rung); qam_decoder_replay launches it on any stream. */
int qam_decoder_capture(qam_decoder* dec, int rung, hipStream_t s);
int qam_decoder_replay(qam_decoder* dec, int rung, hipStream_t s);

/* Frees the host object and its graphs (not dev_mem). */
void qam_decoder_destroy(qam_decoder* dec);

/* qam_decoder_decode_gated is declared after qam_gate below. */

/*
 * qam_escalation_schedule -- which of T decode steps are run again at 8 bits
 *   ([PoD] abstract: escalate the uncertain steps).  Exactly
 *   floor(rate * T + 0.5) steps are marked: those with the largest score,
 *   ties going to the earlier step.  Host only.
 *   scores        (host) fp64 [T], finite.
 *   rate          in [0, 1].
 *   escalate_out  (host) uint8 [T]: 1 = re-run at 8 bits.
 *   n_out         (host, may be NULL) the number marked.
 */
int qam_escalation_schedule(const double* scores, int64_t T, double rate, uint8_t* escalate_out,
                            int64_t* n_out);

/*
 * qam_gate -- the escalation gate on the device ([PoD] abstract: a step is
 *   redone at 8 bits when the low-precision output distribution looks
 *   uncertain, entropy above a threshold or a small top-two margin).  Over
 *   the V logits z of the low pass, in fp64: p = softmax(z); entropy
 *   H = -sum p ln p in nats (0 ln 0 = 0: a -inf logit is a token of
 *   probability 0); margin = p_(1) - p_(2), the two largest probabilities
 *   (ties to the lower index).  escalate = H > tau_entropy or
 *   margin < tau_margin (+inf / -inf switch a test off).  Logits holding a
 *   NaN or +inf, or all -inf, give no distribution: H, margin, p1 and p2
 *   are NaN and escalate = 1.  One launch; the partials of its workgroups
 *   are merged in a fixed order, so the result is the same bits on every
 *   call (within ~1e-12 of the same formulas evaluated in fp64 on a CPU).
 *   logits     (device) fp32 [V], 2 <= V <= 2^31 - 2.
 *   out        (device) one qam_uncertainty, written by the launch.
 *   workspace  (device) qam_gate_workspace_bytes(V) bytes, 256-byte aligned,
 *              zero-filled before its first use; every call leaves its
 *              counter at zero again.  Calls sharing a workspace must be
 *              ordered.
 */
typedef struct qam_uncertainty {
    double  entropy;     /* nats                                       */
    double  margin;      /* p1 - p2                                    */
    double  p1, p2;      /* the two largest probabilities              */
    int64_t top1, top2;  /* their token indices                        */
    int32_t escalate;    /* 1: redo the step at the high depth         */
    int32_t reserved;
} qam_uncertainty;

size_t qam_gate_workspace_bytes(int64_t V);
int qam_gate(const float* logits, int64_t V, double tau_entropy, double tau_margin,
             qam_uncertainty* out, void* workspace, size_t workspace_bytes, hipStream_t s);

/*
 * qam_decoder_decode_gated -- T decode steps with the escalation gate decided
 *   on the device ([PoD] abstract: decode with the top bits, redo the step at
 *   8 bits when the gate fires).  Per step t: h <- inputs[t], replay the
 *   rung_low graph, qam_gate over the logits, read its result into
 *   host_result (one synchronisation of `s`), and if it fired h <- inputs[t]
 *   again and replay the rung_high graph.  Both rungs must have been
 *   captured (qam_decoder_capture).
 *   inputs         (device) fp32 [T][hidden].
 *   gate_workspace (device) qam_gate_workspace_bytes(vocab) bytes, as for
 *                  qam_gate; gate_out (device) one qam_uncertainty.
 *   host_result    (host, pinned memory for speed) one qam_uncertainty.
 *   escalated_out  (host) uint8 [T]: 1 where the step was redone.
 *   Host-synchronous; not for graph capture.  Outputs of the last step stay
 *   in the decoder's buffers.
 *   Errors: QAM_ERR_NULL, QAM_ERR_ARG (T < 0, a rung not captured),
 *   QAM_ERR_ALIGN, QAM_ERR_WORKSPACE, and whatever qam_gate returns; on an
 *   error part way, the steps before it have run and escalated_out holds
 *   their flags.
 */
int qam_decoder_decode_gated(qam_decoder* dec, const float* inputs, int64_t T, int rung_low, int rung_high,
                             double tau_entropy, double tau_margin, void* gate_workspace,
                             size_t gate_workspace_bytes, qam_uncertainty* gate_out,
                             qam_uncertainty* host_result, uint8_t* escalated_out, hipStream_t s);

/*
 * qam_decoder_decode_gated_async -- the same T gated steps with the decision
 *   left on the device: no host synchronisation per step (HIP graphs have no
 *   conditional nodes here, so the branch is a predicate).  Per step t:
 *   h <- inputs[t]; replay the rung_low graph; qam_gate into gate_out;
 *   escalated_dev[t] = gate_out->escalate; h <- inputs[t] again if it fired
 *   (a predicated copy kernel); then a graph of the rung_high step whose
 *   every product kernel reads gate_out->escalate first and exits at once
 *   when it is 0.  That graph is captured on `s` on the first call (and again
 *   when gate_out changes), so `s` must not be the null stream and the call
 *   must not itself be captured.  Everything is enqueued on `s`; the call
 *   returns without waiting.  rung_low must have been captured.
 *   escalated_dev  (device) uint8 [T].
 *   Each step pays the rung_high graph's launches whether or not it fired.
 */
int qam_decoder_decode_gated_async(qam_decoder* dec, const float* inputs, int64_t T, int rung_low, int rung_high,
                                   double tau_entropy, double tau_margin, void* gate_workspace,
                                   size_t gate_workspace_bytes, qam_uncertainty* gate_out, uint8_t* escalated_dev,
                                   hipStream_t s);

/* ---------------------------------------------------------------- draft and verify */
/*
 * Verified speculation ([PoD] abstract: speculation verified at full depth
 * reaches the full-depth output at a similar weight-byte cost).  Reading
 * taken: greedy decoding; the draft model is the stored stack read at the
 * draft rung (D4), the target the same stack read at the verify rung (D8).
 * A round drafts k tokens one step at a time at the draft rung, then runs
 * ONE batched step at the verify rung over the k + 1 inputs (the current
 * token and the k drafts), so the verify pass reads every weight block once
 * for all k + 1 positions.  With t_i the target's token after input i and
 * d_i the i-th draft, the round keeps d_1 .. d_j for the longest prefix with
 * t_{i-1} = d_i, then emits t_j: every emitted token is the target's greedy
 * token, whatever the draft.
 *
 * The decode step here has no attention: a step's output depends on its
 * input alone.  The token-feedback stand-in feeds back the embedding row of
 * the emitted token (a caller table E [vocab][hidden] fp32) as the next
 * step's input.
 *
 * A verifier holds the batched step's buffers over a decoder's weights.
 * Its step is the decoder's chain for B requests at once:
 *   h_r = x_r;  x'_r = rms(h_r)
 *   per layer: qkv = W_qkv x';  x' = qkv[:, :q_dim];  h += W_o x';
 *              x' = rms(h);  u = W_gate_up x';  m = silu(u_gate) * u_up;
 *              h += W_down m;  x' = rms(h)
 *   logits = W_lm x'
 * each product a qam_qmatvec product at B (the pre-pass route for B >= 2,
 * every request's result independent of the others and of its slot): rms in
 * fp64 over the row (x' = fl32(h / sqrt(mean h^2 + eps))), h + y rounded
 * once to fp32, silu(g) u in fp64 rounded once.  For B >= 2 the elementwise
 * steps run inside the pre-pass of the product that consumes them (the
 * residual add and norm, the q columns read in place, the gated product),
 * so a layer is four products of two launches each; for B = 1 each is one
 * small row kernel before its product.
 */
typedef struct qam_verifier qam_verifier;   /* opaque host object */

/* Device bytes of a verifier for batches up to max_batch (1 .. 16). */
size_t qam_verifier_bytes(const qam_decoder_desc* d, int max_batch);

/* qam_verifier_create -- lay out the batched buffers in dev_mem (caller-owned,
 *   256-byte aligned, kept alive with the verifier), zero the workspace
 *   counters on `s` and synchronise.  The decoder must outlive it. */
int qam_verifier_create(qam_decoder* dec, int max_batch, void* dev_mem, size_t dev_bytes, qam_verifier** out,
                        hipStream_t s);

/* (device) the verifier's buffers, row-major with B rows in use:
 *   QAM_VER_X [max_batch][hidden] inputs (read by op 0), QAM_VER_H [..][hidden],
 *   QAM_VER_QKV [..][q_dim + 2 kv_dim], QAM_VER_M [..][ffn],
 *   QAM_VER_XN [..][hidden] the last rms output,
 *   QAM_VER_LOGITS [..][vocab],
 *   QAM_VER_Y [..][max(hidden, 2 ffn)] the o, gate|up and down products'
 *   output (rows packed with the product's row count as stride);
 *   NULL for an unknown id. */
#define QAM_VER_X      0
#define QAM_VER_H      1
#define QAM_VER_QKV    2
#define QAM_VER_M      3
#define QAM_VER_XN     4
#define QAM_VER_LOGITS 5
#define QAM_VER_Y      6
float* qam_verifier_buffer(qam_verifier* v, int which);

/* qam_verifier_run -- enqueue ops first .. first+count-1 of the batched
 *   chain for B requests (1 <= B <= max_batch) at `rung`: 4 n_layers + 2
 *   ops, each forming its product's input from the previous op's output:
 *     op 0         h = x; x' = rms h
 *     op 1 + 4l    (l > 0: h += y; x' = rms h) qkv = W_qkv x'
 *     op 2 + 4l    y = W_o qkv[:, :q_dim]
 *     op 3 + 4l    h += y; x' = rms h; y = W_gate_up x'
 *     op 4 + 4l    m = silu(y_gate) y_up; y = W_down m
 *     last         h += y; x' = rms h; logits = W_lm x'
 *   qam_verifier_step runs them all. */
int qam_verifier_run(qam_verifier* v, int rung, int B, int first, int count, hipStream_t s);
int qam_verifier_step(qam_verifier* v, int rung, int B, hipStream_t s);

/* qam_verifier_capture -- capture qam_verifier_step(v, rung, B) on `s` (not
 *   the null stream) as a HIP graph kept by the verifier, one per (rung, B);
 *   qam_verifier_replay launches it, and qam_decoder_speculate replays the
 *   graph of (verify_rung, k + 1) when there is one. */
int qam_verifier_capture(qam_verifier* v, int rung, int B, hipStream_t s);
int qam_verifier_replay(qam_verifier* v, int rung, int B, hipStream_t s);

/* Frees the host object and its graphs (not dev_mem). */
void qam_verifier_destroy(qam_verifier* v);

/*
 * qam_argmax_rows -- idx[r] = the first index of the largest of
 *   v[r*ld .. r*ld + n-1] (fp32 order; -0 < +0 as bit patterns; rows must
 *   hold no NaN), for r < rows.
 *   v        (device) fp32, ld >= n >= 1, 1 <= rows <= 65535, n < 2^31.
 *   idx_out  (device) int32 [rows].
 *   workspace (device) 8 * rows bytes, 8-byte aligned, zero before the
 *            first use; left zero.  Two launches.
 */
int qam_argmax_rows(const float* v, int64_t rows, int64_t n, int64_t ld, int32_t* idx_out, void* workspace,
                    hipStream_t s);

typedef struct qam_spec_stats {
    int64_t rounds;         /* verify passes                                  */
    int64_t draft_steps;    /* steps at the draft rung (k per round)          */
    int64_t drafted;        /* tokens drafted (= draft_steps)                 */
    int64_t accepted;       /* drafts kept                                    */
    int64_t emitted;        /* tokens emitted (>= n_tokens; the last round's  */
                            /* surplus is dropped from tokens_out)            */
} qam_spec_stats;

/*
 * qam_decoder_speculate -- n_tokens greedy tokens after first_token by
 *   draft-and-verify (above), k drafts per round (1 .. max_batch - 1).
 *   embed       (device) fp32 [vocab][hidden], the feedback table.
 *   draft_rung, verify_rung  rungs 0..4 of {0,2,4,6,8}; the draft steps
 *               replay the decoder's graph of draft_rung when captured.
 *   tokens_out  (host) int32 [n_tokens].
 *   stats       (host, may be NULL).
 *   Per round: k draft steps, each one graph replay, a device argmax and an
 *   embedding-row copy chosen on the device; one batched verify step (a
 *   graph replay when captured); a
 *   device argmax of its k + 1 rows; one kernel that accepts and feeds the
 *   next input; then a read of the round's tokens (one synchronisation of
 *   `s`).  The decoder's own buffers hold the last draft step.
 */
int qam_decoder_speculate(qam_decoder* dec, qam_verifier* v, const float* embed, int32_t first_token,
                          int n_tokens, int k, int draft_rung, int verify_rung, int32_t* tokens_out,
                          qam_spec_stats* stats, hipStream_t s);

/* ---------------------------------------------------------------- diagnostics */

/*
 * Timeline of the batch-1 product (a tracing aid for short, latency-bound
 * launches such as a decode step's).  Only the library built with
 * QAM_TIMELINE (python -m query_adaptive_mixed_amd.build --timeline, giving
 * libqam_timeline.so) records anything; in the product library both calls
 * return QAM_ERR_ARG.
 *
 * qam_timeline_select -- choose up to QAM_TIMELINE_SLOTS matrices by their
 *   planes pointer (slot i: planes[i]) and clear the stamps (synchronous).
 *   Every later single-matrix launch of the batch-1 kernel on a chosen
 *   matrix writes, for each of its first QAM_TIMELINE_GROUPS workgroups and
 *   each wave, the 100 MHz wall clock (wall_clock64) at QAM_TIMELINE_POINTS
 *   points: 0 kernel entry, 1 start of the wave's work, 2 first x sub-chunk
 *   staged, 3 last tile multiplied, 4 row sums formed, 5 the block's waves'
 *   sums combined, 6 split-K arrival counted, 7 wave exit (0 where a wave
 *   never reaches a point).  A later launch on the same matrix overwrites.
 *   n in [0, QAM_TIMELINE_SLOTS]; planes may be NULL when n = 0.
 * qam_timeline_read -- copy the stamps, uint64
 *   [QAM_TIMELINE_SLOTS][QAM_TIMELINE_GROUPS][8 waves][QAM_TIMELINE_POINTS],
 *   to host memory `out` (synchronous); n_words must be at least that count.
 */
#define QAM_TIMELINE_SLOTS  8
#define QAM_TIMELINE_GROUPS 512
#define QAM_TIMELINE_POINTS 8
int qam_timeline_select(const void* const* planes, int n);
int qam_timeline_read(uint64_t* out, size_t n_words);

const char* qam_last_error(void);     /* thread-local, "" if none           */
const char* qam_last_variant(void);   /* kernel variant of the last call     */
const char* qam_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QAM_H */
