// Batched mixed-depth product on the matrix cores: 2 to 32 requests, with
// one level map shared by all of them or one map per request.
//
// [FoQLens] "Progress": every 64-row block is read at its own depth from the
// one stored copy inside the pass (the pages' batched decode reads 32
// requests per step).  With a map per request, block b is read once, to the
// deepest slice any request needs, and every request gets the block's codes
// at its own depth: the residual slices make the code at depth d the sum of
// the first d/2 slices, so the codes for each depth present in the batch are
// built incrementally from the same loaded words and multiplied by the limbs
// of the requests at that depth.
//
// Arithmetic (exact, as in the batch-1 kernel; qmatvec_internal.h): a
// pre-pass turns each request's x, per column chunk, into int8 limbs laid out
// as B operands of v_mfma_i32_16x16x64_i8, 16 columns per MFMA, and lists the
// chunk's uncovered elements (relative error above 2^-15) with their exact
// residuals.  A (chunk, request) is "coarse" when the coarse split (the hi
// part's three limbs and one lo digit, 32 bits of fixed point) leaves at most
// kCoarseListMax elements uncovered, else "fine" (the hi part and the full
// 24-bit lo part, 48 bits).  A set of SS requests has NCGC coarse column
// groups (column 4 rr + l: hi limbs 0..2, then the lo digit of weight 2^16,
// which is the coarse digit or the fine part's top digit) and NCGF fine ones
// (column 2 rr + l: the fine part's low digits 0 and 1, zero for a coarse
// request); sets of one or two requests keep both blocks in one group (the
// fine block from column 4 SS).  Sets of more than four requests multiply
// their coarse groups first and their fine groups in a second pass only when
// a request of the set is fine for the chunk: 4 columns per request instead
// of 6 in the common case.  Sets of up to four always take the fine split (the
// coarse one would save them at most one group).  Codes are the A
// operands (16 rows x 64 columns, exactly the words a lane loads); i32
// accumulation is exact; a request's columns are combined in fp64 after the
// chunk, through an LDS table of the block's 64 x 16 NCG integer sums, and the
// listed residuals are added with their codes in fp64.
//
// A workgroup is one (block, column chunk): wave (ks, h) serves request set h
// on the chunk's tiles ks, ks + KS, ...; the KS waves of a set add their sums
// into the set's table with LDS integer adds (exact in any order).  One row
// per lane then forms the outputs, so y is written coalesced.

#include <algorithm>
#include <vector>

#include "qmatvec_internal.h"

namespace qam {

typedef __attribute__((address_space(1))) const v4i global_v4i;

constexpr int kBadExp = 0x7FFFFFFF;   // exponent marker of a chunk of x with a non-finite value
constexpr int kMaxNCG = 6;            // 16 requests: 4 coarse + 2 fine column groups
constexpr int kCoarseCols = 4;        // coarse B-operand columns per request
constexpr int kFineCols = 2;          // fine B-operand columns per request
constexpr int kCoarseListMax = 4;     // most coarse-uncovered elements a coarse (chunk, request) lists
constexpr int kFineFlag = 1 << 30;    // unc_count bit: the (chunk, request) is fine

// Column groups of a set of SS requests: coarse, fine, both.  Sets of one or
// two requests keep all six columns of a request in one group (the coarse
// block, then the fine block at column 4 SS): there is no MFMA to save.
__host__ __device__ constexpr int ncgc_of_ss(int ss) { return (kCoarseCols * ss + 15) / 16; }
__host__ __device__ constexpr int ncgf_of_ss(int ss) { return (kFineCols * ss + 15) / 16; }
__host__ __device__ constexpr int ncg_of_ss(int ss) {
    return (kCoarseCols + kFineCols) * ss <= 16 ? 1 : ncgc_of_ss(ss) + ncgf_of_ss(ss);
}
// The coarse groups of a total of NCG (every set size gives a distinct total:
// 1-2 requests 1 (shared), 3-4 1 + 1, 5-8 2 + 1, 9-12 3 + 2, 13-16 4 + 2).
__host__ __device__ constexpr int ncgc_of_ncg(int ncg) {
    return ncg <= 2 ? 1 : ncg == 3 ? 2 : ncg == 5 ? 3 : 4;
}
// First column of the fine block in a set's columns.
__host__ __device__ constexpr int fine_base(int ncg, int ss) { return ncg == 1 ? kCoarseCols * ss : 16 * ncgc_of_ncg(ncg); }

struct MItem {
    const uint8_t* planes;
    const float* scales;
    const void* x;             // [B][K]
    float* y;                  // [B][N]
    const uint8_t* level;      // [B][n_blocks] (per request) or [n_blocks]
    int64_t level_stride;      // n_blocks (per request) or 0
    v4i* limbs;                // [n_tiles][NH][NCG][64] 16-byte B operands
    int* exps;                 // [n_chunks][16 NH]
    int* unc_count;            // [n_chunks][16 NH] uncovered elements listed
    int2* unc;                 // [n_chunks][16 NH][tpc 64] (column in the chunk, residual bits)
    double* partials;          // [n_chunks][B][N] (split K only)
    uint32_t* counters;        // [n_blocks]       (split K only)
    int64_t plane_bytes;
    int64_t N, K;
    int n_blocks, n_tiles, tpc, n_chunks;
    int wg_begin;              // grouped launches: first product workgroup of this item
    int pre_begin;             // grouped launches: first pre-pass workgroup of this item
    // the pre-pass's input transform (XMode; fp32 x; zero: plain x)
    int x_mode;
    int64_t x_ld;
    const float* x_add;
    float* x_res;
    float* x_side;
    double x_eps;
};

struct MCommon {
    const MItem* items;        // grouped launches: the descriptor table
    const int* wg_item;        // grouped launches: item of every product workgroup
    const int* pre_item;       // grouped launches: item of every pre-pass workgroup
    uint32_t* status;          // the call's status word
    int B;
    int NH;                    // request sets per workgroup
    int SS;                    // requests per set (<= 16)
    int KS;                    // waves per request set splitting a chunk's tiles
    int NCG;                   // 16-column groups per request set (coarse, then fine)
    int NCGC;                  // coarse groups among them
    int first;                 // refinement launches: slices below this are not read, and y is added to
};

// Rung of request r in block b (0..4 are depths; above 4 is not a rung of
// the product).
template <bool PER_REQ>
__device__ __forceinline__ int rung_of(const MItem& a, int r, int b) {
    return PER_REQ ? (int)a.level[(int64_t)r * a.level_stride + b] : level_of(a.level, b);
}

// ------------------------------------------------------------------ x -> limbs

// Columns c .. c+3 of request r's input, after the item's transform (for
// kXAddNorm the values before scaling, v = h + add).
template <bool XBF16>
__device__ __forceinline__ float4 input4(const MItem& a, int r, int64_t c) {
    if constexpr (XBF16) return x4_value<true>(load_x4_raw<true>(a.x, (int64_t)r * a.K + c));   // plain only
    const float* xf = static_cast<const float*>(a.x);
    switch (a.x_mode) {
        case kXStrided:
            return *reinterpret_cast<const float4*>(xf + (int64_t)r * a.x_ld + c);
        case kXAddNorm: {
            const float4 h = *reinterpret_cast<const float4*>(xf + (int64_t)r * a.K + c);
            const float4 d = *reinterpret_cast<const float4*>(a.x_add + (int64_t)r * a.K + c);
            return float4{h.x + d.x, h.y + d.y, h.z + d.z, h.w + d.w};
        }
        case kXGated: {
            // x' = silu(g) u of gate|up rows 64 (c / 32) + c % 32 and + 32 (c % 4 == 0: one block)
            const float* row = xf + (int64_t)r * a.x_ld + 64 * (c / 32) + c % 32;
            const float4 g4 = *reinterpret_cast<const float4*>(row);
            const float4 u4 = *reinterpret_cast<const float4*>(row + 32);
            const double g[4] = {g4.x, g4.y, g4.z, g4.w}, u[4] = {u4.x, u4.y, u4.z, u4.w};
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (float)(g[i] / (1.0 + exp(-g[i])) * u[i]);
            return float4{o[0], o[1], o[2], o[3]};
        }
        default:
            return x4_value<XBF16>(load_x4_raw<XBF16>(a.x, (int64_t)r * a.K + c));
    }
}

// One workgroup of sixteen wavefronts per (column chunk, request slot
// r < SS NH): the chunk's largest |x| sets the exponent; slots r >= B get zero
// limbs.  The uncovered elements are listed in column order.  Columns go in
// rounds of kPreRound, each thread holding kPreVec groups of four (thread T:
// columns 4T and 4T + 4 kPreThreads of the round); the first round's values
// stay in registers from the maximum to the split.
constexpr int kPreThreads = 1024;
constexpr int kPreVec = 2;
constexpr int kPreRound = 4 * kPreThreads * kPreVec;
static_assert(kPreVec == 2 && 4 * kPreThreads < 65536, "two 16-bit count fields per thread");

template <bool XBF16, bool GROUPED>
__global__ __launch_bounds__(kPreThreads) void limbs_kernel(MItem single, MCommon c) {
    __shared__ float red_m[kPreThreads / 64];
    __shared__ float red_p[kPreThreads / 64];
    __shared__ double red_s[kPreThreads / 64];
    __shared__ int wave_n[kPreThreads / 64];
    __shared__ int clist_n;                    // coarse chunks: elements listed so far ...
    __shared__ int2 clist[kCoarseListMax];     // ... and the list, in no order until sorted
    MItem a;
    int local;
    if constexpr (GROUPED) {
        a = c.items[c.pre_item[blockIdx.x]];
        local = (int)blockIdx.x - a.pre_begin;
    } else {
        a = single;
        local = (int)blockIdx.x;
    }
    const int B = c.B, NH = c.NH, NCG = c.NCG, SS = c.SS;
    const int slots = SS * NH;
    const int chunk = local / slots;
    const int r = local % slots;
    const int T = threadIdx.x;
    const int lane = T & 63, wave = T >> 6;
    const int t0 = chunk * a.tpc;
    const int ncol = min(a.tpc, a.n_tiles - t0) * 64;
    const int64_t col0 = (int64_t)t0 * 64;
    const bool live = r < B;
    const int mode = a.x_mode;
    const bool norm = mode == kXAddNorm;
    float m = 0.0f;
    float poison = 0.0f;   // 0 * x summed: NaN exactly when some x is not finite
    double ssq = 0.0;      // norm transforms: sum of v^2 over the row
    float4 keep[kPreVec];
#pragma unroll
    for (int j = 0; j < kPreVec; ++j) keep[j] = float4{0.0f, 0.0f, 0.0f, 0.0f};
    if (live)
        for (int base = 0; base < ncol; base += kPreRound)
#pragma unroll
            for (int j = 0; j < kPreVec; ++j) {
                const int k = base + 4 * T + 4 * kPreThreads * j;
                if (k < ncol) {
                    const float4 v = input4<XBF16>(a, r, col0 + k);
                    if (base == 0) keep[j] = v;
                    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
                    poison = __builtin_fmaf(v.x, 0.0f, poison);
                    poison = __builtin_fmaf(v.y, 0.0f, poison);
                    poison = __builtin_fmaf(v.z, 0.0f, poison);
                    poison = __builtin_fmaf(v.w, 0.0f, poison);
                    if (norm)
                        ssq += (double)v.x * (double)v.x + (double)v.y * (double)v.y + (double)v.z * (double)v.z +
                               (double)v.w * (double)v.w;
                }
            }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        m = fmaxf(m, __shfl_xor(m, o));
        poison += __shfl_xor(poison, o);
        if (norm) ssq += __shfl_xor(ssq, o);
    }
    if (lane == 0) {
        red_m[wave] = m;
        red_p[wave] = poison;
        red_s[wave] = ssq;
    }
    __syncthreads();
    m = red_m[0];
    poison = red_p[0];
    ssq = red_s[0];
#pragma unroll
    for (int w = 1; w < kPreThreads / 64; ++w) {
        m = fmaxf(m, red_m[w]);
        poison += red_p[w];
        ssq += red_s[w];
    }
    // kXAddNorm: every value is scaled by inv (a positive factor, so the
    // largest |x'| is the largest |v| scaled and rounded alike)
    double inv = 1.0;
    if (norm) {
        inv = 1.0 / sqrt(ssq / (double)a.K + a.x_eps);
        m = (float)((double)m * inv);
    }
    const bool nonfinite = poison != 0.0f || (norm && !(inv <= 1.7976931348623157e308));   // NaN compares unequal
    int e = 0;
    if (m > 0.0f) frexpf(m, &e);
    const XSplit sp = xsplit_of(e);
    // Coarse or fine: count the elements the coarse split leaves uncovered
    // (the first round's values are still in registers).  Sets of up to four
    // requests (one or two column groups) always take the fine split: the
    // coarse one would save them at most one group of MFMAs, less than the
    // count costs these small launches.
    const bool one_group = NCG <= 2;
    int ccount = 0;
    if (live && !nonfinite && !one_group)
        for (int base = 0; base < ncol; base += kPreRound)
#pragma unroll
            for (int j = 0; j < kPreVec; ++j) {
                const int k = base + 4 * T + 4 * kPreThreads * j;
                if (k < ncol) {
                    float4 v = base == 0 ? keep[j] : input4<XBF16>(a, r, col0 + k);
                    if (norm)
                        v = float4{(float)((double)v.x * inv), (float)((double)v.y * inv),
                                   (float)((double)v.z * inv), (float)((double)v.w * inv)};
                    ccount += (int)coarse_uncovered(v.x, sp) + (int)coarse_uncovered(v.y, sp) +
                              (int)coarse_uncovered(v.z, sp) + (int)coarse_uncovered(v.w, sp);
                }
            }
    if (!one_group) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ccount += __shfl_xor(ccount, o);
        if (lane == 0) wave_n[wave] = ccount;
        if (T == 0) clist_n = 0;
        __syncthreads();
        ccount = 0;
#pragma unroll
        for (int w = 0; w < kPreThreads / 64; ++w) ccount += wave_n[w];
        __syncthreads();   // wave_n is written again by the listing
    }
    const bool fine = one_group || ccount > kCoarseListMax;
    const int h = r / SS, rr = r % SS;
    const int FB = fine_base(NCG, SS);
    uint8_t* lb = reinterpret_cast<uint8_t*>(a.limbs);
    int2* list = a.unc + (int64_t)(chunk * slots + r) * a.tpc * 64;
    int listed = 0;
    for (int base = 0; base < ncol; base += kPreRound) {
        float r2[kPreVec][4];
        bool u[kPreVec][4];
        int packed = 0;   // uncovered counts of this thread's groups, 16 bits each
#pragma unroll
        for (int j = 0; j < kPreVec; ++j) {
            const int k = base + 4 * T + 4 * kPreThreads * j;
            const bool in = k < ncol;
            uint32_t wh[4] = {0, 0, 0, 0}, wl[4] = {0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                r2[j][q] = 0.0f;
                u[j][q] = false;
            }
            float4 v = float4{0.0f, 0.0f, 0.0f, 0.0f};
            if (in && live) {
                v = base == 0 ? keep[j] : input4<XBF16>(a, r, col0 + k);
                const int64_t o = (int64_t)r * a.K + col0 + k;
                if (norm) {   // the residual row, then the normalised input (each element is read
                              // before it is written, by the same thread: res may be x)
                    *reinterpret_cast<float4*>(a.x_res + o) = v;
                    v = float4{(float)((double)v.x * inv), (float)((double)v.y * inv), (float)((double)v.z * inv),
                               (float)((double)v.w * inv)};
                }
                if (mode == kXAddNorm || mode == kXGated) *reinterpret_cast<float4*>(a.x_side + o) = v;
            }
            if (in && live && !nonfinite) {
                if (fine) {
                    split_elem(v.x, sp, wh[0], wl[0], r2[j][0], u[j][0]);
                    split_elem(v.y, sp, wh[1], wl[1], r2[j][1], u[j][1]);
                    split_elem(v.z, sp, wh[2], wl[2], r2[j][2], u[j][2]);
                    split_elem(v.w, sp, wh[3], wl[3], r2[j][3], u[j][3]);
                } else {
                    split_coarse(v.x, sp, wh[0], wl[0], r2[j][0], u[j][0]);
                    split_coarse(v.y, sp, wh[1], wl[1], r2[j][1], u[j][1]);
                    split_coarse(v.z, sp, wh[2], wl[2], r2[j][2], u[j][2]);
                    split_coarse(v.w, sp, wh[3], wl[3], r2[j][3], u[j][3]);
                }
            }
            if (in) {
                const int64_t kk = col0 + k;   // columns kk .. kk+3: one tile, one 16-column slice
                const int64_t t = kk >> 6;
                const int kg = (int)((kk & 63) >> 4);
                const int byte = (int)(kk & 15);
                // digits: hi 0..2 and lo 2 to coarse columns 4 rr + 0..3, lo 0..1 to fine
                // columns FB + 2 rr + 0..1
#pragma unroll
                for (int l = 0; l < kCoarseCols + kFineCols; ++l) {
                    const uint32_t* w = l < 3 ? wh : wl;
                    const int sh = l < 3 ? 8 * l : l == 3 ? 16 : 8 * (l - 4);
                    const int col = l < kCoarseCols ? kCoarseCols * rr + l : FB + kFineCols * rr + (l - kCoarseCols);
                    const uint32_t word = ((w[0] >> sh) & 0xFFu) | (((w[1] >> sh) & 0xFFu) << 8) |
                                          (((w[2] >> sh) & 0xFFu) << 16) | (((w[3] >> sh) & 0xFFu) << 24);
                    const int64_t unit = ((t * NH + h) * NCG + (col >> 4)) * 64 + kg * 16 + (col & 15);
                    *reinterpret_cast<uint32_t*>(lb + unit * 16 + byte) = word;
                }
            }
            packed |= ((int)u[j][0] + (int)u[j][1] + (int)u[j][2] + (int)u[j][3]) << (16 * j);
        }
        // uncovered elements of this round, appended in column order: the
        // first groups of all threads, then the second ones (16-bit fields:
        // a round holds at most 4 kPreThreads of each)
        if (!fine) {
            // a coarse chunk lists at most kCoarseListMax elements (counted
            // above): each takes a slot, and the list is sorted at the end
#pragma unroll
            for (int j = 0; j < kPreVec; ++j) {
                const int k = base + 4 * T + 4 * kPreThreads * j;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (u[j][q]) {
                        const int pos = atomicAdd(&clist_n, 1);   // < kCoarseListMax: the count above saw these
                        if (pos < kCoarseListMax) clist[pos] = int2{k + q, __float_as_int(r2[j][q])};
                    }
            }
        } else if (__syncthreads_or(packed)) {
            int incl = packed;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o);
                if (lane >= o) incl += v;
            }
            if (lane == 63) wave_n[wave] = incl;
            __syncthreads();
            int before = 0, total = 0;
#pragma unroll
            for (int w = 0; w < kPreThreads / 64; ++w) {
                const int n = wave_n[w];
                if (w < wave) before += n;
                total += n;
            }
            const int excl = before + incl - packed;
            const int total0 = total & 0xFFFF;
#pragma unroll
            for (int j = 0; j < kPreVec; ++j) {
                int pos = listed + (j == 0 ? (excl & 0xFFFF) : total0 + ((excl >> 16) & 0xFFFF));
                const int k = base + 4 * T + 4 * kPreThreads * j;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (u[j][q]) list[pos++] = int2{k + q, __float_as_int(r2[j][q])};
            }
            listed += total0 + ((total >> 16) & 0xFFFF);
            __syncthreads();   // wave_n is read before the next round writes it
        }
    }
    if (!fine) {   // the coarse list in column order, as the scan would have placed it
        __syncthreads();
        if (T == 0) {
            listed = min(clist_n, kCoarseListMax);
            for (int i = 1; i < listed; ++i)
                for (int m = i; m > 0 && clist[m - 1].x > clist[m].x; --m) {
                    const int2 t = clist[m - 1];
                    clist[m - 1] = clist[m];
                    clist[m] = t;
                }
            for (int i = 0; i < listed; ++i) list[i] = clist[i];
        }
    }
    if (T == 0) {
        a.exps[chunk * slots + r] = nonfinite ? kBadExp : e;
        a.unc_count[chunk * slots + r] = live && !nonfinite ? (listed | (fine ? kFineFlag : 0)) : 0;
    }
}

// ------------------------------------------------------------------ product

// Tiles in flight: two halves of H tiles, each tile NS weight loads and NG
// limb loads per lane (NG: the column groups multiplied, coarse or all).
template <int NS, int NG>
struct MRing {
    static constexpr int H = NS + NG <= 4 ? 2 : 1;
    static constexpr int PF = 2 * H;
};

template <int NS, int NG, int H>
__device__ __forceinline__ void mload(u32x4 (&w)[H][NS], v4i (&x)[H][NG], const uint8_t* wbase, int64_t pb,
                                      int64_t wstride, const v4i* xbase, int64_t xstride, int tile, int last,
                                      int first) {
#pragma unroll
    for (int u = 0; u < H; ++u) {
        const int t = min(tile + u, last);
#pragma unroll
        for (int p = 0; p < NS; ++p)
            w[u][p] = p < first ? u32x4{0u, 0u, 0u, 0u} : load_plane(wbase + p * pb + (int64_t)t * wstride);
#pragma unroll
        for (int g = 0; g < NG; ++g) x[u][g] = *(global_v4i*)(xbase + t * xstride + g * 64);
    }
}

// One tile: for each depth d present among the set's requests, the codes at
// depth d times the limbs of the requests reading d (mcol[g]: depth of the
// request owning this lane's column in group g; gmask[g]: the depths present
// in group g, so a group with no request at d costs no MFMA there); with a
// shared map, the codes at the block's depth NS times every limb.  The first
// NG column groups are multiplied (the coarse ones, or all).
template <int NS, int NCG, int G0, int NG, bool PER_REQ>
__device__ __forceinline__ void mtile(const u32x4 (&w)[NS], const v4i (&xl)[NG], const int (&mcol)[NCG],
                                      const uint32_t (&gmask)[NCG], uint32_t dmask, v4i (&acc)[4][NCG]) {
    uint32_t q[4][4];   // [j][u]: masked slice bits so far, unrotated
#pragma unroll
    for (int p = 0; p < NS; ++p) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t mk = slice_mask(3 - p, u);
            if (p == 0) {
                q[0][u] = w[0].x & mk;
                q[1][u] = w[0].y & mk;
                q[2][u] = w[0].z & mk;
                q[3][u] = w[0].w & mk;
            } else {
                q[0][u] |= w[p].x & mk;
                q[1][u] |= w[p].y & mk;
                q[2][u] |= w[p].z & mk;
                q[3][u] |= w[p].w & mk;
            }
        }
        const bool use = PER_REQ ? ((dmask >> (p + 1)) & 1u) != 0 : p == NS - 1;
        if (use) {
            v4i A[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                A[j] = v4i{(int)q[j][0], (int)rotl32(q[j][1], 2), (int)rotl32(q[j][2], 4), (int)rotl32(q[j][3], 6)};
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                if (PER_REQ && ((gmask[G0 + g] >> (p + 1)) & 1u) == 0) continue;
                v4i bm;
                if constexpr (PER_REQ) {
                    const bool mine = mcol[G0 + g] == p + 1;
                    bm = v4i{mine ? xl[g].x : 0, mine ? xl[g].y : 0, mine ? xl[g].z : 0, mine ? xl[g].w : 0};
                } else {
                    bm = xl[g];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[j][G0 + g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[j], bm, acc[j][G0 + g], 0, 0, 0);
            }
        }
    }
}

// The product over this wave's tiles of the chunk: tiles ks, ks + KS, ...,
// multiplying column groups G0 .. G0 + NG - 1.
template <int NS, int NCG, int G0, int NG, bool PER_REQ>
__device__ __forceinline__ void mproduct(const MItem& a, int NH, int KS, int b, int chunk, int h, int ks, int L,
                                         const int (&mcol)[NCG], const uint32_t (&gmask)[NCG], uint32_t dmask,
                                         int first, v4i (&acc)[4][NCG]) {
    constexpr int H = MRing<NS, NG>::H;
    constexpr int PF = MRing<NS, NG>::PF;
    const int t0 = chunk * a.tpc + ks;
    const int nt_all = min(a.tpc, a.n_tiles - chunk * a.tpc);
    const int nt = nt_all > ks ? (nt_all - ks + KS - 1) / KS : 0;
    if (nt == 0) return;
    const int last = nt - 1;
    const uint8_t* wbase = a.planes + (int64_t)b * 16 * a.K + (int64_t)t0 * kTileBytes + L * 16;
    const int64_t wstride = (int64_t)KS * kTileBytes;
    const int64_t xunit = (int64_t)NH * NCG * 64;        // v4i units per tile
    const v4i* xbase = a.limbs + (int64_t)t0 * xunit + ((int64_t)h * NCG + G0) * 64 + L;
    const int64_t xstride = xunit * KS;
    const int64_t pb = a.plane_bytes;

    __builtin_amdgcn_s_waitcnt(0);
    u32x4 wa[H][NS], wb[H][NS];
    v4i xa[H][NG], xb[H][NG];
    mload<NS, NG, H>(wa, xa, wbase, pb, wstride, xbase, xstride, 0, last, first);
    __builtin_amdgcn_sched_barrier(0);
    mload<NS, NG, H>(wb, xb, wbase, pb, wstride, xbase, xstride, H, last, first);
    __builtin_amdgcn_sched_barrier(0);
    int t = 0;
    for (; t + PF < nt; t += PF) {
#pragma unroll
        for (int u = 0; u < H; ++u) mtile<NS, NCG, G0, NG, PER_REQ>(wa[u], xa[u], mcol, gmask, dmask, acc);
        __builtin_amdgcn_sched_barrier(0);
        mload<NS, NG, H>(wa, xa, wbase, pb, wstride, xbase, xstride, t + PF, last, first);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < H; ++u) mtile<NS, NCG, G0, NG, PER_REQ>(wb[u], xb[u], mcol, gmask, dmask, acc);
        __builtin_amdgcn_sched_barrier(0);
        mload<NS, NG, H>(wb, xb, wbase, pb, wstride, xbase, xstride, t + PF + H, last, first);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Drain: the last ring, whose tail may run past the wave's tiles.  Tiles
    // past them were loaded (clamped to the last one) but are multiplied by
    // zero limbs, so the accumulators see the same straight-line code as in
    // the loop.
#pragma unroll
    for (int u = 0; u < H; ++u) {
        const bool in = t + u < nt;
        v4i z[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) z[g] = in ? xa[u][g] : v4i{0, 0, 0, 0};
        mtile<NS, NCG, G0, NG, PER_REQ>(wa[u], z, mcol, gmask, dmask, acc);
    }
#pragma unroll
    for (int u = 0; u < H; ++u) {
        const bool in = t + H + u < nt;
        v4i z[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) z[g] = in ? xb[u][g] : v4i{0, 0, 0, 0};
        mtile<NS, NCG, G0, NG, PER_REQ>(wb[u], z, mcol, gmask, dmask, acc);
    }
}

// Request r's exact corrections for the uncovered elements of its chunk, for
// the row of lane `row`: code(row, k) at the request's read (slices
// first .. depth-1) times the listed residual, in fp64.  The list (at most
// kDenseListed entries) comes in with one load, lane i holding entry i, and
// the plane words of four elements are in flight together; the terms are
// still added one by one in list order.
__device__ __forceinline__ double listed_correction(const MItem& a, int b, int chunk, int slot, int n, int row,
                                                    int first, int depth, int e) {
    const int2* list = a.unc + (int64_t)slot * a.tpc * 64;
    const int64_t col0 = (int64_t)chunk * a.tpc * 64;
    const int L = (int)threadIdx.x & 63;
    const int2 mine = L < n ? list[L] : make_int2(0, 0);
    // row `row` of tile t: word row >> 4 of lanes (row & 15) + 16 g, g = 0..3
    const uint8_t* rowbase = a.planes + (int64_t)b * 16 * a.K + 16 * (row & 15) + 4 * (row >> 4);
    double part = 0.0;
    for (int i0 = 0; i0 < n; i0 += 4) {
        uint32_t w[4][4];
        int kc[4];
        float res[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = min(i0 + j, n - 1);
            const int64_t k = col0 + __builtin_amdgcn_readlane(mine.x, i);
            res[j] = __int_as_float(__builtin_amdgcn_readlane(mine.y, i));
            kc[j] = (int)(k & 63);
            const uint8_t* wp = rowbase + (k >> 6) * kTileBytes + 256 * (kc[j] >> 4);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[j][q] = (q >= first && q < depth) ? *reinterpret_cast<const uint32_t*>(wp + q * a.plane_bytes) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (i0 + j >= n) break;
            // slice 3 - q of the element's byte, before the rotation by 2u
            const int u = (kc[j] >> 2) & 3;
            uint32_t acc = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t m = 0x03030303u << (2 * (3 - q));
                acc |= w[j][q] & ((m >> (2 * u)) | (m << ((32 - 2 * u) & 31)));
            }
            acc = (acc << (2 * u)) | (acc >> ((32 - 2 * u) & 31));
            part += (double)(int)(int8_t)(uint8_t)(acc >> (8 * (kc[j] & 3))) * (double)res[j];
        }
    }
    return e < kSmallExp ? ldexp(part, -kPrescale) : part;
}

// The same corrections for a chunk with many listed elements: the list,
// sorted by column, is spread tile by tile into the wave's LDS row `r2d`
// (64 residuals, zero where nothing is listed), and the lane of row `row`
// multiplies the row's 64 codes of the tile by it.  Terms are added in
// column order, as in listed_correction (the extra terms are exact zeros), so
// both forms give the same bits; this one reads each tile's words once
// instead of gathering one code per listed element.
constexpr int kDenseListed = 16;

__device__ __forceinline__ void row_tile_words(const uint8_t* tb, int64_t pb, int first, int depth,
                                               uint32_t (&w)[4][4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[g][q] = (q >= first && q < depth) ? *reinterpret_cast<const uint32_t*>(tb + 256 * g + q * pb) : 0u;
}

// (The item's fields come by value: a reference to the item would keep the
// caller's copy of it in scratch memory when this is not inlined.)
__device__ double dense_correction(const uint8_t* planes, int64_t plane_bytes, int64_t K, const int2* unc, int tpc,
                                   int n_tiles, int b, int chunk, int slot, int n, int row, int first, int depth,
                                   int e, float* r2d) {
    const int2* list = unc + (int64_t)slot * tpc * 64;
    const int L = (int)threadIdx.x & 63;
    const int t0 = chunk * tpc;
    const int t1 = min(n_tiles, t0 + tpc);
    // row `row` of tile t: word row >> 4 of lanes (row & 15) + 16 g, g = 0..3
    const uint8_t* rowbase = planes + (int64_t)b * 16 * K + 16 * (row & 15) + 4 * (row >> 4);
    double part = 0.0;
    int p = 0;
    uint32_t cur[4][4], nxt[4][4];
    row_tile_words(rowbase + (int64_t)t0 * kTileBytes, plane_bytes, first, depth, cur);
    for (int t = t0; t < t1 && p < n; ++t) {
        if (t + 1 < t1) row_tile_words(rowbase + (int64_t)(t + 1) * kTileBytes, plane_bytes, first, depth, nxt);
        const int lo = (t - t0) * 64;
        int2 ent = make_int2(0x7fffffff, 0);
        if (p + L < n) ent = list[p + L];
        const bool in = ent.x < lo + 64;   // every earlier entry is consumed: these are the tile's
        const int cnt = __popcll(__ballot(in));
        if (cnt > 0) {
            r2d[L] = 0.0f;
            if (in) r2d[ent.x - lo] = __int_as_float(ent.y);
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    uint32_t acc = 0u;
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc |= cur[g][q] & rotr_const(0x03030303u << (2 * (3 - q)), 2 * u);
                    if (u != 0) acc = rotl32(acc, 2 * u);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        part += (double)(int8_t)(uint8_t)(acc >> (8 * i)) * (double)r2d[16 * g + 4 * u + i];
                }
            p += cnt;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) cur[g][q] = nxt[g][q];
    }
    return e < kSmallExp ? ldexp(part, -kPrescale) : part;
}

// One workgroup = KS x NH wavefronts = one (block, column chunk).
// REFINE: a refinement launch (c.first > 0); without it `first` is the
// constant 0 and the code is that of the plain product.
template <int NCG, bool PER_REQ, bool GROUPED, bool REFINE>
__global__ __launch_bounds__(256) void qmm_kernel(MItem single, MCommon c) {
    extern __shared__ int tab[];   // [NH][64 rows][16 NCG + 1] integer sums, one flag, then r2d rows
    constexpr int TW = 16 * NCG + 1;
    constexpr int NCGC = ncgc_of_ncg(NCG);
    MItem a;
    int local;
    if constexpr (GROUPED) {
        a = c.items[c.wg_item[blockIdx.x]];
        local = (int)blockIdx.x - a.wg_begin;
    } else {
        a = single;
        local = (int)blockIdx.x;
    }
    const int B = c.B, NH = c.NH, KS = c.KS, SS = c.SS;
    const int FB = fine_base(NCG, SS);   // first column of the fine block
    const int first = REFINE ? c.first : 0;
    const int chunk = local % a.n_chunks;
    const int b = local / a.n_chunks;
    const int wave = (int)threadIdx.x >> 6;
    const int h = wave % NH;
    const int ks = wave / NH;
    const int L = (int)threadIdx.x & 63;
    const int nw = NH * KS;
    const int slots = SS * NH;
    // rung of request L (lanes < B); a rung above 4 is flagged, read as
    // nothing and its outputs are NaN; then the depths of the set's requests
    // and columns.  A refinement launch reads nothing for a request at or
    // below its first slice.
    const int rung = L < B ? rung_of<PER_REQ>(a, L, b) : 0;
    const bool bad = rung > 4;
    const uint64_t bad_mask = __ballot(bad);
    if (bad_mask && threadIdx.x == 0 && chunk == 0)
        __hip_atomic_fetch_or(c.status, (uint32_t)QAM_STATUS_BAD_RUNG, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int m_req = bad ? 0 : rung;
    const int m_all = m_req > first ? m_req : 0;
    uint32_t dm_all = 1u << m_all;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) dm_all |= __shfl_xor(dm_all, o);
    dm_all = __builtin_amdgcn_readfirstlane(dm_all);
    if (dm_all == 1u) {   // no request reads any of the block: y = 0 (unchanged when refining), by the first chunk
        if (chunk == 0)
            for (int r = wave; r < B; r += nw) {
                float* yo = &a.y[(int64_t)r * a.N + (int64_t)b * kRows + L];
                if ((bad_mask >> r) & 1) *yo = __builtin_nanf("");
                else if (!REFINE) *yo = 0.0f;
            }
        return;
    }
    const int m_set = __shfl(m_all, (SS * h + (L & 15)) & 63);   // depth of request SS h + (L & 15)
    uint32_t dm = (L < SS && SS * h + L < B) ? (1u << m_set) : 1u;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dm |= __shfl_xor(dm, o);
    dm = __builtin_amdgcn_readfirstlane(dm);
    const int ns = 31 - __builtin_clz(dm);
    int mcol[NCG];
    uint32_t gmask[NCG];
#pragma unroll
    for (int g = 0; g < NCG; ++g) {
        // request (within the set) owning this lane's column of group g
        const int cc = 16 * g + (L & 15);                       // the column in the set
        const bool coarse = NCG == 1 ? cc < kCoarseCols * SS : g < NCGC;
        const int rr = coarse ? cc / kCoarseCols : (cc - FB) / kFineCols;
        const int md = __shfl(m_set, rr & 15);                   // its depth (lane rr holds it)
        mcol[g] = (rr < SS && SS * h + rr < B) ? md : 0;
        uint32_t gm = 1u << mcol[g];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) gm |= __shfl_xor(gm, o);
        gmask[g] = __builtin_amdgcn_readfirstlane(gm);
    }
    for (int i = (int)threadIdx.x; i < NH * 64 * TW; i += (int)blockDim.x) tab[i] = 0;
    v4i acc[4][NCG];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < NCG; ++g) acc[j][g] = v4i{0, 0, 0, 0};
    // Sets of up to four requests always take the fine split: one pass over
    // every group.  Larger sets multiply their coarse groups first and the
    // fine ones in a second pass when a request of the set is fine for the
    // chunk, so no launch waits for the pre-pass's mode before its first loads.
    constexpr bool ALWAYS_FINE = NCG <= 2;
    constexpr int NG1 = ALWAYS_FINE ? NCG : NCGC;
    switch (ns) {
        case 0: break;   // no request of this set reads the block
        case 1: mproduct<1, NCG, 0, NG1, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, gmask, dm, first, acc); break;
        case 2: mproduct<2, NCG, 0, NG1, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, gmask, dm, first, acc); break;
        case 3: mproduct<3, NCG, 0, NG1, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, gmask, dm, first, acc); break;
        default: mproduct<4, NCG, 0, NG1, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, gmask, dm, first, acc); break;
    }
    // the chunk's exponent and listed count (with the fine flag) of every
    // request (lane r: request r) and this lane's row scale, read once the
    // first pass is done (the product's loads wait for nothing the pre-pass
    // wrote), so that their latency passes during the table sums
    int e_all = 0, n_all = 0;
    if (L < slots) {
        e_all = a.exps[chunk * slots + L];
        n_all = a.unc_count[chunk * slots + L];
    }
    const float sc32 = a.scales[b * kRows + L];
    __syncthreads();   // the tables are clear
    // the wave's 64 x 16 NCG integer sums added into its set's table
    int* mine = tab + h * 64 * TW;
    if (ns > 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < NG1; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    atomicAdd(&mine[(16 * j + 4 * (L >> 4) + i) * TW + 16 * g + (L & 15)], acc[j][g][i]);
    }
    if constexpr (!ALWAYS_FINE) {
        // the set's mode: a fine request of the set brings the fine groups in
        const uint64_t fine_bits = __ballot(L < slots && (n_all & kFineFlag) != 0);
        const bool fine = __builtin_amdgcn_readfirstlane(
                              (int)(((fine_bits >> (SS * h)) & ((1ull << SS) - 1)) != 0)) != 0;
        if (fine && ns > 0) {
            switch (ns) {
                case 1: mproduct<1, NCG, NCGC, NCG - NCGC, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, gmask, dm, first, acc); break;
                case 2: mproduct<2, NCG, NCGC, NCG - NCGC, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, gmask, dm, first, acc); break;
                case 3: mproduct<3, NCG, NCGC, NCG - NCGC, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, gmask, dm, first, acc); break;
                default: mproduct<4, NCG, NCGC, NCG - NCGC, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, gmask, dm, first, acc); break;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int g = NCGC; g < NCG; ++g)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        atomicAdd(&mine[(16 * j + 4 * (L >> 4) + i) * TW + 16 * g + (L & 15)], acc[j][g][i]);
        }
    }
    __syncthreads();

    // outputs: one row per lane, requests spread over the waves; the sums of
    // request r are its coarse columns 4 (r mod SS) + l and fine columns
    // 16 NCGC + 2 (r mod SS) + l of set r / SS, combined and scaled into fp64,
    // with the chunk's listed corrections
    const int row = L;
    float* r2d = reinterpret_cast<float*>(tab + NH * 64 * TW + 4) + 64 * wave;   // this wave's residual row
    const double sc = (double)sc32;
    const bool split = a.n_chunks > 1;
    for (int r = wave; r < B; r += nw) {
        const int* t2 = tab + (r / SS) * 64 * TW + row * TW + kCoarseCols * (r % SS);
        const int* t2f = tab + (r / SS) * 64 * TW + row * TW + FB + kFineCols * (r % SS);
        const int slot = chunk * slots + r;
        const int e = __shfl(e_all, r & 63);
        const int mr = __shfl(m_all, r & 63);
        double v = 0.0;
        if (mr != 0) {
            if (e == kBadExp) {
                v = __builtin_nan("");
            } else {
                v = limb_value(t2[0], t2[1], t2[2], t2f[0], t2f[1], t2[3], e);
                const int n = __shfl(n_all, r & 63) & ~kFineFlag;
                if (n > kDenseListed)
                    v += dense_correction(a.planes, a.plane_bytes, a.K, a.unc, a.tpc, a.n_tiles, b, chunk, slot, n, row,
                                          first, mr, e, r2d);
                else if (n > 0)
                    v += listed_correction(a, b, chunk, slot, n, row, first, mr, e);
            }
        }
        if ((bad_mask >> r) & 1) v = __builtin_nan("");
        if (!split) {
            float* yo = &a.y[(int64_t)r * a.N + (int64_t)b * kRows + row];
            if constexpr (!REFINE) *yo = (float)(sc * v);
            else if (mr != 0 || ((bad_mask >> r) & 1)) *yo = (float)((double)*yo + sc * v);
        } else {   // split K: publish the partial with a device-scope write-through store
            __hip_atomic_store(&a.partials[((int64_t)chunk * B + r) * a.N + (int64_t)b * kRows + row], v,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (!split) return;
    // Once the whole workgroup's partial stores are complete, one thread
    // counts the arrival; the last workgroup of the block sums the partials
    // in chunk order.  The signal fences keep the compiler from moving the
    // partial stores past the counter update, or the loads ahead of it.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int* flag = tab + NH * 64 * TW;
    if (threadIdx.x == 0)
        *flag = (int)__hip_atomic_fetch_add(&a.counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (*flag != a.n_chunks - 1) return;
    // The wave's (request, chunk) pairs in request-major order, eight
    // partial loads in flight at a time; each request's sum still runs over
    // its chunks in order.
    const int nc = a.n_chunks;
    const int n_pairs = (B - wave + nw - 1) / nw * nc;
    const double* pbase = a.partials + (int64_t)b * kRows + row;
    double sum = 0.0;
    for (int f0 = 0; f0 < n_pairs; f0 += 8) {
        double pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int f = min(f0 + j, n_pairs - 1);
            const int jr = f / nc, cc = f - jr * nc;
            pv[j] = __hip_atomic_load(pbase + ((int64_t)cc * B + wave + jr * nw) * a.N, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int f = f0 + j;
            if (f >= n_pairs) break;
            sum += pv[j];
            const int jr = f / nc;
            if (f - jr * nc != nc - 1) continue;
            const int r = wave + jr * nw;
            float* yo = &a.y[(int64_t)r * a.N + (int64_t)b * kRows + row];
            if constexpr (!REFINE) *yo = (float)(sc * sum);
            else if (__shfl(m_all, r & 63) != 0 || ((bad_mask >> r) & 1)) *yo = (float)((double)*yo + sc * sum);
            sum = 0.0;
        }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (threadIdx.x == 0) __hip_atomic_store(&a.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ host side

template <int NCG, bool GROUPED>
static void launch_product(const MItem& it, const MCommon& c, bool per_req, int64_t grid, hipStream_t s) {
    const dim3 blk(64 * c.NH * c.KS);
    const size_t lds = ((size_t)c.NH * 64 * (16 * NCG + 1) + 4 + 4 * 64) * sizeof(int);   // + 4 waves' r2d rows
    if (c.first > 0) {
        if (per_req)
            hipLaunchKernelGGL((qmm_kernel<NCG, true, GROUPED, true>), dim3((unsigned)grid), blk, lds, s, it, c);
        else
            hipLaunchKernelGGL((qmm_kernel<NCG, false, GROUPED, true>), dim3((unsigned)grid), blk, lds, s, it, c);
    } else if (per_req) {
        hipLaunchKernelGGL((qmm_kernel<NCG, true, GROUPED, false>), dim3((unsigned)grid), blk, lds, s, it, c);
    } else {
        hipLaunchKernelGGL((qmm_kernel<NCG, false, GROUPED, false>), dim3((unsigned)grid), blk, lds, s, it, c);
    }
}

template <bool GROUPED>
static void launch_mfma(const MItem& it, const MCommon& c, bool xbf16, bool per_req, int64_t pre_grid, int64_t grid,
                        hipStream_t s) {
    if (xbf16)
        hipLaunchKernelGGL((limbs_kernel<true, GROUPED>), dim3((unsigned)pre_grid), dim3(kPreThreads), 0, s, it, c);
    else
        hipLaunchKernelGGL((limbs_kernel<false, GROUPED>), dim3((unsigned)pre_grid), dim3(kPreThreads), 0, s, it, c);
    switch (c.NCG) {   // the totals ncg_of_ss gives
        case 1: launch_product<1, GROUPED>(it, c, per_req, grid, s); break;
        case 2: launch_product<2, GROUPED>(it, c, per_req, grid, s); break;
        case 3: launch_product<3, GROUPED>(it, c, per_req, grid, s); break;
        case 5: launch_product<5, GROUPED>(it, c, per_req, grid, s); break;
        default: launch_product<6, GROUPED>(it, c, per_req, grid, s); break;
    }
}

struct MPlan {
    int NH, SS, NCG, KS, tpc, n_chunks;
    size_t counters, partials, limbs, exps, unc, total;
};

// Plan defaults of the pre-pass route (a group's qam_tuning may change them).
// Wavefronts aimed for per launch (with four waves per set: on the streaming
// stack, two chunks per 28672-column matrix).
constexpr int64_t kMfmaTargetWaves = 256 * 64;
// Waves per request set splitting each chunk's tiles inside a workgroup (at
// most four waves per workgroup): a split inside the workgroup is reduced in
// LDS, one across workgroups through partials in memory.
constexpr int kMfmaKsplit = 4;
constexpr int kMfmaSetMax = 16;

struct MShape {
    int NH, SS, NCG, KS;
};

static MShape mshape(int64_t B, const qam_tuning* t) {
    MShape m{};
    const int set_max = t && t->set_max > 0 ? t->set_max : kMfmaSetMax;
    m.NH = (int)((B + set_max - 1) / set_max);              // request sets, as even as possible
    m.SS = (int)((B + m.NH - 1) / m.NH);
    m.NCG = ncg_of_ss(m.SS);                                  // 16-column groups per set
    const int ks = t && t->ksplit > 0 ? t->ksplit : kMfmaKsplit;
    m.KS = std::max(1, std::min(ks, 4 / m.NH));               // at most four waves per workgroup
    return m;
}

// Shortest column chunk in tiles.  Measured on the batched layer (4096 and
// 14336 columns) and the streaming stack: per-request maps take chunks of at
// least 96 tiles, shared maps 3 B tiles.  A split of K writes B fp64 partials
// per row and chunk and reads them back (16 B bytes per row against 64 bytes
// per row and tile of weights at D8), so short chunks spend a large share of
// the traffic on partials.
static int mfma_min_tiles(int64_t B, bool per_req, const qam_tuning* t) {
    if (t && t->tiles_per_request > 0) return (int)std::min<int64_t>(4096, (int64_t)t->tiles_per_request * B);
    return per_req ? 96 : (int)(3 * B);
}

// Chunking of one matrix on the pre-pass route, for a chunk length goal.
static MPlan mplan_goal(int64_t N, int64_t K, int64_t B, int goal, bool per_req, const qam_tuning* t) {
    MPlan p{};
    const MShape m = mshape(B, t);
    p.NH = m.NH;
    p.SS = m.SS;
    p.NCG = m.NCG;
    p.KS = m.KS;
    const int n_tiles = (int)(K / kTileCols);
    goal = std::max<int>(goal, mfma_min_tiles(B, per_req, t));
    const int want = (n_tiles + goal - 1) / goal;
    int tpc = (n_tiles + want - 1) / want;
    tpc = (tpc + 3) / 4 * 4;
    if (tpc > n_tiles) tpc = n_tiles;
    p.tpc = tpc;
    p.n_chunks = (n_tiles + tpc - 1) / tpc;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t slots = (size_t)p.n_chunks * p.SS * p.NH;
    p.counters = QAM_WS_COUNTER_BYTES;
    p.partials = p.n_chunks > 1 ? up((size_t)p.n_chunks * B * N * sizeof(double)) : 0;
    p.limbs = up((size_t)n_tiles * p.NH * p.NCG * 64 * 16);
    p.exps = up(2 * slots * sizeof(int));                     // exponents, then listed counts
    p.unc = up(slots * (size_t)p.tpc * 64 * sizeof(int2));
    p.total = p.counters + p.partials + p.limbs + p.exps + p.unc;
    return p;
}

static int64_t mfma_target(const qam_tuning* t) { return t && t->target_waves > 0 ? t->target_waves : kMfmaTargetWaves; }

static MPlan mplan(int64_t N, int64_t K, int64_t B, bool per_req) {
    const MShape m = mshape(B, nullptr);
    const int64_t block_tiles = N / kRows * (K / kTileCols) * m.NH * m.KS;
    return mplan_goal(N, K, B, chunk_goal(block_tiles, mfma_target(nullptr), 0), per_req, nullptr);
}

static MItem make_mitem(const void* x, const qam_packed* w, const uint8_t* level_map, float* y, int per_request,
                        const MPlan& p, char* limbs, char* exps, char* unc) {
    MItem it{};
    it.planes = static_cast<const uint8_t*>(w->planes);
    it.scales = w->scales;
    it.x = x;
    it.y = y;
    it.level = level_map;
    it.level_stride = per_request ? w->n_blocks : 0;
    it.plane_bytes = w->N * w->K / 4;
    it.N = w->N;
    it.K = w->K;
    it.n_blocks = (int)w->n_blocks;
    it.n_tiles = (int)(w->K / kTileCols);
    it.tpc = p.tpc;
    it.n_chunks = p.n_chunks;
    it.limbs = reinterpret_cast<v4i*>(limbs);
    it.exps = reinterpret_cast<int*>(exps);
    it.unc_count = reinterpret_cast<int*>(exps) + (size_t)p.n_chunks * p.SS * p.NH;
    it.unc = reinterpret_cast<int2*>(unc);
    return it;
}

static MCommon mcommon(int64_t B, int NH, int SS, int NCG, int KS, uint32_t* status) {
    MCommon c{};
    c.B = (int)B;
    c.NH = NH;
    c.SS = SS;
    c.NCG = NCG;
    c.NCGC = ncgc_of_ncg(NCG);
    c.KS = KS;
    c.status = status;
    return c;
}

// Workspace of the pre-pass route (0 for bad shapes).
size_t qam_mfma_workspace_bytes(int64_t N, int64_t K, int64_t B) {
    if (N <= 0 || K <= 0 || N % kRows || K % kTileCols || K > QAM_MAX_K || B < 1 || B > QAM_MAX_BATCH_MFMA) return 0;
    if (N / kRows > QAM_MAX_BLOCKS) return 0;
    return std::max(mplan(N, K, B, false).total, mplan(N, K, B, true).total);   // either kind of map
}

// The pre-pass route of qam_qmatvec (arguments already checked by the caller).
int qmatvec_mfma(const void* x, int x_dtype, int64_t B, const qam_packed* packed, const uint8_t* level_map,
                 int per_request_maps, float* y, void* workspace, size_t workspace_bytes, hipStream_t s) {
    const MPlan p = mplan(packed->N, packed->K, B, per_request_maps != 0);
    if (int rc = check_workspace(workspace, workspace_bytes, p.total, "qmatvec")) return rc;
    char* ws = static_cast<char*>(workspace);
    char* limbs = ws + p.counters + p.partials;
    MItem it = make_mitem(x, packed, level_map, y, per_request_maps, p, limbs, limbs + p.limbs,
                          limbs + p.limbs + p.exps);
    it.counters = reinterpret_cast<uint32_t*>(ws);
    it.partials = p.partials ? reinterpret_cast<double*>(ws + p.counters) : nullptr;
    const MCommon c = mcommon(B, p.NH, p.SS, p.NCG, p.KS, status_word(ws));
    launch_mfma<false>(it, c, x_dtype == QAM_X_BF16, per_request_maps != 0, (int64_t)p.n_chunks * p.SS * p.NH,
                       (int64_t)it.n_blocks * p.n_chunks, s);
    QAM_HIP_CHECK(hipGetLastError());
    char v[128];
    snprintf(v, sizeof(v), "qmatvec_mfma B=%lld maps=%s tpc=%d chunks=%d sets=%d colgroups=%d ksplit=%d",
             (long long)B, per_request_maps ? "per-request" : "shared", p.tpc, p.n_chunks, p.NH, p.NCG, p.KS);
    set_variant(v);
    return QAM_OK;
}

// The pre-pass route with an input transform (internal: the verify chain).
int qmatvec_mfma_in(const float* x, int64_t B, const qam_packed* packed, const uint8_t* level_map, float* y,
                    const XIn& in, void* workspace, size_t workspace_bytes, hipStream_t s) {
    if (!x || !packed || !packed->planes || !level_map || !y) QAM_FAIL(QAM_ERR_NULL, "qmatvec_in: null pointer");
    if (B < 2 || B > QAM_MAX_BATCH_MFMA) QAM_FAIL(QAM_ERR_ARG, "qmatvec_in: B=%lld outside [2, %d]", (long long)B,
                                                  QAM_MAX_BATCH_MFMA);
    const int64_t N = packed->N, K = packed->K;
    if (N <= 0 || K <= 0 || N % kRows || K % kTileCols || K > QAM_MAX_K || packed->n_blocks != N / kRows)
        QAM_FAIL(QAM_ERR_SHAPE, "qmatvec_in: bad packed shape N=%lld K=%lld", (long long)N, (long long)K);
    const bool norm = in.mode == kXAddNorm;
    switch (in.mode) {
        case kXPlain: break;
        case kXStrided:
            if (in.ld < K || in.ld % 4) QAM_FAIL(QAM_ERR_ARG, "qmatvec_in: row stride %lld", (long long)in.ld);
            break;
        case kXAddNorm:
            if (!in.add || !in.res || !in.side) QAM_FAIL(QAM_ERR_NULL, "qmatvec_in: add-norm needs add, res, side");
            if (!(in.eps >= 0.0)) QAM_FAIL(QAM_ERR_ARG, "qmatvec_in: eps must be >= 0");
            break;
        case kXGated:
            if (!in.side) QAM_FAIL(QAM_ERR_NULL, "qmatvec_in: gated input needs side");
            if (in.ld < 2 * K || in.ld % 4) QAM_FAIL(QAM_ERR_ARG, "qmatvec_in: row stride %lld", (long long)in.ld);
            break;
        default: QAM_FAIL(QAM_ERR_ARG, "qmatvec_in: unknown input mode %d", in.mode);
    }
    if (!aligned(x, 16) || !aligned(in.add, 16) || !aligned(in.res, 16) || !aligned(in.side, 16) || !aligned(y, 4))
        QAM_FAIL(QAM_ERR_ALIGN, "qmatvec_in: inputs must be 16-byte aligned");
    // the whole row in one chunk for the norm (its sum of squares comes first)
    const MPlan p = norm ? mplan_goal(N, K, B, (int)(K / kTileCols), false, nullptr) : mplan(N, K, B, false);
    if (norm && p.n_chunks != 1) QAM_FAIL(QAM_ERR_SHAPE, "qmatvec_in: the norm's row spans %d chunks", p.n_chunks);
    if (int rc = check_workspace(workspace, workspace_bytes, p.total, "qmatvec_in")) return rc;
    char* ws = static_cast<char*>(workspace);
    char* limbs = ws + p.counters + p.partials;
    MItem it = make_mitem(x, packed, level_map, y, 0, p, limbs, limbs + p.limbs, limbs + p.limbs + p.exps);
    it.counters = reinterpret_cast<uint32_t*>(ws);
    it.partials = p.partials ? reinterpret_cast<double*>(ws + p.counters) : nullptr;
    it.x_mode = in.mode;
    it.x_ld = in.ld;
    it.x_add = in.add;
    it.x_res = in.res;
    it.x_side = in.side;
    it.x_eps = in.eps;
    const MCommon c = mcommon(B, p.NH, p.SS, p.NCG, p.KS, status_word(ws));
    launch_mfma<false>(it, c, false, false, (int64_t)p.n_chunks * p.SS * p.NH, (int64_t)it.n_blocks * p.n_chunks, s);
    QAM_HIP_CHECK(hipGetLastError());
    return QAM_OK;
}

// ------------------------------------------------------------------ grouped launches

struct MGroupLayout {
    std::vector<MPlan> plans;
    size_t partials = 0, limbs = 0, exps = 0, unc = 0, table = 0, wgmap = 0, premap = 0, total = 0;
    int64_t n_wg = 0, n_pre = 0, blocks = 0;
    MShape m{};
};

static int mfma_layout(const qam_gemv_item* items, int n_items, int64_t B, bool per_req, const qam_tuning* t,
                       MGroupLayout& g) {
    if (!items || n_items < 1) QAM_FAIL(QAM_ERR_ARG, "group: need at least one item");
    if (B < 2 || B > QAM_MAX_BATCH_MFMA) QAM_FAIL(QAM_ERR_ARG, "group: B=%lld outside [2, %d]", (long long)B, QAM_MAX_BATCH_MFMA);
    g.m = mshape(B, t);
    int64_t block_tiles = 0;
    for (int i = 0; i < n_items; ++i) {
        const qam_packed& w = items[i].w;
        if (w.N <= 0 || w.N % kRows || w.K <= 0 || w.K % kTileCols || w.K > QAM_MAX_K)
            QAM_FAIL(QAM_ERR_SHAPE, "group: item %d has a bad shape", i);
        g.blocks += w.N / kRows;
        block_tiles += w.N / kRows * (w.K / kTileCols) * g.m.NH * g.m.KS;
    }
    if (g.blocks > QAM_MAX_BLOCKS) QAM_FAIL(QAM_ERR_SHAPE, "group: %lld blocks > %d", (long long)g.blocks, QAM_MAX_BLOCKS);
    const int goal = chunk_goal(block_tiles, mfma_target(t), 0);
    for (int i = 0; i < n_items; ++i) {
        const MPlan p = mplan_goal(items[i].w.N, items[i].w.K, B, goal, per_req, t);
        g.plans.push_back(p);
        g.partials += p.partials;
        g.limbs += p.limbs;
        g.exps += p.exps;
        g.unc += p.unc;
        g.n_wg += (int64_t)(items[i].w.N / kRows) * p.n_chunks;
        g.n_pre += (int64_t)p.n_chunks * g.m.SS * g.m.NH;
    }
    if (g.n_wg > 0x7FFFFFFF || g.n_pre > 0x7FFFFFFF) QAM_FAIL(QAM_ERR_SHAPE, "group: too many workgroups");
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    g.table = up((size_t)n_items * sizeof(MItem));
    g.wgmap = up((size_t)g.n_wg * sizeof(int));
    g.premap = up((size_t)g.n_pre * sizeof(int));
    g.total = QAM_WS_COUNTER_BYTES + g.partials + g.limbs + g.exps + g.unc + g.table + g.wgmap + g.premap;
    return QAM_OK;
}

// Device bytes of a group on the pre-pass route: enough for either kind of map.
size_t mfma_group_bytes(const qam_gemv_item* items, int n_items, int64_t B, const qam_tuning* t) {
    MGroupLayout g2;
    if (mfma_layout(items, n_items, B, true, t, g2) != QAM_OK) return 0;
    MGroupLayout g;
    if (mfma_layout(items, n_items, B, false, t, g) != QAM_OK) return 0;
    return std::max(g.total, g2.total);
}

int mfma_group_init(const qam_gemv_item* items, int n_items, int64_t B, int x_dtype, int per_request_maps,
                    const qam_tuning* t, void* dev_mem, size_t dev_bytes, qam_group* out, hipStream_t s) {
    MGroupLayout g;
    if (int rc = mfma_layout(items, n_items, B, per_request_maps != 0, t, g)) return rc;
    if (dev_bytes < g.total) QAM_FAIL(QAM_ERR_WORKSPACE, "group_init: %zu < %zu bytes", dev_bytes, g.total);
    if (!aligned(dev_mem, 256)) QAM_FAIL(QAM_ERR_ALIGN, "group_init: device memory must be 256-byte aligned");
    char* base = static_cast<char*>(dev_mem);
    char* partials = base + QAM_WS_COUNTER_BYTES;
    char* limbs = partials + g.partials;
    char* exps = limbs + g.limbs;
    char* unc = exps + g.exps;
    char* table = unc + g.unc;
    char* wgmap = table + g.table;
    char* premap = wgmap + g.wgmap;
    std::vector<MItem> host_items(n_items);
    std::vector<int> hw((size_t)g.n_wg), hp((size_t)g.n_pre);
    int64_t wg = 0, pre = 0, blk = 0;
    size_t po = 0, lo = 0, eo = 0, uo = 0;
    for (int i = 0; i < n_items; ++i) {
        const qam_gemv_item& gi = items[i];
        if (int rc = check_item(gi.x, x_dtype, B, &gi.w, gi.level_map, gi.y, "group_init", QAM_OUT_STORE)) return rc;
        const MPlan& p = g.plans[i];
        if (gi.level_stride < 0 || (gi.level_stride > 0 && gi.level_stride < gi.w.n_blocks))
            QAM_FAIL(QAM_ERR_ARG, "group_init: item %d level_stride %lld < n_blocks", i, (long long)gi.level_stride);
        MItem it = make_mitem(gi.x, &gi.w, gi.level_map, gi.y, per_request_maps, p, limbs + lo, exps + eo, unc + uo);
        if (per_request_maps && gi.level_stride > 0) it.level_stride = gi.level_stride;
        it.counters = reinterpret_cast<uint32_t*>(base) + blk;
        it.partials = p.partials ? reinterpret_cast<double*>(partials + po) : nullptr;
        po += p.partials;
        lo += p.limbs;
        eo += p.exps;
        uo += p.unc;
        blk += it.n_blocks;
        it.wg_begin = (int)wg;
        it.pre_begin = (int)pre;
        const int64_t n = (int64_t)it.n_blocks * p.n_chunks;
        for (int64_t k = 0; k < n; ++k) hw[(size_t)(wg + k)] = i;
        wg += n;
        const int64_t np = (int64_t)p.n_chunks * g.m.SS * g.m.NH;
        for (int64_t k = 0; k < np; ++k) hp[(size_t)(pre + k)] = i;
        pre += np;
        host_items[i] = it;
    }
    QAM_HIP_CHECK(hipMemsetAsync(base, 0, QAM_WS_COUNTER_BYTES, s));
    QAM_HIP_CHECK(hipMemcpyAsync(table, host_items.data(), sizeof(MItem) * n_items, hipMemcpyHostToDevice, s));
    QAM_HIP_CHECK(hipMemcpyAsync(wgmap, hw.data(), sizeof(int) * hw.size(), hipMemcpyHostToDevice, s));
    QAM_HIP_CHECK(hipMemcpyAsync(premap, hp.data(), sizeof(int) * hp.size(), hipMemcpyHostToDevice, s));
    QAM_HIP_CHECK(hipStreamSynchronize(s));
    *out = qam_group{};
    out->dev_mem = dev_mem;
    out->n_items = n_items;
    out->B = B;
    out->x_dtype = x_dtype;
    out->n_workgroups = g.n_wg;
    out->lds_bytes = 0;
    out->table = table;
    out->wg_map = wgmap;
    out->route = 1;
    out->per_request_maps = per_request_maps;
    out->n_pre_workgroups = g.n_pre;
    out->pre_map = premap;
    out->lens_ready = 0;
    out->sets = g.m.NH;
    out->set_size = g.m.SS;
    out->col_groups = g.m.NCG;
    out->ksplit = g.m.KS;
    return QAM_OK;
}

// first > 0: a refinement launch (slices first.. of each request's depth added to y).
static int mfma_group_run_from(const qam_group* g, int first, hipStream_t s) {
    if (!g->dev_mem || g->sets < 1 || g->sets > 4 || g->set_size < 1 || g->set_size > 16 ||
        (int64_t)g->sets * g->set_size < g->B || g->col_groups != ncg_of_ss(g->set_size) || g->ksplit < 1 ||
        g->ksplit * g->sets > 4)
        QAM_FAIL(QAM_ERR_ARG, "qmatvec_group: corrupt group descriptor");
    MCommon c = mcommon(g->B, g->sets, g->set_size, g->col_groups, g->ksplit, status_word(g->dev_mem));
    c.items = static_cast<const MItem*>(g->table);
    c.wg_item = static_cast<const int*>(g->wg_map);
    c.pre_item = static_cast<const int*>(g->pre_map);
    c.first = first;
    MItem dummy{};
    launch_mfma<true>(dummy, c, g->x_dtype == QAM_X_BF16, g->per_request_maps != 0, g->n_pre_workgroups,
                      g->n_workgroups, s);
    QAM_HIP_CHECK(hipGetLastError());
    char v[128];
    snprintf(v, sizeof(v), "qmatvec_mfma_group%s items=%d B=%lld maps=%s sets=%d colgroups=%d ksplit=%d wg=%lld",
             first ? "_refine" : "", g->n_items, (long long)g->B, g->per_request_maps ? "per-request" : "shared",
             g->sets, g->col_groups, g->ksplit, (long long)g->n_workgroups);
    set_variant(v);
    return QAM_OK;
}

int mfma_group_run(const qam_group* g, hipStream_t s) { return mfma_group_run_from(g, 0, s); }

}  // namespace qam

extern "C" int qam_qmatvec_group_refine(const qam_group* group, int first_slice, hipStream_t s) {
    qam::clear_error();
    if (!group || !group->table || !group->wg_map || !group->pre_map)
        QAM_FAIL(QAM_ERR_NULL, "qmatvec_group_refine: uninitialised group");
    if (group->route != 1 || group->B < 2 || group->B > QAM_MAX_BATCH_MFMA || group->n_workgroups < 1)
        QAM_FAIL(QAM_ERR_ARG, "qmatvec_group_refine: the group must take the pre-pass route");
    if (first_slice < 1 || first_slice > 3) QAM_FAIL(QAM_ERR_ARG, "qmatvec_group_refine: first_slice %d outside [1, 3]", first_slice);
    return qam::mfma_group_run_from(group, first_slice, s);
}
