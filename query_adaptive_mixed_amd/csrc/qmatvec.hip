// Mixed-depth matrix-vector product over the slice planes (the staged-limb
// route: one request).
//
// Each block of 64 output rows is read at its own depth straight from the
// stored bytes inside the pass ("FoQLens", table "Progress"); a block read at
// d bits touches d/2 slice planes, a ZERO block nothing.  Cost is the weight
// bytes read ("Precision on Demand", abstract).
//
// Work decomposition.  A workgroup is one wavefront (or up to eight splitting
// a chunk's tiles) and takes one block of 64 rows and one chunk of columns
// (tiles_per_chunk tiles of 64).  The wave walks its chunk in sub-chunks of
// 16 tiles; the ring of weight loads runs through the whole chunk, and each
// sub-chunk's x is turned into the exact fixed-point form of
// qmatvec_internal.h in LDS (largest |x| of the sub-chunk in [2^(e-1), 2^e);
// hi and lo parts, three signed int8 limbs each).  Each lane owns, per
// 64-column tile and per slice, one 16-byte word group covering 4 rows x 16
// columns; codes are rebuilt in registers (one mask per slice and one rotate
// per four codes) and multiplied into the limbs exactly, in int32, with
// v_mfma_i32_16x16x64_i8 on the matrix cores: the rebuilt words are the A
// operand as they stand, and B-operand column l holds limb l (hi 0..2, lo
// 0..2).  The six column sums are combined into a per-row fp64 sum.  A
// sub-chunk holding an element that the two parts do not carry to 2^-15
// relative error (its range within the sub-chunk exceeds 2^31, e.g. the
// exponentially small tail of a gated activation) is instead staged as fp32
// and multiplied on the vector ALUs in fp32 (per-element exponents; at most
// 256 sequential terms per lane and row, so within 2^-16 of sum|w||x|).  The
// row sums are either written as the
// output (one chunk) or stored as partials; the last wavefront of a block to
// finish sums the partials in chunk order and writes y = fl32(scale * sum).
// No floating-point atomics: results are bit-reproducible.
//
// The same kernel serves one matrix (descriptor passed by value, with its
// fused epilogue) and a group of matrices with independent inputs (descriptor
// table in device memory, one table lookup per workgroup), so a whole weight
// field is one launch.
#include <hip/hip_ext.h>

#include <algorithm>
#include <vector>

#include "lens_rules.h"
#include "qmatvec_internal.h"

namespace qam {

// ------------------------------------------------------------------ timeline

// The timeline build (QAM_TIMELINE) stamps chosen single-matrix launches;
// elsewhere the stamps compile to nothing.
#ifdef QAM_TIMELINE
__constant__ const void* tl_select[QAM_TIMELINE_SLOTS];
__device__ unsigned long long tl_stamps[QAM_TIMELINE_SLOTS][QAM_TIMELINE_GROUPS][8][QAM_TIMELINE_POINTS];
#define QAM_STAMP(P)                                                                                    \
    do {                                                                                                \
        if (tl_row != nullptr && L == 0) tl_row[ks * QAM_TIMELINE_POINTS + (P)] = (unsigned long long)wall_clock64(); \
    } while (0)
#else
#define QAM_STAMP(P) \
    do {             \
    } while (0)
#endif

// ------------------------------------------------------------------ layout

// Sub-chunks of S tiles: each lane loads G = S / 4 groups of four x values.
constexpr int kStageTiles = 16;
constexpr int kStageGroups = kStageTiles / 4;

// Prefetch ring: two halves of H tiles each, up to sixteen 16-byte loads in
// flight per lane.  The wait before one half is computed always follows the
// reload of the other half, so it drains exactly the older half.
template <int NS>
struct Ring {
    static constexpr int raw = 8 / NS;
    static constexpr int Hr = raw >= 4 ? 4 : (raw >= 2 ? 2 : 1);
    static constexpr int H = Hr > kStageTiles / 2 ? kStageTiles / 2 : Hr;   // tiles per half
    static constexpr int PF = 2 * H;                                         // tiles per ring
};

// B operand in LDS: per tile, one 16-byte slot per (limb column c < 6, lane
// group k) at 4 c + k, then 4 zero slots that columns 6..15 read.  After the
// sub-chunk's slots, the [6][64] int32 table of its column sums.  A sub-chunk
// staged as fp32 keeps x of tile t, columns 16 k .. 16 k + 15, in slots
// t * 28 + 4 k .. + 3 (clear of the zero slots).
constexpr int kSlotsPerTile = 4 * (kLimbCols + 1);
constexpr int kZeroSlot = 4 * kLimbCols;
constexpr int kRegionInt4 = kStageTiles * kSlotsPerTile + kLimbCols * 16;   // int4 per wave

// One tile on the matrix cores: for each 16-row group j, the rebuilt codes of
// the lane (row 16j + (L & 15), columns 16(L >> 4) + 0..15) are the A
// operand; the lane's B operand is column L & 15 of the limbs (slot bslot of
// the tile).  acc[j] gets the 16 x 16 int32 product: lane L holds column
// L & 15 of rows 16j + 4(L >> 4) + i.
template <int NS>
__device__ __forceinline__ void tile_mfma(const u32x4* buf, const int4* __restrict__ lt, int bslot, v4i (&acc)[4]) {
    const int4 b4 = lt[bslot];
    const v4i bm = v4i{b4.x, b4.y, b4.z, b4.w};
    uint32_t w[4][NS];
#pragma unroll
    for (int p = 0; p < NS; ++p) {
        w[0][p] = buf[p].x;
        w[1][p] = buf[p].y;
        w[2][p] = buf[p].z;
        w[3][p] = buf[p].w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const v4i A = v4i{(int)assemble<NS, 0>(w[j]), (int)assemble<NS, 1>(w[j]), (int)assemble<NS, 2>(w[j]),
                          (int)assemble<NS, 3>(w[j])};
        acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, bm, acc[j], 0, 0, 0);
    }
}

// One tile in fp32 on the vector ALUs: lane L accumulates, for rows
// 16j + (L & 15), its 16 columns 16(L >> 4) + 4u + i: code (byte i of the
// rebuilt word u) times x, in fp32.  xt: this lane group's four slots of x.
__device__ __forceinline__ float code_byte(uint32_t P, int i) {
    return (float)((int)(P << (24 - 8 * i)) >> 24);
}

template <int NS>
__device__ __forceinline__ void tile_float(const u32x4* buf, const int4* __restrict__ xt, float (&facc)[4]) {
    uint32_t w[4][NS];
#pragma unroll
    for (int p = 0; p < NS; ++p) {
        w[0][p] = buf[p].x;
        w[1][p] = buf[p].y;
        w[2][p] = buf[p].z;
        w[3][p] = buf[p].w;
    }
    // one group of four columns at a time: four x values live, not sixteen
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
        const int4 v = xt[u];
        const float x0 = __int_as_float(v.x), x1 = __int_as_float(v.y), x2 = __int_as_float(v.z),
                    x3 = __int_as_float(v.w);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t acc = 0;
#pragma unroll
            for (int p = 0; p < NS; ++p) {
                const uint32_t m = 0x03030303u << (2 * (3 - p));
                acc |= w[j][p] & (u == 0 ? m : ((m >> (2 * u)) | (m << (32 - 2 * u))));
            }
            const uint32_t P = u == 0 ? acc : ((acc << (2 * u)) | (acc >> (32 - 2 * u)));
            facc[j] = __builtin_fmaf(code_byte(P, 0), x0, facc[j]);
            facc[j] = __builtin_fmaf(code_byte(P, 1), x1, facc[j]);
            facc[j] = __builtin_fmaf(code_byte(P, 2), x2, facc[j]);
            facc[j] = __builtin_fmaf(code_byte(P, 3), x3, facc[j]);
        }
    }
}

template <int NS, int H>
__device__ __forceinline__ void load_half(u32x4 (&h)[H][NS], const uint8_t* base, int64_t pb, int64_t tstride,
                                          int tile, int last) {
#pragma unroll
    for (int u = 0; u < H; ++u) {
        const int t = min(tile + u, last);   // past the sub-chunk: reload its last tile (never computed)
#pragma unroll
        for (int p = 0; p < NS; ++p) h[u][p] = load_plane(base + p * pb + (int64_t)t * tstride);
    }
}

// Orders this wavefront's own LDS accesses: the limb area is private to the
// wave and a wave's LDS instructions execute in issue order, so it is enough
// to keep the compiler from moving accesses across this point (no workgroup
// barrier: the waves of a workgroup run different numbers of sub-chunks).
__device__ __forceinline__ void lds_order() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only: vector loads stay in flight
}

// Largest |x| of a sub-chunk (every lane ends with it) and whether some x is
// not finite (0 * x summed is NaN exactly then).
__device__ __forceinline__ float sub_max(const float4 (&xv)[kStageGroups], bool& bad) {
    float m = 0.0f;
    float poison = 0.0f;
#pragma unroll
    for (int i = 0; i < kStageGroups; ++i) {
        const float4 v = xv[i];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        poison = __builtin_fmaf(v.x, 0.0f, poison);
        poison = __builtin_fmaf(v.y, 0.0f, poison);
        poison = __builtin_fmaf(v.z, 0.0f, poison);
        poison = __builtin_fmaf(v.w, 0.0f, poison);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        m = fmaxf(m, __shfl_xor(m, o));
        poison += __shfl_xor(poison, o);
    }
    bad = __builtin_amdgcn_readfirstlane((int)(poison != 0.0f)) != 0;   // NaN != 0
    return m;
}

__device__ __forceinline__ int exp_of(float m) {
    int e = 0;
    if (m > 0.0f) frexpf(m, &e);
    return __builtin_amdgcn_readfirstlane(e);
}

// Turn this wave's sub-chunk of x into limb words in LDS.  xraw[i] holds the
// x values of group L + 64 i (four columns).  The limb words of limb column
// c and the tile's columns 16k + 4u .. +3 go to word u of slot 4 c + k.  If
// some element of the sub-chunk is uncovered, x is staged as fp32 instead
// (slot t * 28 + (g & 15) for group g of tile t) and the return value is
// true: the sub-chunk runs in fp32.
template <bool XBF16>
__device__ __forceinline__ bool stage_limbs(const u32x4 (&xraw)[kStageGroups], int ngroups, int L,
                                            int4* __restrict__ lds, int& exp, bool& bad, bool want_ssq,
                                            double& ssq) {
    lds_order();   // the last sub-chunk's limb reads come before these writes
    float4 xv[kStageGroups];
#pragma unroll
    for (int i = 0; i < kStageGroups; ++i) xv[i] = x4_value<XBF16>(xraw[i]);
    const float m = sub_max(xv, bad);
    exp = exp_of(m);
    const XSplit sp = xsplit_of(exp);
    bool unc = false;
#pragma unroll
    for (int i = 0; i < kStageGroups; ++i) {
        const int g = L + 64 * i;
        if (g >= ngroups) continue;
        const float4 v = xv[i];
        if (want_ssq) {   // this lane's share of sum x^2 (an RMS-normalised input, one column chunk)
            ssq += (double)v.x * (double)v.x;
            ssq += (double)v.y * (double)v.y;
            ssq += (double)v.z * (double)v.z;
            ssq += (double)v.w * (double)v.w;
        }
        uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
        float r;
        bool u0, u1, u2, u3;
        split_elem(v.x, sp, h0, l0, r, u0);
        split_elem(v.y, sp, h1, l1, r, u1);
        split_elem(v.z, sp, h2, l2, r, u2);
        split_elem(v.w, sp, h3, l3, r, u3);
        unc = unc || u0 || u1 || u2 || u3;
        const int4 hw = limb_words(h0, h1, h2, h3);
        const int4 lw = limb_words(l0, l1, l2, l3);
        // slot (4 c + k) * 4 + u of tile g >> 4, k = (g & 15) >> 2, u = g & 3: 16 c + (g & 15)
        int* wl = reinterpret_cast<int*>(lds) + (g >> 4) * kSlotsPerTile * 4 + (g & 15);
        wl[0] = hw.x;
        wl[16] = hw.y;
        wl[32] = hw.z;
        wl[48] = lw.x;
        wl[64] = lw.y;
        wl[80] = lw.z;
    }
    const bool fp32 = __builtin_amdgcn_readfirstlane((int)(__ballot(unc) != 0)) != 0;
    if (fp32) {
        lds_order();   // the limb writes above come first
#pragma unroll
        for (int i = 0; i < kStageGroups; ++i) {
            const int g = L + 64 * i;
            if (g >= ngroups) continue;
            const float4 v = xv[i];
            lds[(g >> 4) * kSlotsPerTile + (g & 15)] =
                int4{__float_as_int(v.x), __float_as_int(v.y), __float_as_int(v.z), __float_as_int(v.w)};
        }
    }
    lds_order();   // the writes come before the tile loop's reads
    return fp32;
}

// ------------------------------------------------------------------ epilogue

// sum_k x[k]^2 in fp64, in a fixed order: lane partials over a stride of
// 256 columns, then a butterfly (every lane ends with the same value).
template <bool XBF16>
__device__ double sum_squares(const void* x, int64_t K, int L) {
    double s = 0.0;
    for (int64_t k = 4 * L; k < K; k += 256) {
        const float4 v = x4_value<XBF16>(load_x4_raw<XBF16>(x, k));
        s += (double)v.x * (double)v.x;
        s += (double)v.y * (double)v.y;
        s += (double)v.z * (double)v.z;
        s += (double)v.w * (double)v.w;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
    return s;
}

// Writes the block's outputs from the row sum `sum` = c_n . x of lane L's row
// (ssq: sum_k x[k]^2 when have_ssq, else taken here): v = scale * sum
// (divided by the RMS of x when the item asks for an RMS-normalised input),
// then y = fl32(v) (store), y = fl32(y + v) (residual add) or, for rows
// interleaved 32 gate / 32 up per block, one output per pair:
// fl32(silu(gate) * up) with silu(t) = t / (1 + e^-t), all in fp64.
template <bool XBF16, bool EPI>
// `scale` and `y_old` are the row's scale and, when adding, its y before the
// launch (loaded by the caller, ahead of the split-K hand-off where it has one).
__device__ __forceinline__ void finish(const Item& a, int b, int L, double sum, bool have_ssq, double ssq, float scale,
                                       float y_old) {
    const int row = b * kRows + L;
    double v = (double)scale * sum;
    if (EPI && a.rms) {
        const double ss = have_ssq ? ssq : sum_squares<XBF16>(a.x, a.K, L);
        v = v / sqrt(ss / (double)a.K + a.eps);
    }
    if (EPI && a.out_mode == QAM_OUT_GLU) {
        const double up = __shfl(v, (L + 32) & 63);
        if (L < 32) a.y[b * 32 + L] = (float)(v / (1.0 + exp(-v)) * up);
    } else if (EPI && a.out_mode == QAM_OUT_ADD) {
        a.y[row] = (float)((double)y_old + v);
    } else {
        a.y[row] = (float)v;
    }
}

// A ZERO block: every row's sum is 0, so y = 0 (store), y unchanged (add) or
// silu(0) * 0 = 0 (gated pairs); nothing of the block is read.
template <bool EPI>
__device__ __forceinline__ void finish_zero(const Item& a, int b, int L) {
    if (EPI && a.out_mode == QAM_OUT_ADD) return;
    if (EPI && a.out_mode == QAM_OUT_GLU) {
        if (L < 32) a.y[b * 32 + L] = 0.0f;
    } else {
        a.y[(int64_t)b * kRows + L] = 0.0f;
    }
}

// One wavefront: block b, column chunk `chunk`, read at NS slices.  The chunk
// is walked in sub-chunks of kStageTiles tiles; each sub-chunk's exact
// integer sums are scaled into a per-row fp64 sum (exact but for fp64
// rounding across sub-chunks, in a fixed order).
template <int NS, bool XBF16, bool EPI>
__device__ __forceinline__ void wave_body(const Item& a, const Common& c, int4* __restrict__ lds, int b, int chunk,
                                          int L, int ks, int KS, double* red, unsigned long long* tl_row) {
    (void)tl_row;
    QAM_STAMP(1);
    constexpr int H = Ring<NS>::H;
    constexpr int PF = Ring<NS>::PF;
    constexpr int S = kStageTiles;
    constexpr int G = kStageGroups;
    const int tile0 = chunk * a.tpc;
    // the chunk's tiles ks, ks + KS, ... are this wave's (KS waves share a chunk)
    const int ntile_all = min(a.tpc, a.n_tiles - tile0);
    const int ntile = ntile_all > ks ? (ntile_all - ks + KS - 1) / KS : 0;
    const int64_t tstride = (int64_t)KS * kTileBytes;
    const uint8_t* base0 = a.planes + (int64_t)b * 16 * a.K + (int64_t)(tile0 + ks) * kTileBytes + L * 16;
    const int kg = L >> 4;
    const int64_t pb = a.plane_bytes;

    // this lane's B-operand slot, and the zero slots of every tile (written
    // once; staging never touches them)
    const int bslot = 4 * ((L & 15) < kLimbCols ? (L & 15) : kLimbCols) + kg;
    if ((L >> 2) < S) lds[(L >> 2) * kSlotsPerTile + kZeroSlot + (L & 3)] = int4{0, 0, 0, 0};
    int* tab = reinterpret_cast<int*>(lds + S * kSlotsPerTile);   // [6][64 rows] sums of a sub-chunk

    double mine = 0.0;
    bool any_bad = false;
    bool fmode = false;   // this sub-chunk runs in fp32
    double ssq = 0.0;
    // an unsplit RMS-normalised product sees all of x while staging it
    const bool want_ssq = EPI && a.rms && a.n_chunks == 1;

    // x of sub-chunk `sub`, raw, G groups of four values per lane (lanes past
    // the sub-chunk reload its last group, never staged)
    u32x4 xraw[G];
    auto load_x = [&](int sub) {
        const int ngroups = min(S, ntile - sub * S) * 16;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int g = min(L + 64 * i, ngroups - 1);
            const int64_t col = (int64_t)(tile0 + ks + KS * (sub * S + (g >> 4))) * kTileCols + 4 * (g & 15);
            xraw[i] = load_x4_raw<XBF16>(a.x, col);
        }
    };
    int exp = 0;
    bool bad = false;
    auto stage = [&](int sub) {
        fmode = stage_limbs<XBF16>(xraw, min(S, ntile - sub * S) * 16, L, lds, exp, bad, want_ssq, ssq);
    };
    v4i macc[4];
    float facc[4];
    auto clear_acc = [&]() {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            macc[j] = v4i{0, 0, 0, 0};
            facc[j] = 0.0f;
        }
    };
    // The sub-chunk's exact per-row integers, scaled by its exponent into the
    // row's fp64 sum: the six limb columns of every row meet in LDS, then row
    // L's value forms on lane L.
    // In fp32: the four lane groups' partial sums of rows 16j + (L & 15) meet
    // by lane shuffles (in fp64) and lane L keeps row L's.
    auto flush = [&]() {
        if (fmode) {
            double d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                d[j] = (double)facc[j];
                d[j] += __shfl_xor(d[j], 16);
                d[j] += __shfl_xor(d[j], 32);
            }
            mine += kg == 0 ? d[0] : (kg == 1 ? d[1] : (kg == 2 ? d[2] : d[3]));
        } else {
            const int gc = L & 15;
            if (gc < kLimbCols) {
#pragma unroll
                for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(tab + gc * 64 + 16 * j + 4 * kg) = macc[j];
            }
            lds_order();
            mine += limb_value(tab[L], tab[64 + L], tab[128 + L], tab[192 + L], tab[256 + L], tab[320 + L], exp);
        }
        any_bad = any_bad || bad;
    };
#define QAM_TILE(BUF, TT)                                                                  \
    do {                                                                                   \
        if (fmode) tile_float<NS>(BUF, lds + (TT) * kSlotsPerTile + 4 * kg, facc);         \
        else tile_mfma<NS>(BUF, lds + (TT) * kSlotsPerTile, bslot, macc);                  \
    } while (0)
    // A half ring of H tiles, the sub-chunk's mode tested once: straight-line
    // matrix-core tiles accumulate in place (a test per tile made the compiler
    // copy the accumulators back after every tile)
#define QAM_HALF(BUF, TT)                                                                  \
    do {                                                                                   \
        if (fmode) {                                                                       \
            _Pragma("unroll") for (int u = 0; u < H; ++u)                                  \
                tile_float<NS>(BUF[u], lds + ((TT) + u) * kSlotsPerTile + 4 * kg, facc);   \
        } else {                                                                           \
            _Pragma("unroll") for (int u = 0; u < H; ++u)                                  \
                tile_mfma<NS>(BUF[u], lds + ((TT) + u) * kSlotsPerTile, bslot, macc);      \
        }                                                                                  \
    } while (0)

    // One prefetch ring runs through the whole chunk: two halves of H tiles,
    // each reloaded PF tiles ahead right after it is used.  A round that ends
    // a sub-chunk loads the next sub-chunk's x before its first reload and,
    // once its last tile is done, flushes the sums and stages the new limbs,
    // all inside the round (no x kept in registers from one round to the
    // next), so a sub-chunk boundary never drains the weight loads in flight.
    // Every wait below drains only the older half (and x loaded before it).
    static_assert(S % PF == 0, "sub-chunks hold whole ring rounds");
    if (ntile > 0) {
        const int last = ntile - 1;
        // nothing of this wave is in flight here: this wait is free, and it
        // keeps the compiler's wait counting exact through the loop below
        __builtin_amdgcn_s_waitcnt(0);
        load_x(0);
        u32x4 A[H][NS], Bh[H][NS];
        __builtin_amdgcn_sched_barrier(0);   // x loads go out first ...
        load_half<NS, H>(A, base0, pb, tstride, 0, last);
        __builtin_amdgcn_sched_barrier(0);   // ... then half a ring, and only then is x used
        stage(0);
        QAM_STAMP(2);
        load_half<NS, H>(Bh, base0, pb, tstride, H, last);
        __builtin_amdgcn_sched_barrier(0);
        clear_acc();
        int t = 0;
        // steady rounds: every tile of the round is in range and so is the next round's first
        for (; t + PF < ntile; t += PF) {
            const int tl = t % S;
            const bool ends_sub = tl + PF == S;
            if (ends_sub) load_x((t + PF) / S);
            __builtin_amdgcn_sched_barrier(0);
            QAM_HALF(A, tl);
            __builtin_amdgcn_sched_barrier(0);
            load_half<NS, H>(A, base0, pb, tstride, t + PF, last);
            __builtin_amdgcn_sched_barrier(0);
            QAM_HALF(Bh, tl + H);
            __builtin_amdgcn_sched_barrier(0);
            if (ends_sub) {
                flush();
                stage((t + PF) / S);
                clear_acc();
            }
            load_half<NS, H>(Bh, base0, pb, tstride, t + PF + H, last);   // past the end: clamped, never used
            __builtin_amdgcn_sched_barrier(0);
        }
        // the last round, possibly ragged
        const int tl = t % S;
#pragma unroll
        for (int u = 0; u < H; ++u)
            if (t + u < ntile) QAM_TILE(A[u], tl + u);
#pragma unroll
        for (int u = 0; u < H; ++u)
            if (t + H + u < ntile) QAM_TILE(Bh[u], tl + H + u);
        QAM_STAMP(3);
        flush();
        QAM_STAMP(4);
    }
#undef QAM_HALF
#undef QAM_TILE

    const int row = b * kRows + L;   // the row this lane writes
    double part = any_bad ? __builtin_nan("") : mine;   // non-finite x: NaN
    if (KS > 1) {   // the chunk's other waves hand over their row sums; wave 0 adds them in order
        if (ks > 0) {
            red[(ks * 2 + 0) * 64 + L] = part;
            red[(ks * 2 + 1) * 64 + L] = ssq;
        }
        __syncthreads();
        QAM_STAMP(5);
        if (ks > 0) return;
        for (int k2 = 1; k2 < KS; ++k2) {
            part += red[(k2 * 2 + 0) * 64 + L];
            ssq += red[(k2 * 2 + 1) * 64 + L];
        }
    }

    if (a.n_chunks == 1) {
        if (want_ssq) {
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) ssq += __shfl_xor(ssq, o);
        }
        finish<XBF16, EPI>(a, b, L, part, want_ssq, ssq, a.scales[row], EPI && a.out_mode == QAM_OUT_ADD ? a.y[row] : 0.0f);
        return;
    }
    // Split K: publish this chunk's partials, then count the arrival; the last
    // wave of the block sums the partials in chunk order.  The partials are
    // written and read with device-scope (write-through) atomic accesses and
    // the counter is bumped only after those stores have completed, so no
    // cache-wide writeback or invalidate is needed: a device-scope fence here
    // writes back and invalidates the whole L2 of the XCD, thousands of times
    // per launch.  The signal fences keep the compiler from moving the
    // partial stores past the counter update, and the partial loads ahead of
    // it (they emit no instruction).
    __hip_atomic_store(&a.partials[(int64_t)chunk * a.N + row], part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the row's scale and old y, in flight while the stores complete (no
    // other wave writes this row of y before the last arriver)
    const float scale = a.scales[row];
    const float y_old = EPI && a.out_mode == QAM_OUT_ADD ? a.y[row] : 0.0f;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);   // the partial stores are complete before the arrival is counted
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    uint32_t prev = 0;
    if (L == 0) prev = __hip_atomic_fetch_add(&a.counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0);
    QAM_STAMP(6);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (prev != (uint32_t)(a.n_chunks - 1)) return;
    // eight partial loads in flight at a time, added in chunk order
    double sum = 0.0;
    for (int c0 = 0; c0 < a.n_chunks; c0 += 8) {
        double pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            pv[j] = __hip_atomic_load(&a.partials[(int64_t)min(c0 + j, a.n_chunks - 1) * a.N + row], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (c0 + j < a.n_chunks) sum += pv[j];
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (L == 0) __hip_atomic_store(&a.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    finish<XBF16, EPI>(a, b, L, sum, false, ssq, scale, y_old);
}

// One (block, column chunk) unit of item a, `local` being its index within
// the item, run by c.KS wavefronts (at most MAXW); wave k takes the chunk's
// tiles k, k + KS, ...  With a lens map lm (one wavefront per unit), the
// block's rung comes from the lens rules and the chunk-0 unit writes it to
// the item's map; else it is read from the map (or fixed).  A rung above 4
// is not a depth of the product: the unit raises the item's status flag and
// writes NaN outputs (no read of its planes).
template <bool XBF16, int MAXW, bool EPI, bool LENS = false>
__device__ __forceinline__ void run_unit(const Item& a, const Common& c, int local, int4* lds, int tid,
                                         const LensMap* lm = nullptr, unsigned long long* tl_row = nullptr) {
    // per wave: kRegionInt4 int4 (the sub-chunk's limb words, then its column
    // sums); then, with several waves, [KS][2][64] fp64 row sums handed to wave 0
    const int KS = MAXW == 1 ? 1 : c.KS;
    const int ks = MAXW == 1 ? 0 : tid >> 6;
    int4* mylds = lds + ks * kRegionInt4;
    double* red = reinterpret_cast<double*>(lds + KS * kRegionInt4);
    const int chunk = local % a.n_chunks;
    const int b = local / a.n_chunks;
    const int L = tid & 63;
    int lev;
    if constexpr (LENS) {
        static_assert(MAXW == 1, "one wavefront per unit computes the rung");
        lev = lens_block_rung(a.coords, b, L, *lm);
        if (chunk == 0 && L == 0) const_cast<uint8_t*>(a.level)[b] = (uint8_t)lev;
    } else {
        lev = a.fixed_level >= 0 ? a.fixed_level : level_of(a.level, b);
    }
    const int ns = __builtin_amdgcn_readfirstlane(lev);
    switch (ns) {   // uniform over the workgroup: one block
        case 0:   // ZERO: nothing read, y = 0 (written once, by the first chunk's first wave)
            if (chunk == 0 && ks == 0) finish_zero<EPI>(a, b, L);
            return;
        case 1: wave_body<1, XBF16, EPI>(a, c, mylds, b, chunk, L, ks, KS, red, tl_row); return;
        case 2: wave_body<2, XBF16, EPI>(a, c, mylds, b, chunk, L, ks, KS, red, tl_row); return;
        case 3: wave_body<3, XBF16, EPI>(a, c, mylds, b, chunk, L, ks, KS, red, tl_row); return;
        case 4: wave_body<4, XBF16, EPI>(a, c, mylds, b, chunk, L, ks, KS, red, tl_row); return;
        default:   // not a rung of {0,2,4,6,8}: flag it, and write NaN once (no planes read)
            if (chunk == 0 && ks == 0) {
                if (L == 0 && c.status) __hip_atomic_fetch_or(c.status, (uint32_t)QAM_STATUS_BAD_RUNG, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT);
                if (!(EPI && a.out_mode == QAM_OUT_GLU)) a.y[(int64_t)b * kRows + L] = __builtin_nanf("");
                else if (L < 32) a.y[b * 32 + L] = __builtin_nanf("");
            }
            return;
    }
}

// The descriptor of grouped unit u.  The table and the unit map do not change
// while a launch runs, so they are read through the constant address space:
// scalar loads, even after the kernel has stored to global memory.
typedef __attribute__((address_space(4))) const int const_int;
__device__ __forceinline__ Item unit_item(const Common& c, int u) {
    static_assert(sizeof(Item) % 4 == 0, "descriptor in whole dwords");
    const int idx = *(const_int*)(c.wg_item + u);
    const const_u32* src = (const const_u32*)(c.items + idx);
    uint32_t w[sizeof(Item) / 4];
#pragma unroll
    for (int i = 0; i < (int)(sizeof(Item) / 4); ++i) w[i] = src[i];
    Item a;
    __builtin_memcpy(&a, w, sizeof(Item));
    return a;
}

// One workgroup per unit of a group (descriptor table, one lookup per
// workgroup; plain stores, the only output a group's items have).
template <bool XBF16, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void qmatvec_kernel(Common c) {
    extern __shared__ int4 lds[];
    const Item a = unit_item(c, (int)blockIdx.x);
    run_unit<XBF16, MAXW, false>(a, c, (int)blockIdx.x - a.wg_begin, lds, (int)threadIdx.x);
}

// One workgroup per unit of a single matrix, with its epilogue.  The fields
// the first loads depend on come first, as scalars (the rest of the
// descriptor follows by value): the compiler preloads them into scalar
// registers at wave launch (-amdgpu-kernarg-preload-count), so a short,
// dependent launch such as a decode step's issues its first loads without
// waiting for the argument segment.  tiles_tpc = n_tiles | tpc << 16;
// chunks_level_ks = n_chunks | (fixed_level + 1) << 16 | KS << 24.
template <bool XBF16, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void qmatvec_single_kernel(const void* x, const uint8_t* planes, int64_t K,
                                                                   int64_t plane_bytes, const int* run_if,
                                                                   uint32_t tiles_tpc, uint32_t chunks_level_ks,
                                                                   Item single, Common c) {
    extern __shared__ int4 lds[];
#ifdef QAM_TIMELINE
    const unsigned long long t_entry = (unsigned long long)wall_clock64();
#endif
    if (run_if != nullptr && *run_if == 0) return;   // predicated launch, not taken
    Item a = single;
    a.x = x;
    a.planes = planes;
    a.K = K;
    a.plane_bytes = plane_bytes;
    a.n_tiles = (int)(tiles_tpc & 0xFFFFu);
    a.tpc = (int)(tiles_tpc >> 16);
    a.n_chunks = (int)(chunks_level_ks & 0xFFFFu);
    a.fixed_level = (int)((chunks_level_ks >> 16) & 0xFFu) - 1;
    Common cc = c;
    cc.KS = (int)(chunks_level_ks >> 24);
    unsigned long long* tl_row = nullptr;
#ifdef QAM_TIMELINE
    for (int i = 0; i < QAM_TIMELINE_SLOTS; ++i)
        if (tl_select[i] != nullptr && tl_select[i] == (const void*)planes && blockIdx.x < QAM_TIMELINE_GROUPS)
            tl_row = &tl_stamps[i][blockIdx.x][0][0];
    const int tl_wave = (int)threadIdx.x >> 6;
    if (tl_row != nullptr && (threadIdx.x & 63) == 0) tl_row[tl_wave * QAM_TIMELINE_POINTS] = t_entry;
#endif
    run_unit<XBF16, MAXW, true>(a, cc, (int)blockIdx.x, lds, (int)threadIdx.x, nullptr, tl_row);
#ifdef QAM_TIMELINE
    if (tl_row != nullptr && (threadIdx.x & 63) == 0)
        tl_row[tl_wave * QAM_TIMELINE_POINTS + 7] = (unsigned long long)wall_clock64();
#endif
}

// A group whose maps are built in the same launch: every unit computes its
// block's rung from the lens map (kernel argument) before its planes.
template <bool XBF16>
__global__ __launch_bounds__(64) void qmatvec_lens_kernel(Common c, LensMap lm) {
    extern __shared__ int4 lds[];
    const Item a = unit_item(c, (int)blockIdx.x);
    run_unit<XBF16, 1, false, true>(a, c, (int)blockIdx.x - a.wg_begin, lds, (int)threadIdx.x, &lm);
}

// ------------------------------------------------------------------ host side

// Plan defaults of the staged-limb route (a group's qam_tuning may change them).
constexpr int64_t kTargetWaves = 256 * 32;   // wavefronts aimed for per launch
constexpr int kMaxChunkTiles = 64;           // longest column chunk (long waves leave a long tail)
constexpr int kTailPct = 15;                 // share of a group's block tiles planned with short chunks
constexpr int kTailDiv = 2;                  // how much shorter

// every chunk holds a whole number of prefetch rings (Ring<NS>::PF for every NS)
int tpc_align() { return 8; }
size_t lds_bytes_staged() { return (size_t)kRegionInt4 * sizeof(int4); }

// Column chunk length (in tiles) for a launch covering `block_tiles` block x
// tile pairs: enough chunks for about target_waves wavefronts of equal work,
// at most `cap` tiles (cap <= 0: no cap).
int chunk_goal(int64_t block_tiles, int64_t target_waves, int cap) {
    int64_t g = (block_tiles + target_waves - 1) / target_waves;
    if (cap > 0) g = std::min<int64_t>(g, cap);
    return (int)std::max<int64_t>(1, std::min<int64_t>(g, QAM_MAX_K / kTileCols));
}

int staged_goal(int64_t block_tiles, const qam_tuning* t) {
    const int64_t tw = t && t->target_waves > 0 ? t->target_waves : kTargetWaves;
    const int cap = t && t->max_chunk_tiles > 0 ? t->max_chunk_tiles : kMaxChunkTiles;
    return chunk_goal(block_tiles, tw, cap);
}

// Chunking of one matrix: K is cut into the fewest chunks of at most `goal`
// tiles, evened out and rounded up to a multiple of `align` tiles.
Plan make_plan(int64_t N, int64_t K, int goal, int align) {
    Plan p{};
    const int n_blocks = (int)(N / kRows);
    const int n_tiles = (int)(K / kTileCols);
    if (align <= 0) align = tpc_align();
    const int want = (n_tiles + goal - 1) / goal;
    int tpc = (n_tiles + want - 1) / want;
    tpc = (tpc + align - 1) / align * align;
    if (tpc > n_tiles) tpc = n_tiles;
    p.tpc = tpc;
    p.n_chunks = (n_tiles + tpc - 1) / tpc;
    p.n_quads = n_blocks;   // one wavefront-sized workgroup per block and chunk
    p.partial_bytes = p.n_chunks > 1 ? ((size_t)p.n_chunks * N * sizeof(double) + 255) / 256 * 256 : 0;
    return p;
}

// With events, the launch records them at the kernel's own start and end
// (hipExtLaunchKernel), which times the kernel alone.
template <int MAXW>
static void launch_group_k(const Common& c, int64_t grid, int threads, size_t lds, hipStream_t s,
                           hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
    const dim3 g((unsigned)grid), b((unsigned)threads);
    if (e0 || e1) {
        if (c.x_bf16)
            hipExtLaunchKernelGGL((qmatvec_kernel<true, MAXW>), g, b, (uint32_t)lds, s, e0, e1, 0u, c);
        else
            hipExtLaunchKernelGGL((qmatvec_kernel<false, MAXW>), g, b, (uint32_t)lds, s, e0, e1, 0u, c);
        return;
    }
    if (c.x_bf16)
        hipLaunchKernelGGL((qmatvec_kernel<true, MAXW>), g, b, lds, s, c);
    else
        hipLaunchKernelGGL((qmatvec_kernel<false, MAXW>), g, b, lds, s, c);
}

template <int MAXW>
static void launch_single_k(const Item& it, const Common& c, int64_t grid, int threads, size_t lds, hipStream_t s) {
    const uint32_t tiles_tpc = (uint32_t)it.n_tiles | ((uint32_t)it.tpc << 16);
    const uint32_t chunks_level_ks =
        (uint32_t)it.n_chunks | ((uint32_t)(it.fixed_level + 1) << 16) | ((uint32_t)c.KS << 24);
    const dim3 g((unsigned)grid), b((unsigned)threads);
    if (c.x_bf16)
        hipLaunchKernelGGL((qmatvec_single_kernel<true, MAXW>), g, b, lds, s, it.x, it.planes, it.K, it.plane_bytes,
                           it.run_if, tiles_tpc, chunks_level_ks, it, c);
    else
        hipLaunchKernelGGL((qmatvec_single_kernel<false, MAXW>), g, b, lds, s, it.x, it.planes, it.K, it.plane_bytes,
                           it.run_if, tiles_tpc, chunks_level_ks, it, c);
}

void launch_single(const Item& it, const Common& c, int64_t grid, hipStream_t s) {
    // the packed launch fields (16 bits each for tiles, tpc and chunks: K <= QAM_MAX_K)
    static_assert(QAM_MAX_K / kTileCols < 65536, "tile counts fit 16 bits");
    if (c.KS > 1) {   // several waves per (block, chunk)
        const size_t lds = (size_t)c.KS * lds_bytes_staged() + (size_t)c.KS * 2 * 64 * sizeof(double);
        launch_single_k<8>(it, c, grid, 64 * c.KS, lds, s);
        return;
    }
    launch_single_k<1>(it, c, grid, 64, lds_bytes_staged(), s);
}

// Host checks shared by the single and grouped entry points.
int check_item(const void* x, int x_dtype, int64_t B, const qam_packed* packed, const uint8_t* level_map,
               float* y, const char* who, int out_mode) {
    if (!x || !packed || !level_map || !y || !packed->planes) QAM_FAIL(QAM_ERR_NULL, "%s: null pointer", who);
    const int64_t N = packed->N, K = packed->K;
    if (N <= 0 || K <= 0 || N % kRows || K % kTileCols || K > QAM_MAX_K || packed->n_blocks != N / kRows ||
        packed->n_blocks > QAM_MAX_BLOCKS)
        QAM_FAIL(QAM_ERR_SHAPE, "%s: bad packed shape N=%lld K=%lld", who, (long long)N, (long long)K);
    if (B < 1 || B > QAM_MAX_BATCH_MFMA)
        QAM_FAIL(QAM_ERR_ARG, "%s: B=%lld outside [1, %d]", who, (long long)B, QAM_MAX_BATCH_MFMA);
    if (x_dtype != QAM_X_F32 && x_dtype != QAM_X_BF16) QAM_FAIL(QAM_ERR_ARG, "%s: unknown x_dtype %d", who, x_dtype);
    if (!aligned(x, 16) || !aligned(y, 4) || !aligned(packed->planes, 256))
        QAM_FAIL(QAM_ERR_ALIGN, "%s: x must be 16-byte and planes 256-byte aligned", who);
    if (packed->scales != reinterpret_cast<float*>(static_cast<char*>(packed->planes) + N * K))
        QAM_FAIL(QAM_ERR_ARG, "%s: descriptor scales do not follow the planes", who);
    const size_t xbytes = (size_t)B * K * (x_dtype == QAM_X_BF16 ? 2 : 4);
    const char* xc = static_cast<const char*>(x);
    const char* yc = reinterpret_cast<const char*>(y);
    const size_t ybytes = (size_t)B * (out_mode == QAM_OUT_GLU ? N / 2 : N) * 4;
    if (xc < yc + ybytes && yc < xc + xbytes) QAM_FAIL(QAM_ERR_ARG, "%s: x and y overlap", who);
    return QAM_OK;
}

// The workspace of one call: counters and the status word first, then the
// route's own buffers.
int check_workspace(void* workspace, size_t workspace_bytes, size_t need, const char* who) {
    if (!workspace) QAM_FAIL(QAM_ERR_WORKSPACE, "%s: workspace of %zu bytes required", who, need);
    if (workspace_bytes < need) QAM_FAIL(QAM_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, workspace_bytes, need);
    if (!aligned(workspace, 256)) QAM_FAIL(QAM_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
    return QAM_OK;
}

uint32_t* status_word(void* counter_region) {
    return reinterpret_cast<uint32_t*>(static_cast<char*>(counter_region) + QAM_WS_STATUS_OFFSET);
}

Item make_item(const void* x, const qam_packed* packed, const uint8_t* level_map, float* y, const Plan& p) {
    Item it{};
    it.planes = static_cast<const uint8_t*>(packed->planes);
    it.scales = packed->scales;
    it.x = x;
    it.y = y;
    it.level = level_map;
    it.plane_bytes = packed->N * packed->K / 4;
    it.N = packed->N;
    it.K = packed->K;
    it.n_blocks = (int)(packed->N / kRows);
    it.n_tiles = (int)(packed->K / kTileCols);
    it.tpc = p.tpc;
    it.n_chunks = p.n_chunks;
    it.n_quads = p.n_quads;
    it.fixed_level = -1;
    return it;
}

bool mfma_route(int64_t B) { return B > 1; }

}  // namespace qam

using namespace qam;

extern "C" size_t qam_qmatvec_workspace_bytes(int64_t N, int64_t K, int64_t B) {
    if (N <= 0 || K <= 0 || N % kRows || K % kTileCols || K > QAM_MAX_K || N / kRows > QAM_MAX_BLOCKS || B < 1 ||
        B > QAM_MAX_BATCH_MFMA)
        return 0;
    if (mfma_route(B)) return qam_mfma_workspace_bytes(N, K, B);   // the pre-pass route
    const Plan p = make_plan(N, K, staged_goal(N / kRows * (K / kTileCols), nullptr));
    return QAM_WS_COUNTER_BYTES + p.partial_bytes;
}

extern "C" int qam_status(const void* workspace, int clear, uint32_t* status_out, hipStream_t s) {
    clear_error();
    if (!workspace || !status_out) QAM_FAIL(QAM_ERR_NULL, "status: null pointer");
    if (clear != 0 && clear != 1) QAM_FAIL(QAM_ERR_ARG, "status: clear must be 0 or 1");
    uint32_t* w = status_word(const_cast<void*>(workspace));
    QAM_HIP_CHECK(hipMemcpyAsync(status_out, w, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
    if (clear) QAM_HIP_CHECK(hipMemsetAsync(w, 0, sizeof(uint32_t), s));
    QAM_HIP_CHECK(hipStreamSynchronize(s));
    return QAM_OK;
}

static int check_epilogue(const qam_epilogue* ep, const char* who) {
    if (!ep) return QAM_OK;
    if (ep->rms_norm != 0 && ep->rms_norm != 1) QAM_FAIL(QAM_ERR_ARG, "%s: rms_norm must be 0 or 1", who);
    if (ep->out_mode != QAM_OUT_STORE && ep->out_mode != QAM_OUT_ADD && ep->out_mode != QAM_OUT_GLU)
        QAM_FAIL(QAM_ERR_ARG, "%s: unknown out_mode %d", who, ep->out_mode);
    if (!(ep->eps >= 0.0) || ep->eps > 1e300) QAM_FAIL(QAM_ERR_ARG, "%s: eps must be finite and >= 0", who);
    return QAM_OK;
}

extern "C" int qam_qmatvec_ep(const void* x, int x_dtype, int64_t B, const qam_packed* packed,
                              const uint8_t* level_map, const qam_epilogue* ep, float* y, void* workspace,
                              size_t workspace_bytes, hipStream_t s) {
    clear_error();
    if (int rc = check_epilogue(ep, "qmatvec")) return rc;
    const int out_mode = ep ? ep->out_mode : QAM_OUT_STORE;
    if (int rc = check_item(x, x_dtype, B, packed, level_map, y, "qmatvec", out_mode)) return rc;
    if (B != 1) QAM_FAIL(QAM_ERR_ARG, "qmatvec_ep: B=%lld; the fused epilogues take one request", (long long)B);
    const Plan p = make_plan(packed->N, packed->K, staged_goal(packed->n_blocks * (packed->K / kTileCols), nullptr));
    if (int rc = check_workspace(workspace, workspace_bytes, QAM_WS_COUNTER_BYTES + p.partial_bytes, "qmatvec"))
        return rc;
    Item it = make_item(x, packed, level_map, y, p);
    if (ep) {
        it.rms = ep->rms_norm;
        it.out_mode = ep->out_mode;
        it.eps = ep->eps;
    }
    it.counters = static_cast<uint32_t*>(workspace);
    if (p.n_chunks > 1) it.partials = reinterpret_cast<double*>(static_cast<char*>(workspace) + QAM_WS_COUNTER_BYTES);
    Common c{};
    c.B = 1;
    c.x_bf16 = x_dtype == QAM_X_BF16;
    c.KS = 1;
    c.status = status_word(workspace);
    launch_single(it, c, (int64_t)p.n_chunks * p.n_quads, s);
    QAM_HIP_CHECK(hipGetLastError());
    char v[128];
    snprintf(v, sizeof(v), "qmatvec_staged B=1 tpc=%d chunks=%d", p.tpc, p.n_chunks);
    set_variant(v);
    return QAM_OK;
}

extern "C" int qam_qmatvec(const void* x, int x_dtype, int64_t B, const qam_packed* packed, const uint8_t* level_map,
                           int per_request_maps, float* y, void* workspace, size_t workspace_bytes, hipStream_t s) {
    clear_error();
    if (per_request_maps != 0 && per_request_maps != 1) QAM_FAIL(QAM_ERR_ARG, "qmatvec: per_request_maps must be 0 or 1");
    if (!mfma_route(B))
        return qam_qmatvec_ep(x, x_dtype, B, packed, level_map, nullptr, y, workspace, workspace_bytes, s);
    if (int rc = check_item(x, x_dtype, B, packed, level_map, y, "qmatvec", QAM_OUT_STORE)) return rc;
    return qmatvec_mfma(x, x_dtype, B, packed, level_map, per_request_maps, y, workspace, workspace_bytes, s);
}

// ------------------------------------------------------------------ grouped launches

namespace qam {

struct GroupLayout {
    std::vector<Plan> plans;
    size_t partial_bytes = 0, table_bytes = 0, map_bytes = 0, total = 0;
    int64_t n_wg = 0, blocks = 0, block_tiles = 0;
};

static int check_tuning(const qam_tuning* t, const char* who) {
    if (!t) return QAM_OK;
    if (t->target_waves < 0 || t->target_waves > (1 << 20) || (t->target_waves > 0 && t->target_waves < 64))
        QAM_FAIL(QAM_ERR_ARG, "%s: target_waves %d not 0 or in [64, 2^20]", who, t->target_waves);
    if (t->max_chunk_tiles < 0 || t->max_chunk_tiles > QAM_MAX_K / kTileCols)
        QAM_FAIL(QAM_ERR_ARG, "%s: max_chunk_tiles %d outside [0, %d]", who, t->max_chunk_tiles, QAM_MAX_K / kTileCols);
    if (t->tail_pct < -1 || t->tail_pct > 100 || t->tail_div < 0 || t->tail_div > 64)
        QAM_FAIL(QAM_ERR_ARG, "%s: tail_pct %d / tail_div %d out of range", who, t->tail_pct, t->tail_div);
    if (t->ksplit != 0 && t->ksplit != 1 && t->ksplit != 2 && t->ksplit != 4)
        QAM_FAIL(QAM_ERR_ARG, "%s: ksplit %d not 0, 1, 2 or 4", who, t->ksplit);
    if (t->set_max != 0 && (t->set_max < 8 || t->set_max > 16))
        QAM_FAIL(QAM_ERR_ARG, "%s: set_max %d not 0 or in [8, 16]", who, t->set_max);
    if (t->tiles_per_request < 0 || t->tiles_per_request > 64)
        QAM_FAIL(QAM_ERR_ARG, "%s: tiles_per_request %d outside [0, 64]", who, t->tiles_per_request);
    return QAM_OK;
}

static int layout_group(const qam_gemv_item* items, int n_items, const qam_tuning* tun, GroupLayout& g) {
    if (!items || n_items < 1) QAM_FAIL(QAM_ERR_ARG, "group: need at least one item");
    for (int i = 0; i < n_items; ++i) {
        const qam_packed& w = items[i].w;
        if (w.N <= 0 || w.N % kRows || w.K <= 0 || w.K % kTileCols || w.K > QAM_MAX_K)
            QAM_FAIL(QAM_ERR_SHAPE, "group: item %d has a bad shape", i);
        g.blocks += w.N / kRows;
        g.block_tiles += w.N / kRows * (w.K / kTileCols);
    }
    if (g.blocks > QAM_MAX_BLOCKS) QAM_FAIL(QAM_ERR_SHAPE, "group: %lld blocks > %d", (long long)g.blocks, QAM_MAX_BLOCKS);
    // Items are dispatched in order, so the last ones run while the chip
    // drains: those covering the last tail_pct percent of the block tiles
    // take chunks tail_div times shorter, so that the final wavefronts are short.
    const int goal = staged_goal(g.block_tiles, tun);
    const int tail_pct = tun && tun->tail_pct != 0 ? std::max(0, tun->tail_pct) : kTailPct;
    const int tail_div = tun && tun->tail_div > 0 ? tun->tail_div : kTailDiv;
    int64_t before = 0;
    for (int i = 0; i < n_items; ++i) {
        const int64_t bt = items[i].w.N / kRows * (items[i].w.K / kTileCols);
        const bool tail = tail_pct > 0 && (before + bt) * 100 > g.block_tiles * (100 - tail_pct);
        before += bt;
        const Plan p = make_plan(items[i].w.N, items[i].w.K, tail ? std::max(1, goal / tail_div) : goal);
        g.plans.push_back(p);
        g.partial_bytes += p.partial_bytes;
        g.n_wg += (int64_t)p.n_chunks * p.n_quads;
    }
    if (g.n_wg > 0x7FFFFFFF) QAM_FAIL(QAM_ERR_SHAPE, "group: too many workgroups");
    g.table_bytes = ((size_t)n_items * sizeof(Item) + 255) / 256 * 256;
    g.map_bytes = ((size_t)g.n_wg * sizeof(int) + 255) / 256 * 256;
    g.total = QAM_WS_COUNTER_BYTES + g.partial_bytes + g.table_bytes + g.map_bytes;
    return QAM_OK;
}

}  // namespace qam

extern "C" size_t qam_group_bytes_tuned(const qam_gemv_item* items, int n_items, int64_t B, int per_request_maps,
                                        const qam_tuning* tuning) {
    if (per_request_maps != 0 && per_request_maps != 1) return 0;
    if (check_tuning(tuning, "group_bytes") != QAM_OK) return 0;
    if (B < 1 || B > QAM_MAX_BATCH_MFMA) return 0;
    if (mfma_route(B)) return mfma_group_bytes(items, n_items, B, tuning);
    GroupLayout g;
    if (layout_group(items, n_items, tuning, g) != QAM_OK) return 0;
    return g.total;
}

extern "C" size_t qam_group_bytes(const qam_gemv_item* items, int n_items, int64_t B, int per_request_maps) {
    return qam_group_bytes_tuned(items, n_items, B, per_request_maps, nullptr);
}

extern "C" int qam_group_init_tuned(const qam_gemv_item* items, int n_items, int64_t B, int x_dtype,
                                    int per_request_maps, const qam_tuning* tuning, void* dev_mem, size_t dev_bytes,
                                    qam_group* group_out, hipStream_t s) {
    clear_error();
    if (!group_out || !dev_mem) QAM_FAIL(QAM_ERR_NULL, "group_init: null pointer");
    if (per_request_maps != 0 && per_request_maps != 1) QAM_FAIL(QAM_ERR_ARG, "group_init: per_request_maps must be 0 or 1");
    if (int rc = check_tuning(tuning, "group_init")) return rc;
    if (B < 1 || B > QAM_MAX_BATCH_MFMA) QAM_FAIL(QAM_ERR_ARG, "group_init: B=%lld outside [1, %d]", (long long)B,
                                                  QAM_MAX_BATCH_MFMA);
    if (mfma_route(B))
        return mfma_group_init(items, n_items, B, x_dtype, per_request_maps, tuning, dev_mem, dev_bytes, group_out, s);
    GroupLayout g;
    if (int rc = layout_group(items, n_items, tuning, g)) return rc;
    if (dev_bytes < g.total) QAM_FAIL(QAM_ERR_WORKSPACE, "group_init: %zu < %zu bytes", dev_bytes, g.total);
    if (!aligned(dev_mem, 256)) QAM_FAIL(QAM_ERR_ALIGN, "group_init: device memory must be 256-byte aligned");
    char* base = static_cast<char*>(dev_mem);
    char* partials = base + QAM_WS_COUNTER_BYTES;
    char* table = partials + g.partial_bytes;
    char* wgmap = table + g.table_bytes;
    std::vector<Item> host_items(n_items);
    std::vector<int> host_map((size_t)g.n_wg);
    int lens_ready = 1;
    int64_t wg = 0, blk = 0;
    size_t poff = 0;
    for (int i = 0; i < n_items; ++i) {
        const qam_gemv_item& gi = items[i];
        if (int rc = check_item(gi.x, x_dtype, B, &gi.w, gi.level_map, gi.y, "group_init", QAM_OUT_STORE)) return rc;
        const Plan& p = g.plans[i];
        Item it = make_item(gi.x, &gi.w, gi.level_map, gi.y, p);
        it.wg_begin = (int)wg;
        it.coords = gi.coords;
        if (!gi.coords) lens_ready = 0;
        else if (!aligned(gi.coords, 8)) QAM_FAIL(QAM_ERR_ALIGN, "group_init: item %d coords not 8-byte aligned", i);
        if (p.n_chunks > 1) {
            it.counters = reinterpret_cast<uint32_t*>(base) + blk;
            it.partials = reinterpret_cast<double*>(partials + poff);
            poff += p.partial_bytes;
        }
        blk += it.n_blocks;
        const int64_t n = (int64_t)p.n_chunks * p.n_quads;
        for (int64_t k = 0; k < n; ++k) host_map[(size_t)(wg + k)] = i;
        wg += n;
        host_items[i] = it;
    }
    QAM_HIP_CHECK(hipMemsetAsync(base, 0, QAM_WS_COUNTER_BYTES, s));
    QAM_HIP_CHECK(hipMemcpyAsync(table, host_items.data(), sizeof(Item) * n_items, hipMemcpyHostToDevice, s));
    QAM_HIP_CHECK(hipMemcpyAsync(wgmap, host_map.data(), sizeof(int) * host_map.size(), hipMemcpyHostToDevice, s));
    QAM_HIP_CHECK(hipStreamSynchronize(s));
    *group_out = qam_group{};
    group_out->n_items = n_items;
    group_out->B = B;
    group_out->x_dtype = x_dtype;
    group_out->n_workgroups = g.n_wg;
    group_out->lds_bytes = lds_bytes_staged();
    group_out->table = table;
    group_out->wg_map = wgmap;
    group_out->route = 0;
    group_out->per_request_maps = 0;
    group_out->lens_ready = lens_ready;
    group_out->dev_mem = dev_mem;
    return QAM_OK;
}

extern "C" int qam_group_init(const qam_gemv_item* items, int n_items, int64_t B, int x_dtype, int per_request_maps,
                              void* dev_mem, size_t dev_bytes, qam_group* group_out, hipStream_t s) {
    return qam_group_init_tuned(items, n_items, B, x_dtype, per_request_maps, nullptr, dev_mem, dev_bytes, group_out, s);
}

namespace qam {

static Common staged_common(const qam_group* group) {
    Common c{};
    c.items = static_cast<const Item*>(group->table);
    c.wg_item = static_cast<const int*>(group->wg_map);
    c.B = 1;
    c.x_bf16 = group->x_dtype == QAM_X_BF16;
    c.KS = 1;
    c.status = status_word(group->dev_mem);
    return c;
}

// Checks of a group and its lens rules for a launch that builds the maps;
// fills the launch arguments.
static int lens_group_setup(const qam_group* group, const qam_lens* lenses, int n_lenses,
                            const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs, int glass,
                            Common& c, LensMap& lm, const char* who) {
    if (!group || !group->table || !group->wg_map || !group->dev_mem) QAM_FAIL(QAM_ERR_NULL, "%s: uninitialised group", who);
    if (!params || !ladder_bits) QAM_FAIL(QAM_ERR_NULL, "%s: null params/ladder", who);
    if (group->route != 0 || group->B != 1 || group->n_workgroups < 1)
        QAM_FAIL(QAM_ERR_ARG, "%s: the map is built in the launch for one request (the staged-limb route)", who);
    if (!group->lens_ready) QAM_FAIL(QAM_ERR_ARG, "%s: the group's items have no block coordinates", who);
    if (int rc = lens_check_product_ladder(ladder_bits, n_rungs, glass, who)) return rc;
    lm = LensMap{};
    if (int rc = lens_check_map(lenses, n_lenses, params, n_rungs, glass, lm.p, who)) return rc;
    for (int i = 0; i < n_lenses; ++i) {
        lm.t.cx[i] = lenses[i].cx;
        lm.t.cy[i] = lenses[i].cy;
        lm.t.R[i] = lens_radius(*params, lenses[i].r, params->f);
    }
    lm.glass = glass;
    c = staged_common(group);
    return QAM_OK;
}

static void launch_lens(const qam_group* group, const Common& c, const LensMap& lm, hipStream_t s,
                        hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
    const dim3 g((unsigned)group->n_workgroups), b(64u);
    const uint32_t lds = (uint32_t)group->lds_bytes;
    if (c.x_bf16)
        hipExtLaunchKernelGGL((qmatvec_lens_kernel<true>), g, b, lds, s, e0, e1, 0u, c, lm);
    else
        hipExtLaunchKernelGGL((qmatvec_lens_kernel<false>), g, b, lds, s, e0, e1, 0u, c, lm);
}

}  // namespace qam

extern "C" int qam_qmatvec_group_lens(const qam_group* group, const qam_lens* lenses, int n_lenses,
                                      const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs,
                                      int glass, hipStream_t s) {
    clear_error();
    Common c;
    LensMap lm;
    if (int rc = lens_group_setup(group, lenses, n_lenses, params, ladder_bits, n_rungs, glass, c, lm,
                                  "qmatvec_group_lens"))
        return rc;
    launch_lens(group, c, lm, s);
    QAM_HIP_CHECK(hipGetLastError());
    char v[128];
    snprintf(v, sizeof(v), "qmatvec_staged_group_lens items=%d B=1 wg=%lld", group->n_items,
             (long long)group->n_workgroups);
    set_variant(v);
    return QAM_OK;
}

// Runs `n` launches back to back on `s`, each timed by HIP events it records
// at the kernel's own start and end; writes the n durations (ms) and
// synchronises `s`.
template <typename F>
static int time_launches(int n, float* ms_out, hipStream_t s, F launch_one, const char* who) {
    if (!ms_out) QAM_FAIL(QAM_ERR_NULL, "%s: null output", who);
    if (n < 1 || n > 4096) QAM_FAIL(QAM_ERR_ARG, "%s: n=%d outside [1, 4096]", who, n);
    std::vector<hipEvent_t> ev((size_t)2 * n, nullptr);
    hipError_t e = hipSuccess;
    for (size_t i = 0; i < ev.size() && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
    for (int i = 0; i < n && e == hipSuccess; ++i) {
        launch_one(ev[2 * i], ev[2 * i + 1]);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    for (int i = 0; i < n && e == hipSuccess; ++i) e = hipEventElapsedTime(&ms_out[i], ev[2 * i], ev[2 * i + 1]);
    for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
    if (e != hipSuccess) QAM_FAIL(QAM_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
    return QAM_OK;
}

// Benchmark hook: qam_qmatvec_group_lens run `n` times back to back on `s`,
// each launch timed as by qam_group_launch_times.
extern "C" int qam_group_lens_launch_times(const qam_group* group, const qam_lens* lenses, int n_lenses,
                                           const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs,
                                           int glass, int n, float* ms_out, hipStream_t s) {
    clear_error();
    Common c;
    LensMap lm;
    if (int rc = lens_group_setup(group, lenses, n_lenses, params, ladder_bits, n_rungs, glass, c, lm,
                                  "group_lens_launch_times"))
        return rc;
    return time_launches(n, ms_out, s, [&](hipEvent_t e0, hipEvent_t e1) { launch_lens(group, c, lm, s, e0, e1); },
                         "group_lens_launch_times");
}

static int staged_group_ok(const qam_group* group, const char* who) {
    if (!group || !group->table || !group->wg_map || !group->dev_mem) QAM_FAIL(QAM_ERR_NULL, "%s: uninitialised group", who);
    if (group->route != 0 || group->B != 1 || group->n_workgroups < 1)
        QAM_FAIL(QAM_ERR_ARG, "%s: not a staged-limb group (corrupt descriptor?)", who);
    return QAM_OK;
}

// Benchmark hook: runs a staged-limb group `n` times back to back on `s`,
// timing each launch with HIP events recorded at the kernel's own start and
// end; writes the n durations (ms) and synchronises `s`.
extern "C" int qam_group_launch_times(const qam_group* group, int n, float* ms_out, hipStream_t s) {
    clear_error();
    if (int rc = staged_group_ok(group, "group_launch_times")) return rc;
    const Common c = staged_common(group);
    return time_launches(n, ms_out, s, [&](hipEvent_t e0, hipEvent_t e1) {
        launch_group_k<1>(c, group->n_workgroups, 64, group->lds_bytes, s, e0, e1);
    }, "group_launch_times");
}

extern "C" int qam_qmatvec_group(const qam_group* group, hipStream_t s) {
    clear_error();
    if (!group || !group->table || !group->wg_map) QAM_FAIL(QAM_ERR_NULL, "qmatvec_group: uninitialised group");
    if (group->route == 1) {
        if (!group->pre_map || group->B < 2 || group->B > QAM_MAX_BATCH_MFMA || group->n_workgroups < 1)
            QAM_FAIL(QAM_ERR_ARG, "qmatvec_group: corrupt group descriptor");
        return mfma_group_run(group, s);
    }
    if (int rc = staged_group_ok(group, "qmatvec_group")) return rc;
    const Common c = staged_common(group);
    launch_group_k<1>(c, group->n_workgroups, 64, group->lds_bytes, s);
    QAM_HIP_CHECK(hipGetLastError());
    char v[128];
    snprintf(v, sizeof(v), "qmatvec_staged_group items=%d B=1 wg=%lld", group->n_items, (long long)group->n_workgroups);
    set_variant(v);
    return QAM_OK;
}

extern "C" int qam_timeline_select(const void* const* planes, int n) {
    clear_error();
#ifdef QAM_TIMELINE
    if (n < 0 || n > QAM_TIMELINE_SLOTS) QAM_FAIL(QAM_ERR_ARG, "timeline_select: n=%d outside [0, %d]", n, QAM_TIMELINE_SLOTS);
    if (n > 0 && !planes) QAM_FAIL(QAM_ERR_NULL, "timeline_select: null planes");
    const void* h[QAM_TIMELINE_SLOTS] = {};
    for (int i = 0; i < n; ++i) h[i] = planes[i];
    QAM_HIP_CHECK(hipDeviceSynchronize());
    QAM_HIP_CHECK(hipMemcpyToSymbol(HIP_SYMBOL(qam::tl_select), h, sizeof h));
    static const unsigned long long zero[QAM_TIMELINE_GROUPS * 8 * QAM_TIMELINE_POINTS] = {};
    for (int i = 0; i < QAM_TIMELINE_SLOTS; ++i)
        QAM_HIP_CHECK(hipMemcpyToSymbol(HIP_SYMBOL(qam::tl_stamps), zero, sizeof zero, i * sizeof zero));
    return QAM_OK;
#else
    (void)planes;
    (void)n;
    QAM_FAIL(QAM_ERR_ARG, "timeline_select: this library was built without the timeline (QAM_TIMELINE)");
#endif
}

extern "C" int qam_timeline_read(uint64_t* out, size_t n_words) {
    clear_error();
#ifdef QAM_TIMELINE
    const size_t words = (size_t)QAM_TIMELINE_SLOTS * QAM_TIMELINE_GROUPS * 8 * QAM_TIMELINE_POINTS;
    if (!out) QAM_FAIL(QAM_ERR_NULL, "timeline_read: null output");
    if (n_words < words) QAM_FAIL(QAM_ERR_ARG, "timeline_read: %zu words < %zu", n_words, words);
    QAM_HIP_CHECK(hipDeviceSynchronize());
    QAM_HIP_CHECK(hipMemcpyFromSymbol(out, HIP_SYMBOL(qam::tl_stamps), words * sizeof(uint64_t)));
    return QAM_OK;
#else
    (void)out;
    (void)n_words;
    QAM_FAIL(QAM_ERR_ARG, "timeline_read: this library was built without the timeline (QAM_TIMELINE)");
#endif
}
