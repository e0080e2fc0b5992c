// Mixed-depth matrix-vector / small-batch product over the slice planes
// (the staged-limb route: up to 8 requests sharing one level map).
//
// Each block of 64 output rows is read at its own depth straight from the
// stored bytes inside the pass ("FoQLens", table "Progress"); a block read at
// d bits touches d/2 slice planes, a ZERO block nothing.  Cost is the weight
// bytes read ("Precision on Demand", abstract).
//
// Work decomposition.  A workgroup is one wavefront (or, for batch 1, up to
// eight splitting a chunk's tiles) and takes one block of 64 rows and one
// chunk of columns (tiles_per_chunk tiles of 64).  The wave walks its chunk in
// sub-chunks of 16, 8 or 4 tiles (by batch); the ring of weight loads runs
// through the whole chunk, and each sub-chunk's x is turned into an exact
// fixed-point form in LDS:
//     v_k = rint(x_k * 2^(22-e)),   2^(e-1) <= max_sub-chunk |x| < 2^e,
// held as three signed int8 limbs v_k = sum_l s_l 256^l (balanced digits).
// Each lane owns, per 64-column tile and per slice, one 16-byte word group
// covering 4 rows x 16 columns; codes are rebuilt in registers (one mask per
// slice and one rotate per four codes) and multiplied into the limbs exactly,
// in int32, with v_mfma_i32_16x16x64_i8 on the matrix cores: the rebuilt
// words are the A operand as they stand, and B-operand column 3 r + l holds
// limb l of request r (the dot4 form, v_dot4_i32_i8 on the vector ALUs,
// reaches the same integers).  The limb sums are combined into an exact
// integer per row, request and sub-chunk, scaled by 2^(e-22) into an fp64 row
// sum, and either written as the output (one chunk) or stored as a partial;
// the last wavefront of a block to finish sums the partials in chunk order and
// writes y = fl32(scale * sum).  No floating-point atomics: results are
// bit-reproducible, and the two inner products give the same bits.
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

// ------------------------------------------------------------------ x staging

// LDS index (in 16-byte units) of the limb words of 4-column group g of the
// sub-chunk: tile g/16, then the group's position u in the lane's 16 columns,
// then the lane group (L >> 4) that owns it, so that the four lane groups
// reading one u hit four consecutive 16-byte slots.
__device__ __forceinline__ int limb_slot(int g) { return (g & ~15) | ((g & 3) << 2) | ((g >> 2) & 3); }

// ------------------------------------------------------------------ per-wave body

// x is staged in sub-chunks of S tiles (the same for both inner products, so
// that they reach the same integers): each lane loads G = S / 4 groups of four
// values per request.  S is a multiple of every ring length used with NB.
template <int NB>
struct Stage {
    static constexpr int S = NB <= 2 ? 16 : (NB <= 5 ? 8 : 4);
    static constexpr int G = S / 4;
};

// Prefetch ring: two halves of H tiles each, up to sixteen 16-byte loads in
// flight per lane (fewer when a dot4 form's per-request accumulators take the
// registers, or beyond four requests on the matrix cores).  The wait before
// one half is computed always follows the reload of the other half, so it
// drains exactly the older half.
template <int NS, int NB, bool MF>
struct Ring {
    static constexpr int raw = MF ? (NB <= 4 ? 8 : 4) / NS : (NB == 1 ? 8 : 4) / (NS * NB);
    static constexpr int Hr = raw >= 4 ? 4 : (raw >= 2 ? 2 : 1);
    static constexpr int H = Hr > Stage<NB>::S / 2 ? Stage<NB>::S / 2 : Hr;   // tiles per half
    static constexpr int PF = 2 * H;                                           // tiles per ring
};

// Matrix-core limb layout for NB requests: B-operand column 3 r + l holds
// limb l of request r, in NCG groups of 16 columns.  Per tile and group there
// is one 16-byte slot per (real column c, lane group k), at 4 c + k, then,
// when the group has columns past the requests, 4 zero slots that every such
// column reads.
template <int NB>
struct MFLayout {
    static constexpr int cols = 3 * NB;
    static constexpr int NCG = (cols + 15) / 16;
    static constexpr int ncol(int g) { return cols - 16 * g < 16 ? cols - 16 * g : 16; }
    static constexpr int gslots(int g) { return 4 * (ncol(g) + (ncol(g) < 16 ? 1 : 0)); }
    static constexpr int goff(int g) { return g == 0 ? 0 : goff(g - 1) + gslots(g - 1); }
    static constexpr int stride = goff(NCG);                                   // int4 slots per tile
    static constexpr int zero = goff(NCG - 1) + 4 * ncol(NCG - 1);             // zero slots of the last group
    static constexpr bool padded = ncol(NCG - 1) < 16;
};

// int4 of LDS per wave: the larger of the dot4 layout (NB S 16) and the
// matrix-core one (S x stride, then 3 NB x 64 int32 sums).
template <int NB>
constexpr int region_int4() {
    constexpr int d4 = NB * Stage<NB>::S * 16;
    constexpr int mf = Stage<NB>::S * MFLayout<NB>::stride + 3 * NB * 16;
    return d4 > mf ? d4 : mf;
}

// One tile: four groups of four columns, four rows each, NB requests.
template <int NS, int NB>
__device__ __forceinline__ void tile_dots(const u32x4* buf, const int4* __restrict__ lt, int slots,
                                          int (&acc)[NB][4][kLimbs]) {
    uint32_t w[4][NS];
#pragma unroll
    for (int p = 0; p < NS; ++p) {
        w[0][p] = buf[p].x;
        w[1][p] = buf[p].y;
        w[2][p] = buf[p].z;
        w[3][p] = buf[p].w;
    }
    int4 lm[4][NB];
#pragma unroll
    for (int uu = 0; uu < 4; ++uu)
#pragma unroll
        for (int r = 0; r < NB; ++r) lm[uu][r] = lt[r * slots + uu * 4];
#define QAM_GROUP(UU)                                                                          \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                             \
        const int P = (int)assemble<NS, UU>(w[j]);                                              \
        _Pragma("unroll") for (int r = 0; r < NB; ++r) {                                        \
            acc[r][j][0] = __builtin_amdgcn_sdot4(P, lm[UU][r].x, acc[r][j][0], false);         \
            acc[r][j][1] = __builtin_amdgcn_sdot4(P, lm[UU][r].y, acc[r][j][1], false);         \
            acc[r][j][2] = __builtin_amdgcn_sdot4(P, lm[UU][r].z, acc[r][j][2], false);         \
        }                                                                                      \
    }
    QAM_GROUP(0)
    QAM_GROUP(1)
    QAM_GROUP(2)
    QAM_GROUP(3)
#undef QAM_GROUP
}

// One tile on the matrix cores: for each 16-row group j, the rebuilt codes
// of the lane (row 16j + (L & 15), columns 16(L >> 4) + 0..15) are the A
// operand; B operand g of the lane is column 16 g + (L & 15) of the limbs
// (slot bslot[g] of the tile).  acc[g][j] gets the 16 x 16 int32 product:
// lane L holds column 16 g + (L & 15) of rows 16j + 4(L >> 4) + i.
template <int NS, int NB>
__device__ __forceinline__ void tile_mfma(const u32x4* buf, const int4* __restrict__ lt,
                                          const int (&bslot)[MFLayout<NB>::NCG],
                                          v4i (&acc)[MFLayout<NB>::NCG][4]) {
    constexpr int NCG = MFLayout<NB>::NCG;
    v4i bm[NCG];
#pragma unroll
    for (int g = 0; g < NCG; ++g) {
        const int4 b4 = lt[bslot[g]];
        bm[g] = v4i{b4.x, b4.y, b4.z, b4.w};
    }
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
#pragma unroll
        for (int g = 0; g < NCG; ++g) acc[g][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, bm[g], acc[g][j], 0, 0, 0);
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

// Turn this wave's sub-chunk of x into limb words in LDS (see the file comment).
// xraw[r][i] holds the x values of group lane + 64 i of request r.
// Limb layouts: for the dot4 product, group g's limb words as one 16-byte
// slot (limb_slot); for the matrix-core product (MF), MFLayout: the limb
// words of request r, limb l and the tile's columns 16k + 4u .. +3 go to word
// u of slot 4 c + k of the group holding column 3 r + l.
template <int NB, int G, bool XBF16, bool MF>
__device__ __forceinline__ void stage_limbs(const u32x4 (&xraw)[NB][G], int ngroups, int slots, int L,
                                            int4* __restrict__ lds, int (&exps)[NB], bool (&bad)[NB],
                                            bool want_ssq, double (&ssq)[NB]) {
    lds_order();   // the last sub-chunk's limb reads come before these writes
    float4 xv[NB][G];
#pragma unroll
    for (int r = 0; r < NB; ++r)
#pragma unroll
        for (int i = 0; i < G; ++i) xv[r][i] = x4_value<XBF16>(xraw[r][i]);
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        float m = 0.0f;
        float poison = 0.0f;   // 0 * x summed: NaN exactly when some x is not finite
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float4 v = xv[r][i];
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
        int e = 0;
        if (m > 0.0f) frexpf(m, &e);
        exps[r] = __builtin_amdgcn_readfirstlane(e);
        bad[r] = __builtin_amdgcn_readfirstlane((int)(poison != 0.0f)) != 0;   // NaN != 0
        const int sh = kFrac - exps[r];
        const float scale = __uint_as_float((uint32_t)(sh + 127) << 23);     // 2^sh when sh <= 126
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int g = L + 64 * i;
            if (g >= ngroups) continue;
            const float4 v = xv[r][i];
            if (want_ssq) {   // this lane's share of sum x^2 (an RMS-normalised input, one column chunk)
                ssq[r] += (double)v.x * (double)v.x;
                ssq[r] += (double)v.y * (double)v.y;
                ssq[r] += (double)v.z * (double)v.z;
                ssq[r] += (double)v.w * (double)v.w;
            }
            uint32_t w0, w1, w2, w3;
            if (sh <= 126) {
                w0 = limbs_fast(v.x, scale), w1 = limbs_fast(v.y, scale);
                w2 = limbs_fast(v.z, scale), w3 = limbs_fast(v.w, scale);
            } else {   // every |x| of the sub-chunk below 2^-104
                w0 = limbs_of(v.x, sh), w1 = limbs_of(v.y, sh), w2 = limbs_of(v.z, sh), w3 = limbs_of(v.w, sh);
            }
            const int4 lw = limb_words(w0, w1, w2, w3);
            if constexpr (MF) {
                using Y = MFLayout<NB>;
                // (4 c + k) * 4 + u with k = (g & 15) >> 2, u = g & 3 is 16 c + (g & 15)
                int* wl = reinterpret_cast<int*>(lds) + (g >> 4) * Y::stride * 4 + (g & 15);
                const int c0 = 3 * r, c1 = 3 * r + 1, c2 = 3 * r + 2;
                wl[4 * Y::goff(c0 >> 4) + 16 * (c0 & 15)] = lw.x;
                wl[4 * Y::goff(c1 >> 4) + 16 * (c1 & 15)] = lw.y;
                wl[4 * Y::goff(c2 >> 4) + 16 * (c2 & 15)] = lw.z;
            } else {
                lds[r * slots + limb_slot(g)] = lw;
            }
        }
    }
    lds_order();   // the writes come before the tile loop's reads
}

// ------------------------------------------------------------------ epilogue

// sum_k x[r][k]^2 in fp64, in a fixed order: lane partials over a stride of
// 256 columns, then a butterfly (every lane ends with the same value).
template <bool XBF16>
__device__ double sum_squares(const void* x, int64_t K, int r, int L) {
    double s = 0.0;
    for (int64_t k = 4 * L; k < K; k += 256) {
        const float4 v = x4_value<XBF16>(load_x4_raw<XBF16>(x, (int64_t)r * K + k));
        s += (double)v.x * (double)v.x;
        s += (double)v.y * (double)v.y;
        s += (double)v.z * (double)v.z;
        s += (double)v.w * (double)v.w;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
    return s;
}

// Writes the block's outputs from the exact row sums sum[r] = c_n . x_r
// (ssq: sum_k x_r[k]^2 when have_ssq, else taken here):
// v = scale * sum (divided by the RMS of x_r when the item asks for an
// RMS-normalised input), then y = fl32(v) (store), y = fl32(y + v) (residual
// add) or, for rows interleaved 32 gate / 32 up per block, one output per
// pair: fl32(silu(gate) * up) with silu(t) = t / (1 + e^-t), all in fp64.
template <int NB, bool XBF16, bool EPI>
__device__ __forceinline__ void finish(const Item& a, int b, int L, const double (&sum)[NB], bool have_ssq,
                                       const double (&ssq)[NB]) {
    const int row = b * kRows + L;
    const double sc = (double)a.scales[row];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        double v = sc * sum[r];
        if (EPI && a.rms) {
            const double ss = have_ssq ? ssq[r] : sum_squares<XBF16>(a.x, a.K, r, L);
            v = v / sqrt(ss / (double)a.K + a.eps);
        }
        if (EPI && a.out_mode == QAM_OUT_GLU) {
            const double up = __shfl(v, (L + 32) & 63);
            if (L < 32) a.y[(int64_t)r * (a.N / 2) + b * 32 + L] = (float)(v / (1.0 + exp(-v)) * up);
        } else if (EPI && a.out_mode == QAM_OUT_ADD) {
            float* yp = a.y + (int64_t)r * a.N + row;
            *yp = (float)((double)*yp + v);
        } else {
            a.y[(int64_t)r * a.N + row] = (float)v;
        }
    }
}

// A ZERO block: every row's sum is 0, so y = 0 (store), y unchanged (add) or
// silu(0) * 0 = 0 (gated pairs); nothing of the block is read.
template <int NB, bool EPI>
__device__ __forceinline__ void finish_zero(const Item& a, int b, int L) {
    if (EPI && a.out_mode == QAM_OUT_ADD) return;
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        if (EPI && a.out_mode == QAM_OUT_GLU) {
            if (L < 32) a.y[(int64_t)r * (a.N / 2) + b * 32 + L] = 0.0f;
        } else {
            a.y[(int64_t)r * a.N + (int64_t)b * kRows + L] = 0.0f;
        }
    }
}

// One wavefront: block b, column chunk `chunk`, read at NS slices.  The chunk
// is walked in sub-chunks of S tiles; each sub-chunk's exact integer sums are
// scaled into a per-row fp64 sum (exact but for fp64 rounding across
// sub-chunks, in a fixed order).
template <int NS, int NB, bool XBF16, bool MF, bool EPI>
__device__ __forceinline__ void wave_body(const Item& a, const Common& c, int4* __restrict__ lds, int b, int chunk,
                                          int L, int ks, int KS, double* red) {
    constexpr int H = Ring<NS, NB, MF>::H;
    constexpr int PF = Ring<NS, NB, MF>::PF;
    using Y = MFLayout<NB>;
    constexpr int NCG = Y::NCG;
    constexpr int S = Stage<NB>::S;
    constexpr int G = Stage<NB>::G;
    const int B = c.B;
    const int tile0 = chunk * a.tpc;
    // the chunk's tiles ks, ks + KS, ... are this wave's (KS waves share a chunk)
    const int ntile_all = min(a.tpc, a.n_tiles - tile0);
    const int ntile = ntile_all > ks ? (ntile_all - ks + KS - 1) / KS : 0;
    const int64_t tstride = (int64_t)KS * kTileBytes;
    const uint8_t* base0 = a.planes + (int64_t)b * 16 * a.K + (int64_t)(tile0 + ks) * kTileBytes + L * 16;
    const int kg = L >> 4;
    const int slots = S * 16;
    const int64_t pb = a.plane_bytes;

    // MF: this lane's B-operand slot per column group, and the zero slots of
    // every tile (written once; staging never touches them)
    int bslot[NCG];
#pragma unroll
    for (int g = 0; g < NCG; ++g) {
        const int cc = L & 15;
        bslot[g] = Y::goff(g) + 4 * (cc < Y::ncol(g) ? cc : Y::ncol(g)) + kg;
    }
    if constexpr (MF && Y::padded) {
        if ((L >> 2) < S) lds[(L >> 2) * Y::stride + Y::zero + (L & 3)] = int4{0, 0, 0, 0};
    }
    int* tab = reinterpret_cast<int*>(lds + S * Y::stride);   // MF: [3 NB][64 rows] sums of a sub-chunk

    double mine[NB];
    bool any_bad[NB];
    double ssq[NB];
    // an unsplit RMS-normalised product sees all of x while staging it
    const bool want_ssq = EPI && a.rms && a.n_chunks == 1;
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        mine[r] = 0.0;
        any_bad[r] = false;
        ssq[r] = 0.0;
    }

    // x of sub-chunk `sub`, raw, G groups of four values per lane and request
    // (lanes past the sub-chunk reload its last group, never staged)
    u32x4 xraw[NB][G];
    auto load_x = [&](int sub) {
        const int ngroups = min(S, ntile - sub * S) * 16;
#pragma unroll
        for (int r = 0; r < NB; ++r)
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int g = min(L + 64 * i, ngroups - 1);
                const int64_t col = (int64_t)(tile0 + ks + KS * (sub * S + (g >> 4))) * kTileCols + 4 * (g & 15);
                xraw[r][i] = load_x4_raw<XBF16>(a.x, (int64_t)r * a.K + col);
            }
    };
    int exps[NB];
    bool bad[NB];
    auto stage = [&](int sub) {
        stage_limbs<NB, G, XBF16, MF>(xraw, min(S, ntile - sub * S) * 16, slots, L, lds, exps, bad, want_ssq, ssq);
    };
    int acc[NB][4][kLimbs];
    v4i macc[NCG][4];
    auto clear_acc = [&]() {
#pragma unroll
        for (int r = 0; r < NB; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int l = 0; l < kLimbs; ++l) acc[r][j][l] = 0;
#pragma unroll
        for (int g = 0; g < NCG; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) macc[g][j] = v4i{0, 0, 0, 0};
    };
    // The sub-chunk's exact per-row integers, scaled by its exponent into the
    // row's fp64 sum.  dot4: summed over the four lane groups sharing a row;
    // MF: the three limb columns of every row through LDS, then row L's
    // integer on lane L (the same value either way).
    auto flush = [&]() {
        if constexpr (MF) {
#pragma unroll
            for (int g = 0; g < NCG; ++g) {
                const int gc = 16 * g + (L & 15);
                if (gc < 3 * NB) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(tab + gc * 64 + 16 * j + 4 * kg) = macc[g][j];
                }
            }
            lds_order();
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                const double d = (double)tab[(3 * r + 2) * 64 + L] * 65536.0 + (double)tab[(3 * r + 1) * 64 + L] * 256.0 +
                                 (double)tab[3 * r * 64 + L];
                mine[r] += ldexp(d, exps[r] - kFrac);
                any_bad[r] = any_bad[r] || bad[r];
            }
        } else {
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                double d[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    d[j] = (double)acc[r][j][2] * 65536.0 + (double)acc[r][j][1] * 256.0 + (double)acc[r][j][0];
                    d[j] += __shfl_xor(d[j], 16);
                    d[j] += __shfl_xor(d[j], 32);
                }
                const double sel = kg == 0 ? d[0] : (kg == 1 ? d[1] : (kg == 2 ? d[2] : d[3]));
                mine[r] += ldexp(sel, exps[r] - kFrac);
                any_bad[r] = any_bad[r] || bad[r];
            }
        }
    };
#define QAM_TILE(BUF, TT)                                                   \
    do {                                                                    \
        if constexpr (MF) tile_mfma<NS, NB>(BUF, lds + (TT) * Y::stride, bslot, macc); \
        else tile_dots<NS, NB>(BUF, lds + (TT) * 16 + kg, slots, acc);     \
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
#pragma unroll
            for (int u = 0; u < H; ++u) QAM_TILE(A[u], tl + u);
            __builtin_amdgcn_sched_barrier(0);
            load_half<NS, H>(A, base0, pb, tstride, t + PF, last);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < H; ++u) QAM_TILE(Bh[u], tl + H + u);
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
        flush();
    }
#undef QAM_TILE

    const int row = b * kRows + L;          // the row this lane writes: j = L >> 4
    double part[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) part[r] = any_bad[r] ? __builtin_nan("") : mine[r];   // non-finite x: NaN
    if (KS > 1) {   // the chunk's other waves hand over their row sums; wave 0 adds them in order
        if (ks > 0) {
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                red[((ks * NB + r) * 2 + 0) * 64 + L] = part[r];
                red[((ks * NB + r) * 2 + 1) * 64 + L] = ssq[r];
            }
        }
        __syncthreads();
        if (ks > 0) return;
        for (int k2 = 1; k2 < KS; ++k2)
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                part[r] += red[((k2 * NB + r) * 2 + 0) * 64 + L];
                ssq[r] += red[((k2 * NB + r) * 2 + 1) * 64 + L];
            }
    }

    if (a.n_chunks == 1) {
        if (want_ssq) {
#pragma unroll
            for (int r = 0; r < NB; ++r)
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) ssq[r] += __shfl_xor(ssq[r], o);
        }
        finish<NB, XBF16, EPI>(a, b, L, part, want_ssq, ssq);
        return;
    }
    // Split K: publish this chunk's partials, then count the arrival; the last
    // wave of the block sums the partials in chunk order.  The partials are
    // written and read with device-scope (write-through) atomic accesses and
    // the counter is bumped only after those stores have completed, so no
    // cache-wide writeback or invalidate is needed: a device-scope fence here
    // writes back and invalidates the whole L2 of the XCD, thousands of times
    // per launch.
#pragma unroll
    for (int r = 0; r < NB; ++r)
        __hip_atomic_store(&a.partials[((int64_t)chunk * B + r) * a.N + row], part[r], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);   // the partial stores are complete before the arrival is counted
    uint32_t prev = 0;
    if (L == 0) prev = __hip_atomic_fetch_add(&a.counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0);
    if (prev != (uint32_t)(a.n_chunks - 1)) return;
    double sum[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        sum[r] = 0.0;
        for (int cc = 0; cc < a.n_chunks; ++cc)
            sum[r] += __hip_atomic_load(&a.partials[((int64_t)cc * B + r) * a.N + row], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    }
    if (L == 0) __hip_atomic_store(&a.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    finish<NB, XBF16, EPI>(a, b, L, sum, false, ssq);
}

// One (block, column chunk) unit of item a, `local` being its index within
// the item, run by c.KS wavefronts (at most MAXW); wave k takes the chunk's
// tiles k, k + KS, ...  With a lens map lm (one wavefront per unit), the
// block's rung comes from the lens rules and the chunk-0 unit writes it to
// the item's map; else it is read from the map (or fixed).
template <int NB, bool XBF16, int MAXW, bool MF, bool EPI, bool LENS = false>
__device__ __forceinline__ void run_unit(const Item& a, const Common& c, int local, int4* lds, int tid,
                                         const LensMap* lm = nullptr) {
    // per wave: region_int4<NB>() int4 (the sub-chunk's limb words in the
    // layout of the inner product in use; for the matrix cores then 3 NB x 64
    // int32 sums); then, with several waves, [KS][NB][2][64] fp64 row sums
    // handed to wave 0
    const int KS = MAXW == 1 ? 1 : c.KS;
    const int ks = MAXW == 1 ? 0 : tid >> 6;
    const int region = region_int4<NB>();   // int4 per wave
    int4* mylds = lds + ks * region;
    double* red = reinterpret_cast<double*>(lds + KS * region);
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
    const int ns = __builtin_amdgcn_readfirstlane(lev < 4 ? lev : 4);
    switch (ns) {   // uniform over the workgroup: one block
        case 0:   // ZERO: nothing read, y = 0 (written once, by the first chunk's first wave)
            if (chunk == 0 && ks == 0) finish_zero<NB, EPI>(a, b, L);
            return;
        case 1: wave_body<1, NB, XBF16, MF, EPI>(a, c, mylds, b, chunk, L, ks, KS, red); return;
        case 2: wave_body<2, NB, XBF16, MF, EPI>(a, c, mylds, b, chunk, L, ks, KS, red); return;
        case 3: wave_body<3, NB, XBF16, MF, EPI>(a, c, mylds, b, chunk, L, ks, KS, red); return;
        default: wave_body<4, NB, XBF16, MF, EPI>(a, c, mylds, b, chunk, L, ks, KS, red); return;
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

// One workgroup per unit: a single matrix (descriptor by value; with its
// epilogue) or a group (descriptor table, one lookup per workgroup; plain
// stores, the only output a group's items have).
template <int NB, bool GROUPED, bool XBF16, int MAXW, bool MF>
__global__ __launch_bounds__(64 * MAXW) void qmatvec_kernel(Item single, Common c) {
    extern __shared__ int4 lds[];
    if constexpr (GROUPED) {
        const Item a = unit_item(c, (int)blockIdx.x);
        run_unit<NB, XBF16, MAXW, MF, false>(a, c, (int)blockIdx.x - a.wg_begin, lds, (int)threadIdx.x);
    } else {
        run_unit<NB, XBF16, MAXW, MF, true>(single, c, (int)blockIdx.x, lds, (int)threadIdx.x);
    }
}

// A group whose maps are built in the same launch: every unit computes its
// block's rung from the lens map (kernel argument) before its planes.
template <int NB, bool XBF16, bool MF>
__global__ __launch_bounds__(64) void qmatvec_lens_kernel(Common c, LensMap lm) {
    extern __shared__ int4 lds[];
    const Item a = unit_item(c, (int)blockIdx.x);
    run_unit<NB, XBF16, 1, MF, false, true>(a, c, (int)blockIdx.x - a.wg_begin, lds, (int)threadIdx.x, &lm);
}

// ------------------------------------------------------------------ host side

static int64_t g_target_waves = 256 * 32;   // wavefronts aimed for per launch
static int64_t g_max_chunk_tiles = 64;       // longest column chunk of the staged-limb launches

// every chunk holds a whole number of prefetch rings (Ring<NS, B, MF>::PF for every NS and form)
int tpc_align_for(int64_t B) { return B <= 4 ? 8 : 4; }
int stage_tiles_for(int64_t B) { return B <= 2 ? 16 : (B <= 5 ? 8 : 4); }
size_t lds_bytes_for(int64_t B) {
    int r = 0;
    switch (B) {
        case 1: r = region_int4<1>(); break;
        case 2: r = region_int4<2>(); break;
        case 3: r = region_int4<3>(); break;
        case 4: r = region_int4<4>(); break;
        case 5: r = region_int4<5>(); break;
        case 6: r = region_int4<6>(); break;
        case 7: r = region_int4<7>(); break;
        default: r = region_int4<8>(); break;
    }
    return (size_t)r * sizeof(int4);
}

// Inner product of the staged-limb route: 1 = matrix cores, 0 = dot4 on the
// vector ALUs (the same integers, so the same bits).
static int g_staged_mfma = 1;

// Column chunk length (in tiles) for a launch covering `block_tiles` block x
// tile pairs: enough chunks for about g_target_waves wavefronts of equal work.
int chunk_goal(int64_t block_tiles, int64_t target_waves) {
    const bool dflt = target_waves <= 0;
    if (dflt) target_waves = g_target_waves;
    int64_t g = (block_tiles + target_waves - 1) / target_waves;
    if (dflt) g = std::min<int64_t>(g, g_max_chunk_tiles);   // long waves leave a long tail
    return (int)std::max<int64_t>(1, std::min<int64_t>(g, QAM_MAX_K / kTileCols));
}

// Chunking of one matrix: K is cut into the fewest chunks of at most `goal`
// tiles, evened out and rounded up to a whole number of prefetch rings.
Plan make_plan(int64_t N, int64_t K, int64_t B, int goal, int align) {
    Plan p{};
    const int n_blocks = (int)(N / kRows);
    const int n_tiles = (int)(K / kTileCols);
    if (align <= 0) align = tpc_align_for(B);
    const int want = (n_tiles + goal - 1) / goal;
    int tpc = (n_tiles + want - 1) / want;
    tpc = (tpc + align - 1) / align * align;
    if (tpc > n_tiles) tpc = n_tiles;
    p.tpc = tpc;
    p.n_chunks = (n_tiles + tpc - 1) / tpc;
    p.n_quads = n_blocks;   // one wavefront-sized workgroup per block and chunk
    p.partial_bytes = p.n_chunks > 1 ? ((size_t)p.n_chunks * B * N * sizeof(double) + 255) / 256 * 256 : 0;
    return p;
}

// With events, the launch records them at the kernel's own start and end
// (hipExtLaunchKernel), which times the kernel alone.
template <int NB, bool GROUPED, int MAXW, bool MF>
static void launch_k(const Item& it, const Common& c, int64_t grid, int threads, size_t lds, hipStream_t s,
                     hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
    const dim3 g((unsigned)grid), b((unsigned)threads);
    if (e0 || e1) {
        if (c.x_bf16)
            hipExtLaunchKernelGGL((qmatvec_kernel<NB, GROUPED, true, MAXW, MF>), g, b, (uint32_t)lds, s, e0, e1, 0u,
                                  it, c);
        else
            hipExtLaunchKernelGGL((qmatvec_kernel<NB, GROUPED, false, MAXW, MF>), g, b, (uint32_t)lds, s, e0, e1, 0u,
                                  it, c);
        return;
    }
    if (c.x_bf16)
        hipLaunchKernelGGL((qmatvec_kernel<NB, GROUPED, true, MAXW, MF>), g, b, lds, s, it, c);
    else
        hipLaunchKernelGGL((qmatvec_kernel<NB, GROUPED, false, MAXW, MF>), g, b, lds, s, it, c);
}

template <int NB, bool GROUPED>
static void launch_nb(const Item& it, const Common& c, int64_t grid, size_t lds, hipStream_t s, hipEvent_t e0,
                      hipEvent_t e1) {
    if (g_staged_mfma) launch_k<NB, GROUPED, 1, true>(it, c, grid, 64, lds, s, e0, e1);
    else launch_k<NB, GROUPED, 1, false>(it, c, grid, 64, lds, s, e0, e1);
}

template <bool GROUPED>
static void launch(int64_t B, const Item& it, const Common& c, int64_t grid, size_t lds, hipStream_t s,
                   hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
    switch (B) {
        case 1: launch_nb<1, GROUPED>(it, c, grid, lds, s, e0, e1); break;
        case 2: launch_nb<2, GROUPED>(it, c, grid, lds, s, e0, e1); break;
        case 3: launch_nb<3, GROUPED>(it, c, grid, lds, s, e0, e1); break;
        case 4: launch_nb<4, GROUPED>(it, c, grid, lds, s, e0, e1); break;
        case 5: launch_nb<5, GROUPED>(it, c, grid, lds, s, e0, e1); break;
        case 6: launch_nb<6, GROUPED>(it, c, grid, lds, s, e0, e1); break;
        case 7: launch_nb<7, GROUPED>(it, c, grid, lds, s, e0, e1); break;
        default: launch_nb<8, GROUPED>(it, c, grid, lds, s, e0, e1); break;
    }
}

void launch_single(int64_t B, const Item& it, const Common& c, int64_t grid, hipStream_t s) {
    if (B == 1 && c.KS > 1) {   // several waves per (block, chunk): batch 1 only
        const size_t lds = (size_t)c.KS * lds_bytes_for(1) + (size_t)c.KS * 2 * 64 * sizeof(double);
        if (g_staged_mfma)
            launch_k<1, false, 8, true>(it, c, grid, 64 * c.KS, lds, s);
        else
            launch_k<1, false, 8, false>(it, c, grid, 64 * c.KS, lds, s);
        return;
    }
    launch<false>(B, it, c, grid, lds_bytes_for(B), s);
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

}  // namespace qam

using namespace qam;

extern "C" size_t qam_qmatvec_workspace_bytes(int64_t N, int64_t K, int64_t B) {
    if (N <= 0 || K <= 0 || N % kRows || K % kTileCols || K > QAM_MAX_K || N / kRows > QAM_MAX_BLOCKS || B < 1 ||
        B > QAM_MAX_BATCH_MFMA)
        return 0;
    size_t need = 0;
    if (B <= QAM_MAX_BATCH) {   // the staged-limb route
        const Plan p = make_plan(N, K, B, chunk_goal(N / kRows * (K / kTileCols), 0));
        need = p.n_chunks > 1 ? QAM_WS_COUNTER_BYTES + p.partial_bytes : 0;
    }
    if (B > 1) need = std::max(need, qam_mfma_workspace_bytes(N, K, B));   // the pre-pass route
    return need;
}

extern "C" int qam_set_max_chunk_tiles(int t) {
    clear_error();
    if (t < 1 || t > QAM_MAX_K / kTileCols) QAM_FAIL(QAM_ERR_ARG, "set_max_chunk_tiles: %d outside [1, %d]", t, QAM_MAX_K / kTileCols);
    g_max_chunk_tiles = t;
    return QAM_OK;
}

static const char* staged_name() { return g_staged_mfma ? "qmatvec_staged_mfma" : "qmatvec_staged_dot4"; }

extern "C" int qam_set_staged_mfma(int on) {
    clear_error();
    if (on != 0 && on != 1) QAM_FAIL(QAM_ERR_ARG, "set_staged_mfma: %d is not 0 or 1", on);
    g_staged_mfma = on;
    return QAM_OK;
}

extern "C" int qam_set_target_waves(int waves) {
    clear_error();
    if (waves < 64 || waves > (1 << 20)) QAM_FAIL(QAM_ERR_ARG, "set_target_waves: %d outside [64, 2^20]", waves);
    g_target_waves = waves;
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
    if (B > QAM_MAX_BATCH)
        QAM_FAIL(QAM_ERR_ARG, "qmatvec: B=%lld outside [1, %d] for this entry point", (long long)B, QAM_MAX_BATCH);
    const Plan p = make_plan(packed->N, packed->K, B, chunk_goal(packed->n_blocks * (packed->K / kTileCols), 0));
    Item it = make_item(x, packed, level_map, y, p);
    if (ep) {
        it.rms = ep->rms_norm;
        it.out_mode = ep->out_mode;
        it.eps = ep->eps;
    }
    if (p.n_chunks > 1) {
        const size_t need = QAM_WS_COUNTER_BYTES + p.partial_bytes;
        if (!workspace) QAM_FAIL(QAM_ERR_WORKSPACE, "qmatvec: workspace of %zu bytes required", need);
        if (workspace_bytes < need) QAM_FAIL(QAM_ERR_WORKSPACE, "qmatvec: workspace %zu < %zu bytes", workspace_bytes, need);
        if (!aligned(workspace, 256)) QAM_FAIL(QAM_ERR_ALIGN, "qmatvec: workspace must be 256-byte aligned");
        it.counters = static_cast<uint32_t*>(workspace);
        it.partials = reinterpret_cast<double*>(static_cast<char*>(workspace) + QAM_WS_COUNTER_BYTES);
    }
    Common c{};
    c.B = (int)B;
    c.x_bf16 = x_dtype == QAM_X_BF16;
    c.KS = 1;
    const int64_t grid = (int64_t)p.n_chunks * p.n_quads;
    launch_single(B, it, c, grid, s);
    QAM_HIP_CHECK(hipGetLastError());
    char v[128];
    snprintf(v, sizeof(v), "%s B=%lld tpc=%d chunks=%d", staged_name(), (long long)B, p.tpc, p.n_chunks);
    set_variant(v);
    return QAM_OK;
}

// Smallest batch with a shared map that takes the pre-pass route (below it,
// staging the limbs in every row block's wave costs less than the pre-pass
// launch and the limb loads; from 3 requests on it costs more).
static int g_mfma_min_batch = 3;

bool qam::mfma_route(int64_t B, int per_request_maps) {
    return (per_request_maps && B > 1) || B > QAM_MAX_BATCH || B >= g_mfma_min_batch;
}

extern "C" int qam_set_mfma_min_batch(int b) {
    clear_error();
    if (b < 2 || b > QAM_MAX_BATCH + 1) QAM_FAIL(QAM_ERR_ARG, "set_mfma_min_batch: %d outside [2, %d]", b, QAM_MAX_BATCH + 1);
    g_mfma_min_batch = b;
    return QAM_OK;
}

extern "C" int qam_qmatvec(const void* x, int x_dtype, int64_t B, const qam_packed* packed, const uint8_t* level_map,
                           int per_request_maps, float* y, void* workspace, size_t workspace_bytes, hipStream_t s) {
    clear_error();
    if (per_request_maps != 0 && per_request_maps != 1) QAM_FAIL(QAM_ERR_ARG, "qmatvec: per_request_maps must be 0 or 1");
    if (!mfma_route(B, per_request_maps) || B < 1)
        return qam_qmatvec_ep(x, x_dtype, B, packed, level_map, nullptr, y, workspace, workspace_bytes, s);
    if (int rc = check_item(x, x_dtype, B, packed, level_map, y, "qmatvec", QAM_OUT_STORE)) return rc;
    return qmatvec_mfma(x, x_dtype, B, packed, level_map, per_request_maps, y, workspace, workspace_bytes, s);
}

// ------------------------------------------------------------------ grouped launches

namespace qam {

static int g_tail_pct = 15;   // share of a group's block tiles planned with short chunks
static int g_tail_div = 2;    // how much shorter

struct GroupLayout {
    std::vector<Plan> plans;
    size_t partial_bytes = 0, table_bytes = 0, map_bytes = 0, total = 0;
    int64_t n_wg = 0, blocks = 0, block_tiles = 0;
};

static int layout_group(const qam_gemv_item* items, int n_items, int64_t B, GroupLayout& g) {
    if (!items || n_items < 1) QAM_FAIL(QAM_ERR_ARG, "group: need at least one item");
    if (B < 1 || B > QAM_MAX_BATCH) QAM_FAIL(QAM_ERR_ARG, "group: B=%lld outside [1, %d]", (long long)B, QAM_MAX_BATCH);
    for (int i = 0; i < n_items; ++i) {
        const qam_packed& w = items[i].w;
        if (w.N <= 0 || w.N % kRows || w.K <= 0 || w.K % kTileCols || w.K > QAM_MAX_K)
            QAM_FAIL(QAM_ERR_SHAPE, "group: item %d has a bad shape", i);
        g.blocks += w.N / kRows;
        g.block_tiles += w.N / kRows * (w.K / kTileCols);
    }
    if (g.blocks > QAM_MAX_BLOCKS) QAM_FAIL(QAM_ERR_SHAPE, "group: %lld blocks > %d", (long long)g.blocks, QAM_MAX_BLOCKS);
    // Items are dispatched in order, so the last ones run while the chip
    // drains: those covering the last g_tail_pct percent of the block tiles
    // take chunks g_tail_div times shorter, so that the final wavefronts are short.
    const int goal = chunk_goal(g.block_tiles, 0);
    int64_t before = 0;
    for (int i = 0; i < n_items; ++i) {
        const int64_t bt = items[i].w.N / kRows * (items[i].w.K / kTileCols);
        const bool tail = g_tail_pct > 0 && (before + bt) * 100 > g.block_tiles * (100 - g_tail_pct);
        before += bt;
        const Plan p = make_plan(items[i].w.N, items[i].w.K, B, tail ? std::max(1, goal / g_tail_div) : goal);
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

extern "C" int qam_set_tail_split(int pct, int div) {
    clear_error();
    if (pct < 0 || pct > 100 || div < 1 || div > 64) QAM_FAIL(QAM_ERR_ARG, "set_tail_split: pct %d / div %d out of range", pct, div);
    g_tail_pct = pct;
    g_tail_div = div;
    return QAM_OK;
}

extern "C" size_t qam_group_bytes(const qam_gemv_item* items, int n_items, int64_t B, int per_request_maps) {
    if (per_request_maps != 0 && per_request_maps != 1) return 0;
    if (mfma_route(B, per_request_maps)) return mfma_group_bytes(items, n_items, B);
    GroupLayout g;
    if (layout_group(items, n_items, B, g) != QAM_OK) return 0;
    return g.total;
}

extern "C" int qam_group_init(const qam_gemv_item* items, int n_items, int64_t B, int x_dtype, int per_request_maps,
                              void* dev_mem, size_t dev_bytes, qam_group* group_out, hipStream_t s) {
    clear_error();
    if (!group_out || !dev_mem) QAM_FAIL(QAM_ERR_NULL, "group_init: null pointer");
    if (per_request_maps != 0 && per_request_maps != 1) QAM_FAIL(QAM_ERR_ARG, "group_init: per_request_maps must be 0 or 1");
    if (mfma_route(B, per_request_maps))
        return mfma_group_init(items, n_items, B, x_dtype, per_request_maps, dev_mem, dev_bytes, group_out, s);
    GroupLayout g;
    if (int rc = layout_group(items, n_items, B, g)) return rc;
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
    group_out->n_items = n_items;
    group_out->B = B;
    group_out->x_dtype = x_dtype;
    group_out->n_workgroups = g.n_wg;
    group_out->lds_bytes = lds_bytes_for(B);
    group_out->table = table;
    group_out->wg_map = wgmap;
    group_out->route = 0;
    group_out->per_request_maps = 0;
    group_out->n_pre_workgroups = 0;
    group_out->pre_map = nullptr;
    group_out->lens_ready = lens_ready;
    return QAM_OK;
}

namespace qam {

template <int NB, bool MF>
static void launch_lens_k(const Common& c, const LensMap& lm, int64_t grid, size_t lds, hipStream_t s,
                          hipEvent_t e0, hipEvent_t e1) {
    const dim3 g((unsigned)grid), b(64u);
    if (c.x_bf16)
        hipExtLaunchKernelGGL((qmatvec_lens_kernel<NB, true, MF>), g, b, (uint32_t)lds, s, e0, e1, 0u, c, lm);
    else
        hipExtLaunchKernelGGL((qmatvec_lens_kernel<NB, false, MF>), g, b, (uint32_t)lds, s, e0, e1, 0u, c, lm);
}

template <int NB>
static void launch_lens_nb(const Common& c, const LensMap& lm, int64_t grid, size_t lds, hipStream_t s,
                           hipEvent_t e0, hipEvent_t e1) {
    if (g_staged_mfma) launch_lens_k<NB, true>(c, lm, grid, lds, s, e0, e1);
    else launch_lens_k<NB, false>(c, lm, grid, lds, s, e0, e1);
}

// Checks of a group and its lens rules for a launch that builds the maps;
// fills the launch arguments.
static int lens_group_setup(const qam_group* group, const qam_lens* lenses, int n_lenses,
                            const qam_lens_params* params, const uint8_t* ladder_bits, int n_rungs, int glass,
                            Common& c, LensMap& lm, const char* who) {
    if (!group || !group->table || !group->wg_map) QAM_FAIL(QAM_ERR_NULL, "%s: uninitialised group", who);
    if (!params || !ladder_bits) QAM_FAIL(QAM_ERR_NULL, "%s: null params/ladder", who);
    if (group->route != 0 || group->per_request_maps != 0 || group->B < 1 || group->B > QAM_MAX_BATCH ||
        group->n_workgroups < 1)
        QAM_FAIL(QAM_ERR_ARG, "%s: the map is built in the launch on the staged-limb route only (shared map)", who);
    if (!group->lens_ready) QAM_FAIL(QAM_ERR_ARG, "%s: the group's items have no block coordinates", who);
    static const uint8_t kProductLadder[5] = {0, 2, 4, 6, 8};
    if (n_rungs != 5) QAM_FAIL(QAM_ERR_LADDER, "%s: the product ladder has 5 rungs, got %d", who, n_rungs);
    if (int rc = lens_check_ladder(ladder_bits, n_rungs, glass, who)) return rc;
    for (int i = 0; i < 5; ++i)
        if (ladder_bits[i] != kProductLadder[i]) QAM_FAIL(QAM_ERR_LADDER, "%s: ladder must be {0,2,4,6,8}", who);
    lm = LensMap{};
    if (int rc = lens_check_map(lenses, n_lenses, params, n_rungs, glass, lm.p, who)) return rc;
    for (int i = 0; i < n_lenses; ++i) {
        lm.t.cx[i] = lenses[i].cx;
        lm.t.cy[i] = lenses[i].cy;
        lm.t.R[i] = lens_radius(lenses[i].r, params->f);
    }
    lm.glass = glass;
    c = Common{};
    c.items = static_cast<const Item*>(group->table);
    c.wg_item = static_cast<const int*>(group->wg_map);
    c.B = (int)group->B;
    c.x_bf16 = group->x_dtype == QAM_X_BF16;
    c.KS = 1;
    return QAM_OK;
}

static void launch_lens(const qam_group* group, const Common& c, const LensMap& lm, hipStream_t s,
                        hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
    const int64_t grid = group->n_workgroups;
    const size_t lds = group->lds_bytes;
    switch (group->B) {
        case 1: launch_lens_nb<1>(c, lm, grid, lds, s, e0, e1); break;
        default: launch_lens_nb<2>(c, lm, grid, lds, s, e0, e1); break;
    }
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
    if (group->B > 2)
        QAM_FAIL(QAM_ERR_ARG, "qmatvec_group_lens: B=%lld; the map is built in the launch for B <= 2",
                 (long long)group->B);
    launch_lens(group, c, lm, s);
    QAM_HIP_CHECK(hipGetLastError());
    char v[128];
    snprintf(v, sizeof(v), "%s_group_lens items=%d B=%lld wg=%lld", staged_name(), group->n_items,
             (long long)group->B, (long long)group->n_workgroups);
    set_variant(v);
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
    if (group->B > 2) QAM_FAIL(QAM_ERR_ARG, "group_lens_launch_times: B=%lld > 2", (long long)group->B);
    if (!ms_out) QAM_FAIL(QAM_ERR_NULL, "group_lens_launch_times: null output");
    if (n < 1 || n > 4096) QAM_FAIL(QAM_ERR_ARG, "group_lens_launch_times: n=%d outside [1, 4096]", n);
    std::vector<hipEvent_t> ev((size_t)2 * n, nullptr);
    hipError_t e = hipSuccess;
    for (size_t i = 0; i < ev.size() && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
    for (int i = 0; i < n && e == hipSuccess; ++i) {
        launch_lens(group, c, lm, s, ev[2 * i], ev[2 * i + 1]);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    for (int i = 0; i < n && e == hipSuccess; ++i) e = hipEventElapsedTime(&ms_out[i], ev[2 * i], ev[2 * i + 1]);
    for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
    if (e != hipSuccess) QAM_FAIL(QAM_ERR_HIP, "group_lens_launch_times: %s", hipGetErrorString(e));
    return QAM_OK;
}

// Benchmark hook: runs a staged-limb group `n` times back to back on `s`,
// timing each launch with HIP events recorded at the kernel's own start and
// end; writes the n durations (ms) and synchronises `s`.
extern "C" int qam_group_launch_times(const qam_group* group, int n, float* ms_out, hipStream_t s) {
    clear_error();
    if (!group || !group->table || !group->wg_map || !ms_out) QAM_FAIL(QAM_ERR_NULL, "group_launch_times: null pointer");
    if (group->route != 0 || group->B < 1 || group->B > QAM_MAX_BATCH || group->n_workgroups < 1)
        QAM_FAIL(QAM_ERR_ARG, "group_launch_times: only staged-limb groups are timed here");
    if (n < 1 || n > 4096) QAM_FAIL(QAM_ERR_ARG, "group_launch_times: n=%d outside [1, 4096]", n);
    Common c{};
    c.items = static_cast<const Item*>(group->table);
    c.wg_item = static_cast<const int*>(group->wg_map);
    c.B = (int)group->B;
    c.x_bf16 = group->x_dtype == QAM_X_BF16;
    c.KS = 1;
    Item none{};
    std::vector<hipEvent_t> ev((size_t)2 * n, nullptr);
    hipError_t e = hipSuccess;
    for (size_t i = 0; i < ev.size() && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
    for (int i = 0; i < n && e == hipSuccess; ++i) {
        launch<true>(group->B, none, c, group->n_workgroups, group->lds_bytes, s, ev[2 * i], ev[2 * i + 1]);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    for (int i = 0; i < n && e == hipSuccess; ++i) e = hipEventElapsedTime(&ms_out[i], ev[2 * i], ev[2 * i + 1]);
    for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
    if (e != hipSuccess) QAM_FAIL(QAM_ERR_HIP, "group_launch_times: %s", hipGetErrorString(e));
    return QAM_OK;
}

extern "C" int qam_qmatvec_group(const qam_group* group, hipStream_t s) {
    clear_error();
    if (!group || !group->table || !group->wg_map) QAM_FAIL(QAM_ERR_NULL, "qmatvec_group: uninitialised group");
    if (group->route == 1) {
        if (!group->pre_map || group->B < 2 || group->B > QAM_MAX_BATCH_MFMA || group->n_workgroups < 1)
            QAM_FAIL(QAM_ERR_ARG, "qmatvec_group: corrupt group descriptor");
        return mfma_group_run(group, s);
    }
    if (group->route != 0 || group->B < 1 || group->B > QAM_MAX_BATCH || group->n_workgroups < 1)
        QAM_FAIL(QAM_ERR_ARG, "qmatvec_group: corrupt group descriptor");
    Common c{};
    c.items = static_cast<const Item*>(group->table);
    c.wg_item = static_cast<const int*>(group->wg_map);
    c.B = (int)group->B;
    c.x_bf16 = group->x_dtype == QAM_X_BF16;
    c.KS = 1;
    char v[128];
    Item none{};
    launch<true>(group->B, none, c, group->n_workgroups, group->lds_bytes, s);
    QAM_HIP_CHECK(hipGetLastError());
    snprintf(v, sizeof(v), "%s_group items=%d B=%lld wg=%lld", staged_name(), group->n_items, (long long)group->B,
             (long long)group->n_workgroups);
    set_variant(v);
    return QAM_OK;
}
