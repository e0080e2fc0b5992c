// Batched mixed-depth product on the matrix cores: up to 32 requests, with
// one level map shared by all of them or one map per request.
//
// [FoQLens] "Progress": every 64-row block is read at its own depth from the
// one stored copy inside the pass (the pages' batched decode reads 32
// requests per step).  With a map per request, block b is read once, to the
// deepest slice any request needs, and every request gets the block's codes
// at its own depth: the residual slices make the code at depth d the sum of
// the first d/2 slices.  Two forms use that: the per-depth form builds the
// codes for each depth present in the batch incrementally from the same
// loaded words and multiplies them by the limbs of the requests at that
// depth; the per-slice form (selectable by a tuning hook) multiplies each
// slice plane alone by every request's limbs and lets each request add the
// planes it reads.
//
// Arithmetic (exact, as in the batch-1 kernel): a pre-pass turns each
// request's x, per column chunk, into a 24-bit fixed point held as three int8
// limbs, laid out as B operands of v_mfma_i32_16x16x64_i8: column c = 3 rr + l
// of a request set (16 requests at most, SS by the plan) holds limb l of
// request rr, 16 columns per MFMA (NCG column groups per set: 1 for up to 5
// requests, 2 up to 10, 3 up to 16).  Codes are the A operands (16 rows x 64
// columns, exactly the words a lane loads); i32 accumulation is exact; the
// limbs of a request are combined in fp64 after the chunk, through an LDS
// table of the block's 64 x 16 NCG integer sums.
//
// A workgroup is one (block, column chunk).  Per-depth form: wave (ks, h)
// serves request set h on the chunk's tiles ks, ks + KS, ...; the KS tables
// of a set are summed when the outputs are formed.  Per-slice form: wave
// (h, p) takes plane p of the chunk for set h.  Either way one row per lane
// forms the outputs, so y is written coalesced.

#include <algorithm>
#include <vector>

#include "qmatvec_internal.h"

namespace qam {

typedef __attribute__((address_space(1))) const v4i global_v4i;

constexpr int kBadExp = 0x7FFFFFFF;   // exponent marker of a chunk of x with a non-finite value

struct MItem {
    const uint8_t* planes;
    const float* scales;
    const void* x;             // [B][K]
    float* y;                  // [B][N]
    const uint8_t* level;      // [B][n_blocks] (per request) or [n_blocks]
    int64_t level_stride;      // n_blocks (per request) or 0
    v4i* limbs;                // [n_tiles][NH][NCG][64] 16-byte B operands
    int* exps;                 // [n_chunks][16 NH]
    double* partials;          // [n_chunks][B][N] (split K only)
    uint32_t* counters;        // [n_blocks]       (split K only)
    int64_t plane_bytes;
    int64_t N, K;
    int n_blocks, n_tiles, tpc, n_chunks;
    int wg_begin;              // grouped launches: first product workgroup of this item
    int pre_begin;             // grouped launches: first pre-pass workgroup of this item
};

struct MCommon {
    const MItem* items;        // grouped launches: the descriptor table
    const int* wg_item;        // grouped launches: item of every product workgroup
    const int* pre_item;       // grouped launches: item of every pre-pass workgroup
    int B;
    int NH;                    // request sets per workgroup
    int SS;                    // requests per set (<= 16; 3 SS limb columns in NCG groups of 16)
    int KS;                    // waves per request set splitting a chunk's tiles
    int NCG;                   // 16-column groups per request set
    int first;                 // refinement launches: slices below this are not read, and y is added to
};

// Depth (slices read, 0..4) of request r in block b.
template <bool PER_REQ>
__device__ __forceinline__ int depth_of(const MItem& a, int r, int b) {
    const int lev = PER_REQ ? (int)a.level[(int64_t)r * a.level_stride + b] : level_of(a.level, b);
    return lev < 4 ? lev : 4;
}

// ------------------------------------------------------------------ x -> limbs

// One workgroup of four wavefronts per (column chunk, request slot
// r < SS NH): the chunk's largest |x| sets the exponent; slots r >= B get zero
// limbs.
constexpr int kPreThreads = 256;

template <bool XBF16, bool GROUPED>
__global__ __launch_bounds__(kPreThreads) void limbs_kernel(MItem single, MCommon c) {
    __shared__ float red_m[kPreThreads / 64];
    __shared__ float red_p[kPreThreads / 64];
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
    const int t0 = chunk * a.tpc;
    const int ncol = min(a.tpc, a.n_tiles - t0) * 64;
    const int64_t col0 = (int64_t)t0 * 64;
    const bool live = r < B;
    float m = 0.0f;
    float poison = 0.0f;   // 0 * x summed: NaN exactly when some x is not finite
    if (live)
        for (int k = 4 * T; k < ncol; k += 4 * kPreThreads) {
            const float4 v = x4_value<XBF16>(load_x4_raw<XBF16>(a.x, (int64_t)r * a.K + col0 + k));
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
    if ((T & 63) == 0) {
        red_m[T >> 6] = m;
        red_p[T >> 6] = poison;
    }
    __syncthreads();
    m = red_m[0];
    poison = red_p[0];
#pragma unroll
    for (int w = 1; w < kPreThreads / 64; ++w) {
        m = fmaxf(m, red_m[w]);
        poison += red_p[w];
    }
    const bool nonfinite = poison != 0.0f;   // NaN compares unequal
    int e = 0;
    if (m > 0.0f) frexpf(m, &e);
    if (T == 0) a.exps[chunk * slots + r] = nonfinite ? kBadExp : e;
    const int sh = kFrac - e;
    const float scale = __uint_as_float((uint32_t)(sh + 127) << 23);   // 2^sh when sh <= 126
    const int h = r / SS, rr = r % SS;
    uint8_t* lb = reinterpret_cast<uint8_t*>(a.limbs);
    for (int k = 4 * T; k < ncol; k += 4 * kPreThreads) {
        uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
        if (live && !nonfinite) {
            const float4 v = x4_value<XBF16>(load_x4_raw<XBF16>(a.x, (int64_t)r * a.K + col0 + k));
            if (sh <= 126) {
                w0 = limbs_fast(v.x, scale), w1 = limbs_fast(v.y, scale);
                w2 = limbs_fast(v.z, scale), w3 = limbs_fast(v.w, scale);
            } else {   // every |x| of the chunk below 2^-104
                w0 = limbs_of(v.x, sh), w1 = limbs_of(v.y, sh), w2 = limbs_of(v.z, sh), w3 = limbs_of(v.w, sh);
            }
        }
        const int64_t kk = col0 + k;   // columns kk .. kk+3: one tile, one 16-column slice
        const int64_t t = kk >> 6;
        const int kg = (int)((kk & 63) >> 4);
        const int byte = (int)(kk & 15);
#pragma unroll
        for (int l = 0; l < kLimbs; ++l) {
            const int col = 3 * rr + l;          // B-operand column of this limb
            if (col >= 16 * NCG) break;          // beyond the set's columns (padding slots only)
            const uint32_t word = ((w0 >> (8 * l)) & 0xFFu) | (((w1 >> (8 * l)) & 0xFFu) << 8) |
                                  (((w2 >> (8 * l)) & 0xFFu) << 16) | (((w3 >> (8 * l)) & 0xFFu) << 24);
            const int64_t unit = ((t * NH + h) * NCG + (col >> 4)) * 64 + kg * 16 + (col & 15);
            *reinterpret_cast<uint32_t*>(lb + unit * 16 + byte) = word;
        }
    }
}

// ------------------------------------------------------------------ product

// Tiles in flight: two halves of H tiles, each tile NS weight loads and NCG
// limb loads per lane.
template <int NS, int NCG>
struct MRing {
    static constexpr int H = NS + NCG <= 4 ? 2 : 1;
    static constexpr int PF = 2 * H;
};

template <int NS, int NCG, int H>
__device__ __forceinline__ void mload(u32x4 (&w)[H][NS], v4i (&x)[H][NCG], const uint8_t* wbase, int64_t pb,
                                      int64_t wstride, const v4i* xbase, int64_t xstride, int tile, int last,
                                      int first) {
#pragma unroll
    for (int u = 0; u < H; ++u) {
        const int t = min(tile + u, last);
#pragma unroll
        for (int p = 0; p < NS; ++p)
            w[u][p] = p < first ? u32x4{0u, 0u, 0u, 0u} : load_plane(wbase + p * pb + (int64_t)t * wstride);
#pragma unroll
        for (int g = 0; g < NCG; ++g) x[u][g] = *(global_v4i*)(xbase + t * xstride + g * 64);
    }
}

// One tile: for each depth d present among the set's requests (bit d of
// `dmask`), the codes at depth d times the limbs of the requests reading d
// (mcol[g]: depth of the request owning this lane's column in group g).
template <int NS, int NCG, bool PER_REQ>
__device__ __forceinline__ void mtile(const u32x4 (&w)[NS], const v4i (&xl)[NCG], const int (&mcol)[NCG],
                                      uint32_t dmask, v4i (&acc)[4][NCG]) {
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
            v4i bm[NCG];
#pragma unroll
            for (int g = 0; g < NCG; ++g) {
                if constexpr (PER_REQ) {
                    const bool mine = mcol[g] == p + 1;
                    bm[g] = v4i{mine ? xl[g].x : 0, mine ? xl[g].y : 0, mine ? xl[g].z : 0, mine ? xl[g].w : 0};
                } else {
                    bm[g] = xl[g];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4i A = v4i{(int)q[j][0], (int)rotl32(q[j][1], 2), (int)rotl32(q[j][2], 4),
                                  (int)rotl32(q[j][3], 6)};
#pragma unroll
                for (int g = 0; g < NCG; ++g)
                    acc[j][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, bm[g], acc[j][g], 0, 0, 0);
            }
        }
    }
}

// The product over this wave's tiles of the chunk: tiles ks, ks + KS, ...
template <int NS, int NCG, bool PER_REQ>
__device__ __forceinline__ void mproduct(const MItem& a, int NH, int KS, int b, int chunk, int h, int ks, int L,
                                         const int (&mcol)[NCG], uint32_t dmask, int first, v4i (&acc)[4][NCG]) {

    constexpr int H = MRing<NS, NCG>::H;
    constexpr int PF = MRing<NS, NCG>::PF;
    const int t0 = chunk * a.tpc + ks;
    const int nt_all = min(a.tpc, a.n_tiles - chunk * a.tpc);
    const int nt = nt_all > ks ? (nt_all - ks + KS - 1) / KS : 0;
    if (nt == 0) return;
    const int last = nt - 1;
    const uint8_t* wbase = a.planes + (int64_t)b * 16 * a.K + (int64_t)t0 * kTileBytes + L * 16;
    const int64_t wstride = (int64_t)KS * kTileBytes;
    const int64_t xunit = (int64_t)NH * NCG * 64;        // v4i units per tile
    const v4i* xbase = a.limbs + (int64_t)t0 * xunit + (int64_t)h * NCG * 64 + L;
    const int64_t xstride = xunit * KS;
    const int64_t pb = a.plane_bytes;

    __builtin_amdgcn_s_waitcnt(0);
    u32x4 wa[H][NS], wb[H][NS];
    v4i xa[H][NCG], xb[H][NCG];
    mload<NS, NCG, H>(wa, xa, wbase, pb, wstride, xbase, xstride, 0, last, first);
    __builtin_amdgcn_sched_barrier(0);
    mload<NS, NCG, H>(wb, xb, wbase, pb, wstride, xbase, xstride, H, last, first);
    __builtin_amdgcn_sched_barrier(0);
    int t = 0;
    for (; t + PF < nt; t += PF) {
#pragma unroll
        for (int u = 0; u < H; ++u) mtile<NS, NCG, PER_REQ>(wa[u], xa[u], mcol, dmask, acc);
        __builtin_amdgcn_sched_barrier(0);
        mload<NS, NCG, H>(wa, xa, wbase, pb, wstride, xbase, xstride, t + PF, last, first);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < H; ++u) mtile<NS, NCG, PER_REQ>(wb[u], xb[u], mcol, dmask, acc);
        __builtin_amdgcn_sched_barrier(0);
        mload<NS, NCG, H>(wb, xb, wbase, pb, wstride, xbase, xstride, t + PF + H, last, first);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Drain: the last ring, whose tail may run past the wave's tiles.  Tiles
    // past them were loaded (clamped to the last one) but are multiplied by
    // zero limbs, so the accumulators see the same straight-line code as in
    // the loop.
#pragma unroll
    for (int u = 0; u < H; ++u) {
        const bool in = t + u < nt;
        v4i z[NCG];
#pragma unroll
        for (int g = 0; g < NCG; ++g) z[g] = in ? xa[u][g] : v4i{0, 0, 0, 0};
        mtile<NS, NCG, PER_REQ>(wa[u], z, mcol, dmask, acc);
    }
#pragma unroll
    for (int u = 0; u < H; ++u) {
        const bool in = t + H + u < nt;
        v4i z[NCG];
#pragma unroll
        for (int g = 0; g < NCG; ++g) z[g] = in ? xb[u][g] : v4i{0, 0, 0, 0};
        mtile<NS, NCG, PER_REQ>(wb[u], z, mcol, dmask, acc);
    }
}

// One workgroup = KS x NH wavefronts = one (block, column chunk).
// REFINE: a refinement launch (c.first > 0); without it `first` is the
// constant 0 and the code is that of the plain product.
template <int NCG, bool PER_REQ, bool GROUPED, bool REFINE>
__global__ __launch_bounds__(256) void qmm_kernel(MItem single, MCommon c) {
    extern __shared__ int tab[];   // [KS NH][64 rows][16 NCG + 1] integer sums, then one flag
    constexpr int TW = 16 * NCG + 1;
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
    const int first = REFINE ? c.first : 0;
    const int chunk = local % a.n_chunks;
    const int b = local / a.n_chunks;
    const int wave = (int)threadIdx.x >> 6;
    const int h = wave % NH;
    const int ks = wave / NH;
    const int L = (int)threadIdx.x & 63;

    // depth of request L (lanes < B), then of the set's requests and columns;
    // a refinement launch reads nothing for a request at or below its first slice
    const int m_req = L < B ? depth_of<PER_REQ>(a, L, b) : 0;
    const int m_all = m_req > first ? m_req : 0;
    uint32_t dm_all = 1u << m_all;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) dm_all |= __shfl_xor(dm_all, o);
    dm_all = __builtin_amdgcn_readfirstlane(dm_all);
    if (dm_all == 1u) {   // no request reads any of the block: y = 0 (unchanged when refining), by the first chunk
        if (chunk == 0 && !REFINE)
            for (int r = wave; r < B; r += NH * KS) a.y[(int64_t)r * a.N + (int64_t)b * kRows + L] = 0.0f;
        return;
    }
    const int m_set = __shfl(m_all, (SS * h + (L & 15)) & 63);   // depth of request SS h + (L & 15)
    uint32_t dm = (L < SS && SS * h + L < B) ? (1u << m_set) : 1u;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dm |= __shfl_xor(dm, o);
    dm = __builtin_amdgcn_readfirstlane(dm);
    const int ns = 31 - __builtin_clz(dm);
    int mcol[NCG];
#pragma unroll
    for (int g = 0; g < NCG; ++g) {
        const int rr = (16 * g + (L & 15)) / 3;                 // request (within the set) owning this column
        const int md = __shfl(m_set, rr & 15);                   // its depth (lane rr holds it)
        mcol[g] = (rr < SS && SS * h + rr < B) ? md : 0;
    }
    v4i acc[4][NCG];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < NCG; ++g) acc[j][g] = v4i{0, 0, 0, 0};
    switch (ns) {
        case 0: break;   // no request of this set reads the block
        case 1: mproduct<1, NCG, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, dm, first, acc); break;
        case 2: mproduct<2, NCG, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, dm, first, acc); break;
        case 3: mproduct<3, NCG, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, dm, first, acc); break;
        default: mproduct<4, NCG, PER_REQ>(a, NH, KS, b, chunk, h, ks, L, mcol, dm, first, acc); break;
    }
    // the wave's 64 x 16 NCG integer sums into its table
    int* mine = tab + (ks * NH + h) * 64 * TW;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < NCG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) mine[(16 * j + 4 * (L >> 4) + i) * TW + 16 * g + (L & 15)] = acc[j][g][i];
    __syncthreads();

    // outputs: one row per lane, requests spread over the waves; the limbs of
    // request r are columns 3 (r mod 16) + l of set r / 16, summed over the KS
    // tables (exact integers), then scaled into fp64
    const int row = L;
    const double sc = (double)a.scales[b * kRows + row];
    const int slots = SS * NH;
    const bool split = a.n_chunks > 1;
    for (int r = wave; r < B; r += NH * KS) {
        const int hs = r / SS, c0 = 3 * (r % SS);
        int64_t s0 = 0, s1 = 0, s2 = 0;
        for (int k2 = 0; k2 < KS; ++k2) {
            const int* t2 = tab + (k2 * NH + hs) * 64 * TW + row * TW + c0;
            s0 += t2[0];
            s1 += t2[1];
            s2 += t2[2];
        }
        const double d = (double)s2 * 65536.0 + (double)s1 * 256.0 + (double)s0;
        const int e = a.exps[chunk * slots + r];
        const int mr = __shfl(m_all, r & 63);
        const double v = mr == 0 ? 0.0 : (e == kBadExp ? __builtin_nan("") : ldexp(d, e - kFrac));
        if (!split) {
            float* yo = &a.y[(int64_t)r * a.N + (int64_t)b * kRows + row];
            if constexpr (!REFINE) *yo = (float)(sc * v);
            else if (mr != 0) *yo = (float)((double)*yo + sc * v);
        } else   // split K: publish the partial with a device-scope write-through store
            __hip_atomic_store(&a.partials[((int64_t)chunk * B + r) * a.N + (int64_t)b * kRows + row], v,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!split) return;
    // Once the whole workgroup's partial stores are complete, one thread
    // counts the arrival; the last workgroup of the block sums the partials
    // in chunk order.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int* flag = tab + KS * NH * 64 * TW;
    if (threadIdx.x == 0)
        *flag = (int)__hip_atomic_fetch_add(&a.counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*flag != a.n_chunks - 1) return;
    for (int r = wave; r < B; r += NH * KS) {
        double sum = 0.0;
        for (int cc = 0; cc < a.n_chunks; ++cc)
            sum += __hip_atomic_load(&a.partials[((int64_t)cc * B + r) * a.N + (int64_t)b * kRows + row],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float* yo = &a.y[(int64_t)r * a.N + (int64_t)b * kRows + row];
        if constexpr (!REFINE) *yo = (float)(sc * sum);
        else if (__shfl(m_all, r & 63) != 0) *yo = (float)((double)*yo + sc * sum);
    }
    if (threadIdx.x == 0) __hip_atomic_store(&a.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ per-slice partials

// Per-request maps, the per-slice form: the masked bytes of slice plane p
// (digit 3 - p of every code, in place: bits 7-6 as a signed byte, bits 5-4,
// 3-2 or 1-0 as an unsigned one) add up, over the planes a request reads, to
// its code at its depth, so P_p = plane p's bytes times every request's limbs
// needs no masking, and request r's sum is that of P_p over p < d_r(b).  Wave
// p of a set takes plane p over the chunk's tiles; each plane's partials are
// exact int32, so the order of the sum does not matter.

template <int NCG>
struct PRing {
    static constexpr int H = NCG <= 2 ? 2 : 1;   // tiles per half: 4 + 4 NCG registers each
    static constexpr int PF = 2 * H;
};

template <int NCG, int H>
__device__ __forceinline__ void pload(u32x4 (&w)[H], v4i (&x)[H][NCG], const uint8_t* wbase, const v4i* xbase,
                                      int64_t xunit, int tile, int last) {
#pragma unroll
    for (int u = 0; u < H; ++u) {
        const int t = min(tile + u, last);
        w[u] = load_plane(wbase + (int64_t)t * kTileBytes);
#pragma unroll
        for (int g = 0; g < NCG; ++g) x[u][g] = *(global_v4i*)(xbase + t * xunit + g * 64);
    }
}

template <int P, int NCG>
__device__ __forceinline__ void ptile(const u32x4& w, const v4i (&xl)[NCG], v4i (&acc)[4][NCG]) {
    const uint32_t wj[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const v4i A = v4i{(int)(wj[j] & slice_mask(3 - P, 0)), (int)rotl32(wj[j] & slice_mask(3 - P, 1), 2),
                          (int)rotl32(wj[j] & slice_mask(3 - P, 2), 4), (int)rotl32(wj[j] & slice_mask(3 - P, 3), 6)};
#pragma unroll
        for (int g = 0; g < NCG; ++g) acc[j][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, xl[g], acc[j][g], 0, 0, 0);
    }
}

// Plane P of block b over the chunk's tiles, for request set h.
template <int P, int NCG>
__device__ __forceinline__ void pproduct(const MItem& a, int NH, int b, int chunk, int h, int L, v4i (&acc)[4][NCG]) {
    constexpr int H = PRing<NCG>::H;
    constexpr int PF = PRing<NCG>::PF;
    const int t0 = chunk * a.tpc;
    const int nt = min(a.tpc, a.n_tiles - t0);
    const int last = nt - 1;
    const uint8_t* wbase = a.planes + (int64_t)P * a.plane_bytes + (int64_t)b * 16 * a.K + (int64_t)t0 * kTileBytes +
                           L * 16;
    const int64_t xunit = (int64_t)NH * NCG * 64;
    const v4i* xbase = a.limbs + (int64_t)t0 * xunit + (int64_t)h * NCG * 64 + L;
    __builtin_amdgcn_s_waitcnt(0);
    u32x4 wa[H], wb[H];
    v4i xa[H][NCG], xb[H][NCG];
    pload<NCG, H>(wa, xa, wbase, xbase, xunit, 0, last);
    __builtin_amdgcn_sched_barrier(0);
    pload<NCG, H>(wb, xb, wbase, xbase, xunit, H, last);
    __builtin_amdgcn_sched_barrier(0);
    int t = 0;
    for (; t + PF < nt; t += PF) {
#pragma unroll
        for (int u = 0; u < H; ++u) ptile<P, NCG>(wa[u], xa[u], acc);
        __builtin_amdgcn_sched_barrier(0);
        pload<NCG, H>(wa, xa, wbase, xbase, xunit, t + PF, last);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < H; ++u) ptile<P, NCG>(wb[u], xb[u], acc);
        __builtin_amdgcn_sched_barrier(0);
        pload<NCG, H>(wb, xb, wbase, xbase, xunit, t + PF + H, last);
        __builtin_amdgcn_sched_barrier(0);
    }
    // the last ring: tiles past the chunk were loaded (clamped) and are multiplied by zero limbs
#pragma unroll
    for (int u = 0; u < H; ++u) {
        v4i z[NCG];
#pragma unroll
        for (int g = 0; g < NCG; ++g) z[g] = t + u < nt ? xa[u][g] : v4i{0, 0, 0, 0};
        ptile<P, NCG>(wa[u], z, acc);
    }
#pragma unroll
    for (int u = 0; u < H; ++u) {
        v4i z[NCG];
#pragma unroll
        for (int g = 0; g < NCG; ++g) z[g] = t + H + u < nt ? xb[u][g] : v4i{0, 0, 0, 0};
        ptile<P, NCG>(wb[u], z, acc);
    }
}

// One workgroup = 4 NH wavefronts = one (block, column chunk); wave 4h + p
// takes plane p for request set h.  Each wave keeps only the columns of the
// requests that read its plane and adds them into the set's table (LDS
// integer adds: exact, in any order); then one row per lane, as in qmm_kernel.
template <int NCG, bool GROUPED>
__global__ __launch_bounds__(512) void qmm_plane_kernel(MItem single, MCommon c) {
    extern __shared__ int tab[];   // [NH][64 rows][16 NCG + 1] integer sums, then one flag
    constexpr int TW = 16 * NCG + 1;
    MItem a;
    int local;
    if constexpr (GROUPED) {
        a = c.items[c.wg_item[blockIdx.x]];
        local = (int)blockIdx.x - a.wg_begin;
    } else {
        a = single;
        local = (int)blockIdx.x;
    }
    const int B = c.B, NH = c.NH, SS = c.SS;
    const int chunk = local % a.n_chunks;
    const int b = local / a.n_chunks;
    const int wave = (int)threadIdx.x >> 6;
    const int p = wave & 3;
    const int h = wave >> 2;
    const int L = (int)threadIdx.x & 63;
    const int nw = 4 * NH;

    const int m_all = L < B ? depth_of<true>(a, L, b) : 0;   // slices request L reads
    int dmax = m_all;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) dmax = max(dmax, __shfl_xor(dmax, o));
    dmax = __builtin_amdgcn_readfirstlane(dmax);
    if (dmax == 0) {   // no request reads any of the block: y = 0, written once, by the first chunk
        if (chunk == 0)
            for (int r = wave; r < B; r += nw) a.y[(int64_t)r * a.N + (int64_t)b * kRows + L] = 0.0f;
        return;
    }
    // deepest read in this wave's set, and whether the request owning each of
    // this lane's columns reads plane p
    const int m_set = __shfl(m_all, (SS * h + (L & 15)) & 63);
    int dset = (L < SS && SS * h + L < B) ? m_set : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dset = max(dset, __shfl_xor(dset, o));
    dset = __builtin_amdgcn_readfirstlane(dset);
    bool keep[NCG];
#pragma unroll
    for (int g = 0; g < NCG; ++g) {
        const int rr = (16 * g + (L & 15)) / 3;
        const int md = __shfl(m_set, rr & 15);
        keep[g] = rr < SS && SS * h + rr < B && md > p;
    }
    for (int i = (int)threadIdx.x; i < NH * 64 * TW; i += (int)blockDim.x) tab[i] = 0;
    v4i acc[4][NCG];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < NCG; ++g) acc[j][g] = v4i{0, 0, 0, 0};
    if (p < dset) {
        switch (p) {
            case 0: pproduct<0, NCG>(a, NH, b, chunk, h, L, acc); break;
            case 1: pproduct<1, NCG>(a, NH, b, chunk, h, L, acc); break;
            case 2: pproduct<2, NCG>(a, NH, b, chunk, h, L, acc); break;
            default: pproduct<3, NCG>(a, NH, b, chunk, h, L, acc); break;
        }
    }
    __syncthreads();   // the tables are clear
    if (p < dset) {
        int* mine = tab + h * 64 * TW;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < NCG; ++g)
                if (keep[g])
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        atomicAdd(&mine[(16 * j + 4 * (L >> 4) + i) * TW + 16 * g + (L & 15)], acc[j][g][i]);
    }
    __syncthreads();

    const int row = L;
    const double sc = (double)a.scales[b * kRows + row];
    const int slots = SS * NH;
    const bool split = a.n_chunks > 1;
    for (int r = wave; r < B; r += nw) {
        const int* t2 = tab + (r / SS) * 64 * TW + row * TW + 3 * (r % SS);
        const double d = (double)t2[2] * 65536.0 + (double)t2[1] * 256.0 + (double)t2[0];
        const int e = a.exps[chunk * slots + r];
        const int mr = __shfl(m_all, r & 63);
        const double v = mr == 0 ? 0.0 : (e == kBadExp ? __builtin_nan("") : ldexp(d, e - kFrac));
        if (!split)
            a.y[(int64_t)r * a.N + (int64_t)b * kRows + row] = (float)(sc * v);
        else
            __hip_atomic_store(&a.partials[((int64_t)chunk * B + r) * a.N + (int64_t)b * kRows + row], v,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!split) return;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int* flag = tab + NH * 64 * TW;
    if (threadIdx.x == 0)
        *flag = (int)__hip_atomic_fetch_add(&a.counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*flag != a.n_chunks - 1) return;
    for (int r = wave; r < B; r += nw) {
        double sum = 0.0;
        for (int cc = 0; cc < a.n_chunks; ++cc)
            sum += __hip_atomic_load(&a.partials[((int64_t)cc * B + r) * a.N + (int64_t)b * kRows + row],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.y[(int64_t)r * a.N + (int64_t)b * kRows + row] = (float)(sc * sum);
    }
    if (threadIdx.x == 0) __hip_atomic_store(&a.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ host side

// Per-request maps take the per-slice form up to this many requests, the
// per-depth form above.  0 by default: with 96-tile chunks and four waves
// per set the per-depth form is ahead at every batch measured (4 / 8 / 12 /
// 16 requests: 30 / 36 / 43 / 45 us against 31 / 42 / 48 / 50 us for the
// per-slice form); the per-slice form stays selectable (tuning hook) and
// gives the same bits with the same chunks.
static int g_mfma_per_slice_max = 0;


static bool per_slice_form(int64_t B, bool per_req, int NH) { return per_req && B <= g_mfma_per_slice_max && NH <= 2; }

template <int NCG, bool GROUPED>
static void launch_product(const MItem& it, const MCommon& c, bool per_req, int64_t grid, hipStream_t s) {
    if (per_slice_form(c.B, per_req, c.NH)) {
        const size_t lds = ((size_t)c.NH * 64 * (16 * NCG + 1) + 4) * sizeof(int);
        hipLaunchKernelGGL((qmm_plane_kernel<NCG, GROUPED>), dim3((unsigned)grid), dim3(256 * c.NH), lds, s, it, c);
        return;
    }
    const dim3 blk(64 * c.NH * c.KS);
    const size_t lds = ((size_t)c.KS * c.NH * 64 * (16 * NCG + 1) + 4) * sizeof(int);
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
    switch (c.NCG) {
        case 1: launch_product<1, GROUPED>(it, c, per_req, grid, s); break;
        case 2: launch_product<2, GROUPED>(it, c, per_req, grid, s); break;
        default: launch_product<3, GROUPED>(it, c, per_req, grid, s); break;
    }
}

struct MPlan {
    int NH, SS, NCG, KS, tpc, n_chunks;
    size_t counters, partials, limbs, exps, total;
};

// Wavefronts aimed for per launch (with four waves per set: on the streaming
// stack, two chunks per 28672-column matrix; 337 / 405 us at 4 / 8 requests
// against 370 / 430 us at half the target).
static int64_t g_mfma_target_waves = 256 * 64;
// Shortest column chunk, in tiles per request of the batch (0: by form, see
// mfma_min_tiles): a split of K writes B fp64 partials per row and chunk and
// reads them back, 16 B bytes per row against 64 bytes per row and tile of
// weights at D8, so chunks shorter than a few B tiles spend a large share of
// the traffic on partials.
static int g_mfma_tiles_per_request = 0;
// Waves per request set splitting each chunk's tiles inside a workgroup (at
// most four waves per workgroup): a split inside the workgroup is reduced in
// LDS, one across workgroups through partials in memory.
static int g_mfma_ksplit = 4;

// Most requests per set (three limb columns each, in 16-column groups).
static int g_mfma_set_max = 0;   // 0: the default below; else 8..16
static int mfma_set_max(int64_t) { return g_mfma_set_max ? g_mfma_set_max : 16; }
// request sets, as even as possible
static int mfma_sets(int64_t B) { return (int)((B + mfma_set_max(B) - 1) / mfma_set_max(B)); }
static int mfma_ss(int64_t B) { return (int)((B + mfma_sets(B) - 1) / mfma_sets(B)); }
// 16-column groups per set (three limb columns per request)
static int mfma_ncg(int64_t B) { return (3 * mfma_ss(B) + 15) / 16; }
// waves per set splitting a chunk: at most four waves per workgroup
static int mfma_ks(int64_t B) { return std::max(1, std::min(g_mfma_ksplit, 4 / mfma_sets(B))); }

// Shortest column chunk in tiles.  Measured on the batched layer (4096 and
// 14336 columns) and the streaming stack: per-request maps take chunks of at
// least 96 tiles (per-depth form, 4 / 8 / 12 / 16 / 32 requests: 30 / 36 /
// 43 / 45 / 75 us, against 35 / 42 / 52 / 56 / 90 us with 32-tile chunks);
// shared maps 3 B tiles (404 us against 430 us at 8 requests on the stack).
static int mfma_min_tiles(int64_t B, bool per_req) {
    if (g_mfma_tiles_per_request > 0) return (int)std::min<int64_t>(4096, (int64_t)g_mfma_tiles_per_request * B);
    return per_req ? 96 : (int)(3 * B);
}

// Chunking of one matrix on the pre-pass route, for a chunk length goal.
static MPlan mplan_goal(int64_t N, int64_t K, int64_t B, int goal, bool per_req) {
    MPlan p{};
    p.NH = mfma_sets(B);
    p.SS = mfma_ss(B);
    p.NCG = mfma_ncg(B);
    p.KS = mfma_ks(B);
    const int n_tiles = (int)(K / kTileCols);
    goal = std::max<int>(goal, mfma_min_tiles(B, per_req));
    const int want = (n_tiles + goal - 1) / goal;
    int tpc = (n_tiles + want - 1) / want;
    tpc = (tpc + 3) / 4 * 4;
    if (tpc > n_tiles) tpc = n_tiles;
    p.tpc = tpc;
    p.n_chunks = (n_tiles + tpc - 1) / tpc;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    p.counters = QAM_WS_COUNTER_BYTES;
    p.partials = p.n_chunks > 1 ? up((size_t)p.n_chunks * B * N * sizeof(double)) : 0;
    p.limbs = up((size_t)n_tiles * p.NH * p.NCG * 64 * 16);
    p.exps = up((size_t)p.n_chunks * p.SS * p.NH * sizeof(int));
    p.total = p.counters + p.partials + p.limbs + p.exps;
    return p;
}

static MPlan mplan(int64_t N, int64_t K, int64_t B, bool per_req) {
    const int64_t block_tiles = N / kRows * (K / kTileCols) * mfma_sets(B) * mfma_ks(B);
    return mplan_goal(N, K, B, chunk_goal(block_tiles, g_mfma_target_waves), per_req);
}

static MItem make_mitem(const void* x, const qam_packed* w, const uint8_t* level_map, float* y, int per_request,
                        const MPlan& p) {
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
    return it;
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
    if (!workspace) QAM_FAIL(QAM_ERR_WORKSPACE, "qmatvec: workspace of %zu bytes required", p.total);
    if (workspace_bytes < p.total) QAM_FAIL(QAM_ERR_WORKSPACE, "qmatvec: workspace %zu < %zu bytes", workspace_bytes, p.total);
    if (!aligned(workspace, 256)) QAM_FAIL(QAM_ERR_ALIGN, "qmatvec: workspace must be 256-byte aligned");
    char* ws = static_cast<char*>(workspace);
    MItem it = make_mitem(x, packed, level_map, y, per_request_maps, p);
    it.counters = reinterpret_cast<uint32_t*>(ws);
    it.partials = p.partials ? reinterpret_cast<double*>(ws + p.counters) : nullptr;
    it.limbs = reinterpret_cast<v4i*>(ws + p.counters + p.partials);
    it.exps = reinterpret_cast<int*>(ws + p.counters + p.partials + p.limbs);
    MCommon c{};
    c.B = (int)B;
    c.NH = p.NH;
    c.SS = p.SS;
    c.KS = p.KS;
    c.NCG = p.NCG;
    launch_mfma<false>(it, c, x_dtype == QAM_X_BF16, per_request_maps != 0, (int64_t)p.n_chunks * p.SS * p.NH,
                       (int64_t)it.n_blocks * p.n_chunks, s);
    QAM_HIP_CHECK(hipGetLastError());
    char v[128];
    snprintf(v, sizeof(v), "qmatvec_mfma B=%lld maps=%s form=%s tpc=%d chunks=%d sets=%d colgroups=%d ksplit=%d",
             (long long)B, per_request_maps ? "per-request" : "shared",
             per_slice_form(B, per_request_maps != 0, p.NH) ? "slice" : "depth", p.tpc, p.n_chunks, p.NH, p.NCG, p.KS);
    set_variant(v);
    return QAM_OK;
}

// ------------------------------------------------------------------ grouped launches

struct MGroupLayout {
    std::vector<MPlan> plans;
    size_t partials = 0, limbs = 0, exps = 0, table = 0, wgmap = 0, premap = 0, total = 0;
    int64_t n_wg = 0, n_pre = 0, blocks = 0;
    int NH = 1, SS = 16, NCG = 1, KS = 1;
};

static int mfma_layout(const qam_gemv_item* items, int n_items, int64_t B, bool per_req, MGroupLayout& g) {
    if (!items || n_items < 1) QAM_FAIL(QAM_ERR_ARG, "group: need at least one item");
    if (B < 2 || B > QAM_MAX_BATCH_MFMA) QAM_FAIL(QAM_ERR_ARG, "group: B=%lld outside [2, %d]", (long long)B, QAM_MAX_BATCH_MFMA);
    g.NH = mfma_sets(B);
    g.SS = mfma_ss(B);
    g.NCG = mfma_ncg(B);
    g.KS = mfma_ks(B);
    int64_t block_tiles = 0;
    for (int i = 0; i < n_items; ++i) {
        const qam_packed& w = items[i].w;
        if (w.N <= 0 || w.N % kRows || w.K <= 0 || w.K % kTileCols || w.K > QAM_MAX_K)
            QAM_FAIL(QAM_ERR_SHAPE, "group: item %d has a bad shape", i);
        g.blocks += w.N / kRows;
        block_tiles += w.N / kRows * (w.K / kTileCols) * g.NH * g.KS;
    }
    if (g.blocks > QAM_MAX_BLOCKS) QAM_FAIL(QAM_ERR_SHAPE, "group: %lld blocks > %d", (long long)g.blocks, QAM_MAX_BLOCKS);
    const int goal = chunk_goal(block_tiles, g_mfma_target_waves);
    for (int i = 0; i < n_items; ++i) {
        const MPlan p = mplan_goal(items[i].w.N, items[i].w.K, B, goal, per_req);
        g.plans.push_back(p);
        g.partials += p.partials;
        g.limbs += p.limbs;
        g.exps += p.exps;
        g.n_wg += (int64_t)(items[i].w.N / kRows) * p.n_chunks;
        g.n_pre += (int64_t)p.n_chunks * g.SS * g.NH;
    }
    if (g.n_wg > 0x7FFFFFFF || g.n_pre > 0x7FFFFFFF) QAM_FAIL(QAM_ERR_SHAPE, "group: too many workgroups");
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    g.table = up((size_t)n_items * sizeof(MItem));
    g.wgmap = up((size_t)g.n_wg * sizeof(int));
    g.premap = up((size_t)g.n_pre * sizeof(int));
    g.total = QAM_WS_COUNTER_BYTES + g.partials + g.limbs + g.exps + g.table + g.wgmap + g.premap;
    return QAM_OK;
}

// Device bytes of a group on the pre-pass route: enough for either kind of map.
size_t mfma_group_bytes(const qam_gemv_item* items, int n_items, int64_t B) {
    MGroupLayout g2;
    if (mfma_layout(items, n_items, B, true, g2) != QAM_OK) return 0;
    MGroupLayout g;
    if (mfma_layout(items, n_items, B, false, g) != QAM_OK) return 0;
    g.total = std::max(g.total, g2.total);
    return g.total;
}

int mfma_group_init(const qam_gemv_item* items, int n_items, int64_t B, int x_dtype, int per_request_maps,
                    void* dev_mem, size_t dev_bytes, qam_group* out, hipStream_t s) {
    MGroupLayout g;
    if (int rc = mfma_layout(items, n_items, B, per_request_maps != 0, g)) return rc;
    if (dev_bytes < g.total) QAM_FAIL(QAM_ERR_WORKSPACE, "group_init: %zu < %zu bytes", dev_bytes, g.total);
    if (!aligned(dev_mem, 256)) QAM_FAIL(QAM_ERR_ALIGN, "group_init: device memory must be 256-byte aligned");
    char* base = static_cast<char*>(dev_mem);
    char* partials = base + QAM_WS_COUNTER_BYTES;
    char* limbs = partials + g.partials;
    char* exps = limbs + g.limbs;
    char* table = exps + g.exps;
    char* wgmap = table + g.table;
    char* premap = wgmap + g.wgmap;
    std::vector<MItem> host_items(n_items);
    std::vector<int> hw((size_t)g.n_wg), hp((size_t)g.n_pre);
    int64_t wg = 0, pre = 0, blk = 0;
    size_t po = 0, lo = 0, eo = 0;
    for (int i = 0; i < n_items; ++i) {
        const qam_gemv_item& gi = items[i];
        if (int rc = check_item(gi.x, x_dtype, B, &gi.w, gi.level_map, gi.y, "group_init", QAM_OUT_STORE)) return rc;
        const MPlan& p = g.plans[i];
        if (gi.level_stride < 0 || (gi.level_stride > 0 && gi.level_stride < gi.w.n_blocks))
            QAM_FAIL(QAM_ERR_ARG, "group_init: item %d level_stride %lld < n_blocks", i, (long long)gi.level_stride);
        MItem it = make_mitem(gi.x, &gi.w, gi.level_map, gi.y, per_request_maps, p);
        if (per_request_maps && gi.level_stride > 0) it.level_stride = gi.level_stride;
        it.counters = reinterpret_cast<uint32_t*>(base) + blk;
        it.partials = p.partials ? reinterpret_cast<double*>(partials + po) : nullptr;
        it.limbs = reinterpret_cast<v4i*>(limbs + lo);
        it.exps = reinterpret_cast<int*>(exps + eo);
        po += p.partials;
        lo += p.limbs;
        eo += p.exps;
        blk += it.n_blocks;
        it.wg_begin = (int)wg;
        it.pre_begin = (int)pre;
        const int64_t n = (int64_t)it.n_blocks * p.n_chunks;
        for (int64_t k = 0; k < n; ++k) hw[(size_t)(wg + k)] = i;
        wg += n;
        const int64_t np = (int64_t)p.n_chunks * g.SS * g.NH;
        for (int64_t k = 0; k < np; ++k) hp[(size_t)(pre + k)] = i;
        pre += np;
        host_items[i] = it;
    }
    QAM_HIP_CHECK(hipMemsetAsync(base, 0, QAM_WS_COUNTER_BYTES, s));
    QAM_HIP_CHECK(hipMemcpyAsync(table, host_items.data(), sizeof(MItem) * n_items, hipMemcpyHostToDevice, s));
    QAM_HIP_CHECK(hipMemcpyAsync(wgmap, hw.data(), sizeof(int) * hw.size(), hipMemcpyHostToDevice, s));
    QAM_HIP_CHECK(hipMemcpyAsync(premap, hp.data(), sizeof(int) * hp.size(), hipMemcpyHostToDevice, s));
    QAM_HIP_CHECK(hipStreamSynchronize(s));
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
    out->sets = g.NH;
    out->set_size = g.SS;
    out->col_groups = g.NCG;
    return QAM_OK;
}

// first > 0: a refinement launch (slices first.. of each request's depth added to y).
static int mfma_group_run_from(const qam_group* g, int first, hipStream_t s) {
    if (g->sets < 1 || g->sets > 4 || g->set_size < 1 || g->set_size > 16 || (int64_t)g->sets * g->set_size < g->B ||
        g->col_groups < 1 || g->col_groups > 3 || 3 * g->set_size > 16 * g->col_groups)
        QAM_FAIL(QAM_ERR_ARG, "qmatvec_group: corrupt group descriptor");
    MCommon c{};
    c.items = static_cast<const MItem*>(g->table);
    c.wg_item = static_cast<const int*>(g->wg_map);
    c.pre_item = static_cast<const int*>(g->pre_map);
    c.B = (int)g->B;
    c.NH = g->sets;
    c.SS = g->set_size;
    c.NCG = g->col_groups;
    c.KS = std::max(1, std::min(g_mfma_ksplit, 4 / c.NH));
    c.first = first;
    MItem dummy{};
    launch_mfma<true>(dummy, c, g->x_dtype == QAM_X_BF16, g->per_request_maps != 0, g->n_pre_workgroups,
                      g->n_workgroups, s);
    QAM_HIP_CHECK(hipGetLastError());
    char v[128];
    snprintf(v, sizeof(v), "qmatvec_mfma_group%s items=%d B=%lld maps=%s form=%s wg=%lld", first ? "_refine" : "",
             g->n_items, (long long)g->B,
             g->per_request_maps ? "per-request" : "shared",
             per_slice_form(g->B, g->per_request_maps != 0, g->sets) ? "slice" : "depth", (long long)g->n_workgroups);
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
    if (qam::per_slice_form(group->B, group->per_request_maps != 0, group->sets))
        QAM_FAIL(QAM_ERR_ARG, "qmatvec_group_refine: not available in the per-slice form");
    return qam::mfma_group_run_from(group, first_slice, s);
}

extern "C" int qam_set_mfma_per_slice_max(int b) {
    qam::clear_error();
    if (b < 0 || b > QAM_MAX_BATCH_MFMA) QAM_FAIL(QAM_ERR_ARG, "set_mfma_per_slice_max: %d outside [0, %d]", b,
                                                  QAM_MAX_BATCH_MFMA);
    qam::g_mfma_per_slice_max = b;
    return QAM_OK;
}

extern "C" int qam_set_mfma_set_max(int n) {
    qam::clear_error();
    if (n != 0 && (n < 8 || n > 16)) QAM_FAIL(QAM_ERR_ARG, "set_mfma_set_max: %d not 0 or in [8, 16]", n);
    qam::g_mfma_set_max = n;
    return QAM_OK;
}

extern "C" int qam_set_mfma_ksplit(int ks) {
    qam::clear_error();
    if (ks != 1 && ks != 2 && ks != 4) QAM_FAIL(QAM_ERR_ARG, "set_mfma_ksplit: %d not 1, 2 or 4", ks);
    qam::g_mfma_ksplit = ks;
    return QAM_OK;
}

extern "C" int qam_set_mfma_tiles_per_request(int t) {
    qam::clear_error();
    if (t < 0 || t > 64) QAM_FAIL(QAM_ERR_ARG, "set_mfma_tiles_per_request: %d outside [0, 64]", t);
    qam::g_mfma_tiles_per_request = t;
    return QAM_OK;
}

extern "C" int qam_set_mfma_target_waves(int waves) {
    qam::clear_error();
    if (waves < 64 || waves > (1 << 20)) QAM_FAIL(QAM_ERR_ARG, "set_mfma_target_waves: %d outside [64, 2^20]", waves);
    qam::g_mfma_target_waves = waves;
    return QAM_OK;
}

