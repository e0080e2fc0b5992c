// Level maps decided by the layer itself from its own read at the base depth
// (FoQLens, section "FoQZones, the mechanism", the variant in which the layer
// decides): each block of 64 output rows gets the reduced draft score
//   s^_c = ((|y_c|^2 Delta_c^2) Delta_c^2) / w_c,
// with y_c its 64 outputs of the base read, Delta_c^2 the mean squared row
// scale of its rows (the step of the stored 8-bit codes) and w_c = 64 K its
// weights, and then a rung:
//   threshold: glass + #{j in 1 .. kappa - glass : s^ >= lambda 16^j};
//   share:     the floor(f n_blocks) blocks of largest s^ (equal scores in
//              block order, NaN never) rise to kappa, the rest stay at the
//              glass;
// kappa = glass + floor(g (m - glass)).  Scores and levels stay on the device.
//
// The score is fp64 with the rows summed in order (the squares of fp32 values
// are exact in fp64) and, like every file of the library, compiled with
// -ffp-contract=off, so it is the same bits as the same sums written out on a
// CPU; the rungs then follow from exact comparisons.
#include <math.h>

#include "qam_common.h"

namespace qam {

constexpr int kLayerThreads = 256;

// Requests of at most this many blocks are scored and ranked by one workgroup
// of layer_group_kernel in one launch (nb^2 / 1024 comparisons per thread);
// larger ones rank over many workgroups after the score launch.
constexpr int64_t kLayerFusedMax = 512;

// The reduced score of block c of request r: its 64 outputs and 64 scales
// are 16 float4 loads each (a block's rows are contiguous, 256 bytes), all
// issued before the sums, which run over the rows in order.
__device__ __forceinline__ double block_score(const float* __restrict__ y, const float* __restrict__ scales,
                                              int64_t r, int64_t c, int64_t N, double w) {
    const float4* yv = reinterpret_cast<const float4*>(y + r * N + c * 64);
    const float4* sv = reinterpret_cast<const float4*>(scales + c * 64);
    float4 a[16], s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        a[i] = yv[i];
        s[i] = sv[i];
    }
    double energy = 0.0, step2 = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        energy = energy + (double)a[i].x * (double)a[i].x;
        energy = energy + (double)a[i].y * (double)a[i].y;
        energy = energy + (double)a[i].z * (double)a[i].z;
        energy = energy + (double)a[i].w * (double)a[i].w;
        step2 = step2 + (double)s[i].x * (double)s[i].x;
        step2 = step2 + (double)s[i].y * (double)s[i].y;
        step2 = step2 + (double)s[i].z * (double)s[i].z;
        step2 = step2 + (double)s[i].w * (double)s[i].w;
    }
    step2 = step2 / 64.0;
    const double draft = energy * step2;
    return (draft * step2) / w;
}

// Threshold rule on a score: glass + #{j in 1 .. lifts : score >= lambda 16^j}.
__device__ __forceinline__ int threshold_rung(double score, double lambda, int glass, int lifts) {
    int lv = glass;
    for (int j = 1; j <= lifts; ++j)
        if (score >= lambda * ldexp(1.0, 4 * j)) ++lv;
    return lv;
}

// (v, b) ranks ahead of (key, c): larger score, or equal score and lower index.
__device__ __forceinline__ bool ranks_ahead(double v, int64_t b, double key, int64_t c) {
    return v > key || (v == key && b < c);
}

// Blocks of sc[lo, hi) ahead of (key, c), hi <= kLayerFusedMax: four
// independent counts (integer, so their order does not matter), so that
// several LDS reads are in flight at once.
__device__ __forceinline__ int count_ahead_range(const double* sc, int lo, int hi, double key, int c) {
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
    int b = lo;
    for (; b + 4 <= hi; b += 4) {
        r0 += ranks_ahead(sc[b], b, key, c);
        r1 += ranks_ahead(sc[b + 1], b + 1, key, c);
        r2 += ranks_ahead(sc[b + 2], b + 2, key, c);
        r3 += ranks_ahead(sc[b + 3], b + 3, key, c);
    }
    for (; b < hi; ++b) r0 += ranks_ahead(sc[b], b, key, c);
    return r0 + r1 + r2 + r3;
}


// One thread per (request, block): the score and, in threshold mode, the rung.
__global__ void __launch_bounds__(kLayerThreads)
layer_score_kernel(const float* __restrict__ y, const float* __restrict__ scales, int64_t B, int64_t nb,
                   int64_t N, double w, int mode, double lambda, int glass, int lifts, double* __restrict__ shat,
                   uint8_t* __restrict__ level) {
    const int64_t idx = (int64_t)blockIdx.x * kLayerThreads + threadIdx.x;
    if (idx >= B * nb) return;
    const int64_t r = idx / nb, c = idx - r * nb;
    const double score = block_score(y, scales, r, c, N, w);
    shat[idx] = score;
    if (mode == QAM_LAYER_THRESHOLD) level[idx] = (uint8_t)threshold_rung(score, lambda, glass, lifts);
}

// Share rule: one thread per (request, block); its rank is the number of
// blocks of the request ahead of it (larger score, or equal score and lower
// index), counted over the request's scores staged through LDS.
__global__ void __launch_bounds__(kLayerThreads)
layer_share_kernel(const double* __restrict__ shat, int64_t nb, int64_t k, int glass, int kappa,
                   uint8_t* __restrict__ level) {
    __shared__ double tile[kLayerThreads];
    const int64_t r = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * kLayerThreads + threadIdx.x;
    const double* row = shat + r * nb;
    const double key = c < nb ? row[c] : NAN;
    int64_t rank = 0;
    for (int64_t b0 = 0; b0 < nb; b0 += kLayerThreads) {
        const int64_t b = b0 + threadIdx.x;
        tile[threadIdx.x] = b < nb ? row[b] : NAN;
        __syncthreads();
        const int n = (int)(nb - b0 < kLayerThreads ? nb - b0 : kLayerThreads);
        for (int t = 0; t < n; ++t) {
            const double v = tile[t];
            rank += ranks_ahead(v, b0 + t, key, c);
        }
        __syncthreads();
    }
    if (c < nb) level[r * nb + c] = (uint8_t)((!isnan(key) && rank < k) ? kappa : glass);
}

// One matrix of a grouped call, as the kernel sees it.
struct LayerItem {
    const float* y;
    const float* scales;
    double* shat;
    uint8_t* level;
    int64_t N, nb;
    double w;
    int64_t k;            // share mode: blocks that rise per request
};

struct LayerGroupArgs {
    LayerItem items[QAM_LAYER_GROUP_MAX];
    int64_t B;
    int mode, glass, lifts, kappa;
    double lambda;
};

constexpr int kLayerGroupThreads = 1024;

// Every matrix of a group in one launch: a workgroup per (item, request),
// each scoring that request's blocks (at most kLayerFusedMax) and, in share
// mode, ranking them in LDS, four adjacent lanes per block each counting a
// quarter of the blocks (integer counts, summed by two lane shuffles); the
// same arithmetic as the single-matrix kernels.
__global__ void __launch_bounds__(kLayerGroupThreads) layer_group_kernel(LayerGroupArgs g) {
    __shared__ double sc[kLayerFusedMax];
    const int64_t item = blockIdx.x / g.B, r = blockIdx.x - item * g.B;
    const LayerItem& it = g.items[item];
    const int64_t nb = it.nb;
    for (int64_t c = threadIdx.x; c < nb; c += kLayerGroupThreads) {
        const double score = block_score(it.y, it.scales, r, c, it.N, it.w);
        it.shat[r * nb + c] = score;
        if (g.mode == QAM_LAYER_THRESHOLD) it.level[r * nb + c] = (uint8_t)threshold_rung(score, g.lambda, g.glass, g.lifts);
        else sc[c] = score;
    }
    if (g.mode == QAM_LAYER_THRESHOLD) return;
    __syncthreads();
    const int n = (int)nb;
    // 4 n (block, quarter) pairs; the trip count is the same for every lane
    for (int base = 0; base < 4 * n; base += kLayerGroupThreads) {
        const int idx = base + (int)threadIdx.x;
        const bool on = idx < 4 * n;
        const int c = idx >> 2, q = idx & 3;
        const double key = on ? sc[c] : 0.0;
        int part = on ? count_ahead_range(sc, (q * n) >> 2, ((q + 1) * n) >> 2, key, c) : 0;
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        if (on && q == 0) it.level[r * nb + c] = (uint8_t)((!isnan(key) && part < it.k) ? g.kappa : g.glass);
    }
}

}  // namespace qam

using namespace qam;

// Checks shared by the entry points (error text names `who`).
static int check_layer(const qam_packed* w, int64_t B, const qam_layer_rule* rule, int n_rungs, int glass,
                       const char* who) {
    const int64_t N = w->N, K = w->K, nb = w->n_blocks;
    if (!w->scales) QAM_FAIL(QAM_ERR_NULL, "%s: null scales", who);
    if (N <= 0 || K <= 0 || N % 64 || K % 64 || K > QAM_MAX_K || nb != N / 64 || nb > QAM_MAX_BLOCKS)
        QAM_FAIL(QAM_ERR_SHAPE, "%s: bad packed shape N=%lld K=%lld", who, (long long)N, (long long)K);
    if (B < 0 || B > 65535) QAM_FAIL(QAM_ERR_ARG, "%s: B=%lld outside [0, 65535]", who, (long long)B);
    if (n_rungs < 1 || n_rungs > QAM_MAX_RUNGS || glass < 0 || glass >= n_rungs)
        QAM_FAIL(QAM_ERR_LADDER, "%s: glass %d outside a ladder of %d rungs", who, glass, n_rungs);
    if (rule->mode != QAM_LAYER_THRESHOLD && rule->mode != QAM_LAYER_SHARE)
        QAM_FAIL(QAM_ERR_ARG, "%s: unknown mode %d", who, rule->mode);
    if (!(rule->g >= 0.0 && rule->g <= 1.0)) QAM_FAIL(QAM_ERR_ARG, "%s: g outside [0, 1]", who);
    if (rule->mode == QAM_LAYER_THRESHOLD && isnan(rule->lambda)) QAM_FAIL(QAM_ERR_ARG, "%s: lambda is NaN", who);
    if (rule->mode == QAM_LAYER_SHARE && !(rule->share >= 0.0 && rule->share <= 1.0))
        QAM_FAIL(QAM_ERR_ARG, "%s: share outside [0, 1]", who);
    if (!aligned(w->scales, 16)) QAM_FAIL(QAM_ERR_ALIGN, "%s: scales must be 16-byte aligned", who);
    return QAM_OK;
}

extern "C" int qam_layer_levels(const float* y_base, int64_t B, const qam_packed* w, const qam_layer_rule* rule,
                                int n_rungs, int glass, double* shat_out, uint8_t* level_out, hipStream_t s) {
    clear_error();
    if (!w || !rule || ((!y_base || !shat_out || !level_out) && B > 0))
        QAM_FAIL(QAM_ERR_NULL, "layer_levels: null pointer");
    if (int rc = check_layer(w, B, rule, n_rungs, glass, "layer_levels")) return rc;
    if (!aligned(y_base, 16) || !aligned(shat_out, 8))
        QAM_FAIL(QAM_ERR_ALIGN, "layer_levels: y_base must be 16-byte, shat_out 8-byte aligned");
    const int64_t N = w->N, K = w->K, nb = w->n_blocks;
    const int m = n_rungs - 1;
    const int kappa = glass + (int)floor(rule->g * (double)(m - glass));
    if (B == 0) {
        set_variant("layer_levels");
        return QAM_OK;
    }
    const double wc = (double)(64 * K);
    if (rule->mode == QAM_LAYER_SHARE && nb <= kLayerFusedMax) {
        // one workgroup per request scores and ranks its blocks: the grouped kernel with one item
        LayerGroupArgs g{};
        LayerItem& it = g.items[0];
        it.y = y_base;
        it.scales = w->scales;
        it.shat = shat_out;
        it.level = level_out;
        it.N = N;
        it.nb = nb;
        it.w = wc;
        it.k = (int64_t)floor(rule->share * (double)nb);
        g.B = B;
        g.mode = rule->mode;
        g.glass = glass;
        g.lifts = kappa - glass;
        g.kappa = kappa;
        g.lambda = rule->lambda;
        hipLaunchKernelGGL(layer_group_kernel, dim3((unsigned)B), dim3(kLayerGroupThreads), 0, s, g);
        QAM_HIP_CHECK(hipGetLastError());
        set_variant("layer_levels_share_fused");
        return QAM_OK;
    }
    const int64_t n = B * nb;
    const unsigned grid = (unsigned)((n + kLayerThreads - 1) / kLayerThreads);
    hipLaunchKernelGGL(layer_score_kernel, dim3(grid), dim3(kLayerThreads), 0, s, y_base, w->scales, B, nb, N, wc,
                       rule->mode, rule->lambda, glass, kappa - glass, shat_out, level_out);
    QAM_HIP_CHECK(hipGetLastError());
    if (rule->mode == QAM_LAYER_SHARE) {
        const int64_t k = (int64_t)floor(rule->share * (double)nb);
        const dim3 g2((unsigned)((nb + kLayerThreads - 1) / kLayerThreads), (unsigned)B);
        hipLaunchKernelGGL(layer_share_kernel, g2, dim3(kLayerThreads), 0, s, shat_out, nb, k, glass, kappa,
                           level_out);
        QAM_HIP_CHECK(hipGetLastError());
    }
    set_variant(rule->mode == QAM_LAYER_SHARE ? "layer_levels_share" : "layer_levels_threshold");
    return QAM_OK;
}

extern "C" int qam_layer_levels_group(const qam_layer_item* items, int n_items, int64_t B,
                                      const qam_layer_rule* rule, int n_rungs, int glass, hipStream_t s) {
    clear_error();
    if (!items || !rule) QAM_FAIL(QAM_ERR_NULL, "layer_levels_group: null pointer");
    if (n_items < 1 || n_items > QAM_LAYER_GROUP_MAX)
        QAM_FAIL(QAM_ERR_ARG, "layer_levels_group: %d items outside [1, %d]", n_items, QAM_LAYER_GROUP_MAX);
    LayerGroupArgs g{};
    for (int i = 0; i < n_items; ++i) {
        const qam_layer_item& q = items[i];
        if ((!q.y_base || !q.shat_out || !q.level_out) && B > 0)
            QAM_FAIL(QAM_ERR_NULL, "layer_levels_group: item %d: null pointer", i);
        if (int rc = check_layer(&q.w, B, rule, n_rungs, glass, "layer_levels_group")) return rc;
        if (q.w.n_blocks > kLayerFusedMax)
            QAM_FAIL(QAM_ERR_SHAPE, "layer_levels_group: item %d has %lld blocks, more than %lld", i,
                     (long long)q.w.n_blocks, (long long)kLayerFusedMax);
        if (!aligned(q.y_base, 16) || !aligned(q.shat_out, 8))
            QAM_FAIL(QAM_ERR_ALIGN, "layer_levels_group: item %d: y_base must be 16-byte, shat_out 8-byte aligned", i);
        LayerItem& it = g.items[i];
        it.y = q.y_base;
        it.scales = q.w.scales;
        it.shat = q.shat_out;
        it.level = q.level_out;
        it.N = q.w.N;
        it.nb = q.w.n_blocks;
        it.w = (double)(64 * q.w.K);
        it.k = (int64_t)floor(rule->share * (double)q.w.n_blocks);
    }
    const int kappa = glass + (int)floor(rule->g * (double)(n_rungs - 1 - glass));
    g.B = B;
    g.mode = rule->mode;
    g.glass = glass;
    g.lifts = kappa - glass;
    g.kappa = kappa;
    g.lambda = rule->lambda;
    if (B > 0) {
        hipLaunchKernelGGL(layer_group_kernel, dim3((unsigned)(n_items * B)), dim3(kLayerGroupThreads), 0, s, g);
        QAM_HIP_CHECK(hipGetLastError());
    }
    set_variant("layer_levels_group");
    return QAM_OK;
}
