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
// in one launch (nb^2 / 256 comparisons per thread); larger ones rank over
// many workgroups after the score launch.
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

// Share rule for a request of at most kLayerFusedMax blocks, one workgroup
// per request: the scores go to LDS (and shat), then each block's rank is
// counted there.
__global__ void __launch_bounds__(kLayerThreads)
layer_share_fused_kernel(const float* __restrict__ y, const float* __restrict__ scales, int64_t nb, int64_t N,
                         double w, int64_t k, int glass, int kappa, double* __restrict__ shat,
                         uint8_t* __restrict__ level) {
    __shared__ double sc[kLayerFusedMax];
    const int64_t r = blockIdx.x;
    for (int64_t c = threadIdx.x; c < nb; c += kLayerThreads) {
        const double score = block_score(y, scales, r, c, N, w);
        shat[r * nb + c] = score;
        sc[c] = score;
    }
    __syncthreads();
    for (int64_t c = threadIdx.x; c < nb; c += kLayerThreads) {
        const double key = sc[c];
        int64_t rank = 0;
        for (int64_t b = 0; b < nb; ++b) rank += ranks_ahead(sc[b], b, key, c);
        level[r * nb + c] = (uint8_t)((!isnan(key) && rank < k) ? kappa : glass);
    }
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

}  // namespace qam

using namespace qam;

extern "C" int qam_layer_levels(const float* y_base, int64_t B, const qam_packed* w, const qam_layer_rule* rule,
                                int n_rungs, int glass, double* shat_out, uint8_t* level_out, hipStream_t s) {
    clear_error();
    if (!w || !rule || !w->scales || ((!y_base || !shat_out || !level_out) && B > 0))
        QAM_FAIL(QAM_ERR_NULL, "layer_levels: null pointer");
    const int64_t N = w->N, K = w->K, nb = w->n_blocks;
    if (N <= 0 || K <= 0 || N % 64 || K % 64 || K > QAM_MAX_K || nb != N / 64 || nb > QAM_MAX_BLOCKS)
        QAM_FAIL(QAM_ERR_SHAPE, "layer_levels: bad packed shape N=%lld K=%lld", (long long)N, (long long)K);
    if (B < 0 || B > 65535) QAM_FAIL(QAM_ERR_ARG, "layer_levels: B=%lld outside [0, 65535]", (long long)B);
    if (n_rungs < 1 || n_rungs > QAM_MAX_RUNGS || glass < 0 || glass >= n_rungs)
        QAM_FAIL(QAM_ERR_LADDER, "layer_levels: glass %d outside a ladder of %d rungs", glass, n_rungs);
    if (rule->mode != QAM_LAYER_THRESHOLD && rule->mode != QAM_LAYER_SHARE)
        QAM_FAIL(QAM_ERR_ARG, "layer_levels: unknown mode %d", rule->mode);
    if (!(rule->g >= 0.0 && rule->g <= 1.0)) QAM_FAIL(QAM_ERR_ARG, "layer_levels: g outside [0, 1]");
    if (rule->mode == QAM_LAYER_THRESHOLD && isnan(rule->lambda))
        QAM_FAIL(QAM_ERR_ARG, "layer_levels: lambda is NaN");
    if (rule->mode == QAM_LAYER_SHARE && !(rule->share >= 0.0 && rule->share <= 1.0))
        QAM_FAIL(QAM_ERR_ARG, "layer_levels: share outside [0, 1]");
    if (!aligned(y_base, 16) || !aligned(w->scales, 16) || !aligned(shat_out, 8))
        QAM_FAIL(QAM_ERR_ALIGN, "layer_levels: y_base and scales must be 16-byte, shat_out 8-byte aligned");
    const int m = n_rungs - 1;
    const int kappa = glass + (int)floor(rule->g * (double)(m - glass));
    if (B == 0) {
        set_variant("layer_levels");
        return QAM_OK;
    }
    const double wc = (double)(64 * K);
    if (rule->mode == QAM_LAYER_SHARE && nb <= kLayerFusedMax) {
        const int64_t k = (int64_t)floor(rule->share * (double)nb);
        hipLaunchKernelGGL(layer_share_fused_kernel, dim3((unsigned)B), dim3(kLayerThreads), 0, s, y_base,
                           w->scales, nb, N, wc, k, glass, kappa, shat_out, level_out);
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
