// The escalation gate on the device: entropy and top-two margin of the low
// pass's output distribution ("Precision on Demand: Escalating Weight Bits at
// Uncertain Decoding Steps in a Small Local Model", abstract: redo a step at
// 8 bits when the low-precision output looks uncertain, entropy above a
// threshold or a small top-two margin).
//
// With m = max z, e_i = exp(z_i - m), S = sum e_i and T = sum e_i (z_i - m),
// the softmax entropy -sum p ln p is ln S - T / S, and the largest
// probability is 1 / S.  Each workgroup reduces its slice of the logits to
// (m_g, S_g, T_g, its top two) relative to its own maximum; the last
// workgroup to finish rescales them to the global maximum, in slice order,
// and writes the result.  Every sum has a fixed order, so the result is the
// same bits on every call.
#include <math.h>

#include "qam_common.h"

namespace qam {

constexpr int kGateThreads = 256;
constexpr int kGateMaxGroups = 256;   // at most one partial per thread of the merging workgroup
constexpr int64_t kGatePerGroup = 1024;   // logits per workgroup (at most kGateMaxGroups groups)
constexpr int kGateBatch = 4;             // loads a thread has in flight

struct GatePartial {
    double m, S, T;        // max of the slice, sum of exp(z - m), sum of exp(z - m) (z - m)
    float v1, v2;          // the slice's two largest logits ...
    int32_t i1, i2;        // ... and their indices (ties to the lower index)
    int32_t bad;           // a NaN or +inf in the slice
    int32_t pad;
};

static_assert(sizeof(GatePartial) == 48, "partial layout");
static_assert(kGateMaxGroups <= kGateThreads, "the merge takes one partial per thread");

// (v, i) ranks ahead of (w, j): larger value, or equal value and lower index.
__device__ __forceinline__ bool ahead(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

// Merge the top two (a1, a2) with (b1, b2) into (a1, a2).
__device__ __forceinline__ void merge2(float& a1, int& ai1, float& a2, int& ai2, float b1, int bi1, float b2, int bi2) {
    if (ahead(b1, bi1, a1, ai1)) {
        // b1 leads; the runner-up is the better of a1 and b2
        if (ahead(a1, ai1, b2, bi2)) {
            a2 = a1;
            ai2 = ai1;
        } else {
            a2 = b2;
            ai2 = bi2;
        }
        a1 = b1;
        ai1 = bi1;
    } else if (ahead(b1, bi1, a2, ai2)) {
        a2 = b1;
        ai2 = bi1;
    }
}

// Sum over the workgroup in a fixed tree order; every thread gets the sum.
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double s = red[0];
    for (int k = 1; k < kGateThreads / 64; ++k) s += red[k];
    return s;
}

// Maximum over the workgroup; every thread gets it.
__device__ __forceinline__ double block_max(double v, double* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double s = red[0];
    for (int k = 1; k < kGateThreads / 64; ++k) s = fmax(s, red[k]);
    return s;
}

// The top two (and the NaN / +inf flag) over the workgroup; every thread gets them.
struct Top2 {
    float v1, v2;
    int i1, i2;
    int bad;
};
__device__ __forceinline__ void block_top2(Top2& t, Top2* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float b1 = __shfl_xor(t.v1, o), b2 = __shfl_xor(t.v2, o);
        const int bi1 = __shfl_xor(t.i1, o), bi2 = __shfl_xor(t.i2, o);
        merge2(t.v1, t.i1, t.v2, t.i2, b1, bi1, b2, bi2);
        t.bad |= __shfl_xor(t.bad, o);
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = t;
    __syncthreads();
    t = red[0];
    for (int k = 1; k < kGateThreads / 64; ++k) {
        merge2(t.v1, t.i1, t.v2, t.i2, red[k].v1, red[k].i1, red[k].v2, red[k].i2);
        t.bad |= red[k].bad;
    }
}

__global__ __launch_bounds__(kGateThreads) void gate_kernel(const float* __restrict__ z, int64_t V, int64_t per,
                                                            double tau_h, double tau_m, GatePartial* parts,
                                                            uint32_t* counter, qam_uncertainty* out) {
    constexpr int NW = kGateThreads / 64;
    __shared__ double red[NW];
    __shared__ Top2 tred[NW];
    __shared__ int last;
    const int g = blockIdx.x;
    const int64_t lo = (int64_t)g * per;
    const int64_t hi = min(V, lo + per);
    const int T = threadIdx.x;

    // pass 1: the slice's top two (the first is its maximum) and whether it
    // holds a NaN or +inf
    float v1 = -INFINITY, v2 = -INFINITY;
    int i1 = INT32_MAX, i2 = INT32_MAX;
    int bad = 0;
    float keep[kGateBatch];   // the first batch, reused by pass 2 (the whole slice when it fits)
    for (int64_t k0 = lo + T; k0 < hi; k0 += kGateBatch * kGateThreads) {
        float v[kGateBatch];
#pragma unroll
        for (int j = 0; j < kGateBatch; ++j) {   // the batch's loads go out together
            const int64_t k = k0 + (int64_t)j * kGateThreads;
            v[j] = k < hi ? z[k] : -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < kGateBatch; ++j) {
            const int64_t k = k0 + (int64_t)j * kGateThreads;
            if (k < hi) {
                if (isnan(v[j]) || v[j] == INFINITY) bad = 1;
                merge2(v1, i1, v2, i2, v[j], (int)k, -INFINITY, INT32_MAX);
            }
            if (k0 == lo + T) keep[j] = v[j];
        }
    }
    Top2 tp{v1, v2, i1, i2, bad};
    block_top2(tp, tred);
    v1 = tp.v1, v2 = tp.v2, i1 = tp.i1, i2 = tp.i2, bad = tp.bad;

    // pass 2: sums relative to the slice's maximum (-inf logits add nothing)
    const double md = (double)v1;
    double S = 0.0, Tt = 0.0;
    if (v1 != -INFINITY && !bad) {
        for (int64_t k0 = lo + T; k0 < hi; k0 += kGateBatch * kGateThreads) {
            float v[kGateBatch];
#pragma unroll
            for (int j = 0; j < kGateBatch; ++j) {
                const int64_t k = k0 + (int64_t)j * kGateThreads;
                v[j] = k0 == lo + T ? keep[j] : (k < hi ? z[k] : -INFINITY);
            }
#pragma unroll
            for (int j = 0; j < kGateBatch; ++j) {   // in index order, as loaded
                const double d = (double)v[j] - md;
                if (d != -INFINITY) {
                    const double e = exp(d);
                    S += e;
                    Tt += e * d;
                }
            }
        }
    }
    S = block_sum(S, red);
    Tt = block_sum(Tt, red);

    if (T == 0) {
        GatePartial* pp = parts + g;
        __hip_atomic_store(&pp->m, md, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&pp->S, S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&pp->T, Tt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&pp->v1, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&pp->v2, v2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&pp->i1, i1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&pp->i2, i2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&pp->bad, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the partial is stored before it is counted: the signal fences keep
        // the compiler from moving the stores past the wait or the counter
        // update (they emit no instruction), and the wait holds the hardware
        // to it (device-scope stores are written through to L2 in order of
        // completion, and the counter update is issued after they complete)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        last = (int)(__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     gridDim.x - 1);
    }
    __syncthreads();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // no partial load moves ahead of the count
    if (!last) return;

    // the last workgroup: every partial is in; thread k takes partial k
    // (G <= the workgroup size) and the workgroup reduces them in a fixed
    // tree order
    const int G = (int)gridDim.x;
    double mk = -INFINITY, Sk = 0.0, Tk = 0.0;
    Top2 tk{-INFINITY, -INFINITY, INT32_MAX, INT32_MAX, 0};
    if (T < G) {
        const GatePartial* pp = parts + T;
        mk = __hip_atomic_load(&pp->m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        Sk = __hip_atomic_load(&pp->S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        Tk = __hip_atomic_load(&pp->T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tk.v1 = __hip_atomic_load(&pp->v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tk.v2 = __hip_atomic_load(&pp->v2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tk.i1 = __hip_atomic_load(&pp->i1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tk.i2 = __hip_atomic_load(&pp->i2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tk.bad = __hip_atomic_load(&pp->bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const double M = block_max(mk, red);
    block_top2(tk, tred);
    // each slice's sums rescaled to the global maximum (an all -inf slice adds nothing)
    double Sc = 0.0, Tc = 0.0;
    if (T < G && mk != -INFINITY && M != -INFINITY && !tk.bad) {
        const double sh = mk - M;   // <= 0
        const double f = exp(sh);
        Sc = f * Sk;
        Tc = f * (Tk + sh * Sk);
    }
    const double Sa = block_sum(Sc, red);
    const double Ta = block_sum(Tc, red);
    if (T != 0) return;
    qam_uncertainty r{};
    r.top1 = tk.i1;
    r.top2 = tk.i2;
    if (tk.bad || M == -INFINITY) {
        r.entropy = r.margin = r.p1 = r.p2 = __builtin_nan("");
        r.escalate = 1;
    } else {
        r.entropy = log(Sa) - Ta / Sa;
        r.p1 = 1.0 / Sa;
        r.p2 = exp((double)tk.v2 - M) / Sa;
        r.margin = r.p1 - r.p2;
        r.escalate = (r.entropy > tau_h || r.margin < tau_m) ? 1 : 0;
    }
    *out = r;
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static int gate_groups(int64_t V) {
    const int64_t g = (V + kGatePerGroup - 1) / kGatePerGroup;
    return (int)std::max<int64_t>(1, std::min<int64_t>(kGateMaxGroups, g));
}

}  // namespace qam

using namespace qam;

extern "C" size_t qam_gate_workspace_bytes(int64_t V) {
    if (V < 2 || V > INT32_MAX - 1) return 0;
    return 256 + (size_t)gate_groups(V) * sizeof(GatePartial);
}

extern "C" int qam_gate(const float* logits, int64_t V, double tau_entropy, double tau_margin, qam_uncertainty* out,
                        void* workspace, size_t workspace_bytes, hipStream_t s) {
    clear_error();
    if (!logits || !out || !workspace) QAM_FAIL(QAM_ERR_NULL, "gate: null pointer");
    if (V < 2 || V > INT32_MAX - 1) QAM_FAIL(QAM_ERR_SHAPE, "gate: V=%lld outside [2, 2^31 - 2]", (long long)V);
    if (isnan(tau_entropy) || isnan(tau_margin)) QAM_FAIL(QAM_ERR_ARG, "gate: NaN threshold");
    const size_t need = qam_gate_workspace_bytes(V);
    if (workspace_bytes < need) QAM_FAIL(QAM_ERR_WORKSPACE, "gate: workspace %zu < %zu bytes", workspace_bytes, need);
    if (!aligned(workspace, 256) || !aligned(logits, 4) || !aligned(out, 8))
        QAM_FAIL(QAM_ERR_ALIGN, "gate: workspace must be 256-byte, logits 4-byte and out 8-byte aligned");
    const int G = gate_groups(V);
    const int64_t per = (V + G - 1) / G;
    uint32_t* counter = static_cast<uint32_t*>(workspace);
    GatePartial* parts = reinterpret_cast<GatePartial*>(static_cast<char*>(workspace) + 256);
    hipLaunchKernelGGL(gate_kernel, dim3((unsigned)G), dim3(kGateThreads), 0, s, logits, V, per, tau_entropy,
                       tau_margin, parts, counter, out);
    QAM_HIP_CHECK(hipGetLastError());
    set_variant("gate_fp64");
    return QAM_OK;
}
