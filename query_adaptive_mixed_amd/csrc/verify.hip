// Draft and verify: the decoder's chain for a batch of requests (the verify
// pass), a row argmax, and the greedy draft-and-verify loop.
//
// [PoD] "Precision on Demand" abstract: speculation verified at full depth
// reaches the full-depth output at a similar weight-byte cost.  The draft
// is the stored stack read at a low rung, the target the same stack at a
// high rung; one batched verify pass reads every block once for all the
// drafted positions.

#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "decoder_internal.h"

using namespace qam;

struct qam_verifier {
    qam_decoder* dec = nullptr;
    int max_batch = 0;
    int64_t H = 0, Q = 0, KV = 0, F = 0, V = 0;
    float *x = nullptr, *h = nullptr, *qkv = nullptr, *m = nullptr, *xn = nullptr, *y = nullptr,
          *logits = nullptr;
    char* ws = nullptr;
    size_t ws_bytes = 0;
    uint64_t* keys = nullptr;     // [max_batch + 1] argmax keys, zero between uses
    int32_t* drafts = nullptr;    // [max_batch]
    int32_t* round = nullptr;     // [max_batch + 2]: count, then the round's tokens
    hipGraph_t graph[5][17] = {};   // captured verify passes by (rung, B)
    hipGraphExec_t exec[5][17] = {};
    ~qam_verifier() {
        for (int r = 0; r < 5; ++r)
            for (int b = 0; b < 17; ++b) {
                if (exec[r][b]) (void)hipGraphExecDestroy(exec[r][b]);
                if (graph[r][b]) (void)hipGraphDestroy(graph[r][b]);
            }
    }
};

namespace {

constexpr size_t kAlign = 256;
constexpr int kGlueThreads = 256;
constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxPerBlock = kArgmaxThreads * 16;
size_t up256(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ------------------------------------------------------------------ device

__device__ double block_sum(double v, double* red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x / 64, l = threadIdx.x % 64;
    if (l == 0) red[w] = v;
    __syncthreads();
    double t = 0.0;
    for (int i = 0; i < kGlueThreads / 64; ++i) t += red[i];   // same order in every thread
    __syncthreads();
    return t;
}

enum GlueMode { kInit = 0, kAddNorm = 1, kGlu = 2 };

struct GlueArgs {
    const float* x;    // kInit: inputs [B][n]; kAddNorm, kGlu: y [B][ld]
    float* h;          // residual [B][n] (kInit, kAddNorm)
    float* out;        // kInit, kAddNorm: x' [B][n]; kGlu: m [B][n]
    int64_t n;         // row length written
    int64_t ld;        // row stride of x
    double eps;
};

// One workgroup per request row.
template <int MODE>
__global__ void __launch_bounds__(kGlueThreads) glue_kernel(GlueArgs a) {
    __shared__ double red[kGlueThreads / 64];
    const int64_t r = blockIdx.x;
    const int64_t n = a.n;
    if constexpr (MODE == kGlu) {
        // block b of the gate|up product: rows 64b..64b+31 gate, 64b+32..64b+63 up
        for (int64_t j = threadIdx.x; j < n; j += kGlueThreads) {
            const int64_t b = j / 32, i = j % 32;
            const double g = a.x[r * a.ld + 64 * b + i];
            const double u = a.x[r * a.ld + 64 * b + 32 + i];
            a.out[r * n + j] = (float)(g / (1.0 + exp(-g)) * u);
        }
        return;
    } else {
        double ss = 0.0;
        for (int64_t i = threadIdx.x; i < n; i += kGlueThreads) {
            float v;
            if constexpr (MODE == kInit) v = a.x[r * n + i];
            else v = a.h[r * n + i] + a.x[r * a.ld + i];
            a.h[r * n + i] = v;
            ss += (double)v * (double)v;
        }
        const double inv = 1.0 / sqrt(block_sum(ss, red) / (double)n + a.eps);
        for (int64_t i = threadIdx.x; i < n; i += kGlueThreads)
            a.out[r * n + i] = (float)((double)a.h[r * n + i] * inv);
    }
}

// Orderable key: larger float first, then the smaller index.
__device__ __forceinline__ uint64_t argmax_key(float f, uint32_t i) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - i);
}

__device__ __forceinline__ int32_t key_index(uint64_t k) { return (int32_t)(0xFFFFFFFFu - (uint32_t)k); }

// grid (ceil(n / kArgmaxPerBlock), rows): each workgroup folds its slice of a
// row into keys[row] with one 64-bit atomic max.
__global__ void __launch_bounds__(kArgmaxThreads) argmax_kernel(const float* v, int64_t n, int64_t ld,
                                                                 uint64_t* keys) {
    __shared__ uint64_t red[kArgmaxThreads / 64];
    const int64_t row = blockIdx.y;
    const int64_t lo = (int64_t)blockIdx.x * kArgmaxPerBlock;
    const int64_t hi = std::min<int64_t>(n, lo + kArgmaxPerBlock);
    uint64_t best = 0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kArgmaxThreads) {
        const uint64_t k = argmax_key(v[row * ld + i], (uint32_t)i);
        best = k > best ? k : best;
    }
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t t = __shfl_xor(best, o);
        best = t > best ? t : best;
    }
    if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kArgmaxThreads / 64; ++w) best = red[w] > best ? red[w] : best;
        atomicMax(reinterpret_cast<unsigned long long*>(&keys[row]), (unsigned long long)best);
    }
}

// idx[r] from keys[r], which are set back to zero.
__global__ void argmax_finish_kernel(uint64_t* keys, int64_t rows, int32_t* idx) {
    for (int64_t r = threadIdx.x; r < rows; r += blockDim.x) {
        idx[r] = key_index(keys[r]);
        keys[r] = 0;
    }
}

// A draft step's token: dst = E[token], token recorded, key cleared.
__global__ void __launch_bounds__(kGlueThreads) embed_kernel(uint64_t* key, const float* E, int64_t H, float* dst,
                                                              int32_t* token_out) {
    __shared__ int32_t tok;
    if (threadIdx.x == 0) {
        tok = key_index(*key);
        *key = 0;
        *token_out = tok;
    }
    __syncthreads();
    for (int64_t i = threadIdx.x; i < H; i += kGlueThreads) dst[i] = E[(int64_t)tok * H + i];
}

// The verify decision: keys[0..k] hold the target's tokens after inputs
// 0..k, drafts[0..k-1] the drafts.  Keeps the agreeing prefix, emits the
// target's token after it, writes the next input row x0 = E[that token].
__global__ void __launch_bounds__(kGlueThreads) accept_kernel(uint64_t* keys, const int32_t* drafts, int k,
                                                               const float* E, int64_t H, float* x0,
                                                               int32_t* round_out) {
    __shared__ int32_t next;
    if (threadIdx.x == 0) {
        int j = 0;
        while (j < k && key_index(keys[j]) == drafts[j]) ++j;
        for (int i = 0; i < j; ++i) round_out[1 + i] = drafts[i];
        next = key_index(keys[j]);
        round_out[1 + j] = next;
        round_out[0] = j + 1;
        for (int i = 0; i <= k; ++i) keys[i] = 0;
    }
    __syncthreads();
    for (int64_t i = threadIdx.x; i < H; i += kGlueThreads) x0[i] = E[(int64_t)next * H + i];
}

// ------------------------------------------------------------------ host

struct VLayout {
    size_t ws = 0, x = 0, h = 0, qkv = 0, m = 0, xn = 0, y = 0, logits = 0, keys = 0, drafts = 0, round = 0,
           total = 0, ws_bytes = 0;
};

int vlayout(const qam_decoder_desc* d, int max_batch, VLayout& lo) {
    if (!d) QAM_FAIL(QAM_ERR_NULL, "verifier: null description");
    if (max_batch < 1 || max_batch > 16) QAM_FAIL(QAM_ERR_ARG, "verifier: max_batch=%d outside [1, 16]", max_batch);
    if (qam_decoder_bytes(d) == 0) QAM_FAIL(QAM_ERR_SHAPE, "verifier: invalid decoder description");
    const int64_t H = d->hidden, Q = d->q_dim, KV = d->kv_dim, F = d->ffn, V = d->vocab, B = max_batch;
    const int64_t shapes[5][2] = {{Q + 2 * KV, H}, {H, Q}, {2 * F, H}, {H, F}, {V, H}};
    size_t ws = 0;
    for (int64_t b = 1; b <= B; ++b)
        for (const auto& sh : shapes) {
            const size_t need = qam_qmatvec_workspace_bytes(sh[0], sh[1], b);
            if (need == 0) QAM_FAIL(QAM_ERR_SHAPE, "verifier: no workspace for %lld x %lld", (long long)sh[0],
                                    (long long)sh[1]);
            ws = std::max(ws, need);
        }
    size_t off = 0;
    lo.ws = off;      off += up256(ws);
    lo.ws_bytes = up256(ws);
    lo.x = off;       off += up256((size_t)B * H * 4);
    lo.h = off;       off += up256((size_t)B * H * 4);
    lo.qkv = off;     off += up256((size_t)B * (Q + 2 * KV) * 4);
    lo.m = off;       off += up256((size_t)B * F * 4);
    lo.xn = off;      off += up256((size_t)B * H * 4);
    lo.y = off;       off += up256((size_t)B * std::max(H, 2 * F) * 4);
    lo.logits = off;  off += up256((size_t)B * V * 4);
    lo.keys = off;    off += up256((size_t)(B + 1) * 8);
    lo.drafts = off;  off += up256((size_t)B * 4);
    lo.round = off;   off += up256((size_t)(B + 2) * 4);
    lo.total = off;
    return QAM_OK;
}

template <int MODE>
int glue(const qam_verifier* v, int B, const float* x, float* h, float* out, int64_t n, int64_t ld, hipStream_t s) {
    GlueArgs a{x, h, out, n, ld, v->dec->d.eps};
    hipLaunchKernelGGL(glue_kernel<MODE>, dim3((unsigned)B), dim3(kGlueThreads), 0, s, a);
    QAM_HIP_CHECK(hipGetLastError());
    return QAM_OK;
}

int product(qam_verifier* v, int rung, int B, const qam_packed& w, const float* x, float* y, hipStream_t s) {
    return qam_qmatvec(x, QAM_X_F32, B, &w, v->dec->maps[rung], 0, y, v->ws, v->ws_bytes, s);
}

// A product of the chain with its input's elementwise step: at B = 1 a glue
// kernel and the staged product, from two requests on the pre-pass route's
// pre-pass, which forms the product's input itself.
int product_in(qam_verifier* v, int rung, int B, const qam_packed& w, const XIn& in, const float* x, float* y,
               hipStream_t s) {
    if (B > 1) return qmatvec_mfma_in(x, B, &w, v->dec->maps[rung], y, in, v->ws, v->ws_bytes, s);
    const int64_t K = w.K;
    int rc = QAM_OK;
    switch (in.mode) {
        case kXStrided:   // row stride is moot for one row
            return product(v, rung, B, w, x, y, s);
        case kXAddNorm:
            rc = glue<kAddNorm>(v, B, in.add, in.res, in.side, K, K, s);
            break;
        case kXGated:
            rc = glue<kGlu>(v, B, x, nullptr, in.side, K, in.ld, s);
            break;
        default:
            return product(v, rung, B, w, x, y, s);
    }
    return rc ? rc : product(v, rung, B, w, in.side, y, s);
}

// The chain, op by op (n_layers L):
//   op 0            h = x; xn = rmsnorm(h)
//   op 1 + 4l       layer l > 0: h += y, xn = rmsnorm(h); then qkv = Wqkv xn
//   op 2 + 4l       y = Wo q (q: the first q_dim columns of qkv)
//   op 3 + 4l       h += y, xn = rmsnorm(h); y = Wgu xn
//   op 4 + 4l       m = silu(gate) up of y; y = Wdown m
//   op 4L + 1       h += y, xn = rmsnorm(h); logits = Whead xn
// Each op forms its own input from the previous op's output, so the
// elementwise steps ride in the products' pre-passes.
int run_ops(qam_verifier* v, int rung, int B, int first, int count, hipStream_t s) {
    const int n_ops = 4 * v->dec->d.n_layers + 2;
    if (rung < 0 || rung > 4) QAM_FAIL(QAM_ERR_ARG, "verifier: rung %d outside 0..4", rung);
    if (B < 1 || B > v->max_batch) QAM_FAIL(QAM_ERR_ARG, "verifier: B=%d outside [1, %d]", B, v->max_batch);
    if (first < 0 || count < 0 || first > n_ops || count > n_ops - first)
        QAM_FAIL(QAM_ERR_ARG, "verifier: ops [%d, %d) outside the chain of %d", first, first + count, n_ops);
    const int64_t H = v->H, Q = v->Q, KV = v->KV, F = v->F;
    XIn add_norm;   // h += y, xn = rmsnorm(h)
    add_norm.mode = kXAddNorm;
    add_norm.add = v->y;
    add_norm.res = v->h;
    add_norm.side = v->xn;
    add_norm.eps = v->dec->d.eps;
    XIn strided_q;
    strided_q.mode = kXStrided;
    strided_q.ld = Q + 2 * KV;
    XIn gated;
    gated.mode = kXGated;
    gated.ld = 2 * F;
    gated.side = v->m;
    for (int op = first; op < first + count; ++op) {
        int rc = QAM_OK;
        if (op == 0) {
            rc = glue<kInit>(v, B, v->x, v->h, v->xn, H, H, s);
        } else if (op == n_ops - 1) {
            rc = product_in(v, rung, B, v->dec->d.lm_head, add_norm, v->h, v->logits, s);
        } else {
            const qam_decoder_layer& L = v->dec->layers[(size_t)(op - 1) / 4];
            switch ((op - 1) % 4) {
                case 0:
                    rc = op == 1 ? product(v, rung, B, L.qkv, v->xn, v->qkv, s)
                                 : product_in(v, rung, B, L.qkv, add_norm, v->h, v->qkv, s);
                    break;
                case 1: rc = product_in(v, rung, B, L.o, strided_q, v->qkv, v->y, s); break;
                case 2: rc = product_in(v, rung, B, L.gate_up, add_norm, v->h, v->y, s); break;
                default: rc = product_in(v, rung, B, L.down, gated, v->y, v->y, s); break;
            }
        }
        if (rc) return rc;
    }
    return QAM_OK;
}

int launch_argmax(const float* x, int64_t rows, int64_t n, int64_t ld, uint64_t* keys, hipStream_t s) {
    const unsigned chunks = (unsigned)((n + kArgmaxPerBlock - 1) / kArgmaxPerBlock);
    hipLaunchKernelGGL(argmax_kernel, dim3(chunks, (unsigned)rows), dim3(kArgmaxThreads), 0, s, x, n, ld, keys);
    QAM_HIP_CHECK(hipGetLastError());
    return QAM_OK;
}

}  // namespace

extern "C" size_t qam_verifier_bytes(const qam_decoder_desc* d, int max_batch) {
    VLayout lo;
    if (vlayout(d, max_batch, lo) != QAM_OK) return 0;
    return lo.total;
}

extern "C" int qam_verifier_create(qam_decoder* dec, int max_batch, void* dev_mem, size_t dev_bytes,
                                   qam_verifier** out, hipStream_t s) {
    clear_error();
    if (!dec || !dev_mem || !out) QAM_FAIL(QAM_ERR_NULL, "verifier_create: null pointer");
    *out = nullptr;
    VLayout lo;
    if (int rc = vlayout(&dec->d, max_batch, lo)) return rc;
    if (dev_bytes < lo.total) QAM_FAIL(QAM_ERR_WORKSPACE, "verifier_create: %zu < %zu bytes", dev_bytes, lo.total);
    if (!aligned(dev_mem, kAlign)) QAM_FAIL(QAM_ERR_ALIGN, "verifier_create: device memory must be 256-byte aligned");
    qam_verifier* v = new (std::nothrow) qam_verifier();
    if (!v) QAM_FAIL(QAM_ERR_ARG, "verifier_create: out of host memory");
    char* base = static_cast<char*>(dev_mem);
    v->dec = dec;
    v->max_batch = max_batch;
    v->H = dec->d.hidden, v->Q = dec->d.q_dim, v->KV = dec->d.kv_dim, v->F = dec->d.ffn, v->V = dec->d.vocab;
    v->ws = base + lo.ws;
    v->ws_bytes = lo.ws_bytes;
    v->x = reinterpret_cast<float*>(base + lo.x);
    v->h = reinterpret_cast<float*>(base + lo.h);
    v->qkv = reinterpret_cast<float*>(base + lo.qkv);
    v->m = reinterpret_cast<float*>(base + lo.m);
    v->xn = reinterpret_cast<float*>(base + lo.xn);
    v->y = reinterpret_cast<float*>(base + lo.y);
    v->logits = reinterpret_cast<float*>(base + lo.logits);
    v->keys = reinterpret_cast<uint64_t*>(base + lo.keys);
    v->drafts = reinterpret_cast<int32_t*>(base + lo.drafts);
    v->round = reinterpret_cast<int32_t*>(base + lo.round);
    hipError_t e = hipMemsetAsync(v->ws, 0, QAM_WS_COUNTER_BYTES, s);
    if (e == hipSuccess) e = hipMemsetAsync(v->keys, 0, (size_t)(max_batch + 1) * 8, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        delete v;
        QAM_FAIL(QAM_ERR_HIP, "verifier_create: %s", hipGetErrorString(e));
    }
    *out = v;
    return QAM_OK;
}

extern "C" float* qam_verifier_buffer(qam_verifier* v, int which) {
    if (!v) return nullptr;
    switch (which) {
        case QAM_VER_X: return v->x;
        case QAM_VER_H: return v->h;
        case QAM_VER_QKV: return v->qkv;
        case QAM_VER_M: return v->m;
        case QAM_VER_XN: return v->xn;
        case QAM_VER_LOGITS: return v->logits;
        case QAM_VER_Y: return v->y;
        default: return nullptr;
    }
}

extern "C" int qam_verifier_run(qam_verifier* v, int rung, int B, int first, int count, hipStream_t s) {
    clear_error();
    if (!v) QAM_FAIL(QAM_ERR_NULL, "verifier_run: null verifier");
    return run_ops(v, rung, B, first, count, s);
}

extern "C" int qam_verifier_step(qam_verifier* v, int rung, int B, hipStream_t s) {
    clear_error();
    if (!v) QAM_FAIL(QAM_ERR_NULL, "verifier_step: null verifier");
    if (int rc = run_ops(v, rung, B, 0, 4 * v->dec->d.n_layers + 2, s)) return rc;
    char buf[96];
    snprintf(buf, sizeof(buf), "verifier_step rung=%d B=%d", rung, B);
    set_variant(buf);
    return QAM_OK;
}

extern "C" int qam_verifier_capture(qam_verifier* v, int rung, int B, hipStream_t s) {
    clear_error();
    if (!v) QAM_FAIL(QAM_ERR_NULL, "verifier_capture: null verifier");
    if (!s) QAM_FAIL(QAM_ERR_ARG, "verifier_capture: the null stream cannot be captured");
    if (rung < 0 || rung > 4 || B < 1 || B > v->max_batch)
        QAM_FAIL(QAM_ERR_ARG, "verifier_capture: rung %d / B %d out of range", rung, B);
    QAM_HIP_CHECK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    const int rc = run_ops(v, rung, B, 0, 4 * v->dec->d.n_layers + 2, s);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &g);
    if (rc != QAM_OK) {
        if (g) (void)hipGraphDestroy(g);
        return rc;
    }
    if (e != hipSuccess) QAM_FAIL(QAM_ERR_HIP, "verifier_capture: %s", hipGetErrorString(e));
    hipGraphExec_t x = nullptr;
    const hipError_t ei = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (ei != hipSuccess) {
        (void)hipGraphDestroy(g);
        QAM_FAIL(QAM_ERR_HIP, "verifier_capture: instantiate: %s", hipGetErrorString(ei));
    }
    if (v->exec[rung][B]) (void)hipGraphExecDestroy(v->exec[rung][B]);
    if (v->graph[rung][B]) (void)hipGraphDestroy(v->graph[rung][B]);
    v->graph[rung][B] = g;
    v->exec[rung][B] = x;
    return QAM_OK;
}

extern "C" int qam_verifier_replay(qam_verifier* v, int rung, int B, hipStream_t s) {
    clear_error();
    if (!v) QAM_FAIL(QAM_ERR_NULL, "verifier_replay: null verifier");
    if (rung < 0 || rung > 4 || B < 1 || B > v->max_batch || !v->exec[rung][B])
        QAM_FAIL(QAM_ERR_ARG, "verifier_replay: rung %d, B %d was not captured", rung, B);
    QAM_HIP_CHECK(hipGraphLaunch(v->exec[rung][B], s));
    return QAM_OK;
}

extern "C" void qam_verifier_destroy(qam_verifier* v) { delete v; }

extern "C" int qam_argmax_rows(const float* v, int64_t rows, int64_t n, int64_t ld, int32_t* idx_out,
                               void* workspace, hipStream_t s) {
    clear_error();
    if (!v || !idx_out || !workspace) QAM_FAIL(QAM_ERR_NULL, "argmax_rows: null pointer");
    if (rows < 1 || rows > 65535 || n < 1 || n >= ((int64_t)1 << 31) || ld < n)
        QAM_FAIL(QAM_ERR_ARG, "argmax_rows: rows=%lld n=%lld ld=%lld", (long long)rows, (long long)n, (long long)ld);
    if (!aligned(workspace, 8) || !aligned(v, 4) || !aligned(idx_out, 4))
        QAM_FAIL(QAM_ERR_ALIGN, "argmax_rows: misaligned pointer");
    uint64_t* keys = static_cast<uint64_t*>(workspace);
    if (int rc = launch_argmax(v, rows, n, ld, keys, s)) return rc;
    hipLaunchKernelGGL(argmax_finish_kernel, dim3(1), dim3(256), 0, s, keys, rows, idx_out);
    QAM_HIP_CHECK(hipGetLastError());
    set_variant("argmax_rows");
    return QAM_OK;
}

extern "C" int qam_decoder_speculate(qam_decoder* dec, qam_verifier* v, const float* embed, int32_t first_token,
                                     int n_tokens, int k, int draft_rung, int verify_rung, int32_t* tokens_out,
                                     qam_spec_stats* stats, hipStream_t s) {
    clear_error();
    if (!dec || !v || !embed || (!tokens_out && n_tokens > 0)) QAM_FAIL(QAM_ERR_NULL, "speculate: null pointer");
    if (v->dec != dec) QAM_FAIL(QAM_ERR_ARG, "speculate: the verifier belongs to another decoder");
    if (k < 1 || k > v->max_batch - 1) QAM_FAIL(QAM_ERR_ARG, "speculate: k=%d outside [1, %d]", k, v->max_batch - 1);
    if (n_tokens < 0) QAM_FAIL(QAM_ERR_ARG, "speculate: n_tokens < 0");
    if (first_token < 0 || first_token >= v->V) QAM_FAIL(QAM_ERR_ARG, "speculate: first_token %d outside the vocab", first_token);
    for (int r : {draft_rung, verify_rung})
        if (r < 0 || r > 4) QAM_FAIL(QAM_ERR_ARG, "speculate: rung %d outside 0..4", r);
    if (!aligned(embed, 4)) QAM_FAIL(QAM_ERR_ALIGN, "speculate: embed not 4-byte aligned");
    const int64_t H = v->H, V = v->V;
    qam_spec_stats st{};
    std::vector<int32_t> round((size_t)v->max_batch + 2);
    QAM_HIP_CHECK(hipMemcpyAsync(v->x, embed + (int64_t)first_token * H, H * sizeof(float),
                                 hipMemcpyDeviceToDevice, s));
    int64_t have = 0;
    while (have < n_tokens) {
        for (int i = 1; i <= k; ++i) {
            QAM_HIP_CHECK(hipMemcpyAsync(dec->h, v->x + (int64_t)(i - 1) * H, H * sizeof(float),
                                         hipMemcpyDeviceToDevice, s));
            if (dec->exec[draft_rung]) {
                QAM_HIP_CHECK(hipGraphLaunch(dec->exec[draft_rung], s));
            } else if (int rc = qam_decoder_run(dec, draft_rung, 0, 4 * dec->d.n_layers + 1, s)) {
                return rc;
            }
            uint64_t* dkey = v->keys + v->max_batch;
            if (int rc = launch_argmax(dec->logits, 1, V, V, dkey, s)) return rc;
            hipLaunchKernelGGL(embed_kernel, dim3(1), dim3(kGlueThreads), 0, s, dkey, embed, H, v->x + (int64_t)i * H,
                               v->drafts + (i - 1));
            QAM_HIP_CHECK(hipGetLastError());
        }
        if (v->exec[verify_rung][k + 1]) {
            QAM_HIP_CHECK(hipGraphLaunch(v->exec[verify_rung][k + 1], s));
        } else if (int rc = run_ops(v, verify_rung, k + 1, 0, 4 * dec->d.n_layers + 2, s)) {
            return rc;
        }
        if (int rc = launch_argmax(v->logits, k + 1, V, V, v->keys, s)) return rc;
        hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(kGlueThreads), 0, s, v->keys, v->drafts, k, embed, H, v->x,
                           v->round);
        QAM_HIP_CHECK(hipGetLastError());
        QAM_HIP_CHECK(hipMemcpyAsync(round.data(), v->round, (size_t)(k + 2) * sizeof(int32_t),
                                     hipMemcpyDeviceToHost, s));
        QAM_HIP_CHECK(hipStreamSynchronize(s));
        const int got = round[0];
        if (got < 1 || got > k + 1) QAM_FAIL(QAM_ERR_HIP, "speculate: round emitted %d tokens", got);
        for (int i = 0; i < got && have < n_tokens; ++i) tokens_out[have++] = round[(size_t)1 + i];
        st.rounds += 1;
        st.draft_steps += k;
        st.drafted += k;
        st.accepted += got - 1;
        st.emitted += got;
    }
    if (stats) *stats = st;
    char buf[96];
    snprintf(buf, sizeof(buf), "decoder_speculate k=%d rungs=%d/%d", k, draft_rung, verify_rung);
    set_variant(buf);
    return QAM_OK;
}
