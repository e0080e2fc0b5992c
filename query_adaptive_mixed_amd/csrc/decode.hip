// Decode driver: one step of a decoder-only model as a chain of mixed-depth
// products with fused epilogues, eager or replayed from a HIP graph, and the
// host-side escalation schedule.
//
// [PoD] "Precision on Demand" abstract: 8-bit weights are stored once, each
// step is decoded with their top 4 bits, and a step whose output looks
// uncertain is decoded again at 8 bits; cost is counted in weight bytes read
// per token.  In the ladder {0,2,4,6,8} those two depths are rungs 2 and 4,
// every block at the same rung.

#include <algorithm>
#include <cmath>
#include <new>
#include <numeric>
#include <vector>

#include "decoder_internal.h"

using namespace qam;

namespace {

constexpr size_t kAlign = 256;
// Longest column chunk of a step's products, in tiles: a product with few
// row blocks and many columns (the down projection) is cut into several
// chunks so that its waves stay short.
size_t up256(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// The five launches of one layer (or the lm_head) in chain order.
struct Op {
    const qam_packed* w;
    const float* x;
    float* y;
    int rms, out_mode;
    int kind;   // 0 q|k|v, 1 o, 2 gate|up, 3 down, 4 the head
};

std::vector<Op> chain(const qam_decoder& dec) {
    std::vector<Op> ops;
    ops.reserve(4 * dec.layers.size() + 1);
    for (const qam_decoder_layer& L : dec.layers) {
        ops.push_back({&L.qkv, dec.h, dec.qkv, 1, QAM_OUT_STORE, 0});
        ops.push_back({&L.o, dec.qkv, dec.h, 0, QAM_OUT_ADD, 1});
        ops.push_back({&L.gate_up, dec.h, dec.m, 1, QAM_OUT_GLU, 2});
        ops.push_back({&L.down, dec.m, dec.h, 0, QAM_OUT_ADD, 3});
    }
    ops.push_back({&dec.d.lm_head, dec.h, dec.logits, 1, QAM_OUT_STORE, 4});
    return ops;
}

// Launch shape of each kind of product: waves per (block, chunk) and the
// longest column chunk in tiles.  The description's waves_per_block and
// max_chunk_tiles, when set, apply to every product.  By default the o
// projection (few blocks) takes up to 32 tiles in one chunk over 8 waves, so
// that it needs no split-K hand-off; the head (thousands of blocks) runs one
// wave per block; the others run 4 waves over chunks of at most 16 tiles.  On
// the Qwen3-0.6B shapes these defaults make a D4 step 0.675 ms against 0.699
// ms with 4 waves and 16-tile chunks everywhere.
struct OpShape {
    int ks, max_chunk;
};

OpShape op_shape(const qam_decoder_desc& d, int kind) {
    static const OpShape def[5] = {{4, 16}, {8, 32}, {4, 16}, {4, 16}, {1, 16}};
    OpShape sh = def[kind];
    if (d.waves_per_block) sh.ks = d.waves_per_block;
    if (d.max_chunk_tiles) sh.max_chunk = d.max_chunk_tiles;
    return sh;
}

Plan plan_of(const qam_packed& w, int64_t target_waves, int max_chunk) {
    // chunks of whole D8 rings (2 tiles) so that small matrices spread over
    // many wavefronts: a decode step is a chain of short, latency-bound launches
    return make_plan(w.N, w.K, chunk_goal(w.n_blocks * (w.K / kTileCols), target_waves, max_chunk), 2);
}

bool same_shape(const qam_packed& w, int64_t N, int64_t K) {
    return w.N == N && w.K == K && w.n_blocks == N / kRows && w.planes &&
           w.scales == reinterpret_cast<float*>(static_cast<char*>(w.planes) + N * K);
}

struct Layout {
    size_t ws = 0, h = 0, qkv = 0, m = 0, logits = 0, maps = 0, total = 0;
    int64_t max_blocks = 0;
};

int layout(const qam_decoder_desc* d, Layout& lo) {
    if (!d || !d->layers) QAM_FAIL(QAM_ERR_NULL, "decoder: null description");
    if (d->n_layers < 1 || d->n_layers > 4096) QAM_FAIL(QAM_ERR_ARG, "decoder: n_layers=%d", d->n_layers);
    const int64_t H = d->hidden, Q = d->q_dim, KV = d->kv_dim, F = d->ffn, V = d->vocab;
    if (H <= 0 || Q <= 0 || KV <= 0 || F <= 0 || V <= 0 || H % 64 || Q % 64 || KV % 64 || F % 32 || V % 64 ||
        H > QAM_MAX_K || Q > QAM_MAX_K || F > QAM_MAX_K)
        QAM_FAIL(QAM_ERR_SHAPE, "decoder: hidden, q_dim, kv_dim, vocab must be multiples of 64 and ffn of 32");
    if (!(d->eps >= 0.0) || d->eps > 1e300) QAM_FAIL(QAM_ERR_ARG, "decoder: eps must be finite and >= 0");
    if (d->target_waves < 0) QAM_FAIL(QAM_ERR_ARG, "decoder: target_waves < 0");
    if (d->waves_per_block != 0 && d->waves_per_block != 1 && d->waves_per_block != 2 && d->waves_per_block != 4 &&
        d->waves_per_block != 8)
        QAM_FAIL(QAM_ERR_ARG, "decoder: waves_per_block must be 0, 1, 2, 4 or 8");
    if (d->max_chunk_tiles < 0 || d->max_chunk_tiles > QAM_MAX_K / 64)
        QAM_FAIL(QAM_ERR_ARG, "decoder: max_chunk_tiles %d outside [0, %d]", d->max_chunk_tiles, QAM_MAX_K / 64);
    const int64_t tw = d->target_waves ? d->target_waves : 16;
    size_t partial = 0;
    auto need = [&](const qam_packed& w, int kind) {
        lo.max_blocks = std::max<int64_t>(lo.max_blocks, w.n_blocks);
        partial = std::max(partial, plan_of(w, tw, op_shape(*d, kind).max_chunk).partial_bytes);
    };
    for (int l = 0; l < d->n_layers; ++l) {
        const qam_decoder_layer& L = d->layers[l];
        if (!same_shape(L.qkv, Q + 2 * KV, H) || !same_shape(L.o, H, Q) || !same_shape(L.gate_up, 2 * F, H) ||
            !same_shape(L.down, H, F))
            QAM_FAIL(QAM_ERR_SHAPE, "decoder: layer %d has a matrix of the wrong shape", l);
        need(L.qkv, 0), need(L.o, 1), need(L.gate_up, 2), need(L.down, 3);
    }
    if (!same_shape(d->lm_head, V, H)) QAM_FAIL(QAM_ERR_SHAPE, "decoder: lm_head must be [vocab][hidden]");
    need(d->lm_head, 4);
    if (lo.max_blocks > QAM_MAX_BLOCKS) QAM_FAIL(QAM_ERR_SHAPE, "decoder: a matrix has more than %d blocks", QAM_MAX_BLOCKS);
    size_t off = 0;
    lo.ws = off;      off += up256(QAM_WS_COUNTER_BYTES + partial);
    lo.h = off;       off += up256((size_t)H * 4);
    lo.qkv = off;     off += up256((size_t)(Q + 2 * KV) * 4);
    lo.m = off;       off += up256((size_t)F * 4);
    lo.logits = off;  off += up256((size_t)V * 4);
    lo.maps = off;    off += 5 * up256((size_t)lo.max_blocks);
    lo.total = off;
    return QAM_OK;
}

int enqueue(qam_decoder* dec, int rung, int first, int count, hipStream_t s, const int* run_if = nullptr) {
    if (rung < 0 || rung > 4) QAM_FAIL(QAM_ERR_ARG, "decoder: rung %d outside 0..4", rung);
    const std::vector<Op> ops = chain(*dec);
    if (first < 0 || count < 0 || first > (int)ops.size() || count > (int)ops.size() - first)
        QAM_FAIL(QAM_ERR_ARG, "decoder: products [%d, %d) outside the chain of %zu", first, first + count, ops.size());
    Common c{};
    c.B = 1;
    c.x_bf16 = 0;
    c.status = status_word(dec->ws);
    for (int i = first; i < first + count; ++i) {
        const Op& op = ops[(size_t)i];
        const OpShape sh = op_shape(dec->d, op.kind);
        const Plan p = plan_of(*op.w, dec->target_waves, sh.max_chunk);
        c.KS = sh.ks;   // waves per (block, chunk)
        Item it = make_item(op.x, op.w, dec->maps[rung], op.y, p);
        it.fixed_level = rung;   // the map is uniform: the kernel takes the rung, not the map bytes
        it.rms = op.rms;
        it.out_mode = op.out_mode;
        it.eps = dec->d.eps;
        if (p.n_chunks > 1) {
            it.counters = reinterpret_cast<uint32_t*>(dec->ws);
            it.partials = reinterpret_cast<double*>(dec->ws + QAM_WS_COUNTER_BYTES);
        }
        it.counters = reinterpret_cast<uint32_t*>(dec->ws);
        it.run_if = run_if;
        launch_single(it, c, (int64_t)p.n_chunks * p.n_quads, s);
    }
    QAM_HIP_CHECK(hipGetLastError());
    return QAM_OK;
}

// h = x when *flag (the re-run of an escalated step starts from its input).
__global__ void __launch_bounds__(256) copy_if_kernel(const int* flag, const float* x, float* h, int64_t n) {
    if (*flag == 0) return;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        h[i] = x[i];
}

// out = (*flag != 0), one byte.
__global__ void flag_byte_kernel(const int* flag, uint8_t* out) { *out = *flag != 0 ? 1 : 0; }

// Capture the step at `rung` with every product predicated on *flag.
int capture_predicated(qam_decoder* dec, int rung, const int* flag, hipStream_t s) {
    QAM_HIP_CHECK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    const int rc = enqueue(dec, rung, 0, 4 * dec->d.n_layers + 1, s, flag);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &g);
    if (rc != QAM_OK) {
        if (g) (void)hipGraphDestroy(g);
        return rc;
    }
    if (e != hipSuccess) QAM_FAIL(QAM_ERR_HIP, "decoder: predicated capture: %s", hipGetErrorString(e));
    hipGraphExec_t x = nullptr;
    const hipError_t ei = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (ei != hipSuccess) {
        (void)hipGraphDestroy(g);
        QAM_FAIL(QAM_ERR_HIP, "decoder: predicated capture: instantiate: %s", hipGetErrorString(ei));
    }
    if (dec->pexec[rung]) (void)hipGraphExecDestroy(dec->pexec[rung]);
    if (dec->pgraph[rung]) (void)hipGraphDestroy(dec->pgraph[rung]);
    dec->pgraph[rung] = g;
    dec->pexec[rung] = x;
    dec->pflag[rung] = flag;
    return QAM_OK;
}

}  // namespace

extern "C" size_t qam_decoder_bytes(const qam_decoder_desc* d) {
    Layout lo;
    if (layout(d, lo) != QAM_OK) return 0;
    return lo.total;
}

extern "C" int qam_decoder_create(const qam_decoder_desc* d, void* dev_mem, size_t dev_bytes, qam_decoder** out,
                                  hipStream_t s) {
    clear_error();
    if (!out || !dev_mem) QAM_FAIL(QAM_ERR_NULL, "decoder_create: null pointer");
    *out = nullptr;
    Layout lo;
    if (int rc = layout(d, lo)) return rc;
    if (dev_bytes < lo.total) QAM_FAIL(QAM_ERR_WORKSPACE, "decoder_create: %zu < %zu bytes", dev_bytes, lo.total);
    if (!aligned(dev_mem, kAlign)) QAM_FAIL(QAM_ERR_ALIGN, "decoder_create: device memory must be 256-byte aligned");
    qam_decoder* dec = new (std::nothrow) qam_decoder();
    if (!dec) QAM_FAIL(QAM_ERR_ARG, "decoder_create: out of host memory");
    dec->d = *d;
    dec->layers.assign(d->layers, d->layers + d->n_layers);
    dec->d.layers = dec->layers.data();
    dec->target_waves = d->target_waves ? d->target_waves : 16;
    char* base = static_cast<char*>(dev_mem);
    dec->ws = base + lo.ws;
    dec->h = reinterpret_cast<float*>(base + lo.h);
    dec->qkv = reinterpret_cast<float*>(base + lo.qkv);
    dec->m = reinterpret_cast<float*>(base + lo.m);
    dec->logits = reinterpret_cast<float*>(base + lo.logits);
    hipError_t e = hipMemsetAsync(dec->ws, 0, QAM_WS_COUNTER_BYTES, s);
    for (int r = 0; r < 5 && e == hipSuccess; ++r) {
        dec->maps[r] = reinterpret_cast<uint8_t*>(base + lo.maps + r * up256((size_t)lo.max_blocks));
        e = hipMemsetAsync(dec->maps[r], r, (size_t)lo.max_blocks, s);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        delete dec;
        QAM_FAIL(QAM_ERR_HIP, "decoder_create: %s", hipGetErrorString(e));
    }
    *out = dec;
    return QAM_OK;
}

extern "C" float* qam_decoder_buffer(qam_decoder* dec, int which) {
    if (!dec) return nullptr;
    switch (which) {
        case QAM_DEC_H: return dec->h;
        case QAM_DEC_QKV: return dec->qkv;
        case QAM_DEC_M: return dec->m;
        case QAM_DEC_LOGITS: return dec->logits;
        default: return nullptr;
    }
}

extern "C" int qam_decoder_step(qam_decoder* dec, int rung, hipStream_t s) {
    clear_error();
    if (!dec) QAM_FAIL(QAM_ERR_NULL, "decoder_step: null decoder");
    if (int rc = enqueue(dec, rung, 0, 4 * dec->d.n_layers + 1, s)) return rc;
    char v[96];
    snprintf(v, sizeof(v), "decoder_step rung=%d launches=%d", rung, 4 * dec->d.n_layers + 1);
    set_variant(v);
    return QAM_OK;
}

extern "C" int qam_decoder_run(qam_decoder* dec, int rung, int first, int count, hipStream_t s) {
    clear_error();
    if (!dec) QAM_FAIL(QAM_ERR_NULL, "decoder_run: null decoder");
    return enqueue(dec, rung, first, count, s);
}

extern "C" int qam_decoder_capture(qam_decoder* dec, int rung, hipStream_t s) {
    clear_error();
    if (!dec) QAM_FAIL(QAM_ERR_NULL, "decoder_capture: null decoder");
    if (!s) QAM_FAIL(QAM_ERR_ARG, "decoder_capture: the null stream cannot be captured");
    if (rung < 0 || rung > 4) QAM_FAIL(QAM_ERR_ARG, "decoder_capture: rung %d outside 0..4", rung);
    QAM_HIP_CHECK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    const int rc = enqueue(dec, rung, 0, 4 * dec->d.n_layers + 1, s);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &g);
    if (rc != QAM_OK) {
        if (g) (void)hipGraphDestroy(g);
        return rc;
    }
    if (e != hipSuccess) QAM_FAIL(QAM_ERR_HIP, "decoder_capture: %s", hipGetErrorString(e));
    hipGraphExec_t x = nullptr;
    const hipError_t ei = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (ei != hipSuccess) {
        (void)hipGraphDestroy(g);
        QAM_FAIL(QAM_ERR_HIP, "decoder_capture: instantiate: %s", hipGetErrorString(ei));
    }
    if (dec->exec[rung]) (void)hipGraphExecDestroy(dec->exec[rung]);
    if (dec->graph[rung]) (void)hipGraphDestroy(dec->graph[rung]);
    dec->graph[rung] = g;
    dec->exec[rung] = x;
    return QAM_OK;
}

extern "C" int qam_decoder_replay(qam_decoder* dec, int rung, hipStream_t s) {
    clear_error();
    if (!dec) QAM_FAIL(QAM_ERR_NULL, "decoder_replay: null decoder");
    if (rung < 0 || rung > 4 || !dec->exec[rung]) QAM_FAIL(QAM_ERR_ARG, "decoder_replay: rung %d was not captured", rung);
    QAM_HIP_CHECK(hipGraphLaunch(dec->exec[rung], s));
    return QAM_OK;
}

extern "C" int qam_decoder_decode_gated(qam_decoder* dec, const float* inputs, int64_t T, int rung_low,
                                        int rung_high, double tau_entropy, double tau_margin, void* gate_workspace,
                                        size_t gate_workspace_bytes, qam_uncertainty* gate_out,
                                        qam_uncertainty* host_result, uint8_t* escalated_out, hipStream_t s) {
    clear_error();
    if (!dec || !gate_out || !host_result || ((!inputs || !escalated_out) && T > 0))
        QAM_FAIL(QAM_ERR_NULL, "decoder_decode_gated: null pointer");
    if (T < 0) QAM_FAIL(QAM_ERR_ARG, "decoder_decode_gated: T < 0");
    for (int r : {rung_low, rung_high})
        if (r < 0 || r > 4 || !dec->exec[r]) QAM_FAIL(QAM_ERR_ARG, "decoder_decode_gated: rung %d was not captured", r);
    if (!aligned(inputs, 4)) QAM_FAIL(QAM_ERR_ALIGN, "decoder_decode_gated: inputs not 4-byte aligned");
    const int64_t H = dec->d.hidden, V = dec->d.vocab;
    if (gate_workspace_bytes < qam_gate_workspace_bytes(V))
        QAM_FAIL(QAM_ERR_WORKSPACE, "decoder_decode_gated: gate workspace %zu < %zu bytes", gate_workspace_bytes,
                 qam_gate_workspace_bytes(V));
    for (int64_t t = 0; t < T; ++t) {
        const float* x = inputs + t * H;
        QAM_HIP_CHECK(hipMemcpyAsync(dec->h, x, H * sizeof(float), hipMemcpyDeviceToDevice, s));
        QAM_HIP_CHECK(hipGraphLaunch(dec->exec[rung_low], s));
        if (int rc = qam_gate(dec->logits, V, tau_entropy, tau_margin, gate_out, gate_workspace,
                              gate_workspace_bytes, s))
            return rc;
        QAM_HIP_CHECK(hipMemcpyAsync(host_result, gate_out, sizeof(qam_uncertainty), hipMemcpyDeviceToHost, s));
        QAM_HIP_CHECK(hipStreamSynchronize(s));
        escalated_out[t] = host_result->escalate ? 1 : 0;
        if (host_result->escalate) {
            QAM_HIP_CHECK(hipMemcpyAsync(dec->h, x, H * sizeof(float), hipMemcpyDeviceToDevice, s));
            QAM_HIP_CHECK(hipGraphLaunch(dec->exec[rung_high], s));
        }
    }
    QAM_HIP_CHECK(hipStreamSynchronize(s));
    set_variant("decoder_decode_gated");
    return QAM_OK;
}

extern "C" int qam_decoder_decode_gated_async(qam_decoder* dec, const float* inputs, int64_t T, int rung_low,
                                              int rung_high, double tau_entropy, double tau_margin,
                                              void* gate_workspace, size_t gate_workspace_bytes,
                                              qam_uncertainty* gate_out, uint8_t* escalated_dev, hipStream_t s) {
    clear_error();
    if (!dec || !gate_out || ((!inputs || !escalated_dev) && T > 0))
        QAM_FAIL(QAM_ERR_NULL, "decoder_decode_gated_async: null pointer");
    if (T < 0) QAM_FAIL(QAM_ERR_ARG, "decoder_decode_gated_async: T < 0");
    if (!s) QAM_FAIL(QAM_ERR_ARG, "decoder_decode_gated_async: needs a stream other than the null stream");
    if (rung_low < 0 || rung_low > 4 || !dec->exec[rung_low])
        QAM_FAIL(QAM_ERR_ARG, "decoder_decode_gated_async: rung %d was not captured", rung_low);
    if (rung_high < 0 || rung_high > 4) QAM_FAIL(QAM_ERR_ARG, "decoder_decode_gated_async: rung %d", rung_high);
    if (!aligned(inputs, 4) || !aligned(gate_out, 8))
        QAM_FAIL(QAM_ERR_ALIGN, "decoder_decode_gated_async: misaligned inputs or gate_out");
    const int64_t H = dec->d.hidden, V = dec->d.vocab;
    if (gate_workspace_bytes < qam_gate_workspace_bytes(V))
        QAM_FAIL(QAM_ERR_WORKSPACE, "decoder_decode_gated_async: gate workspace %zu < %zu bytes", gate_workspace_bytes,
                 qam_gate_workspace_bytes(V));
    const int* flag = &gate_out->escalate;
    if (!dec->pexec[rung_high] || dec->pflag[rung_high] != flag)
        if (int rc = capture_predicated(dec, rung_high, flag, s)) return rc;
    const unsigned cgrid = (unsigned)std::min<int64_t>(64, (H + 255) / 256);
    for (int64_t t = 0; t < T; ++t) {
        const float* x = inputs + t * H;
        QAM_HIP_CHECK(hipMemcpyAsync(dec->h, x, H * sizeof(float), hipMemcpyDeviceToDevice, s));
        QAM_HIP_CHECK(hipGraphLaunch(dec->exec[rung_low], s));
        if (int rc = qam_gate(dec->logits, V, tau_entropy, tau_margin, gate_out, gate_workspace,
                              gate_workspace_bytes, s))
            return rc;
        hipLaunchKernelGGL(flag_byte_kernel, dim3(1), dim3(1), 0, s, flag, escalated_dev + t);
        hipLaunchKernelGGL(copy_if_kernel, dim3(cgrid), dim3(256), 0, s, flag, x, dec->h, H);
        QAM_HIP_CHECK(hipGetLastError());
        QAM_HIP_CHECK(hipGraphLaunch(dec->pexec[rung_high], s));
    }
    set_variant("decoder_decode_gated_async");
    return QAM_OK;
}

extern "C" void qam_decoder_destroy(qam_decoder* dec) {
    if (!dec) return;
    for (int r = 0; r < 5; ++r) {
        if (dec->exec[r]) (void)hipGraphExecDestroy(dec->exec[r]);
        if (dec->graph[r]) (void)hipGraphDestroy(dec->graph[r]);
        if (dec->pexec[r]) (void)hipGraphExecDestroy(dec->pexec[r]);
        if (dec->pgraph[r]) (void)hipGraphDestroy(dec->pgraph[r]);
    }
    delete dec;
}

extern "C" int qam_escalation_schedule(const double* scores, int64_t T, double rate, uint8_t* escalate_out,
                                       int64_t* n_out) {
    clear_error();
    if (!scores || !escalate_out) QAM_FAIL(QAM_ERR_NULL, "escalation_schedule: null pointer");
    if (T < 0) QAM_FAIL(QAM_ERR_ARG, "escalation_schedule: T < 0");
    if (!(rate >= 0.0 && rate <= 1.0)) QAM_FAIL(QAM_ERR_ARG, "escalation_schedule: rate outside [0, 1]");
    for (int64_t t = 0; t < T; ++t)
        if (!std::isfinite(scores[t])) QAM_FAIL(QAM_ERR_ARG, "escalation_schedule: score %lld not finite", (long long)t);
    const int64_t n = (int64_t)std::floor(rate * (double)T + 0.5);
    std::vector<int64_t> order((size_t)T);
    std::iota(order.begin(), order.end(), (int64_t)0);
    // largest score first; equal scores keep step order (the earlier step wins)
    std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return scores[a] > scores[b]; });
    std::fill(escalate_out, escalate_out + T, (uint8_t)0);
    for (int64_t i = 0; i < n; ++i) escalate_out[order[(size_t)i]] = 1;
    if (n_out) *n_out = n;
    return QAM_OK;
}
