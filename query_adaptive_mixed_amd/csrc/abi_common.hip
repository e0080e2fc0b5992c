// Thread-local diagnostics and small host-side helpers of the C ABI.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "qam_common.h"

namespace qam {

static thread_local std::string g_error;
static thread_local std::string g_variant;

void set_error(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
}

void clear_error() { g_error.clear(); }

void set_variant(const std::string& v) { g_variant = v; }

}  // namespace qam

extern "C" {

const char* qam_last_error(void) { return qam::g_error.c_str(); }

const char* qam_last_variant(void) { return qam::g_variant.c_str(); }

const char* qam_version(void) { return "qam 0.1 gfx950"; }

size_t qam_packed_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return 0;
    return (size_t)N * (size_t)K + 4 * (size_t)N;
}

int qam_describe_packed(void* packed_buf, int64_t N, int64_t K, qam_packed* desc_out) {
    qam::clear_error();
    if (!packed_buf || !desc_out) QAM_FAIL(QAM_ERR_NULL, "describe_packed: null pointer");
    if (N <= 0 || K <= 0 || N % QAM_ROWS_PER_BLOCK || K % 64 || K > QAM_MAX_K)
        QAM_FAIL(QAM_ERR_SHAPE, "describe_packed: N=%lld K=%lld must be positive multiples of 64, K <= %d",
                 (long long)N, (long long)K, QAM_MAX_K);
    if (!qam::aligned(packed_buf, 256)) QAM_FAIL(QAM_ERR_ALIGN, "describe_packed: buffer not 256-byte aligned");
    desc_out->N = N;
    desc_out->K = K;
    desc_out->n_blocks = N / QAM_ROWS_PER_BLOCK;
    desc_out->planes = packed_buf;
    desc_out->scales = reinterpret_cast<float*>(static_cast<char*>(packed_buf) + N * K);
    return QAM_OK;
}

int qam_map_weight_bytes(const uint8_t* level, int64_t n_blocks, int64_t K, const uint8_t* ladder_bits,
                         int n_rungs, double* mean_bits, int64_t* weight_bytes) {
    qam::clear_error();
    if (n_blocks < 0 || K <= 0) QAM_FAIL(QAM_ERR_SHAPE, "map_weight_bytes: bad n_blocks/K");
    if ((n_blocks > 0 && !level) || !ladder_bits) QAM_FAIL(QAM_ERR_NULL, "map_weight_bytes: null pointer");
    if (n_rungs < 1 || n_rungs > QAM_MAX_RUNGS) QAM_FAIL(QAM_ERR_LADDER, "map_weight_bytes: bad rung count");
    // rule 7: bits = sum_b w_b bits(b) / sum_b w_b, with w_b = 64 K for every block
    int64_t bit_sum = 0;
    for (int64_t b = 0; b < n_blocks; ++b) {
        if (level[b] >= n_rungs) QAM_FAIL(QAM_ERR_ARG, "map_weight_bytes: rung %d out of range", (int)level[b]);
        bit_sum += (int64_t)ladder_bits[level[b]];
    }
    const int64_t wb = (int64_t)QAM_ROWS_PER_BLOCK * K;
    if (mean_bits) *mean_bits = n_blocks ? (double)(bit_sum * wb) / (double)(n_blocks * wb) : 0.0;
    if (weight_bytes) *weight_bytes = bit_sum * wb / 8;
    return QAM_OK;
}

}  // extern "C"
