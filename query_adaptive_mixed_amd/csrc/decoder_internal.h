// The decoder's host object, shared by the decode driver and the batched
// verify step.
#pragma once

#include <vector>

#include "qmatvec_internal.h"

struct qam_decoder {
    qam_decoder_desc d{};
    std::vector<qam_decoder_layer> layers;
    float *h = nullptr, *qkv = nullptr, *m = nullptr, *logits = nullptr;
    uint8_t* maps[5] = {};
    char* ws = nullptr;            // counters, then fp64 partials
    int64_t target_waves = 16;
    hipGraph_t graph[5] = {};
    hipGraphExec_t exec[5] = {};
    // steps whose products run only when a device flag is nonzero, by rung
    hipGraph_t pgraph[5] = {};
    hipGraphExec_t pexec[5] = {};
    const int* pflag[5] = {};      // the flag each predicated graph reads
};
