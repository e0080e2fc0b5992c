// qam_qmatvec_noalloc: qam_qmatvec with its workspace in a file-scope device
// array, for callers that cannot allocate device memory.
//
// The array is a static object of this library's code object: the loader
// gives every GPU its own zero-filled copy when the code object is loaded
// there, and it lives until the process ends.  In host code the name
// `scratch` is only a host-side shadow of the device symbol, so the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
#include <mutex>

#include "qam_common.h"
#include "qmatvec_internal.h"

namespace qam {

__device__ __align__(256) unsigned char scratch[QAM_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_setup_mutex;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch`, per device

// Zero n 32-bit words with vector stores (a kernel, so the clear can sit in
// a captured graph, where a memset node is not wanted).
__global__ void __launch_bounds__(256) clear_words(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Device address of the current device's copy of `scratch`.  The first call
// on a device looks the address up and enqueues a clear of the counter region
// on `s`, ahead of the work that call enqueues.
int scratch_of_current_device(void** out, hipStream_t s) {
    int dev = -1;
    QAM_HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) QAM_FAIL(QAM_ERR_ARG, "qmatvec_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_setup_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        QAM_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p || !aligned(p, 256)) QAM_FAIL(QAM_ERR_HIP, "qmatvec_noalloc: bad scratch address on device %d", dev);
        const int64_t words = QAM_WS_COUNTER_BYTES / 4;
        hipLaunchKernelGGL(clear_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                           static_cast<uint32_t*>(p), words);
        QAM_HIP_CHECK(hipGetLastError());
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QAM_OK;
}

}  // namespace
}  // namespace qam

extern "C" int qam_qmatvec_noalloc(const void* x, int x_dtype, int64_t B, const qam_packed* packed,
                                   const uint8_t* level_map, int per_request_maps, float* y, hipStream_t s) {
    qam::clear_error();
    if (per_request_maps != 0 && per_request_maps != 1)
        QAM_FAIL(QAM_ERR_ARG, "qmatvec_noalloc: per_request_maps must be 0 or 1");
    if (int rc = qam::check_item(x, x_dtype, B, packed, level_map, y, "qmatvec_noalloc", QAM_OUT_STORE)) return rc;
    const size_t need = qam_qmatvec_workspace_bytes(packed->N, packed->K, B);
    if (need == 0 || need > (size_t)QAM_SCRATCH_BYTES)
        QAM_FAIL(QAM_ERR_WORKSPACE, "qmatvec_noalloc: N=%lld K=%lld B=%lld needs %zu bytes of scratch, limit %d",
                 (long long)packed->N, (long long)packed->K, (long long)B, need, QAM_SCRATCH_BYTES);
    void* ws = nullptr;
    if (int rc = qam::scratch_of_current_device(&ws, s)) return rc;
    return qam_qmatvec(x, x_dtype, B, packed, level_map, per_request_maps, y, ws, (size_t)QAM_SCRATCH_BYTES, s);
}
