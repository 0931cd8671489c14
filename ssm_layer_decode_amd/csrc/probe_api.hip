// probe_api.hip -- the C ABI of the measurement library librssm_probes.so
// (include/rssm_probes.h): argument checks, then the probe kernels of
// probe_kernels.hip.  Not part of the decode method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rssm_probes.h"
#include "rssm_launch.h"

namespace {
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
rssm_status hip_status(hipError_t e) { return e == hipSuccess ? RSSM_OK : RSSM_EHIP; }
}  // namespace

extern "C" {

rssm_status rssm_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!dst || !src || !aligned16(dst) || !aligned16(src) || bytes % 16 != 0) return RSSM_EINVAL;
    return hip_status(rssm::launch_probe_copy(dst, src, bytes, (hipStream_t)stream));
}

rssm_status rssm_probe_read(const void* src, size_t bytes, float* sink, void* stream) {
    if (!src || !sink || !aligned16(src) || bytes % 16 != 0) return RSSM_EINVAL;
    return hip_status(rssm::launch_probe_read(src, bytes, sink, (hipStream_t)stream));
}

rssm_status rssm_probe_read_chunked(const void* src, size_t bytes, void* dst, size_t write_bytes, float* sink,
                                    void* stream) {
    if (!src || !sink || !aligned16(src) || bytes == 0 || bytes % 32768 != 0) return RSSM_EINVAL;
    if (write_bytes % 16 != 0 || write_bytes > 4096) return RSSM_EINVAL;
    if (write_bytes > 0 && (!dst || !aligned16(dst))) return RSSM_EINVAL;
    if (bytes / 32768 > 0x7fffffffull) return RSSM_EINVAL;
    return hip_status(rssm::launch_probe_read_chunked(src, bytes, dst, write_bytes, sink, (hipStream_t)stream));
}

}  // extern "C"
