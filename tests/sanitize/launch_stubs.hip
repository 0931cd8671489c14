// Launchers for the host-only sanitizer build of the C ABI: the driver's calls
// are all rejected on the host or touch no kernel, so reaching a launcher is a
// failure and aborts.
#include <cstdio>
#include <cstdlib>

#include "rssm_launch.h"

namespace rssm {
static hipError_t never(const char* name) {
    std::fprintf(stderr, "launcher %s reached\n", name);
    std::abort();
}
hipError_t launch_decode(const StepArgs&, int, int, int, bool, int, int, size_t, hipStream_t) { return never("decode"); }
hipError_t launch_decode_split(const StepArgs&, int, int, int, int, int, size_t, hipStream_t) {
    return never("decode_split");
}
hipError_t launch_fold(const StepArgs&, int, int, int, bool, int, int, size_t, hipStream_t) { return never("fold"); }
hipError_t launch_commit(const StepArgs&, int, int, int, bool, int, int, size_t, hipStream_t) { return never("commit"); }
hipError_t launch_commit_static(const StepArgs&, int, int, int, bool, int, int, size_t, hipStream_t) {
    return never("commit_static");
}
hipError_t launch_verify(const StepArgs&, int, int, int, int, bool, int, size_t, hipStream_t) { return never("verify"); }
hipError_t launch_prefill(const StepArgs&, int, int, int, int, int, size_t, hipStream_t) { return never("prefill"); }
hipError_t launch_refresh(const StepArgs&, int, int, int, int, hipStream_t) { return never("refresh"); }
hipError_t launch_reset(const StepArgs&, int, int, int, int, hipStream_t) { return never("reset"); }
hipError_t launch_conv_decode(const ConvArgs&, int, int, int, int, size_t, hipStream_t) { return never("conv_decode"); }
hipError_t launch_conv_verify(const ConvArgs&, int, int, int, int, size_t, hipStream_t) { return never("conv_verify"); }
hipError_t launch_conv_commit(const ConvArgs&, hipStream_t) { return never("conv_commit"); }
hipError_t launch_probe_copy(void*, const void*, size_t, hipStream_t) { return never("probe_copy"); }
hipError_t launch_probe_read(const void*, size_t, float*, hipStream_t) { return never("probe_read"); }
hipError_t launch_probe_read_chunked(const void*, size_t, void*, size_t, float*, hipStream_t) {
    return never("probe_read_chunked");
}
}  // namespace rssm
