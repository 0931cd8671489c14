// rssm_launch.h -- launcher entry points implemented next to the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include "rssm_args.h"

namespace rssm {
hipError_t launch_decode(const StepArgs& A, int N, int in_dtype, int rc, bool multi, int ck, int grid, size_t lds,
                         hipStream_t s);
// Decode of two-head tiles whose non-flush steps read an fp8 or MXFP4 copy, 128 threads per head
// (key dims 64 and 128, windows up to 16, at most 128 rows per head).
hipError_t launch_decode_split(const StepArgs& A, int N, int in_dtype, int rc, int ck, int grid, size_t lds,
                               hipStream_t s);
hipError_t launch_fold(const StepArgs& A, int N, int in_dtype, int rc, bool multi, int ck, int grid, size_t lds,
                       hipStream_t s);
hipError_t launch_commit(const StepArgs& A, int N, int in_dtype, int rc, bool multi, int ck, int fold_grid,
                         size_t lds, hipStream_t s);
// The same with the fold list in the library's own device array (A.work unused).
hipError_t launch_commit_static(const StepArgs& A, int N, int in_dtype, int rc, bool multi, int ck, int fold_grid,
                                size_t lds, hipStream_t s);
// rd: read format (RC_NONE / RC_F16 for the checkpoint itself, else the copy's)
hipError_t launch_verify(const StepArgs& A, int N, int in_dtype, int rd, int tt, bool multi, int grid, size_t lds, hipStream_t s);
// Prefill of T prompt tokens (A.T), then the key appends; np rows per thread per head.
hipError_t launch_prefill(const StepArgs& A, int N, int in_dtype, int ck, int np, int grid, size_t lds, hipStream_t s);
hipError_t launch_refresh(const StepArgs& A, int N, int rc, int ck, int grid, hipStream_t s);
hipError_t launch_reset(const StepArgs& A, int N, int rc, int ck, int grid, hipStream_t s);

hipError_t launch_conv_decode(const ConvArgs& A, int N, int in_dtype, int sf, int grid, size_t lds, hipStream_t s);
hipError_t launch_conv_verify(const ConvArgs& A, int N, int in_dtype, int tt, int grid, size_t lds, hipStream_t s);
hipError_t launch_conv_commit(const ConvArgs& A, hipStream_t s);

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t s);
hipError_t launch_probe_read_chunked(const void* src, size_t bytes, void* dst, size_t write_bytes, float* sink,
                                     hipStream_t s);
}  // namespace rssm
