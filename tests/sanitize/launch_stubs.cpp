// Test support (not part of the library): stand-ins for the kernel
// launchers, so that the C ABI's host code (argument validation, dispatch,
// status and error reporting in api.cpp) can be built with the host address
// and undefined-behaviour sanitizers and run on a machine without a GPU.
// Every launch reports hipErrorInvalidValue; the workspace sizes follow the
// library's rules for the preparation and weight quantization (NVFP4 only)
// and report no K-split workspace for products.
#include "../../sparsity_prep_amd/csrc/kernels.h"

namespace sharq {

hipError_t launch_prepare(const PrepArgs &, void *, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_prepare_noalloc(const PrepArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_prepare_swiglu(const PrepArgs &, void *, hipStream_t) { return hipErrorInvalidValue; }
size_t prepare_workspace_bytes(int64_t T, int fmt) { return fmt == kFmtNv ? (size_t)(T > 0 ? T : 1) * 16 : 0; }
hipError_t launch_quantize_weight(const QuantWArgs &, void *, hipStream_t) { return hipErrorInvalidValue; }
size_t quantize_weight_workspace_bytes(int64_t E, int64_t nout, int fmt) {
    return fmt == kFmtNv ? (size_t)(E * nout > 0 ? E * nout : 1) * sizeof(float) : 0;
}
hipError_t launch_linear(const LinearArgs &, void *, size_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_linear_swiglu(const LinearArgs &, hipStream_t) { return hipErrorInvalidValue; }
size_t linear_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int) { return 0; }

}  // namespace sharq
