// Many-query (prefill) path: placeholder until the MFMA scoring kernels land.
#include "topo_internal.h"

namespace topo {

size_t prefill_workspace_bytes(int32_t, int32_t, int64_t, int64_t, int32_t, int32_t, int32_t) { return 256; }

hipError_t launch_prefill(const PrefillLaunch&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace topo
