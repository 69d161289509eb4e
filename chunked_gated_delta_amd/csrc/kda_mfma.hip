// Matrix-core path (bf16 MFMA on gfx950).  Not available yet: the host falls
// back to nothing -- kda_chunk_fwd picks the vector path when this says no.
#include "kda_internal.h"

namespace kda {

bool mfma_supported(const Params&) { return false; }

size_t mfma_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_mfma(const Params&, hipStream_t, hipEvent_t, hipEvent_t) { return hipErrorNotSupported; }

}  // namespace kda
