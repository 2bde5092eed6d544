// bf16 matrix-core engine (placeholder until the MFMA kernels land).
#include "flce_internal.h"

namespace flce {

hipError_t mfma_logits(const Plan&, const Work&, const ChunkArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t mfma_dh(const Plan&, const Work&, const ChunkArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t mfma_dw(const Plan&, const Work&, const ChunkArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace flce
