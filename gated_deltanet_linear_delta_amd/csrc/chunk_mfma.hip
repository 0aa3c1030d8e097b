// Fused matrix-core chunkwise kernel (bf16 inputs) -- placeholder until the kernel lands.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {

bool chunk_mfma_supported(const ChunkArgs&) { return false; }
hipError_t launch_chunk_mfma(const ChunkArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace gdn
