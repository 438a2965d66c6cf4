// kda_chunk_mfma.hip -- MFMA chunked prefill (bf16 inputs, dk = dv = 128,
// chunk = 64).  Placeholder until the kernel lands: reports no support, so
// the ABI layer uses the generic path.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

bool chunk_mfma_supports(const ChunkArgs&) { return false; }

hipError_t launch_chunk_mfma(const ChunkArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kda
