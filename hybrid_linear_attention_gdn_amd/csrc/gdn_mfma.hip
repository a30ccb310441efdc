// MFMA kernel family (bf16 inputs, d = 112): placeholder until written.
#include "gdn_internal.h"

namespace gdn {

size_t mfma_chunk_bytes_M() { return 0; }
size_t mfma_chunk_bytes_P() { return 0; }
size_t mfma_chunk_bytes_cs() { return 0; }

hipError_t launch_mfma(const Plan &, const Args &) { return hipErrorNotSupported; }

}  // namespace gdn
