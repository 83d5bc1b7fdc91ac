// MFMA split-K decode (placeholder until the gfx950 kernel lands).
#include "kernels.hpp"

namespace mla {

bool mfma_decode_supported(const mla_dims &, int) { return false; }
int mfma_row_block() { return 64; }
hipError_t launch_absorb_mfma_layout(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_splitk_mfma(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mla
