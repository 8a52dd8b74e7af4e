// Matrix-core attention path: not enabled yet; every shape takes the vector path.
#include "attn_mfma.hpp"

namespace msa {

bool attn_mfma_applicable(const AttnArgs&) { return false; }
size_t attn_mfma_workspace(msa_dtype, int64_t, int, int, int, int, int64_t, int) { return 0; }
hipError_t launch_attn_mfma(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace msa
