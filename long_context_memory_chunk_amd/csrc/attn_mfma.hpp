// Matrix-core attention path (bf16 prefill): declarations shared with attn.hip.
#pragma once

#include "launch.hpp"

namespace msa {

bool attn_mfma_applicable(const AttnArgs& a);
size_t attn_mfma_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D,
                           int64_t max_rows, int L);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st);

}  // namespace msa
