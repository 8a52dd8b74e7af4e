// Matrix-core attention paths (bf16 prefill and decode): declarations shared
// with attn.hip.
#pragma once

#include "launch.hpp"

namespace msa {

bool attn_mfma_applicable(const AttnArgs& a);
size_t attn_mfma_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D,
                           int64_t max_rows, int L);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st);

// attn_decode_mfma.hip: keys per chunk, and the launch over P key partitions
// of nc chunks each, writing the partial (m, l, o) of every row and partition.
constexpr int kDecodeChunk = 128;
hipError_t launch_decode_mfma(const AttnArgs& a, float* part_o, float2* part_ml, int P, int nc, hipStream_t st);

}  // namespace msa
