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
// The same over the memory rows only, its P partitions written as partials
// p_base .. p_base + P - 1 of P_total per row.
hipError_t launch_decode_mfma_mem(const AttnArgs& a, float* part_o, float2* part_ml, int P, int nc, int p_base,
                                  int P_total, hipStream_t st);
// One launch: the device gather's copy (n_copy workgroups; the one-query copy
// if `one`) beside the attention over the local keys only, whose P partitions
// are written as partials 0 .. P - 1 of P_total per row.  a.KVmem and
// a.mem_off are not read.  With attn_rows (4 or 8: one-query copy of a
// one-token query, hkv <= 8), copy workgroup w takes attn_rows rows and writes
// their partial as index P + w, so n_copy = P_total - P (workgroups past the
// gathered rows write none; the combine is told to read only those that do).
hipError_t launch_gather_local_attn(const GatherCopyArgs& gc, bool one, int attn_rows, int n_copy,
                                    const AttnArgs& a, float* part_o, float2* part_ml, int P, int nc, int P_total,
                                    hipStream_t st);

}  // namespace msa
