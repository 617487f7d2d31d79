// csa_indexer_scores: lightning-indexer relevance of every compressed entry,
// written as fp32 scores (-inf for entries the query cannot see yet).
//
// The kernel (indexer_core.hpp) runs the MXFP4 contraction on the CDNA4
// block-scaled matrix cores.  Products of E2M1 values times power-of-two
// scales are exact and fp32 sums of them stay exact while every partial sum
// is an integer multiple of the smallest product below 2^24 of it, so for
// such inputs the scores equal the exact scores bit for bit.  Decode (one
// query) is a pure stream of the keys: 68 B per entry for d_I = 128.
#include "indexer_core.hpp"

extern "C" csa_status_t csa_indexer_scores(const uint8_t* q_codes, const uint8_t* q_e8m0, const float* w,
                                           const uint8_t* k_codes, const uint8_t* k_e8m0, const int32_t* q_pos0,
                                           int32_t B, int32_t T_q, int32_t H_I, int32_t d_I, int32_t cap, int32_t m,
                                           float* scores, void* stream) {
  if (!scores) return CSA_EINVAL;
  const csa_status_t s = csa_ix::check_indexer_args(q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, H_I, d_I,
                                                    cap, m);
  if (s != CSA_OK) return s;
  if (B == 0 || T_q == 0 || cap == 0) return CSA_OK;
  const hipError_t err = csa_ix::launch_indexer<csa_ix::kScoresF32>(
      H_I, q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, B, T_q, d_I, cap, m, scores, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? CSA_OK : CSA_EHIP;
}
