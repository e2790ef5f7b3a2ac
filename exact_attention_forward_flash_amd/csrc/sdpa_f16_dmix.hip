// Instantiations of the 16-bit attention kernel for the SDPA entry point with value width
// different from the query/key width: f16, (Dqk, Dv) = (64, 96) and (128, 64).
#include "wf_internal.hpp"

namespace wf {
#define E(DQK, DV, HPW, MASK, CAUSAL) WF_ATTN_ENTRY(_Float16, DT_F16, DQK, DQK, DV, 8, HPW, MASK, CAUSAL, MODE_DENSE)
#define DIMS(DQK, DV)                                                                              \
  E(DQK, DV, 1, MASK_NONE, false), E(DQK, DV, 2, MASK_NONE, false), E(DQK, DV, 4, MASK_NONE, false), \
  E(DQK, DV, 1, MASK_NONE, true),  E(DQK, DV, 2, MASK_NONE, true),  E(DQK, DV, 4, MASK_NONE, true),  \
  E(DQK, DV, 1, MASK_BOOL, false), E(DQK, DV, 1, MASK_HALF, false), E(DQK, DV, 1, MASK_F32, false)
static const AttnEntry kTable[] = {DIMS(64, 96), DIMS(128, 64)};
#undef DIMS
#undef E
const AttnEntry* attn_table_sdpa_f16_dmix(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
