// Instantiations of the 16-bit attention kernel for the SDPA entry point: f16, head dim 64.
#include "wf_internal.hpp"

namespace wf {
#define E(NW, HPW, MASK, CAUSAL) WF_ATTN_ENTRY(_Float16, DT_F16, 64, 64, 64, NW, HPW, MASK, CAUSAL, MODE_DENSE)
static const AttnEntry kTable[] = {
    E(8, 1, MASK_NONE, false), E(8, 2, MASK_NONE, false), E(8, 4, MASK_NONE, false),
    E(8, 1, MASK_NONE, true),  E(8, 2, MASK_NONE, true),  E(8, 4, MASK_NONE, true),
    E(8, 1, MASK_BOOL, false), E(8, 1, MASK_HALF, false), E(8, 1, MASK_F32, false),
    E(4, 1, MASK_NONE, false), E(4, 2, MASK_NONE, false), E(4, 4, MASK_NONE, false),
    E(4, 1, MASK_NONE, true),  E(4, 2, MASK_NONE, true),  E(4, 4, MASK_NONE, true),
    // masked calls without the lse: Q prescaled, scores relative to the reference max
    WF_ATTN_ENTRY(_Float16, DT_F16, 64, 64, 64, 8, 1, MASK_BOOL, false, MODE_DENSE_PM),
    WF_ATTN_ENTRY(_Float16, DT_F16, 64, 64, 64, 8, 1, MASK_HALF, false, MODE_DENSE_PM),
};
#undef E
const AttnEntry* attn_table_sdpa_f16_d64(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
