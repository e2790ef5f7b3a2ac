// Instantiations of the persistent dense attention kernel: f16, head dim 64.
#include "wf_internal.hpp"

namespace wf {
#define E(HPW, CAUSAL, SUM16) WF_ATTN_P_ENTRY(_Float16, DT_F16, 64, HPW, CAUSAL, SUM16)
// SUM16: row sums over the 16-bit weights (calls without the lse), else fp32 sums.
static const AttnEntry kTable[] = {
    E(1, false, true),  E(2, false, true),  E(4, false, true),  E(4, true, true),
    E(1, false, false), E(2, false, false), E(4, false, false), E(4, true, false),
};
#undef E
const AttnEntry* attn_table_p_f16_d64(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
