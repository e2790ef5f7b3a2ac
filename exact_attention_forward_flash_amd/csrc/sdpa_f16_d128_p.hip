// Instantiations of the persistent dense attention kernel: f16, head dim 128.
#include "wf_internal.hpp"

namespace wf {
#define E(HPW, CAUSAL) WF_ATTN_P_ENTRY(_Float16, DT_F16, 128, HPW, CAUSAL)
static const AttnEntry kTable[] = {E(1, false), E(2, false), E(4, false), E(4, true)};
#undef E
const AttnEntry* attn_table_p_f16_d128(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
