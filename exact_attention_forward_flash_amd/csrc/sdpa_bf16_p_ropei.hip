// Instantiations of the persistent dense attention kernel that turns Q by a rotary table as
// it is read (used by the rotary entry point when the call takes the persistent kernel):
// bf16, head dims 64 and 128.
#include "wf_internal.hpp"
namespace wf {
#define E(D, HPW, CAUSAL, SUM16, ROPE) WF_ATTN_PR_ENTRY(__bf16, DT_BF16, D, HPW, CAUSAL, SUM16, ROPE)
// ROPE 2: interleaved over the first rot dims.
static const AttnEntry kTable[] = {
    E(128, 1, false, true, 2),  E(128, 2, false, true, 2),  E(128, 4, false, true, 2),  E(128, 4, true, true, 2),
    E(128, 1, false, false, 2), E(128, 2, false, false, 2), E(128, 4, false, false, 2), E(128, 4, true, false, 2),
    E(64, 1, false, true, 2),  E(64, 2, false, true, 2),  E(64, 4, false, true, 2),  E(64, 4, true, true, 2),
    E(64, 1, false, false, 2), E(64, 2, false, false, 2), E(64, 4, false, false, 2), E(64, 4, true, false, 2),
};
#undef E
const AttnEntry* attn_table_p_ropei_bf16(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
