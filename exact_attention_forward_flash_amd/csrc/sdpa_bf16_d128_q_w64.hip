// Instantiations of the persistent 64-query-wave attention kernel: bf16, head dim 128.
// Built with the compiler-generated MFMAs forced to the VGPR form (the S^T products; the O^T
// products are written out with AGPR accumulators).
#include "wf_internal.hpp"

namespace wf {
#define E(HPW, CAUSAL) WF_ATTN_Q_ENTRY(__bf16, DT_BF16, 128, HPW, CAUSAL)
static const AttnEntry kTable[] = {E(1, false), E(2, false), E(4, false), E(4, true)};
#undef E
const AttnEntry* attn_table_q_bf16_d128(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
