// Instantiations of the 64-query-wave attention kernel for the SDPA entry point: bf16,
// head dim 128. Built with the compiler-generated MFMAs forced to the VGPR form.
#include "wf_internal.hpp"

namespace wf {
#define E(HPW, MASK, CAUSAL) WF_ATTN_W_ENTRY(__bf16, DT_BF16, 128, 128, 128, HPW, MASK, CAUSAL, MODE_DENSE)
static const AttnEntry kTable[] = {
    E(1, MASK_NONE, false), E(2, MASK_NONE, false), E(4, MASK_NONE, false),
    E(1, MASK_NONE, true),  E(2, MASK_NONE, true),  E(4, MASK_NONE, true),
    E(1, MASK_BOOL, false), E(1, MASK_HALF, false), E(1, MASK_F32, false),
};
#undef E
const AttnEntry* attn_table_w_bf16_d128(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
