// Instantiations for the packed varlen MLA prefill with value width 64: score width 64 (nope)
// + 64 (rope), HPW query heads of a KV head sharing each K/V tile.
#include "wf_internal.hpp"

namespace wf {
#define E(T, DT, HPW, CAUSAL) WF_ATTN_ENTRY(T, DT, 128, 64, 64, 8, HPW, MASK_NONE, CAUSAL, MODE_VARLEN)
#define ALL(T, DT) E(T, DT, 1, false), E(T, DT, 1, true), E(T, DT, 2, false), E(T, DT, 2, true), \
                   E(T, DT, 4, false), E(T, DT, 4, true)
static const AttnEntry kTable[] = {ALL(__bf16, DT_BF16), ALL(_Float16, DT_F16)};
#undef ALL
#undef E
const AttnEntry* attn_table_mla_v64(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
