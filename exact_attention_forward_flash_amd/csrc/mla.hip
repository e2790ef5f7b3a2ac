// Instantiations for the packed varlen MLA prefill: score width 128 (nope) + 64 (rope), value
// width 128, persistent work groups over a device-built tile schedule. HPW query heads of a
// KV head share each K/V tile (HPW 4 / 2 / 1: 64 / 128 / 256 query rows per work item).
#include "wf_internal.hpp"

namespace wf {
#define E(T, DT, HPW, CAUSAL) WF_ATTN_ENTRY(T, DT, 192, 128, 128, 8, HPW, MASK_NONE, CAUSAL, MODE_VARLEN)
#define ALL(T, DT) E(T, DT, 1, false), E(T, DT, 1, true), E(T, DT, 2, false), E(T, DT, 2, true), \
                   E(T, DT, 4, false), E(T, DT, 4, true)
static const AttnEntry kTable[] = {ALL(__bf16, DT_BF16), ALL(_Float16, DT_F16)};
#undef ALL
#undef E
const AttnEntry* attn_table_mla(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
