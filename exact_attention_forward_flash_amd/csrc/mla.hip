// Instantiations for the packed varlen MLA prefill: score width 128 (nope) + 64 (rope),
// value width 128, persistent work groups over a device-built tile schedule.
#include "wf_internal.hpp"

namespace wf {
#define E(T, DT, CAUSAL) WF_ATTN_ENTRY(T, DT, 192, 128, 128, 8, 1, MASK_NONE, CAUSAL, MODE_VARLEN)
static const AttnEntry kTable[] = {
    E(__bf16, DT_BF16, false), E(__bf16, DT_BF16, true),
    E(_Float16, DT_F16, false), E(_Float16, DT_F16, true),
};
#undef E
const AttnEntry* attn_table_mla(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
