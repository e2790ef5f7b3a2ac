// Instantiations for split-KV attention (block KV cache attend): each work group covers a
// contiguous range of key tiles and writes an fp32 partial result plus its log-sum-exp.
#include "wf_internal.hpp"

namespace wf {
#define E(T, DT, D, NW) WF_ATTN_ENTRY(T, DT, D, D, D, NW, 1, MASK_NONE, false, MODE_SPLIT)
static const AttnEntry kTable[] = {
    E(__bf16, DT_BF16, 64, 4), E(__bf16, DT_BF16, 128, 4),
    E(_Float16, DT_F16, 64, 4), E(_Float16, DT_F16, 128, 4),
};
#undef E
const AttnEntry* attn_table_split(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
}  // namespace wf
