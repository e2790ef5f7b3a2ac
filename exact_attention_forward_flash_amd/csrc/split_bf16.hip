// Instantiations for split-KV attention (bf16): each work group covers a contiguous range of
// key tiles of one (batch, KV head, head group, query tile) item and writes an fp32 partial
// result plus its log-sum-exp, which split_combine_kernel merges. Used by the block KV cache
// attend (one query head per group) and by decode (HPW query heads of a KV group share each
// K/V tile; causal = the queries are the last Lq of the keys).
#include "wf_internal.hpp"

namespace wf {
#define E(D, HPW, CAUSAL) WF_ATTN_ENTRY(__bf16, DT_BF16, D, D, D, 4, HPW, MASK_NONE, CAUSAL, MODE_SPLIT)
static const AttnEntry kTable[] = {
    E(64, 1, false),  E(64, 2, false),  E(64, 4, false),
    E(64, 1, true),   E(64, 2, true),   E(64, 4, true),
    E(128, 1, false), E(128, 2, false), E(128, 4, false),
    E(128, 1, true),  E(128, 2, true),  E(128, 4, true),
};
#undef E
// packed (query head, position) rows: the G*Lq queries of a KV head share one work item
#define P(D, CAUSAL) WF_ATTN_ENTRY(__bf16, DT_BF16, D, D, D, 4, 1, MASK_NONE, CAUSAL, MODE_SPLITP)
static const AttnEntry kTableP[] = {P(64, false), P(64, true), P(128, false), P(128, true)};
#undef P
const AttnEntry* attn_table_split_bf16(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}
const AttnEntry* attn_table_splitp_bf16(int* n) {
  *n = (int)(sizeof(kTableP) / sizeof(kTableP[0]));
  return kTableP;
}
}  // namespace wf
