// Host driver for the decode split plan: reads "n_rows hq hkv d window
// max_position" lines, prints "pages_per_split max_splits workspace_bytes".
#include <cstdio>

#include "../../decoder_attention_paged_amd/csrc/decode_plan.h"

int main() {
    int n, hq, hkv, d, w, mp;
    while (std::scanf("%d %d %d %d %d %d", &n, &hq, &hkv, &d, &w, &mp) == 6) {
        const dap::DecodePlan p = dap::decode_plan(n, hq, hkv, d, w, mp);
        std::printf("%d %d %zu\n", p.pages_per_split, p.max_splits, p.workspace_bytes);
    }
    return 0;
}
