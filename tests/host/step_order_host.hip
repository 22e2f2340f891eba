// Host driver for the fused step's block order (step_order.h): reads
// "n_pre n_dec" lines and prints, per case, the number of workgroups and
// then each launched index's role and id ("p<id>" or "d<id>").
#include <cstdio>

#include <hip/hip_runtime.h>

#include "../../decoder_attention_paged_amd/csrc/step_order.h"

int main() {
    unsigned n_pre, n_dec;
    while (std::scanf("%u %u", &n_pre, &n_dec) == 2) {
        const unsigned n = dap::step_blocks(n_pre, n_dec);
        std::printf("%u", n);
        for (unsigned x = 0; x < n; ++x) {
            const dap::StepRole r = dap::step_role(x, n_pre, n_dec);
            std::printf(" %c%u", r.prefill ? 'p' : 'd', r.id);
        }
        std::printf("\n");
    }
    return 0;
}
