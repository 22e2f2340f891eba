// Block order of the fused step kernel: which workgroups are decode chunks
// and which prefill tiles. Host and device arithmetic only.
//
// Workgroups go in groups of 8 consecutive indices (one per XCD: the
// dispatcher deals consecutive workgroups out to the XCDs in turn). Every
// decode group comes first, in the decode kernel's own order, and the
// prefill groups after them: the prefill tiles then fill the CUs that the
// decode's last round leaves idle as its chunks finish unevenly, instead of
// delaying the decode's start or taking wave slots its page reads need.
// Within each kind the ids keep their order and an id's position mod 8
// equals the id mod 8, so each kind keeps its standalone XCD placement.
#pragma once

namespace dap {

constexpr unsigned kStepGroup = 8;

struct StepRole {
    bool prefill;
    unsigned id;     // prefill block id in [0, 8 ceil(n_pre/8)), or decode block id in [0, 8 ceil(n_dec/8))
};

__host__ __device__ inline unsigned step_groups(unsigned n) { return (n + kStepGroup - 1) / kStepGroup; }

// Workgroups to launch for n_pre prefill and n_dec decode blocks (each kind
// rounded up to whole groups; the extra ids are past n_pre / n_dec).
__host__ __device__ inline unsigned step_blocks(unsigned n_pre, unsigned n_dec) {
    return (step_groups(n_pre) + step_groups(n_dec)) * kStepGroup;
}

__host__ __device__ inline StepRole step_role(unsigned x, unsigned n_pre, unsigned n_dec) {
    (void)n_pre;
    const unsigned dg = step_groups(n_dec);
    if (x < dg * kStepGroup) return {false, x};
    return {true, x - dg * kStepGroup};
}

}  // namespace dap
