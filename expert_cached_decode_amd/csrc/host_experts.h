// Host-side expert compute for the decode host branch (plain C++, no HIP).
#pragma once
#include <stdint.h>

namespace ec {

struct HostPool;

// One batch of host-list experts of one layer step.
struct HostJob {
    const uint8_t* expert_base[1024]; // per host-list index: expert start in the host pool
    int n_experts;
    const int32_t* rewritten; // [T*k] slot or -(1 + host index)
    int T, k, H, I, wdtype;
    const void* x;            // [T][H] f32 (wdtype f32) or bf16
    float* y;                 // [T][H][k] written for host-side pairs (t, j) only (the k partial
                              // sums of one output element are adjacent for the merge)
    float* act;               // scratch [T*k][I]
};

HostPool* host_pool_create(int threads);
void host_pool_destroy(HostPool* p);
void host_pool_run(HostPool* p, const HostJob& job);

} // namespace ec
