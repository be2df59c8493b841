// Prefill MoE layer: full-layer double-buffered expert upload overlapped with
// a grouped expert GEMM (host-side orchestration + kernel launchers).
#pragma once
#include "ec_internal.h"

namespace ec {

struct PrefillState {
    int Tp = 0;              // prefill_max_tokens (0: disabled)
    uint8_t* buf[2] = {nullptr, nullptr}; // two full-layer expert buffers
    int buf_layer[2] = {-1, -1};          // layer uploaded (or being uploaded) into each buffer
    bool used[2] = {false, false};        // a compute has been enqueued on the buffer
    int last = 1;                         // buffer of the previous compute
    hipEvent_t loaded[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr};
    int32_t* ids = nullptr;  // [Tp*k]
    float* w = nullptr;      // [Tp*k]
    int32_t* cnt = nullptr;  // [E]
    int32_t* segc = nullptr; // [ceil(Tp*k / 512)][E] per-segment counts, then their column prefix sums
    int32_t* off = nullptr;  // [E+1] row offsets of each expert's group
    int32_t* toff = nullptr; // [E+1] tile offsets (64-row tiles)
    int32_t* perm = nullptr; // [Tp*k] grouped row -> pair index t*k+j
    uint16_t* act = nullptr; // [Tp*k][I] bf16 SwiGLU activations, grouped order
    float* y = nullptr;      // [Tp*k][H] expert outputs per pair
};

struct PrefillCall {
    const uint8_t* host_pool;
    int P;                   // layers held by the host pool (layer l reads pool layer l % P)
    int layer, L, E, k, H, I, T, wdtype;
    uint64_t layer_bytes, expert_bytes;
    const void* x;
    const float* logits;
    void* out;
    hipStream_t compute, copy;
    int overlap;
};

void prefill_carve(PrefillState& p, Carve& d, int Tp, int E, int k, int H, int I, uint64_t layer_bytes);
hipError_t prefill_init(PrefillState& p);
void prefill_reset_device(PrefillState& p, hipStream_t s);
void prefill_destroy(PrefillState& p);
hipError_t prefill_layer(PrefillState& p, const PrefillCall& c);

} // namespace ec
