// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>

namespace kda {

// Validated problem, passed by value to the kernels.
struct Params {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* S0;   // may be null (zero state)
    void* o;
    float* S_T;        // may be null
    int B, T, H, Dk, Dv;
    float scale;
    int o_f32;         // bf16 inputs with a float32 output
};

hipError_t launch_fwd_bf16(const Params& p, hipStream_t stream);  // Dk = Dv = 128, chunk 32
hipError_t launch_fwd_f32(const Params& p, hipStream_t stream);   // Dk = Dv in {64, 128}, chunk 16
hipError_t launch_state_copy(const Params& p, hipStream_t stream); // T = 0: S_T = S0 (or 0)

}  // namespace kda
