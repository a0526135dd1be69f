// fa_kernels.hpp -- internal interface between the C ABI (fa_api.cpp) and the
// kernel translation units.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
    const void *Q, *K, *V;
    void *O;
    float *LSE;
    int B, H, Nq, Nk, d;
    float scale;
    int causal, dtype;
    void *stream;
};

struct BwdArgs {
    const void *Q, *K, *V, *O, *dO;
    const float *LSE;
    void *dQ, *dK, *dV;
    int B, H, Nq, Nk, d;
    float scale;
    int causal, dtype;
    float *Dvec;  // [B*H*Nq] workspace: rowsum(dO * O)
    void *stream;
};

hipError_t launch_fwd(const FwdArgs &a);
constexpr int kBwdStages = 3;
// stage < 0 runs every stage in order.
hipError_t launch_bwd(const BwdArgs &a, int stage);
const char *describe_fwd();
const char *describe_bwd();

}  // namespace fa
