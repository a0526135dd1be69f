// fa_kernels.hpp -- internal interface between the C ABI (fa_api.cpp) and the
// kernel translation units.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "fa_types.hpp"

namespace fa {

struct FwdArgs {
    const void *Q, *K, *V;
    void *O;
    float *LSE;
    int B, H, Nq, Nk, d;
    float scale;
    int causal, dtype;
    void *stream;
    // split-KV: num_splits > 1 key ranges of keys_per_split keys (a multiple
    // of fwd_key_tile(d)), partial states in caller workspace, then a merge
    int num_splits = 1, keys_per_split = 0;
    float *Upart = nullptr, *Mpart = nullptr, *Lpart = nullptr;
    Dropout drop{0u, 0u, 0u, 1.f};  // t = 0: no dropout
    // fp16 V^T tiles in the key loop's LDS layout (fwd_packed_v_bytes), or
    // nullptr: the key loop converts and transposes V itself
    uint16_t *Vpk = nullptr;
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
    Dropout drop{0u, 0u, 0u, 1.f};  // t = 0: no dropout
};

// Compute units of the current device (the grid of the persistent kernels).
int compute_units();
hipError_t launch_fwd(const FwdArgs &a);
int fwd_key_tile(int d);  // keys per tile of the forward's key loop for head dim d
int fwd_query_tile();  // query rows per forward workgroup
size_t fwd_packed_v_bytes(int B, int H, int Nk, int d);  // bytes of the packed V^T tiles
constexpr int kBwdStages = 3;
// stage < 0 runs every stage in order.
hipError_t launch_bwd(const BwdArgs &a, int stage);
const char *describe_fwd();
const char *describe_bwd();

}  // namespace fa
