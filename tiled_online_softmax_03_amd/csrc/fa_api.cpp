// fa_api.cpp -- the libfa C ABI: argument checks, workspace sizing and
// dispatch to the gfx950 kernels.  Declarations and the full contract are in
// include/fa.h.
#include "fa.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "fa_kernels.hpp"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t pad256(size_t n) { return (n + 255) & ~(size_t)255; }

// Shape / scalar checks shared by fa_fwd and fa_bwd.
fa_status check_common(int B, int H, int Nq, int Nk, int d, float scale, int dtype) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_BF16 && dtype != FA_F16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
    const int64_t n = (Nq > Nk ? Nq : Nk);
    if ((int64_t)B * H * n * d >= kMaxElems) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_bwd_workspace_size(int B, int H, int Nq, int Nk, int d);

fa_status fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H, int Nq,
                 int Nk, int d, float scale, int causal, int dtype, void *stream) {
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
        return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    fa::FwdArgs a{Q, K, V, O, LSE, B, H, Nq, Nk, d, scale, causal ? 1 : 0, dtype, stream};
    return fa::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int H, int Nq, int Nk, int d) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
    const size_t rows = (size_t)B * H * Nq;
    return pad256(rows * sizeof(float));
}

static fa_status bwd_impl(int stage, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                          const float *LSE, void *dQ, void *dK, void *dV, int B, int H, int Nq, int Nk, int d,
                          float scale, int causal, int dtype, void *workspace, size_t workspace_bytes,
                          void *stream) {
    if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV || !workspace) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(LSE) ||
        !aligned16(dQ) || !aligned16(dK) || !aligned16(dV))
        return FA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if (workspace_bytes < fa_bwd_workspace_size(B, H, Nq, Nk, d)) return FA_ERR_INVALID_ARG;
    float *Dvec = static_cast<float *>(workspace);
    fa::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal ? 1 : 0, dtype, Dvec, stream};
    return fa::launch_bwd(a, stage) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_bwd(const void *Q, const void *K, const void *V, const void *O, const void *dO, const float *LSE,
                 void *dQ, void *dK, void *dV, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                 int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return bwd_impl(-1, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal, dtype, workspace,
                    workspace_bytes, stream);
}

int fa_bwd_num_stages(void) { return fa::kBwdStages; }

fa_status fa_bwd_stage(int stage, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                       const float *LSE, void *dQ, void *dK, void *dV, int B, int H, int Nq, int Nk, int d,
                       float scale, int causal, int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (stage < 0 || stage >= fa::kBwdStages) return FA_ERR_INVALID_ARG;
    return bwd_impl(stage, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal, dtype, workspace,
                    workspace_bytes, stream);
}

const char *fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_HIP: return "FA_ERR_HIP";
        default: return "FA_UNKNOWN_STATUS";
    }
}

const char *fa_describe(int d, int dtype, int causal) {
    if ((d != 64 && d != 128) || dtype < FA_BF16 || dtype > FA_F32) return "unsupported";
    static const char *names[] = {"bf16", "f16", "f32"};
    thread_local char buf[512];
    snprintf(buf, sizeof buf, "d=%d dtype=%s causal=%d | fwd: %s | bwd: %s", d, names[dtype], causal ? 1 : 0,
             fa::describe_fwd(), fa::describe_bwd());
    return buf;
}

}  // extern "C"
