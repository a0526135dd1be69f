// fa_api.cpp -- the libfa C ABI: argument checks, workspace sizing and
// dispatch to the gfx950 kernels.  Declarations and the full contract are in
// include/fa.h.
#include "fa.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "fa_kernels.hpp"

// Device scratch of fa_bwd_noalloc: the D = rowsum(dO * O) rows live here
// instead of in a caller workspace.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` only names the symbol:
// its device address comes from hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) float scratch[FA_NOALLOC_MAX_ROWS];

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;
constexpr int kDescribeBytes = 2048;  // fa_describe's buffer (the longest description is well below it)

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

// Dropout parameters for a rate; t = 0 means none.
fa::Dropout make_dropout(int t, unsigned long long seed) {
    fa::Dropout dr{(uint32_t)(seed & 0xffffffffull), (uint32_t)(seed >> 32), (uint32_t)t, 1.f};
    if (t > 0) dr.keep_scale = 256.f / (float)(256 - t);
    return dr;
}

}  // namespace

extern "C" {

size_t fa_bwd_workspace_size(int B, int H, int Nq, int Nk, int d);

int fa_dropout_threshold(float dropout_p) {
    if (!isfinite(dropout_p) || dropout_p < 0.f || dropout_p >= 1.f) return -1;
    const int t = (int)floorf(dropout_p * 256.f + 0.5f);
    return t > 255 ? 255 : t;
}

static fa_status fwd_impl(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H, int Nq,
                          int Nk, int d, float scale, int causal, int dtype, fa::Dropout drop, void *stream) {
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
        return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    fa::FwdArgs a{Q, K, V, O, LSE, B, H, Nq, Nk, d, scale, causal ? 1 : 0, dtype, stream};
    a.drop = drop;
    return fa::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H, int Nq,
                 int Nk, int d, float scale, int causal, int dtype, void *stream) {
    return fwd_impl(Q, K, V, O, LSE, B, H, Nq, Nk, d, scale, causal, dtype, make_dropout(0, 0), stream);
}

size_t fa_fwd_workspace_size(int B, int H, int Nq, int Nk, int d) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || (d != 64 && d != 128)) return 0;
    return pad256(fa::fwd_packed_v_bytes(B, H, Nk, d));
}

fa_status fa_fwd_ws(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H, int Nq, int Nk,
                    int d, float scale, int causal, int dtype, void *workspace, size_t workspace_bytes,
                    void *stream) {
    if (!Q || !K || !V || !O || !LSE || !workspace) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
        return FA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if (workspace_bytes < fa_fwd_workspace_size(B, H, Nq, Nk, d)) return FA_ERR_INVALID_ARG;
    fa::FwdArgs a{Q, K, V, O, LSE, B, H, Nq, Nk, d, scale, causal ? 1 : 0, dtype, stream};
    a.Vpk = static_cast<uint16_t *>(workspace);
    return fa::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_dropout(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H, int Nq,
                         int Nk, int d, float scale, int causal, int dtype, float dropout_p, unsigned long long seed,
                         void *stream) {
    const int t = fa_dropout_threshold(dropout_p);
    if (t < 0) return FA_ERR_INVALID_ARG;
    return fwd_impl(Q, K, V, O, LSE, B, H, Nq, Nk, d, scale, causal, dtype, make_dropout(t, seed), stream);
}

size_t fa_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || num_splits < 1 || num_splits > FA_MAX_SPLITS) return 0;
    if (num_splits == 1) return 0;
    const size_t rows = (size_t)B * H * Nq * (size_t)num_splits;
    return pad256(rows * (size_t)d * sizeof(float)) + 2 * pad256(rows * sizeof(float));
}

fa_status fa_fwd_splitkv(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int H, int Nq,
                         int Nk, int d, float scale, int causal, int dtype, int num_splits, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_INVALID_ARG;
    if (num_splits == 1) return fa_fwd(Q, K, V, O, LSE, B, H, Nq, Nk, d, scale, causal, dtype, stream);
    if (!Q || !K || !V || !O || !LSE || !workspace) return FA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
        return FA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    const size_t need = fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, num_splits);
    if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
    const int BQ = fa::fwd_query_tile(), BC = fa::fwd_key_tile(d);
    const int64_t grid = (int64_t)B * H * ((Nq + BQ - 1) / BQ) * num_splits;
    if (grid >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
    const size_t rows = (size_t)B * H * Nq * (size_t)num_splits;
    char *ws = static_cast<char *>(workspace);
    float *U = reinterpret_cast<float *>(ws);
    float *M = reinterpret_cast<float *>(ws + pad256(rows * (size_t)d * sizeof(float)));
    float *L = reinterpret_cast<float *>(ws + pad256(rows * (size_t)d * sizeof(float)) + pad256(rows * sizeof(float)));
    // under the causal mask only keys 0 .. Nq - 1 can be kept: the ranges cover those
    const int Nk_used = (causal && Nk > Nq) ? Nq : Nk;
    const int n_kt = (Nk_used + BC - 1) / BC;
    const int tiles_per_split = (n_kt + num_splits - 1) / num_splits;
    fa::FwdArgs a{Q, K, V, O, LSE, B, H, Nq, Nk, d, scale, causal ? 1 : 0, dtype, stream};
    a.num_splits = num_splits;
    a.keys_per_split = tiles_per_split * BC;
    a.Upart = U;
    a.Mpart = M;
    a.Lpart = L;
    return fa::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_num_splits(int B, int H, int Nq, int Nk, int d, int causal) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || (d != 64 && d != 128)) return 0;
    // Under the causal mask no query row sees a key past Nq - 1 (key j is kept for
    // query i only when j <= i), so ranges beyond that would only be empty.
    if (causal && Nk > Nq) Nk = Nq;
    // Measured on MI355X (one head of 4096 x 4096, d64; 8 heads of one query
    // against 8192 keys; 32 heads of 128 queries against 32768 keys): the
    // best count gives about one workgroup per CU and keeps 8 or more key
    // tiles per range; beyond that the extra prologues and the merge cost more
    // than the added parallelism gains.  (512 keys = 8 tiles of 64 at d = 128, 4 of
    // 128 at d = 64.)
    constexpr int kCUs = 256, kMinKeysPerSplit = 512;
    const int BQ = fa::fwd_query_tile(), BC = fa::fwd_key_tile(d);
    const int64_t wgs = (int64_t)B * H * ((Nq + BQ - 1) / BQ);
    if (wgs >= kCUs) return 1;
    const int n_kt = (Nk + BC - 1) / BC;
    int64_t g = (kCUs + wgs - 1) / wgs;
    const int64_t g_max = (int64_t)n_kt * BC / kMinKeysPerSplit;
    if (g > g_max) g = g_max;
    if (g > FA_MAX_SPLITS) g = FA_MAX_SPLITS;
    return g < 1 ? 1 : (int)g;
}

size_t fa_bwd_workspace_size(int B, int H, int Nq, int Nk, int d) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
    const size_t rows = (size_t)B * H * Nq;
    return pad256(rows * sizeof(float));
}

// Pointer checks of the backward: none null, all 16-byte aligned.
static bool bwd_ptrs_ok(const void *Q, const void *K, const void *V, const void *O, const void *dO, const float *LSE,
                        const void *dQ, const void *dK, const void *dV) {
    if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return false;
    return aligned16(Q) && aligned16(K) && aligned16(V) && aligned16(O) && aligned16(dO) && aligned16(LSE) &&
           aligned16(dQ) && aligned16(dK) && aligned16(dV);
}

static fa_status bwd_impl(int stage, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                          const float *LSE, void *dQ, void *dK, void *dV, int B, int H, int Nq, int Nk, int d,
                          float scale, int causal, int dtype, void *workspace, size_t workspace_bytes,
                          void *stream, fa::Dropout drop = make_dropout(0, 0)) {
    if (!workspace || !bwd_ptrs_ok(Q, K, V, O, dO, LSE, dQ, dK, dV)) return FA_ERR_INVALID_ARG;
    if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if (workspace_bytes < fa_bwd_workspace_size(B, H, Nq, Nk, d)) return FA_ERR_INVALID_ARG;
    float *Dvec = static_cast<float *>(workspace);
    fa::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal ? 1 : 0, dtype, Dvec, stream};
    a.drop = drop;
    return fa::launch_bwd(a, stage) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_bwd_dropout(const void *Q, const void *K, const void *V, const void *O, const void *dO, const float *LSE,
                         void *dQ, void *dK, void *dV, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                         int dtype, float dropout_p, unsigned long long seed, void *workspace,
                         size_t workspace_bytes, void *stream) {
    const int t = fa_dropout_threshold(dropout_p);
    if (t < 0) return FA_ERR_INVALID_ARG;
    return bwd_impl(-1, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal, dtype, workspace,
                    workspace_bytes, stream, make_dropout(t, seed));
}

fa_status fa_bwd(const void *Q, const void *K, const void *V, const void *O, const void *dO, const float *LSE,
                 void *dQ, void *dK, void *dV, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                 int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return bwd_impl(-1, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal, dtype, workspace,
                    workspace_bytes, stream);
}

// Device address of this GPU's `scratch`, looked up once per device with that
// device current (the first fa_bwd_noalloc call on it); nullptr if the lookup
// fails.
static void *noalloc_scratch(int *hip_err) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *ptr[kMaxDevices];
    static bool done[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *hip_err = 1;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!done[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            *hip_err = 1;
            return nullptr;  // not cached: a later call tries again
        }
        ptr[dev] = p;
        done[dev] = true;
    }
    return ptr[dev];
}

fa_status fa_bwd_noalloc(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                         const float *LSE, void *dQ, void *dK, void *dV, int B, int H, int Nq, int Nk, int d,
                         float scale, int causal, int dtype, void *stream) {
    // the same argument checks as fa_bwd first, so a bad call never touches the scratch
    if (!bwd_ptrs_ok(Q, K, V, O, dO, LSE, dQ, dK, dV)) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if ((int64_t)B * H * Nq > (int64_t)FA_NOALLOC_MAX_ROWS) return FA_ERR_UNSUPPORTED;
    int hip_err = 0;
    void *ws = noalloc_scratch(&hip_err);
    if (!ws) return FA_ERR_HIP;
    return bwd_impl(-1, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal, dtype, ws,
                    (size_t)FA_NOALLOC_MAX_ROWS * sizeof(float), stream);
}

int fa_bwd_num_stages(void) { return fa::kBwdStages; }

fa_status fa_bwd_stage(int stage, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                       const float *LSE, void *dQ, void *dK, void *dV, int B, int H, int Nq, int Nk, int d,
                       float scale, int causal, int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (stage < 0 || stage >= fa::kBwdStages) return FA_ERR_INVALID_ARG;
    return bwd_impl(stage, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Nq, Nk, d, scale, causal, dtype, workspace,
                    workspace_bytes, stream);
}

#define FA_STR2(x) #x
#define FA_STR(x) FA_STR2(x)
const char *fa_build_info(void) {
    return "HIP " FA_STR(HIP_VERSION_MAJOR) "." FA_STR(HIP_VERSION_MINOR) "." FA_STR(HIP_VERSION_PATCH)
           ", clang " __clang_version__ ", offload arch gfx950";
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
    thread_local char buf[kDescribeBytes];
    const int n = snprintf(buf, sizeof buf, "d=%d dtype=%s causal=%d | fwd: %s | bwd: %s", d, names[dtype],
                           causal ? 1 : 0, fa::describe_fwd(), fa::describe_bwd());
    // the kernel descriptions are fixed strings: one that did not fit is a bug of this file
    return (n < 0 || n >= (int)sizeof buf) ? "fa_describe: description longer than its buffer" : buf;
}

}  // extern "C"
