/*
 * fa.h -- C ABI of libfa: exact scaled-dot-product attention, computed the
 * FlashAttention way, for AMD Instinct MI355X (gfx950).
 *
 * Operation (definition: lumenova.space "research-attention", section 01;
 * the Attention(Q,K,V) formula of the jrdollar31.pages.dev "Flash Attention"
 * notes), for every batch b and head h independently:
 *
 *     S   = scale * Q K^T                 Q: [Nq, d], K: [Nk, d]
 *     P   = softmax over each row of S    (keys j > i removed when causal)
 *     O   = P V                           V: [Nk, d], O: [Nq, d]
 *     LSE = m + ln(l)  per query row, m = row max of S, l = sum_j exp(S_j - m)
 *
 * The forward never forms S or P in memory: it runs the running-state
 * recurrence (m, l, unnormalised O) over key tiles (research-attention,
 * section 02; page 1 "Flash Attention 原理与实现", section "Forward 的 Tiling
 * 策略") and saves LSE, which is enough to rebuild P later
 * (research-attention, section 04).  The backward recomputes P from Q, K and
 * LSE (page 1, section "Backward 的 Tiling 策略") and returns
 * dV = P^T dO, dQ = scale * dS K, dK = scale * dS^T Q with the softmax
 * gradient dS = P * (dO V^T - rowsum(dO * O)).
 *
 * Conventions shared by every entry point:
 *  - Tensors are caller-owned DEVICE pointers, contiguous row-major
 *    [B, H, N, d] (d fastest), base address 16-byte aligned.  LSE is
 *    [B, H, Nq] float32, natural log, in units of the scaled scores.
 *  - dtype selects the element type of Q, K, V, O, dO, dQ, dK, dV.
 *    FA_F32 reads and writes float32 but rounds the matrix-core operands
 *    (Q, K, V, dO, and the probabilities) to 16-bit first, so it is not a
 *    true-fp32 attention.  Accumulation is float32 in every mode.
 *  - The forward multiplies the probabilities with V on the fp16 matrix core,
 *    converting bf16 (and bf16-rounded fp32) V to fp16: V must satisfy
 *    |V| <= 65504, the fp16 range (for bf16 data: |V| <= 65280, the largest
 *    bf16 number in it).  Inside that range the conversion is exact down to
 *    2^-14, and below that it keeps fp16's subnormal precision (absolute
 *    error <= 2^-25).  A larger value becomes infinity there, and every
 *    output row that gives its key weight comes out non-finite; no error is
 *    returned (the library does not read V on the host).  The backward is
 *    not limited by this.
 *  - causal != 0 keeps key j for query i exactly when j <= i (top-left
 *    alignment, for any Nq and Nk).  Key 0 is always kept, so no row is empty.
 *  - d must be 64 or 128.  B, H, Nq, Nk >= 1 need not be multiples of any
 *    tile size.  B*H*max(Nq,Nk)*d must stay below 2^31 elements.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *    enqueue work on it: they do not synchronise, allocate or keep state
 *    (fa_bwd_noalloc's fixed device array aside), and may be called from
 *    several host threads.  fa_bwd must be ordered after
 *    the fa_fwd that produced O and LSE (same stream, or an event).
 *  - Errors: argument problems are detected on the host before anything is
 *    enqueued and returned as FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED;
 *    FA_ERR_HIP means a launch was rejected by the HIP runtime.  No entry
 *    point aborts or throws across the ABI.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, size <= 0, scale not finite and > 0, workspace too small */
    FA_ERR_UNSUPPORTED = 2, /* head dim or dtype the library has no kernel for, size too large */
    FA_ERR_HIP = 3          /* the HIP runtime rejected a launch */
} fa_status;

typedef enum fa_dtype {
    FA_BF16 = 0,
    FA_F16 = 1,
    FA_F32 = 2
} fa_dtype;

/*
 * Forward.  Reads Q [B,H,Nq,d], K [B,H,Nk,d], V [B,H,Nk,d]; writes
 * O [B,H,Nq,d] (dtype) and LSE [B,H,Nq] (float32).  `scale` multiplies
 * Q K^T before masking and softmax (1/sqrt(d) in the usual definition); it
 * must be finite and positive.  O and LSE must not overlap the inputs.
 */
fa_status fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal,
                 int dtype, void *stream);

/*
 * Forward with a caller-owned workspace: the same O and LSE as fa_fwd, bit
 * for bit, and faster at long key sequences.  A first kernel writes V once
 * into the workspace as fp16 tiles already transposed and placed the way the
 * key loop keeps them in LDS (fp32 inputs are rounded to bf16 first, as
 * everywhere); the key loop then copies each tile in as it is instead of
 * converting and transposing V itself in every workgroup.
 *  - workspace: device memory of at least fa_fwd_workspace_size() bytes
 *    (B*H*ceil(Nk/tile)*tile*d*2, padded to 256), 256-byte aligned; contents
 *    on entry do not matter, on return unspecified.
 *  - When it pays: the packing pass reads and writes V once, and it saves
 *    each workgroup (256 query rows) its own conversion of every V tile, so
 *    the gain grows with the query tiles per head.  At d = 128 on bf16/fp16
 *    data the key loop is also a different kernel (four waves of 64 query
 *    rows, one per SIMD), with the same results.  Measured on MI355X:
 *    4096 rows +7-9 %, 65536 causal rows +12-14 % (d = 128, bf16); 1024
 *    rows against 8192 keys (d = 64, fp16) 7 % slower than fa_fwd.
 *  - Everything else as fa_fwd; FA_ERR_INVALID_ARG also for a null,
 *    misaligned or too small workspace.
 */
size_t fa_fwd_workspace_size(int B, int H, int Nq, int Nk, int d); /* 0 for invalid sizes */
fa_status fa_fwd_ws(const void *Q, const void *K, const void *V, void *O, float *LSE,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Split-KV forward: the same result as fa_fwd (O and LSE, up to rounding
 * order) computed by cutting the keys into `num_splits` ranges of whole key
 * tiles, one workgroup per (query tile, range), each producing the running
 * state (m, l, u) of its range, followed by a merge of the states with the
 * rule that combines key blocks (lumenova.space "research-attention",
 * section 02: m* = max m_g, l = sum exp(m_g - m*) l_g, O = sum exp(m_g - m*)
 * u_g / l).  For shapes with few query tiles -- a single head, a short
 * query block against a long key sequence -- this fills the GPU where fa_fwd
 * cannot.
 *  - num_splits >= 1 and <= FA_MAX_SPLITS; 1 is exactly fa_fwd (workspace
 *    unused, may be NULL).  Ranges past the last key are empty and harmless.
 *  - workspace: caller-owned device memory of at least
 *    fa_fwd_splitkv_workspace_size() bytes, 256-byte aligned, contents on
 *    entry irrelevant, on return unspecified.  Layout: u [G][B*H*Nq][d]
 *    float32, then m and l [G][B*H*Nq] float32 each, G = num_splits.
 *  - Two launches on `stream` (partial states, merge); same argument rules
 *    and errors as fa_fwd, plus FA_ERR_INVALID_ARG for a bad num_splits or a
 *    short / misaligned workspace.
 */
#define FA_MAX_SPLITS 256
size_t fa_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits);
fa_status fa_fwd_splitkv(const void *Q, const void *K, const void *V, void *O, float *LSE,
                         int B, int H, int Nq, int Nk, int d, float scale, int causal,
                         int dtype, int num_splits, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * A split count for fa_fwd_splitkv on one MI355X (256 CUs): 1 when fa_fwd
 * already launches a workgroup per CU, otherwise enough ranges for about one
 * workgroup per CU, keeping at least 512 keys per range.  Returns 0 for
 * invalid sizes.
 */
int fa_fwd_num_splits(int B, int H, int Nq, int Nk, int d, int causal);

/*
 * Attention with dropout on the probabilities (inverted dropout), for
 * training runs that must keep the dropout rate over the same forward and
 * backward range (lumenova.space "research-attention", section 06; the pages
 * leave dropout out of the derivation itself, section 01):
 *   O = (Z * P / (1 - rate)) V, LSE as without dropout;
 *   the backward draws Z again and returns the gradients of that O.
 * Z is not stored: element (b*H + h, query i, key j) is kept unless byte
 * j % 4 of word i % 4 of Philox4x32-10 (Salmon et al., "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC 2011) at counter (j / 4, i / 4, b*H + h, 0)
 * with key (seed & 0xffffffff, seed >> 32) is below t, where
 * t = fa_dropout_threshold(dropout_p); the realised rate is t / 256 and the
 * survivors are scaled by 256 / (256 - t).  The same seed and shape give the
 * same mask in fa_fwd_dropout and fa_bwd_dropout (and on every call).
 *  - dropout_p in [0, 1), finite; t = 0 (dropout_p < 1/512) is exactly
 *    fa_fwd / fa_bwd.  Otherwise FA_ERR_INVALID_ARG.
 *  - Everything else as fa_fwd / fa_bwd (same workspace for the backward).
 */
int fa_dropout_threshold(float dropout_p); /* t in 0..255, or -1 if dropout_p is not in [0, 1) */
fa_status fa_fwd_dropout(const void *Q, const void *K, const void *V, void *O, float *LSE,
                         int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                         float dropout_p, unsigned long long seed, void *stream);
fa_status fa_bwd_dropout(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                         const float *LSE, void *dQ, void *dK, void *dV,
                         int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                         float dropout_p, unsigned long long seed,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace fa_bwd needs for this shape: the float32 row
 * statistic D = rowsum(dO * O) [B,H,Nq], padded to 256 bytes.  Returns 0
 * for invalid sizes.
 */
size_t fa_bwd_workspace_size(int B, int H, int Nq, int Nk, int d);

/*
 * Backward.  Reads Q, K, V, the forward's O and LSE, and the upstream
 * gradient dO [B,H,Nq,d]; writes dQ [B,H,Nq,d], dK and dV [B,H,Nk,d]
 * (dtype).  `workspace` is caller-owned device memory of at least
 * fa_bwd_workspace_size() bytes, 256-byte aligned; its contents on entry
 * do not matter and on return are unspecified.  Same scale/causal/dtype as
 * the forward.  No atomics are used: dQ, dK and dV are bitwise
 * reproducible for a given input, launch and device.
 */
fa_status fa_bwd(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                 const float *LSE, void *dQ, void *dK, void *dV,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_bwd split into its kernel launches, for callers that schedule or time
 * them one by one.  fa_bwd_num_stages() returns the number of stages;
 * running fa_bwd_stage(0..n-1, ...) in order on one stream, with the same
 * arguments and workspace, is exactly fa_bwd.  In general stage 0 computes
 * D = rowsum(dO * O) into the workspace, stage 1 is the K/V-stationary pass
 * that writes dK and dV, stage 2 the Q-stationary pass that writes dQ
 * (stages 1 and 2 both read D).  At d = 128 on bf16/fp16 data stage 0 is
 * the Q-stationary pass, which writes dQ and forms D itself, stage 1 the
 * K/V-stationary pass, and stage 2 launches nothing.  Same argument checks
 * as fa_bwd; an unknown stage returns FA_ERR_INVALID_ARG.
 */
int fa_bwd_num_stages(void);

fa_status fa_bwd_stage(int stage, const void *Q, const void *K, const void *V, const void *O, const void *dO,
                       const float *LSE, void *dQ, void *dK, void *dV,
                       int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The same kernels and results as
 * fa_bwd, bit for bit; the D = rowsum(dO * O) rows that fa_bwd keeps in the
 * caller's workspace live in a fixed device array of the library instead:
 * FA_NOALLOC_MAX_ROWS floats (16 MiB), one copy per GPU, held until the
 * process ends.
 *  - B*H*Nq must not exceed FA_NOALLOC_MAX_ROWS: larger calls return
 *    FA_ERR_UNSUPPORTED without launching anything.
 *  - Every call on one GPU uses that GPU's one array, which keeps the last
 *    call's contents: calls that overlap on one GPU (concurrent streams,
 *    several host threads without ordering) race and may return wrong
 *    gradients.  Calls ordered on one stream are safe.
 *  - The first call on a device (with that device current, hipSetDevice)
 *    looks the array's device address up once; FA_ERR_HIP if that fails.
 *  - Everything else (arguments, checks, errors) as fa_bwd.
 */
#define FA_NOALLOC_MAX_ROWS (4 * 1024 * 1024)
fa_status fa_bwd_noalloc(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                         const float *LSE, void *dQ, void *dK, void *dV,
                         int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                         void *stream);

/* Static string naming the HIP and compiler versions the library was built
 * with and its target, for measurement records. */
const char *fa_build_info(void);

/* Static, human-readable name of a status code ("FA_OK", ...). */
const char *fa_status_string(int status);

/*
 * Description of the kernels fa_fwd / fa_bwd would launch for this
 * head dim, dtype and mask (kernel names, tile sizes, waves per workgroup),
 * or "unsupported".  The string lives in thread-local storage and stays
 * valid until the same thread calls fa_describe again.
 */
const char *fa_describe(int d, int dtype, int causal);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
