// fa_bwd.hip -- attention backward for gfx950.
//
// Method: page 1 "Flash Attention 原理与实现", section "Backward 的 Tiling
// 策略": S and P are recomputed block by block from Q, K and the saved
// statistics instead of being stored; dV = P^T dO, dP = dO V^T, dQ = dS K,
// dK = dS^T Q.  P is rebuilt as exp(s - LSE) (lumenova.space
// "research-attention", section 04).  The softmax gradient is the standard
// vector-Jacobian product dS = P * (dP - D) with D_i = sum_j P_ij dP_ij, and
// D_i = rowsum(dO_i * O_i) because O_i = sum_j P_ij V_j.  The cross-block sums
// of dQ and dK use the second option of page 1's section "实际实现中的注意事项"
// (item 3): partial sums kept on chip, no atomics.
//
// Three launches on the caller's stream, each a stage of fa_bwd_stage:
//   0. bwd_pre_kernel   D = rowsum(dO * O) in fp32.
//   1. bwd_dkdv_kernel  K/V-stationary: a workgroup owns 128 keys of one head
//                       (8 waves, two per SIMD: 4 key groups x 2 query halves;
//                       K and V rows in LDS) and walks
//                       the query tiles, recomputing S, P, dP and dS, and
//                       accumulating dV^T += dO^T P and dK^T += Q^T dS in
//                       registers.  Q and dO are staged row-major through LDS
//                       (double-buffered); their transposes are read with
//                       ds_read_b64_tr_b16.  For d = 128 16-bit data without
//                       dropout, bwd_dkdv_kv_kernel does the same with four
//                       waves, one per SIMD, whose K and V fragments stay in
//                       registers for the whole pass.
//   2. bwd_dq_kernel    Q-stationary: a workgroup owns 256 query rows (32 per
//                       wave, Q and dO rows held in VGPRs) and streams K/V
//                       tiles like the forward: S^T = K Q^T, dP^T = V dO^T,
//                       dS^T, dQ^T += K^T dS^T.  For d = 128 16-bit data
//                       without dropout, bwd_dq_kv_kernel: four waves, one per
//                       SIMD, 64 rows each, so every K/V fragment read from
//                       LDS feeds two products.
// dQ, dK and dV are therefore deterministic.  The price is that S and dP are
// formed twice (7 matrix products instead of 5).
//
// Dropout (DROP = true): with keep flags Z drawn again from the counter-based
// generator the forward used (fa_common.hpp), dV takes P~ = Z P / (1 - rate),
// dP becomes Z (dO V^T) / (1 - rate), and dS = P (dP - D) with the undropped
// P; D = rowsum(dO * O) still equals sum_j P_ij dP_ij because O is the
// dropped forward's output.
#include <algorithm>
#include <type_traits>

#include "fa_common.hpp"
#include "fa_kernels.hpp"

// Query rows per step of the dK/dV pass at d = 64 (64 at d = 128).
#ifndef FA_DKDV_ROWS_D64
#define FA_DKDV_ROWS_D64 128
#endif
// The d = 128 16-bit dK/dV pass without dropout keeps K and V in registers
// (bwd_dkdv_kv_kernel); 0 selects the two-waves-per-SIMD pass for it too.
#ifndef FA_DKDV_KV
#define FA_DKDV_KV 1
#endif
// The d = 128 16-bit dQ pass without dropout takes 64 query rows per wave
// (bwd_dq_kv_kernel); 0 selects the two-waves-per-SIMD pass for it too.
#ifndef FA_DQ_KV
#define FA_DQ_KV 1
#endif

namespace fa {

// Floats of eight consecutive stored elements, without rounding fp32 data.
template <int E>
__device__ __forceinline__ void load8_stored(const void *base, int64_t elem, float out[8]) {
    if constexpr (E == ELT_F32) {
        const f32x4_t *p = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(base) + elem);
        const f32x4_t a = p[0], b = p[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
    } else {
        load8_float<E>(base, elem, out);
    }
}

// ---------------------------------------------------------------- 0. D = rowsum(dO * O)
template <int D, int E>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const void *__restrict__ O, const void *__restrict__ dO,
                                                      float *__restrict__ Dvec, int64_t rows) {
    constexpr int NCH = D / 8;      // lanes per row
    constexpr int RPB = 256 / NCH;  // rows per block
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / NCH;
    const int c = tid % NCH;
    float acc = 0.f;
    if (row < rows) {
        float o[8], go[8];
        load8_stored<E>(O, row * D + c * 8, o);
        load8_float<E>(dO, row * D + c * 8, go);  // dO as the products see it
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(o[e], go[e], acc);
    }
#pragma unroll
    for (int off = NCH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && c == 0) Dvec[row] = acc;
}

// ---------------------------------------------------------------- 1. dK, dV
// Eight waves = 4 key groups x 2 query halves.  Wave w owns keys
// k0 + 32*(w % 4) .. +31 and, in every 64-row query step, rows 32*(w / 4) ..
// +31 of it; the two waves of a key group (which share a SIMD) keep separate
// dK^T / dV^T partial sums that are added through LDS at the end.  K and V
// fragments are read from LDS, so no VGPRs hold them.
template <int D, int E, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv_kernel(const void *__restrict__ Q, const void *__restrict__ K, const void *__restrict__ V,
                     const void *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Dvec,
                     void *__restrict__ dK, void *__restrict__ dV, int BH, int Nq, int Nk, float scale,
                     float scale_log2, int n_kt, Dropout dr) {
    constexpr int NW = 8, NT = 512;
    constexpr int NKG = 4;        // key groups
    constexpr int BKC = 32 * NKG; // keys per workgroup
    // Query rows per step: at d = 64 every product carries half the work of
    // d = 128, so a step takes twice the rows (each wave walks its half in
    // 32-row blocks) to keep the barrier, the staging and the exponentials the
    // same share of the time.
    constexpr int BQ = D == 64 ? FA_DKDV_ROWS_D64 : 64;
    constexpr int QH = BQ / 2;    // rows of one query half in a step
    static_assert(QH % 32 == 0, "query halves are whole 32-row blocks");
    constexpr int NCH = D / 8;    // 16-byte chunks per row
    constexpr int NKS = D / 16;   // k-steps over the head dim
    constexpr int NDB = D / 32;   // 32-row blocks of dK^T / dV^T
    constexpr bool DMA = E != ELT_F32;  // 16-bit Q / dO go global -> LDS directly
    constexpr int CH_PER_T = DMA ? 1 : BQ * NCH / NT;  // register staging (fp32 -> bf16)
    static_assert(BQ * NCH % NT == 0 && BKC * NCH % NT == 0, "staging split");

    // Q/dO tiles (double-buffered), this workgroup's K and V rows, row statistics.
    // After the loop the same space holds the query-half partial sums (needs
    // NKG * 2 * NDB * 16 * 64 floats = 128 KiB for d = 128).
    constexpr int QBYTES = 2 * 2 * BQ * D * 2, KVBYTES = 2 * BKC * D * 2, STATS = 2 * 2 * BQ * 4;
    constexpr int XBYTES = NKG * 2 * NDB * 16 * 64 * 4;
    constexpr int LDS_BYTES = (QBYTES + KVBYTES + STATS) > XBYTES ? (QBYTES + KVBYTES + STATS) : XBYTES;
    __shared__ __attribute__((aligned(16))) unsigned char lds_raw[LDS_BYTES];
    uint16_t (*Qs)[BQ * D] = reinterpret_cast<uint16_t (*)[BQ * D]>(lds_raw);
    uint16_t (*dOs)[BQ * D] = reinterpret_cast<uint16_t (*)[BQ * D]>(lds_raw + 2 * BQ * D * 2);
    uint16_t *Ks = reinterpret_cast<uint16_t *>(lds_raw + QBYTES);
    uint16_t *Vs = reinterpret_cast<uint16_t *>(lds_raw + QBYTES + BKC * D * 2);
    float (*lse2)[BQ] = reinterpret_cast<float (*)[BQ]>(lds_raw + QBYTES + KVBYTES);
    float (*dvec)[BQ] = reinterpret_cast<float (*)[BQ]>(lds_raw + QBYTES + KVBYTES + 2 * BQ * 4);
    float *xchg = reinterpret_cast<float *>(lds_raw);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int kg = wave % NKG, qh = wave / NKG;

    int bh, kt;
    if constexpr (CAUSAL) {
        // low key tiles meet the most query rows: dispatch them first
        const int L = blockIdx.x;
        kt = L / BH;
        bh = L % BH;
    } else {
        const int L = xcd_remap(blockIdx.x, gridDim.x);
        bh = L / n_kt;
        kt = L % n_kt;
    }
    const int64_t q_head = (int64_t)bh * Nq * D;
    const int64_t k_head = (int64_t)bh * Nk * D;
    const int k0 = kt * BKC;
    const int kw0 = k0 + kg * 32;  // first key of this wave
    const int kw = kw0 + l32;      // this lane's key

    const int n_qt = (Nq + BQ - 1) / BQ;
    const int qt_begin = CAUSAL ? min(k0 / BQ, n_qt) : 0;  // earlier rows see none of these keys

    // ---- this workgroup's K and V rows into LDS (row-major, swizzled; zero past Nk)
#pragma unroll
    for (int j = 0; j < BKC * NCH / NT; ++j) {
        const int i = tid + j * NT;
        const int row = i / NCH, c = i % NCH;
        u32x4_t kz = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
        if (k0 + row < Nk) {
            kz = load8_operand<E>(K, k_head + (int64_t)(k0 + row) * D + c * 8);
            vz = load8_operand<E>(V, k_head + (int64_t)(k0 + row) * D + c * 8);
        }
        *reinterpret_cast<u32x4_t *>(&Ks[tile_off<D>(row, c * 8)]) = kz;
        *reinterpret_cast<u32x4_t *>(&Vs[tile_off<D>(row, c * 8)]) = vz;
    }

    // ---- staging of one query tile
    const void *Qh = static_cast<const char *>(Q) + q_head * (E == ELT_F32 ? 4 : 2);
    const void *dOh = static_cast<const char *>(dO) + q_head * (E == ELT_F32 ? 4 : 2);
    u32x4_t qreg[CH_PER_T], dreg[CH_PER_T];
    float lreg = 0.f, dvreg = 0.f;
    int qt_next_row0 = 0;
    auto load_tile = [&](int qt, int buf) __attribute__((always_inline)) {
        const int q0 = qt * BQ;
        qt_next_row0 = q0;
        // Only the waves whose threads store the row statistics load them (one
        // 64-lane load each instead of one per wave), ahead of the copies so
        // that the copies share the basic block of the products that follow.
        if (__builtin_amdgcn_readfirstlane(wave) < BQ / 64) {
            const int qq = min(q0 + (tid & (BQ - 1)), Nq - 1);
            lreg = LSE[(int64_t)bh * Nq + qq];
            dvreg = Dvec[(int64_t)bh * Nq + qq];
        }
        if constexpr (DMA) {
            dma_tile<D, BQ, NW>(Qh, q0, Nq, Qs[buf], wave, lane);
            dma_tile<D, BQ, NW>(dOh, q0, Nq, dOs[buf], wave, lane);
        } else {
#pragma unroll
            for (int j = 0; j < CH_PER_T; ++j) {
                const int i = tid + j * NT;
                const int row = i / NCH, c = i % NCH;
                const int qq = q0 + row;
                qreg[j] = u32x4_t{0u, 0u, 0u, 0u};
                dreg[j] = u32x4_t{0u, 0u, 0u, 0u};
                if (qq < Nq) {
                    qreg[j] = load8_operand<E>(Q, q_head + (int64_t)qq * D + c * 8);
                    dreg[j] = load8_operand<E>(dO, q_head + (int64_t)qq * D + c * 8);
                }
            }
        }
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
        if constexpr (!DMA) {
#pragma unroll
            for (int j = 0; j < CH_PER_T; ++j) {
                const int i = tid + j * NT;
                const int row = i / NCH, c = i % NCH;
                *reinterpret_cast<u32x4_t *>(&Qs[buf][tile_off<D>(row, c * 8)]) = qreg[j];
                *reinterpret_cast<u32x4_t *>(&dOs[buf][tile_off<D>(row, c * 8)]) = dreg[j];
            }
        }
        if (tid < BQ) {
            const bool real = qt_next_row0 + tid < Nq;
            lse2[buf][tid] = real ? lreg * kLog2e : INFINITY;  // P = 0 on padding rows
            dvec[buf][tid] = real ? (DROP ? dvreg : -dvreg) : 0.f;  // -D: the dP chains start from it
        }
    };

    f32x16_t dvT[NDB], dkT[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) { dvT[db] = f32x16_t{}; dkT[db] = f32x16_t{}; }

    if (qt_begin < n_qt) {
        load_tile(qt_begin, 0);
        store_tile(0);
    }
    wait_vmem();
    __syncthreads();

    // One query tile; BUF (compile-time) is the LDS buffer it reads, so every LDS
    // address is a fixed offset from a per-lane base.
    auto step = [&](int qt, auto buf_c) __attribute__((always_inline)) {
        constexpr int buf = decltype(buf_c)::value;
        const bool more = qt + 1 < n_qt;
        // The prefetch goes out on every step (the last step copies its own tile
        // into the idle buffer again): no branch separates it from the products.
        load_tile(more ? qt + 1 : qt, buf ^ 1);  // in flight during this step's math
        const uint16_t *qs = Qs[buf];
        const uint16_t *ds = dOs[buf];
        // (The d = 128 branch keeps a single block in this exact form: the compiler's
        // schedule of the d = 128 kernel was measured 7 % slower when it was
        // written as the one-iteration case of the loop below.)
        if constexpr (QH == 32) {
            const int q0 = qt * BQ + qh * 32;

            if (!CAUSAL || q0 + 31 >= kw0) {  // else every row of the block precedes this wave's keys
                // S = Q K^T and dP = dO V^T: lane = key, register r -> query q0 + 8*(r/4) + 4*g + r%4
                f32x16_t s = f32x16_t{}, dp = f32x16_t{};
                if constexpr (!DROP) {
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const f32x4_t D4 = *reinterpret_cast<const f32x4_t *>(&dvec[buf][qh * 32 + 8 * rq + 4 * g]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) dp[4 * rq + i] = D4[i];  // -D of the block's rows
                    }
                }
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int qoff = tile_off<D>(qh * 32 + l32, 16 * ks + 8 * g);
                    const int koff = tile_off<D>(kg * 32 + l32, 16 * ks + 8 * g);
                    s = mfma_in<E>(*reinterpret_cast<const u32x4_t *>(&qs[qoff]),
                                   *reinterpret_cast<const u32x4_t *>(&Ks[koff]), s);
                    dp = mfma_in<E>(*reinterpret_cast<const u32x4_t *>(&ds[qoff]),
                                    *reinterpret_cast<const u32x4_t *>(&Vs[koff]), dp);
                }
                // P = exp2(s*c - LSE*log2e), dS = P (dP - D)
                uint32_t pp[8], dd[8];
                uint32_t keep16 = 0xffffu;  // dropout keep flags: bit 4rq + i, query q0 + 8rq + 4g + i
                if constexpr (DROP) keep16 = dropout_keep_key_lane(dr, (uint32_t)bh, (uint32_t)(q0 + 4 * g), (uint32_t)kw, lane);
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const f32x4_t L4 = *reinterpret_cast<const f32x4_t *>(&lse2[buf][qh * 32 + 8 * rq + 4 * g]);
                    const f32x4_t D4 = *reinterpret_cast<const f32x4_t *>(&dvec[buf][qh * 32 + 8 * rq + 4 * g]);
                    const uint32_t keep = (keep16 >> (4 * rq)) & 0xfu;  // bit i: query q0 + 8rq + 4g + i kept
                    float p[4], t[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 4 * rq + i;
                        float pv = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -L4[i]));
                        if (CAUSAL && kw > q0 + 8 * rq + 4 * g + i) pv = 0.f;
                        if constexpr (DROP) {
                            const bool kept = (keep >> i) & 1u;
                            p[i] = kept ? pv * dr.keep_scale : 0.f;
                            t[i] = pv * ((kept ? dp[r] * dr.keep_scale : 0.f) - D4[i]);
                        } else {
                            p[i] = pv;
                            t[i] = pv * dp[r];  // dp holds dP - D
                        }
                    }
                    pp[2 * rq] = pack_in<E>(p[0], p[1]);
                    pp[2 * rq + 1] = pack_in<E>(p[2], p[3]);
                    dd[2 * rq] = pack_in<E>(t[0], t[1]);
                    dd[2 * rq + 1] = pack_in<E>(t[2], t[3]);
                }
                // dV^T += dO^T P and dK^T += Q^T dS; k-step h covers query rows 16h..16h+15 of the block
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4_t bp = {pp[4 * h], pp[4 * h + 1], pp[4 * h + 2], pp[4 * h + 3]};
                    const u32x4_t bs = {dd[4 * h], dd[4 * h + 1], dd[4 * h + 2], dd[4 * h + 3]};
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        dvT[db] = mfma_in<E>(tr_operand<D>(ds, qh * 32 + 16 * h, 32 * db, lane), bp, dvT[db]);
                        dkT[db] = mfma_in<E>(tr_operand<D>(qs, qh * 32 + 16 * h, 32 * db, lane), bs, dkT[db]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int sub = 0; sub < QH / 32; ++sub) {
                const int r0 = qh * QH + 32 * sub;  // first row of this 32-row block in the tile
                const int q0 = qt * BQ + r0;

                if (!CAUSAL || q0 + 31 >= kw0) {  // else every row of the block precedes this wave's keys
                    // S = Q K^T and dP = dO V^T: lane = key, register r -> query q0 + 8*(r/4) + 4*g + r%4
                    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
                    if constexpr (!DROP) {
#pragma unroll
                        for (int rq = 0; rq < 4; ++rq) {
                            const f32x4_t D4 = *reinterpret_cast<const f32x4_t *>(&dvec[buf][r0 + 8 * rq + 4 * g]);
#pragma unroll
                            for (int i = 0; i < 4; ++i) dp[4 * rq + i] = D4[i];  // -D of the block's rows
                        }
                    }
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const int qoff = tile_off<D>(r0 + l32, 16 * ks + 8 * g);
                        const int koff = tile_off<D>(kg * 32 + l32, 16 * ks + 8 * g);
                        s = mfma_in<E>(*reinterpret_cast<const u32x4_t *>(&qs[qoff]),
                                       *reinterpret_cast<const u32x4_t *>(&Ks[koff]), s);
                        dp = mfma_in<E>(*reinterpret_cast<const u32x4_t *>(&ds[qoff]),
                                        *reinterpret_cast<const u32x4_t *>(&Vs[koff]), dp);
                    }
                    // P = exp2(s*c - LSE*log2e), dS = P (dP - D)
                    uint32_t pp[8], dd[8];
                    uint32_t keep16 = 0xffffu;  // dropout keep flags: bit 4rq + i, query q0 + 8rq + 4g + i
                    if constexpr (DROP) keep16 = dropout_keep_key_lane(dr, (uint32_t)bh, (uint32_t)(q0 + 4 * g), (uint32_t)kw, lane);
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const f32x4_t L4 = *reinterpret_cast<const f32x4_t *>(&lse2[buf][r0 + 8 * rq + 4 * g]);
                        const f32x4_t D4 = *reinterpret_cast<const f32x4_t *>(&dvec[buf][r0 + 8 * rq + 4 * g]);
                        const uint32_t keep = (keep16 >> (4 * rq)) & 0xfu;  // bit i: query q0 + 8rq + 4g + i kept
                        float p[4], t[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = 4 * rq + i;
                            float pv = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -L4[i]));
                            if (CAUSAL && kw > q0 + 8 * rq + 4 * g + i) pv = 0.f;
                            if constexpr (DROP) {
                                const bool kept = (keep >> i) & 1u;
                                p[i] = kept ? pv * dr.keep_scale : 0.f;
                                t[i] = pv * ((kept ? dp[r] * dr.keep_scale : 0.f) - D4[i]);
                            } else {
                                p[i] = pv;
                                t[i] = pv * dp[r];  // dp holds dP - D
                            }
                        }
                        pp[2 * rq] = pack_in<E>(p[0], p[1]);
                        pp[2 * rq + 1] = pack_in<E>(p[2], p[3]);
                        dd[2 * rq] = pack_in<E>(t[0], t[1]);
                        dd[2 * rq + 1] = pack_in<E>(t[2], t[3]);
                    }
                    // dV^T += dO^T P and dK^T += Q^T dS; k-step h covers query rows 16h..16h+15 of the block
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const u32x4_t bp = {pp[4 * h], pp[4 * h + 1], pp[4 * h + 2], pp[4 * h + 3]};
                        const u32x4_t bs = {dd[4 * h], dd[4 * h + 1], dd[4 * h + 2], dd[4 * h + 3]};
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            dvT[db] = mfma_in<E>(tr_operand<D>(ds, r0 + 16 * h, 32 * db, lane), bp, dvT[db]);
                            dkT[db] = mfma_in<E>(tr_operand<D>(qs, r0 + 16 * h, 32 * db, lane), bs, dkT[db]);
                        }
                    }
                }
            }
        }
        store_tile(buf ^ 1);
        wait_vmem();
        __syncthreads();
    };
    for (int qt = qt_begin; qt < n_qt; qt += 2) {
        step(qt, std::integral_constant<int, 0>{});
        if (qt + 1 < n_qt) step(qt + 1, std::integral_constant<int, 1>{});
    }

    // ---- add the two query halves' partial sums (LDS, lane-major: conflict-free)
    __syncthreads();  // every wave is done with the tiles the exchange area overlays
    float *x = xchg + (size_t)kg * (2 * NDB * 16 * 64);
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                x[((0 * NDB + db) * 16 + r) * 64 + lane] = dkT[db][r];
                x[((1 * NDB + db) * 16 + r) * 64 + lane] = dvT[db][r];
            }
    }
    __syncthreads();
    if (qh == 0 && kw < Nk) {
        // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane = key, register r -> head dim 32db + 8*(r/4) + 4*g + r%4
        const int64_t row = k_head + (int64_t)kw * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                float a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * rq + i;
                    a[i] = (dkT[db][r] + x[((0 * NDB + db) * 16 + r) * 64 + lane]) * scale;
                    b[i] = dvT[db][r] + x[((1 * NDB + db) * 16 + r) * 64 + lane];
                }
                const int col = db * 32 + 8 * rq + 4 * g;
                store4<E>(dK, row + col, a[0], a[1], a[2], a[3]);
                store4<E>(dV, row + col, b[0], b[1], b[2], b[3]);
            }
    }
}

// ---------------------------------------------------------------- 1'. dK, dV with K and V in registers
// The d = 128 16-bit pass without dropout.  Four waves, one per SIMD, each
// owning 32 keys for the whole pass, so its K and V fragments (the B operands
// of S = Q K^T and dP = dO V^T) stay in registers and the only LDS operands
// are the streamed Q and dO rows: a third less LDS traffic per product than
// the two-waves-per-SIMD pass above, which reads K and V from LDS.  With one
// wave per SIMD nothing hides a stall but the wave's own instruction stream,
// so the step is written as a fixed program:
//  * V is held negated: the dP accumulator starts from D and ends as D - dP,
//    so dS = P (dP - D) = -(P * acc) is one multiply per element; dK is
//    accumulated with that sign and flipped together with the final scale.
//  * dV^T and dK^T accumulate in AGPRs (mfma_acc), the S and dP products in
//    VGPRs where the softmax gradient reads them.
//  * Q and dO tiles of BQ rows are double-buffered in LDS.  The copies
//    global -> LDS are issued as inline assembly, invisible to the compiler,
//    which would otherwise wait for them before the first transposed LDS read
//    of the step (it cannot tell that read from the copy's target); the step
//    waits for them once, at its end, before the barrier.  (The compiler uses
//    no M0 of its own in this kernel, so the copies may set it.)
//  * A step is BQ / 32 row blocks; each block is 16 S/dP products (A) and 16
//    dV/dK products (B), ordered A0 A1 B0 A2 B1 ... so that every block's
//    softmax gradient runs beside the products of the next group, one pair
//    of elements per two products; the LDS operand of each product is read
//    LEAD products ahead.  A scheduling barrier after every product keeps
//    this order.
//  * LDS addresses are one per-lane offset per operand shape plus an
//    immediate (tensor and row block); the stage is added once per step.
//  * Non-causal launches are persistent: one workgroup per compute unit walks
//    the key blocks, and each block's K and V rows reach LDS (where the waves
//    read their fragments) during the last step of the block before it,
//    together with its first Q/dO tile and that tile's statistics.
#ifndef FA_KV_ROWS
#define FA_KV_ROWS 64  // query rows per step (128 measured 2 % slower)
#endif
#ifndef FA_KV_LEAD
#define FA_KV_LEAD 3
#endif
template <int E, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kv_kernel(const void *__restrict__ Q, const void *__restrict__ K, const void *__restrict__ V,
                        const void *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Dvec,
                        void *__restrict__ dK, void *__restrict__ dV, int BH, int Nq, int Nk, float scale,
                        float scale_log2, int n_kt) {
    constexpr int D = 128, NW = 4, BQ = FA_KV_ROWS, BKC = 32 * NW;
    constexpr int NB = BQ / 32;       // 32-row blocks per step
    constexpr int NP = 32 * NB;       // matrix products per step
    constexpr int NKS = D / 16;       // k-steps over the head dim
    constexpr int NDB = D / 32;       // 32-row blocks of dK^T / dV^T
    constexpr int TILE = BQ * D * 2;  // bytes of one tile of BQ rows
    constexpr int NCP = BQ / 16;      // 1 KiB copies per wave per tensor per tile
    constexpr int ST = 4 * TILE;      // row statistics: stage s at ST + s * 8 BQ (LSE * log2 e, then D)
    constexpr int LEAD = FA_KV_LEAD, NSLOT = LEAD + 1;
    static_assert(E != ELT_F32, "16-bit operands are copied global -> LDS as they are");
    static_assert(BQ == 64 || BQ == 128, "two or four row blocks per step");
    static_assert(BQ * 2 == 64 * NW || BQ == 64 * NW / 4, "one statistics row of 64 per wave or half the waves");
    // stage s: Q at 2 s TILE, dO at (2 s + 1) TILE; statistics; then the K and V
    // rows of the workgroup's key block (KV, 2 x BKC rows of 256 bytes, tile_off
    // layout), copied global -> LDS while the item before it computes
    constexpr int KV = ST + 2 * 8 * BQ + 512, KVB = BKC * D * 2;
    __shared__ __attribute__((aligned(16))) unsigned char lds[KV + 2 * KVB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;

    // Work items are key blocks.  Causal: one per workgroup, the low key tiles
    // (which meet the most query rows) first.  Otherwise the workgroups are
    // persistent: workgroup w takes the blocks it * gridDim.x + xcd_remap(w), and
    // each item's K/V rows and first Q/dO tile are copied while the item before
    // it computes.
    const int n_items = BH * n_kt;
    auto item_of = [&](int it) -> int {
        if constexpr (CAUSAL) return it == 0 ? (int)blockIdx.x : -1;
        const int L = it * (int)gridDim.x + xcd_remap(blockIdx.x, gridDim.x);
        return L < n_items ? L : -1;
    };
    auto decode = [&](int L, int &bh_, int &kt_) __attribute__((always_inline)) {
        if constexpr (CAUSAL) {
            kt_ = L / BH;
            bh_ = L % BH;
        } else {
            bh_ = L / n_kt;
            kt_ = L % n_kt;
        }
    };
    const int n_qt = (Nq + BQ - 1) / BQ;
    // the current item (updated at the top of the item loop)
    int bh = 0, kt = 0, k0 = 0, kw = 0, kwg = 0, qt_begin = 0;
    int64_t k_head = 0;

    // Per-lane LDS byte offsets in a tile (tile_off<128> layout):
    //  a_off[ks]: the A operand (row l32, head dims 16ks + 8g .. +7);
    //  t_off[db][hf]: the transposed read of rows 4g + j/4 + 8 hf, columns
    //  32 db + 16 ((lane / 16) % 2) + 4 (j % 4), j = lane % 16.
    uint32_t a_off[NKS], t_off[NDB][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) a_off[ks] = 2u * (uint32_t)tile_off<D>(l32, 16 * ks + 8 * g);
    {
        const int j = lane & 15;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                t_off[db][hf] = 2u * (uint32_t)tile_off<D>(4 * g + (j >> 2) + 8 * hf, 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3));
    }
    const uint32_t st_off = (uint32_t)ST + 16u * (uint32_t)g;  // statistics of rows 4g + 8 rq + i

    // Copies of a tile: blocks of 4 rows (1 KiB), NCP per wave per tensor;
    // lane l fetches row 4b + l/16, 16-byte chunk (l % 16) ^ swz(row), which the
    // swizzle places at byte 16 l of the block.  Block b = wave + 4 jb, so the
    // swizzle of a lane's row is the same for every jb.
    auto q_base = [&](int bh_) { return static_cast<const uint16_t *>(Q) + (int64_t)bh_ * Nq * D; };
    auto do_base = [&](int bh_) { return static_cast<const uint16_t *>(dO) + (int64_t)bh_ * Nq * D; };
    const int cp_row = wave * 4 + lane / 16;  // + 16 jb
    const uint32_t cp_col = (uint32_t)((lane & 15) ^ swz<D>(cp_row)) * 16u;  // byte offset of the chunk in its row
    // Row statistics of a tile: wave w loads 64 rows of one of them (LSE for
    // w < NW / 2, D for the rest; at BQ = 64 waves 1 and 3 load rows nobody
    // uses), one value per lane.
    const int st_kind = wave / (NW / 2), st_part = wave % (NW / 2);
    auto st_base = [&](int bh_) { return (st_kind == 0 ? LSE : Dvec) + (int64_t)bh_ * Nq; };
    float sreg = 0.f;
    int st_row0 = 0;
    auto fetch_stats = [&](int qt, const float *src) __attribute__((always_inline)) {
        st_row0 = qt * BQ + 64 * st_part;
        sreg = src[min(st_row0 + lane, Nq - 1)];
    };
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 in the clobber list: see the kernel's notes
    // copy jb of this wave's share of the Q and dO rows of tile qt (of the head
    // at Qb, dOb), into stage s
    auto fetch_copy = [&](int qt, int s, int jb, const uint16_t *Qb, const uint16_t *dOb)
        __attribute__((always_inline)) {
        const int grow = min(qt * BQ + cp_row + 16 * jb, Nq - 1);  // rows past Nq re-read row Nq - 1 (zero weight)
        const uint32_t off = (uint32_t)grow * (uint32_t)(D * 2) + cp_col;  // bytes from the head's first row
        const uint32_t dq = (uint32_t)(2 * s * TILE + (wave + NW * jb) * 1024);
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(Qb), "s"(dq)
                     : "memory", "m0");
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(dOb),
                     "s"(dq + (uint32_t)TILE)
                     : "memory", "m0");
    };
    // the K and V rows of key block kt_ of head bh_ into the KV region: 32
    // blocks of 4 rows per tensor, 8 per wave; rows past Nk re-read row Nk - 1
    // (their results are never stored)
    auto fetch_kv = [&](int bh_, int kt_) __attribute__((always_inline)) {
        const uint16_t *Kb = static_cast<const uint16_t *>(K) + (int64_t)bh_ * Nk * D;
        const uint16_t *Vb = static_cast<const uint16_t *>(V) + (int64_t)bh_ * Nk * D;
#pragma unroll
        for (int jb = 0; jb < BKC / 16; ++jb) {
            const int grow = min(kt_ * BKC + cp_row + 16 * jb, Nk - 1);
            const uint32_t off = (uint32_t)grow * (uint32_t)(D * 2) + cp_col;
            const uint32_t dk = (uint32_t)(KV + (wave + NW * jb) * 1024);
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(Kb),
                         "s"(dk)
                         : "memory", "m0");
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(Vb),
                         "s"(dk + (uint32_t)KVB)
                         : "memory", "m0");
        }
    };
#pragma clang diagnostic pop
    // The statistics of the last fetch into stage s, once their loads landed
    // (a store in every wave: no branch sinks the loads to the end of the
    // step).  Rows past Nq get LSE = inf (P = 0) and D = 0.
    auto put_stats = [&](int s) __attribute__((always_inline)) {
        const bool real = st_row0 + lane < Nq;
        const float v = st_kind == 0 ? (real ? sreg * kLog2e : INFINITY) : (real ? sreg : 0.f);
        uint32_t at = (uint32_t)(ST + s * 8 * BQ + st_kind * 4 * BQ + 256 * st_part);
        if (256 * st_part >= 4 * BQ) at = (uint32_t)(ST + 2 * 8 * BQ + 256 * st_kind);  // unused rows (BQ = 64)
        *reinterpret_cast<float *>(lds + at + 4 * lane) = v;
    };

    f32x16_t dvT[NDB], dkT[NDB];
    u32x4_t kf[NKS], vn[NKS];  // K and -V fragments: lane = key, k = head-dim index 16*ks + 8*g + v

    // Position of group G (16 products) in the step's order A0 A1 B0 A2 B1 ... B(NB-1):
    // is it an A group, and of which block.
    auto grp_is_a = [](int G) constexpr { return G == 0 || (G != 2 * NB - 1 && G % 2 == 1); };
    auto grp_block = [](int G) constexpr { return G == 0 ? 0 : G == 2 * NB - 1 ? NB - 1 : G % 2 == 1 ? (G + 1) / 2 : (G - 2) / 2; };
    // first product of A(b); the softmax gradient of block b starts one product
    // into the group after A(b)
    auto a_start = [](int b) constexpr { return b == 0 ? 0 : 16 * (2 * b - 1); };
    auto v_start = [](int b) constexpr { return b == 0 ? 17 : 16 * 2 * b + 1; };

    // One query tile in stage s (its statistics at offset 8 BQ s); the next
    // tile's copies go into the other stage, which every wave finished reading
    // before this step's barrier.  MASK: apply the causal mask (the tile
    // reaches this workgroup's keys).
    auto step_pipe = [&](int qt, int s, int qn, const uint16_t *Qn, const uint16_t *dOn, auto mask_c)
        __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_c)::value;
        const uint32_t sb = (uint32_t)(2 * s * TILE), stb = (uint32_t)(s * 8 * BQ);
        uint32_t ao[NKS], to[NDB][2];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) ao[ks] = a_off[ks] + sb;
#pragma unroll
        for (int db = 0; db < NDB; ++db) { to[db][0] = t_off[db][0] + sb; to[db][1] = t_off[db][1] + sb; }
        const uint32_t so = st_off + stb;
        const int q0 = qt * BQ;
        u32x4_t opr[NSLOT];
        f32x16_t sc[NB], dp[NB];
        f32x4_t L4[NB][4];
        float pv[NB][16], tv[NB][16];
        uint32_t pp[NB][8], dd[NB][8];
        // operand of product i into its slot
        auto rd = [&](int i) __attribute__((always_inline)) {
            const int G = i / 16, j = i % 16, b = grp_block(G);
            if (grp_is_a(G)) {  // S / dP of block b: one 16-byte read
                const int ks = j / 2, w = j % 2;
                opr[i % NSLOT] = *reinterpret_cast<const u32x4_t *>(lds + ao[ks] + w * TILE + b * 32 * 256);
            } else {  // dV / dK of block b: two transposed reads
                const int h = j / 8, db = (j % 8) / 2, w = j % 2;
                const unsigned off = (w == 0 ? TILE : 0) + (b * 32 + 16 * h) * 256;
                const u32x2_t x0 = ds_read_tr16(reinterpret_cast<const uint16_t *>(lds + to[db][0] + off));
                const u32x2_t x1 = ds_read_tr16(reinterpret_cast<const uint16_t *>(lds + to[db][1] + off));
                opr[i % NSLOT] = u32x4_t{x0[0], x0[1], x1[0], x1[1]};
            }
        };
        auto mm = [&](int i) __attribute__((always_inline)) {
            const int G = i / 16, j = i % 16, b = grp_block(G);
            const u32x4_t a = opr[i % NSLOT];
            if (grp_is_a(G)) {
                const int ks = j / 2, w = j % 2;
                if (w == 0) sc[b] = mfma_in<E>(a, kf[ks], ks == 0 ? f32x16_t{} : sc[b]);
                else dp[b] = mfma_in<E>(a, vn[ks], dp[b]);
            } else {
                const int h = j / 8, db = (j % 8) / 2, w = j % 2;
                if (w == 0) mfma_acc<E>(dvT[db], a, u32x4_t{pp[b][4 * h], pp[b][4 * h + 1], pp[b][4 * h + 2], pp[b][4 * h + 3]});
                else mfma_acc<E>(dkT[db], a, u32x4_t{dd[b][4 * h], dd[b][4 * h + 1], dd[b][4 * h + 2], dd[b][4 * h + 3]});
            }
        };
        // D of block b's rows into its dP accumulator; LSE * log2 e of its rows
        auto rd_dinit = [&](int b, int rq) __attribute__((always_inline)) {
            const f32x4_t D4 = *reinterpret_cast<const f32x4_t *>(lds + so + 4 * BQ + 4 * (32 * b + 8 * rq));
#pragma unroll
            for (int k = 0; k < 4; ++k) dp[b][4 * rq + k] = D4[k];
        };
        auto rd_lse = [&](int b, int rq) __attribute__((always_inline)) {
            L4[b][rq] = *reinterpret_cast<const f32x4_t *>(lds + so + 4 * (32 * b + 8 * rq));
        };
        // elements e, e + 1 of block b's softmax gradient in two halves, each
        // pair of instructions independent (no wait after an exponential)
        auto pair_exp = [&](int b, int e) __attribute__((always_inline)) {
            const int rq = e / 4, k = e % 4;
            const float x0 = fmaf(sc[b][e], scale_log2, -L4[b][rq][k]);
            const float x1 = fmaf(sc[b][e + 1], scale_log2, -L4[b][rq][k + 1]);
            float p0 = __builtin_amdgcn_exp2f(x0), p1 = __builtin_amdgcn_exp2f(x1);
            if (MASK) {  // rows q0 + c + 4g and the next one against this lane's key
                const int c = 32 * b + 8 * rq + k;
                if (kwg > q0 + c) p0 = 0.f;
                if (kwg > q0 + c + 1) p1 = 0.f;
            }
            pv[b][e] = p0;
            pv[b][e + 1] = p1;
        };
        auto pair_grad = [&](int b, int e) __attribute__((always_inline)) {
            tv[b][e] = pv[b][e] * dp[b][e];
            tv[b][e + 1] = pv[b][e + 1] * dp[b][e + 1];
            pp[b][e / 2] = pack_in<E>(pv[b][e], pv[b][e + 1]);
            dd[b][e / 2] = pack_in<E>(tv[b][e], tv[b][e + 1]);
        };

#pragma unroll
        for (int rq = 0; rq < 4; ++rq) rd_dinit(0, rq);
        static_for<LEAD>([&](auto ic) __attribute__((always_inline)) { rd(decltype(ic)::value); });
        __builtin_amdgcn_sched_barrier(0);
        static_for<NP>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            mm(i);
            if constexpr (i + LEAD < NP) rd(i + LEAD);
            // the next tile's copies, during the first products
            if constexpr (i >= 1 && i <= NCP) fetch_copy(qn, s ^ 1, i - 1, Qn, dOn);
            static_for<NB>([&](auto bc) __attribute__((always_inline)) {
                constexpr int b = decltype(bc)::value;
                // block b's D, ten products ahead of its first dP product
                if constexpr (b > 0 && i >= a_start(b) - 10 && i < a_start(b) - 6) rd_dinit(b, i - (a_start(b) - 10));
                // each row group's statistics four products ahead of its elements
                constexpr int e0 = v_start(b);
                if constexpr (i >= e0 - 4 && i < e0 + 12 && (i - (e0 - 4)) % 4 == 0) rd_lse(b, (i - (e0 - 4)) / 4);
                if constexpr (i >= e0 && i < e0 + 16) {
                    if constexpr ((i - e0) % 2 == 0) pair_exp(b, i - e0);
                    else pair_grad(b, i - e0 - 1);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    int L = item_of(0);
    int base = 0;  // the stage of the current item's first tile
    if (L >= 0) {  // the first item's K/V rows, first tile and its statistics
        decode(L, bh, kt);
        const int qb0 = CAUSAL ? min(kt * BKC / BQ, n_qt) : 0;
        fetch_kv(bh, kt);
        if (qb0 < n_qt) {
            fetch_stats(qb0, st_base(bh));
#pragma unroll
            for (int jb = 0; jb < NCP; ++jb) fetch_copy(qb0, 0, jb, q_base(bh), do_base(bh));
            wait_vmem();
            put_stats(0);
        }
        wait_vmem();
        __syncthreads();
    }
    for (int it = 0; L >= 0; ++it) {
        const int Ln = item_of(it + 1);
        int bhn = 0, ktn = 0;
        decode(L, bh, kt);
        if (Ln >= 0) decode(Ln, bhn, ktn);
        k_head = (int64_t)bh * Nk * D;
        k0 = kt * BKC;
        kw = k0 + wave * 32 + l32;  // this lane's key
        kwg = kw - 4 * g;           // the key less the lane's 4g offset in the score registers' row order
        qt_begin = CAUSAL ? min(k0 / BQ, n_qt) : 0;  // earlier rows see none of these keys
        const uint16_t *Qh = q_base(bh), *dOh = do_base(bh);
        const float *sth = st_base(bh);
        // the next item's first tile (rows 0: it is non-causal)
        const uint16_t *Qx = Ln >= 0 ? q_base(bhn) : Qh, *dOx = Ln >= 0 ? do_base(bhn) : dOh;
        const float *stx = Ln >= 0 ? st_base(bhn) : sth;

        // K and -V fragments from the KV region (the swizzle depends on the
        // row's low four bits, so the wave's rows 32 wave + l32 sit at the A
        // operand offsets plus 8 KiB per wave); every wave holds them before
        // the region takes the next item's rows
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            kf[ks] = *reinterpret_cast<const u32x4_t *>(lds + KV + 8192 * wave + a_off[ks]);
            vn[ks] = *reinterpret_cast<const u32x4_t *>(lds + KV + KVB + 8192 * wave + a_off[ks]) ^ 0x80008000u;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();

#pragma unroll
        for (int db = 0; db < NDB; ++db) { dvT[db] = f32x16_t{}; dkT[db] = f32x16_t{}; }
        mfma_wait<3>();  // the zeroed accumulators, before mfma_acc reads them

        auto step = [&](int qt, auto mask_c) __attribute__((always_inline)) {
            const int s = (base + qt - qt_begin) & 1;
            const bool last = qt + 1 == n_qt;
            if (last && Ln >= 0) fetch_kv(bhn, ktn);  // the next item's rows, beside this last step
            // the next tile, or past the last one the next item's first tile (or,
            // with no next item, this tile again into the idle stage, so every
            // step issues the same copies and no branch splits the step)
            const int qn = last ? (Ln >= 0 ? 0 : qt) : qt + 1;
            fetch_stats(qn, last ? stx : sth);
            step_pipe(qt, s, qn, last ? Qx : Qh, last ? dOx : dOh, mask_c);
            // the next tile's copies and statistics have landed: publish them
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            put_stats(s ^ 1);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        // Causal: the first tiles reach this workgroup's keys and take the masked
        // program, in a loop of their own (one loop holding both programs needs
        // more registers than the file has); the rest need no mask.
        const int qt_mask_end = CAUSAL ? min(n_qt, (k0 + BKC + BQ - 1) / BQ) : qt_begin;
        for (int qt = qt_begin; qt < qt_mask_end; ++qt) step(qt, std::true_type{});
        for (int qt = qt_mask_end; qt < n_qt; ++qt) step(qt, std::false_type{});
        base = (base + n_qt - qt_begin) & 1;

        // the accumulators were last written by matrix products the compiler does
        // not see (mfma_acc): give them their result latency before any read
        mfma_drain();
        if (kw < Nk) {
            // dK = scale * dK^T (accumulated negated), dV = dV^T: lane = key,
            // register r -> head dim 32db + 8*(r/4) + 4*g + r%4
            const int64_t row = k_head + (int64_t)kw * D;
            const float nscale = -scale;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int col = db * 32 + 8 * rq + 4 * g;
                    store4<E>(dK, row + col, dkT[db][4 * rq] * nscale, dkT[db][4 * rq + 1] * nscale,
                              dkT[db][4 * rq + 2] * nscale, dkT[db][4 * rq + 3] * nscale);
                    store4<E>(dV, row + col, dvT[db][4 * rq], dvT[db][4 * rq + 1], dvT[db][4 * rq + 2],
                              dvT[db][4 * rq + 3]);
                }
        }
        L = Ln;
    }
}

// ---------------------------------------------------------------- 2. dQ
template <int D, int BC, int E, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(512) void bwd_dq_kernel(const void *__restrict__ Q, const void *__restrict__ K,
                                                     const void *__restrict__ V, const void *__restrict__ dO,
                                                     const float *__restrict__ LSE, const float *__restrict__ Dvec,
                                                     void *__restrict__ dQ, int BH, int Nq, int Nk, float scale,
                                                     float scale_log2, int n_qt, Dropout dr) {
    constexpr int NW = 8, NT = 512;
    constexpr int BR = 32 * NW;   // query rows per workgroup
    constexpr int NKB = BC / 32;  // 32-key blocks per tile
    constexpr int NCH = D / 8;
    constexpr int NKS = D / 16;
    constexpr int NDB = D / 32;
    constexpr bool DMA = E != ELT_F32;  // 16-bit K / V go global -> LDS directly
    constexpr int CH = BC * NCH;        // 16-byte chunks per K (and V) tile
    constexpr int CH_PER_T = DMA ? 1 : (CH + NT - 1) / NT;

    // One __shared__ object per buffer (see the dK/dV pass): the transposed reads of
    // K must be distinguishable from the copies filling the other buffers.
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[BC * D], Ks1[BC * D], Vs0[BC * D], Vs1[BC * D];
    auto kbuf = [&](int b) __attribute__((always_inline)) { return b ? Ks1 : Ks0; };
    auto vbuf = [&](int b) __attribute__((always_inline)) { return b ? Vs1 : Vs0; };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    int bh, qt;
    if constexpr (CAUSAL) {
        const int L = blockIdx.x;  // longest rows first
        qt = n_qt - 1 - L / BH;
        bh = L % BH;
    } else {
        const int L = xcd_remap(blockIdx.x, gridDim.x);
        bh = L / n_qt;
        qt = L % n_qt;
    }
    const int64_t q_head = (int64_t)bh * Nq * D;
    const int64_t k_head = (int64_t)bh * Nk * D;
    const int q_wave0 = qt * BR + wave * 32;
    const int q = q_wave0 + l32;  // this lane's query row
    const int q_ld = q < Nq ? q : Nq - 1;

    int k_end = Nk;
    if constexpr (CAUSAL) k_end = min(Nk, min(qt * BR + BR, Nq));
    const int n_kt = (k_end + BC - 1) / BC;

    // Q^T and dO^T fragments (B operands, k = head-dim index 16*ks + 8*g + v) and the
    // row statistics, loaded before any tile prefetch.
    u32x4_t qf[NKS], df[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        qf[ks] = load8_operand<E>(Q, q_head + (int64_t)q_ld * D + 16 * ks + 8 * g);
        df[ks] = load8_operand<E>(dO, q_head + (int64_t)q_ld * D + 16 * ks + 8 * g);
    }
    const float lse2 = LSE[(int64_t)bh * Nq + q_ld] * kLog2e;
    const float dv = Dvec[(int64_t)bh * Nq + q_ld];

    const void *Kh = static_cast<const char *>(K) + k_head * (E == ELT_F32 ? 4 : 2);
    const void *Vh = static_cast<const char *>(V) + k_head * (E == ELT_F32 ? 4 : 2);
    u32x4_t kreg[CH_PER_T], vreg[CH_PER_T];
    auto load_tile = [&](int k0, int buf) __attribute__((always_inline)) {
        if constexpr (DMA) {
            dma_tile<D, BC, NW>(Kh, k0, Nk, kbuf(buf), wave, lane);
            dma_tile<D, BC, NW>(Vh, k0, Nk, vbuf(buf), wave, lane);
        } else {
#pragma unroll
            for (int j = 0; j < CH_PER_T; ++j) {
                const int i = tid + j * NT;
                const int row = i / NCH, c = i % NCH;
                kreg[j] = u32x4_t{0u, 0u, 0u, 0u};
                vreg[j] = u32x4_t{0u, 0u, 0u, 0u};
                if (i < CH && k0 + row < Nk) {
                    kreg[j] = load8_operand<E>(K, k_head + (int64_t)(k0 + row) * D + c * 8);
                    vreg[j] = load8_operand<E>(V, k_head + (int64_t)(k0 + row) * D + c * 8);
                }
            }
        }
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
        if constexpr (!DMA) {
#pragma unroll
            for (int j = 0; j < CH_PER_T; ++j) {
                const int i = tid + j * NT;
                const int row = i / NCH, c = i % NCH;
                if (i < CH) {
                    *reinterpret_cast<u32x4_t *>(&kbuf(buf)[tile_off<D>(row, c * 8)]) = kreg[j];
                    *reinterpret_cast<u32x4_t *>(&vbuf(buf)[tile_off<D>(row, c * 8)]) = vreg[j];
                }
            }
        }
    };

    f32x16_t dqT[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dqT[db] = f32x16_t{};

    load_tile(0, 0);
    store_tile(0);
    wait_vmem();
    __syncthreads();

    auto step = [&](int kt, auto buf_c) __attribute__((always_inline)) {
        constexpr int buf = decltype(buf_c)::value;
        const int k0 = kt * BC;
        const bool more = kt + 1 < n_kt;
        if (more) load_tile(k0 + BC, buf ^ 1);

        if (!CAUSAL || k0 <= q_wave0 + 31) {
            const bool ragged = k0 + BC > Nk;
            const bool diag = CAUSAL && (k0 + BC - 1 > q_wave0);
            // One 32-key block at a time (S, dP and dS of 32 keys live at once,
            // which keeps the kernel within 256 VGPRs without spills).
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                // S^T = K Q^T and dP^T = V dO^T: lane = query, register r -> key k0 + 32kb + 8*(r/4) + 4*g + r%4
                f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int off = tile_off<D>(kb * 32 + l32, 16 * ks + 8 * g);
                    s = mfma_in<E>(*reinterpret_cast<const u32x4_t *>(&kbuf(buf)[off]), qf[ks], s);
                    dp = mfma_in<E>(*reinterpret_cast<const u32x4_t *>(&vbuf(buf)[off]), df[ks], dp);
                }
                // masked scores -> -inf (P = 0), in a branch of its own taken only on the
                // ragged or diagonal tile
                if (ragged || diag) {
                    keep_branch();
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + 8 * (r / 4) + 4 * g + (r % 4);
                        if (key >= Nk || (CAUSAL && key > q)) s[r] = -INFINITY;
                    }
                }
                uint32_t keep = 0xffffu;  // bit r: register r survives dropout
                if constexpr (DROP)
                    keep = dropout_keep_query_lane(dr, (uint32_t)bh, (uint32_t)q, (uint32_t)(k0 + 32 * kb + 4 * g), lane);
                uint32_t dd[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float t[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int r = 2 * i + e;
                        const float pv = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -lse2));
                        if constexpr (DROP)
                            t[e] = pv * (((keep >> r) & 1u ? dp[r] * dr.keep_scale : 0.f) - dv);
                        else
                            t[e] = pv * (dp[r] - dv);
                    }
                    dd[i] = pack_in<E>(t[0], t[1]);
                }
                // dQ^T += K^T dS^T; k-step kst covers keys k0 + 16kst .. k0 + 16kst + 15
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kst = 2 * kb + h;
                    const u32x4_t b = {dd[4 * h], dd[4 * h + 1], dd[4 * h + 2], dd[4 * h + 3]};
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        dqT[db] = mfma_in<E>(tr_operand<D>(kbuf(buf), 16 * kst, 32 * db, lane), b, dqT[db]);
                }
            }
        }
        if (more) store_tile(buf ^ 1);
        wait_vmem();
        __syncthreads();
    };
    for (int kt = 0; kt < n_kt; kt += 2) {
        step(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < n_kt) step(kt + 1, std::integral_constant<int, 1>{});
    }

    // ---- dQ = scale * (dQ^T)^T: lane = query, register r -> head dim 32db + 8*(r/4) + 4*g + r%4
    if (q < Nq) {
        const int64_t row = q_head + (int64_t)q * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq)
                store4<E>(dQ, row + db * 32 + 8 * rq + 4 * g, dqT[db][4 * rq] * scale, dqT[db][4 * rq + 1] * scale,
                          dqT[db][4 * rq + 2] * scale, dqT[db][4 * rq + 3] * scale);
    }
}

// ---------------------------------------------------------------- 2'. dQ with 64 query rows per wave
// The d = 128 16-bit pass without dropout.  Four waves, one per SIMD, each
// owning 64 query rows (two 32-row blocks) of the workgroup's 256: every K and
// V fragment read from LDS feeds the products of both blocks, which halves
// the LDS reads per product of the two-waves-per-SIMD pass above.  Q^T and
// dO^T fragments stay in registers, dQ^T accumulates in AGPRs (mfma_acc),
// S^T and dP^T land in VGPRs where the softmax gradient reads them.  K/V
// tiles of 64 keys are double-buffered in LDS, copied global -> LDS by inline
// assembly and waited for once per step, before the barrier (the compiler
// uses no M0 of its own here).  A step is two 32-key blocks, each 32 S/dP
// products (A) and 16 dQ products (B), ordered A0 A1 B0 B1: block 0's
// softmax gradient runs beside A1, block 1's beside B0 and the first half of
// B1 (B1's first eight products need only keys 0..15 of the block).
// Non-causal launches are persistent: one workgroup per compute unit walks the
// query tiles, and each tile's Q rows (read from LDS into AGPRs) and first K/V
// tile reach LDS while the tile before it computes.
template <int E, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kv_kernel(const void *__restrict__ Q, const void *__restrict__ K, const void *__restrict__ V,
                      const void *__restrict__ O, const void *__restrict__ dO, const float *__restrict__ LSE,
                      float *__restrict__ Dvec, void *__restrict__ dQ, int BH, int Nq, int Nk, float scale,
                      float scale_log2, int n_qt) {
    constexpr int D = 128, NW = 4, BR = 64 * NW, BC = 64;
    constexpr int NKS = D / 16;       // k-steps over the head dim
    constexpr int NDB = D / 32;       // 32-column blocks of dQ^T
    constexpr int TILE = BC * D * 2;  // bytes of one K (or V) tile
    constexpr int NCP = BC / 16;      // 1 KiB copies per wave per tensor per tile
    constexpr int NP = 96;            // matrix products per step
    constexpr int LEAD = FA_KV_LEAD, NSLOT = LEAD + 1;
    static_assert(E != ELT_F32, "16-bit operands are copied global -> LDS as they are");
    // stage s: K at 2 s TILE, V at (2 s + 1) TILE; the workgroup's Q tile (BR
    // rows, tile_off layout) at QS, copied while the item before it computes
    constexpr int QS = 4 * TILE;
    __shared__ __attribute__((aligned(16))) unsigned char lds[QS + BR * D * 2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;

    // Work items are query tiles.  Causal: one per workgroup, the longest rows
    // first.  Otherwise the workgroups are persistent: workgroup w takes the
    // tiles it * gridDim.x + xcd_remap(w), and each item's Q tile and first
    // K/V tile are copied while the item before it computes.
    const int n_items = BH * n_qt;
    auto item_of = [&](int it) -> int {
        if constexpr (CAUSAL) return it == 0 ? (int)blockIdx.x : -1;
        const int L = it * (int)gridDim.x + xcd_remap(blockIdx.x, gridDim.x);
        return L < n_items ? L : -1;
    };
    auto decode = [&](int L, int &bh_, int &qt_) __attribute__((always_inline)) {
        if constexpr (CAUSAL) {
            qt_ = n_qt - 1 - L / BH;
            bh_ = L % BH;
        } else {
            bh_ = L / n_qt;
            qt_ = L % n_qt;
        }
    };
    auto k_tiles = [&](int qt_) {  // key tiles of query tile qt_
        const int k_end = CAUSAL ? min(Nk, min(qt_ * BR + BR, Nq)) : Nk;
        return (k_end + BC - 1) / BC;
    };

    // Per-lane LDS byte offsets in a tile (tile_off<128> layout):
    //  a_off[ks]: the A operand (key row l32 of a 32-key block, head dims
    //  16ks + 8g .. +7); t_off[db][hf]: the transposed read of key rows
    //  4g + j/4 + 8 hf, head dims 32 db + 16 ((lane / 16) % 2) + 4 (j % 4).
    uint32_t a_off[NKS], t_off[NDB][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) a_off[ks] = 2u * (uint32_t)tile_off<D>(l32, 16 * ks + 8 * g);
    {
        const int j = lane & 15;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                t_off[db][hf] = 2u * (uint32_t)tile_off<D>(4 * g + (j >> 2) + 8 * hf, 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3));
    }

    // Copies global -> LDS in blocks of 4 rows (1 KiB), block b = wave + 4 jb
    // (the same swizzle for every jb).  A K/V tile: NCP blocks per wave per
    // tensor, key rows past Nk re-read row Nk - 1 (their scores are masked).
    // The Q tile: BR / 16 blocks per wave, rows past Nq re-read row Nq - 1
    // (never stored).
    const int cp_row = wave * 4 + lane / 16;  // + 16 jb
    const uint32_t cp_col = (uint32_t)((lane & 15) ^ swz<D>(cp_row)) * 16u;
    auto k_base = [&](int bh_) { return static_cast<const uint16_t *>(K) + (int64_t)bh_ * Nk * D; };
    auto v_base = [&](int bh_) { return static_cast<const uint16_t *>(V) + (int64_t)bh_ * Nk * D; };
    auto q_base = [&](int bh_) { return static_cast<const uint16_t *>(Q) + (int64_t)bh_ * Nq * D; };
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 in the clobber list: see the kernel's notes
    auto fetch_copy = [&](int kt, int s, int jb, const uint16_t *Kb, const uint16_t *Vb) __attribute__((always_inline)) {
        const int grow = min(kt * BC + cp_row + 16 * jb, Nk - 1);
        const uint32_t off = (uint32_t)grow * (uint32_t)(D * 2) + cp_col;  // bytes from the head's first row
        const uint32_t dk = (uint32_t)(2 * s * TILE + (wave + NW * jb) * 1024);
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(Kb), "s"(dk)
                     : "memory", "m0");
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(Vb),
                     "s"(dk + (uint32_t)TILE)
                     : "memory", "m0");
    };
    auto copy_q = [&](int q0, const uint16_t *Qb) __attribute__((always_inline)) {
#pragma unroll
        for (int jb = 0; jb < BR / 16; ++jb) {
            const int grow = min(q0 + cp_row + 16 * jb, Nq - 1);
            const uint32_t off = (uint32_t)grow * (uint32_t)(D * 2) + cp_col;
            const uint32_t dq = (uint32_t)(QS + (wave + NW * jb) * 1024);
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(Qb), "s"(dq)
                         : "memory", "m0");
        }
    };
#pragma clang diagnostic pop

    // the current item (updated at the top of the item loop)
    int bh = 0, qt = 0, q_w0 = 0, n_kt = 0;
    int64_t q_head = 0;
    u32x4_t qf[2][NKS], df[2][NKS];
    float lse2[2], dv[2];
    int klim[2];
    f32x16_t dqT[2][NDB];
    int base = 0;  // the stage of the current item's first key tile
    int L = item_of(0);
    if (L >= 0) {  // the first item's Q tile and first K/V tile
        int bh0, qt0;
        decode(L, bh0, qt0);
        copy_q(qt0 * BR, q_base(bh0));
        if (k_tiles(qt0) > 0) {
#pragma unroll
            for (int jb = 0; jb < NCP; ++jb) fetch_copy(0, 0, jb, k_base(bh0), v_base(bh0));
        }
        wait_vmem();
        __syncthreads();
    }
    for (int it = 0; L >= 0; ++it) {
    const int Ln = item_of(it + 1);
    int bhn = 0, qtn = 0;
    decode(L, bh, qt);
    if (Ln >= 0) decode(Ln, bhn, qtn);
    q_head = (int64_t)bh * Nq * D;
    q_w0 = qt * BR + 64 * wave;  // first row of this wave
    n_kt = k_tiles(qt);
    const uint16_t *Kh = k_base(bh), *Vh = v_base(bh);
    // the next item's first tile (non-causal: every item has n_kt >= 1, and its
    // last step copies it)
    const uint16_t *Kx = Ln >= 0 ? k_base(bhn) : Kh, *Vx = Ln >= 0 ? v_base(bhn) : Vh;

    // Q^T fragments (B operands, k = head-dim index 16*ks + 8*g + v, lane = row
    // q_w0 + 32 r + l32) from the Q tile into AGPRs: the swizzle depends on the
    // row's low four bits, so they sit at the A operand offsets plus 256 bytes
    // per row of 64 wave + 32 r (the per-wave part opaque per item, so the sums
    // are formed here).
    {
        uint32_t qb = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char *)lds) +
                      (uint32_t)(QS + 64 * 256 * wave);
        asm volatile("" : "+s"(qb));
        uint32_t qa[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qa[ks] = qb + a_off[ks];
        lds_read_agpr(qf, qa);
    }
    // dO^T fragments of both row blocks and the rows' statistics.  This pass
    // runs first and forms D = rowsum(dO * O) itself ([RA] section 04's D
    // term): each lane adds its 64 head dims of the row in fp32, the permlane32
    // swap adds the two halves (the same sum in both lanes), and the g = 0
    // lanes store it for the dK/dV pass that follows.
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int q = q_w0 + 32 * r + l32;
        const int q_ld = q < Nq ? q : Nq - 1;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) df[r][ks] = load8_operand<E>(dO, q_head + (int64_t)q_ld * D + 16 * ks + 8 * g);
        lse2[r] = LSE[(int64_t)bh * Nq + q_ld] * kLog2e;
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            float o8[8];
            load8_float<E>(O, q_head + (int64_t)q_ld * D + 16 * ks + 8 * g, o8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = df[r][ks][i];
                acc = fmaf(o8[2 * i], E == ELT_BF16 ? bf16_lo(w) : f16_lo(w), acc);
                acc = fmaf(o8[2 * i + 1], E == ELT_BF16 ? bf16_hi(w) : f16_hi(w), acc);
            }
        }
        dv[r] = half_sum(acc);
        if (g == 0 && q < Nq) Dvec[(int64_t)bh * Nq + q] = dv[r];
    }
    // last key each lane's rows see (past Nk, or causal past the row), less
    // the lane's 4g offset in the score registers' key order
#pragma unroll
    for (int r = 0; r < 2; ++r) klim[r] = (CAUSAL ? min(q_w0 + 32 * r + l32, Nk - 1) : Nk - 1) - 4 * g;
    // every wave holds its Q^T: the tile's space takes the next item's
    __syncthreads();
    if (Ln >= 0) copy_q(qtn * BR, q_base(bhn));

#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int db = 0; db < NDB; ++db) dqT[r][db] = f32x16_t{};
    mfma_wait<3>();  // the zeroed accumulators, before mfma_acc reads them

    // One key tile in stage s: products 0..31 A(block 0), 32..63 A(block 1),
    // 64..79 B(block 0), 80..95 B(block 1).  A product i < 64: k-step ks =
    // (i % 32) / 4, tensor w = (i % 4) / 2 (K: S^T, V: dP^T), row block i % 2.
    // B product j = (i - 64) % 16: k-step h = j / 8, db = (j % 8) / 2, row block j % 2.
    // MASK: apply the mask of keys past Nk and, causal, of keys after the row.
    auto step_pipe = [&](int kt, int s, int kn, const uint16_t *Kn, const uint16_t *Vn, auto mask_c)
        __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_c)::value;
        const uint32_t sb = (uint32_t)(2 * s * TILE);
        uint32_t ao[NKS], to[NDB][2];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) ao[ks] = a_off[ks] + sb;
#pragma unroll
        for (int db = 0; db < NDB; ++db) { to[db][0] = t_off[db][0] + sb; to[db][1] = t_off[db][1] + sb; }
        const int k0 = kt * BC;
        u32x4_t opr[NSLOT];
        f32x16_t sc[2][2], dp[2][2];  // [key block][row block]
        float pv[2][2][16];
        uint32_t dd[2][2][8];
        // Product i is issued in slot n; its operand goes through ring entry
        // (n / 2) % NSLOT.  An A product's operand is shared by the two row
        // blocks (products i, i + 1, i even): read once.
        auto rd = [&](int n, int i) __attribute__((always_inline)) {
            if (i < 64) {
                if (i % 2 == 0) {
                    const int kb = i / 32, ks = (i % 32) / 4, w = (i % 4) / 2;
                    opr[(n / 2) % NSLOT] = *reinterpret_cast<const u32x4_t *>(lds + ao[ks] + w * TILE + kb * 32 * 256);
                }
            } else {
                const int kb = (i - 64) / 16, j = (i - 64) % 16, h = j / 8, db = (j % 8) / 2;
                if (j % 2 == 0) {
                    const unsigned off = (kb * 32 + 16 * h) * 256;
                    const u32x2_t x0 = ds_read_tr16(reinterpret_cast<const uint16_t *>(lds + to[db][0] + off));
                    const u32x2_t x1 = ds_read_tr16(reinterpret_cast<const uint16_t *>(lds + to[db][1] + off));
                    opr[(n / 2) % NSLOT] = u32x4_t{x0[0], x0[1], x1[0], x1[1]};
                }
            }
        };
        auto mm = [&](int n, int i) __attribute__((always_inline)) {
            const u32x4_t a = opr[(n / 2) % NSLOT];
            if (i < 64) {
                const int kb = i / 32, ks = (i % 32) / 4, w = (i % 4) / 2, r = i % 2;
                if (w == 0) {  // S^T: Q^T from AGPRs
                    if (ks == 0) sc[kb][r] = mfma_bagpr_first<E>(a, qf[r][ks]);
                    else mfma_bagpr<E>(sc[kb][r], a, qf[r][ks]);
                } else {  // dP^T: dO^T from VGPRs
                    dp[kb][r] = mfma_in<E>(a, df[r][ks], ks == 0 ? f32x16_t{} : dp[kb][r]);
                }
            } else {
                const int kb = (i - 64) / 16, j = (i - 64) % 16, h = j / 8, db = (j % 8) / 2, r = j % 2;
                mfma_acc<E>(dqT[r][db], a, u32x4_t{dd[kb][r][4 * h], dd[kb][r][4 * h + 1], dd[kb][r][4 * h + 2], dd[kb][r][4 * h + 3]});
            }
        };
        // elements e, e + 1 (register pair) of key block kb, row block r:
        // P = exp2(s c - LSE log2 e), dS = P (dP - D), in two halves
        auto pair_exp = [&](int kb, int r, int e) __attribute__((always_inline)) {
            float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][r][e], scale_log2, -lse2[r]));
            float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][r][e + 1], scale_log2, -lse2[r]));
            if (MASK) {  // keys k0 + c + 4g and the next one against the row's last key
                const int c = 32 * kb + 8 * (e / 4) + (e % 4);
                if (k0 + c > klim[r]) p0 = 0.f;
                if (k0 + c + 1 > klim[r]) p1 = 0.f;
            }
            pv[kb][r][e] = p0;
            pv[kb][r][e + 1] = p1;
        };
        auto pair_grad = [&](int kb, int r, int e) __attribute__((always_inline)) {
            const float t0 = pv[kb][r][e] * (dp[kb][r][e] - dv[r]);
            const float t1 = pv[kb][r][e + 1] * (dp[kb][r][e + 1] - dv[r]);
            dd[kb][r][e / 2] = pack_in<E>(t0, t1);
        };
        // the 16 pairs of a key block (8 per row block), in the order the B
        // products need them: keys 0..15 of both row blocks first
        auto vwork = [&](int kb, int u) __attribute__((always_inline)) {  // u = 0..31
            const int pr = u / 2, half = u % 2;             // pair pr = 0..15
            const int h = pr / 8, r = (pr / 4) % 2, e = 8 * h + 2 * (pr % 4);
            if (half == 0) pair_exp(kb, r, e);
            else pair_grad(kb, r, e);
        };

        // Slot n issues product perm(n).  The masked program (the ragged or
        // diagonal tile, one per row tile at most) runs A0 B0 A1 B1 with each
        // softmax gradient between its A and B groups: fewer values live at
        // once than with the overlap, which the extra mask arithmetic needs.
        auto perm = [](int n) constexpr {
            if (!MASK) return n;
            return n < 32 ? n : n < 48 ? n + 32 : n < 80 ? n - 16 : n;
        };
        static_for<LEAD>([&](auto ic) __attribute__((always_inline)) {
            constexpr int n = 2 * decltype(ic)::value;
            rd(n, perm(n));
            rd(n + 1, perm(n + 1));
        });
        __builtin_amdgcn_sched_barrier(0);
        static_for<NP>([&](auto nc) __attribute__((always_inline)) {
            constexpr int n = decltype(nc)::value;
            if constexpr (MASK && (n == 32 || n == 80)) {
                // the whole softmax gradient of the key block whose S/dP products
                // just finished, after their result latency (mfma_bagpr)
                mfma_drain();
                static_for<32>([&](auto uc) __attribute__((always_inline)) { vwork(n == 32 ? 0 : 1, decltype(uc)::value); });
                __builtin_amdgcn_sched_barrier(0);
            }
            mm(n, perm(n));
            if constexpr (n % 2 == 1 && (n + 1) / 2 + LEAD - 1 < NP / 2) {
                constexpr int m = n + 1 + 2 * (LEAD - 1);  // the pair LEAD pairs ahead
                rd(m, perm(m));
                rd(m + 1, perm(m + 1));
            }
            if constexpr (n >= 1 && n <= NCP) fetch_copy(kn, s ^ 1, n - 1, Kn, Vn);
            if constexpr (!MASK) {
                // block 0's softmax beside A(block 1) (32 units in 32 slots);
                // block 1's beside B(block 0) and the first half of B(block 1):
                // 32 units in 24 slots, two per slot in the first eight
                // (the first reads of a key block's scores wait for the result
                // latency of its last S^T products, which the compiler does not see)
                if constexpr (n == 33 || n == 65) mfma_wait<7>();
                if constexpr (n >= 33 && n < 65) vwork(0, n - 33);
                if constexpr (n >= 65 && n < 73) {
                    vwork(1, 2 * (n - 65));
                    vwork(1, 2 * (n - 65) + 1);
                }
                if constexpr (n >= 73 && n < 89) vwork(1, n - 73 + 16);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    auto step = [&](int kt, auto mask_c) __attribute__((always_inline)) {
        const bool last = kt + 1 == n_kt;
        // the next tile, or past the last one the next item's first tile (with
        // no next item, this tile again into the idle stage)
        const int kn = last ? (Ln >= 0 ? 0 : kt) : kt + 1;
        step_pipe(kt, (base + kt) & 1, kn, last ? Kx : Kh, last ? Vx : Vh, mask_c);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // Tiles that need no mask come first: every key exists and, causal, every
    // key precedes the workgroup's first row.  The rest take the masked program
    // in a loop of their own (one loop holding both programs needs more
    // registers than the file has).
    int n_full = Nk / BC;
    if constexpr (CAUSAL) n_full = min(n_full, (qt * BR + 1) / BC);
    n_full = min(n_full, n_kt);
    for (int kt = 0; kt < n_full; ++kt) step(kt, std::false_type{});
    for (int kt = n_full; kt < n_kt; ++kt) step(kt, std::true_type{});
    base = (base + n_kt) & 1;
    if (n_kt == 0 && Ln >= 0) {  // no step to copy the next item's first tile
#pragma unroll
        for (int jb = 0; jb < NCP; ++jb) fetch_copy(0, base, jb, Kx, Vx);
        wait_vmem();
        __syncthreads();
    }

    mfma_drain();  // mfma_acc results, before they are read
    // dQ = scale * (dQ^T)^T: lane = row, register r -> head dim 32db + 8*(r/4) + 4*g + r%4
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int q = q_w0 + 32 * r + l32;
        if (q < Nq) {
            const int64_t row = q_head + (int64_t)q * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq)
                    store4<E>(dQ, row + db * 32 + 8 * rq + 4 * g, dqT[r][db][4 * rq] * scale,
                              dqT[r][db][4 * rq + 1] * scale, dqT[r][db][4 * rq + 2] * scale,
                              dqT[r][db][4 * rq + 3] * scale);
        }
    }
    L = Ln;
    }
}

// Keys per tile of the dQ pass: at d = 64 a tile carries half the matrix work
// of d = 128, so it takes twice the keys (the 32-key blocks inside keep the
// registers the same).
template <int D, int E>
constexpr int dq_keys() { return E == ELT_F32 ? 32 : D == 64 ? 128 : 64; }
template <int D, int E, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs &a, int stage) {
    hipStream_t st = (hipStream_t)a.stream;
    const int BH = a.B * a.H;
    const int64_t rows = (int64_t)BH * a.Nq;
    const float sl2 = a.scale * kLog2e;
    const bool drop = a.drop.t > 0;
    // d = 128 on 16-bit data without dropout: the dQ pass runs first and forms
    // D itself (stage 0), then the dK/dV pass (stage 1); stage 2 launches nothing
    const bool dq_first = D == 128 && E != ELT_F32 && FA_DQ_KV && !drop;
    if (dq_first) {
        if (stage < 0 || stage == 0) {
            const int n_qt = (a.Nq + 255) / 256;
            if constexpr (D == 128 && E != ELT_F32)
                // causal: one query tile per workgroup; otherwise one persistent
                // workgroup per compute unit walks the tiles
                hipLaunchKernelGGL((bwd_dq_kv_kernel<E, CAUSAL>),
                                   dim3(CAUSAL ? BH * n_qt : std::min(BH * n_qt, compute_units())), dim3(256), 0, st,
                                   a.Q, a.K, a.V, a.O, a.dO, a.LSE, a.Dvec, a.dQ, BH, a.Nq, a.Nk, a.scale, sl2, n_qt);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    } else if (stage < 0 || stage == 0) {
        constexpr int RPB = 256 / (D / 8);
        hipLaunchKernelGGL((bwd_pre_kernel<D, E>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, a.O,
                           a.dO, a.Dvec, rows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stage < 0 || stage == 1) {
        const int n_kt = (a.Nk + 127) / 128;
        if constexpr (D == 128 && E != ELT_F32 && FA_DKDV_KV) {
            if (!drop) {
                // causal: one key block per workgroup; otherwise one persistent
                // workgroup per compute unit walks the blocks
                const int items = BH * n_kt;
                const int grid = CAUSAL ? items : std::min(items, compute_units());
                hipLaunchKernelGGL((bwd_dkdv_kv_kernel<E, CAUSAL>), dim3(grid), dim3(256), 0, st, a.Q, a.K, a.V,
                                   a.dO, a.LSE, a.Dvec, a.dK, a.dV, BH, a.Nq, a.Nk, a.scale, sl2, n_kt);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
                goto dq;
            }
        }
        if (drop)
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, E, CAUSAL, true>), dim3(BH * n_kt), dim3(512), 0, st, a.Q, a.K, a.V,
                               a.dO, a.LSE, a.Dvec, a.dK, a.dV, BH, a.Nq, a.Nk, a.scale, sl2, n_kt, a.drop);
        else
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, E, CAUSAL, false>), dim3(BH * n_kt), dim3(512), 0, st, a.Q, a.K, a.V,
                               a.dO, a.LSE, a.Dvec, a.dK, a.dV, BH, a.Nq, a.Nk, a.scale, sl2, n_kt, Dropout{});
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
dq:
    if ((stage < 0 || stage == 2) && !dq_first) {
        const int n_qt = (a.Nq + 255) / 256;
        constexpr int BC = dq_keys<D, E>();
        if (drop)
            hipLaunchKernelGGL((bwd_dq_kernel<D, BC, E, CAUSAL, true>), dim3(BH * n_qt), dim3(512), 0, st, a.Q, a.K, a.V,
                               a.dO, a.LSE, a.Dvec, a.dQ, BH, a.Nq, a.Nk, a.scale, sl2, n_qt, a.drop);
        else
            hipLaunchKernelGGL((bwd_dq_kernel<D, BC, E, CAUSAL, false>), dim3(BH * n_qt), dim3(512), 0, st, a.Q, a.K, a.V,
                               a.dO, a.LSE, a.Dvec, a.dQ, BH, a.Nq, a.Nk, a.scale, sl2, n_qt, Dropout{});
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D, int E>
static hipError_t launch_bwd_c(const BwdArgs &a, int stage) {
    return a.causal ? launch_bwd_t<D, E, true>(a, stage) : launch_bwd_t<D, E, false>(a, stage);
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs &a, int stage) {
    switch (a.dtype) {
        case ELT_BF16: return launch_bwd_c<D, ELT_BF16>(a, stage);
        case ELT_F16: return launch_bwd_c<D, ELT_F16>(a, stage);
        default: return launch_bwd_c<D, ELT_F32>(a, stage);
    }
}

hipError_t launch_bwd(const BwdArgs &a, int stage) {
    return a.d == 64 ? launch_bwd_d<64>(a, stage) : launch_bwd_d<128>(a, stage);
}

const char *describe_bwd() {
    return "bwd_pre_kernel (D=rowsum(dO*O)) -> bwd_dkdv_kernel<D, 8 waves = 4 key groups x 2 query halves, "
           "128 keys, 64-row query steps (128 at d=64), double-buffered Q/dO, transposed LDS reads> -> "
           "bwd_dq_kernel<D, 8 waves x 32 rows, 64-key tiles (128 at d=64)>; d=128 16-bit without dropout: "
           "bwd_dq_kv_kernel<4 waves, one per SIMD, persistent (non-causal), 64 rows each, Q^T and dQ "
           "accumulators in AGPRs, 64-key tiles "
           "as a fixed program, forms D itself> -> bwd_dkdv_kv_kernel<4 waves, one per SIMD, persistent (non-causal), "
           "32 keys each with K/V "
           "fragments in registers, dV/dK accumulators in AGPRs, 64-row steps as a fixed product/softmax program>; "
           "no atomics";
}

}  // namespace fa
