// fa_fwd.hip -- attention forward for gfx950.
//
// Method: page 1 "Flash Attention 原理与实现", section "Forward 的 Tiling
// 策略" (Q in row blocks, K/V streamed in key blocks, per-row running
// statistics) with the single-exponential state update of lumenova.space
// "research-attention", section 02 (m' = max(m, max s), alpha = exp(m - m'),
// p = exp(s - m'), l' = alpha l + sum p, u' = alpha u + sum p v, one division
// at the end) and LSE = m + ln l saved for the backward (same page, section 04).
//
// MI355X mapping (one workgroup = NW waves = 32*NW query rows of one head,
// two waves per SIMD):
//  * Each wave keeps its 32 query rows in VGPRs for the whole key loop.
//  * K and V tiles of BC keys are double-buffered in LDS, shared by all
//    waves; the next tile is fetched while the current one is in use.  K
//    stays row-major (XOR-swizzled 16-byte chunks) and is copied global ->
//    LDS directly; V is converted to fp16 and written transposed, so the
//    P*V product reads each operand with one 16-byte LDS read.
//  * Scores are formed transposed, S^T = K Q^T, so each lane owns one query
//    row: the row max and row sum are in-lane reductions plus one
//    permlane32 swap, and the rescale of the accumulator is one multiply per
//    register with a lane-uniform factor.
//  * O^T += V^T P^T runs on the fp16 matrix core: P is rounded to fp16
//    (11-bit significand) rather than bf16, which keeps the output within a
//    1e-3 relative-L2 budget; V converts from bf16 to fp16 exactly.
//  * Softmax runs in base 2 with the scale folded into one FMA:
//    p = exp2(s * scale*log2e - m2), m2 the running max in log2 units.
//
// Split-KV (SPLIT = true): the keys are cut into ranges of whole tiles, one
// workgroup per (query tile, range), and each writes its unnormalised state
// (u, m, l) for its rows instead of O and LSE; fwd_merge_kernel then combines
// the ranges with the same merge rule the key loop applies tile by tile
// (lumenova.space "research-attention", section 02): m* = max m_g,
// l = sum 2^(m_g - m*) l_g, O = sum 2^(m_g - m*) u_g / l.  This gives shapes
// with few query tiles (one head, or a short query block against a long key
// sequence) enough workgroups for 256 CUs.
//
// Dropout (DROP = true): the row sum l takes the undropped P (the softmax is
// not changed), the P V product takes P with the dropped elements zeroed,
// and the epilogue multiplies by 1 / (1 - rate) together with 1 / l.  The
// four lanes of a quad (four consecutive query rows) share the generator calls
// of each 32-key block (fa_common.hpp, dropout_keep_query_lane).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

// V^T tile in LDS: [D][BC] fp16.  Each row holds, per 16-key group kst, two
// 16-byte chunks: chunk 2*kst + g carries keys 16kst + 4g + 0..3 and
// 16kst + 8 + 4g + 0..3, exactly the eight k-slots lane group g feeds to the
// PV matrix product, so one ds_read_b128 fetches a whole operand.
//
// Placement (64 banks of 4 bytes): row `col` is stored at vt_row(col) with its
// chunks XORed by vt_xor(col), chosen so that both access shapes are free of
// bank conflicts:
//  * operand reads: 16 lanes read 16 consecutive rows at one chunk;
//  * the transposed stores (vblock below): 32 lanes write 8 bytes each into
//    16 rows four apart, at two chunk halves.
// With 64 keys a row is 128 bytes (half the banks): (row parity, chunk) must
// be a bijection both on col bits 0..3 (reads) and on bits 2..5 (stores);
// parity = bit 0 ^ bit 4, chunk xor = bits 1..3 ^ bit 5 does both.  With 128
// keys a row spans all banks and the chunk alone must be distinct.
template <int BC>
__device__ __forceinline__ int vt_row(int col) {
    if constexpr (BC == 64) return col ^ ((col >> 4) & 1);
    return col;
}
template <int BC>
__device__ __forceinline__ int vt_xor(int col) {
    if constexpr (BC == 64) return ((col >> 1) & 7) ^ ((col >> 5) & 1);
    return (col + col / (BC / 8)) % (BC / 8);
}

// Thread -> (key quad u, column quad c4) of the V staging: each 32-lane half
// of a wave covers 16 consecutive column quads of two key quads two apart (the
// two chunk halves), which the V^T layout above stores without bank
// conflicts; each 16-lane group still reads a contiguous row segment.
template <int D, int BC>
__device__ __forceinline__ void vblock(int tid, int &c4, int &u) {
    static_assert((BC / 4) * (D / 4) == 512 && (D == 128 || D == 64), "one V block per thread of 8 waves");
    const int w = tid >> 6, l = tid & 63;
    const int c4lo = l & 15, h = (l >> 4) & 1, hi = l >> 5;
    if constexpr (D == 128) {
        c4 = c4lo + 16 * hi;
        u = 4 * (w >> 1) + 2 * h + (w & 1);
    } else {
        c4 = c4lo;
        u = 4 * w + 2 * h + hi;
    }
}

// V^T tiles prepared once per call for fa_fwd_ws: tile (bh, kt) of BC keys is
// written to Vpk exactly as the key loop keeps it in LDS (fp16, [D][BC],
// vt_row / vt_xor placement, zero past Nk), so the loop copies it global ->
// LDS with no conversion or transposition of its own.  One workgroup per
// tile: the same per-thread 4-key x 4-column blocks as the in-loop staging,
// written transposed into LDS, then copied out 16 bytes per lane.
template <int D, int BC, int E>
__global__ __launch_bounds__(512) void v_pack_kernel(const void *__restrict__ V, uint16_t *__restrict__ Vpk, int Nk,
                                                     int n_kt) {
    static_assert((BC / 4) * (D / 4) == 512 && D * BC * 2 == 16 * 1024, "one block per thread, 16 KiB tiles");
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * BC];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / n_kt, k0 = (blockIdx.x % n_kt) * BC;
    const int64_t k_head = (int64_t)bh * Nk * D;
    int c4, u;  // keys k0 + 4u .. +3, columns 4c4 .. 4c4+3
    vblock<D, BC>(tid, c4, u);
    float v[4][4];  // [key][column], in the operand precision
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int key = k0 + 4 * u + k;
        if constexpr (E == ELT_F32) {
            f32x4_t x = {0.f, 0.f, 0.f, 0.f};
            if (key < Nk) x = *reinterpret_cast<const f32x4_t *>(static_cast<const float *>(V) + k_head + (int64_t)key * D + 4 * c4);
            const uint32_t w0 = pack_bf16(x[0], x[1]), w1 = pack_bf16(x[2], x[3]);  // fp32 operands are bf16
            v[k][0] = bf16_lo(w0); v[k][1] = bf16_hi(w0); v[k][2] = bf16_lo(w1); v[k][3] = bf16_hi(w1);
        } else {
            u32x2_t w = {0u, 0u};
            if (key < Nk) w = *reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(V) + k_head + (int64_t)key * D + 4 * c4);
            if constexpr (E == ELT_BF16) {
                v[k][0] = bf16_lo(w[0]); v[k][1] = bf16_hi(w[0]); v[k][2] = bf16_lo(w[1]); v[k][3] = bf16_hi(w[1]);
            } else {
                v[k][0] = f16_lo(w[0]); v[k][1] = f16_hi(w[0]); v[k][2] = f16_lo(w[1]); v[k][3] = f16_hi(w[1]);
            }
        }
    }
    const int kst = u / 4, qd = u % 4;
    const int chunk = 2 * kst + (qd & 1), half = qd >> 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int col = 4 * c4 + e;
        *reinterpret_cast<u32x2_t *>(&Vt[vt_row<BC>(col) * BC + ((chunk ^ vt_xor<BC>(col)) * 8) + half * 4]) =
            u32x2_t{pack_f16(v[0][e], v[1][e]), pack_f16(v[2][e], v[3][e])};
    }
    __syncthreads();
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(Vpk + (int64_t)blockIdx.x * (D * BC));
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(Vt);
    dst[tid] = src[tid];
    dst[tid + 512] = src[tid + 512];
}

// Rescale threshold (log2 units): the running maximum used for the
// exponentials is only moved when a new score exceeds it by more than this,
// so p = exp2(s*c - m_used) stays below 2^8 (far inside fp16 range) and the
// accumulator is rescaled only on the rare tiles that raise the maximum.
// O = u / l and LSE = m_used + log2 l hold for any m_used, so this changes no
// result beyond rounding.
constexpr float kRescaleThreshold = 8.f;

// Starting value of the running maximum: finite, so that a row whose keys in
// a range are all masked (possible under split-KV with the causal mask)
// gives p = exp2(-inf - m) = 0 rather than exp2(-inf + inf) = NaN, and so
// that the first real score always moves it (the accumulator is then
// multiplied by exp2(-huge) = 0, which it already is).
constexpr float kMaxInit = -3.402823466e38f;

// Partial-state outputs of a split-KV launch: R = B*H*Nq rows, G ranges.
struct SplitOut {
    float *U;  // [G][R][D] unnormalised accumulator u
    float *M;  // [G][R] running maximum, log2 units
    float *L;  // [G][R] row sum l
    int keys_per_split;  // a multiple of the key tile
};

template <int D, int BC, int NW, int E, bool CAUSAL, bool SPLIT, bool DROP, bool PREV = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_kernel(const void *__restrict__ Q, const void *__restrict__ K,
                                                      const void *__restrict__ V, void *__restrict__ O,
                                                      float *__restrict__ LSE, int BH, int Nq, int Nk,
                                                      float scale_log2, int n_qt, SplitOut part, Dropout dr,
                                                      const uint16_t *__restrict__ Vpk) {
    static_assert(!(SPLIT && DROP), "split-KV has no dropout variant");
    static_assert(!PREV || (!SPLIT && !DROP), "packed V^T tiles serve the plain forward");
    constexpr int BR = 32 * NW;    // query rows per workgroup
    constexpr int NT = NW * 64;    // threads
    constexpr int NCH = D / 8;     // 16-byte chunks per K row
    constexpr int NKB = BC / 32;   // 32-key blocks per tile
    constexpr int NDB = D / 32;    // 32-column blocks of O
    constexpr int NKS = D / 16;    // k-steps of the QK^T product
    constexpr bool DMA = E != ELT_F32;  // 16-bit K goes global -> LDS directly
    // K register staging (fp32 inputs only): 16-byte chunks per thread
    constexpr int KCH_PER_T = (BC * NCH + NT - 1) / NT;
    // V staging: blocks of 4 keys x 4 columns per thread
    constexpr int VBLK = (BC / 4) * (D / 4);
    constexpr int VBLK_PER_T = (VBLK + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BC * D];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * BC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    int bh, qt, split = 0;
    if constexpr (SPLIT) {
        // key range outermost, so the workgroups of one range (same K/V rows) run together
        const int L = blockIdx.x, per = BH * n_qt;
        split = L / per;
        bh = (L % per) / n_qt;
        qt = (L % per) % n_qt;
    } else if constexpr (CAUSAL) {
        // longest rows first: the last query tiles see the most keys
        const int L = blockIdx.x;
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
    if constexpr (CAUSAL) k_end = min(Nk, min(qt * BR + BR, Nq));  // keys <= last query of the workgroup
    int k_begin = 0;
    if constexpr (SPLIT) {
        k_begin = split * part.keys_per_split;
        k_end = min(k_end, k_begin + part.keys_per_split);
    }
    const int n_kt = k_end > k_begin ? (k_end - k_begin + BC - 1) / BC : 0;

    // Q^T fragments: B operand of S^T = K Q^T, k = head-dim index 16*ks + 8*g + v.
    // Loaded before any tile prefetch so waiting for them never waits on a prefetch.
    u32x4_t qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = load8_operand<E>(Q, q_head + (int64_t)q_ld * D + 16 * ks + 8 * g);

    // ---- tile staging.  K: DMA (16-bit) or registers (fp32 -> bf16).  V: registers,
    // converted to fp16 and written transposed.
    const void *Kh = static_cast<const char *>(K) + k_head * (E == ELT_F32 ? 4 : 2);
    u32x4_t kreg[DMA ? 1 : KCH_PER_T];
    uint32_t vraw[VBLK_PER_T][4][2];  // [block][key][2 words of 4 columns] in the input type
    float vf32[E == ELT_F32 ? VBLK_PER_T : 1][4][4];
    auto load_tile = [&](int k0, int buf) __attribute__((always_inline)) {
        if constexpr (DMA) {
            dma_tile<D, BC, NW>(Kh, k0, Nk, Ks[buf], wave, lane);
        } else {
#pragma unroll
            for (int j = 0; j < KCH_PER_T; ++j) {
                const int i = tid + j * NT;
                const int row = i / NCH, c = i % NCH;
                kreg[j] = u32x4_t{0u, 0u, 0u, 0u};
                if (i < BC * NCH && k0 + row < Nk) kreg[j] = load8_operand<E>(K, k_head + (int64_t)(k0 + row) * D + c * 8);
            }
        }
        if constexpr (PREV) {
            // the packed V^T tile: 16 KiB copied as is, 1 KiB per wave instruction
            const uint16_t *src = Vpk + ((int64_t)bh * ((Nk + BC - 1) / BC) + k0 / BC) * (D * BC);
#pragma unroll
            for (int b = wave; b < D * BC / 512; b += NW)
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + b * 512 + lane * 8),
                                                 (__attribute__((address_space(3))) void *)(&Vt[buf][b * 512]), 16, 0, 0);
            return;
        }
        // Interior tiles (every key exists) take an unguarded path: a uniform branch
        // instead of one exec-masked load per key.
        auto load_v = [&](auto guarded_c) __attribute__((always_inline)) {
            constexpr bool guarded = decltype(guarded_c)::value;
#pragma unroll
            for (int j = 0; j < VBLK_PER_T; ++j) {
                const int i = tid + j * NT;
                int c4, u;  // keys 4u..4u+3, columns 4c4..4c4+3
                vblock<D, BC>(i, c4, u);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int key = k0 + 4 * u + k;
                    const bool ok = (VBLK % NT == 0 || i < VBLK) && (!guarded || key < Nk);
                    if constexpr (E == ELT_F32) {
                        f32x4_t x = {0.f, 0.f, 0.f, 0.f};
                        if (ok) x = *reinterpret_cast<const f32x4_t *>(static_cast<const float *>(V) + k_head + (int64_t)key * D + 4 * c4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) vf32[j][k][e] = x[e];
                    } else {
                        u32x2_t w = {0u, 0u};
                        if (ok) w = *reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(V) + k_head + (int64_t)key * D + 4 * c4);
                        vraw[j][k][0] = w[0];
                        vraw[j][k][1] = w[1];
                    }
                }
            }
        };
        if (k0 + BC <= Nk) load_v(std::false_type{});
        else load_v(std::true_type{});
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
        if constexpr (!DMA) {
#pragma unroll
            for (int j = 0; j < KCH_PER_T; ++j) {
                const int i = tid + j * NT;
                const int row = i / NCH, c = i % NCH;
                if (i < BC * NCH) *reinterpret_cast<u32x4_t *>(&Ks[buf][tile_off<D>(row, c * 8)]) = kreg[j];
            }
        }
        if constexpr (PREV) return;  // V^T arrived by copy
#pragma unroll
        for (int j = 0; j < VBLK_PER_T; ++j) {
            const int i = tid + j * NT;
            int c4, u;
            vblock<D, BC>(i, c4, u);
            if (i < VBLK) {
                float v[4][4];  // [key][column]
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if constexpr (E == ELT_F32) {
                        // the operand precision of fp32 data is bf16
                        const uint32_t w0 = pack_bf16(vf32[j][k][0], vf32[j][k][1]);
                        const uint32_t w1 = pack_bf16(vf32[j][k][2], vf32[j][k][3]);
                        v[k][0] = bf16_lo(w0); v[k][1] = bf16_hi(w0); v[k][2] = bf16_lo(w1); v[k][3] = bf16_hi(w1);
                    } else if constexpr (E == ELT_BF16) {
                        v[k][0] = bf16_lo(vraw[j][k][0]); v[k][1] = bf16_hi(vraw[j][k][0]);
                        v[k][2] = bf16_lo(vraw[j][k][1]); v[k][3] = bf16_hi(vraw[j][k][1]);
                    } else {
                        v[k][0] = f16_lo(vraw[j][k][0]); v[k][1] = f16_hi(vraw[j][k][0]);
                        v[k][2] = f16_lo(vraw[j][k][1]); v[k][3] = f16_hi(vraw[j][k][1]);
                    }
                }
                const int kst = u / 4, qd = u % 4;  // 16-key group, key quad inside it
                const int chunk = 2 * kst + (qd & 1), half = qd >> 1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int col = 4 * c4 + e;
                    *reinterpret_cast<u32x2_t *>(&Vt[buf][vt_row<BC>(col) * BC + ((chunk ^ vt_xor<BC>(col)) * 8) + half * 4]) =
                        u32x2_t{pack_f16(v[0][e], v[1][e]), pack_f16(v[2][e], v[3][e])};
                }
            }
        }
    };

    f32x16_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16_t{};
    float m_used = kMaxInit, l_run = 0.f;
    const f16x2_t ones = {(_Float16)1.f, (_Float16)1.f};

    if (n_kt > 0) {  // (workgroup-uniform: an empty key range skips straight to the epilogue)
        load_tile(k_begin, 0);
        store_tile(0);
    }
    wait_vmem();
    __syncthreads();

    // One key tile; BUF is the LDS buffer it reads (compile-time, so every LDS
    // address is a fixed offset from a per-lane base).
    auto step = [&](int kt, auto buf_c) __attribute__((always_inline)) {
        constexpr int buf = decltype(buf_c)::value;
        const int k0 = k_begin + kt * BC;
        const bool more = kt + 1 < n_kt;
        if (more) load_tile(k0 + BC, buf ^ 1);  // in flight during this tile's math
        if (!CAUSAL || k0 <= q_wave0 + 31) {  // else the tile lies above the diagonal for every row of this wave
            // dropout keep flags first: they do not depend on the scores, so the
            // generator's vector work can run beside the S^T products
            uint32_t keepv[NKB];  // bit r: register r of block kb survives dropout
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                keepv[kb] = DROP ? dropout_keep_query_lane(dr, (uint32_t)bh, (uint32_t)q,
                                                           (uint32_t)(k0 + 32 * kb + 4 * g), lane) : 0u;
            // ---- S^T = K Q^T : lane = query, register r -> key 8*(r/4) + 4*g + r%4 of each 32-key block
            f32x16_t s[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {  // independent accumulation chains back to back
                    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(&Ks[buf][tile_off<D>(kb * 32 + l32, 16 * ks + 8 * g)]);
                    s[kb] = mfma_in<E>(a, qf[ks], s[kb]);
                }

            const bool ragged = k0 + BC > Nk;
            const bool diag = CAUSAL && (k0 + BC - 1 > q_wave0);
            if (ragged || diag) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + kb * 32 + 8 * (r / 4) + 4 * g + (r % 4);
                        if (key >= Nk || (CAUSAL && key > q)) s[kb][r] = -INFINITY;
                    }
            }

            // ---- tile max; move the reference maximum only when it grows past the threshold
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = half_max(mx) * scale_log2;  // scale > 0, so max commutes with it
            if (__ballot(mx > m_used + kRescaleThreshold) != 0) {  // wave-uniform branch
                const float m_new = fmaxf(m_used, mx);
                const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
                m_used = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            }

            // ---- P = exp2(s*c - m_used) rounded to fp16; l += sum of the rounded values
            // (under dropout, pk then loses its dropped elements: l keeps them)
            uint32_t pk[NKB][8];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const uint32_t keep = keepv[kb];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * i], scale_log2, -m_used));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * i + 1], scale_log2, -m_used));
                    pk[kb][i] = pack_f16(p0, p1);
                    l_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk[kb][i]), ones, l_run, false);
                    if constexpr (DROP)
                        pk[kb][i] &= ((keep >> (2 * i)) & 1u ? 0x0000ffffu : 0u) |
                                     ((keep >> (2 * i + 1)) & 1u ? 0xffff0000u : 0u);
                }
            }

            // ---- O^T += V^T P^T (fp16 matrix core).  k-step kst covers keys
            // 16*kst .. 16*kst+15; slot (g, v) holds key 16*kst + 4g + v (v < 4)
            // or 16*kst + 8 + 4g + (v-4), matching the S^T register order.
#pragma unroll
            for (int kst = 0; kst < BC / 16; ++kst) {
                const int kb = kst / 2, h = kst % 2;
                const u32x4_t b = {pk[kb][4 * h], pk[kb][4 * h + 1], pk[kb][4 * h + 2], pk[kb][4 * h + 3]};
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int col = db * 32 + l32;
                    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(
                        &Vt[buf][vt_row<BC>(col) * BC + (((2 * kst + g) ^ vt_xor<BC>(col)) * 8)]);
                    o[db] = mfma_f16(a, b, o[db]);
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

    const float l_tot = half_sum(l_run);
    if constexpr (SPLIT) {
        // ---- partial state of this key range: u (unnormalised), m (log2 units), l
        if (q < Nq) {
            const int64_t R = (int64_t)BH * Nq;
            const int64_t prow = (int64_t)split * R + (int64_t)bh * Nq + q;
            float *urow = part.U + prow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq)
                    *reinterpret_cast<f32x4_t *>(urow + db * 32 + 8 * rq + 4 * g) =
                        f32x4_t{o[db][4 * rq], o[db][4 * rq + 1], o[db][4 * rq + 2], o[db][4 * rq + 3]};
            if (g == 0) {
                part.M[prow] = m_used;
                part.L[prow] = l_tot;
            }
        }
        return;
    }
    // ---- epilogue: O = u / l (times 1 / (1 - rate) under dropout), LSE = (m_used + log2 l) * ln 2
    const float inv = (DROP ? dr.keep_scale : 1.f) / l_tot;
    if (q < Nq) {
        const int64_t orow = q_head + (int64_t)q * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq)
                store4<E>(O, orow + db * 32 + 8 * rq + 4 * g, o[db][4 * rq] * inv, o[db][4 * rq + 1] * inv,
                          o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
        if (g == 0) LSE[(int64_t)bh * Nq + q] = (m_used + __builtin_log2f(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------- 64 query rows per wave
// fa_fwd_ws at d = 128 on 16-bit data.  Four waves, one per SIMD, each owning
// 64 query rows (two 32-row blocks) of the workgroup's 256, so every K or V^T
// fragment read from LDS feeds two products (fwd_kernel reads one per
// product).  Q^T fragments and the O^T accumulators sit in AGPRs, the scores
// in VGPRs where the softmax reads them.  The results are fwd_kernel's bits:
// every accumulator takes the same products in the same order, the maximum
// and the rescale decision are made per tile and per 32-row block as there,
// and each row sum adds the same fp16 values in the same order.
//
// With one wave per SIMD only the wave's own instruction stream keeps the
// matrix core busy, so a step (tile j of 64 keys) is a fixed program of 64
// products with a scheduling barrier after each:
//   products  0..31  S^T(j) = K Q^T, key block 0 then 1 (one K fragment for
//                    both row blocks);
//   products 32..47  O^T += V^T P^T for keys 32..63 of tile j - 1, held over
//                    from the previous step (their V^T fragments wait in
//                    registers);
//   products 48..63  O^T += V^T P^T for keys 0..31 of tile j.
// Beside them run the in-lane maxima of key block 0 (products 18..25) and
// 1 (34..37), the rescale vote (38), and the exponentials, one per product:
// tile j - 1's keys 48..63 (0..15), then tile j's keys 0..31 (16..47) and
// 32..47 (48..63), keys in the score registers' order.  The held-over
// products cover the latency of the last S^T results, which the maxima and
// the vote wait for.  The exponentials of keys 0..31 use the reference
// maximum as it stands; when the vote moves it (rare after the first tile),
// a branch before product 48 -- every product of tile j - 1 issued by then --
// rescales O and l and computes them again.
// K and V^T tiles are double-buffered in LDS and copied global -> LDS by
// inline assembly (the compiler uses no M0 of its own here), waited for once
// per step before the barrier.  Ragged and causal-diagonal tiles take a
// variant that masks each key block's scores, and takes its maxima, once its
// S^T products are done.
template <int E, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_r64_kernel(const void *__restrict__ Q, const void *__restrict__ K, void *__restrict__ O,
                    float *__restrict__ LSE, int BH, int Nq, int Nk, float scale_log2, int n_qt,
                    const uint16_t *__restrict__ Vpk) {
    constexpr int D = 128, NW = 4, BR = 64 * NW, BC = 64;
    constexpr int NKS = D / 16, NDB = D / 32, NKG = BC / 16;
    constexpr int TILE = BC * D * 2;       // bytes of a K tile or of a V^T tile
    constexpr int VS = 2 * TILE;           // K stage s at s TILE, V^T stage s at VS + s TILE
    constexpr int QS = 4 * TILE;           // the Q tile (BR rows, tile_off<D> layout): 4 TILE bytes
    constexpr int NCP = TILE / 1024 / NW;  // 1 KiB copies per wave per tile and tensor
    constexpr int LEAD = 3, NSLOT = LEAD + 1;
    static_assert(E != ELT_F32, "16-bit K is copied global -> LDS as it is");
    static_assert(BR * D * 2 == 4 * TILE, "the Q tile fills four tile-sized stages");
    __shared__ __attribute__((aligned(16))) unsigned char lds[8 * TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;


    // LDS byte offsets in a stage: a_off[ks] the K fragment (key row l32 of a
    // 32-key block, head dims 16 ks + 8 g .. +7; key block 1 adds 8 KiB);
    // v_off[p][kg] the V^T fragment of head dim 32 db + l32 with db % 2 = p
    // (db / 2 adds 8 KiB), keys of 16-key group kg.
    uint32_t a_off[NKS], v_off[2][NKG];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) a_off[ks] = 2u * (uint32_t)tile_off<D>(l32, 16 * ks + 8 * g);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int kg = 0; kg < NKG; ++kg) {
            const int col = 32 * p + l32;
            v_off[p][kg] = (uint32_t)VS + 2u * (uint32_t)(vt_row<BC>(col) * BC + (((2 * kg + g) ^ vt_xor<BC>(col)) * 8));
        }

    // Copies global -> LDS in 1 KiB blocks, block b = wave + 4 jb: K rows 4b ..
    // 4b + 3 of a tile with the swizzle applied on the global side (rows past
    // Nk re-read row Nk - 1, whose scores are masked), V^T tiles as they are,
    // Q rows the same way as K (rows past Nq re-read row Nq - 1, never stored).
    const int n_kt_all = (Nk + BC - 1) / BC;  // tiles per head in the packed V^T
    const int cp_row = wave * 4 + lane / 16;
    const uint32_t cp_col = (uint32_t)((lane & 15) ^ swz<D>(cp_row)) * 16u;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 in the clobber list: see the kernel's notes
    auto copy_tile = [&](int kt, int s, int jb, const uint16_t *Kb, const unsigned char *Vb)
        __attribute__((always_inline)) {
        const int grow = min(kt * BC + cp_row + 16 * jb, Nk - 1);
        const uint32_t koff = (uint32_t)grow * (uint32_t)(D * 2) + cp_col;
        const uint32_t voff = (uint32_t)kt * (uint32_t)TILE + (uint32_t)((wave + NW * jb) * 1024 + lane * 16);
        const uint32_t dk = (uint32_t)(s * TILE + (wave + NW * jb) * 1024);
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(koff), "s"(Kb), "s"(dk)
                     : "memory", "m0");
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(Vb),
                     "s"(dk + (uint32_t)VS)
                     : "memory", "m0");
    };
    auto copy_q = [&](int q0, const uint16_t *Qb) __attribute__((always_inline)) {
#pragma unroll
        for (int jb = 0; jb < BR / 16; ++jb) {
            const int grow = min(q0 + cp_row + 16 * jb, Nq - 1);
            const uint32_t qoff = (uint32_t)grow * (uint32_t)(D * 2) + cp_col;
            const uint32_t dq = (uint32_t)(QS + (wave + NW * jb) * 1024);
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(qoff), "s"(Qb), "s"(dq)
                         : "memory", "m0");
        }
    };
#pragma clang diagnostic pop

    // Work items are query tiles.  Causal: one per workgroup, the longest rows
    // first.  Otherwise the workgroups are persistent: workgroup w takes the
    // tiles it * gridDim.x + xcd_remap(w), so that in every round an XCD's
    // workgroups hold consecutive tiles (the same heads' K and V in its L2),
    // and each item's Q tile and first K/V tile are copied while the item
    // before it still computes.
    const int n_items = BH * n_qt;
    auto item_of = [&](int it) -> int {
        if constexpr (CAUSAL) return it == 0 ? (int)blockIdx.x : -1;
        const int L = it * (int)gridDim.x + xcd_remap(blockIdx.x, gridDim.x);
        return L < n_items ? L : -1;
    };
    auto decode = [&](int L, int &bh, int &qt) __attribute__((always_inline)) {
        if constexpr (CAUSAL) {
            qt = n_qt - 1 - L / BH;
            bh = L % BH;
        } else {
            bh = L / n_qt;
            qt = L % n_qt;
        }
    };
    auto k_base = [&](int bh) { return static_cast<const uint16_t *>(K) + (int64_t)bh * Nk * D; };
    auto v_base = [&](int bh) {
        return reinterpret_cast<const unsigned char *>(Vpk) + (int64_t)bh * n_kt_all * TILE;
    };
    auto q_base = [&](int bh) { return static_cast<const uint16_t *>(Q) + (int64_t)bh * Nq * D; };

    int L = item_of(0);
    int base = 0;  // the LDS stage of the current item's first tile
    if (L >= 0) {  // the first item's Q tile and first K / V tile
        int bh0, qt0;
        decode(L, bh0, qt0);
        copy_q(qt0 * BR, q_base(bh0));
#pragma unroll
        for (int jb = 0; jb < NCP; ++jb) copy_tile(0, 0, jb, k_base(bh0), v_base(bh0));
    }
    for (int it = 0; L >= 0; ++it) {
        const int Ln = item_of(it + 1);
        int bh, qt, bhn = 0, qtn = 0;
        decode(L, bh, qt);
        if (Ln >= 0) decode(Ln, bhn, qtn);
        const int64_t q_head = (int64_t)bh * Nq * D;
        const int q_w0 = qt * BR + 64 * wave;  // first row of this wave
        const int k_end = CAUSAL ? min(Nk, min(qt * BR + BR, Nq)) : Nk;
        const int n_kt = (k_end + BC - 1) / BC;
        const uint16_t *Kh = k_base(bh);
        const unsigned char *Vh = v_base(bh);
        // the next item's first tile goes where this item's tile n_kt would
        const uint16_t *Kx = Ln >= 0 ? k_base(bhn) : Kh;
        const unsigned char *Vx = Ln >= 0 ? v_base(bhn) : Vh;

        // this item's Q tile and first tile are in LDS once every wave's copies
        // are (for later items the previous item's step ends already waited
        // for them: its first step for the Q tile, its last for the K/V tile)
        if (it == 0) {
            wait_vmem();
            __syncthreads();
        }
        // Q^T fragments (B operands of S^T = K Q^T, k = head dim 16 ks + 8 g + v)
        // of both row blocks, from the Q tile into AGPRs.  The swizzle depends
        // on the row's low four bits only, so the wave's fragment ks of row
        // block r sits at the K fragment's offset a_off[ks] plus 256 bytes per
        // row of 64 wave + 32 r.  The wave's part is made opaque per item so
        // the eight sums are formed here, not kept live over the item loop.
        uint32_t qb = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char *)lds) +
                      (uint32_t)(QS + 64 * 256 * wave);
        asm volatile("" : "+s"(qb));
        uint32_t qa[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qa[ks] = qb + a_off[ks];
        u32x4_t qf[2][NKS];
        lds_read_agpr(qf, qa);
        // last key each lane's rows see (past Nk, or causal past the row), less
        // the lane's 4g offset in the score registers' key order
        int klim[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) klim[r] = (CAUSAL ? min(q_w0 + 32 * r + l32, Nk - 1) : Nk - 1) - 4 * g;
        // every wave holds its Q: the tile's space takes the next item's
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
        if (Ln >= 0) copy_q(qtn * BR, q_base(bhn));

        f32x16_t o[2][NDB];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[r][db] = f32x16_t{};
        float m_used[2] = {kMaxInit, kMaxInit}, l_run[2] = {0.f, 0.f};
        const f16x2_t ones = {(_Float16)1.f, (_Float16)1.f};
        // Scores of the current tile [key block][row block]; P as fp16 pairs, the
        // B operand of each 16-key group [row block][group]; V^T fragments of the
        // held-over groups 2 and 3 [group - 2][db].  Before the first tile the
        // held-over part is empty: scores -inf (P = 0) and V^T = 0.
        f32x16_t sc[2][2];
        u32x4_t pk[2][NKG], vt[2][NDB];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[1][r][e] = -INFINITY;
            pk[r][2] = u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int db = 0; db < NDB; ++db) vt[h][db] = u32x4_t{0u, 0u, 0u, 0u};
        mfma_wait<3>();  // the zeroed accumulators, before mfma_acc reads them

        // The exponentials run as a stream of 32 pairs per step, one pair per two
        // products.  Pair P: P < 8 the previous tile's group 3 (row block P / 4),
        // then groups 0, 1, 2 of this tile (row block (P % 8) / 4); t = P % 4 picks
        // register elements 8 (group % 2) + 2t, + 1 of key block group / 2.  Each
        // element's exponential is issued in a slot of its own (pa) and the pair is
        // packed to fp16 and added to the row sum a slot later (pb), so the wave
        // never waits on the transcendental unit's latency.
        auto pair_of = [](int P, int &kg, int &r, int &t) constexpr {
            kg = P < 8 ? 3 : (P - 8) / 8;
            r = (P % 8) / 4;
            t = P % 4;
        };
        float xp[2][2];  // the two exponentials of pairs in flight, by P % 2
        xp[1][0] = xp[1][1] = 0.f;  // "pair 31 of the tile before the first": P = 0
        auto pa = [&](int P, int h) __attribute__((always_inline)) {
            int kg, r, t;
            pair_of(P, kg, r, t);
            const int e = 8 * (kg % 2) + 2 * t + h;
            xp[P % 2][h] = __builtin_amdgcn_exp2f(fmaf(sc[kg / 2][r][e], scale_log2, -m_used[r]));
        };
        auto pb = [&](int P) __attribute__((always_inline)) {
            int kg, r, t;
            pair_of(P, kg, r, t);
            // (the word is cast, not the vector element: a cast of an element of a
            // vector lvalue reads element 0)
            const uint32_t w = pack_f16(xp[P % 2][0], xp[P % 2][1]);
            pk[r][kg][t] = w;
            l_run[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), ones, l_run[r], false);
        };

        // One step over tile kt in stage s, copying tile kn of the head at Kn / Vn
        // (this item's next tile, or the next item's first) into stage s ^ 1.
        auto step = [&](int kt, int s, int kn, const uint16_t *Kn, const unsigned char *Vn, auto mask_c)
            __attribute__((always_inline)) {
            constexpr bool MASK = decltype(mask_c)::value;
            const uint32_t sb = (uint32_t)(s * TILE);
            uint32_t ao[NKS], vo[2][NKG];
    #pragma unroll
            for (int ks = 0; ks < NKS; ++ks) ao[ks] = a_off[ks] + sb;
    #pragma unroll
            for (int p = 0; p < 2; ++p)
    #pragma unroll
                for (int kg = 0; kg < NKG; ++kg) vo[p][kg] = v_off[p][kg] + sb;
            const int k0 = kt * BC;
            u32x4_t opr[NSLOT];
            float mx[2] = {-INFINITY, -INFINITY}, mt[2], l_prev[2];
            uint64_t vote[2];
            // operand of product pair u (products 2u, 2u + 1, one per row block):
            // u < 16 K fragment (key block u / 8, k-step u % 8); 16..23 held-over
            // V^T in registers; 24..31 V^T fragment (group (u - 24) / 4, db (u - 24) % 4)
            auto rd = [&](int u) __attribute__((always_inline)) {
                if (u < 16) opr[u % NSLOT] = *reinterpret_cast<const u32x4_t *>(lds + ao[u % 8] + (u / 8) * 32 * 256);
                else if (u >= 24) {
                    const int kg = (u - 24) / 4, db = (u - 24) % 4;
                    opr[u % NSLOT] = *reinterpret_cast<const u32x4_t *>(lds + vo[db % 2][kg] + (db / 2) * 8192);
                }
            };
            auto mm = [&](int i) __attribute__((always_inline)) {
                const int u = i / 2, r = i % 2;
                if (u < 16) {
                    const int kb = u / 8, ks = u % 8;
                    if (ks == 0) sc[kb][r] = mfma_bagpr_first<E>(opr[u % NSLOT], qf[r][0]);
                    else mfma_bagpr<E>(sc[kb][r], opr[u % NSLOT], qf[r][ks]);
                } else if (u < 24) {
                    const int kg = 2 + (u - 16) / 4, db = (u - 16) % 4;
                    mfma_acc<ELT_F16>(o[r][db], vt[kg - 2][db], pk[r][kg]);
                } else {
                    const int kg = (u - 24) / 4, db = (u - 24) % 4;
                    mfma_acc<ELT_F16>(o[r][db], opr[u % NSLOT], pk[r][kg]);
                }
            };
            // in-lane maximum over elements 4c .. 4c + 3 of key block kb, row block r
            auto maxq = [&](int kb, int r, int c) __attribute__((always_inline)) {
                mx[r] = max3(max3(mx[r], sc[kb][r][4 * c], sc[kb][r][4 * c + 1]), sc[kb][r][4 * c + 2], sc[kb][r][4 * c + 3]);
            };
            auto do_vote = [&]() __attribute__((always_inline)) {
    #pragma unroll
                for (int r = 0; r < 2; ++r) {
                    mt[r] = half_max(mx[r]) * scale_log2;  // scale > 0: max commutes with it
                    vote[r] = __ballot(mt[r] > m_used[r] + kRescaleThreshold);
                }
            };
            // masked tiles: the scores of every key past Nk or after the row -> -inf
            auto mask_block = [&](int kb) __attribute__((always_inline)) {
    #pragma unroll
                for (int r = 0; r < 2; ++r)
    #pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (k0 + 32 * kb + 8 * (e / 4) + (e % 4) > klim[r]) sc[kb][r][e] = -INFINITY;
            };

            static_for<LEAD>([&](auto c) __attribute__((always_inline)) { rd(decltype(c)::value); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<64>([&](auto nc) __attribute__((always_inline)) {
                constexpr int n = decltype(nc)::value;
                if constexpr (MASK && (n == 16 || n == 32)) {
                    // mask a key block once its S^T products are done, and take its maxima
                    mfma_drain();
                    mask_block(n / 16 - 1);
    #pragma unroll
                    for (int c = 0; c < 8; ++c) maxq(n / 16 - 1, c / 4, c % 4);
                    if constexpr (n == 32) do_vote();
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (!MASK && n == 16) mfma_wait<7>();  // key block 0's S^T results, before pa reads them
                if constexpr (n == 48) {
                    // every product of the previous tile is issued: move the reference
                    // maximum where the vote says so, rescale O and l, and redo the
                    // exponentials of groups 0 and 1
                    if ((vote[0] | vote[1]) != 0) {
                        keep_branch();
                        // the accumulators' wait states, with the accumulators as
                        // operands so that no copy of them is taken before it
                        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                                     : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]),
                                       "+a"(o[1][1]), "+a"(o[1][2]), "+a"(o[1][3])
                                     :
                                     : "memory");
    #pragma unroll
                        for (int r = 0; r < 2; ++r) {
                            // a block that did not vote keeps its maximum: alpha = 1, exact
                            const float m_new = vote[r] != 0 ? fmaxf(m_used[r], mt[r]) : m_used[r];
                            const float alpha = __builtin_amdgcn_exp2f(m_used[r] - m_new);
                            m_used[r] = m_new;
                            l_run[r] = l_prev[r] * alpha;
    #pragma unroll
                            for (int db = 0; db < NDB; ++db) o[r][db] *= alpha;
                        }
    #pragma unroll
                        for (int P = 8; P < 24; ++P) {
                            pa(P, 0);
                            pa(P, 1);
                            pb(P);
                        }
                    }
                    mfma_wait<1>();  // P and the rescaled accumulators, before the products read them
                }
                mm(n);
                if constexpr (n % 2 == 1) {
                    constexpr int u = n / 2 + LEAD;
                    if constexpr (u < 32) rd(u);
                }
                if constexpr (n >= 1 && n <= NCP) copy_tile(kn, s ^ 1, n - 1, Kn, Vn);
                // the exponential stream: pair n / 2 - 1 finished (but pair 23's,
                // which must precede the branch before product 48), pair n / 2 started
                if constexpr (n % 2 == 0 && n != 48) pb(n == 0 ? 31 : n / 2 - 1);
                pa(n / 2, n % 2);
                if constexpr (n == 47) pb(23);
                if constexpr (n == 17) { l_prev[0] = l_run[0]; l_prev[1] = l_run[1]; }  // before group 0's sums
                if constexpr (!MASK) {
                    if constexpr (n == 34) mfma_wait<7>();  // key block 1's S^T results, before the maxima read them
                    if constexpr (n >= 18 && n < 26) maxq(0, (n - 18) / 4, (n - 18) % 4);
                    if constexpr (n >= 34 && n < 38) {
                        maxq(1, (n - 34) / 2, 2 * ((n - 34) % 2));
                        maxq(1, (n - 34) / 2, 2 * ((n - 34) % 2) + 1);
                    }
                    if constexpr (n == 38) do_vote();
                }
                // V^T fragments of groups 2, 3 for the next step
                if constexpr (n >= 48 && n % 2 == 0) {
                    constexpr int x = (n - 48) / 2, kg = 2 + x / 4, db = x % 4;
                    vt[kg - 2][db] = *reinterpret_cast<const u32x4_t *>(lds + vo[db % 2][kg] + (db / 2) * 8192);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };


        // Tiles that need no mask first: every key exists and, causal, precedes
        // the workgroup's first row.  The rest take the masked variant in a loop of
        // their own.  The last step copies the next item's first tile.
        int n_full = Nk / BC;
        if constexpr (CAUSAL) n_full = min(n_full, (qt * BR + 1) / BC);
        n_full = min(n_full, n_kt);
        int kt = 0;
        for (; kt < n_full; ++kt) {
            const bool last = kt + 1 == n_kt;
            step(kt, (base + kt) & 1, last ? 0 : kt + 1, last ? Kx : Kh, last ? Vx : Vh, std::false_type{});
        }
        for (; kt < n_kt; ++kt) {
            const bool last = kt + 1 == n_kt;
            step(kt, (base + kt) & 1, last ? 0 : kt + 1, last ? Kx : Kh, last ? Vx : Vh, std::true_type{});
        }
        base = (base + n_kt) & 1;

        // the last tile's group 2 sums and group 3, then its held-over products
        pb(31);
        static_for<8>([&](auto c) __attribute__((always_inline)) {
            constexpr int P = decltype(c)::value;
            pa(P, 0);
            pa(P, 1);
            pb(P);
        });
        mfma_wait<1>();
        static_for<16>([&](auto c) __attribute__((always_inline)) {
            constexpr int i = decltype(c)::value, kg = 2 + i / 8, db = (i % 8) / 2, r = i % 2;
            mfma_acc<ELT_F16>(o[r][db], vt[kg - 2][db], pk[r][kg]);
            __builtin_amdgcn_sched_barrier(0);
        });
        mfma_drain();  // mfma_acc results, before they are read

        // ---- epilogue: O = u / l, LSE = (m_used + log2 l) * ln 2
    #pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float l_tot = half_sum(l_run[r]);
            const float inv = 1.f / l_tot;
            const int q = q_w0 + 32 * r + l32;
            if (q < Nq) {
                const int64_t orow = q_head + (int64_t)q * D;
    #pragma unroll
                for (int db = 0; db < NDB; ++db)
    #pragma unroll
                    for (int rq = 0; rq < 4; ++rq)
                        store4<E>(O, orow + db * 32 + 8 * rq + 4 * g, o[r][db][4 * rq] * inv, o[r][db][4 * rq + 1] * inv,
                                  o[r][db][4 * rq + 2] * inv, o[r][db][4 * rq + 3] * inv);
                if (g == 0) LSE[(int64_t)bh * Nq + q] = (m_used[r] + __builtin_log2f(l_tot)) * kLn2;
            }
        }

        L = Ln;
    }
}

// fa_fwd_ws at d = 128 on 16-bit data takes fwd_r64_kernel; 0 selects fwd_kernel.
#ifndef FA_FWD_R64
#define FA_FWD_R64 1
#endif

// Launch shape: waves per workgroup (32 query rows each) and keys per tile.
#ifndef FA_FWD_WAVES
#define FA_FWD_WAVES 8
#endif
#ifndef FA_FWD_KEYS
#define FA_FWD_KEYS 64
#endif
// Keys per tile: at d = 64 each tile carries half the matrix work of d = 128, so
// it takes twice as many keys to keep the per-tile costs (barrier, staging) the
// same fraction of the time.
#ifndef FA_FWD_KEYS_D64
#define FA_FWD_KEYS_D64 128
#endif
template <int D>
constexpr int fwd_keys() { return D == 64 ? FA_FWD_KEYS_D64 : FA_FWD_KEYS; }

// Merge of the split-KV partial states: one thread per 4 columns of a row.
template <int D, int E>
__global__ __launch_bounds__(256) void fwd_merge_kernel(SplitOut part, int G, int64_t R, void *__restrict__ O,
                                                        float *__restrict__ LSE) {
    constexpr int TPR = D / 4;       // threads per row
    constexpr int RPB = 256 / TPR;   // rows per block
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c4 = threadIdx.x % TPR;
    if (row >= R) return;
    // (unrolled so that the independent loads of several ranges are in flight together)
    float m_star = kMaxInit;
#pragma unroll 8
    for (int gi = 0; gi < G; ++gi) m_star = fmaxf(m_star, part.M[gi * R + row]);
    float l = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int gi = 0; gi < G; ++gi) {
        const float a = __builtin_amdgcn_exp2f(part.M[gi * R + row] - m_star);
        l = fmaf(a, part.L[gi * R + row], l);
        const f32x4_t u = *reinterpret_cast<const f32x4_t *>(part.U + (gi * R + row) * D + 4 * c4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(a, u[e], acc[e]);
    }
    const float inv = 1.f / l;
    store4<E>(O, row * D + 4 * c4, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    if (c4 == 0) LSE[row] = (m_star + __builtin_log2f(l)) * kLn2;
}

// Compute units of the current device (cached per device; every MI355X has
// 256).  Callers on several host threads may race to fill an entry: they
// store the same value, through an atomic.
int compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int D, int E, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs &a) {
    constexpr int BC = fwd_keys<D>(), NW = FA_FWD_WAVES, BR = 32 * NW;
    const int n_qt = (a.Nq + BR - 1) / BR;
    const int BH = a.B * a.H;
    const dim3 block(NW * 64);
    const float sl2 = a.scale * kLog2e;
    hipStream_t st = (hipStream_t)a.stream;
    if (a.drop.t > 0) {
        hipLaunchKernelGGL((fwd_kernel<D, BC, NW, E, CAUSAL, false, true>), dim3(BH * n_qt), block, 0, st, a.Q, a.K,
                           a.V, a.O, a.LSE, BH, a.Nq, a.Nk, sl2, n_qt, SplitOut{}, a.drop, nullptr);
        return hipGetLastError();
    }
    if (a.num_splits <= 1 && a.Vpk) {
        // V^T tiles packed once, then copied as they are by the key loop
        const int n_kt = (a.Nk + BC - 1) / BC;
        hipLaunchKernelGGL((v_pack_kernel<D, BC, E>), dim3(BH * n_kt), dim3(512), 0, st, a.V, a.Vpk, a.Nk, n_kt);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if constexpr (D == 128 && E != ELT_F32 && BC == 64 && BR == 256 && FA_FWD_R64) {
            // 64 query rows per wave, one wave per SIMD, over the same 256-row tiles
            // causal: one query tile per workgroup; otherwise one persistent
            // workgroup per compute unit walks the tiles
            const int items = BH * n_qt;
            const int grid = CAUSAL ? items : std::min(items, compute_units());
            hipLaunchKernelGGL((fwd_r64_kernel<E, CAUSAL>), dim3(grid), dim3(256), 0, st, a.Q, a.K, a.O, a.LSE,
                               BH, a.Nq, a.Nk, sl2, n_qt, a.Vpk);
            return hipGetLastError();
        }
        hipLaunchKernelGGL((fwd_kernel<D, BC, NW, E, CAUSAL, false, false, true>), dim3(BH * n_qt), block, 0, st, a.Q,
                           a.K, a.V, a.O, a.LSE, BH, a.Nq, a.Nk, sl2, n_qt, SplitOut{}, Dropout{}, a.Vpk);
        return hipGetLastError();
    }
    if (a.num_splits <= 1) {
        hipLaunchKernelGGL((fwd_kernel<D, BC, NW, E, CAUSAL, false, false>), dim3(BH * n_qt), block, 0, st, a.Q, a.K,
                           a.V, a.O, a.LSE, BH, a.Nq, a.Nk, sl2, n_qt, SplitOut{}, Dropout{}, nullptr);
        return hipGetLastError();
    }
    const int G = a.num_splits;
    const SplitOut part{a.Upart, a.Mpart, a.Lpart, a.keys_per_split};
    hipLaunchKernelGGL((fwd_kernel<D, BC, NW, E, CAUSAL, true, false>), dim3(BH * n_qt * G), block, 0, st, a.Q, a.K,
                       a.V, a.O, a.LSE, BH, a.Nq, a.Nk, sl2, n_qt, part, Dropout{}, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t R = (int64_t)BH * a.Nq;
    constexpr int RPB = 256 / (D / 4);
    hipLaunchKernelGGL((fwd_merge_kernel<D, E>), dim3((unsigned)((R + RPB - 1) / RPB)), dim3(256), 0, st, part, G,
                       R, a.O, a.LSE);
    return hipGetLastError();
}

template <int D, int E>
static hipError_t launch_fwd_c(const FwdArgs &a) {
    return a.causal ? launch_fwd_t<D, E, true>(a) : launch_fwd_t<D, E, false>(a);
}

template <int D>
static hipError_t launch_fwd_d(const FwdArgs &a) {
    switch (a.dtype) {
        case ELT_BF16: return launch_fwd_c<D, ELT_BF16>(a);
        case ELT_F16: return launch_fwd_c<D, ELT_F16>(a);
        default: return launch_fwd_c<D, ELT_F32>(a);
    }
}

hipError_t launch_fwd(const FwdArgs &a) { return a.d == 64 ? launch_fwd_d<64>(a) : launch_fwd_d<128>(a); }

int fwd_key_tile(int d) { return d == 64 ? fwd_keys<64>() : fwd_keys<128>(); }
int fwd_query_tile() { return 32 * FA_FWD_WAVES; }
size_t fwd_packed_v_bytes(int B, int H, int Nk, int d) {
    const int BC = fwd_key_tile(d);
    return (size_t)B * H * ((Nk + BC - 1) / BC) * (size_t)BC * d * 2;
}

const char *describe_fwd() {
    return "fwd_kernel<D, keys per tile 64 (d=128) / 128 (d=64), waves=8 (256 query rows, 32 per wave), "
           "double-buffered K/V^T in LDS, S^T=KQ^T bf16/f16 MFMA 32x32x16, PV fp16 MFMA, lazy rescale>; "
           "fa_fwd_ws: v_pack_kernel (V -> fp16 V^T tiles in the LDS layout), then the key loop copies them; "
           "at d=128 on bf16/fp16 the key loop is fwd_r64_kernel<4 waves, one per SIMD, 64 query rows each, "
           "fixed 64-product program per 64-key tile, the last 32 keys' PV products held over to the next tile; "
           "non-causal: one persistent workgroup per CU over the query tiles>";
}

}  // namespace fa
