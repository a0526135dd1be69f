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
           "fa_fwd_ws: v_pack_kernel (V -> fp16 V^T tiles in the LDS layout), then the key loop copies them";
}

}  // namespace fa
