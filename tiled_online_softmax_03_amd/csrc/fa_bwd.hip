// fa_bwd.hip -- attention backward for gfx950.
//
// Method: page 1 "Flash Attention 原理与实现", section "Backward 的 Tiling
// 策略" (recompute S and P block by block instead of storing them; dV = P^T dO,
// dP = dO V^T, dQ = dS K, dK = dS^T Q; dQ and dK summed across blocks, by
// atomics or partial sums -- section "实际实现中的注意事项", item 3), with P
// rebuilt from the saved LSE as exp(s - LSE) (lumenova.space
// "research-attention", section 04).  The softmax gradient is the standard
// vector-Jacobian product dS = P * (dP - D), D_i = sum_j P_ij dP_ij, and
// D_i = rowsum(dO_i * O_i) because O_i = sum_j P_ij V_j.
//
// Three launches on the caller's stream:
//   1. bwd_pre_kernel   D = rowsum(dO * O) (fp32), zero the fp32 dQ accumulator.
//   2. bwd_dkdv_kernel  K/V-stationary: a workgroup owns 32*NW keys of one head
//                       (32 per wave, K and V rows kept in VGPRs), walks the
//                       query tiles, recomputes P, accumulates dV^T and dK^T in
//                       registers, and adds dS K into the dQ accumulator with
//                       fp32 atomics after exchanging dS through LDS.
//   3. bwd_dq_kernel    dQ = scale * accumulator, rounded to the output type.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

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

// ---------------------------------------------------------------- 1. preprocess
template <int D, int E>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const void *__restrict__ O, const void *__restrict__ dO,
                                                      float *__restrict__ Dvec, float *__restrict__ dQacc,
                                                      int64_t rows) {
    constexpr int NCH = D / 8;        // lanes per row
    constexpr int RPB = 256 / NCH;    // rows per block
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
        f32x4_t *z = reinterpret_cast<f32x4_t *>(dQacc + row * D + c * 8);
        z[0] = f32x4_t{};
        z[1] = f32x4_t{};
    }
#pragma unroll
    for (int off = NCH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && c == 0) Dvec[row] = acc;
}

// ---------------------------------------------------------------- 2. dK, dV (+ dQ atomics)

// Row-major 16-bit tile with rows of W elements: 16-byte chunk c of row r is
// stored at chunk c ^ rswz<W>(r) so that 16 rows read at one chunk spread
// over all banks.
template <int W>
__device__ __forceinline__ int rswz(int row) { return (row / (128 / W)) % (W / 8); }
// Transposed 16-bit tile with rows of W elements read in 8-byte units (4
// elements): unit u of row c is stored at unit u ^ tswz<W>(c).
template <int W>
__device__ __forceinline__ int tswz(int col) { return (col / (128 / W)) % (W / 4); }

__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <int D, int NW, int E, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(
    const void *__restrict__ Q, const void *__restrict__ K, const void *__restrict__ V,
    const void *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Dvec,
    float *__restrict__ dQacc, void *__restrict__ dK, void *__restrict__ dV, int BH, int Nq, int Nk,
    float scale, float scale_log2, int n_kt) {
    constexpr int BKC = 32 * NW;  // keys per workgroup
    constexpr int BQ = 32;        // queries per step
    constexpr int NT = NW * 64;
    constexpr int NCH = D / 8;    // 16-byte chunks per row of Q / dO / K
    constexpr int NKS = D / 16;   // k-steps over the head dim
    constexpr int NDB = D / 32;   // 32-row blocks of dK^T / dV^T
    static_assert(NW % NDB == 0 || NDB % NW == 0, "wave / column-block split");

    __shared__ __attribute__((aligned(16))) uint16_t Qs[BQ * D];    // [q][d]
    __shared__ __attribute__((aligned(16))) uint16_t dOs[BQ * D];   // [q][d]
    __shared__ __attribute__((aligned(16))) uint16_t Qt[D * BQ];    // [d][q]
    __shared__ __attribute__((aligned(16))) uint16_t dOt[D * BQ];   // [d][q]
    __shared__ __attribute__((aligned(16))) uint16_t Kt[D * BKC];   // [d][key], whole workgroup
    __shared__ __attribute__((aligned(16))) uint16_t dSs[BQ * BKC]; // [q][key]
    __shared__ __attribute__((aligned(16))) float lse2[BQ];
    __shared__ __attribute__((aligned(16))) float dvec[BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

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
    const int kw = k0 + wave * 32 + l32;  // this lane's key
    const int kw_ld = kw < Nk ? kw : Nk - 1;

    // K and V rows of this lane's key as B operands (k = head-dim index 16*ks + 8*g + v)
    u32x4_t kf[NKS], vf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        u32x4_t kz = load8_operand<E>(K, k_head + (int64_t)kw_ld * D + 16 * ks + 8 * g);
        u32x4_t vz = load8_operand<E>(V, k_head + (int64_t)kw_ld * D + 16 * ks + 8 * g);
        if (kw >= Nk) { kz = u32x4_t{0u, 0u, 0u, 0u}; vz = kz; }
        kf[ks] = kz;
        vf[ks] = vz;
    }
    // K^T of the whole workgroup into LDS for the dQ product: Kt[d][key]
    for (int i = tid; i < (BKC / 4) * NCH; i += NT) {
        const int c = i % NCH, u = i / NCH;  // keys 4u..4u+3, head dims 8c..8c+7
        u32x4_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int key = k0 + 4 * u + k;
            w[k] = key < Nk ? load8_operand<E>(K, k_head + (int64_t)key * D + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int dcol = c * 8 + e;
            const int wi = e / 2;
            const u32x2_t val = (e & 1) ? u32x2_t{hi16x2(w[0][wi], w[1][wi]), hi16x2(w[2][wi], w[3][wi])}
                                        : u32x2_t{lo16x2(w[0][wi], w[1][wi]), lo16x2(w[2][wi], w[3][wi])};
            // 8-byte unit u of row dcol; rows hold BKC keys -> 16-byte chunk u/2
            const int chunk = (u / 2) ^ rswz<BKC>(dcol);
            *reinterpret_cast<u32x2_t *>(&Kt[dcol * BKC + chunk * 8 + (u & 1) * 4]) = val;
        }
    }

    f32x16_t dvT[NDB], dkT[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) { dvT[db] = f32x16_t{}; dkT[db] = f32x16_t{}; }

    const int n_qt = (Nq + BQ - 1) / BQ;
    const int qt_begin = CAUSAL ? min(k0 / BQ, n_qt) : 0;

    // dQ work split: wave w covers column block (w % NDB) over key slice (w / NDB)
    constexpr int WPB = NW >= NDB ? NW / NDB : 1;  // waves per column block
    constexpr int KSL = BKC / WPB;                 // keys per slice
    const int dq_db = wave % NDB, dq_ks = wave / NDB;

    for (int qt = qt_begin; qt < n_qt; ++qt) {
        const int q0 = qt * BQ;
        __syncthreads();  // previous step done with every tile below
        // ---- stage Q and dO: row-major and transposed copies
        for (int i = tid; i < 2 * (BQ / 4) * NCH; i += NT) {
            const int which = i / ((BQ / 4) * NCH);  // 0: Q, 1: dO
            const int j = i % ((BQ / 4) * NCH);
            const int c = j % NCH, u = j / NCH;      // rows 4u..4u+3, head dims 8c..8c+7
            const void *src = which ? dO : Q;
            uint16_t *rm = which ? dOs : Qs;
            uint16_t *tr = which ? dOt : Qt;
            u32x4_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int qq = q0 + 4 * u + k;
                w[k] = qq < Nq ? load8_operand<E>(src, q_head + (int64_t)qq * D + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
                const int row = 4 * u + k;
                *reinterpret_cast<u32x4_t *>(&rm[row * D + ((c ^ rswz<D>(row)) * 8)]) = w[k];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int dcol = c * 8 + e;
                const int wi = e / 2;
                const u32x2_t val = (e & 1) ? u32x2_t{hi16x2(w[0][wi], w[1][wi]), hi16x2(w[2][wi], w[3][wi])}
                                            : u32x2_t{lo16x2(w[0][wi], w[1][wi]), lo16x2(w[2][wi], w[3][wi])};
                *reinterpret_cast<u32x2_t *>(&tr[dcol * BQ + ((u ^ tswz<BQ>(dcol)) * 4)]) = val;
            }
        }
        if (tid < BQ) {
            const int qq = q0 + tid;
            lse2[tid] = qq < Nq ? LSE[(int64_t)bh * Nq + qq] * kLog2e : INFINITY;  // P = 0 on padding rows
            dvec[tid] = qq < Nq ? Dvec[(int64_t)bh * Nq + qq] : 0.f;
        }
        __syncthreads();

        // ---- S = Q K^T and dP = dO V^T: lane = key, register r -> query 8*(r/4) + 4*g + r%4
        f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int ch = ((2 * ks + g) ^ rswz<D>(l32)) * 8;
            const u32x4_t qa = *reinterpret_cast<const u32x4_t *>(&Qs[l32 * D + ch]);
            const u32x4_t da = *reinterpret_cast<const u32x4_t *>(&dOs[l32 * D + ch]);
            s = mfma_in<E>(qa, kf[ks], s);
            dp = mfma_in<E>(da, vf[ks], dp);
        }
        // ---- P = exp(s*scale - LSE), dS = P * (dP - D)
        uint32_t pp[8], ds[8];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const f32x4_t L4 = *reinterpret_cast<const f32x4_t *>(&lse2[8 * rq + 4 * g]);
            const f32x4_t D4 = *reinterpret_cast<const f32x4_t *>(&dvec[8 * rq + 4 * g]);
            float p[4], t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * rq + i;
                const int qq = q0 + 8 * rq + 4 * g + i;
                float pv = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -L4[i]));
                if (CAUSAL && kw > qq) pv = 0.f;
                p[i] = pv;
                t[i] = pv * (dp[r] - D4[i]);
            }
            pp[2 * rq] = pack_in<E>(p[0], p[1]);
            pp[2 * rq + 1] = pack_in<E>(p[2], p[3]);
            ds[2 * rq] = pack_in<E>(t[0], t[1]);
            ds[2 * rq + 1] = pack_in<E>(t[2], t[3]);
            // dS into LDS as [q][key] for the dQ product
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 8 * rq + 4 * g + i;
                const int key = wave * 32 + l32;
                const int chunk = (key / 8) ^ rswz<BKC>(row);
                const uint32_t word = ds[2 * rq + i / 2];
                dSs[row * BKC + chunk * 8 + (key % 8)] = (uint16_t)((i & 1) ? (word >> 16) : (word & 0xffffu));
            }
        }
        // ---- dV^T += dO^T P and dK^T += Q^T dS (k = query; slot (g, v) -> 16h + 4g + v or 16h + 8 + 4g + v-4)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4_t bp = {pp[4 * h], pp[4 * h + 1], pp[4 * h + 2], pp[4 * h + 3]};
            const u32x4_t bs = {ds[4 * h], ds[4 * h + 1], ds[4 * h + 2], ds[4 * h + 3]};
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int dcol = db * 32 + l32;
                const int sw = tswz<BQ>(dcol);
                const int o1 = dcol * BQ + (((4 * h + g) ^ sw) * 4), o2 = dcol * BQ + (((4 * h + 2 + g) ^ sw) * 4);
                const u32x2_t a1 = *reinterpret_cast<const u32x2_t *>(&dOt[o1]);
                const u32x2_t a2 = *reinterpret_cast<const u32x2_t *>(&dOt[o2]);
                const u32x2_t b1 = *reinterpret_cast<const u32x2_t *>(&Qt[o1]);
                const u32x2_t b2 = *reinterpret_cast<const u32x2_t *>(&Qt[o2]);
                dvT[db] = mfma_in<E>(u32x4_t{a1[0], a1[1], a2[0], a2[1]}, bp, dvT[db]);
                dkT[db] = mfma_in<E>(u32x4_t{b1[0], b1[1], b2[0], b2[1]}, bs, dkT[db]);
            }
        }
        __syncthreads();  // dS of every wave in LDS

        // ---- dQ[q][d] += dS[q][key] K[key][d] over this wave's key slice and column block
        {
            f32x16_t acc = f32x16_t{};
            const int dcol = dq_db * 32 + l32;
#pragma unroll
            for (int kk = 0; kk < KSL / 16; ++kk) {
                const int kc = (dq_ks * KSL) / 8 + 2 * kk + g;  // 16-byte chunk of 8 keys
                const u32x4_t a = *reinterpret_cast<const u32x4_t *>(&dSs[l32 * BKC + ((kc ^ rswz<BKC>(l32)) * 8)]);
                const u32x4_t b = *reinterpret_cast<const u32x4_t *>(&Kt[dcol * BKC + ((kc ^ rswz<BKC>(dcol)) * 8)]);
                acc = mfma_in<E>(a, b, acc);
            }
            if (NW >= NDB || wave < NDB) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qq = q0 + 8 * (r / 4) + 4 * g + (r % 4);
                    if (qq < Nq) unsafeAtomicAdd(&dQacc[q_head + (int64_t)qq * D + dcol], acc[r]);
                }
            }
        }
    }

    // ---- dK = scale * dK^T^T, dV = dV^T^T: lane = key, register r -> head dim 32db + 8*(r/4) + 4*g + r%4
    if (kw < Nk) {
        const int64_t row = k_head + (int64_t)kw * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int col = db * 32 + 8 * rq + 4 * g;
                store4<E>(dK, row + col, dkT[db][4 * rq] * scale, dkT[db][4 * rq + 1] * scale,
                          dkT[db][4 * rq + 2] * scale, dkT[db][4 * rq + 3] * scale);
                store4<E>(dV, row + col, dvT[db][4 * rq], dvT[db][4 * rq + 1], dvT[db][4 * rq + 2],
                          dvT[db][4 * rq + 3]);
            }
    }
}

// ---------------------------------------------------------------- 3. dQ finalise
template <int E>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float *__restrict__ dQacc, void *__restrict__ dQ,
                                                     int64_t n8, float scale) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f32x4_t *p = reinterpret_cast<const f32x4_t *>(dQacc + i * 8);
    const f32x4_t a = p[0], b = p[1];
    store4<E>(dQ, i * 8, a[0] * scale, a[1] * scale, a[2] * scale, a[3] * scale);
    store4<E>(dQ, i * 8 + 4, b[0] * scale, b[1] * scale, b[2] * scale, b[3] * scale);
}

template <int D, int E, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs &a) {
    constexpr int NW = 4, BKC = 32 * NW;
    hipStream_t st = (hipStream_t)a.stream;
    const int BH = a.B * a.H;
    const int64_t rows = (int64_t)BH * a.Nq;
    {
        constexpr int RPB = 256 / (D / 8);
        hipLaunchKernelGGL((bwd_pre_kernel<D, E>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, a.O,
                           a.dO, a.Dvec, a.dQacc, rows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        const int n_kt = (a.Nk + BKC - 1) / BKC;
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, E, CAUSAL>), dim3(BH * n_kt), dim3(NW * 64), 0, st, a.Q, a.K, a.V,
                           a.dO, a.LSE, a.Dvec, a.dQacc, a.dK, a.dV, BH, a.Nq, a.Nk, a.scale, a.scale * kLog2e, n_kt);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        const int64_t n8 = rows * D / 8;
        hipLaunchKernelGGL((bwd_dq_kernel<E>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, a.dQacc, a.dQ, n8,
                           a.scale);
        return hipGetLastError();
    }
}

template <int D, int E>
static hipError_t launch_bwd_c(const BwdArgs &a) {
    return a.causal ? launch_bwd_t<D, E, true>(a) : launch_bwd_t<D, E, false>(a);
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs &a) {
    switch (a.dtype) {
        case ELT_BF16: return launch_bwd_c<D, ELT_BF16>(a);
        case ELT_F16: return launch_bwd_c<D, ELT_F16>(a);
        default: return launch_bwd_c<D, ELT_F32>(a);
    }
}

hipError_t launch_bwd(const BwdArgs &a) { return a.d == 64 ? launch_bwd_d<64>(a) : launch_bwd_d<128>(a); }

const char *describe_bwd() {
    return "bwd_pre_kernel -> bwd_dkdv_kernel<D, waves=4 (128 keys), query step 32, fp32 dQ atomics> -> bwd_dq_kernel";
}

}  // namespace fa
