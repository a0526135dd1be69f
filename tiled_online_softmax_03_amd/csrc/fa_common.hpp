// fa_common.hpp -- device helpers shared by the libfa kernels (gfx950 only).
//
// Matrix-core conventions used throughout (CDNA3/CDNA4 32x32 MFMA, wave64):
//   v_mfma_f32_32x32x16_{bf16,f16}: D[32x32] += A[32x16] * B[16x32]
//   A operand: lane l holds A[row = l%32][k in slot (l/32, v)], v = 0..7
//   B operand: lane l holds B[k in slot (l/32, v)][col = l%32]
//   C/D      : lane l, register r (0..15) holds D[8*(r/4) + 4*(l/32) + r%4][l%32]
// The contraction index k only has to be assigned to the same (l/32, v) slot
// in A and B, so the kernels pick whatever k order makes their loads cheap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_types.hpp"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Element type of the tensors crossing the ABI.
enum Elt : int { ELT_BF16 = 0, ELT_F16 = 1, ELT_F32 = 2 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_f16(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// The 16-bit operand type of a matrix product on data of element type E:
// fp16 data stays fp16, bf16 stays bf16, fp32 is rounded to bf16.
template <int E>
__device__ __forceinline__ f32x16_t mfma_in(u32x4_t a, u32x4_t b, f32x16_t c) {
    if constexpr (E == ELT_F16) return mfma_f16(a, b, c);
    else return mfma_bf16(a, b, c);
}

// acc += A B with the accumulator pinned to accumulation registers (AGPRs),
// for accumulators that only ever feed matrix products.  The compiler does not
// see the product's latency, so a reader of acc outside these products must
// wait for it (the callers put the wait states in front of such reads), and
// the B operand must have been written at least two instructions earlier.
template <int E>
__device__ __forceinline__ void mfma_acc(f32x16_t &acc, u32x4_t a, u32x4_t b) {
    if constexpr (E == ELT_F16)
        asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states for the result of matrix products the compiler does not see
// (mfma_acc, mfma_bagpr) before vector code reads or overwrites their
// registers: a 16-pass product needs 19 on this family, 32 leaves margin.
// (The scheduling barriers keep vector code from being moved above the wait:
// the asm only orders memory operations.)
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
// A shorter wait (n + 1 wait states, n = 0..7) for the same purpose, where the
// schedule already places other instructions in between.
template <int N>
__device__ __forceinline__ void mfma_wait() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop %0" ::"n"(N) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// acc (+)= A B with the B operand held in AGPRs (a fragment that only feeds
// matrix products) and the accumulator in VGPRs, where vector code reads it.
// As for mfma_acc, the compiler does not see the latency: a vector read of
// acc must come several products later (the callers' schedules place it at
// least two products after the last write).
template <int E>
__device__ __forceinline__ void mfma_bagpr(f32x16_t &acc, u32x4_t a, u32x4_t b) {
    if constexpr (E == ELT_F16)
        asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
// 16 bytes of global memory loaded straight into an AGPR tuple.  The load is
// still in flight when this returns: wait_agpr_loads must run before anything
// reads the result (it takes every such tuple as an operand, so no use can be
// placed ahead of it).
__device__ __forceinline__ u32x4_t load16_agpr(const void *p) {
    u32x4_t v;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=a"(v) : "v"(p) : "memory");
    return v;
}
// Wait for the loads of load16_agpr into the 16 tuples of f[2][8].
__device__ __forceinline__ void wait_agpr_loads(u32x4_t (&f)[2][8]) {
    asm volatile("s_waitcnt vmcnt(0)"
                 : "+a"(f[0][0]), "+a"(f[0][1]), "+a"(f[0][2]), "+a"(f[0][3]), "+a"(f[0][4]), "+a"(f[0][5]),
                   "+a"(f[0][6]), "+a"(f[0][7]), "+a"(f[1][0]), "+a"(f[1][1]), "+a"(f[1][2]), "+a"(f[1][3]),
                   "+a"(f[1][4]), "+a"(f[1][5]), "+a"(f[1][6]), "+a"(f[1][7])
                 :
                 : "memory");
}

// Sixteen 16-byte LDS reads straight into AGPRs: f[r][k] from byte address
// a[k] + 8192 r.  The wait for them sits in the same block, so the tuples hold
// their values when it returns and no VALU copy stands between them and the
// products that read them.
__device__ __forceinline__ void lds_read_agpr(u32x4_t (&f)[2][8], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b128 %0, %16\n\tds_read_b128 %1, %17\n\tds_read_b128 %2, %18\n\tds_read_b128 %3, %19\n\t"
        "ds_read_b128 %4, %20\n\tds_read_b128 %5, %21\n\tds_read_b128 %6, %22\n\tds_read_b128 %7, %23\n\t"
        "ds_read_b128 %8, %16 offset:8192\n\tds_read_b128 %9, %17 offset:8192\n\t"
        "ds_read_b128 %10, %18 offset:8192\n\tds_read_b128 %11, %19 offset:8192\n\t"
        "ds_read_b128 %12, %20 offset:8192\n\tds_read_b128 %13, %21 offset:8192\n\t"
        "ds_read_b128 %14, %22 offset:8192\n\tds_read_b128 %15, %23 offset:8192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=a"(f[0][0]), "=a"(f[0][1]), "=a"(f[0][2]), "=a"(f[0][3]), "=a"(f[0][4]), "=a"(f[0][5]), "=a"(f[0][6]),
          "=a"(f[0][7]), "=a"(f[1][0]), "=a"(f[1][1]), "=a"(f[1][2]), "=a"(f[1][3]), "=a"(f[1][4]), "=a"(f[1][5]),
          "=a"(f[1][6]), "=a"(f[1][7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}

// A fragment moved to AGPRs once, where mfma_bagpr reads it (the compiler
// would otherwise keep it in VGPRs and copy it over before every product).
__device__ __forceinline__ u32x4_t to_agpr(u32x4_t v) {
    uint32_t x0, x1, x2, x3;
    asm("v_accvgpr_write_b32 %0, %1" : "=a"(x0) : "v"(v[0]));
    asm("v_accvgpr_write_b32 %0, %1" : "=a"(x1) : "v"(v[1]));
    asm("v_accvgpr_write_b32 %0, %1" : "=a"(x2) : "v"(v[2]));
    asm("v_accvgpr_write_b32 %0, %1" : "=a"(x3) : "v"(v[3]));
    return u32x4_t{x0, x1, x2, x3};
}
template <int E>
__device__ __forceinline__ f32x16_t mfma_bagpr_first(u32x4_t a, u32x4_t b) {  // acc = A B
    f32x16_t d;
    if constexpr (E == ELT_F16)
        asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
    return d;
}

// Round-to-nearest-even packing of two floats (low half = a).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    f32x2_t x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    f32x2_t x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2_t));
}
template <int E>
__device__ __forceinline__ uint32_t pack_in(float a, float b) {
    if constexpr (E == ELT_F16) return pack_f16(a, b);
    else return pack_bf16(a, b);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t u) {
    return (float)__builtin_bit_cast(f16x2_t, u)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t u) {
    return (float)__builtin_bit_cast(f16x2_t, u)[1];
}

// Largest of three floats in one v_max3_f32.  The scores it takes are never
// NaN, so the quieting the compiler would add in front of fmaxf (the IEEE mode
// treats signalling NaNs specially) is left out.
__device__ __forceinline__ float max3(float a, float b, float c) {
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// Both halves' value combined: lanes l and l^32 exchange through
// v_permlane32_swap; the two results are {own, partner} in some order.
__device__ __forceinline__ float half_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Eight consecutive elements of an E-typed row as four 32-bit words of the
// 16-bit MFMA operand type (fp32 is rounded to bf16 on the way).
template <int E>
__device__ __forceinline__ u32x4_t load8_operand(const void *base, int64_t elem) {
    if constexpr (E == ELT_F32) {
        const f32x4_t *p = reinterpret_cast<const f32x4_t *>(static_cast<const float *>(base) + elem);
        f32x4_t a = p[0], b = p[1];
        return u32x4_t{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]),
                       pack_bf16(b[2], b[3])};
    } else {
        return *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(base) + elem);
    }
}

// Eight consecutive elements of an E-typed row as floats.  fp32 data is first
// rounded to bf16, the operand precision it is given everywhere else.
template <int E>
__device__ __forceinline__ void load8_float(const void *base, int64_t elem, float out[8]) {
    if constexpr (E == ELT_F32) {
        u32x4_t w = load8_operand<E>(base, elem);
#pragma unroll
        for (int i = 0; i < 4; ++i) { out[2 * i] = bf16_lo(w[i]); out[2 * i + 1] = bf16_hi(w[i]); }
    } else {
        u32x4_t w = *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(base) + elem);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (E == ELT_BF16) { out[2 * i] = bf16_lo(w[i]); out[2 * i + 1] = bf16_hi(w[i]); }
            else { out[2 * i] = f16_lo(w[i]); out[2 * i + 1] = f16_hi(w[i]); }
        }
    }
}

// Store four consecutive floats to an E-typed row (RNE for 16-bit types).
template <int E>
__device__ __forceinline__ void store4(void *base, int64_t elem, float a, float b, float c, float d) {
    if constexpr (E == ELT_F32) {
        *reinterpret_cast<f32x4_t *>(static_cast<float *>(base) + elem) = f32x4_t{a, b, c, d};
    } else if constexpr (E == ELT_BF16) {
        *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(base) + elem) = u32x2_t{pack_bf16(a, b), pack_bf16(c, d)};
    } else {
        *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(base) + elem) = u32x2_t{pack_f16(a, b), pack_f16(c, d)};
    }
}

// Row-major 16-bit LDS tile with rows of W elements: 16-byte chunk c of row r
// is stored at chunk c ^ swz<W>(r).  LDS has 64 four-byte banks (256 bytes).
// Two access shapes must spread over them:
//  * ds_read_b128 of one chunk from consecutive rows: swz is a bijection on
//    the low row bits (16 rows for W = 128, 8 for W = 64);
//  * ds_read_b64_tr_b16 of an 8-row x 64-byte block (rows r0 + 0..7, four
//    aligned chunks): the rows must cover all four 64-byte bank groups.  For
//    W = 128 a row is exactly 256 bytes, so the group is picked by swz bits 2-3
//    and these come from row & 3; for W = 64 two rows share the 256 bytes and
//    row & 1 selects the half, (row >> 1) & 1 the group inside it.
// (A swizzle that keeps the 8 rows in two bank groups halves the transposed
// read rate.)
template <int W>
__device__ __forceinline__ int swz(int row) {
    if constexpr (W / 8 >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    return ((row & 3) << 1) | ((row >> 2) & 1);
}

// Element offset of (row, col) in such a tile; col must be a multiple of 4.
template <int W>
__device__ __forceinline__ int tile_off(int row, int col) {
    return row * W + (((col >> 3) ^ swz<W>(row)) << 3) + (col & 7);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives
// halfword (i % 4) of the 8-byte chunks addressed by lanes i/4, i/4 + 4,
// i/4 + 8 and i/4 + 12 of its group, in that order.
__device__ __forceinline__ u32x2_t ds_read_tr16(const uint16_t *p) {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)p);
    return __builtin_bit_cast(u32x2_t, v);
}

// MFMA A operand holding T^T, read transposed from a row-major swizzled LDS
// tile T[k][m] (rows of W elements): lane l gets m = m0 + l%32 and the k
// slots v = 0..3 -> row r0 + 4g + v, v = 4..7 -> row r0 + 8 + 4g + (v-4),
// g = l/32 -- the row order of a 32x32 accumulator's registers 8h..8h+7.
template <int W>
__device__ __forceinline__ u32x4_t tr_operand(const uint16_t *T, int r0, int m0, int lane) {
    const int j = lane & 15, g = lane >> 5;
    const int col = m0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
    const int row = r0 + 4 * g + (j >> 2);
    const u32x2_t a = ds_read_tr16(T + tile_off<W>(row, col));
    const u32x2_t b = ds_read_tr16(T + tile_off<W>(row + 8, col));
    return u32x4_t{a[0], a[1], b[0], b[1]};
}

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N - 1>{}),
// in order: a loop whose index is a compile-time constant in every copy.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// An empty statement with a side effect: placed in a rarely taken uniform
// branch it stops the compiler from flattening the branch into per-element
// selects that would then run on every tile.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Wait until every vector-memory operation of this wave has completed,
// including global -> LDS copies (which the compiler does not track).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Copy rows [row0, row0 + R) of a row-major 16-bit global matrix with rows of
// W elements into an LDS tile in tile_off<W> layout, using
// global_load_lds_dwordx4: one wave instruction fills 1 KiB of LDS, lane l
// the 16 bytes at 16*l, so each lane fetches the global chunk that the
// swizzle places there.  Rows at or past `nrows` re-read row nrows-1 (finite
// data; callers give such rows zero weight).  Blocks are spread over the
// NWAVES waves of the workgroup.  Completion: wait_vmem() then a barrier.
template <int W, int R, int NWAVES>
__device__ __forceinline__ void dma_tile(const void *g, int row0, int nrows, uint16_t *lds, int wave, int lane) {
    constexpr int RPB = 512 / W;  // rows per 1 KiB block
    constexpr int NBLK = R / RPB;
    static_assert(R % RPB == 0, "tile rows must fill whole 1 KiB blocks");
    const int r_in = lane / (W / 8), p = lane % (W / 8);
#pragma unroll
    for (int j = 0; j < (NBLK + NWAVES - 1) / NWAVES; ++j) {
        const int b = wave + j * NWAVES;
        if (NBLK % NWAVES != 0 && b >= NBLK) break;
        const int r = b * RPB + r_in;
        const int c = p ^ swz<W>(r);
        int grow = row0 + r;
        grow = grow < nrows ? grow : nrows - 1;
        const uint16_t *src = static_cast<const uint16_t *>(g) + (int64_t)grow * W + c * 8;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)(lds + b * 512), 16, 0, 0);
    }
}

// ---- attention dropout (inverted dropout on P, the mask drawn again in the
// backward).  The generator is Philox4x32 with 10 rounds from Salmon, Moraes,
// Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011):
// per round, counter words 0 and 2 are multiplied by two fixed odd constants,
// the high product halves are XORed with the other two words and the key,
// the low halves carried over; the key moves by two Weyl increments between
// rounds.  Element (bh, query i, key j) is decided by byte j % 4 (least
// significant first) of word i % 4 of the output for counter
// (j / 4, i / 4, bh, 0) and key (seed low, seed high): dropped when the byte
// is below t (rate t / 256).  Parameters: struct Dropout (fa_types.hpp).
__device__ __forceinline__ u32x4_t philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
    constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;    // multipliers of words 0 and 2
    constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;  // key increments
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t hiA = __umulhi(kMulA, c0), loA = kMulA * c0;
        const uint32_t hiB = __umulhi(kMulB, c2), loB = kMulB * c2;
        c0 = hiB ^ c1 ^ k0;
        c1 = loB;
        c2 = hiA ^ c3 ^ k1;
        c3 = loA;
        k0 += kWeylA;
        k1 += kWeylB;
    }
    return u32x4_t{c0, c1, c2, c3};
}

// Bit e set: byte e of w is below t, i.e. that element is dropped.  Bytes 0/2
// and 1/3 go through a packed 16-bit subtraction; the sign bit of byte - t is
// set exactly when byte < t (both in 0..255).  t2 = t | t << 16.
__device__ __forceinline__ uint32_t dropped_bytes(uint32_t w, uint32_t t2) {
    typedef short s16x2_t __attribute__((ext_vector_type(2)));
    const uint32_t dl = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2_t, w & 0x00ff00ffu) -
                                                         __builtin_bit_cast(s16x2_t, t2));
    const uint32_t dh = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2_t, (w >> 8) & 0x00ff00ffu) -
                                                         __builtin_bit_cast(s16x2_t, t2));
    return ((dl >> 15) & 1u) | ((dh >> 14) & 2u) | ((dl >> 29) & 4u) | ((dh >> 28) & 8u);
}

// x from lane (this lane ^ s) of the same quad (s = 1, 2, 3; DPP quad permutation).
template <int S>
__device__ __forceinline__ uint32_t quad_xor(uint32_t x) {
    constexpr int ctrl = S == 1 ? 0xB1 : S == 2 ? 0x4E : 0x1B;  // [1,0,3,2] [2,3,0,1] [3,2,1,0]
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, ctrl, 0xF, 0xF, false);
}

// The four lanes of a quad hold four consecutive queries (or keys) and need the
// same four generator calls of a 16-query x 4-key (or 4-query x 16-key) strip;
// lane w evaluates call w alone and the keep flags travel through three quad
// exchanges.  `packed` holds, for each of the quad's lanes w', a nibble at bits
// 4w' .. 4w'+3; the result gathers nibble (this lane) of lane (this lane ^ s)
// into bits 4(this lane ^ s) .. +3.
__device__ __forceinline__ uint32_t quad_gather_nibbles(uint32_t packed, uint32_t w) {
    const uint32_t sh = 4u * w;
    uint32_t keep = ((packed >> sh) & 0xfu) << sh;
    keep |= ((quad_xor<1>(packed) >> sh) & 0xfu) << (4u * (w ^ 1u));
    keep |= ((quad_xor<2>(packed) >> sh) & 0xfu) << (4u * (w ^ 2u));
    keep |= ((quad_xor<3>(packed) >> sh) & 0xfu) << (4u * (w ^ 3u));
    return keep;
}

// Keep flags of a lane that owns query q (q % 4 == lane % 4) for the 16 keys
// kbase + 8 rq + e (rq, e = 0..3; kbase % 4 == 0): bit 4 rq + e.
__device__ __forceinline__ uint32_t dropout_keep_query_lane(const Dropout &dr, uint32_t bh, uint32_t q, uint32_t kbase,
                                                            int lane) {
    const uint32_t w = (uint32_t)lane & 3u, t2 = dr.t | (dr.t << 16);
    const u32x4_t out = philox4x32_10((kbase + 8u * w) >> 2, q >> 2, bh, 0u, dr.k0, dr.k1);  // key group rq = w
    uint32_t packed = 0;  // nibble i: keep flags of the group's 4 keys for query 4(q/4) + i
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= (~dropped_bytes(out[i], t2) & 0xfu) << (4 * i);
    return quad_gather_nibbles(packed, w);
}

// Keep flags of a lane that owns key j (j % 4 == lane % 4) for the 16 queries
// qbase + 8 rq + i (rq, i = 0..3; qbase % 4 == 0): bit 4 rq + i.
__device__ __forceinline__ uint32_t dropout_keep_key_lane(const Dropout &dr, uint32_t bh, uint32_t qbase, uint32_t j,
                                                          int lane) {
    const uint32_t w = (uint32_t)lane & 3u, t2 = dr.t | (dr.t << 16);
    const u32x4_t out = philox4x32_10(j >> 2, (qbase + 8u * w) >> 2, bh, 0u, dr.k0, dr.k1);  // query group rq = w
    uint32_t packed = 0;  // nibble e: keep flags of the group's 4 queries for key 4(j/4) + e
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t kept = ~dropped_bytes(out[i], t2);  // bit e: key e kept for query i
#pragma unroll
        for (int e = 0; e < 4; ++e) packed |= ((kept >> e) & 1u) << (4 * e + i);
    }
    return quad_gather_nibbles(packed, w);
}

// Map a hardware workgroup index to a logical one so that consecutive
// logical indices land on the same XCD.  Workgroups are handed to the eight
// XCDs round-robin; this is a bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int p, int n) {
    const int per = n / 8, rem = n % 8;
    const int xcd = p % 8, slot = p / 8;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

}  // namespace fa
