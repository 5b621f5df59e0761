// Device helpers shared by the gfx950 kernels of libgdn: vector types, bf16
// conversion and hi/lo splitting, and 16x16 MFMA tile products.
//
// MFMA lane layouts used throughout (wave64, gfx950):
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) + e] and
//     B[8*(l/16) + e][l%16] for e < 8; the accumulator holds
//     D[4*(l/16) + e][l%16] for e < 4.
//   v_mfma_f32_16x16x16_bf16: lane l holds A[l%16][4*(l/16) + e] and
//     B[4*(l/16) + e][l%16] for e < 4 (used for a k remainder of 16);
//     same accumulator layout.
//   v_mfma_f32_16x16x4_f32:   lane l holds A[l%16][l/16] and B[l/16][l%16];
//     same accumulator layout.
// Every operand buffer is stored "k-contiguous": A as [row][k] and B as
// [col][k], so one lane's 8 bf16 values are one 16-byte LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

struct alignas(16) U16x8 { u16 v[8]; };

__device__ __forceinline__ u16 bf16_bits(float x) {
    __bf16 h = (__bf16)x;                    // round to nearest even
    return __builtin_bit_cast(u16, h);
}
__device__ __forceinline__ float bf16_to_f32(u16 b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi); x - hi is exact in fp32.
__device__ __forceinline__ void split_bf16(float x, u16 &hi, u16 &lo) {
    hi = bf16_bits(x);
    lo = bf16_bits(x - bf16_to_f32(hi));
}

// Two floats to two bf16 (round to nearest even) in one 32-bit word, low
// half first: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt2_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, bf16x2));
}
// Packed split of two floats: hi = bf16 pair, lo = bf16 pair of the residuals.
__device__ __forceinline__ void split2_bf16(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = cvt2_bf16(a, b);
    lo = cvt2_bf16(a - __builtin_bit_cast(float, hi << 16), b - __builtin_bit_cast(float, hi & 0xffff0000u));
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i reads 4 bf16 D_i[0..3] at its own 8-byte address; lane j
// receives {D_{4e + j/4}[j % 4] : e = 0..3}.  So if lane i of a group points
// at row r0 + i/4, columns c0 + 4*(i%4) of a row-major matrix M, lane j gets
// the column c0 + j, rows r0 .. r0+3: M^T read as an MFMA operand fragment.
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
__device__ __forceinline__ shortx4 ld_tr16(const u16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p));
}

// x + (x from lane l ^ 16), x + (x from lane l ^ 32), in registers: gfx950's
// permlane swaps exchange 16-lane rows 0 <-> 1 and 2 <-> 3 (the 32-lane
// halves) between their two operands; with both operands x, every lane ends
// up with its own value in one result and its partner's in the other.  (The
// two results are copied out to plain variables before use.)
__device__ __forceinline__ float add_xor16(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned a0 = r[0], a1 = r[1];
    return __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
}
__device__ __forceinline__ float add_xor32(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned a0 = r[0], a1 = r[1];
    return __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations (lgkmcnt(0)) but leaves its global loads and stores in flight
// (vmcnt and expcnt at their maxima), unlike __syncthreads(), which also
// waits for every outstanding global operation.  The empty asm statements
// keep the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);     // vmcnt(63) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---- bf16 tile products ---------------------------------------------------
// acc += A(16 x kdim) * B(kdim x 16); A at `a` with row stride lda (elements),
// B stored transposed at `b` ([col][k]) with row stride ldb.  kdim % 16 == 0:
// 32-wide steps, then one 16-wide step for a remainder of 16.
__device__ __forceinline__ bf16x8 ld8(const u16 *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const U16x8 *>(p));
}
__device__ __forceinline__ shortx4 ld4(const u16 *p) {
    return *reinterpret_cast<const shortx4 *>(p);
}

// Split operands: (ahi + alo)(bhi + blo) ~= ahi bhi + ahi blo + alo bhi.
// A null `alo` or `blo` means that operand is exact in bf16.
__device__ __forceinline__ void mma_bf16_split(floatx4 &acc, const u16 *ahi, const u16 *alo, int lda,
                                               const u16 *bhi, const u16 *blo, int ldb, int kdim) {
    const int l = lane_id();
    const int ra = (l & 15) * lda, rb = (l & 15) * ldb;
    int kk = 0;
    for (; kk + 32 <= kdim; kk += 32) {
        const int oa = ra + kk + 8 * (l >> 4), ob = rb + kk + 8 * (l >> 4);
        bf16x8 ah = ld8(ahi + oa), bh = ld8(bhi + ob);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        if (blo) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, ld8(blo + ob), acc, 0, 0, 0);
        if (alo) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld8(alo + oa), bh, acc, 0, 0, 0);
    }
    if (kk < kdim) {
        const int oa = ra + kk + 4 * (l >> 4), ob = rb + kk + 4 * (l >> 4);
        shortx4 ah = ld4(ahi + oa), bh = ld4(bhi + ob);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
        if (blo) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, ld4(blo + ob), acc, 0, 0, 0);
        if (alo) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ld4(alo + oa), bh, acc, 0, 0, 0);
    }
}

__device__ __forceinline__ void mma_bf16(floatx4 &acc, const u16 *a, int lda, const u16 *b, int ldb,
                                         int kdim) {
    mma_bf16_split(acc, a, nullptr, lda, b, nullptr, ldb, kdim);
}

// acc += A * (bhi + blo) with A exact in bf16 and stored transposed
// ([k][row], stride lda): each lane gathers its 8 A values one by one.
__device__ __forceinline__ void mma_bf16_at_split(floatx4 &acc, const u16 *a, int lda, const u16 *bhi,
                                                  const u16 *blo, int ldb, int kdim) {
    const int l = lane_id();
    const int rb = (l & 15) * ldb;
    int kk = 0;
    for (; kk + 32 <= kdim; kk += 32) {
        const u16 *pa = a + (kk + 8 * (l >> 4)) * lda + (l & 15);
        U16x8 av;
#pragma unroll
        for (int e = 0; e < 8; ++e) av.v[e] = pa[e * lda];
        const bf16x8 ah = __builtin_bit_cast(bf16x8, av);
        const int ob = rb + kk + 8 * (l >> 4);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, ld8(bhi + ob), acc, 0, 0, 0);
        if (blo) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, ld8(blo + ob), acc, 0, 0, 0);
    }
    if (kk < kdim) {
        const u16 *pa = a + (kk + 4 * (l >> 4)) * lda + (l & 15);
        shortx4 ah;
#pragma unroll
        for (int e = 0; e < 4; ++e) ah[e] = (short)pa[e * lda];
        const int ob = rb + kk + 4 * (l >> 4);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, ld4(bhi + ob), acc, 0, 0, 0);
        if (blo) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, ld4(blo + ob), acc, 0, 0, 0);
    }
}

// ---- fp32 tile products ---------------------------------------------------
// acc += A(16 x kdim) * B(kdim x 16), A [row][k] stride lda, B [col][k]
// stride ldb, fp32, kdim % 4 == 0.
__device__ __forceinline__ void mma_f32(floatx4 &acc, const float *a, int lda, const float *b, int ldb,
                                        int kdim) {
    const int l = lane_id();
    const float *pa = a + (l & 15) * lda + (l >> 4);
    const float *pb = b + (l & 15) * ldb + (l >> 4);
    for (int kk = 0; kk < kdim; kk += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[kk], pb[kk], acc, 0, 0, 0);
}

// hi and lo bf16 of 4 consecutive values (a 16-deep MFMA operand)
__device__ __forceinline__ void split4(const floatx4 &x, shortx4 &hi, shortx4 &lo) {
    uint2 h, o;
    split2_bf16(x[0], x[1], h.x, o.x);
    split2_bf16(x[2], x[3], h.y, o.y);
    hi = __builtin_bit_cast(shortx4, h);
    lo = __builtin_bit_cast(shortx4, o);
}

// 16x16 MFMA steps of 32 (bf16x8 operands) and 16 (4 x bf16) k values
__device__ __forceinline__ floatx4 mfma32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(shortx4 a, shortx4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// bf16 fragment of two accumulator tiles, in the permuted order (hi only).
__device__ __forceinline__ bf16x8 frag_hi(const floatx4 &t0, const floatx4 &t1) {
    return __builtin_bit_cast(bf16x8, uint4{cvt2_bf16(t0[0], t0[1]), cvt2_bf16(t0[2], t0[3]),
                                            cvt2_bf16(t1[0], t1[1]), cvt2_bf16(t1[2], t1[3])});
}
// hi and lo fragments of two accumulator tiles (permuted order), or of 8
// consecutive values (natural order).
__device__ __forceinline__ void frag_split(const floatx4 &t0, const floatx4 &t1, bf16x8 &hi, bf16x8 &lo) {
    uint4 h, o;
    split2_bf16(t0[0], t0[1], h.x, o.x);
    split2_bf16(t0[2], t0[3], h.y, o.y);
    split2_bf16(t1[0], t1[1], h.z, o.z);
    split2_bf16(t1[2], t1[3], h.w, o.w);
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, o);
}

// acc += A * B with B stored row-major ([k][col], stride ldb).
__device__ __forceinline__ void mma_f32_bn(floatx4 &acc, const float *a, int lda, const float *b, int ldb,
                                           int kdim) {
    const int l = lane_id();
    const float *pa = a + (l & 15) * lda + (l >> 4);
    const float *pb = b + (l >> 4) * ldb + (l & 15);
    for (int kk = 0; kk < kdim; kk += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[kk], pb[kk * ldb], acc, 0, 0, 0);
}

}  // namespace gdn
