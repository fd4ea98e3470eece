// attn_common.h -- device helpers shared by the bf16 attention kernels
// (internal to libhd.so).
#pragma once

#include "hd_internal.h"

namespace hd {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Direct-to-LDS 16-byte load: lane l's 16 bytes from gptr land at LDS byte
// address lds_base + 16*l.  Issued as a two-instruction asm block (M0 holds
// the wave-uniform LDS base) so that the compiler's wait-count pass does not
// treat the in-flight copy into one buffer as aliasing the transposed reads of
// the other buffer; the kernel waits for it explicitly (vmcnt(0) + barrier)
// before the tile is read.  No other code in these kernels uses M0.
__device__ __forceinline__ void lds_dma16(const void *gptr, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gptr)
                 : "memory", "m0");
}

// Same copy from a wave-uniform base (scalar registers) plus a 32-bit per-lane
// byte offset (no 64-bit address arithmetic per lane).
__device__ __forceinline__ void lds_dma16_s(const void *base, unsigned voff, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(base)
                 : "memory", "m0");
}

// Direct-to-LDS 4-byte load: lane l's dword from base + voff lands at LDS
// byte address lds_base + 4*l (same conventions as lds_dma16_s).
__device__ __forceinline__ void lds_dma4_s(const void *base, unsigned voff, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_base), "v"(voff), "s"(base)
                 : "memory", "m0");
}

__device__ __forceinline__ unsigned lds_addr(const char *p) {
    return (unsigned)(size_t)((__attribute__((address_space(3))) const char *)p);
}

constexpr bf16x2 kOnes2 = {(bf16)1.0f, (bf16)1.0f};

__device__ __forceinline__ int swz128(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// Swizzle of V tiles read with ds_read_b64_tr_b16: a 32-lane group reads 4
// consecutive rows x 4 consecutive 16-byte chunks; XOR-ing row r's chunk index
// with 4*(r%4) + (r/4)%4 puts the four rows in four different 64-byte quarters
// of the 256-byte bank window (and is a permutation over any 16 rows).
__device__ __forceinline__ int swzv(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Rotary embedding (rotate-half) of a query row held as MFMA operands: lane
// half hi holds dims 16*ks + 8*hi + e (e < 8) in qop[ks]; dim c pairs with
// c + D/2, i.e. k-step ks with ks + D/32 of the same lane.  The angle pos*f_c
// is taken in turns (ft[c] = f_c / 2 pi), reduced to [-1/2, 1/2] in double
// and fed to the hardware sine / cosine, whose input is in turns.  ft is read
// at lane-uniform indices only (both halves' entries, then a select).
template <int D>
__device__ __forceinline__ void rope_rotate_q(bf16x8 (&qop)[D / 16], int64_t pos, const double *ft, int hi) {
    constexpr int KH = D / 32;
    const double dpos = (double)pos;
#pragma unroll
    for (int ks = 0; ks < KH; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double f = hi ? ft[16 * ks + 8 + e] : ft[16 * ks + e];
            const double turns = dpos * f;
            const float red = (float)(turns - rint(turns));
            const float sn = __builtin_amdgcn_sinf(red), cs = __builtin_amdgcn_cosf(red);
            const float x0 = (float)qop[ks][e], x1 = (float)qop[ks + KH][e];
            qop[ks][e] = (bf16)(x0 * cs - x1 * sn);
            qop[ks + KH][e] = (bf16)(x1 * cs + x0 * sn);
        }
}

__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// One ds_read_b64_tr_b16 from an LDS address.
__device__ __forceinline__ s16x4 lds_read_tr16(const char *addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(addr));
}

}  // namespace hd
