// device.h -- small gfx950 building blocks shared by the HIP kernels: vector
// types, 16-bit element traits, MFMA wrappers, the LDS transpose read and
// wavefront exchanges.  Nothing here is attention-specific.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Buffer resource word 3 for raw (untyped) buffer access on gfx950.  A buffer load
// past the descriptor's num_records returns zero without a memory access.
constexpr int kBufferRsrcWord3 = 0x00020000;

// ---------------------------------------------------------------- 16-bit types

template <typename T> struct Elem;

template <> struct Elem<__bf16> {
    typedef bf16x8 vec8;
    static __device__ __forceinline__ float to_float(uint16_t h) {
        return __uint_as_float((uint32_t)h << 16);
    }
    // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    static __device__ __forceinline__ uint16_t from_float(float f) {
        return __builtin_bit_cast(uint16_t, (__bf16)f);
    }
    // two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
    static __device__ __forceinline__ uint32_t pack2(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    }
    // acc + the two bf16 values of a packed pair (one v_dot2_f32_bf16 against 1, 1)
    static __device__ __forceinline__ float sum2(uint32_t packed, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                               bf16x2{(__bf16)1.f, (__bf16)1.f}, acc, false);
    }
    // 32x32x16: A [32 x 16], B [16 x 32], 8 elements per lane each
    static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // 16x16x32: A [16 x 32], B [32 x 16]
    static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Elem<_Float16> {
    typedef f16x8 vec8;
    static __device__ __forceinline__ float to_float(uint16_t h) {
        return (float)__builtin_bit_cast(_Float16, h);
    }
    static __device__ __forceinline__ uint16_t from_float(float f) {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    }
    // acc + the two fp16 values of a packed pair (one v_dot2_f32_f16 against 1, 1)
    static __device__ __forceinline__ float sum2(uint32_t packed, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed),
                                      f16x2{(_Float16)1.f, (_Float16)1.f}, acc, false);
    }
    static __device__ __forceinline__ f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <typename T>
__device__ __forceinline__ typename Elem<T>::vec8 as_vec8(u32x4 raw) {
    return __builtin_bit_cast(typename Elem<T>::vec8, raw);
}

// ------------------------------------------------------------------- memory

__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}
// Streaming load for data read exactly once (the nontemporal hint sets the load's
// nt bit): on MI355X a plain read stream reaches ~6.3 TB/s and a nontemporal one
// ~7.0 TB/s (microbench/ceilings.hip).
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane j
// names 8 bytes (four 16-bit elements E[j][0..3]); lane i of the group receives
// { E[4e + i/4][i % 4] : e = 0..3 }.  Measured on gfx950 with a lane/element
// probe.  `p` must point into LDS (8-byte aligned).
__device__ __forceinline__ u32x2 lds_read_tr16(void* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// ------------------------------------------------------------ wave exchanges

__device__ __forceinline__ float xor_shfl(float x, int mask) {
    return __shfl_xor(x, mask, 64);
}

// Max and sum of x over the lane pair (l, l ^ 32), in VALU (v_permlane32_swap): no
// LDS round trip, unlike a cross-lane shuffle.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Wait for outstanding LDS operations of this wave (s_waitcnt lgkmcnt(0)) and keep
// the compiler from moving LDS accesses across this point.
__device__ __forceinline__ void lds_wave_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
}

}  // namespace skv
