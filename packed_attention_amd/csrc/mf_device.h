// Device-side helpers for the gfx950 kernels of libmf.so: vector types,
// bf16 <-> fp32 conversion and wavefront (64-lane) reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// 16-byte global load/store of 8 bf16 values held as 4 packed dwords.
__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st16(uint16_t* p, u32x4_t v) {
    *reinterpret_cast<u32x4_t*>(p) = v;
}

// Raw buffer resource over [base, base + bytes): a buffer load whose offset
// falls outside the range returns zeros instead of touching memory, which
// lets ragged tiles load without branches.  The range is clamped to 4 GiB-1,
// so every in-range offset is an address inside the caller's tensor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : uint32_t(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// 16-byte store through a buffer resource; stores whose offset falls
// outside the resource's range are dropped.
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, u32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                          r, voff, soff, 0);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane
// group, lane j points at a row of 4 consecutive 16-bit elements; lane i
// receives element i%4 of the rows pointed at by lanes i/4, 4+i/4, 8+i/4 and
// 12+i/4 (in that order).
__device__ __forceinline__ s16x4_t lds_read_tr16_b64(const void* p) {
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Direct global->LDS load of 16 bytes per lane through a buffer resource:
// lane i's bytes land at lds + 16*i (lds must be the same for the whole
// wavefront); out-of-range offsets deposit zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 16, voff,
                                             soff, 0, 0);
}

// Exact widening of the two bf16 halves of a dword.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Unpack 8 bf16 (4 dwords) to fp32, element order preserved.
__device__ __forceinline__ void unpack8(u32x4_t v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf_lo(v[i]);
        f[2 * i + 1] = bf_hi(v[i]);
    }
}

// Round two fp32 values to bf16 (round-to-nearest-even, v_cvt_pk_bf16_f32)
// and pack them into one dword, `a` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t v = {a, b};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4_t pack8(const float* f) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return r;
}

// DPP lane permutation within rows of 16 lanes (all rows and banks enabled).
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wavefront; every lane receives the same total
// (bitwise: each step adds two values in an order-independent way).  A
// butterfly inside each row of 16 lanes with DPP (swap neighbours, swap
// pairs, mirror within 8, mirror within 16), then v_permlane16_swap adds row
// pairs and v_permlane32_swap the two halves: eight VALU instructions, no
// LDS traffic.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

}  // namespace mf
