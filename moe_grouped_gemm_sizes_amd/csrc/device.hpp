// device.hpp -- gfx950 building blocks shared by the grouped-GEMM kernels.
//
// Everything here targets CDNA4 (gfx950) directly:
//   - MFMA 16x16x32 bf16 and 16x16x128 f8f6f4 (e4m3 operands, unit block
//     scales, so the hardware scale is 2^0).
//   - LDS transpose reads ds_read_b64_tr_b8 / _b16 for operands whose
//     reduction axis is strided in memory.
//   - Buffer loads straight into LDS (buffer_load_dwordx4 ... lds).  The
//     buffer resource's byte range clamps every access, so reads past a
//     tile's valid rows return zeros and never touch memory.
//
// Lane layouts, measured on gfx950 with small-integer operands:
//   MFMA 16x16xK:  A operand lane l -> row l%16, k-slot group l/16;
//                  B operand lane l -> col l%16, same k-slot groups;
//                  D lane l -> col l%16, rows 4*(l/16) + v for v = 0..3.
//   ds_read_b64_tr_b8:  within each 16-lane group, lane t = 8h+i receives
//                  byte i of the 8-byte chunk addressed by lane 2v+h, v = 0..7.
//   ds_read_b64_tr_b16: within each 16-lane group, lane t = 4h+i receives
//                  element i of the 8-byte chunk addressed by lane 4v+h, v = 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moegg {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

#define MOEGG_LDS __attribute__((address_space(3)))

// ----------------------------------------------------------------- buffers

// Raw buffer resource over [base, base + bytes).  Accesses at or past
// `bytes` read as zero and writes there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes from rsrc+voffset into LDS at lds_base + 16 * lane.
// lds_base must be wave-uniform.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t voffset, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MOEGG_LDS void*)lds_base, 16, voffset, 0, 0, 0);
}


// Same, with a wave-uniform scalar offset added to the address.  The range
// check counts soffset as well (measured on gfx950: a load whose step offset
// sat in soffset past a one-row resource read zeros), so a resource must span
// every step's bytes; rows past the valid ones are masked through voffset.
__device__ __forceinline__ void load16_to_lds_so(__amdgpu_buffer_rsrc_t rs, uint32_t voffset, uint32_t soffset,
                                                 void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MOEGG_LDS void*)lds_base, 16, voffset, soffset, 0, 0);
}

// load16_to_lds_so with a cache-policy immediate: CP_NT (non-temporal) marks
// data read once -- a weight panel no other tile will read again -- so that
// it streams instead of holding lines the other operands reuse.  Measured on
// the decode workload, its weight stream runs 1.35x faster with it (bf16
// weights: 208 -> 154 us; e4m3: 138 -> 92 us); where panels are shared by
// several tiles it costs (17 % on the fp8 GEMM's full tiles).
constexpr int CP_DEFAULT = 0, CP_NT = 2;
template <int CP>
__device__ __forceinline__ void load16_to_lds_cp(__amdgpu_buffer_rsrc_t rs, uint32_t voffset, uint32_t soffset,
                                                 void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MOEGG_LDS void*)lds_base, 16, voffset, soffset, 0, CP);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ----------------------------------------------------------------- LDS reads

__device__ __forceinline__ v4i lds_read_b128(const void* p) {
    return *(const MOEGG_LDS v4i*)(p);
}

__device__ __forceinline__ v2i lds_read_tr8(const void* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((MOEGG_LDS v2i*)(p));
}

__device__ __forceinline__ v2i lds_read_tr16(const void* p) {
    v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOEGG_LDS v4s*)(p));
    return __builtin_bit_cast(v2i, r);
}

// ----------------------------------------------------------------- MFMA

// D = A * B + C for 16x16x128 e4m3 operands (32 bytes per lane each).
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// D = A * B + C for 16x16x32 bf16 operands (16 bytes per lane each).
__device__ __forceinline__ v4f mfma_bf16(v4i a, v4i b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                   0, 0, 0);
}

// ----------------------------------------------------------------- conversion

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

}  // namespace moegg
