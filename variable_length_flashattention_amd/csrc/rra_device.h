// Device-side helpers shared by the gfx950 kernels of librra.
// Wave64 only.  MFMA operand layouts used below (checked on gfx950):
//   v_mfma_f32_32x32x16_bf16: A lane l holds row l%32, k = 8*(l/32)+e (e<8);
//     B lane l holds col l%32, same k; C reg r of lane l is
//     row 8*(r/4) + 4*(l/32) + r%4, col l%32.
//   v_mfma_f32_16x16x32_bf16: A row l%16, k = 8*(l/16)+e; B col l%16, same k;
//     C reg r is row 4*(l/16)+r, col l%16.
//   v_mfma_f32_16x16x16_bf16 (1k): as 16x16x32 with 4 k-elements per lane.
//   ds_read_b64_tr_b16: within each 16-lane group, lane j supplies the address
//     of 4 consecutive b16 in "row" j/4, columns 4*(j%4)..+3 of a 4x16 tile;
//     lane i of the group receives column i, rows 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rra {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// The same as a streaming load: the non-temporal hint, for data read once
// (the decode's K/V rows), so that it does not displace reused lines from
// the caches.
__device__ __forceinline__ u32x4 load16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Round two floats to bf16 (nearest-even) and pack lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __attribute__((ext_vector_type(2))) float f2;
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
    f2 v = {lo, hi};
    b2 r = __builtin_convertvector(v, b2);
    return __builtin_bit_cast(uint32_t, r);
}
// lo + hi of a packed bf16 pair, added to acc in fp32 (one v_dot2_f32_bf16
// against (1, 1); the products are exact).
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, pair), __builtin_bit_cast(b2, 0x3F803F80u), acc,
                                           false);
}
// The two floats a packed bf16 pair represents.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations are outstanding and leaves the other counters alone.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Raw buffer descriptor over `base` (byte addressing, no stride, 2^31-1 bytes
// in range; the data-format field is the one the CDNA buffer loads expect).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}
// 16 bytes per lane from buffer `r` at byte offset voff + soff straight into
// LDS: lane l writes lds + 16*l (lds is wave-uniform).
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff, int32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// 4 bytes per lane from buffer `r` at byte offset voff + soff straight into
// LDS: lane l writes lds + 4*l (lds is wave-uniform).
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff, int32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff, soff, 0, 0);
}

// max of three floats in one instruction.  Operands are finite or -inf here,
// so the NaN canonicalisation the compiler would add around fmaxf is not needed.
__device__ __forceinline__ float max3f(float a, float b, float c)
{
    float r;
    __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Values of lanes l and l^32 combined (both halves get the result).
__device__ __forceinline__ float max_across_halves(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                              false, false);
    const float a = __builtin_bit_cast(float, (uint32_t)p[0]), b = __builtin_bit_cast(float, (uint32_t)p[1]);
    return max3f(a, b, b);
}
__device__ __forceinline__ float sum_across_halves(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                              false, false);
    return __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
}

__device__ __forceinline__ int wave_sum_i32(int x)
{
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
__device__ __forceinline__ int64_t wave_sum_i64(int64_t x)
{
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
__device__ __forceinline__ int wave_max_i32(int x)
{
    for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
    return x;
}

}  // namespace rra
