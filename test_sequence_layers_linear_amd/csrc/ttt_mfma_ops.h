// ttt_mfma_ops.h -- bf16 MFMA operand helpers for the d = 64 kernels on
// gfx950 (16x16 tiles; lane l, c = l % 16, g = l / 16):
//   C/D tile    : lane holds rows 4g..4g+3 of column c.
//   A operand   : lane holds row c, k-slots of group g.
//   B operand   : lane holds column c, k-slots of group g.
#pragma once

#include "ttt_internal.h"

namespace ttt {
namespace mfma {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format)
constexpr int kBufferDword3 = 0x00020000;
// bytes of one 64-element bf16 row
constexpr int kRowBytes = 128;
// cache-policy operand of a buffer load or store on gfx950: non-temporal
constexpr int kNonTemporal = 2;

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// A 16x16x16 product whose result feeds a 16x16x32 product as the
// accumulator (or the reverse) needs more wait states between the two than
// the compiler inserts; such products are issued as 16x16x32 with the upper
// four k-slots zero, so that every accumulation chain has one shape.
__device__ __forceinline__ f32x4 mfma16_as32(bf16x4 a, bf16x4 b, f32x4 c)
{
    const u32x2 aw = __builtin_bit_cast(u32x2, a), bw = __builtin_bit_cast(u32x2, b);
    return mfma32(__builtin_bit_cast(bf16x8, u32x4{aw[0], aw[1], 0u, 0u}),
                  __builtin_bit_cast(bf16x8, u32x4{bw[0], bw[1], 0u, 0u}), c);
}

// fp32 -> bf16 (round to nearest even), two values per conversion
__device__ __forceinline__ uint32_t cvt2(float a, float b)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi)
{
    return __builtin_bit_cast(bf16x8, u32x4{cvt2(lo[0], lo[1]), cvt2(lo[2], lo[3]),
                                            cvt2(hi[0], hi[1]), cvt2(hi[2], hi[3])});
}

__device__ __forceinline__ bf16x4 pack4(f32x4 x)
{
    return __builtin_bit_cast(bf16x4, u32x2{cvt2(x[0], x[1]), cvt2(x[2], x[3])});
}

// bf16 bits -> fp32, eight values of a 16-byte segment
__device__ __forceinline__ void unpack8(u32x4 x, float (&f)[8])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(x[e] << 16);
        f[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
    }
}

// Row numbering of a 64-row fp32 accumulator kept as four 16-row tiles: row
// m of tile mt is input index rho(mt, m), so that the registers of tiles 2s
// and 2s + 1, rounded to bf16, are the B operand of a 16x16x32 product over
// the inputs [32s, 32s + 32) with k-slot (g, e) <-> 32s + 8g + e.
__device__ __forceinline__ int rho(int mt, int m)
{
    return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives, as
// element k (k = 0..3), element i % 4 of the 8-byte block addressed by lane
// 4k + i / 4 of its group.
__device__ __forceinline__ bf16x4 read_tr16(const unsigned char* p)
{
    typedef __bf16 lds_bf16x4 __attribute__((ext_vector_type(4)));
    const auto q = (__attribute__((address_space(3))) lds_bf16x4*)(
        (__attribute__((address_space(3))) unsigned char*)(p));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(q);
}

// byte offset of 16-byte segment `seg` of row `r` in a swizzled row-major
// tile of 64-element bf16 rows (conflict-free 16-byte operand reads)
__device__ __forceinline__ int swz(int r, int seg) { return r * kRowBytes + ((seg ^ (r & 7)) << 4); }

// Buffer resource over `bytes` bytes from `base`: loads past the end read
// zero, stores past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                             static_cast<int>(bytes), kBufferDword3);
}

}  // namespace mfma
}  // namespace ttt
