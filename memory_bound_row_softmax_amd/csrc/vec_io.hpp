// vec_io.hpp -- load/store layer: 128-bit chunks, bf16 <-> fp32, per-element fallback.
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%), section 硬件感知的加载与存储策略,
// asks that every thread move a multiple of 128 bits per access (4 x fp32 or 8 x bf16)
// so that loads and stores coalesce, with dtype conversion and the tail mask folded
// into the load.  The pages stage data through shared memory with asynchronous
// copies; here chunks go straight into VGPRs (the LDS only carries per-wave partial
// results).
//
// Every access goes through a buffer resource (base address + size in bytes): a
// 16-byte chunk per lane is one buffer_load_dwordx4 / buffer_store_dwordx4, and an
// offset at or past the end of the resource reads 0 and drops the write in
// hardware, so loads past the end of a row or of the matrix need no branch.  The
// whole offset is passed in the per-lane VGPR operand (the scalar offset operand is
// not part of the hardware range check).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Element types.  VPC = values per 16-byte chunk.
struct F32 {
    static constexpr int VPC = 4;
    static constexpr int BYTES = 4;
};
struct BF16 {
    static constexpr int VPC = 8;
    static constexpr int BYTES = 2;
};

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format; no
// swizzle, no index stride).
constexpr int kBufferWord3 = 0x00020000;

// Cache-policy bits of gfx950 buffer instructions: 1 = sc0, 2 = nt, 16 = sc1.
// Streamed data (every element read once, or written once) is loaded and stored
// with the non-temporal hint: on MI355X it raised read streams from about 6.2 to
// 7.1 TB/s and, with non-temporal stores as well, gave the best one-read-one-write
// rates of the policies tried.  Data reused across rows (the RMSNorm weight) keeps
// the default policy so that it stays in L2.
#ifndef RR_STREAM_LOAD_POLICY
#define RR_STREAM_LOAD_POLICY 2
#endif
#ifndef RR_STREAM_STORE_POLICY
#define RR_STREAM_STORE_POLICY 2
#endif
constexpr int kStreamLoad = RR_STREAM_LOAD_POLICY;
constexpr int kStreamStore = RR_STREAM_STORE_POLICY;
constexpr int kReuseLoad = 0;

struct Buf {
    __amdgpu_buffer_rsrc_t rsrc;
};

// `bytes` must be at most 2^32 - 1; callers pass one row or a few rows.
__device__ __forceinline__ Buf make_buf(const void *base, uint32_t bytes) {
    return {__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                              kBufferWord3)};
}

template <int POLICY>
__device__ __forceinline__ u32x4 buf_load16(Buf b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(b.rsrc, (int)off, 0, POLICY);
}
__device__ __forceinline__ void buf_store16(Buf b, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, b.rsrc, (int)off, 0, kStreamStore);
}

// Chunk -> VPC floats.  bf16 widens exactly: its 16 bits are the top half of an fp32.
template <class E>
__device__ __forceinline__ void decode(u32x4 c, float *f);

template <>
__device__ __forceinline__ void decode<F32>(u32x4 c, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(c[i]);
}

template <>
__device__ __forceinline__ void decode<BF16>(u32x4 c, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(c[i] << 16);
        f[2 * i + 1] = __uint_as_float(c[i] & 0xFFFF0000u);
    }
}

// VPC floats -> chunk.  bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <class E>
__device__ __forceinline__ u32x4 encode(const float *f);

template <>
__device__ __forceinline__ u32x4 encode<F32>(const float *f) {
    u32x4 c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __float_as_uint(f[i]);
    return c;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <>
__device__ __forceinline__ u32x4 encode<BF16>(const float *f) {
    u32x4 c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return c;
}

// Per-element access (rows that are not 16-byte aligned); `off` in bytes.
template <class E, int POLICY>
__device__ __forceinline__ float buf_load_elem(Buf b, uint32_t off) {
    if constexpr (E::BYTES == 4)
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(b.rsrc, (int)off, 0, POLICY));
    else
        return __uint_as_float(
            (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(b.rsrc, (int)off, 0, POLICY) << 16);
}

template <class E>
__device__ __forceinline__ void buf_store_elem(Buf b, uint32_t off, float v);

template <>
__device__ __forceinline__ void buf_store_elem<F32>(Buf b, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), b.rsrc, (int)off, 0, kStreamStore);
}

template <>
__device__ __forceinline__ void buf_store_elem<BF16>(Buf b, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16x2(v, 0.0f) & 0xFFFFu),
                                          b.rsrc, (int)off, 0, kStreamStore);
}

}  // namespace rr
