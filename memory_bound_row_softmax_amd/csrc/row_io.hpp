// row_io.hpp -- a lane's share of a row: which chunks it owns, loads, masks, stores.
//
// Lane l of a group of R lanes owns chunks chunk0 + i * R + l for i = 0..C-1
// (chunk = 16 bytes).  For a fixed i the R lanes touch R consecutive chunks, so
// each load instruction of a wave covers contiguous memory (1 KiB when R >= 64).
// All C loads are issued before any value is used and none sits behind a branch
// (except on the per-element path of unaligned fp32 rows, whose values need no
// conversion after the load).
//
// A RowView is a buffer resource plus the byte offset of the row inside it: one
// row per resource when a row has at least one whole wave (the resource is then
// wave-uniform and lives in scalar registers), the block's rows when several rows
// share a wave.  Reads past the end of the resource return 0 in hardware.  When a
// lane's part is not full (N does not fill the configuration), mask_part() puts a
// neutral value in the registers that hold no element of the row.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "vec_io.hpp"

namespace rr {

struct RowView {
    Buf buf;
    uint32_t base;     // byte offset of the row inside buf
    uint32_t end = 0;  // byte offset inside buf where the row (or a split row's share)
                       // ends; 0 if not known (the per-element path then reads and
                       // writes element by element throughout)
};

// Whether every element owned by lanes chunk0 .. chunk0 + C * R - 1 lies in the row.
template <class E, int C, int R>
__device__ __forceinline__ bool part_full(int chunk0, int N) {
    return (int64_t)(chunk0 + C * R) * E::VPC <= (int64_t)N;
}

// The part of a row that member `member` of the G workgroups of a split row holds:
// chunks [chunk0, chunk0 + S) with S = ceil(row chunks / G) rounded up to whole
// waves (64 chunks), so the G workgroups get equal shares even when the row does
// not fill the configuration; `nend` is the end of that part in elements (at most
// N; at or below chunk0 * VPC when the member holds nothing).  A lane still owns
// chunks chunk0 + i * R + l (i < C); those at or past `nend` belong to the next
// member and are masked, and the member's buffer resources end at `nend`, so they
// are neither read nor written.  With G = 1: the whole row.
template <int VPC, int CR, int G>
__device__ __forceinline__ void member_span(int member, int N, int *chunk0, int *nend) {
    if constexpr (G == 1) {
        *chunk0 = 0;
        *nend = N;
    } else {
        static_assert(CR % 64 == 0, "a member's part is whole waves");
        const int total = (N + VPC - 1) / VPC;
        int span = (total + G - 1) / G;
        span = (span + 63) & ~63;
        if (span > CR) span = CR;  // N beyond P * R * G: never planned
        const int c0 = member * span;
        const int64_t end = (int64_t)(c0 + span) * VPC;
        *chunk0 = c0;
        *nend = (int)(end < (int64_t)N ? end : (int64_t)N);
    }
}

// A buffer offset past every resource: loads there return 0 and touch no memory.
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

// The 16 bytes of `c` moved down by `s` bytes (s < 16), zeros shifted in at the
// top: byte j of the result is byte j + s of c.  Written as one 128-bit shift,
// which the backend expands into shifts and selects; a select in the source whose
// operand is a loaded value would be turned into a branch around that use, and the
// wait for the load would then sit inside the branch.
__device__ __forceinline__ u32x4 shift_down_bytes(u32x4 c, uint32_t s) {
    using u128 = unsigned __int128;
    const u128 w = ((u128)c[0] | ((u128)c[1] << 32) | ((u128)c[2] << 64) | ((u128)c[3] << 96)) >>
                   (8u * s);
    return u32x4{(uint32_t)w, (uint32_t)(w >> 32), (uint32_t)(w >> 64), (uint32_t)(w >> 96)};
}

// POLICY: kStreamLoad for data read once, kReuseLoad for data read by every row.
template <class E, int C, int R, bool VEC, int POLICY = kStreamLoad>
__device__ __forceinline__ void load_part(RowView rv, int chunk0, int l, float *v) {
    constexpr int VPC = E::VPC;
    if constexpr (VEC) {
        u32x4 raw[C];
#pragma unroll
        for (int i = 0; i < C; ++i)
            raw[i] = buf_load16<POLICY>(rv.buf, rv.base + (uint32_t)(chunk0 + i * R + l) * 16u);
#pragma unroll
        for (int i = 0; i < C; ++i) decode<E>(raw[i], v + i * VPC);
    } else if constexpr (E::BYTES == 4) {
        // fp32 rows that are not 16-byte aligned: a chunk that lies wholly inside the
        // row is one 16-byte load at an element-aligned offset (buffer instructions
        // take those on gfx950; measured at 93-95 % of the aligned rate), and the
        // chunk that holds the row's end is read element by element.  The branch
        // costs nothing here, since an fp32 chunk needs no conversion after the load.
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const uint32_t first = (uint32_t)(chunk0 + i * R + l) * VPC;
            const uint32_t byte0 = rv.base + first * E::BYTES;
            if (byte0 + 16u <= rv.end) {
                decode<E>(buf_load16<POLICY>(rv.buf, byte0), v + i * VPC);
            } else {
#pragma unroll
                for (int e = 0; e < VPC; ++e)
                    v[i * VPC + e] = buf_load_elem<E, POLICY>(rv.buf, byte0 + e * E::BYTES);
            }
        }
    } else if (R >= 64 || __builtin_amdgcn_readfirstlane(rv.end - rv.base) >= 16u) {
        // bf16 rows that are not 16-byte aligned.  Widening bf16 to fp32 is ALU work
        // on the loaded words; behind a per-lane branch it would make the wave wait
        // for the load inside the branch, before the next loads are issued.  So each
        // chunk is one 16-byte load at an element-aligned offset with no branch: the
        // range check zeroes every dword that crosses the end of a resource, so the
        // chunk that holds the row's end reads the 16 bytes that end at `end`, and
        // its elements are shifted into place after the load; chunks wholly past the
        // end read 0.  The loads of a part then stay in flight together, as in the
        // aligned path.  This needs rows of at least 16 bytes: plans with whole waves
        // per row (R >= 64) are only made for those, and smaller lane groups test it
        // (end - base is one row there, the same in every lane).
        u32x4 raw[C];
        uint32_t sh[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const uint32_t first = (uint32_t)(chunk0 + i * R + l) * VPC;
            const uint32_t byte0 = rv.base + first * E::BYTES;
            const bool past = byte0 >= rv.end;
            const bool tail = byte0 + 16u > rv.end;
            const uint32_t off = past ? kOutOfRange : (tail ? rv.end - 16u : byte0);
            sh[i] = (tail && !past) ? byte0 - off : 0u;
            raw[i] = buf_load16<POLICY>(rv.buf, off);
        }
#pragma unroll
        for (int i = 0; i < C; ++i) decode<E>(shift_down_bytes(raw[i], sh[i]), v + i * VPC);
    } else {
        // bf16 rows shorter than 16 bytes: element by element
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const uint32_t first = (uint32_t)(chunk0 + i * R + l) * VPC;
            const uint32_t byte0 = rv.base + first * E::BYTES;
#pragma unroll
            for (int e = 0; e < VPC; ++e)
                v[i * VPC + e] = buf_load_elem<E, POLICY>(rv.buf, byte0 + e * E::BYTES);
        }
    }
}

// The 128-bit loads of load_part without the conversion: the lane's chunks land as
// raw 32-bit words in v[0 .. 4C), bit for bit (for bf16 that is half of v; the
// rest is left unwritten, so a buffer in flight holds only P/2 live registers).
// widen_part() later turns them into the P fp32 values load_part would give.
template <class E, int C, int R, int POLICY = kStreamLoad>
__device__ __forceinline__ void load_part_raw(RowView rv, int chunk0, int l, float *v) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const u32x4 raw =
            buf_load16<POLICY>(rv.buf, rv.base + (uint32_t)(chunk0 + i * R + l) * 16u);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[4 * i + q] = __uint_as_float(raw[q]);
    }
}

// In place: the raw words of load_part_raw -> P fp32 values.  Word k holds
// elements 2k and 2k + 1 (bf16), so going from the last element down never
// overwrites a word that is still to be read.
template <class E, int C>
__device__ __forceinline__ void widen_part(float *v) {
    if constexpr (E::BYTES == 2) {
#pragma unroll
        for (int j = C * E::VPC - 1; j >= 0; --j) {
            const uint32_t w = __float_as_uint(v[j / 2]);
            v[j] = __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
        }
    }
}

// Registers that hold no element of the row get `fill`.
// OPAQUE (persistent kernels, whose row loop keeps chunk0 and N fixed): the lane's
// count of elements left in the row passes through an empty asm statement, so that
// the comparisons stay inside the row loop, where they run only for a part that is
// not full.  Left to itself, the compiler hoists all P comparisons out of the loop,
// and their P lane masks and element indices stay live in registers for every row
// (116 spilled scalar registers and some 15 vector registers in the 64-value fp32
// stream kernel).
template <class E, int C, int R, bool OPAQUE = false>
__device__ __forceinline__ void mask_part(int chunk0, int l, int N, float fill, float *v) {
    constexpr int VPC = E::VPC;
    if constexpr (OPAQUE) {
        int left = N - (chunk0 + l) * VPC;  // negative or zero: nothing of the row
        asm volatile("" : "+v"(left));
#pragma unroll
        for (int i = 0; i < C; ++i) {
#pragma unroll
            for (int e = 0; e < VPC; ++e)
                if (i * R * VPC + e >= left) v[i * VPC + e] = fill;
        }
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int first = (chunk0 + i * R + l) * VPC;
#pragma unroll
            for (int e = 0; e < VPC; ++e)
                if (first + e >= N) v[i * VPC + e] = fill;
        }
    }
}

// BOUNDED: the buffer resource holds only this row (or this split-row member's part)
// and ends where it ends, as in the persistent kernels; the hardware's range check
// then drops the stores of chunks past it, and whole waves per row store every chunk
// with no predicate.  Left to a per-chunk predicate in a row loop, the compiler hoists
// the chunks' comparisons out of the loop and keeps their lane masks live (spilled
// scalar registers).  Otherwise (block kernels, whose lane groups of fewer than 64
// lanes share one buffer across rows) each chunk is stored only if it lies in the row.
template <class E, int C, int R, bool VEC, bool BOUNDED = false>
__device__ __forceinline__ void store_part(RowView rv, int chunk0, int l, int N, bool valid,
                                           bool full, const float *v) {
    constexpr int VPC = E::VPC;
    if constexpr (VEC) {
        if constexpr (BOUNDED && R >= 64) {
            if (valid) {
#pragma unroll
                for (int i = 0; i < C; ++i)
                    buf_store16(rv.buf, rv.base + (uint32_t)(chunk0 + i * R + l) * 16u,
                                encode<E>(v + i * VPC));
            }
        } else {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                const int c = chunk0 + i * R + l;
                if (valid && (full || c * VPC < N))
                    buf_store16(rv.buf, rv.base + (uint32_t)c * 16u, encode<E>(v + i * VPC));
            }
        }
    } else {
        // As for the loads: whole chunks inside the row (and inside [0, N), the end of
        // this workgroup's part) are one 16-byte store, the rest element by element.
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int first = (chunk0 + i * R + l) * VPC;
            const uint32_t byte0 = rv.base + (uint32_t)first * E::BYTES;
            if (byte0 + 16u <= rv.end && first + VPC <= N) {
                if (valid) buf_store16(rv.buf, byte0, encode<E>(v + i * VPC));
            } else {
#pragma unroll
                for (int e = 0; e < VPC; ++e)
                    if (valid && (full || first + e < N))
                        buf_store_elem<E>(rv.buf, byte0 + (uint32_t)e * E::BYTES, v[i * VPC + e]);
            }
        }
    }
}

}  // namespace rr
